// Key-split prefill for causal or windowed launches whose one-tile-per-head
// grid leaves CUs idle (head_dim 128, fixed lengths; the host takes it where
// the paired launch would fill at most half of the CUs).
//
// It computes what fwd_prefill.hip computes (S = scale Q K^T, P = softmax(S),
// O = P V with the online softmax of "FlashAttention完整说明", section 二.1, and
// the per-row LSE of section 二.2), with another split of the work.  Under a
// causal mask the 64-row query tiles of a head carry very different numbers of
// key blocks (tile t sees t + 1 of them at s_q = s_k); pairing a light and a
// heavy tile per work group evens the work groups out, but inside one the SIMD
// that holds a light tile's wave and a heavy tile's wave runs most steps with
// one busy wave, and a lone wave leaves the MFMA unit idle while it waits for
// LDS and runs its exponentials; and a small grid leaves CUs with nothing to
// do.  Here a work group has 4 slots of 2 waves
// (32 rows each); a slot takes one 64-row tile and every kgn-th 32-key block
// of the tile's visible range, starting at block kg.  The host picks kgn per
// tile (heavy tiles get up to 4 slots, all in one work group) and packs the
// tiles into work groups so that the largest per-slot block count is as small
// as the slots allow; every SIMD (waves w and w + 4: two different slots) then
// keeps two busy waves.  The slots of one tile merge their (m, l, O) through
// LDS at the end with the log-sum-exp merge.
//
// Per slot the loop is the plain loop of the other kernel with 32-key blocks:
// S^T = K Q^T on v_mfma_f32_32x32x16 with Q^T in registers, K and V by DMA into
// the slot's own double-buffered LDS stages (8 KiB each), the lazy-reference
// exp2 softmax, O^T += V^T P^T with V^T from transposing LDS reads.
#include "device_common.h"
#include "kernels.h"
#include "tiles.h"

namespace exattn {
namespace {

constexpr float kLazyTau = 8.0f;   // move a row's reference only when its max grows by > 2^8
constexpr float kSumCap = 256.0f;  // 2^tau: a block sum below it means every p <= 2^tau

template <bool BF16, bool SOFTCAP>
__global__ void __launch_bounds__(512) prefill_slots_kernel(const SlotParams sp) {
  using E = Elem<BF16>;
  constexpr int D = 128, BN = 32;
  constexpr int KS = D / 16;                 // k-steps of the score MFMA
  constexpr int DT = D / 32;                 // 32-wide head-dim tiles of O^T
  constexpr int DCH = D / 8;                 // 16-byte chunks per row
  constexpr int KTILE = BN * D * 2;          // bytes of a K (or V) block
  constexpr int SLOT_LDS = 4 * KTILE;        // K and V, two stages
  constexpr int ROWS_PER_KB = 1024 / (D * 2);
  constexpr int KINST = KTILE / 1024 / 2;    // DMA slices per wave per block
  constexpr int XO = 8 * DT * 16 * 64 * 4;   // every wave's O^T
  constexpr int XM = 8 * 2 * 64 * 4;         // every wave's (m, l)
  constexpr int LDS = 4 * SLOT_LDS > XO + XM ? 4 * SLOT_LDS : XO + XM;
  static_assert(LDS <= 160 * 1024 && 4 * 64 * D * 2 <= LDS, "LDS budget (stages, partials, O tile)");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];
  static_assert(offsetof(SlotParams, slot) % 32 == 0, "a work group's 4 pairs are one 32-byte load");
  const FwdParams p = sp.f;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = wave >> 1;  // waves 2 s, 2 s + 1: rows 0-31 and 32-63 of slot s's tile
  const int rh = wave & 1;
  const int hsel = lane >> 5;
  const int l32 = lane & 31;
  uint8_t* const ssm = smem + slot * SLOT_LDS;

  // ---- schedule: grid (query head, batch entry, work group of the unit).
  // Work groups are dispatched in linear order, x fastest, round-robin over the
  // 8 XCDs (id % 8): when h_q x batch is a multiple of 8 every work group of a
  // head (and the heads of one KV head) reads its K / V through one XCD's L2.
  const int h = blockIdx.x, b = blockIdx.y, wgi = blockIdx.z;
  const int hk = p.group == 1 ? h : h / p.group;
  const int sq = p.s_q, sk = p.s_k, off = sk - sq;
  // visible 32-key blocks of a 64-row tile (bottom-right aligned masks)
  auto tile_range = [&](int t, int& lo, int& hi) {
    const int t0 = 64 * t, t1 = min(t0 + 64, sq) - 1;
    int kmin = 0, kmax = sk - 1;
    if (p.wl >= 0) kmin = max(0, t0 + off - p.wl);
    if (p.wr >= 0) kmax = min(kmax, t1 + off + p.wr);
    lo = 0;
    hi = 0;
    if (kmax >= kmin) {
      lo = kmin / BN;
      hi = kmax / BN + 1;
    }
  };
  const u32x8_t ws8 = *reinterpret_cast<const u32x8_t*>(sp.slot + 8 * wgi);
  // the work group's longest slot (uniform)
  const int steps = (int)max(max(ws8[1], ws8[3]), max(ws8[5], ws8[7]));
  const uint32_t e = slot == 0 ? ws8[0] : slot == 1 ? ws8[2] : slot == 2 ? ws8[4] : ws8[6];
  const int nb = (int)(slot == 0 ? ws8[1] : slot == 1 ? ws8[3] : slot == 2 ? ws8[5] : ws8[7]);
  const bool used = (e >> 24) & 1u;
  const int tile = (int)(e & 0xffffu);
  const int kg = (int)((e >> 16) & 7u);
  const int kgn = max(1, (int)((e >> 19) & 7u));
  int lo, hi_;
  tile_range(tile, lo, hi_);
  auto blk = [&](int i) { return lo + kg + kgn * i; };

  const int64_t qoff = (int64_t)b * p.q_sb, koff = (int64_t)b * p.k_sb, voff = (int64_t)b * p.v_sb;
  const int q0 = 64 * tile;
  const int q_last = min(q0 + 64, sq) - 1;
  const int qrow = q0 + 32 * rh + l32;
  const bool valid = used && qrow < sq;

  // ---- Q^T fragments: lane holds Q[qrow][16 ks + 8 hsel .. +7] for every ks.
  u32x4_t qf[KS];
  if (valid) {
    const uint16_t* qp = p.q + qoff + (int64_t)h * p.q_sh + (int64_t)qrow * p.q_ss + 8 * hsel;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const u32x4_t*)(qp + 16 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = u32x4_t{0, 0, 0, 0};
  }

  // ---- K and V blocks by DMA into the slot's stages: wave rh of the slot
  // fills 1 KiB slices 2 i + rh; lane l writes slot l of the slice (row l / DCH,
  // stored chunk l % DCH), fetching global chunk (l % DCH) ^ swizzle(row).
  const uint16_t* kgp = p.k + koff + (int64_t)hk * p.k_sh;
  const uint16_t* vgp = p.v + voff + (int64_t)hk * p.v_sh;
  uint32_t kofs[KINST], vofs[KINST];
#pragma unroll
  for (int i = 0; i < KINST; ++i) {
    const int row = (2 * i + rh) * ROWS_PER_KB + lane / DCH;
    kofs[i] = (uint32_t)(row * p.k_ss + 8 * ((lane % DCH) ^ kswz<D>(row))) * 2u;
    vofs[i] = (uint32_t)(row * p.v_ss + 8 * ((lane % DCH) ^ vswz<D>(row))) * 2u;
  }
  auto issue_k = [&](int n, uint8_t* dst) {
    const __amdgpu_buffer_rsrc_t rk = block_rsrc<D>(kgp, p.k_ss, n * BN, sk, BN);
#pragma unroll
    for (int i = 0; i < KINST; ++i) buffer_load_lds16(rk, dst + (2 * i + rh) * 1024, kofs[i]);
  };
  auto issue_v = [&](int n, uint8_t* dst) {
    const __amdgpu_buffer_rsrc_t rv = block_rsrc<D>(vgp, p.v_ss, n * BN, sk, BN);
#pragma unroll
    for (int i = 0; i < KINST; ++i) buffer_load_lds16(rv, dst + (2 * i + rh) * 1024, vofs[i]);
  };
  uint8_t* const k0 = ssm;
  uint8_t* const k1 = ssm + KTILE;
  uint8_t* const v0 = ssm + 2 * KTILE;
  uint8_t* const v1 = ssm + 3 * KTILE;
  if (nb > 0) {
    issue_k(blk(0), k0);
    issue_v(blk(0), v0);
  }

  // ---- loop-invariant LDS operand addresses (as in the other prefill kernel).
  const int krow = row_key(l32);
  const int ksw = kswz<D>(krow);
  int kaddr[8];
#pragma unroll
  for (int bq = 0; bq < 8; ++bq) kaddr[bq] = krow * (D * 2) + 32 * (bq ^ (ksw >> 1)) + 16 * (hsel ^ (ksw & 1));
  const int gi = lane >> 4, li = lane & 15;
  int vtr[2][DT];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int key = 8 * (gi >> 1) + 4 * half + (li >> 2);
      const int dcol = 32 * dt + 16 * (gi & 1) + 4 * (li & 3);
      vtr[half][dt] = key * (D * 2) + 16 * ((dcol >> 3) ^ vswz<D>(key)) + 2 * (dcol & 7);
    }

  // ---- masks: keys <= full_r and >= full_l are visible to every row of the
  // tile; this lane's row sees keys mlo + 8 hsel .. mhi + 8 hsel.
  const int qpos = min(qrow, sq - 1);
  const int full_r = p.wr >= 0 ? min(sk - 1, q0 + off + p.wr) : sk - 1;
  const int full_l = p.wl >= 0 ? q_last + off - p.wl : -0x3fffffff;
  const int mhi = (p.wr >= 0 ? min(sk - 1, qpos + off + p.wr) : sk - 1) - 8 * hsel;
  const int mlo = (p.wl >= 0 ? qpos + off - p.wl : -0x3fffffff) - 8 * hsel;

  f32x16_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16_t{};
  float m_ref = kNegInf;  // reference max (log2 domain) of this lane's row
  float l_run = 0.f;      // this lane's share of the row sum, relative to m_ref

  auto exps = [&](const f32x16_t& s, u32x4_t (&pf)[2], float base) {
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float x0, x1;
      if constexpr (SOFTCAP) {
        const float a0 = s[r], a1 = s[r + 1];
        x0 = a0 == kNegInf ? kNegInf : p.cap_out_log2 * tanh_exp2(a0 * p.cap_in) - base;
        x1 = a1 == kNegInf ? kNegInf : p.cap_out_log2 * tanh_exp2(a1 * p.cap_in) - base;
      } else {
        x0 = __builtin_fmaf(s[r], p.scale_log2, -base);
        x1 = __builtin_fmaf(s[r + 1], p.scale_log2, -base);
      }
      x0 = fast_exp2(x0);
      x1 = fast_exp2(x1);
      pf[r >> 3][(r & 7) >> 1] = E::pack2(x0, x1);
      psum += x0 + x1;
    }
    return psum;
  };
  auto slow = [&](const f32x16_t& s, u32x4_t (&pf)[2]) {
    float mraw = s[0];
#pragma unroll
    for (int r = 0; r < 16; ++r) mraw = fmaxf(mraw, s[r]);
    mraw = halves_max(mraw);
    float m_blk;
    if constexpr (SOFTCAP)
      m_blk = mraw == kNegInf ? kNegInf : p.cap_out_log2 * tanh_exp2(mraw * p.cap_in);
    else
      m_blk = mraw * p.scale_log2;
    const bool need = m_blk > m_ref + kLazyTau;
    const float m_new = need ? m_blk : m_ref;
    const float alpha = need ? fast_exp2(m_ref - m_new) : 1.f;
    if (__ballot(need && m_ref != kNegInf) != 0) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    }
    l_run *= alpha;
    m_ref = m_new;
    return exps(s, pf, m_ref == kNegInf ? 0.f : m_ref);
  };
  auto v_operand = [&](const uint8_t* __restrict__ vs_, int c, int dt) {
    const int rows = 16 * c * (D * 2);
    const u32x2_t lo2 = lds_read_tr16(vs_ + vtr[0][dt] + rows);
    const u32x2_t hi2 = lds_read_tr16(vs_ + vtr[1][dt] + rows);
    return u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]};
  };
  // S^T of one 32-key block: all 8 K reads go out ahead of the MFMAs
  auto qk = [&](const uint8_t* __restrict__ ks_, f32x16_t& s) {
    s = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = E::mfma32x32x16(*(const u32x4_t*)(ks_ + kaddr[ks]), qf[ks], s);
    __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, KS, 0);
  };
  // softmax of the block into P^T, then O^T += V^T P^T
  auto softmax_pv = [&](const uint8_t* __restrict__ vs_, const f32x16_t& s) {
    u32x4_t pf[2];
    u32x4_t vpre[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vpre[dt] = v_operand(vs_, 0, dt);
    float psum = 0.f;
    bool ok = false;
    if (__ballot(m_ref == kNegInf) == 0) {
      psum = exps(s, pf, m_ref);
      ok = __ballot(!(psum <= kSumCap)) == 0;
    }
    if (!ok) psum = slow(s, pf);
    l_run += psum;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        oacc[dt] = E::mfma32x32x16(c == 0 ? vpre[dt] : v_operand(vs_, c, dt), pf[c], oacc[dt]);
  };
  // step i: DMA of the slot's next block into the other stage (K now, V after
  // the score MFMAs), then block i
  auto step = [&](const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc, uint8_t* __restrict__ kn,
                  uint8_t* __restrict__ vn, int i) {
    const bool more = i + 1 < nb;
    if (more) issue_k(blk(i + 1), kn);
    if (i < nb) {
      f32x16_t s;
      qk(kc, s);
      __builtin_amdgcn_sched_barrier(0);
      if (more) issue_v(blk(i + 1), vn);
      const int kb = blk(i) * BN;
      if (kb + BN - 1 > full_r || kb < full_l) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 16 * (r >> 3) + (r & 7);
          if (kk > mhi - kb || kk < mlo - kb) s[r] = kNegInf;
        }
      }
      softmax_pv(vc, s);
    }
  };
  if (p.q_sign != 0u) {  // negative softmax scale: negate Q exactly, use |scale|
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] ^= u32x4_t{p.q_sign, p.q_sign, p.q_sign, p.q_sign};
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
  for (int i = 0; i < steps; i += 2) {
    wait_vmem_all();
    __syncthreads();
    step(k0, v0, k1, v1, i);
    if (i + 1 < steps) {
      wait_vmem_all();
      __syncthreads();
      step(k1, v1, k0, v0, i + 1);
    }
  }
  wait_vmem_all();

  // ---- epilogue.  The slots of a split tile publish (m, l) and O^T through
  // LDS (the stages are free after the barrier); wave (kg, rh) then merges the
  // head-dim tiles dt with dt % kgn == kg of its 32 rows from the kgn partials
  // with the log-sum-exp merge (a tile held by one slot keeps its registers).
  // O = O^T / l, rounded, goes through an LDS tile so that global stores
  // cover whole rows (16 lanes x 16 bytes per row instead of 32 rows x 8
  // bytes per instruction), and kg 0 writes LSE = (m + log2 l) ln 2.  Empty
  // rows give 0 and -inf.
  const float l_tot = halves_sum(l_run);
  float* const xm = reinterpret_cast<float*>(smem + XO);
  f32x4_t* const xo4 = reinterpret_cast<f32x4_t*>(smem);  // [wave][d tile][r / 4][lane][r % 4]
  __syncthreads();
  if (kgn > 1) {
    xm[(wave * 2 + 0) * 64 + lane] = m_ref;
    xm[(wave * 2 + 1) * 64 + lane] = l_tot;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      if (dt % kgn != kg) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          xo4[((wave * DT + dt) * 4 + r4) * 64 + lane] =
              f32x4_t{oacc[dt][4 * r4], oacc[dt][4 * r4 + 1], oacc[dt][4 * r4 + 2], oacc[dt][4 * r4 + 3]};
      }
  }
  __syncthreads();
  const int first = slot - kg;  // the tile's first slot
  float m_fin = m_ref, l_fin = l_tot;
  if (kgn > 1) {
    float mm = kNegInf;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < kgn) mm = fmaxf(mm, xm[((2 * (first + k) + rh) * 2 + 0) * 64 + lane]);
    const float bm = mm == kNegInf ? 0.f : mm;
    float wt[4];  // weight of each partial relative to bm (0 for an empty one)
    float lw = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int wk = 2 * (first + k) + rh;
      wt[k] = k < kgn ? fast_exp2(xm[(wk * 2 + 0) * 64 + lane] - bm) : 0.f;
      if (k < kgn) lw += wt[k] * xm[(wk * 2 + 1) * 64 + lane];
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      if (dt % kgn == kg) {
        f32x16_t acc = oacc[dt] * (kg == 0 ? wt[0] : kg == 1 ? wt[1] : kg == 2 ? wt[2] : wt[3]);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (k < kgn && k != kg) {
            const int wk = 2 * (first + k) + rh;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const f32x4_t o1 = xo4[((wk * DT + dt) * 4 + r4) * 64 + lane];
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[4 * r4 + e] += wt[k] * o1[e];
            }
          }
        oacc[dt] = acc;
      }
    m_fin = mm;
    l_fin = lw;
  }
  __syncthreads();  // the O tile overwrites the published partials
  constexpr int OROW = D * 2;  // bytes per row of the O tile: 64 rows per slot
  const float inv = l_fin > 0.f ? 1.0f / l_fin : 0.f;
  const int orow = 64 * first + 32 * rh + l32;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    if (dt % kgn == kg) {
#pragma unroll
      for (int J = 0; J < 4; ++J) {  // head dims 32 dt + 8 J + 4 hsel + 0..3
        u32x2_t w;
        w[0] = E::pack2(oacc[dt][4 * J] * inv, oacc[dt][4 * J + 1] * inv);
        w[1] = E::pack2(oacc[dt][4 * J + 2] * inv, oacc[dt][4 * J + 3] * inv);
        const int chunk = 4 * dt + J;
        *(u32x2_t*)(smem + orow * OROW + 16 * (chunk ^ kswz<D>(orow)) + 8 * hsel) = w;
      }
    }
  __syncthreads();
  if (kg == 0 && valid && hsel == 0 && p.lse != nullptr)
    p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + qrow] =
        l_fin > 0.f ? (m_fin + fast_log2(l_fin)) * kLn2 : kNegInf;
  // O tile -> global, 16 bytes per thread: rows 64 s .. 64 s + 63 belong to
  // the tile whose first slot is s
#pragma unroll
  for (int it = 0; it < 4 * 64 * DCH / 512; ++it) {
    const int idx = it * 512 + tid;
    const int row = idx / DCH, chunk = idx % DCH;
    const int rs = row >> 6;
    const uint32_t es = rs == 0 ? ws8[0] : rs == 1 ? ws8[2] : rs == 2 ? ws8[4] : ws8[6];
    const int grow = 64 * (int)(es & 0xffffu) + (row & 63);
    if (((es >> 24) & 1u) && ((es >> 16) & 7u) == 0 && grow < sq) {
      const u32x4_t v = *(const u32x4_t*)(smem + row * OROW + 16 * (chunk ^ kswz<D>(row)));
      *(u32x4_t*)(p.o + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)grow * p.o_ss + 8 * chunk) = v;
    }
  }
}

}  // namespace

hipError_t launch_prefill_slots(const SlotParams& sp, bool bf16, bool softcap, hipStream_t stream) {
  const dim3 grid(sp.f.h_q, sp.f.batch, sp.n_wg);
  if (bf16) {
    if (softcap)
      hipLaunchKernelGGL((prefill_slots_kernel<true, true>), grid, dim3(512), 0, stream, sp);
    else
      hipLaunchKernelGGL((prefill_slots_kernel<true, false>), grid, dim3(512), 0, stream, sp);
  } else {
    if (softcap)
      hipLaunchKernelGGL((prefill_slots_kernel<false, true>), grid, dim3(512), 0, stream, sp);
    else
      hipLaunchKernelGGL((prefill_slots_kernel<false, false>), grid, dim3(512), 0, stream, sp);
  }
  return hipGetLastError();
}

}  // namespace exattn
