// Prefill forward at head_dim 256 with the head dims split between two waves.
//
// It computes what fwd_prefill.hip computes (S = scale Q K^T, P = softmax(S),
// O = P V with the online softmax of "FlashAttention完整说明", section 二.1, and
// the per-row LSE of section 二.2).  At d = 256 one wave holding 32 rows needs
// Q^T (64 registers) and O^T (128) besides its scores and operands, more than
// the 256 registers a wave gets when two waves share a SIMD, so the general
// kernel runs one wave per SIMD there, and a lone wave leaves the MFMA unit
// idle while it waits for LDS and runs its exponentials.  Here two waves share
// 32 rows: wave half hh holds Q^T and O^T for head dims 128 hh .. 128 hh + 127
// only.  Per 32-key block each computes its half of S^T = K Q^T (the sum over
// its 128 dims), the two halves are added through LDS (own + partner: the same
// sum bitwise in both waves), both run the same masks and online softmax on the
// same scores, and each accumulates O^T += V^T P^T for its half of the dims.
// No MFMA work is repeated; the exponentials are, which at d = 256 costs what
// d = 128 costs once.  A work group is 8 waves, two per SIMD: phase group
// pg = wave >> 2, half hh = (wave >> 1) & 1, and the waves of a group cover
// 32-row slices.  With one key group a tile has 128 rows (the slices of both
// phase groups) and every wave takes every key block; with two, a tile has 64
// rows and phase group g takes the key blocks n_lo + g + 2 j, the two partial
// results merging at the end.  Phase group 1 runs half a block behind group 0
// (one barrier apart), so each SIMD holds one wave computing its S^T half beside
// one running its exponentials and PV.  Measured on MI355X against the general
// kernel's one-wave-per-SIMD launch: b2 s1024 h8 non-causal 45 -> 30 us (two
// key groups), b4 s2048 h16 non-causal and b2 s4096 h16 causal 2-4% faster
// (one key group).  A version taking the PV of block j - 1 beside the softmax
// of block j measured the same on the first and 8-10% slower on the others;
// one with QK and PV in one phase and the softmax in the other measured 5%
// slower on all.
//
// K and V blocks go by DMA into double-buffered LDS stages (16 KiB each), with
// the chunk swizzles of the other kernels; V^T comes from transposing LDS
// reads; scores stay in the log2 domain with a lazy reference (moved only when
// a block's max exceeds it by more than 2^8).
#include "device_common.h"
#include "kernels.h"
#include "tiles.h"

namespace exattn {
namespace {

// Work-group barrier ordering LDS accesses only: unlike __syncthreads it does not
// wait for outstanding global loads, so a DMA into another stage stays in flight.
// The scheduling barriers keep the compiler from moving arithmetic (MFMAs)
// across it, which would merge the phases it separates.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// 16 bytes per lane from global memory into LDS at lds + 16 * lane (lds
// wave-uniform; the descriptor is that of block_rsrc).  Issued from inline asm
// so that the compiler does not track it: tracked, every LDS read after it
// waits for it (the compiler cannot tell that the read is from another stage),
// which would stall each phase on the next block's load.  Callers wait for it
// with s_waitcnt vmcnt before the barrier that publishes the stage.
__device__ __forceinline__ void dma16(const uint16_t* g, int64_t ss, int kb, int sk, int rows, uint8_t* lds,
                                      uint32_t voffset) {
  const int64_t last = (int64_t)min(sk - 1 - kb, rows - 1) * ss + 256;  // elements to the end of the last row
  const uint64_t base = (uint64_t)(g + (int64_t)kb * ss);
  const u32x4_t rsrc = {(uint32_t)base, (uint32_t)(base >> 32) & 0xffffu, (uint32_t)(last * 2), 0x00020000u};
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}

constexpr float kLazyTau = 8.0f;   // move a row's reference only when its max grows by > 2^8
constexpr float kSumCap = 256.0f;  // 2^tau: a block sum below it means every p <= 2^tau

template <bool BF16, bool SOFTCAP, int NG>
__global__ void __launch_bounds__(512) prefill_dsplit_kernel(const FwdParams p) {
  using E = Elem<BF16>;
  constexpr int D = 256, DH = 128, BN = 32;
  constexpr int TM = 64 * (3 - NG);         // rows per tile: 128 or 64
  constexpr int KS = DH / 16;               // k-steps of this wave's half of the score MFMA
  constexpr int DT = DH / 32;               // 32-wide head-dim tiles of this wave's O^T
  constexpr int DCH = D / 8;                // 16-byte chunks per row
  constexpr int KTILE = BN * D * 2;         // bytes of a K (or V) block: 16 KiB
  constexpr int ROWS_PER_KB = 1024 / (D * 2);
  constexpr int KINST = KTILE / 1024 / 4;   // DMA slices per wave per K (or V) block
  constexpr int STAGES = NG * 4 * KTILE;    // per group: K and V, two stages each
  constexpr int XS = 8 * 16 * 64 * 4;       // every wave's half scores
  constexpr int LDS = STAGES + XS;
  static_assert(KINST >= 1 && LDS <= 160 * 1024, "LDS budget");
  static_assert(TM * D * 2 + (NG - 1) * (8 * 2 * 16 * 64 * 4 + 8 * 2 * 64 * 4) <= STAGES, "epilogue");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pg = wave >> 2;         // phase group: SIMD s holds waves s (group 0) and s + 4 (group 1)
  const int hh = (wave >> 1) & 1;   // head-dim half; the partner is wave ^ 2
  const int rs = NG == 1 ? 2 * pg + (wave & 1) : (wave & 1);  // 32-row slice of the tile
  const int kg = NG == 1 ? 0 : pg;  // key group: blocks n_lo + kg, n_lo + kg + NG, ...
  const int hsel = lane >> 5;
  const int l32 = lane & 31;

  // ---- grid (query head, batch entry or sequence, tile), heaviest tile first.
  const int h = blockIdx.x, b = blockIdx.y;
  const int qt = p.n_qt - 1 - (int)blockIdx.z;
  const int hk = p.group == 1 ? h : h / p.group;
  int sq = p.s_q, sk = p.s_k;
  int64_t qoff, koff, voff, ooff, lseoff;
  if (p.cu_q != nullptr) {
    const int qs = p.cu_q[b], ks = p.cu_k[b];
    sq = p.cu_q[b + 1] - qs;
    sk = p.cu_k[b + 1] - ks;
    qoff = (int64_t)qs * p.q_ss;
    ooff = (int64_t)qs * p.o_ss;
    koff = (int64_t)ks * p.k_ss;
    voff = (int64_t)ks * p.v_ss;
    lseoff = qs;
  } else {
    qoff = (int64_t)b * p.q_sb;
    ooff = (int64_t)b * p.o_sb;
    koff = (int64_t)b * p.k_sb;
    voff = (int64_t)b * p.v_sb;
    lseoff = (int64_t)b * p.lse_sb;
  }
  const int q0 = TM * qt;
  if (q0 >= sq) return;  // uniform: a shorter sequence has no rows here
  const int off = sk - sq;
  const int q_last = min(q0 + TM, sq) - 1;
  const int qrow = q0 + 32 * rs + l32;
  const bool valid = qrow < sq;

  // ---- Q^T fragments of this half: lane holds Q[qrow][128 hh + 16 ks + 8 hsel .. +7].
  u32x4_t qf[KS];
  if (valid) {
    const uint16_t* qp = p.q + qoff + (int64_t)h * p.q_sh + (int64_t)qrow * p.q_ss + DH * hh + 8 * hsel;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const u32x4_t*)(qp + 16 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = u32x4_t{0, 0, 0, 0};
  }

  // ---- visible 32-key blocks [lo, hi) of the tile's rows (bottom-right aligned).
  int kmin = 0, kmax = sk - 1;
  if (p.wl >= 0) kmin = max(0, q0 + off - p.wl);
  if (p.wr >= 0) kmax = min(kmax, q_last + off + p.wr);
  const int n_lo = kmax >= kmin ? kmin / BN : 0;
  const int n_hi = kmax >= kmin ? kmax / BN + 1 : 0;

  // ---- K and V by DMA: the 4 waves of a phase group fill 1 KiB slices
  // (wave & 3) + 4 i of a block; lane l writes slot l of the slice (row l / DCH,
  // stored chunk l % DCH), fetching global chunk (l % DCH) ^ swizzle(row).  With
  // one key group, group 0 loads the K blocks and group 1 the V blocks; with
  // two, each group loads both of its own blocks.
  const uint16_t* kgp = p.k + koff + (int64_t)hk * p.k_sh;
  const uint16_t* vgp = p.v + voff + (int64_t)hk * p.v_sh;
  uint32_t kofs[KINST], vofs[KINST];
#pragma unroll
  for (int i = 0; i < KINST; ++i) {
    const int row = (4 * i + (wave & 3)) * ROWS_PER_KB + lane / DCH;
    kofs[i] = (uint32_t)(row * p.k_ss + 8 * ((lane % DCH) ^ kswz<D>(row))) * 2u;
    vofs[i] = (uint32_t)(row * p.v_ss + 8 * ((lane % DCH) ^ vswz<D>(row))) * 2u;
  }
  uint8_t* const kst = smem + kg * 4 * KTILE;  // K stages 0, 1, then V stages 0, 1
  uint8_t* const vst = kst + 2 * KTILE;
  // DMA of the group's block ordinal j (block n_lo + kg + NG j) into stage j & 1
  auto issue = [&](int j, const int st) __attribute__((always_inline)) {
    const int n = n_lo + kg + NG * j;
    if (NG == 2 || pg == 0) {
#pragma unroll
      for (int i = 0; i < KINST; ++i)
        dma16(kgp, p.k_ss, n * BN, sk, BN, kst + st * KTILE + (4 * i + (wave & 3)) * 1024, kofs[i]);
    }
    if (NG == 2 || pg == 1) {
#pragma unroll
      for (int i = 0; i < KINST; ++i)
        dma16(vgp, p.v_ss, n * BN, sk, BN, vst + st * KTILE + (4 * i + (wave & 3)) * 1024, vofs[i]);
    }
  };
  // blocks of this wave's key group
  const int nb_g = NG == 1 ? n_hi - n_lo : max(0, (n_hi - n_lo - kg + 1) / 2);
  const int nb_0 = NG == 1 ? n_hi - n_lo : (n_hi - n_lo + 1) / 2;  // group 0's, the larger count
  f32x4_t* const xs4 = reinterpret_cast<f32x4_t*>(smem + STAGES);  // [wave][r4][lane]
  if (nb_g > 0) issue(0, 0);

  // ---- loop-invariant LDS operand addresses.
  // K operand of MFMA ks: key row_key(l32), head dims 128 hh + 16 ks + 8 hsel ..
  // +7, i.e. chunk 16 hh + 2 ks + hsel, stored at that ^ kswz(key).
  const int krow = row_key(l32);
  const int ksw = kswz<D>(krow);
  int kaddr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    kaddr[ks] = kg * 4 * KTILE + krow * (D * 2) + 32 * (8 * hh + (ks ^ (ksw >> 1))) + 16 * (hsel ^ (ksw & 1));
  // V^T operand of MFMA (c, dt): head dims 128 hh + 32 dt + ..., keys 16 c + ...
  const int gi = lane >> 4, li = lane & 15;
  // (the second read of an operand is 4 keys further: the same swizzle, +2 KiB)
  int vtr[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int key = 8 * (gi >> 1) + (li >> 2);
    const int dcol = DH * hh + 32 * dt + 16 * (gi & 1) + 4 * (li & 3);
    vtr[dt] = (kg * 4 + 2) * KTILE + key * (D * 2) + 16 * ((dcol >> 3) ^ vswz<D>(key)) + 2 * (dcol & 7);
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

  auto exps = [&](const f32x16_t& s, u32x4_t (&pf)[2], float base) __attribute__((always_inline)) {
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
  auto slow = [&](const f32x16_t& s, u32x4_t (&pf)[2]) __attribute__((always_inline)) {
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
  // (stage st; the addresses above hold the group's stage base)
  auto v_operand = [&](int st, int c, int dt) __attribute__((always_inline)) {
    const int rows = st * KTILE + 16 * c * (D * 2);
    const u32x2_t lo2 = lds_read_tr16(smem + vtr[dt] + rows);
    const u32x2_t hi2 = lds_read_tr16(smem + vtr[dt] + rows + 4 * (D * 2));
    return u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]};
  };
  // softmax of the block's full scores into P^T, then this half's O^T += V^T P^T
  auto softmax_pv = [&](const u32x4_t (&vop)[2][DT], const f32x16_t& s) __attribute__((always_inline)) {
    u32x4_t pf[2];
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
        oacc[dt] = E::mfma32x32x16(vop[c][dt], pf[c], oacc[dt]);
  };
  // The S^T half of the group's block ordinal j (stage j & 1) -> s, published
  // to the partner through this wave's exchange slot.
  auto qk_part = [&](const int st, f32x16_t& s) __attribute__((always_inline)) {
    u32x4_t kop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kop[ks] = *(const u32x4_t*)(smem + st * KTILE + kaddr[ks]);
    s = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = E::mfma32x32x16(kop[ks], qf[ks], s);
    __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);  // all K reads first
    __builtin_amdgcn_sched_group_barrier(0x008, KS, 0);
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      xs4[(wave * 4 + r4) * 64 + lane] = f32x4_t{s[4 * r4], s[4 * r4 + 1], s[4 * r4 + 2], s[4 * r4 + 3]};
  };
  // The partner's half added, masks, softmax, and O^T += V^T P^T for block ordinal j.
  auto pv_part = [&](int j, const int st, f32x16_t& s) __attribute__((always_inline)) {
    f32x4_t o[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) o[r4] = xs4[((wave ^ 2) * 4 + r4) * 64 + lane];
    u32x4_t vop[2][DT];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vop[c][dt] = v_operand(st, c, dt);
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * r4 + e] += o[r4][e];
    const int kb = (n_lo + kg + NG * j) * BN;
    if (kb + BN - 1 > full_r || kb < full_l) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 16 * (r >> 3) + (r & 7);
        if (kk > mhi - kb || kk < mlo - kb) s[r] = kNegInf;
      }
    }
    softmax_pv(vop, s);
  };
  if (p.q_sign != 0u) {  // negative softmax scale: negate Q exactly, use |scale|
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] ^= u32x4_t{p.q_sign, p.q_sign, p.q_sign, p.q_sign};
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
  // Every wave runs the same loop: per block ordinal j, a barrier, the DMA of
  // block j + 1 and the S^T half of block j, a barrier, then softmax and PV of
  // block j.  Group 1 passes one barrier before its loop, so it runs half a
  // block behind group 0: while one wave of a SIMD runs its QK MFMAs the other
  // runs its exponentials and PV.  Between barriers 2j and 2j + 1 group 0 takes
  // QK(j) and group 1 PV(j - 1); between 2j + 1 and 2j + 2 group 0 takes PV(j)
  // and group 1 QK(j).  A group waits for its own DMA before the barrier that
  // opens its QK phase; the barriers themselves wait for LDS only, so a DMA in
  // flight crosses them.  With one key group both groups take every block
  // (group 0 loads K, group 1 V); with two, group g takes blocks n_lo + g + 2 j.
  // A stage is reloaded only after the barrier that ends its last reader's
  // phase.  All waves pass 2 nb_0 + 1 barriers: the loop's, group 1's first,
  // and filler ones at the end.
  f32x16_t s;
  auto body = [&](int j, const int st) __attribute__((always_inline)) {
    wait_vmem_all();
    lds_barrier();
    if (j + 1 < nb_g) issue(j + 1, st ^ 1);
    qk_part(st, s);
    lds_barrier();
    pv_part(j, st, s);
  };
  if (pg == 1) lds_barrier();
  for (int j = 0; j < nb_g; j += 2) {  // two ordinals per pass: constant stage offsets
    body(j, 0);
    if (j + 1 < nb_g) body(j + 1, 1);
  }
  for (int k = 2 * nb_g + pg; k < 2 * nb_0 + 1; ++k) lds_barrier();
  wait_vmem_all();
  __syncthreads();  // the stages are free

  // ---- epilogue.  Both halves of a row hold the same (m, l).  With two key
  // groups the groups' (m, l, O^T) are merged first (the log-sum-exp merge of
  // the online softmax), group kg finalizing d tiles 2 kg and 2 kg + 1 of its
  // half.  O = O^T / l, rounded, goes through an LDS tile so that global stores
  // cover whole rows; LSE = (m + log2 l) ln 2.  Empty rows give 0 and -inf.
  uint8_t* const otile = smem;
  const int orow = 32 * rs + l32;
  auto put = [&](const f32x16_t& o, int dt, float inv) __attribute__((always_inline)) {
#pragma unroll
    for (int J = 0; J < 4; ++J) {  // head dims 128 hh + 32 dt + 8 J + 4 hsel + 0..3
      u32x2_t w;
      w[0] = E::pack2(o[4 * J] * inv, o[4 * J + 1] * inv);
      w[1] = E::pack2(o[4 * J + 2] * inv, o[4 * J + 3] * inv);
      const int chunk = 16 * hh + 4 * dt + J;
      *(u32x2_t*)(otile + orow * (D * 2) + 16 * (chunk ^ kswz<D>(orow)) + 8 * hsel) = w;
    }
  };
  float l_tot = halves_sum(l_run);
  float m_fin = m_ref;
  if constexpr (NG == 1) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) put(oacc[dt], dt, inv);
  } else {
    // [wave][j][r4][lane] f32x4 of the two d tiles the partner group finalizes
    f32x4_t* const xo4 = reinterpret_cast<f32x4_t*>(smem + TM * D * 2);
    float* const xm = reinterpret_cast<float*>(smem + TM * D * 2 + 8 * 2 * 16 * 64 * 4);  // [wave][2][lane]
    const int pw = wave ^ 4;
    auto send = [&](int dt0) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          xo4[((wave * 2 + j) * 4 + r4) * 64 + lane] =
              f32x4_t{oacc[dt0 + j][4 * r4], oacc[dt0 + j][4 * r4 + 1], oacc[dt0 + j][4 * r4 + 2],
                      oacc[dt0 + j][4 * r4 + 3]};
    };
    if (kg == 0)
      send(2);
    else
      send(0);
    xm[(wave * 2 + 0) * 64 + lane] = m_ref;
    xm[(wave * 2 + 1) * 64 + lane] = l_tot;
    __syncthreads();
    const float m_o = xm[(pw * 2 + 0) * 64 + lane];
    const float l_o = xm[(pw * 2 + 1) * 64 + lane];
    const float mm = fmaxf(m_ref, m_o);
    const float a_s = m_ref == kNegInf ? 0.f : fast_exp2(m_ref - mm);
    const float a_o = m_o == kNegInf ? 0.f : fast_exp2(m_o - mm);
    l_tot = l_tot * a_s + l_o * a_o;
    m_fin = mm;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    auto fin = [&](int dt0) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f32x16_t o;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4_t x = xo4[((pw * 2 + j) * 4 + r4) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[4 * r4 + e] = oacc[dt0 + j][4 * r4 + e] * a_s + x[e] * a_o;
        }
        put(o, dt0 + j, inv);
      }
    };
    if (kg == 0)
      fin(0);
    else
      fin(2);
  }
  __syncthreads();
  if (hh == 0 && kg == 0 && valid && hsel == 0 && p.lse != nullptr)
    p.lse[lseoff + (int64_t)h * p.lse_sh + qrow] = l_tot > 0.f ? (m_fin + fast_log2(l_tot)) * kLn2 : kNegInf;
#pragma unroll
  for (int it = 0; it < TM * DCH / 512; ++it) {
    const int idx = it * 512 + tid;
    const int row = idx / DCH, chunk = idx % DCH;
    if (q0 + row < sq) {
      const u32x4_t val = *(const u32x4_t*)(otile + row * (D * 2) + 16 * (chunk ^ kswz<D>(row)));
      *(u32x4_t*)(p.o + ooff + (int64_t)h * p.o_sh + (int64_t)(q0 + row) * p.o_ss + 8 * chunk) = val;
    }
  }
}

template <bool BF16, int NG>
void launch_ng(const FwdParams& p, bool softcap, hipStream_t stream) {
  const dim3 grid(p.h_q, p.batch, p.n_qt);
  if (softcap)
    hipLaunchKernelGGL((prefill_dsplit_kernel<BF16, true, NG>), grid, dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_dsplit_kernel<BF16, false, NG>), grid, dim3(512), 0, stream, p);
}

}  // namespace

hipError_t launch_prefill_dsplit(const FwdParams& p, bool bf16, int groups, bool softcap,
                                 hipStream_t stream) {
  if (groups != 1 && groups != 2) return hipErrorInvalidValue;
  if (bf16) {
    if (groups == 1)
      launch_ng<true, 1>(p, softcap, stream);
    else
      launch_ng<true, 2>(p, softcap, stream);
  } else {
    if (groups == 1)
      launch_ng<false, 1>(p, softcap, stream);
    else
      launch_ng<false, 2>(p, softcap, stream);
  }
  return hipGetLastError();
}

}  // namespace exattn
