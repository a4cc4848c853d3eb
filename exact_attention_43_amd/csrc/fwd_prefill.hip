// Prefill forward kernel: exact attention, tiled, with an online softmax.
//
// What it computes is S = scale * Q K^T, P = softmax(S), O = P V per query head
// ("FlashAttention完整说明", section 一, equations (1)-(3)).  Q/K/V are cut into
// tiles that fit on chip and the per-tile results are merged by the running
// max / running sum rescaling of the online softmax, so the full S and P never
// exist in device memory (same page, section 二.1).  Only O and the per-row
// log-sum-exp are written (same page, section 二.2).
//
// gfx950 design (not the pages' CUDA design):
// - work group = 4 waves x 32 query rows = 128 rows of one query head; KV
//   blocks of 64 keys;
// - the wave computes S^T = K Q^T with v_mfma_f32_32x32x16 (bf16/f16, fp32
//   accumulate): K is the A operand read from LDS, Q^T the B operand held in
//   registers for the whole loop.  In the 32x32 accumulator layout every lane
//   owns ONE query row, so row max and row sum are in-lane, plus one
//   exchange between the two 32-lane halves;
// - the A-operand row -> key map is permuted so that accumulator registers
//   8c..8c+7 of lane half H are 8 consecutive keys (16c + 8H + 0..7); rounded
//   to 16 bits they are directly the B operand (P^T) of O^T = V^T P^T;
// - K tiles go from global memory straight into LDS (global_load_lds_dwordx4,
//   no staging registers); V tiles are staged in registers and written to LDS
//   transposed, so the V^T operand is one ds_read_b128 per MFMA (a measured
//   1.6x cheaper per byte than the LDS transpose read);
// - 16-byte chunks are XOR-swizzled per row, which keeps every operand read
//   and every V^T write free of bank conflicts, and makes all LDS addresses
//   loop-invariant;
// - software pipeline: the MFMAs of S(n+1) = K(n+1) Q^T are issued before the
//   softmax of block n, so the VALU work of one block overlaps the matrix work
//   of the next; K/V tiles are double-buffered, one barrier per block;
// - scores stay in the log2 domain: p = 2^(s * scale * log2 e - m) is one FMA
//   and one v_exp_f32;
// - lazy rescaling: the reference max m of a row only moves when a block's max
//   exceeds it by more than 2^8, so O is rescaled rarely (exact: O and the sum
//   always share one reference);
// - masks (bottom-right causal, window, sequence tail) are evaluated only on
//   KV blocks that straddle a boundary; blocks outside every row's window are
//   never visited;
// - query tiles are issued heaviest first, and the tiles of one head land on
//   one XCD (work group id modulo 8), so their K/V re-reads hit that XCD's L2.
#include "device_common.h"
#include "kernels.h"

namespace exattn {
namespace {

constexpr int kBM = 128;  // query rows per work group
constexpr int kBN = 64;   // keys per KV block
constexpr int kThreads = 256;
constexpr float kLazyTau = 8.0f;  // rescale only when the row max grows by > 2^8

// K tile: row `key` is D*2 bytes; 16-byte chunk c is stored at c ^ kswz(key).
// The 8 lanes of one A-operand read phase read keys {b..b+3, b+8..b+11}; the
// swizzle gives them distinct low 3 bits.
__device__ __forceinline__ int kswz(int key) { return (key & 3) | (((key >> 3) & 1) << 2); }

// V^T tile: row d holds the block's 64 keys (8 chunks of 8 keys, 128 bytes);
// chunk kc is stored at kc ^ vswz(d).  Bijective on each aligned group of 8
// rows (conflict-free operand reads) and spreads the 16 lanes of a transposed
// 8-byte write over distinct banks.
__device__ __forceinline__ int vswz(int d) { return (d ^ (2 * (d >> 3))) & 7; }

// A-operand row m of a 32-key tile -> key: row 8J + 4H + I is key 16(J/2) + 8H + 4(J%2) + I.
__device__ __forceinline__ int row_key(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

// max / sum over the two 32-lane halves, broadcast to all lanes.  (The
// compiler folds the two results of v_permlane32_swap(x, x) into one, so the
// exchange goes through ds_bpermute.)
__device__ __forceinline__ float halves_max(float x) { return fmaxf(x, xor32(x)); }
__device__ __forceinline__ float halves_sum(float x) { return x + xor32(x); }

// Buffer descriptor for the rows kb .. sk-1 of one head (row stride ss
// elements): loads past the last valid element return zeros (the hardware
// range check of raw buffer loads is per dword).  Word 3 is the gfx9 default.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint16_t* g, int64_t ss, int kb,
                                                             int sk) {
  const int64_t last = (int64_t)(sk - 1 - kb) * ss + D;  // elements up to the end of row sk-1
  return __builtin_amdgcn_make_buffer_rsrc((void*)(g + (int64_t)kb * ss), 0, (int)(last * 2),
                                           0x00020000);
}

// 16 bytes per lane from a buffer into LDS at lds + 16 * lane (lds must be
// wave-uniform), and 16 bytes per lane into registers.  Kept out of lambdas:
// the host pass of the compiler drops the kernel stub when these builtins sit
// in a lambda body.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, uint8_t* lds,
                                                  uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16,
                                           voffset, 0, 0, 0);
}
__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t rs, uint32_t voffset) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voffset, 0, 0));
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <bool BF16, int D, bool SOFTCAP>
__global__ void __launch_bounds__(kThreads) prefill_kernel(const FwdParams p) {
  using E = Elem<BF16>;
  constexpr int DCH = D / 8;                   // 16-byte chunks per row
  constexpr int KS = D / 16;                   // k-steps of the 32x32x16 MFMA over head_dim
  constexpr int DT = D / 32;                   // 32-wide head_dim tiles of O^T
  constexpr int KTILE = kBN * D * 2;           // bytes
  constexpr int VTILE = D * kBN * 2;
  constexpr int ROWS_PER_KB = 1024 / (D * 2);  // K rows per 1 KiB direct-load slice
  constexpr int KINST = KTILE / 4096;          // direct loads per wave per K tile
  constexpr int G4 = DCH / 4;                  // 4-chunk groups per V row
  constexpr int VUNITS = 64 * G4;              // (4 keys x 8 columns) V pieces per tile
  constexpr int VLD = (VUNITS + kThreads - 1) / kThreads;
  static_assert(KINST >= 1 && KTILE % 4096 == 0, "tile/thread mismatch");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * KTILE + 2 * VTILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hsel = lane >> 5;  // which 32-lane half
  const int l32 = lane & 31;

  // ---- tile scheduler: heaviest query tiles first; (batch, head) fastest.
  const int units = p.batch * p.h_q;
  const int bid = blockIdx.x;
  const int qt = p.n_qt - 1 - bid / units;
  const int u = bid % units;
  int b, h;
  if (p.xcd_group) {
    // u % 8 picks the XCD; it depends only on the KV unit, so the query heads
    // sharing one K/V also share one L2.
    const int x = u & 7;
    const int rest = u >> 3;
    const int j = rest % p.group;
    const int kvu = (rest / p.group) * 8 + x;
    b = kvu / p.h_kv;
    h = (kvu % p.h_kv) * p.group + j;
  } else {
    b = u / p.h_q;
    h = u % p.h_q;
  }
  const int hk = h / p.group;

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
  const int q0 = qt * kBM;
  if (q0 >= sq) return;  // uniform across the work group

  const uint16_t* qg = p.q + qoff + (int64_t)h * p.q_sh;
  const uint16_t* kg = p.k + koff + (int64_t)hk * p.k_sh;
  const uint16_t* vg = p.v + voff + (int64_t)hk * p.v_sh;
  uint16_t* og = p.o + ooff + (int64_t)h * p.o_sh;
  float* lseg = p.lse != nullptr ? p.lse + lseoff + (int64_t)h * p.lse_sh : nullptr;

  // ---- visible key range of the whole tile (bottom-right aligned).
  const int off = sk - sq;
  const int q_last = min(q0 + kBM, sq) - 1;
  int kmin = 0, kmax = sk - 1;
  if (p.wl >= 0) kmin = max(0, q0 + off - p.wl);
  if (p.wr >= 0) kmax = min(kmax, q_last + off + p.wr);
  int n_lo = 0, n_hi = 0;
  if (kmax >= kmin) {
    n_lo = kmin / kBN;
    n_hi = kmax / kBN + 1;
  }

  // ---- Q^T fragments: lane holds Q[row][16 ks + 8 hsel .. +7] for every ks.
  const int qrow = q0 + wave * 32 + l32;
  u32x4_t qf[KS];
  if (qrow < sq) {
    const uint16_t* qp = qg + (int64_t)qrow * p.q_ss + 8 * hsel;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const u32x4_t*)(qp + 16 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = u32x4_t{0, 0, 0, 0};
  }
  if (p.q_sign != 0u) {  // negative softmax scale: negate Q exactly, use |scale|
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] ^= u32x4_t{p.q_sign, p.q_sign, p.q_sign, p.q_sign};
  }

  // ---- loop-invariant LDS addresses.
  // K operand: tile t2 row key = 32 t2 + row_key(l32); chunk 2 ks + hsel lives
  // at (2 ks + hsel) ^ kswz = 2 (ks ^ s1) + (hsel ^ s0); with ks = 4 a + bq the
  // offset is 128 a + 32 (bq ^ s1) + 16 (hsel ^ s0), so 4 bases cover all ks.
  const int krow = row_key(l32);
  const int ksw = kswz(krow);
  int kaddr[4];
#pragma unroll
  for (int bq = 0; bq < 4; ++bq)
    kaddr[bq] = krow * (D * 2) + 32 * (bq ^ (ksw >> 1)) + 16 * (hsel ^ (ksw & 1));
  // V^T operand: row d = 32 dt + l32 (vswz does not depend on dt); chunk
  // kc = 4 t2 + 2 c + hsel for MFMA (t2, c).
  int vaddr[4];
  {
    const int vs = vswz(l32);
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int c = 0; c < 2; ++c) vaddr[2 * t2 + c] = l32 * (kBN * 2) + 16 * ((4 * t2 + 2 * c + hsel) ^ vs);
  }

  // ---- K/V loads through buffer descriptors built per KV block: the base is
  // the block's first row and the range ends after the last valid row, so rows
  // past the sequence end read as zeros (hardware range check, no tail code).

  // K goes straight into LDS: wave `wave`, instruction i fills 1 KiB slice
  // 4 i + wave; lane l writes slot l = (row l / DCH of the slice, stored chunk
  // l % DCH), so it fetches global chunk (l % DCH) ^ kswz(row).  Lane offsets
  // are loop-invariant bytes (token strides are checked on the host).
  uint32_t kofs_ld[KINST];
#pragma unroll
  for (int i = 0; i < KINST; ++i) {
    const int row = (4 * i + wave) * ROWS_PER_KB + lane / DCH;
    kofs_ld[i] = (uint32_t)(row * p.k_ss + 8 * ((lane % DCH) ^ (kswz(row) & (DCH - 1)))) * 2u;
  }
  auto issue_k = [&](int n, int stage) {
    __amdgpu_buffer_rsrc_t rs = block_rsrc<D>(kg, p.k_ss, n * kBN, sk);
    uint8_t* dst = smem + stage * KTILE;
#pragma unroll
    for (int i = 0; i < KINST; ++i)
      buffer_load_lds16(rs, dst + (4 * i + wave) * 1024, kofs_ld[i]);
  };

  // V is staged in registers: unit un -> (kq, dc) with dc = a + 4 dc_hi,
  // kq = b + 4 kq_hi, a = un & 3, b = (un >> 2) & 3, c = un >> 4, dc_hi = c % G4,
  // kq_hi = c / G4.  One wave instruction covers whole rows (coalesced) and each
  // 16-lane group's transposed 8-byte writes hit 16 distinct bank slots.
  int vkq[VLD], vdc[VLD];
  uint32_t vofs[VLD][4];
#pragma unroll
  for (int i = 0; i < VLD; ++i) {
    const int un = tid + i * kThreads;
    const int cc = un >> 4;
    vdc[i] = (un & 3) + 4 * (cc % G4);
    vkq[i] = ((un >> 2) & 3) + 4 * (cc / G4);
#pragma unroll
    for (int r = 0; r < 4; ++r) vofs[i][r] = (uint32_t)((4 * vkq[i] + r) * p.v_ss + 8 * vdc[i]) * 2u;
  }
  u32x4_t vst[VLD][4];
  auto issue_v = [&](int n) {
    __amdgpu_buffer_rsrc_t rs = block_rsrc<D>(vg, p.v_ss, n * kBN, sk);
#pragma unroll
    for (int i = 0; i < VLD; ++i)
      if (VUNITS % kThreads == 0 || tid + i * kThreads < VUNITS)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vst[i][r] = buffer_load16(rs, vofs[i][r]);
  };
  auto store_v = [&](int stage) {
    uint8_t* vs_ = smem + 2 * KTILE + stage * VTILE;
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      if (VUNITS % kThreads == 0 || tid + i * kThreads < VUNITS) {
        const int kq = vkq[i];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int d = 8 * vdc[i] + t;
          *(u32x2_t*)(vs_ + d * (kBN * 2) + 16 * ((kq >> 1) ^ vswz(d)) + 8 * (kq & 1)) =
              column4(vst[i][0], vst[i][1], vst[i][2], vst[i][3], t);
        }
      }
    }
  };

  auto qk = [&](int stage, f32x16_t (&s)[2]) {
    const uint8_t* ks_ = smem + stage * KTILE;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) s[t2] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const u32x4_t a =
            *(const u32x4_t*)(ks_ + kaddr[ks & 3] + 128 * (ks >> 2) + t2 * 32 * (D * 2));
        s[t2] = E::mfma32x32x16(a, qf[ks], s[t2]);
      }
  };

  f32x16_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16_t{};
  float m_ref = kNegInf;  // reference max (log2 domain) of this lane's row
  float l_run = 0.f;      // this lane's share of the row sum, relative to m_ref

  // One pipeline step: S(n+1) on the MFMAs while block n is softmaxed, then
  // O += P(n) V(n).  s_c holds S(n) on entry; s_n receives S(n+1).
  auto step = [&](int n, f32x16_t (&s_c)[2], f32x16_t (&s_n)[2]) {
    const int j = n - n_lo;
    const bool has_next = n + 1 < n_hi;
    // K(n+1) has landed in LDS, V^T(n) is written; every wave is done with block n-1.
    wait_vmem_all();
    __syncthreads();
    if (n + 2 < n_hi) issue_k(n + 2, j & 1);
    if (has_next) {
      issue_v(n + 1);
      qk((j + 1) & 1, s_n);
    }

    // ---- softmax of block n (overlaps the MFMAs above).
    const int kb = n * kBN;
    const bool need_mask = (kb + kBN > sk) || (p.wr >= 0 && kb + kBN - 1 > q0 + off + p.wr) ||
                           (p.wl >= 0 && kb < q_last + off - p.wl);
    if (need_mask) {
      const int hi = (p.wr >= 0 ? min(sk - 1, qrow + off + p.wr) : sk - 1) - kb - 8 * hsel;
      const int lo = (p.wl >= 0 ? qrow + off - p.wl : -0x3fffffff) - kb - 8 * hsel;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 32 * t2 + 16 * (r >> 3) + (r & 7);  // key - kb - 8 hsel
          if (kk > hi || kk < lo) s_c[t2][r] = kNegInf;
        }
    }
    float mraw = s_c[0][0];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mraw = fmaxf(mraw, s_c[t2][r]);
    mraw = halves_max(mraw);
    float m_blk;
    if constexpr (SOFTCAP)
      m_blk = mraw == kNegInf ? kNegInf : p.cap_out_log2 * tanh_exp2(mraw * p.cap_in);
    else
      m_blk = mraw * p.scale_log2;
    // Lazy rescale: move the reference only when the block max exceeds it by
    // more than 2^tau (never while the block is fully masked: m_blk = -inf).
    const bool need = m_blk > m_ref + kLazyTau;
    const float m_new = need ? m_blk : m_ref;
    const float alpha = need ? fast_exp2(m_ref - m_new) : 1.f;  // 0 when m_ref = -inf
    if (__ballot(need && m_ref != kNegInf) != 0) {
      // rare: a row that already holds mass moves its reference
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    }
    l_run *= alpha;
    m_ref = m_new;
    const float base = m_ref == kNegInf ? 0.f : m_ref;
    float psum = 0.f;
    u32x4_t pf[2][2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float x0, x1;
        if constexpr (SOFTCAP) {
          // masked scores are -inf and must stay so (tanh(-inf) would give -1)
          const float a0 = s_c[t2][r], a1 = s_c[t2][r + 1];
          x0 = a0 == kNegInf ? kNegInf : p.cap_out_log2 * tanh_exp2(a0 * p.cap_in) - base;
          x1 = a1 == kNegInf ? kNegInf : p.cap_out_log2 * tanh_exp2(a1 * p.cap_in) - base;
        } else {
          x0 = __builtin_fmaf(s_c[t2][r], p.scale_log2, -base);
          x1 = __builtin_fmaf(s_c[t2][r + 1], p.scale_log2, -base);
        }
        x0 = fast_exp2(x0);
        x1 = fast_exp2(x1);
        psum += x0 + x1;
        // P^T fragment: the B operand of MFMA (t2, c) is registers 8c .. 8c+7 of tile t2.
        pf[t2][r >> 3][(r & 7) >> 1] = E::pack2(x0, x1);
      }
    l_run += psum;

    // ---- O^T += V^T P^T.
    const uint8_t* vs_ = smem + 2 * KTILE + (j & 1) * VTILE;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const u32x4_t a = *(const u32x4_t*)(vs_ + vaddr[2 * t2 + c] + dt * 32 * (kBN * 2));
          oacc[dt] = E::mfma32x32x16(a, pf[t2][c], oacc[dt]);
        }

    if (has_next) store_v((j + 1) & 1);
  };

  f32x16_t sa[2], sb[2];
  if (n_lo < n_hi) {
    issue_k(n_lo, 0);
    issue_v(n_lo);
    if (n_lo + 1 < n_hi) issue_k(n_lo + 1, 1);
    wait_vmem_all();
    store_v(0);
    __syncthreads();
    qk(0, sa);
  }
  int n = n_lo;
  for (; n + 1 < n_hi; n += 2) {
    step(n, sa, sb);
    step(n + 1, sb, sa);
  }
  if (n < n_hi) step(n, sa, sb);

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2; empty rows: 0 and -inf.
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (qrow < sq) {
    uint16_t* op = og + (int64_t)qrow * p.o_ss;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        u32x2_t w;
        w[0] = E::pack2(oacc[dt][4 * J] * inv, oacc[dt][4 * J + 1] * inv);
        w[1] = E::pack2(oacc[dt][4 * J + 2] * inv, oacc[dt][4 * J + 3] * inv);
        *(u32x2_t*)(op + 32 * dt + 8 * J + 4 * hsel) = w;
      }
    if (hsel == 0 && lseg != nullptr)
      lseg[qrow] = l_tot > 0.f ? (m_ref + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}

template <bool BF16, int D>
hipError_t launch_d(const FwdParams& p, bool softcap, int grid, hipStream_t stream) {
  if (softcap)
    hipLaunchKernelGGL((prefill_kernel<BF16, D, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_kernel<BF16, D, false>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_t(const FwdParams& p, int head_dim, bool softcap, int grid, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<BF16, 64>(p, softcap, grid, stream);
    case 128: return launch_d<BF16, 128>(p, softcap, grid, stream);
    case 256: return launch_d<BF16, 256>(p, softcap, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int prefill_rows_per_tile() { return kBM; }

hipError_t launch_prefill(const FwdParams& p, bool bf16, int head_dim, bool softcap, int grid,
                          hipStream_t stream) {
  return bf16 ? launch_t<true>(p, head_dim, softcap, grid, stream)
              : launch_t<false>(p, head_dim, softcap, grid, stream);
}

}  // namespace exattn
