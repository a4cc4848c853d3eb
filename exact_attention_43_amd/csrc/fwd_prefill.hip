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
// - a work group owns 128 query rows of one query head.  It has NG groups of
//   4 waves; every group covers all 128 rows (32 per wave) and the groups split
//   the KV blocks between them (group g takes blocks n_lo + g, n_lo + g + NG,
//   ...), each with its own double-buffered K/V tiles.  With NG = 2 every SIMD
//   runs two waves: one wave's softmax issues while the other's MFMAs run, and
//   LDS reads reach about 200 B/clk/CU instead of about 120 with one wave per
//   SIMD (measured).  The groups' partial (m, l, O) are merged through LDS at
//   the end, the same log-sum-exp merge as between tiles, each group
//   finalizing half of the head dims; O then leaves through an LDS tile so
//   that global stores cover whole rows;
// - the wave computes S^T = K Q^T with v_mfma_f32_32x32x16 (bf16/f16, fp32
//   accumulate): K is the A operand read from LDS, Q^T the B operand held in
//   registers for the whole loop.  In the 32x32 accumulator layout every lane
//   owns ONE query row, so row max and row sum are in-lane, plus one exchange
//   between the two 32-lane halves;
// - the A-operand row -> key map is permuted so that accumulator registers
//   8c..8c+7 of lane half H are 8 consecutive keys (16c + 8H + 0..7); rounded
//   to 16 bits they are directly the B operand (P^T) of O^T = V^T P^T;
// - K and V tiles go from global memory straight into LDS (buffer_load ...
//   lds, no staging registers).  V stays row-major: the V^T operand is two
//   transposing LDS reads (ds_read_b64_tr_b16) per MFMA;
// - 16-byte chunks are XOR-swizzled per row, which keeps the operand reads
//   free of bank conflicts and all LDS addresses loop-invariant;
// - with one group and d = 128 the loop is software-pipelined: the QK MFMAs of
//   block i are interleaved with the exponentials of block i - 1;
// - loads use per-block buffer descriptors whose range ends at the last key of
//   the sequence: the hardware range check returns zeros past the end, so
//   block tails need no extra code;
// - scores stay in the log2 domain: p = 2^(s * scale * log2 e - m) is one FMA
//   and one v_exp_f32;
// - lazy rescaling: a row's reference max m only moves when a block's max
//   exceeds it by more than 2^8, so O is rescaled rarely (exact: O and the sum
//   always share one reference);
// - masks (bottom-right causal, window, sequence tail) are evaluated only on
//   KV blocks that straddle a boundary; blocks outside every row's window are
//   never visited;
// - query tiles are issued heaviest first, and the tiles of one head land on
//   one XCD (work group id modulo 8), so their K/V re-reads hit that XCD's L2.
#include "device_common.h"
#include "kernels.h"
#include "tiles.h"

namespace exattn {
namespace {

constexpr int kBM = 128;          // query rows per work group
constexpr float kLazyTau = 8.0f;  // rescale only when the row max grows by > 2^8
constexpr float kSumCap = 256.0f;  // 2^tau: a block sum below it means every p <= 2^tau

// Keys per KV block.  The number of groups per work group (NG, a template
// parameter) is chosen per launch: two groups (8 waves, 128 KiB of LDS, one
// work group per CU) split one tile's KV blocks when the grid is small; one
// group (4 waves, 64 KiB, two work groups per CU) when there are at least two
// work groups per CU, which then run unsynchronised (measured faster there).
// d = 256 always takes one group (its tiles need 128 KiB).
template <int D> struct Cfg { static constexpr int BN = 64; };

// Scores of keys outside [lo, hi] (relative to the block's first key plus
// 8 hsel) -> -inf.  Register r of tile t2 holds key 32 t2 + 16 (r / 8) + r % 8.
template <int NT2>
__device__ __forceinline__ void mask_keys(f32x16_t (&s)[NT2], int hi, int lo) {
#pragma unroll
  for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = 32 * t2 + 16 * (r >> 3) + (r & 7);
      if (kk > hi || kk < lo) s[t2][r] = kNegInf;
    }
}

// PAIR: a two-group work group takes a light and a heavy 64-row tile (launch
// shape chosen on the host); its own instances carry the idle-pair DMA.
template <bool BF16, int D, bool SOFTCAP, int NG, bool PAIR>
__global__ void __launch_bounds__(256 * NG)
prefill_kernel(const FwdParams p) {
  using E = Elem<BF16>;
  constexpr int BN = Cfg<D>::BN;
  constexpr int NT2 = BN / 32;                 // 32-key MFMA tiles per KV block
  constexpr int DCH = D / 8;                   // 16-byte chunks per row
  constexpr int KS = D / 16;                   // k-steps of the 32x32x16 MFMA over head_dim
  constexpr int DT = D / 32;                   // 32-wide head_dim tiles of O^T
  constexpr int KTILE = BN * D * 2;            // bytes
  constexpr int VTILE = D * BN * 2;
  constexpr int GROUP_LDS = 2 * KTILE + 2 * VTILE;
  constexpr int ROWS_PER_KB = 1024 / (D * 2);  // K rows per 1 KiB direct-load slice
  constexpr int KINST = KTILE / 4096;          // direct loads per wave per K tile
  static_assert(KINST >= 1 && KTILE % 4096 == 0, "tile/thread mismatch");
  static_assert(NG * GROUP_LDS <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NG * GROUP_LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;   // KV-block group
  const int wg = wave & 3;     // wave within the group
  const int hsel = lane >> 5;  // which 32-lane half
  const int l32 = lane & 31;
  uint8_t* gsm = smem + grp * GROUP_LDS;

  // ---- fast start for dense launches with one tile per query head on the
  // (unit, batch, tile) grid: the Q loads go out first, addressed from the
  // block index and a few kernel arguments, ahead of the rest of the set-up
  // (the general path below reaches them after a few hundred scalar
  // instructions and dependent loads of kernel arguments).  Same rows and
  // values as the general path.
  u32x4_t qf[KS];
  const bool fast_q = p.grid3 != 0 && p.pack == 0 && p.cu_q == nullptr;
  if (fast_q) {
    const int qt_ = p.n_qt - 1 - (int)blockIdx.z;
    const int n64_ = (p.s_q + 63) / 64;
    const int ta = PAIR ? qt_ : 2 * qt_, tb = PAIR ? n64_ - 1 - qt_ : 2 * qt_ + 1;
    const bool a_ = PAIR ? (wg >> 1) == grp : wg < 2;
    const int row = 64 * (a_ ? ta : tb) + 32 * (wg & 1) + l32;
    if (2 * qt_ < n64_ && (a_ || (tb > ta && tb < n64_)) && row < p.s_q) {
      const uint16_t* qp = p.q + (int64_t)blockIdx.y * p.q_sb + (int64_t)blockIdx.x * p.q_sh +
                           (int64_t)row * p.q_ss + 8 * hsel;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const u32x4_t*)(qp + 16 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = u32x4_t{0, 0, 0, 0};
    }
  }

  // ---- tile scheduler: heaviest query tiles first; (batch, head) fastest.
  // Packed GQA (p.pack): a unit is one KV head, and its tiles hold the rows of
  // all `group` query heads that read it, head fastest: virtual row R is
  // position R / group of query head hk * group + R % group.  Unpacked, a unit
  // is one query head and virtual row R is position R.  Work groups are
  // dispatched (and spread over the XCDs, work group id modulo 8) in linear
  // order, x fastest; a three-dimensional grid (unit, batch, tile) gives that
  // same order without the integer divisions of a linear id, which cost a few
  // hundred scalar instructions ahead of the first load.
  const bool pack = p.pack != 0;
  const int G = pack ? p.group : 1;
  int qt, b, h, hk;
  if (p.grid3 != 0) {
    qt = p.n_qt - 1 - (int)blockIdx.z;
    b = blockIdx.y;
    h = pack ? (int)blockIdx.x * p.group : (int)blockIdx.x;  // packed: the group's first query head
    hk = pack || p.group == 1 ? (int)blockIdx.x : h / p.group;
  } else {
    const int units = p.batch * (pack ? p.h_kv : p.h_q);
    const int bid = blockIdx.x;
    qt = p.n_qt - 1 - bid / units;
    const int u = bid % units;
    if (pack) {
      b = u / p.h_kv;
      h = (u % p.h_kv) * p.group;
    } else if (p.xcd_group) {
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
    hk = h / p.group;
  }
  // Virtual row -> position and head offset.  Rows divide through a float
  // reciprocal, exact after the +-1 correction for rows below 2^22 (the host
  // limits packed launches to that); unpacked rows are positions.
  const float rcp_g = __builtin_amdgcn_rcpf((float)G);
  auto vpos = [&](int r) {
    if (!pack) return r;
    int q = (int)((float)r * rcp_g);
    q += (q + 1) * G <= r ? 1 : 0;
    q -= q * G > r ? 1 : 0;
    return q;
  };
  auto vhead = [&](int r) { return pack ? r - vpos(r) * G : 0; };

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
  // ---- the work group's 128 rows are two 64-row tiles: 2 qt and 2 qt + 1,
  // or, when pairing (two groups), tiles j and n64 - 1 - j, a light and a heavy
  // one under a causal mask, so every work group carries about the same work.
  // Paired, group 0's waves 0-1 and group 1's waves 2-3 take tile j and the
  // others tile n64 - 1 - j, so each SIMD (waves w and w + 4) holds one wave of
  // each tile; otherwise waves 0-1 of each group take the first tile.
  const int sqv = sq * G;  // virtual rows
  const int n64 = (sqv + 63) / 64;
  if (2 * qt >= n64) return;  // uniform across the work group
  static_assert(!PAIR || NG == 2, "pairing needs two groups");
  constexpr bool paired = PAIR;
  const int tile_a = paired ? qt : 2 * qt;
  const int tile_b = paired ? n64 - 1 - qt : 2 * qt + 1;
  const bool b_valid = tile_b > tile_a && tile_b < n64;  // an odd tile count leaves one alone
  const bool my_a = paired ? (wg >> 1) == grp : wg < 2;
  const bool my_valid = my_a || b_valid;
  const int q0 = 64 * (my_a ? tile_a : tile_b);   // first row of this wave's tile
  const int q_last = min(q0 + 64, sqv) - 1;

  // ---- Q^T fragments: lane holds Q[row][16 ks + 8 hsel .. +7] for every ks.
  // Issued first: the burst of Q reads from memory is the longest wait of the
  // prologue, and everything up to the loop except the first KV DMA can be
  // computed under it.
  const int qrow = q0 + 32 * (wg & 1) + l32;  // virtual row of this lane
  const int qpos = vpos(qrow);                 // its position
  const int qhead = h + vhead(qrow);           // its query head
  if (!fast_q) {
    if (my_valid && qrow < sqv) {
      const uint16_t* qp = p.q + qoff + (int64_t)qhead * p.q_sh + (int64_t)qpos * p.q_ss + 8 * hsel;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const u32x4_t*)(qp + 16 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = u32x4_t{0, 0, 0, 0};
    }
  }
  const uint16_t* kg = p.k + koff + (int64_t)hk * p.k_sh;
  const uint16_t* vg = p.v + voff + (int64_t)hk * p.v_sh;

  // ---- visible key blocks [lo, hi) of a 64-row tile (bottom-right aligned);
  // the groups walk the union over both tiles, a wave computes its own tile's.
  const int off = sk - sq;
  auto block_range = [&](int tile, int& lo, int& hi) {
    const int t0 = vpos(64 * tile), t1 = vpos(min(64 * tile + 64, sqv) - 1);
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
  int a_lo, a_hi, b_lo = 0, b_hi = 0;
  block_range(tile_a, a_lo, a_hi);
  if (b_valid) block_range(tile_b, b_lo, b_hi);
  int n_lo = a_lo, n_hi = a_hi;
  if (b_valid && b_hi > b_lo) {
    n_lo = a_hi > a_lo ? min(a_lo, b_lo) : b_lo;
    n_hi = max(a_hi, b_hi);
  }
  // Group g takes the blocks whose index is g modulo NG, counted from key 0
  // (not from the tile's first block): a row then sums the same blocks in the
  // same group whatever tile holds it, so its result does not depend on the
  // tiling (packed or not).  Block n_lo - 1 may be loaded and never computed.
  if (n_hi > n_lo) n_lo -= n_lo % NG;
  const int w_lo = my_a ? a_lo : b_lo;                    // this wave's blocks
  const int w_hi = my_valid ? (my_a ? a_hi : b_hi) : 0;

  // ---- K and V straight into LDS by DMA: wave wg of the group, instruction i
  // fills 1 KiB slice 4 i + wg; lane l writes slot l = (row l / DCH of the
  // slice, stored chunk l % DCH), so it fetches global chunk (l % DCH) ^
  // swizzle(row).  Lane offsets are loop-invariant bytes (token strides are
  // checked on the host).
  uint32_t kofs_ld[KINST], vofs_ld[KINST];
#pragma unroll
  for (int i = 0; i < KINST; ++i) {
    const int row = (4 * i + wg) * ROWS_PER_KB + lane / DCH;
    kofs_ld[i] = (uint32_t)(row * p.k_ss + 8 * ((lane % DCH) ^ kswz<D>(row))) * 2u;
    vofs_ld[i] = (uint32_t)(row * p.v_ss + 8 * ((lane % DCH) ^ vswz<D>(row))) * 2u;
  }
  auto issue_k = [&](int n, uint8_t* kdst) {
    const __amdgpu_buffer_rsrc_t rk = block_rsrc<D>(kg, p.k_ss, n * BN, sk, BN);
#pragma unroll
    for (int i = 0; i < KINST; ++i) buffer_load_lds16(rk, kdst + (4 * i + wg) * 1024, kofs_ld[i]);
  };
  auto issue_v = [&](int n, uint8_t* vdst) {
    const __amdgpu_buffer_rsrc_t rv = block_rsrc<D>(vg, p.v_ss, n * BN, sk, BN);
#pragma unroll
    for (int i = 0; i < KINST; ++i) buffer_load_lds16(rv, vdst + (4 * i + wg) * 1024, vofs_ld[i]);
  };
  uint8_t* const k0 = gsm;
  uint8_t* const k1 = gsm + KTILE;
  uint8_t* const v0 = gsm + 2 * KTILE;
  uint8_t* const v1 = gsm + 2 * KTILE + VTILE;
  // The first block of the group: K and V (plain loop) or K only (the
  // software-pipelined loop loads V(b_i) in step i).
  constexpr bool kPipelined = NG == 1 && D == 128 && !SOFTCAP;
  if (n_lo + grp < n_hi) {
    issue_k(n_lo + grp, k0);
    if constexpr (!kPipelined) issue_v(n_lo + grp, v0);
  }

  // ---- loop-invariant LDS addresses.
  // K operand: tile t2 row key = 32 t2 + row_key(l32); chunk 2 ks + hsel lives
  // at (2 ks + hsel) ^ kswz = 2 (ks ^ s1) + (hsel ^ s0) with s1 < NKA; with
  // ks = NKA a + bq the offset is 32 NKA a + 32 (bq ^ s1) + 16 (hsel ^ s0), so
  // NKA bases cover all ks.
  constexpr int NKA = D == 64 ? 4 : 8;
  const int krow = row_key(l32);
  const int ksw = kswz<D>(krow);
  int kaddr[NKA];
#pragma unroll
  for (int bq = 0; bq < NKA; ++bq)
    kaddr[bq] = krow * (D * 2) + 32 * (bq ^ (ksw >> 1)) + 16 * (hsel ^ (ksw & 1));
  // V operand (A of O^T += V^T P^T, from V stored row-major in LDS): for MFMA
  // (t2, c) the lane of d row d0 + i in 16-lane group gi (d0 = 32 dt + 16
  // (gi & 1), lane half H = gi >> 1) needs V[k + t][d0 + i], t = 0..7, with
  // k = 32 t2 + 16 c + 8 H.  Two transposing reads give keys k..k+3 and
  // k+4..k+7: source lane s of the group addresses the 4 values
  // V[k + 4 half + (s >> 2)][d0 + 4 (s & 3) .. + 3].  The key row offset and the
  // swizzle depend only on the lane and on half, the chunk on dt; t2 and c add
  // whole rows.
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

  // The partner wave's share (slices 4 i + (wg ^ 2): the other tile's wave of
  // the group), issued together with this wave's own share in steps where
  // only the partner has a block to compute.
  uint32_t kofs_pt[KINST], vofs_pt[KINST];
#pragma unroll
  for (int i = 0; i < KINST; ++i) {
    const int row = (4 * i + (wg ^ 2)) * ROWS_PER_KB + lane / DCH;
    kofs_pt[i] = (uint32_t)(row * p.k_ss + 8 * ((lane % DCH) ^ kswz<D>(row))) * 2u;
    vofs_pt[i] = (uint32_t)(row * p.v_ss + 8 * ((lane % DCH) ^ vswz<D>(row))) * 2u;
  }
  auto issue_kv_both = [&](int n, uint8_t* kdst, uint8_t* vdst) {
    const __amdgpu_buffer_rsrc_t rk = block_rsrc<D>(kg, p.k_ss, n * BN, sk, BN);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc<D>(vg, p.v_ss, n * BN, sk, BN);
#pragma unroll
    for (int i = 0; i < KINST; ++i) {
      buffer_load_lds16(rk, kdst + (4 * i + wg) * 1024, kofs_ld[i]);
      buffer_load_lds16(rk, kdst + (4 * i + (wg ^ 2)) * 1024, kofs_pt[i]);
    }
#pragma unroll
    for (int i = 0; i < KINST; ++i) {
      buffer_load_lds16(rv, vdst + (4 * i + wg) * 1024, vofs_ld[i]);
      buffer_load_lds16(rv, vdst + (4 * i + (wg ^ 2)) * 1024, vofs_pt[i]);
    }
  };

  f32x16_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16_t{};
  float m_ref = kNegInf;  // reference max (log2 domain) of this lane's row
  float l_run = 0.f;      // this lane's share of the row sum, relative to m_ref

  // p = 2^(score - base) for the block, rounded into the P^T operand (the B
  // operand of MFMA (t2, c) is registers 8c .. 8c+7 of tile t2).  Returns this
  // lane's fp32 sum of p: the row sum, and so the LSE, is taken before rounding
  // (a sum of the 16-bit values can be off by 2^-9 relative, too much for LSE).
  auto exps = [&](const f32x16_t (&s)[NT2], u32x4_t (&pf)[NT2][2], float base) {
    float psum = 0.f;
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float x0, x1;
        if constexpr (SOFTCAP) {
          // masked scores are -inf and must stay so (tanh(-inf) would give -1)
          const float a0 = s[t2][r], a1 = s[t2][r + 1];
          x0 = a0 == kNegInf ? kNegInf : p.cap_out_log2 * tanh_exp2(a0 * p.cap_in) - base;
          x1 = a1 == kNegInf ? kNegInf : p.cap_out_log2 * tanh_exp2(a1 * p.cap_in) - base;
        } else {
          x0 = __builtin_fmaf(s[t2][r], p.scale_log2, -base);
          x1 = __builtin_fmaf(s[t2][r + 1], p.scale_log2, -base);
        }
        x0 = fast_exp2(x0);
        x1 = fast_exp2(x1);
        pf[t2][r >> 3][(r & 7) >> 1] = E::pack2(x0, x1);
        psum += x0 + x1;
      }
    return psum;
  };

  // ---- the pieces of one KV block: S^T = K Q^T, the mask, the online softmax
  // and O^T += V^T P^T.
  // K operand of MFMA (ks, t2): keys 32 t2 + row_key(lane), head dims 16 ks + 8 hsel + 0..7.
  auto k_operand = [&](const uint8_t* __restrict__ ks_, int ks, int t2) {
    return *(const u32x4_t*)(ks_ + kaddr[ks % NKA] + 32 * NKA * (ks / NKA) + t2 * 32 * (D * 2));
  };
  // Eight K reads go out ahead of the MFMAs, then one more per MFMA (d >= 128).
  // Left to itself the scheduler keeps two in flight and waits for each pair
  // right before its MFMAs, which exposes the LDS latency in every k-step
  // whenever a SIMD has no second wave to fill it (measured 2-3% faster at
  // d = 128; at d = 64, with 8 reads per block, the default order measured
  // 1.4% faster).
  auto qk = [&](const uint8_t* __restrict__ ks_, f32x16_t (&s)[NT2]) {
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2) s[t2] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int t2 = 0; t2 < NT2; ++t2) s[t2] = E::mfma32x32x16(k_operand(ks_, ks, t2), qf[ks], s[t2]);
    if constexpr (D >= 128) {
      constexpr int NQ = KS * NT2, PF = 8;
      __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + PF < NQ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };
  // scores outside the causal / window bounds or past the last key -> -inf
  // (only blocks that straddle a bound carry any)
  // Keys <= full_r and >= full_l are visible to every row of the wave's tile,
  // so only blocks that reach past them carry a mask; this lane's row sees
  // keys mlo + 8 hsel .. mhi + 8 hsel.
  const int full_r = p.wr >= 0 ? min(sk - 1, vpos(q0) + off + p.wr) : sk - 1;
  const int full_l = p.wl >= 0 ? vpos(q_last) + off - p.wl : -0x3fffffff;
  const int mhi = (p.wr >= 0 ? min(sk - 1, qpos + off + p.wr) : sk - 1) - 8 * hsel;
  const int mlo = (p.wl >= 0 ? qpos + off - p.wl : -0x3fffffff) - 8 * hsel;
  // The exponentials are first taken against the current reference; the
  // block's row max is needed only when a lane's block sum exceeds 2^tau (some
  // p may exceed 2^tau, or overflowed) or a row has no reference yet (then the
  // sum is inf or NaN).  Then the reference moves lazily (only when the block
  // max exceeds it by more than 2^tau, never while the block is fully masked),
  // O and l are rescaled and the exponentials recomputed.  Exact in all cases:
  // O and l always share the reference, and every p stays <= 2^tau.
  auto slow = [&](const f32x16_t (&s)[NT2], u32x4_t (&pf)[NT2][2]) {
    float mraw = s[0][0];
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mraw = fmaxf(mraw, s[t2][r]);
    mraw = halves_max(mraw);
    float m_blk;
    if constexpr (SOFTCAP)
      m_blk = mraw == kNegInf ? kNegInf : p.cap_out_log2 * tanh_exp2(mraw * p.cap_in);
    else
      m_blk = mraw * p.scale_log2;
    const bool need = m_blk > m_ref + kLazyTau;
    const float m_new = need ? m_blk : m_ref;
    const float alpha = need ? fast_exp2(m_ref - m_new) : 1.f;  // 0 when m_ref = -inf
    if (__ballot(need && m_ref != kNegInf) != 0) {
      // a row that already holds mass moves its reference
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    }
    l_run *= alpha;
    m_ref = m_new;
    return exps(s, pf, m_ref == kNegInf ? 0.f : m_ref);
  };
  auto sum_too_big = [](float psum) { return __ballot(!(psum <= kSumCap)) != 0; };  // also inf, NaN
  auto v_operand = [&](const uint8_t* __restrict__ vs_, int t2, int c, int dt) {
    const int rows = (32 * t2 + 16 * c) * (D * 2);
    const u32x2_t lo = lds_read_tr16(vs_ + vtr[0][dt] + rows);
    const u32x2_t hi = lds_read_tr16(vs_ + vtr[1][dt] + rows);
    u32x4_t a;
    a[0] = lo[0];
    a[1] = lo[1];
    a[2] = hi[0];
    a[3] = hi[1];
    return a;
  };
  auto pv = [&](const uint8_t* __restrict__ vs_, const u32x4_t (&pf)[NT2][2]) {
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] = E::mfma32x32x16(v_operand(vs_, t2, c, dt), pf[t2][c], oacc[dt]);
  };
  // softmax of a block's scores s into pf, then O^T += V^T P^T.  The V^T
  // operands of the first key slice are read before the exponentials, so their
  // LDS latency passes under the VALU work instead of ahead of the first MFMA.
  auto softmax_pv = [&](const uint8_t* __restrict__ vs_, const f32x16_t (&s)[NT2]) {
    u32x4_t pf[NT2][2];
    u32x4_t vpre[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vpre[dt] = v_operand(vs_, 0, 0, dt);
    float psum = 0.f;
    bool ok = false;
    if (__ballot(m_ref == kNegInf) == 0) {  // some row without a reference: straight to the max
      psum = exps(s, pf, m_ref);
      ok = !sum_too_big(psum);
    }
    if (!ok) psum = slow(s, pf);
    l_run += psum;
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          oacc[dt] = E::mfma32x32x16(t2 == 0 && c == 0 ? vpre[dt] : v_operand(vs_, t2, c, dt),
                                     pf[t2][c], oacc[dt]);
  };

  const int nblk = n_hi - n_lo;
  const int steps = (nblk + NG - 1) / NG;
  // group g works on blocks b_i = n_lo + g + NG i, i < nb
  const int nb = nblk > grp ? (nblk - grp + NG - 1) / NG : 0;
  auto blk = [&](int i) { return n_lo + grp + NG * i; };
  auto active = [&](int i) { return blk(i) >= w_lo && blk(i) < w_hi; };  // uniform per wave
  // Consume Q (and apply the sign of a negative scale) just before the loop,
  // after the first DMA is on its way: the compiler then waits for the Q loads
  // only, once.  Otherwise it cannot tell that the loop's own waits covered
  // them and waits inside every step for all newer loads, the next block's
  // prefetch included.
  auto pin_q = [&] {
    if (p.q_sign != 0u) {  // negative softmax scale: negate Q exactly, use |scale|
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] ^= u32x4_t{p.q_sign, p.q_sign, p.q_sign, p.q_sign};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
  };

  if constexpr (kPipelined) {
    // ---- software-pipelined loop (one group: large grids).  Step i computes
    // S(b_i) = K(b_i) Q^T and, with the exponentials of S(b_{i-1}) issued
    // between those MFMAs, the softmax and O += P V of b_{i-1}.  One SIMD
    // overlaps MFMAs with VALU work only when the instruction streams it holds
    // mix them finely; block-sized phases of MFMA and of VALU work, in step on
    // every wave after the barrier, leave one of the two units idle.  K(b_i)
    // lives in K stage i & 1, V(b_i) in V stage i & 1; step i loads K(b_{i+1})
    // and V(b_i) (their stages were last read in step i - 1).  With two groups
    // (small grids, few blocks per tile), and at d = 64 (twice the VALU work
    // per MFMA), the extra step and the discarded work at each end cost more
    // than the overlap gains (measured), so those take the plain loop; softcap
    // needs more registers than two waves per SIMD leave.
    constexpr int NA = KS * NT2;        // MFMAs of S^T = K Q^T per block
    constexpr int EPM = 16 * NT2 / NA;  // exponentials per such MFMA
    static_assert(EPM >= 2 && EPM % 2 == 0, "exponential pairs per MFMA");
    constexpr int VPM = EPM / 2 * 7;  // VALU instructions per MFMA: 2 FMA, 2 exp, 1 pack, 2 add
    // S(b_i) = K Q^T interleaved with the exponentials of S(b_{i-1}) = sc
    // against the current reference, then the check, the softmax fix-up if
    // needed and O += P(b_{i-1}) V(b_{i-1}).
    auto fused = [&](const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vp,
                     const f32x16_t (&sc)[NT2], f32x16_t (&sn)[NT2], bool ap) {
      u32x4_t pf[NT2][2];
      float psum = 0.f;
      const float base = m_ref;
#pragma unroll
      for (int t2 = 0; t2 < NT2; ++t2) sn[t2] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int t2 = 0; t2 < NT2; ++t2) {
          const int mi = ks * NT2 + t2;
          sn[t2] = E::mfma32x32x16(k_operand(kc, ks, t2), qf[ks], sn[t2]);
#pragma unroll
          for (int u = 0; u < EPM; u += 2) {
            const int e = mi * EPM + u, t = e >> 4, r = e & 15;
            const float x0 = fast_exp2(__builtin_fmaf(sc[t][r], p.scale_log2, -base));
            const float x1 = fast_exp2(__builtin_fmaf(sc[t][r + 1], p.scale_log2, -base));
            pf[t][r >> 3][(r & 7) >> 1] = E::pack2(x0, x1);
            psum += x0 + x1;
          }
        }
      // order: two K operand reads ahead, then per MFMA one more read and its
      // share of the exponentials
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int mi = 0; mi < NA; ++mi) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (mi + 2 < NA) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, VPM, 0);
      }
      // consume the exponentials here: LLVM would otherwise sink them below
      // the branch that follows, out of the MFMA stream
#pragma unroll
      for (int t = 0; t < NT2; ++t) asm volatile("" ::"v"(pf[t][0]), "v"(pf[t][1]));
      asm volatile("" ::"v"(psum));
      if (ap) {
        if (sum_too_big(psum)) psum = slow(sc, pf);
        l_run += psum;
        pv(vp, pf);
      }
    };
    // kc: K(b_i); vp: V(b_{i-1}); kn: stage for K(b_{i+1}); vc: stage for V(b_i)
    auto step = [&](const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vp,
                    uint8_t* __restrict__ kn, uint8_t* __restrict__ vc, int i,
                    const f32x16_t (&sc)[NT2], f32x16_t (&sn)[NT2]) {
      if (i + 1 < nb) issue_k(blk(i + 1), kn);
      if (i < nb) issue_v(blk(i), vc);
      const bool ai = i < nb && active(i);
      const bool ap = i > 0 && i <= nb && active(i - 1);
      // A wave's first block (no previous one) still runs the exponentials, on
      // stale registers, and its last runs S = K Q^T on a stale stage: both
      // results are discarded.  Branching around them instead costs registers.
      if (ai || ap) fused(kc, vp, sc, sn, ap);
      if (ai) {
        const int kb = blk(i) * BN;
        if (kb + BN - 1 > full_r || kb < full_l) mask_keys(sn, mhi - kb, mlo - kb);
      }
    };
    pin_q();
    f32x16_t sa[NT2], sb[NT2];
    // Unrolled by two so each call sees fixed stages and score registers.
    // Before each step: K(b_i) and V(b_{i-1}) have landed, and every wave is
    // done with the previous step.
    int i = 0;
    for (; i + 1 <= steps; i += 2) {
      wait_vmem_all();
      __syncthreads();
      step(k0, v1, k1, v0, i, sb, sa);
      wait_vmem_all();
      __syncthreads();
      step(k1, v0, k0, v1, i + 1, sa, sb);
    }
    if (i <= steps) {
      wait_vmem_all();
      __syncthreads();
      step(k0, v1, k1, v0, i, sb, sa);
    }
  } else {
    // ---- plain loop: step i, group g works on block b_i; K(b_i) and V(b_i)
    // live in stage i & 1.  A step starts the DMA of the group's next block
    // into the other stage and computes block b_i.  The stages never overlap;
    // restrict tells the compiler so, which lets the operand reads of this
    // step proceed while the DMA into the other stage is in flight (without
    // it every LDS read waits for all outstanding DMA).
    // Who issues the DMA of the group's next block.  A wave stalls at issue
    // while the CU's vector memory path drains the queue (about 20 cycles per
    // 1 KiB instruction): all waves issuing both tiles at once after the
    // barrier stalled each about 1100 cycles before its first K read (measured
    // with cycle stamps at the causal b2 s1024 h16 d128 shape).  So each wave
    // issues its share of K at the start of the step and its share of V after
    // its score MFMAs; and in a light + heavy pairing, in a step where only
    // one tile's wave of a group pair has a block to compute, the idle wave
    // issues both shares at the start and the busy one none (measured -4% at
    // that shape, -6% at b1 s2048 causal; only paired instances carry this).
    const bool o_valid = !my_a || b_valid;  // the partner's tile exists
    const int o_lo = my_a ? b_lo : a_lo, o_hi = o_valid ? (my_a ? b_hi : a_hi) : 0;
    auto step = [&](const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
                    uint8_t* __restrict__ kn, uint8_t* __restrict__ vn, int n) {
      const bool more = n + NG < n_hi;
      const bool mine_ = n >= w_lo && n < w_hi;
      // 0: own share (K now, V after the score MFMAs); 1: own and the partner's
      // (this wave idle, the partner busy); 2: none (this wave busy, the partner idle)
      int mode = 0;
      if constexpr (PAIR && !SOFTCAP) {
        const bool other = n >= o_lo && n < o_hi;
        mode = mine_ == other ? 0 : (mine_ ? 2 : 1);
      }
      if (more && mode == 0) issue_k(n + NG, kn);
      if (more && mode == 1) issue_kv_both(n + NG, kn, vn);
      if (n >= w_lo && n < w_hi) {  // uniform per wave
        f32x16_t s[NT2];
        qk(kc, s);
        __builtin_amdgcn_sched_barrier(0);
        if (more && mode == 0) issue_v(n + NG, vn);
        const int kb = n * BN;
        if (kb + BN - 1 > full_r || kb < full_l) mask_keys(s, mhi - kb, mlo - kb);
        softmax_pv(vc, s);
      } else if (more && mode == 0) {
        issue_v(n + NG, vn);
      }
    };
    pin_q();
    int i = 0;
    for (; i + 1 < steps; i += 2) {
      const int n = n_lo + NG * i + grp;
      wait_vmem_all();
      __syncthreads();
      step(k0, v0, k1, v1, n);
      wait_vmem_all();
      __syncthreads();
      step(k1, v1, k0, v0, n + NG);
    }
    if (i < steps) {
      wait_vmem_all();
      __syncthreads();
      step(k0, v0, k1, v1, n_lo + NG * i + grp);
    }
  }

  // ---- epilogue.  The tile buffers are free after the barrier.  With two
  // groups, the two waves that hold the same 32 rows merge their (m, l, O)
  // with the log-sum-exp merge, each finalizing half of the head dims from
  // what its partner hands over through LDS.  Then O = O^T / l, rounded, goes
  // through an LDS tile so that global stores cover whole rows (16 lanes x
  // 16 bytes per row piece instead of 32 rows x 8 bytes per instruction), and
  // LSE = (m + log2 l) ln 2.  Empty rows give 0 and -inf.
  constexpr int DTH = DT / NG;                           // d tiles a wave finalizes
  constexpr int XM_BYTES = NG > 1 ? 4 * NG * 2 * 64 * 4 : 0;          // m, l
  constexpr int XO_BYTES = NG > 1 ? 4 * NG * DTH * 16 * 64 * 4 : 0;   // half of O^T
  constexpr int OROW = D * 2;                            // bytes per row of the O tile
  static_assert(XM_BYTES + XO_BYTES + kBM * OROW <= NG * GROUP_LDS, "epilogue buffers");
  float* const xm = reinterpret_cast<float*>(smem);
  float* const xo = reinterpret_cast<float*>(smem + XM_BYTES);
  uint8_t* const otile = smem + XM_BYTES + XO_BYTES;
  const int rs = (my_a ? 0 : 2) + (wg & 1);  // which 32 of the work group's 128 rows
  const int orow = 32 * rs + l32;            // this lane's row in the O tile
  float l_tot = halves_sum(l_run);
  __syncthreads();
  // rounds O^T tile dt (scaled by inv) into the O tile
  auto put = [&](int dt, float inv) {
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      u32x2_t w;
      w[0] = E::pack2(oacc[dt][4 * J] * inv, oacc[dt][4 * J + 1] * inv);
      w[1] = E::pack2(oacc[dt][4 * J + 2] * inv, oacc[dt][4 * J + 3] * inv);
      const int chunk = 4 * dt + J;
      *(u32x2_t*)(otile + orow * OROW + 16 * (chunk ^ kswz<D>(orow)) + 8 * hsel) = w;
    }
  };
  if constexpr (NG > 1) {
    // half h of the head dims (d tiles h DTH ..) is finalized by group h
    auto merge = [&](int h) {
      const int ex = rs * NG + grp, pe = rs * NG + (1 - h);
      xm[(ex * 2 + 0) * 64 + lane] = m_ref;
      xm[(ex * 2 + 1) * 64 + lane] = l_tot;
      // four values per lane and access: [slot][d tile][r / 4][lane][r % 4]
      f32x4_t* const xo4 = reinterpret_cast<f32x4_t*>(xo);
#pragma unroll
      for (int j = 0; j < DTH; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x16_t& src = oacc[(1 - h) * DTH + j];
          xo4[((ex * DTH + j) * 4 + r4) * 64 + lane] =
              f32x4_t{src[4 * r4], src[4 * r4 + 1], src[4 * r4 + 2], src[4 * r4 + 3]};
        }
      __syncthreads();
      const float m1 = xm[(pe * 2 + 0) * 64 + lane];
      const float l1 = xm[(pe * 2 + 1) * 64 + lane];
      const float mm = fmaxf(m_ref, m1);
      const float bm = mm == kNegInf ? 0.f : mm;
      const float a0 = fast_exp2(m_ref - bm);  // 0 for an empty side
      const float a1 = fast_exp2(m1 - bm);
#pragma unroll
      for (int j = 0; j < DTH; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4_t o1 = xo4[((pe * DTH + j) * 4 + r4) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            oacc[h * DTH + j][4 * r4 + e] = oacc[h * DTH + j][4 * r4 + e] * a0 + o1[e] * a1;
        }
      // the same terms in both groups, so both get the same l and m
      l_tot = l_tot * a0 + l1 * a1;
      m_ref = mm;
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
      if (my_valid) {
#pragma unroll
        for (int j = 0; j < DTH; ++j) put(h * DTH + j, inv);
      }
    };
    if (grp == 0)
      merge(0);
    else
      merge(1);
  } else {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (my_valid) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) put(dt, inv);
    }
  }
  __syncthreads();
  // LSE after the barrier: the barrier's release fence waits for every
  // outstanding store, so a store issued before it made all waves wait for a
  // write round trip to memory.
  if (grp == 0 && my_valid && qrow < sqv && hsel == 0 && p.lse != nullptr)
    p.lse[lseoff + (int64_t)qhead * p.lse_sh + qpos] =
        l_tot > 0.f ? (m_ref + fast_log2(l_tot)) * kLn2 : kNegInf;
  // O tile -> global, 16 bytes per thread: rows 0-63 are tile_a, 64-127 tile_b
  constexpr int NTH = 256 * NG;
  static_assert(kBM * DCH % NTH == 0, "O tile copy");
#pragma unroll
  for (int it = 0; it < kBM * DCH / NTH; ++it) {
    const int idx = it * NTH + tid;
    const int row = idx / DCH, chunk = idx % DCH;
    const int grow = 64 * (row < 64 ? tile_a : tile_b) + (row & 63);  // virtual row
    if ((row < 64 || b_valid) && grow < sqv) {
      const u32x4_t v = *(const u32x4_t*)(otile + row * OROW + 16 * (chunk ^ kswz<D>(row)));
      uint16_t* op = p.o + ooff + (int64_t)(h + vhead(grow)) * p.o_sh + (int64_t)vpos(grow) * p.o_ss;
      *(u32x4_t*)(op + 8 * chunk) = v;
    }
  }
}

template <bool BF16, int D, bool SOFTCAP, int NG>
void launch_s(const FwdParams& p, dim3 grid, hipStream_t stream) {
  const dim3 block(256 * NG);
  if constexpr (NG == 2) {
    if (p.pair_tiles != 0) {
      hipLaunchKernelGGL((prefill_kernel<BF16, D, SOFTCAP, 2, true>), grid, block, 0, stream, p);
      return;
    }
  }
  hipLaunchKernelGGL((prefill_kernel<BF16, D, SOFTCAP, NG, false>), grid, block, 0, stream, p);
}

template <bool BF16, int D, int NG>
hipError_t launch_g(const FwdParams& p, bool softcap, dim3 grid, hipStream_t stream) {
  if (softcap)
    launch_s<BF16, D, true, NG>(p, grid, stream);
  else
    launch_s<BF16, D, false, NG>(p, grid, stream);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_t(const FwdParams& p, int head_dim, bool softcap, dim3 grid, int groups,
                    hipStream_t stream) {
  switch (head_dim) {
    case 64:
      return groups == 1 ? launch_g<BF16, 64, 1>(p, softcap, grid, stream)
                         : launch_g<BF16, 64, 2>(p, softcap, grid, stream);
    case 128:
      return groups == 1 ? launch_g<BF16, 128, 1>(p, softcap, grid, stream)
                         : launch_g<BF16, 128, 2>(p, softcap, grid, stream);
    case 256: return launch_g<BF16, 256, 1>(p, softcap, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int prefill_rows_per_tile() { return kBM; }

hipError_t launch_prefill(const FwdParams& p_in, bool bf16, int head_dim, bool softcap, int grid,
                          int groups, hipStream_t stream) {
  // (unit, batch, tile) grid where the dimensions allow it; the XCD-grouped
  // GQA order and grids past the y / z limits index a linear grid.
  FwdParams p = p_in;
  const int upb = p.pack ? p.h_kv : p.h_q;  // units per batch entry
  p.grid3 = !p.xcd_group && p.batch <= 65535 && p.n_qt <= 65535 ? 1 : 0;
  const dim3 g = p.grid3 ? dim3(upb, p.batch, p.n_qt) : dim3(grid);
  return bf16 ? launch_t<true>(p, head_dim, softcap, g, groups, stream)
              : launch_t<false>(p, head_dim, softcap, g, groups, stream);
}

}  // namespace exattn
