// Backward of exact attention: dQ, dK, dV from Q, K, V, O, dO and the forward's
// LSE, by recomputing S and P tile by tile ("FlashAttention完整说明", section
// 二.2: the forward keeps only O and the softmax statistics, the backward
// recomputes the rest).  With P = exp(S - LSE) and D_i = dO_i . O_i:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,
//   dK = scale dS^T Q;
// a KV head's dK and dV sum over the query heads that read it.
//
// gfx950 design, deterministic (no atomics):
// - bwd_dq_kernel (launched first, below) also forms each query row's
//   statistics, D_i = dO_i . O_i and LSE in the log2 domain, from the O and dO
//   rows it loads, and stores them for the dK/dV kernel;
// - bwd_dkdv_kernel: a work group owns 128 keys (32 per wave) of one KV head and
//   walks the query blocks (32 rows) of every query head in its group.  K and V
//   of its keys stay in registers; Q, dO and the rows' statistics stream
//   through double-buffered LDS by DMA.  Per block a wave computes S = Q K^T and
//   dP = dO V^T (queries x keys, Q and dO the A operands with the row
//   permutation that makes 8 consecutive accumulator registers 8 consecutive
//   queries), then dV^T += dO^T P and dK^T += Q^T dS with P and dS rounded in
//   place as the B operand and dO^T / Q^T read transposed from LDS;
// - bwd_dq_kernel: a group of 2 waves owns 64 query rows (32 per wave) of one query
//   head and walks its KV blocks (64 keys) like the forward: S^T = K Q^T and
//   dP^T = V dO^T with Q^T and dO^T in registers, dS^T rounded in place as the
//   B operand of dQ^T += K^T dS^T, K^T read transposed from LDS; for small grids
//   two groups split the blocks (32 keys each) and add their partial dQ in LDS.
// The row statistics make P exact without a running max: LSE is final.
#include "device_common.h"
#include "kernels.h"
#include "tiles.h"

namespace exattn {
namespace {

constexpr int kBwdRows = 32;   // query rows per block of the dK/dV kernel
constexpr int kBwdKeys = 128;  // keys per work group of the dK/dV kernel
constexpr int kDqWaves = 2;    // waves (32 query rows each) per work group of the dQ kernel
constexpr int kDqRows = 32 * kDqWaves;
// keys per block of the dQ kernel: 64, or 32 when two wave groups split the keys
// (their four K/V stages then fit 64 KiB of LDS, two work groups per CU)
template <int NG>
constexpr int dq_keys() { return NG == 1 ? 64 : 32; }

// Is key j visible from query row i (bottom-right offset off = s_k - s_q)?
__device__ __forceinline__ bool visible_key(int i, int j, int sq, int sk, int off, int wl, int wr) {
  return i < sq && j < sk && (wr < 0 || j <= i + off + wr) && (wl < 0 || j >= i + off - wl);
}

// Tiles read both as A operands (16 lanes: 16 rows, one 16-byte chunk each)
// and transposed (lanes of one read: 4 consecutive rows x 2 or 4 adjacent
// chunks): chunk c of row r is stored at c ^ qswz(r).  Over 16 rows qswz takes
// 16 distinct values (8 per row parity for 128-byte rows, two of which share a
// 256-byte bank row), and 4 consecutive rows differ in bits 2-3 (bit 2 for the
// rows of one parity at d = 64), so both read shapes hit distinct bank groups.
template <int D>
__device__ __forceinline__ int qswz(int r) {
  if constexpr (D == 64)
    return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  else
    return 4 * (r & 3) + ((r >> 2) & 3);
}

// The two 16-bit values of a 32-bit word as floats.
template <bool BF16>
__device__ __forceinline__ float lo_f32(uint32_t w) {
  if constexpr (BF16)
    return __builtin_bit_cast(float, w << 16);
  else
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <bool BF16>
__device__ __forceinline__ float hi_f32(uint32_t w) {
  if constexpr (BF16)
    return __builtin_bit_cast(float, w & 0xffff0000u);
  else
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Softcap: P = 2^(c log2 e tanh(s scale / c) - LSE log2 e), and the gradient
// through c tanh(x / c) multiplies dS by 1 - tanh^2.  p_out: P; f_out: that
// factor (1 without softcap).
template <bool SOFTCAP>
__device__ __forceinline__ void probs(float s, float lse2, const BwdParams& p, float& p_out, float& f_out) {
  if constexpr (SOFTCAP) {
    const float t = tanh_exp2(s * p.cap_in);
    p_out = fast_exp2(__builtin_fmaf(t, p.cap_out_log2, -lse2));
    f_out = 1.0f - t * t;
  } else {
    p_out = fast_exp2(__builtin_fmaf(s, p.scale_log2, -lse2));
    f_out = 1.0f;
  }
}

// Token offsets of sequence b (varlen) or its batch offsets, and its lengths.
struct SeqSpan {
  int sq, sk;
  int64_t q, dout, o, dq;  // element offsets of the sequence's first query row
  int64_t k, v, dk, dv;    // ... and of its first key row
};
__device__ __forceinline__ SeqSpan seq_span(const BwdParams& p, int b) {
  SeqSpan r;
  if (p.cu_q != nullptr) {
    const int qs = p.cu_q[b], ks = p.cu_k[b];
    r.sq = p.cu_q[b + 1] - qs;
    r.sk = p.cu_k[b + 1] - ks;
    r.q = (int64_t)qs * p.q_ss, r.dout = (int64_t)qs * p.do_ss, r.o = (int64_t)qs * p.o_ss;
    r.dq = (int64_t)qs * p.dq_ss;
    r.k = (int64_t)ks * p.k_ss, r.v = (int64_t)ks * p.v_ss, r.dk = (int64_t)ks * p.dk_ss;
    r.dv = (int64_t)ks * p.dv_ss;
  } else {
    r.sq = p.s_q, r.sk = p.s_k;
    r.q = (int64_t)b * p.q_sb, r.dout = (int64_t)b * p.do_sb, r.o = (int64_t)b * p.o_sb;
    r.dq = (int64_t)b * p.dq_sb;
    r.k = (int64_t)b * p.k_sb, r.v = (int64_t)b * p.v_sb, r.dk = (int64_t)b * p.dk_sb;
    r.dv = (int64_t)b * p.dv_sb;
  }
  return r;
}

// dK, dV for 128 keys of one KV head (4 waves x 32 keys).
// DS: head-dim slices.  At d = 256 a wave's K and V (128 registers) and its
// dK and dV accumulators (256) leave too few of its 512 for the rest, so the
// work groups of a key tile split dK and dV into two halves of the head dims
// (DS = 2), each recomputing S and dP (a third more products).
template <bool BF16, int D, bool SOFTCAP, int DS>
__global__ void __launch_bounds__(256) bwd_dkdv_kernel(const BwdParams p) {
  using E = Elem<BF16>;
  constexpr int KS = D / 16;                   // k-steps over head_dim
  constexpr int DT = D / 32 / DS;              // 32-wide head_dim tiles of this work group's slice
  constexpr int DCH = D / 8;                   // 16-byte chunks per row
  constexpr int TILE = kBwdRows * D * 2;       // bytes of a Q (or dO) tile
  constexpr int ROWS_PER_KB = 1024 / (D * 2);  // rows per 1 KiB DMA slice
  constexpr int SLICES = TILE / 1024;          // DMA slices per tile
  constexpr int STAGE = 2 * TILE + 2 * 128;    // Q, dO, lse2[32], D[32]
  static_assert(SLICES >= 4 && SLICES % 4 == 0, "slices per wave");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hsel = lane >> 5;
  const int l32 = lane & 31;

  const int n_kt = (p.s_k + kBwdKeys - 1) / kBwdKeys;
  const int dsl = (int)blockIdx.x % DS;   // head-dim slice: dims 32 DT dsl ..
  const int bid = (int)blockIdx.x / DS;
  const int kt = bid % n_kt;
  const int hk = (bid / n_kt) % p.h_kv;
  const int b = bid / (n_kt * p.h_kv);
  const SeqSpan sp = seq_span(p, b);
  const int sq = sp.sq, sk = sp.sk, off = sk - sq;
  const int sqm = p.s_q;  // row stride of the statistics (the longest sequence)
  const int k0 = kt * kBwdKeys;
  if (k0 >= sk) return;  // uniform: a shorter sequence has no keys here
  const int kcol = k0 + 32 * wave + l32;  // this lane's key

  // ---- K and V of this lane's key as B operands: K[kcol][16 ks + 8 hsel .. +7].
  u32x4_t kf[KS], vf[KS];
  {
    const uint16_t* kp = p.k + sp.k + (int64_t)kcol * p.k_ss + (int64_t)hk * p.k_sh + 8 * hsel;
    const uint16_t* vp = p.v + sp.v + (int64_t)kcol * p.v_ss + (int64_t)hk * p.v_sh + 8 * hsel;
    const bool in = kcol < sk;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = in ? *(const u32x4_t*)(kp + 16 * ks) : u32x4_t{0, 0, 0, 0};
      vf[ks] = in ? *(const u32x4_t*)(vp + 16 * ks) : u32x4_t{0, 0, 0, 0};
    }
  }

  // ---- query rows that see any of keys k0 .. k0 + 127 (per head the same).
  const int k1 = min(k0 + kBwdKeys, sk) - 1;
  const int wr = p.wr;
  int i_lo = 0, i_hi = sq - 1;
  if (wr >= 0) i_lo = max(0, k0 - off - wr);
  if (p.wl >= 0) i_hi = min(sq - 1, k1 - off + p.wl);
  const int qb_lo = i_lo / kBwdRows;
  const int qb_hi = i_hi >= i_lo ? i_hi / kBwdRows + 1 : qb_lo;  // exclusive
  const int nqb = qb_hi - qb_lo;
  const int g = p.group;
  const int steps = nqb * g;  // (head, query block) pairs

  // ---- DMA: tile row r, stored chunk (lane % DCH) at r * D * 2 + 16 * ((lane % DCH) ^ qswz(r)).
  uint32_t q_ofs[SLICES / 4], d_ofs[SLICES / 4];
#pragma unroll
  for (int i = 0; i < SLICES / 4; ++i) {
    const int row = (4 * i + wave) * ROWS_PER_KB + lane / DCH;
    q_ofs[i] = (uint32_t)(row * p.q_ss + 8 * ((lane % DCH) ^ qswz<D>(row))) * 2u;
    d_ofs[i] = (uint32_t)(row * p.do_ss + 8 * ((lane % DCH) ^ qswz<D>(row))) * 2u;
  }
  const uint16_t* const qb_ptr = p.q + sp.q;
  const uint16_t* const db_ptr = p.dout + sp.dout;
  const float* const sb_ptr = p.ws_stats + (int64_t)b * p.h_q * sqm * 2;
  auto issue = [&](int st, uint8_t* dst) {
    const int h = hk * g + st / nqb;
    const int q0 = (qb_lo + st % nqb) * kBwdRows;
    const __amdgpu_buffer_rsrc_t rq = block_rsrc<D>(qb_ptr + (int64_t)h * p.q_sh, p.q_ss, q0, sq, kBwdRows);
    const __amdgpu_buffer_rsrc_t rd = block_rsrc<D>(db_ptr + (int64_t)h * p.do_sh, p.do_ss, q0, sq, kBwdRows);
    // the rows' statistics: 32 (lse2, D) pairs, 256 bytes, by lanes 0-15 of wave 0
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(sb_ptr + ((int64_t)h * sqm + q0) * 2), 0, 8 * min(kBwdRows, sq - q0), 0x00020000);
#pragma unroll
    for (int i = 0; i < SLICES / 4; ++i) {
      buffer_load_lds16(rq, dst + (4 * i + wave) * 1024, q_ofs[i]);
      buffer_load_lds16(rd, dst + TILE + (4 * i + wave) * 1024, d_ofs[i]);
    }
    if (wave == 0 && lane < 16) buffer_load_lds16(rs, dst + 2 * TILE, 16u * lane);
  };

  // ---- loop-invariant LDS addresses.
  // A operand of S = Q K^T (and dP = dO V^T): row m = l32 is query row_key(l32)
  // of the block, chunk 2 ks + hsel.
  const int arow = row_key(l32);
  int aaddr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) aaddr[ks] = arow * (D * 2) + 16 * ((2 * ks + hsel) ^ qswz<D>(arow));
  // Transposed A operands (dO^T, Q^T; rows = head dims, k = 8 consecutive
  // queries per lane half) for MFMA (c, dt): two transposing reads of 4 rows.
  const int gi = lane >> 4, li = lane & 15;
  int tr[2][DT];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int row = 8 * (gi >> 1) + 4 * half + (li >> 2);
      const int dcol = 32 * (DT * dsl + dt) + 16 * (gi & 1) + 4 * (li & 3);
      tr[half][dt] = row * (D * 2) + 16 * ((dcol >> 3) ^ qswz<D>(row)) + 2 * (dcol & 7);
    }

  f32x16_t dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dk[dt] = dv[dt] = f32x16_t{};

  // One (head, query block) pair: stage stg holds its tiles; the next pair's
  // DMA into nxt is issued once this pair's first products are under way.
  auto block = [&](int st, const uint8_t* __restrict__ stg, uint8_t* __restrict__ nxt) {
    const uint8_t* qt = stg;
    const uint8_t* dt_ = stg + TILE;
    const float* stats = reinterpret_cast<const float*>(stg + 2 * TILE);  // (lse2, D) per row
    const int q0 = (qb_lo + st % nqb) * kBwdRows;
    f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = E::mfma32x32x16(*(const u32x4_t*)(qt + aaddr[ks]), kf[ks], s);
      dp = E::mfma32x32x16(*(const u32x4_t*)(dt_ + aaddr[ks]), vf[ks], dp);
    }
    if (st + 1 < steps) issue(st + 1, nxt);
    // register 8c + u of lane half H holds query q0 + 16 c + 8 H + u.  A block whose
    // 32 x 32 pairs are all visible (rows and keys in range, inside the causal /
    // window band) skips the mask.
    const int kc0 = k0 + 32 * wave;
    const bool full = q0 + kBwdRows <= sq && kc0 + 32 <= sk && (wr < 0 || kc0 + 31 <= q0 + off + wr) &&
                      (p.wl < 0 || kc0 >= q0 + kBwdRows - 1 + off - p.wl);
    u32x4_t pb[2], sb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int qi = 16 * c + 8 * hsel;
      f32x4_t rs[4];  // rows qi + 2 j, qi + 2 j + 1: (lse2, D, lse2, D)
#pragma unroll
      for (int j = 0; j < 4; ++j) rs[j] = *(const f32x4_t*)(stats + 2 * (qi + 2 * j));
      float pv[8], sv[8], fv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) probs<SOFTCAP>(s[8 * c + u], rs[u >> 1][2 * (u & 1)], p, pv[u], fv[u]);
      if (!full) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (!visible_key(q0 + qi + u, kcol, sq, sk, off, p.wl, wr)) pv[u] = 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        sv[u] = pv[u] * (dp[8 * c + u] - rs[u >> 1][2 * (u & 1) + 1]);
        if constexpr (SOFTCAP) sv[u] *= fv[u];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pb[c][e] = E::pack2(pv[2 * e], pv[2 * e + 1]);
        sb[c][e] = E::pack2(sv[2 * e], sv[2 * e + 1]);
      }
    }
    // dV^T += dO^T P, dK^T += Q^T dS: k = queries 16 c + 8 H + 0..7
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int rows = 16 * c * (D * 2);
        u32x4_t ad, aq;
        const u32x2_t d0 = lds_read_tr16(dt_ + tr[0][dt] + rows), d1 = lds_read_tr16(dt_ + tr[1][dt] + rows);
        const u32x2_t q0v = lds_read_tr16(qt + tr[0][dt] + rows), q1v = lds_read_tr16(qt + tr[1][dt] + rows);
        ad[0] = d0[0], ad[1] = d0[1], ad[2] = d1[0], ad[3] = d1[1];
        aq[0] = q0v[0], aq[1] = q0v[1], aq[2] = q1v[0], aq[3] = q1v[1];
        dv[dt] = E::mfma32x32x16(ad, pb[c], dv[dt]);
        dk[dt] = E::mfma32x32x16(aq, sb[c], dk[dt]);
      }
  };

  uint8_t* const st0 = smem;
  uint8_t* const st1 = smem + STAGE;
  if (steps > 0) issue(0, st0);
  for (int st = 0; st < steps; st += 2) {
    wait_vmem_all();
    __syncthreads();
    block(st, st0, st1);
    if (st + 1 < steps) {
      wait_vmem_all();
      __syncthreads();
      block(st + 1, st1, st0);
    }
  }

  // ---- dK = scale (dK^T)^T, dV = (dV^T)^T: lane holds head dims 32 dt + 8 J + 4 H + 0..3.
  if (kcol < sk) {
    uint16_t* kq = p.dk + sp.dk + (int64_t)kcol * p.dk_ss + (int64_t)hk * p.dk_sh;
    uint16_t* vq = p.dv + sp.dv + (int64_t)kcol * p.dv_ss + (int64_t)hk * p.dv_sh;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        u32x2_t wk, wv;
        wk[0] = E::pack2(dk[dt][4 * J] * p.scale, dk[dt][4 * J + 1] * p.scale);
        wk[1] = E::pack2(dk[dt][4 * J + 2] * p.scale, dk[dt][4 * J + 3] * p.scale);
        wv[0] = E::pack2(dv[dt][4 * J], dv[dt][4 * J + 1]);
        wv[1] = E::pack2(dv[dt][4 * J + 2], dv[dt][4 * J + 3]);
        *(u32x2_t*)(kq + 32 * (DT * dsl + dt) + 8 * J + 4 * hsel) = wk;
        *(u32x2_t*)(vq + 32 * (DT * dsl + dt) + 8 * J + 4 * hsel) = wv;
      }
  }
}

// dK, dV for 32 x (8 / NSET) keys of one KV head with 8 waves (d = 128):
// NSET sets of 8 / NSET waves (32 keys each) take turns over the (query head,
// query block) steps, each set with its own double-buffered Q / dO stage.  K
// and V of the keys are loaded once into LDS and read there as the B operands,
// which leaves a wave about 230 registers, so two waves share each SIMD: one
// wave's LDS reads and exponentials run under the other's products.  The sets'
// partial dK, dV are added through LDS at the end in a fixed order
// (deterministic).
// NSET = 2: 128 keys per work group, the rows' statistics ride with the Q / dO
// DMA.  NSET = 4: 64 keys, twice the work groups, issued heaviest first: under
// a causal mask the first key tiles see the most query rows, and with more
// work groups than CUs the dispatcher hands the light tiles to the CUs that
// finish first (with 128-key tiles the grid is often one work group per CU and
// the heaviest tile alone sets the time).  The 4 sets' stages fill the 160 KiB
// of LDS, so the statistics come from memory into registers instead.
template <bool BF16, int D, bool SOFTCAP, int NSET>
__global__ void __launch_bounds__(512) bwd_dkdv2_kernel(const BwdParams p) {
  using E = Elem<BF16>;
  constexpr int KS = D / 16;                   // k-steps over head_dim
  constexpr int DT = D / 32;                   // 32-wide head_dim tiles
  constexpr int DCH = D / 8;                   // 16-byte chunks per row
  constexpr int TILE = kBwdRows * D * 2;       // bytes of a Q (or dO) tile
  constexpr int ROWS_PER_KB = 1024 / (D * 2);  // rows per 1 KiB DMA slice
  constexpr int SLICES = TILE / 1024;          // DMA slices per Q tile
  static_assert(NSET == 2 || NSET == 4, "2 or 4 sets");
  constexpr int WPS = 8 / NSET;                // waves per set
  constexpr int KEYS = 32 * WPS;               // keys per work group
  constexpr bool kStatsLds = NSET == 2;        // statistics through LDS (else from memory)
  constexpr int STAGE = 2 * TILE + (kStatsLds ? 2 * 128 : 0);  // Q, dO (, lse2[32], D[32])
  constexpr int KVT = KEYS * D * 2;            // bytes of the K (or V) tile
  constexpr int KVSL = KVT / 1024;             // DMA slices per K tile
  static_assert(SLICES % WPS == 0 && KVSL % 8 == 0, "slices per wave");
  constexpr int LDS_MAIN = 2 * KVT + NSET * 2 * STAGE;
  constexpr int LDS_RED = 4 * 2 * DT * 16 * 64 * 4;  // 4 waves' dK and dV partials
  constexpr int LDS = LDS_MAIN > LDS_RED ? LDS_MAIN : LDS_RED;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int set = wave / WPS;  // which steps: set, set + NSET, ...
  const int w4 = wave % WPS;   // which 32 keys
  const int hsel = lane >> 5;
  const int l32 = lane & 31;

  const int n_kt = (p.s_k + KEYS - 1) / KEYS;
  const int bid = blockIdx.x;
  int kt, hk, b;
  if constexpr (NSET == 2) {
    kt = bid % n_kt;
    hk = (bid / n_kt) % p.h_kv;
    b = bid / (n_kt * p.h_kv);
  } else {  // key tiles major: tile 0 of every (batch, KV head) first
    const int units = p.batch * p.h_kv;
    kt = bid / units;
    hk = bid % units % p.h_kv;
    b = bid % units / p.h_kv;
  }
  const SeqSpan sp = seq_span(p, b);
  const int sq = sp.sq, sk = sp.sk, off = sk - sq;
  const int sqm = p.s_q;  // row stride of the statistics (the longest sequence)
  const int k0 = kt * KEYS;
  if (k0 >= sk) return;  // uniform: a shorter sequence has no keys here
  const int kcol = k0 + 32 * w4 + l32;  // this lane's key

  // ---- K and V of the keys into LDS (row = key, chunk c at c ^ kswz(key)),
  // 1 KiB slices, slice wave + 8 i by each wave; keys past the end read as 0.
  uint8_t* const kt_lds = smem;
  uint8_t* const vt_lds = smem + KVT;
  {
    const __amdgpu_buffer_rsrc_t rk =
        block_rsrc<D>(p.k + sp.k + (int64_t)hk * p.k_sh, p.k_ss, k0, sk, KEYS);
    const __amdgpu_buffer_rsrc_t rv =
        block_rsrc<D>(p.v + sp.v + (int64_t)hk * p.v_sh, p.v_ss, k0, sk, KEYS);
#pragma unroll
    for (int i = 0; i < KVSL / 8; ++i) {
      const int sl = wave + 8 * i;
      const int row = sl * ROWS_PER_KB + lane / DCH;
      const int ch = (lane % DCH) ^ kswz<D>(row);
      buffer_load_lds16(rk, kt_lds + sl * 1024, (uint32_t)(row * p.k_ss + 8 * ch) * 2u);
      buffer_load_lds16(rv, vt_lds + sl * 1024, (uint32_t)(row * p.v_ss + 8 * ch) * 2u);
    }
  }

  // ---- query rows that see any of keys k0 .. k0 + KEYS - 1 (per head the same).
  const int k1 = min(k0 + KEYS, sk) - 1;
  const int wr = p.wr;
  int i_lo = 0, i_hi = sq - 1;
  if (wr >= 0) i_lo = max(0, k0 - off - wr);
  if (p.wl >= 0) i_hi = min(sq - 1, k1 - off + p.wl);
  const int qb_lo = i_lo / kBwdRows;
  const int qb_hi = i_hi >= i_lo ? i_hi / kBwdRows + 1 : qb_lo;  // exclusive
  const int nqb = qb_hi - qb_lo;
  const int g = p.group;
  const int steps = nqb * g;  // (head, query block) pairs; set s takes s, s + NSET, ...

  // ---- Q / dO DMA of this set: tile row r, stored chunk (lane % DCH) at
  // r * D * 2 + 16 * ((lane % DCH) ^ qswz(r)); slices w4 + WPS i.
  uint32_t q_ofs[SLICES / WPS], d_ofs[SLICES / WPS];
#pragma unroll
  for (int i = 0; i < SLICES / WPS; ++i) {
    const int row = (WPS * i + w4) * ROWS_PER_KB + lane / DCH;
    q_ofs[i] = (uint32_t)(row * p.q_ss + 8 * ((lane % DCH) ^ qswz<D>(row))) * 2u;
    d_ofs[i] = (uint32_t)(row * p.do_ss + 8 * ((lane % DCH) ^ qswz<D>(row))) * 2u;
  }
  const uint16_t* const qb_ptr = p.q + sp.q;
  const uint16_t* const db_ptr = p.dout + sp.dout;
  const float* const sb_ptr = p.ws_stats + (int64_t)b * p.h_q * sqm * 2;
  // the (lse2, D) pairs of step st's 32 rows; rows past the end read as 0
  auto stats_rsrc = [&](int st) {
    const int h = hk * g + st / nqb;
    const int q0 = (qb_lo + st % nqb) * kBwdRows;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(sb_ptr + ((int64_t)h * sqm + q0) * 2), 0,
                                             8 * min(kBwdRows, sq - q0), 0x00020000);
  };
  auto issue = [&](int st, uint8_t* dst) {
    const int h = hk * g + st / nqb;
    const int q0 = (qb_lo + st % nqb) * kBwdRows;
    const __amdgpu_buffer_rsrc_t rq = block_rsrc<D>(qb_ptr + (int64_t)h * p.q_sh, p.q_ss, q0, sq, kBwdRows);
    const __amdgpu_buffer_rsrc_t rd = block_rsrc<D>(db_ptr + (int64_t)h * p.do_sh, p.do_ss, q0, sq, kBwdRows);
#pragma unroll
    for (int i = 0; i < SLICES / WPS; ++i) {
      buffer_load_lds16(rq, dst + (WPS * i + w4) * 1024, q_ofs[i]);
      buffer_load_lds16(rd, dst + TILE + (WPS * i + w4) * 1024, d_ofs[i]);
    }
    if constexpr (kStatsLds) {
      if (w4 == 0 && lane < 16) buffer_load_lds16(stats_rsrc(st), dst + 2 * TILE, 16u * lane);
    }
  };

  // ---- loop-invariant LDS addresses.
  // A operand of S = Q K^T (and dP = dO V^T): row m = l32 is query row_key(l32)
  // of the block, chunk 2 ks + hsel.
  const int arow = row_key(l32);
  int aaddr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) aaddr[ks] = arow * (D * 2) + 16 * ((2 * ks + hsel) ^ qswz<D>(arow));
  // B operand (K or V of this lane's key, head dims 16 ks + 8 hsel .. +7).
  const int krow = 32 * w4 + l32;
  int baddr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) baddr[ks] = krow * (D * 2) + 16 * ((2 * ks + hsel) ^ kswz<D>(krow));
  // Transposed A operands (dO^T, Q^T; rows = head dims, k = 8 consecutive
  // queries per lane half) for MFMA (c, dt): two transposing reads of 4 rows.
  const int gi = lane >> 4, li = lane & 15;
  int tr[2][DT];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int row = 8 * (gi >> 1) + 4 * half + (li >> 2);
      const int dcol = 32 * dt + 16 * (gi & 1) + 4 * (li & 3);
      tr[half][dt] = row * (D * 2) + 16 * ((dcol >> 3) ^ qswz<D>(row)) + 2 * (dcol & 7);
    }

  f32x16_t dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dk[dt] = dv[dt] = f32x16_t{};

  // One (head, query block) pair: stage stg holds its tiles; the set's next
  // pair's DMA into nxt is issued once this pair's first products are under way.
  auto block = [&](int st, const uint8_t* __restrict__ stg, uint8_t* __restrict__ nxt) {
    const uint8_t* qt = stg;
    const uint8_t* dt_ = stg + TILE;
    const float* stats = reinterpret_cast<const float*>(stg + 2 * TILE);  // (lse2, D) per row
    const int q0 = (qb_lo + st % nqb) * kBwdRows;
    // from memory: rows 16 c + 8 hsel + 2 j, + 1 as (lse2, D, lse2, D), issued
    // now and first needed after the products
    f32x4_t rsm[2][4];
    if constexpr (!kStatsLds) {
      const __amdgpu_buffer_rsrc_t rsr = stats_rsrc(st);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          rsm[c][j] = __builtin_bit_cast(f32x4_t, buffer_load16(rsr, (uint32_t)(8 * (16 * c + 8 * hsel + 2 * j))));
    }
    f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = E::mfma32x32x16(*(const u32x4_t*)(qt + aaddr[ks]), *(const u32x4_t*)(kt_lds + baddr[ks]), s);
      dp = E::mfma32x32x16(*(const u32x4_t*)(dt_ + aaddr[ks]), *(const u32x4_t*)(vt_lds + baddr[ks]), dp);
    }
    if (st + NSET < steps) issue(st + NSET, nxt);
    const int kc0 = k0 + 32 * w4;
    const bool full = q0 + kBwdRows <= sq && kc0 + 32 <= sk && (wr < 0 || kc0 + 31 <= q0 + off + wr) &&
                      (p.wl < 0 || kc0 >= q0 + kBwdRows - 1 + off - p.wl);
    u32x4_t pb[2], sb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int qi = 16 * c + 8 * hsel;
      f32x4_t rs[4];  // rows qi + 2 j, qi + 2 j + 1: (lse2, D, lse2, D)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (kStatsLds)
          rs[j] = *(const f32x4_t*)(stats + 2 * (qi + 2 * j));
        else
          rs[j] = rsm[c][j];
      }
      float pv[8], sv[8], fv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) probs<SOFTCAP>(s[8 * c + u], rs[u >> 1][2 * (u & 1)], p, pv[u], fv[u]);
      if (!full) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (!visible_key(q0 + qi + u, kcol, sq, sk, off, p.wl, wr)) pv[u] = 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        sv[u] = pv[u] * (dp[8 * c + u] - rs[u >> 1][2 * (u & 1) + 1]);
        if constexpr (SOFTCAP) sv[u] *= fv[u];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pb[c][e] = E::pack2(pv[2 * e], pv[2 * e + 1]);
        sb[c][e] = E::pack2(sv[2 * e], sv[2 * e + 1]);
      }
    }
    // dV^T += dO^T P, dK^T += Q^T dS: k = queries 16 c + 8 H + 0..7
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int rows = 16 * c * (D * 2);
        u32x4_t ad, aq;
        const u32x2_t d0 = lds_read_tr16(dt_ + tr[0][dt] + rows), d1 = lds_read_tr16(dt_ + tr[1][dt] + rows);
        const u32x2_t q0v = lds_read_tr16(qt + tr[0][dt] + rows), q1v = lds_read_tr16(qt + tr[1][dt] + rows);
        ad[0] = d0[0], ad[1] = d0[1], ad[2] = d1[0], ad[3] = d1[1];
        aq[0] = q0v[0], aq[1] = q0v[1], aq[2] = q1v[0], aq[3] = q1v[1];
        dv[dt] = E::mfma32x32x16(ad, pb[c], dv[dt]);
        dk[dt] = E::mfma32x32x16(aq, sb[c], dk[dt]);
      }
  };

  uint8_t* const st0 = smem + 2 * KVT + set * 2 * STAGE;
  uint8_t* const st1 = st0 + STAGE;
  if (set < steps) issue(set, st0);
  // every wave runs the same number of iterations and meets every barrier;
  // the first barrier also publishes the K and V tiles
  const int iters = (steps + NSET - 1) / NSET;
  for (int t = 0; t < iters; t += 2) {
    wait_vmem_all();
    __syncthreads();
    if (set + NSET * t < steps) block(set + NSET * t, st0, st1);
    if (t + 1 < iters) {
      wait_vmem_all();
      __syncthreads();
      if (set + NSET * (t + 1) < steps) block(set + NSET * (t + 1), st1, st0);
    }
  }
  wait_vmem_all();  // the K / V DMA when there was no step

  // ---- the sets hand their partial dK^T, dV^T on through LDS (everything in
  // LDS is free once every wave has passed the barrier): with 2 sets set 1 to
  // set 0; with 4 sets 2 -> 0 and 3 -> 1, then 1 -> 0, so the sum is always
  // (s0 + s2) + (s1 + s3).
  __syncthreads();
  float* const red = reinterpret_cast<float*>(smem);  // [publishing wave][dk, dv][dt][j][lane][4]
  auto slot = [&](int pw, int which, int dt, int j) {
    return red + ((((pw * 2 + which) * DT + dt) * 4 + j) * 64 + lane) * 4;
  };
  auto publish = [&](int pw) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *(f32x4_t*)slot(pw, 0, dt, j) = f32x4_t{dk[dt][4 * j], dk[dt][4 * j + 1], dk[dt][4 * j + 2], dk[dt][4 * j + 3]};
        *(f32x4_t*)slot(pw, 1, dt, j) = f32x4_t{dv[dt][4 * j], dv[dt][4 * j + 1], dv[dt][4 * j + 2], dv[dt][4 * j + 3]};
      }
  };
  auto absorb = [&](int pw) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4_t a = *(const f32x4_t*)slot(pw, 0, dt, j);
        const f32x4_t c = *(const f32x4_t*)slot(pw, 1, dt, j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dk[dt][4 * j + e] += a[e];
          dv[dt][4 * j + e] += c[e];
        }
      }
  };
  if constexpr (NSET == 4) {
    // All 8 waves finalize: wave (set s, w4) owns head-dim tile s of its 32
    // keys.  It publishes the 3 tiles the other sets own, sums its own tile
    // over the 4 sets in the fixed order (s0 + s2) + (s1 + s3), and writes it,
    // rounded, into a [64 keys][128 dims] LDS tile that all threads then store
    // as whole rows (16 bytes per thread); dK first, then dV.
    static_assert(DT == NSET, "one head-dim tile per set");
    static_assert(8 * DT * 16 * 64 * 4 + 2 * KEYS * D * 2 <= LDS, "partials and two output tiles");
    float* const part = reinterpret_cast<float*>(smem);  // [wave][dt][j][lane][4]
    uint8_t* const tile_k = smem + 8 * DT * 16 * 64 * 4;
    uint8_t* const tile_v = tile_k + KEYS * D * 2;
    auto pslot = [&](int w, int dt, int j) { return part + (((w * DT + dt) * 4 + j) * 64 + lane) * 4; };
    auto publish_m = [&](const f32x16_t(&m)[DT]) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        if (dt != set) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *(f32x4_t*)pslot(wave, dt, j) = f32x4_t{m[dt][4 * j], m[dt][4 * j + 1], m[dt][4 * j + 2], m[dt][4 * j + 3]};
        }
    };
    // this wave's tile summed over the sets, rounded into the output tile,
    // 4 registers (one row group J) at a time
    auto finalize = [&](const f32x16_t(&m)[DT], uint8_t* tile, float mul) {
      const int key = 32 * w4 + l32;
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        f32x4_t x[4];  // set t's values of registers 4 J .. 4 J + 3
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (t == set) {
            x[t] = f32x4_t{m[0][4 * J], m[0][4 * J + 1], m[0][4 * J + 2], m[0][4 * J + 3]};
#pragma unroll
            for (int dt = 1; dt < DT; ++dt)
              if (dt == set) x[t] = f32x4_t{m[dt][4 * J], m[dt][4 * J + 1], m[dt][4 * J + 2], m[dt][4 * J + 3]};
          } else {
            x[t] = *(const f32x4_t*)pslot(t * WPS + w4, set, J);
          }
        }
        const f32x4_t r = (x[0] + x[2]) + (x[1] + x[3]);
        u32x2_t w;  // head dims 32 set + 8 J + 4 hsel + 0..3
        w[0] = E::pack2(r[0] * mul, r[1] * mul);
        w[1] = E::pack2(r[2] * mul, r[3] * mul);
        const int chunk = 4 * set + J;
        *(u32x2_t*)(tile + key * (D * 2) + 16 * (chunk ^ kswz<D>(key)) + 8 * hsel) = w;
      }
    };
    // the output tile to global memory, 16 bytes per thread, whole rows
    auto store_tile = [&](const uint8_t* tile, uint16_t* base, int64_t ss, int64_t sh) {
#pragma unroll
      for (int it = 0; it < KEYS * DCH / 512; ++it) {
        const int idx = it * 512 + tid;
        const int key = idx / DCH, chunk = idx % DCH;
        if (k0 + key < sk) {
          const u32x4_t val = *(const u32x4_t*)(tile + key * (D * 2) + 16 * (chunk ^ kswz<D>(key)));
          *(u32x4_t*)(base + (int64_t)(k0 + key) * ss + (int64_t)hk * sh + 8 * chunk) = val;
        }
      }
    };
    publish_m(dk);
    __syncthreads();
    finalize(dk, tile_k, p.scale);
    __syncthreads();  // every dK partial read: the region takes dV's
    publish_m(dv);
    store_tile(tile_k, p.dk + sp.dk, p.dk_ss, p.dk_sh);
    __syncthreads();
    finalize(dv, tile_v, 1.0f);
    __syncthreads();
    store_tile(tile_v, p.dv + sp.dv, p.dv_ss, p.dv_sh);
    return;
  } else {
    if (set == 1) publish(w4);
    __syncthreads();
    if (set != 0) return;
    absorb(w4);
  }

  // ---- dK = scale (dK^T)^T, dV = (dV^T)^T: lane holds head dims 32 dt + 8 J + 4 H + 0..3.
  if (kcol < sk) {
    uint16_t* kq = p.dk + sp.dk + (int64_t)kcol * p.dk_ss + (int64_t)hk * p.dk_sh;
    uint16_t* vq = p.dv + sp.dv + (int64_t)kcol * p.dv_ss + (int64_t)hk * p.dv_sh;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        u32x2_t wk, wv;
        wk[0] = E::pack2(dk[dt][4 * J] * p.scale, dk[dt][4 * J + 1] * p.scale);
        wk[1] = E::pack2(dk[dt][4 * J + 2] * p.scale, dk[dt][4 * J + 3] * p.scale);
        wv[0] = E::pack2(dv[dt][4 * J], dv[dt][4 * J + 1]);
        wv[1] = E::pack2(dv[dt][4 * J + 2], dv[dt][4 * J + 3]);
        *(u32x2_t*)(kq + 32 * dt + 8 * J + 4 * hsel) = wk;
        *(u32x2_t*)(vq + 32 * dt + 8 * J + 4 * hsel) = wv;
      }
  }
}

// dQ for 64 query rows of one query head (2 waves x 32 rows; two work groups
// share a CU, which measured 3% faster than one of 4 waves).
template <bool BF16, int D, int NG, bool SOFTCAP>
__global__ void __launch_bounds__(64 * kDqWaves * NG) bwd_dq_kernel(const BwdParams p) {
  using E = Elem<BF16>;
  constexpr int BN = dq_keys<NG>();
  constexpr int NT2 = BN / 32;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int DCH = D / 8;
  constexpr int KTILE = BN * D * 2;
  constexpr int ROWS_PER_KB = 1024 / (D * 2);
  constexpr int NW = kDqWaves;
  constexpr int KINST = KTILE / (1024 * NW);  // DMA instructions per wave per tile
  static_assert(KINST >= 1, "tile / wave mismatch");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NG * 4 * KTILE];  // per group: K, V double-buffered

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wv / NW;   // key-block group: blocks n_lo + grp, + NG, ...
  const int wave = wv % NW;  // row slice of the tile
  const int hsel = lane >> 5;
  const int l32 = lane & 31;

  const int n_qt = (p.s_q + kDqRows - 1) / kDqRows;
  const int units = p.batch * p.h_q;
  const int qt = n_qt - 1 - (int)blockIdx.x / units;  // heaviest (last) tiles first
  const int u = blockIdx.x % units;
  const int b = u / p.h_q, h = u % p.h_q;
  const int hk = h / p.group;
  const SeqSpan sp = seq_span(p, b);
  const int sq = sp.sq, sk = sp.sk, off = sk - sq;
  const int sqm = p.s_q;  // row stride of the statistics
  const int q0 = qt * kDqRows;
  if (q0 >= sq) return;  // uniform: a shorter sequence has no rows here
  const int q0w = q0 + 32 * wave;  // this wave's first row
  const int qrow = q0w + l32;

  // ---- visible key blocks of the tile.
  const int t1 = min(q0 + kDqRows, sq) - 1;
  int kmin = 0, kmax = sk - 1;
  if (p.wl >= 0) kmin = max(0, q0 + off - p.wl);
  if (p.wr >= 0) kmax = min(kmax, t1 + off + p.wr);
  const int n_lo = kmax >= kmin ? kmin / BN : 0;
  const int n_hi = kmax >= kmin ? kmax / BN + 1 : 0;

  // ---- Q^T and dO^T as B operands: lane holds row qrow, head dims 16 ks + 8 hsel .. +7.
  u32x4_t qf[KS], df[KS];
  {
    const bool in = qrow < sq;
    const uint16_t* qp = p.q + sp.q + (int64_t)qrow * p.q_ss + (int64_t)h * p.q_sh + 8 * hsel;
    const uint16_t* dp = p.dout + sp.dout + (int64_t)qrow * p.do_ss + (int64_t)h * p.do_sh + 8 * hsel;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = in ? *(const u32x4_t*)(qp + 16 * ks) : u32x4_t{0, 0, 0, 0};
      df[ks] = in ? *(const u32x4_t*)(dp + 16 * ks) : u32x4_t{0, 0, 0, 0};
    }
  }
  // O of this lane's row in the layout of dO^T (for D_i = dO_i . O_i), and its LSE
  u32x4_t of[KS];
  float lse_in = kNegInf;
  {
    const bool in = qrow < sq;
    const uint16_t* op = p.o + sp.o + (int64_t)qrow * p.o_ss + (int64_t)h * p.o_sh + 8 * hsel;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) of[ks] = in ? *(const u32x4_t*)(op + 16 * ks) : u32x4_t{0, 0, 0, 0};
    const int64_t lb = p.cu_q != nullptr ? (int64_t)h * p.lse_sh + p.cu_q[b]
                                         : (int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh;
    if (in) lse_in = p.lse[lb + qrow];
  }
  float lse2, drow;  // the row's statistics, formed below

  const uint16_t* kg = p.k + sp.k + (int64_t)hk * p.k_sh;
  const uint16_t* vg = p.v + sp.v + (int64_t)hk * p.v_sh;
  uint32_t kofs[KINST], vofs[KINST];
#pragma unroll
  for (int i = 0; i < KINST; ++i) {
    const int row = (NW * i + wave) * ROWS_PER_KB + lane / DCH;
    kofs[i] = (uint32_t)(row * p.k_ss + 8 * ((lane % DCH) ^ qswz<D>(row))) * 2u;
    vofs[i] = (uint32_t)(row * p.v_ss + 8 * ((lane % DCH) ^ qswz<D>(row))) * 2u;
  }
  auto issue = [&](int n, uint8_t* kdst, uint8_t* vdst) {
    const __amdgpu_buffer_rsrc_t rk = block_rsrc<D>(kg, p.k_ss, n * BN, sk, BN);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc<D>(vg, p.v_ss, n * BN, sk, BN);
#pragma unroll
    for (int i = 0; i < KINST; ++i) {
      buffer_load_lds16(rk, kdst + (NW * i + wave) * 1024, kofs[i]);
      buffer_load_lds16(rv, vdst + (NW * i + wave) * 1024, vofs[i]);
    }
  };

  // A operand of S^T = K Q^T and dP^T = V dO^T: tile t2 row m = l32 is key
  // 32 t2 + row_key(l32), chunk 2 ks + hsel.
  const int krow = row_key(l32);
  int aaddr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) aaddr[ks] = krow * (D * 2) + 16 * ((2 * ks + hsel) ^ qswz<D>(krow));
  // K^T operand (rows = head dims, k = 8 consecutive keys per lane half).
  const int gi = lane >> 4, li = lane & 15;
  int tr[2][DT];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int row = 8 * (gi >> 1) + 4 * half + (li >> 2);
      const int dcol = 32 * dt + 16 * (gi & 1) + 4 * (li & 3);
      tr[half][dt] = row * (D * 2) + 16 * ((dcol >> 3) ^ qswz<D>(row)) + 2 * (dcol & 7);
    }

  f32x16_t dq[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dq[dt] = f32x16_t{};

  auto block = [&](int n, const uint8_t* __restrict__ kt, const uint8_t* __restrict__ vt) {
    f32x16_t s[NT2], dp[NT2];
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2) s[t2] = dp[t2] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int t2 = 0; t2 < NT2; ++t2) {
        const int o = aaddr[ks] + t2 * 32 * (D * 2);
        s[t2] = E::mfma32x32x16(*(const u32x4_t*)(kt + o), qf[ks], s[t2]);
        dp[t2] = E::mfma32x32x16(*(const u32x4_t*)(vt + o), df[ks], dp[t2]);
      }
    // register 8c + u of lane half H in tile t2 holds key n BN + 32 t2 + 16 c + 8 H + u.
    // A block whose 32 x BN pairs are all visible skips the mask.
    const int kb0 = n * BN;
    const bool full = q0w + 32 <= sq && kb0 + BN <= sk && (p.wr < 0 || kb0 + BN - 1 <= q0w + off + p.wr) &&
                      (p.wl < 0 || kb0 >= q0w + 31 + off - p.wl);
    u32x4_t sb[NT2][2];
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float sv[8], fv[8];
#pragma unroll
        for (int uu = 0; uu < 8; ++uu) probs<SOFTCAP>(s[t2][8 * c + uu], lse2, p, sv[uu], fv[uu]);
        if (!full) {
#pragma unroll
          for (int uu = 0; uu < 8; ++uu)
            if (!visible_key(qrow, kb0 + 32 * t2 + 16 * c + 8 * hsel + uu, sq, sk, off, p.wl, p.wr)) sv[uu] = 0.f;
        }
#pragma unroll
        for (int uu = 0; uu < 8; ++uu) {
          sv[uu] *= dp[t2][8 * c + uu] - drow;
          if constexpr (SOFTCAP) sv[uu] *= fv[uu];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sb[t2][c][e] = E::pack2(sv[2 * e], sv[2 * e + 1]);
      }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int rows = (32 * t2 + 16 * c) * (D * 2);
          const u32x2_t lo = lds_read_tr16(kt + tr[0][dt] + rows), hi = lds_read_tr16(kt + tr[1][dt] + rows);
          u32x4_t a;
          a[0] = lo[0], a[1] = lo[1], a[2] = hi[0], a[3] = hi[1];
          dq[dt] = E::mfma32x32x16(a, sb[t2][c], dq[dt]);
        }
  };

  uint8_t* const k0s = smem + grp * 4 * KTILE;
  uint8_t* const k1s = k0s + KTILE;
  uint8_t* const v0s = k0s + 2 * KTILE;
  uint8_t* const v1s = k0s + 3 * KTILE;
  auto step = [&](const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
                  uint8_t* __restrict__ kn, uint8_t* __restrict__ vn, int n) {
    if (n + NG < n_hi) issue(n + NG, kn, vn);
    block(n, kc, vc);
  };
  // The rows' statistics, (LSE log2 e, D_i): LSE -inf (a row without keys) becomes +inf, so
  // that exp2(s - lse2) = 0 everywhere.  The waves of group 0 store them for the dK/dV
  // kernel, which runs after this one.  Computed after the first K/V DMA is issued, so
  // that waiting for O does not delay it.
  auto row_stats = [&]() __attribute__((always_inline)) {
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(lo_f32<BF16>(of[ks][e]), lo_f32<BF16>(df[ks][e]), acc);
        acc = __builtin_fmaf(hi_f32<BF16>(of[ks][e]), hi_f32<BF16>(df[ks][e]), acc);
      }
    drow = acc + xor32(acc);  // the lane halves hold the two halves of the head dims
    lse2 = lse_in == kNegInf ? __builtin_inff() : lse_in * kLog2e;
    if (grp == 0 && hsel == 0 && qrow < sq) {
      f32x2_t st;
      st[0] = lse2, st[1] = drow;
      *(f32x2_t*)(p.ws_stats + 2 * (((int64_t)b * p.h_q + h) * sqm + qrow)) = st;
    }
  };
  if constexpr (NG == 1) {
    if (n_lo < n_hi) issue(n_lo, k0s, v0s);
    row_stats();
    for (int n = n_lo; n < n_hi; n += 2) {
      wait_vmem_all();
      __syncthreads();
      step(k0s, v0s, k1s, v1s, n);
      if (n + 1 < n_hi) {
        wait_vmem_all();
        __syncthreads();
        step(k1s, v1s, k0s, v0s, n + 1);
      }
    }
  } else {
    // both groups run the same number of iterations so that every wave meets every barrier
    const int iters = (n_hi - n_lo + NG - 1) / NG;
    const int nf = n_lo + grp;
    if (nf < n_hi) issue(nf, k0s, v0s);
    row_stats();
    for (int t = 0; t < iters; t += 2) {
      wait_vmem_all();
      __syncthreads();
      if (nf + NG * t < n_hi) step(k0s, v0s, k1s, v1s, nf + NG * t);
      if (t + 1 < iters) {
        wait_vmem_all();
        __syncthreads();
        if (nf + NG * (t + 1) < n_hi) step(k1s, v1s, k0s, v0s, nf + NG * (t + 1));
      }
    }
    // Every group finalizes: wave (group g, slice w) owns head-dim tiles
    // g HT .. (g + 1) HT - 1 of its 32 rows (HT = DT / NG).  It publishes the
    // other tiles through LDS (the stages are free once every wave has passed
    // the barrier), sums its own tiles over the groups in a fixed order (g0 + g1;
    // with 4 groups (g0 + g2) + (g1 + g3)), and rounds them into an LDS tile of
    // the 64 rows that all threads then store as whole rows (16 bytes per thread).
    static_assert(NG == 2 || NG == 4, "two or four groups");
    constexpr int HT = DT / NG;      // head-dim tiles per group
    constexpr int PT = DT - HT;      // tiles a wave publishes
    static_assert(HT >= 1, "a head-dim tile per group");
    constexpr int XQ = NG * NW * PT * 16 * 64 * 4;
    static_assert(XQ + kDqRows * D * 2 <= (int)sizeof(smem), "partials and the output tile");
    __syncthreads();
    float* const xq = reinterpret_cast<float*>(smem);  // [group][wave][published tile][j][lane][4]
    uint8_t* const otile = smem + XQ;                  // [64 rows][D] 16-bit, chunks swizzled
    auto xslot = [&](int g, int w, int t, int j) { return xq + ((((g * NW + w) * PT + t) * 4 + j) * 64 + lane) * 4; };
    // slot of tile dt among group g's published tiles
    auto pidx = [](int g, int dt) { return dt < g * HT ? dt : dt - HT; };
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      if (dt / HT != grp) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *(f32x4_t*)xslot(grp, wave, pidx(grp, dt), j) =
              f32x4_t{dq[dt][4 * j], dq[dt][4 * j + 1], dq[dt][4 * j + 2], dq[dt][4 * j + 3]};
      }
    __syncthreads();
    const int orow = 32 * wave + l32;  // this lane's row in the tile
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      if (dt / HT == grp) {
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          f32x4_t x[NG];  // group g's partial of registers 4 J .. 4 J + 3
#pragma unroll
          for (int g = 0; g < NG; ++g)
            x[g] = g == grp ? f32x4_t{dq[dt][4 * J], dq[dt][4 * J + 1], dq[dt][4 * J + 2], dq[dt][4 * J + 3]}
                            : *(const f32x4_t*)xslot(g, wave, pidx(g, dt), J);
          f32x4_t r;
          if constexpr (NG == 2)
            r = x[0] + x[1];
          else
            r = (x[0] + x[2]) + (x[1] + x[3]);
          u32x2_t w;  // head dims 32 dt + 8 J + 4 hsel + 0..3
          w[0] = E::pack2(r[0] * p.scale, r[1] * p.scale);
          w[1] = E::pack2(r[2] * p.scale, r[3] * p.scale);
          const int chunk = 4 * dt + J;
          *(u32x2_t*)(otile + orow * (D * 2) + 16 * (chunk ^ qswz<D>(orow)) + 8 * hsel) = w;
        }
      }
    __syncthreads();
    constexpr int NTH = 64 * NW * NG;
    static_assert(kDqRows * DCH % NTH == 0, "output tile copy");
#pragma unroll
    for (int it = 0; it < kDqRows * DCH / NTH; ++it) {
      const int idx = it * NTH + tid;
      const int row = idx / DCH, chunk = idx % DCH;
      if (q0 + row < sq) {
        const u32x4_t val = *(const u32x4_t*)(otile + row * (D * 2) + 16 * (chunk ^ qswz<D>(row)));
        *(u32x4_t*)(p.dq + sp.dq + (int64_t)(q0 + row) * p.dq_ss + (int64_t)h * p.dq_sh + 8 * chunk) = val;
      }
    }
    return;
  }
  // ---- dQ = scale (dQ^T)^T: lane holds head dims 32 dt + 8 J + 4 H + 0..3 of row qrow.
  if (qrow < sq) {
    uint16_t* op = p.dq + sp.dq + (int64_t)qrow * p.dq_ss + (int64_t)h * p.dq_sh;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        u32x2_t wq;
        wq[0] = E::pack2(dq[dt][4 * J] * p.scale, dq[dt][4 * J + 1] * p.scale);
        wq[1] = E::pack2(dq[dt][4 * J + 2] * p.scale, dq[dt][4 * J + 3] * p.scale);
        *(u32x2_t*)(op + 32 * dt + 8 * J + 4 * hsel) = wq;
      }
  }
}

template <bool BF16, int D, bool SOFTCAP>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
  // The dQ kernel runs first: it also writes every query row's statistics
  // (LSE log2 e, dO . O), which the dK/dV kernel reads.  A kernel whose grid
  // would be empty is skipped: with no query rows dK and dV are zero (the dK/dV
  // kernel sees no query block), with no keys dQ is zero (the dQ kernel sees no
  // key block).
  hipError_t e = hipSuccess;
  const int n_qt = (p.s_q + kDqRows - 1) / kDqRows;
  if (n_qt > 0) {
    const int grid = n_qt * p.h_q * p.batch;
    // Fewer than 1024 tiles leave under two waves per SIMD on 256 CUs: split each
    // tile's key blocks between two wave groups then.  At d = 256 the one-group
    // kernel's 64-key blocks need more registers than a wave has: two groups of
    // 32-key blocks always.
    bool two = true;
    if constexpr (D != 256) two = grid < 1024;
    if (two) {
      hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, 2, SOFTCAP>), dim3(grid), dim3(64 * kDqWaves * 2), 0, stream, p);
    } else {
      if constexpr (D != 256)
        hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, 1, SOFTCAP>), dim3(grid), dim3(64 * kDqWaves), 0, stream, p);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int n_kt = (p.s_k + kBwdKeys - 1) / kBwdKeys;
  if (n_kt > 0) {
    // d = 128: the 8-wave kernel (measured 13-18% faster over the whole backward
    // at the causal training shape and longer sequences); d = 64: the 4-wave one,
    // whose work groups already share a CU two at a time (the 8-wave kernel
    // measured 6% slower there); d = 256: the 4-wave one in two head-dim slices.
    // At d = 128 a mask bounded on one side only (causal, or one window edge)
    // makes the key tiles' work uneven: 64-key tiles in 4 sets then (whole
    // backward 10-18% faster at causal shapes); otherwise 128-key tiles in 2
    // sets, which read each Q / dO block for twice the keys (the 64-key tiles
    // measured 7% slower without a mask).
    if constexpr (D == 256)
      hipLaunchKernelGGL((bwd_dkdv_kernel<BF16, D, SOFTCAP, 2>), dim3(n_kt * p.h_kv * p.batch * 2), dim3(256), 0,
                         stream, p);
    else if constexpr (D == 128) {
      if ((p.wr >= 0) != (p.wl >= 0))
        hipLaunchKernelGGL((bwd_dkdv2_kernel<BF16, D, SOFTCAP, 4>), dim3(((p.s_k + 63) / 64) * p.h_kv * p.batch),
                           dim3(512), 0, stream, p);
      else
        hipLaunchKernelGGL((bwd_dkdv2_kernel<BF16, D, SOFTCAP, 2>), dim3(n_kt * p.h_kv * p.batch), dim3(512), 0,
                           stream, p);
    }
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<BF16, D, SOFTCAP, 1>), dim3(n_kt * p.h_kv * p.batch), dim3(256), 0,
                         stream, p);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

template <int D, bool SOFTCAP>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
  return p.bf16 ? launch_bwd_t<true, D, SOFTCAP>(p, stream) : launch_bwd_t<false, D, SOFTCAP>(p, stream);
}

hipError_t launch_bwd(const BwdParams& p, int head_dim, bool softcap, hipStream_t stream) {
  if (head_dim == 64) return softcap ? launch_bwd_d<64, true>(p, stream) : launch_bwd_d<64, false>(p, stream);
  if (head_dim == 128) return softcap ? launch_bwd_d<128, true>(p, stream) : launch_bwd_d<128, false>(p, stream);
  if (head_dim == 256) return softcap ? launch_bwd_d<256, true>(p, stream) : launch_bwd_d<256, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace exattn
