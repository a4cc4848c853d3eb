// FP8 forward of exact attention with a bf16 output (Inference Cookbook FAQ
// Q20: FP8 inside, BF16 out, since the normalised result and the V descale
// need more precision than FP8 holds; FAQ Q10 gives FP8 a 1e-2 tolerance).
//
// Inputs Q, K, V are OCP FP8 E4M3 codes with one fp32 descale factor each:
// the real value is code x descale.  S = scale q_descale k_descale (Q K^T) is
// formed on the FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales:
// exact products, sums a little shorter than fp32), the softmax runs in fp32
// with a running max and sum as in the bf16 forward ("FlashAttention完整说明",
// section 二.1), and O = P V takes P rounded to bf16 against V widened exactly
// from FP8 to bf16 in registers (every E4M3 value is a bf16 value).  Rounding
// P to E4M3 instead (3 mantissa bits) would move rows that see few keys by
// several percent, beyond the tolerance.  O is scaled by v_descale / l and
// written as bf16; LSE is the natural log of the sum of exp over the row's
// final scores.
//
// Layout per work group: NW waves x 32 query rows of one query head; a wave's
// lane owns one query row (S^T = K Q^T, Q^T the B operand from registers).
// With NG = 2 a second group of NW waves takes every other key block of the
// same rows, and the groups' (max, sum, O) merge through LDS at the end.  With
// one group (large grids) and no softcap the loop is software-pipelined: the
// QK MFMAs of a block are interleaved with the exponentials of the block
// before, against a lazy reference max.
// Key blocks of 64 rows stream by DMA into double-buffered LDS as FP8.  K is
// read as A operands; V is read with the 8-bit transposing read, whose lane i
// receives byte i % 8 of 8 rows (the rows of source lanes 2 e + i / 8 of its
// 16-lane group), and widened to bf16 in registers as the PV A operand.
#include "device_common.h"
#include "kernels.h"
#include "tiles.h"

namespace exattn {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

constexpr int kF8Keys = 64;  // keys per block

// FP8 K tile (rows of D bytes): 16-byte chunk c of row r at c ^ f8swz(r).  An
// A-operand read takes 16 bytes of 16 rows at one chunk; with 128-byte rows
// (d = 128) two rows share a 256-byte bank row, so rows of one parity need 8
// distinct positions; with 64-byte rows four rows share one, so 4.
template <int D>
__device__ __forceinline__ int f8swz(int r) {
  if constexpr (D == 128)
    return (r >> 1) & 7;
  else
    return (r >> 2) & 3;
}

// FP8 V tile (rows of D bytes), read by 8-bit transposing reads: the 32 lanes
// served together read 8 consecutive rows x 2 adjacent 16-byte chunks (c, c+1,
// c even).  Chunk c of row r sits at c ^ v8swz(r): rows of one parity (d = 128,
// two rows per 256-byte bank row) or of one residue mod 4 (d = 64) differ in
// bits 1-2 of the swizzle, so the 16 chunks land in 16 bank groups.
template <int D>
__device__ __forceinline__ int v8swz(int r) {
  if constexpr (D == 128)
    return 2 * ((r >> 1) & 3);
  else
    return 2 * ((r >> 2) & 1);
}

__device__ __forceinline__ bool f8_visible(int i, int j, int sk, int off, int wl, int wr) {
  return j < sk && (wr < 0 || j <= i + off + wr) && (wl < 0 || j >= i + off - wl);
}

// Buffer descriptor over `bytes` bytes from base: loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bytes_rsrc(const uint8_t* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
}

// Two FP8 E4M3 codes (bytes 0-1 or 2-3 of w) as two bf16 in one word (exact).
template <bool HI>
__device__ __forceinline__ uint32_t f8pair_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// 8 bytes of one 16-lane group's transposing read of the FP8 V tile (see the
// file comment for which bytes each lane receives).
__device__ __forceinline__ u32x2_t lds_read_tr8(const uint8_t* p) {
  return __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)(p)));
}

constexpr float kLazyTau = 8.0f;   // the pipelined loop moves a row's reference only when its max grows by > 2^8
constexpr float kSumCap = 256.0f;  // 2^tau: a lane's block sum below it means every p <= 2^tau

template <int D, int NW, int NG, bool SOFTCAP, bool PIPE>
__global__ void __launch_bounds__(64 * NW * NG) fp8_prefill_kernel(const Fp8Params p) {
  constexpr int BN = kF8Keys;
  constexpr int NT2 = BN / 32;       // 32-key tiles per block
  constexpr int KS = D / 64;         // 64-wide k-steps over head_dim (QK)
  constexpr int DT = D / 32;         // 32-wide head_dim tiles of O^T
  constexpr int F8TILE = BN * D;     // bytes of an FP8 K or V tile
  constexpr int STAGE = 2 * F8TILE;  // K and V
  constexpr int SLICES = F8TILE / 1024;
  static_assert(SLICES % NW == 0, "DMA slices per wave");
  constexpr int ROWS_PER_KB = 1024 / D;
  constexpr int CH = D / 16;         // 16-byte chunks per FP8 row
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NG * 2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wv / NW;   // key-block group: blocks n_lo + grp, + NG, ...
  const int wave = wv % NW;  // row slice of the tile
  const int hsel = lane >> 5;
  const int l32 = lane & 31;

  const int rows_wg = 32 * NW;
  const int n_qt = (p.s_q + rows_wg - 1) / rows_wg;
  const int units = p.batch * p.h_q;
  // Tiles heaviest (last) first.  With two groups under a one-sided mask (causal),
  // where the whole grid is resident at once (two work groups per CU), the second
  // half of the grid runs lightest first instead: work groups i and i + grid/2 tend to
  // share a CU, and then carry a heavy and a light tile (measured 22.2 -> 21.4 us at
  // causal b2 s1024 h16 d128, -3% at b4 s1024 h8).
  int qt;
  {
    const int kq = (int)blockIdx.x / units;
    const int half = (n_qt + 1) / 2;
    if (NG == 2 && (p.wr >= 0) != (p.wl >= 0))
      qt = kq < half ? n_qt - 1 - kq : kq - half;
    else
      qt = n_qt - 1 - kq;
  }
  const int u = blockIdx.x % units;
  const int b = u / p.h_q, h = u % p.h_q;
  const int hk = h / p.group;
  // a batch entry's rows: from the batch strides, or (varlen, FAQ Q8) the token
  // span cu[b] .. cu[b + 1] - 1 of the packed tensors
  int sq = p.s_q, sk = p.s_k;
  int64_t qoff, koff, voff, ooff, lseoff;
  if (p.cu_q != nullptr) {
    const int qs = p.cu_q[b], ks = p.cu_k[b];
    sq = p.cu_q[b + 1] - qs;
    sk = p.cu_k[b + 1] - ks;
    qoff = (int64_t)qs * p.q_ss;
    koff = (int64_t)ks * p.k_ss;
    voff = (int64_t)ks * p.v_ss;
    ooff = (int64_t)qs * p.o_ss;
    lseoff = qs;
  } else {
    qoff = (int64_t)b * p.q_sb;
    koff = (int64_t)b * p.k_sb;
    voff = (int64_t)b * p.v_sb;
    ooff = (int64_t)b * p.o_sb;
    lseoff = (int64_t)b * p.lse_sb;
  }
  const int off = sk - sq;
  const int q0 = qt * rows_wg;
  if (q0 >= sq) return;  // uniform: a shorter sequence has no rows here
  const int q0w = q0 + 32 * wave;
  const int qrow = q0w + l32;

  // ---- key blocks any row of the tile sees.
  const int t1 = min(q0 + rows_wg, sq) - 1;
  int kmin = 0, kmax = sk - 1;
  if (p.wl >= 0) kmin = max(0, q0 + off - p.wl);
  if (p.wr >= 0) kmax = min(kmax, t1 + off + p.wr);
  const int n_lo = kmax >= kmin ? kmin / BN : 0;
  const int n_hi = kmax >= kmin ? kmax / BN + 1 : 0;

  // ---- Q^T as B operand of the 64-wide k-steps: lane half H of step s holds head
  // dims 64 s + 32 H .. + 31 (32 bytes); K's A operands use the same assignment,
  // so every dim meets itself.
  i32x8_t qf[KS];
  {
    const bool in = qrow < sq;
    const uint8_t* qp = p.q + qoff + (int64_t)qrow * p.q_ss + (int64_t)h * p.q_sh + 32 * hsel;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t lo = in ? *(const u32x4_t*)(qp + 64 * ks) : u32x4_t{0, 0, 0, 0};
      const u32x4_t hi = in ? *(const u32x4_t*)(qp + 64 * ks + 16) : u32x4_t{0, 0, 0, 0};
      qf[ks] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  }

  // ---- DMA of the FP8 K and V tiles: row r, chunk c at r * D + 16 * (c ^ swz(r)).
  const uint8_t* kg = p.k + koff + (int64_t)hk * p.k_sh;
  const uint8_t* vg = p.v + voff + (int64_t)hk * p.v_sh;
  uint32_t kofs[SLICES / NW], vofs[SLICES / NW];
#pragma unroll
  for (int i = 0; i < SLICES / NW; ++i) {
    const int row = (NW * i + wave) * ROWS_PER_KB + lane / CH;
    kofs[i] = (uint32_t)(row * p.k_ss + 16 * ((lane % CH) ^ f8swz<D>(row)));
    vofs[i] = (uint32_t)(row * p.v_ss + 16 * ((lane % CH) ^ v8swz<D>(row)));
  }
  auto issue = [&](int n, uint8_t* dst) {
    const int kb = n * BN;
    const int64_t lastk = (int64_t)min(sk - 1 - kb, BN - 1) * p.k_ss + D;
    const int64_t lastv = (int64_t)min(sk - 1 - kb, BN - 1) * p.v_ss + D;
    const __amdgpu_buffer_rsrc_t rk = bytes_rsrc(kg + (int64_t)kb * p.k_ss, lastk);
    const __amdgpu_buffer_rsrc_t rv = bytes_rsrc(vg + (int64_t)kb * p.v_ss, lastv);
#pragma unroll
    for (int i = 0; i < SLICES / NW; ++i) {
      buffer_load_lds16(rk, dst + (NW * i + wave) * 1024, kofs[i]);
      buffer_load_lds16(rv, dst + F8TILE + (NW * i + wave) * 1024, vofs[i]);
    }
  };

  // ---- LDS addresses.  K A operand of tile t2, step s: row m = l32 is key
  // 32 t2 + row_key(l32), bytes 64 s + 32 H .. + 31 = chunks 4 s + 2 H, + 1.
  const int krow = row_key(l32);
  int kaddr[KS][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 2; ++e) kaddr[ks][e] = krow * D + 16 * ((4 * ks + 2 * hsel + e) ^ f8swz<D>(krow));
  // V^T operand of O^T += V^T P^T for dim tile dt and 16 keys: group g = lane / 16
  // covers dims 32 dt + 16 (g & 1) .. + 15 and keys 8 (g >> 1) .. + 7; as a source
  // lane, lane i of the group reads key 8 (g >> 1) + i / 2, dims + 8 (i & 1) .. + 7.
  const int gi = lane >> 4, li = lane & 15;
  const int vrow = 8 * (gi >> 1) + (li >> 1);
  int vaddr[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    vaddr[dt] = vrow * D + 16 * ((2 * dt + (gi & 1)) ^ v8swz<D>(vrow)) + 8 * (li & 1);

  float m = -__builtin_inff(), l = 0.f;  // running max (log2 domain) and sum
  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16_t{};

  auto block = [&](int n, const uint8_t* __restrict__ kt, const uint8_t* __restrict__ vt,
                   uint8_t* __restrict__ nxt) {
    // S^T = K Q^T on the FP8 MFMA (unit block scales: E8M0 127)
    f32x16_t s[NT2];
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2) s[t2] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int t2 = 0; t2 < NT2; ++t2) {
        const u32x4_t lo = *(const u32x4_t*)(kt + kaddr[ks][0] + t2 * 32 * D);
        const u32x4_t hi = *(const u32x4_t*)(kt + kaddr[ks][1] + t2 * 32 * D);
        const i32x8_t a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        s[t2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[ks], s[t2], 0, 0, 0, 127, 0, 127);
      }
    if (n + NG < n_hi) issue(n + NG, nxt);
    // the V reads do not depend on P: issue them all now, under the softmax
    u32x2_t vw[NT2][2][DT];
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vw[t2][c][dt] = lds_read_tr8(vt + vaddr[dt] + (32 * t2 + 16 * c) * D);
    // scores in the log2 domain; register 8c + u of tile t2 is key n BN + 32 t2 + 16 c + 8 H + u
    const int kb0 = n * BN;
    const bool full = q0w + 32 <= sq && kb0 + BN <= sk && (p.wr < 0 || kb0 + BN - 1 <= q0w + off + p.wr) &&
                      (p.wl < 0 || kb0 >= q0w + 31 + off - p.wl);
    float mx = -__builtin_inff();
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x;
        if constexpr (SOFTCAP)  // c tanh(s / c) before the mask (FAQ Q22), in the log2 domain
          x = p.cap_out_log2 * tanh_exp2(s[t2][r] * p.cap_in);
        else
          x = s[t2][r] * p.scale_log2;
        if (!full) {
          const int key = kb0 + 32 * t2 + 16 * (r >> 3) + 8 * hsel + (r & 7);
          if (!f8_visible(qrow, key, sk, off, p.wl, p.wr)) x = -__builtin_inff();
        }
        s[t2][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = halves_max(mx);
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;  // rows that see nothing yet
    const float alpha = fast_exp2(m - m_use);
    m = m_new;
    float rs = 0.f;
    u32x4_t pb[NT2][2];
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float pv[8];
#pragma unroll
        for (int uu = 0; uu < 8; ++uu) {
          pv[uu] = fast_exp2(s[t2][8 * c + uu] - m_use);
          rs += pv[uu];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) pb[t2][c][e] = Elem<true>::pack2(pv[2 * e], pv[2 * e + 1]);
      }
    l = l * alpha + halves_sum(rs);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {  // the running max grew for some row
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    // O^T += V^T P^T, V^T widened from FP8 in registers
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const u32x2_t w = vw[t2][c][dt];
          u32x4_t a;
          a[0] = f8pair_bf16<false>(w[0]), a[1] = f8pair_bf16<true>(w[0]);
          a[2] = f8pair_bf16<false>(w[1]), a[3] = f8pair_bf16<true>(w[1]);
          o[dt] = Elem<true>::mfma32x32x16(a, pb[t2][c], o[dt]);
        }
  };

  // Group grp takes blocks n_lo + grp, + NG, ...; both groups run the same number
  // of iterations so that every wave meets every barrier.
  uint8_t* const s0 = smem + grp * 2 * STAGE;
  uint8_t* const s1 = s0 + STAGE;
  if constexpr (PIPE) {
    // ---- software-pipelined loop (one group, no softcap, scale != 0): step i
    // computes S(b_i) = K(b_i) Q^T with the exponentials of S(b_{i-1})
    // interleaved between its MFMAs, then the check, the softmax fix-up if
    // needed and O += P V of b_{i-1}.  The exponentials use a lazy reference
    // m_ref (moved only when a block's max exceeds it by more than 2^8, so O and
    // the sum always share one reference), which needs no block max up front.
    // K(b_i) and V(b_i) live in stage i & 1; step i loads K(b_{i+1}) and V(b_i)
    // (their stage parts were last read in step i - 1).  Scores stay raw until
    // the exponentials, exp2(s scale - m_ref) being one FMA and one exp; a
    // masked score is set to -inf x sign(scale), which the FMA turns into -inf.
    static_assert(NG == 1 && !SOFTCAP, "pipelined loop: one group, no softcap");
    constexpr int NA = KS * NT2;        // FP8 MFMAs of S^T = K Q^T per block
    constexpr int EPM = 16 * NT2 / NA;  // exponentials per such MFMA
    static_assert(EPM >= 2 && EPM % 2 == 0, "exponential pairs per MFMA");
    const float mval = p.scale_log2 > 0.f ? -__builtin_inff() : __builtin_inff();
    const int nb = n_hi - n_lo;
    float m_ref = -__builtin_inff();  // reference (log2 domain) of this lane's row
    float l_run = 0.f;                // this lane's share of the row sum against m_ref
    auto exps = [&](const f32x16_t (&sc)[NT2], u32x4_t (&pf)[NT2][2], float base) {
      float psum = 0.f;
#pragma unroll
      for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float x0 = fast_exp2(__builtin_fmaf(sc[t2][r], p.scale_log2, -base));
          const float x1 = fast_exp2(__builtin_fmaf(sc[t2][r + 1], p.scale_log2, -base));
          pf[t2][r >> 3][(r & 7) >> 1] = Elem<true>::pack2(x0, x1);
          psum += x0 + x1;
        }
      return psum;
    };
    // the block's max exceeds the reference by more than 2^8 for some row, or
    // the reference is unset: move it (rescaling O and the sum) and redo the
    // exponentials
    auto slow = [&](const f32x16_t (&sc)[NT2], u32x4_t (&pf)[NT2][2]) {
      float mb = -__builtin_inff();
#pragma unroll
      for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
        for (int r = 0; r < 16; ++r) mb = fmaxf(mb, sc[t2][r] * p.scale_log2);
      mb = halves_max(mb);
      const bool need = mb > m_ref + kLazyTau;
      const float m_new = need ? mb : m_ref;
      const float alpha = need ? fast_exp2(m_ref - m_new) : 1.f;  // 0 when m_ref = -inf
      if (__builtin_amdgcn_ballot_w64(need && m_ref != -__builtin_inff()) != 0) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      }
      l_run *= alpha;
      m_ref = m_new;
      return exps(sc, pf, m_ref == -__builtin_inff() ? 0.f : m_ref);
    };
    // S(b_i) into sn from K stage kc, interleaved with the exponentials of sc =
    // S(b_{i-1}); then (ap) its check and O += P V from V stage vp
    auto fused = [&](const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vp, const f32x16_t (&sc)[NT2],
                     f32x16_t (&sn)[NT2], bool ap) {
      // K(b_i) operands first, then V(b_{i-1}) (needed only after the
      // exponentials): LDS reads complete in order
      i32x8_t ka[KS][NT2];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int t2 = 0; t2 < NT2; ++t2) {
          const u32x4_t lo = *(const u32x4_t*)(kc + kaddr[ks][0] + t2 * 32 * D);
          const u32x4_t hi = *(const u32x4_t*)(kc + kaddr[ks][1] + t2 * 32 * D);
          ka[ks][t2] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
      u32x2_t vw[NT2][2][DT];
#pragma unroll
      for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) vw[t2][c][dt] = lds_read_tr8(vp + vaddr[dt] + (32 * t2 + 16 * c) * D);
      u32x4_t pf[NT2][2];
      float psum = 0.f;
      const float base = m_ref;
#pragma unroll
      for (int t2 = 0; t2 < NT2; ++t2) sn[t2] = f32x16_t{};
      // one MFMA, then its share of the exponentials, in this order: a wave
      // issues its exponentials while its MFMAs run (the scheduling barriers
      // keep the compiler from regrouping them)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int t2 = 0; t2 < NT2; ++t2) {
          const int mi = ks * NT2 + t2;
          __builtin_amdgcn_sched_barrier(0);
          sn[t2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka[ks][t2], qf[ks], sn[t2], 0, 0, 0, 127, 0, 127);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < EPM; u += 2) {
            const int e = mi * EPM + u, t = e >> 4, r = e & 15;
            const float x0 = fast_exp2(__builtin_fmaf(sc[t][r], p.scale_log2, -base));
            const float x1 = fast_exp2(__builtin_fmaf(sc[t][r + 1], p.scale_log2, -base));
            pf[t][r >> 3][(r & 7) >> 1] = Elem<true>::pack2(x0, x1);
            psum += x0 + x1;
          }
        }
      __builtin_amdgcn_sched_barrier(0);
      // consume the exponentials and the scores here: LLVM would otherwise sink
      // the exponentials below the branch that follows and the score MFMAs
      // below the PV products, out of one instruction stream
#pragma unroll
      for (int t = 0; t < NT2; ++t) asm volatile("" ::"v"(pf[t][0]), "v"(pf[t][1]));
      asm volatile("" ::"v"(psum));
#pragma unroll
      for (int t2 = 0; t2 < NT2; ++t2) asm volatile("" ::"v"(sn[t2][0]));  // one word waits for the MFMA
      if (ap) {
        if (__builtin_amdgcn_ballot_w64(!(psum <= kSumCap)) != 0) psum = slow(sc, pf);  // also inf, NaN
        l_run += psum;
#pragma unroll
        for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              const u32x2_t w = vw[t2][c][dt];
              u32x4_t av;
              av[0] = f8pair_bf16<false>(w[0]), av[1] = f8pair_bf16<true>(w[0]);
              av[2] = f8pair_bf16<false>(w[1]), av[3] = f8pair_bf16<true>(w[1]);
              o[dt] = Elem<true>::mfma32x32x16(av, pf[t2][c], o[dt]);
            }
      }
    };
    auto issue_k = [&](int n, uint8_t* dst) {
      const int kb = n * BN;
      const int64_t lastk = (int64_t)min(sk - 1 - kb, BN - 1) * p.k_ss + D;
      const __amdgpu_buffer_rsrc_t rk = bytes_rsrc(kg + (int64_t)kb * p.k_ss, lastk);
#pragma unroll
      for (int i = 0; i < SLICES / NW; ++i) buffer_load_lds16(rk, dst + (NW * i + wave) * 1024, kofs[i]);
    };
    auto issue_v = [&](int n, uint8_t* dst) {
      const int kb = n * BN;
      const int64_t lastv = (int64_t)min(sk - 1 - kb, BN - 1) * p.v_ss + D;
      const __amdgpu_buffer_rsrc_t rv = bytes_rsrc(vg + (int64_t)kb * p.v_ss, lastv);
#pragma unroll
      for (int i = 0; i < SLICES / NW; ++i) buffer_load_lds16(rv, dst + F8TILE + (NW * i + wave) * 1024, vofs[i]);
    };
    // step i: kc = the stage of b_i (K read, V(b_i) loaded into it), vp = the
    // stage of b_{i-1} (V read); the other stage takes K(b_{i+1})
    auto step = [&](uint8_t* __restrict__ kc, uint8_t* __restrict__ vp, int i, const f32x16_t (&sc)[NT2],
                    f32x16_t (&sn)[NT2]) {
      uint8_t* const kn = kc == s0 ? s1 : s0;
      if (i + 1 < nb) issue_k(n_lo + i + 1, kn);
      if (i < nb) issue_v(n_lo + i, kc);
      // A wave's first step still runs the exponentials, on stale registers, and
      // its last runs S = K Q^T on a stale stage: both results are discarded.
      fused(kc, vp + F8TILE, sc, sn, i > 0);
      if (i < nb) {
        const int kb0 = (n_lo + i) * BN;
        const bool full = q0w + 32 <= sq && kb0 + BN <= sk && (p.wr < 0 || kb0 + BN - 1 <= q0w + off + p.wr) &&
                          (p.wl < 0 || kb0 >= q0w + 31 + off - p.wl);
        if (!full) {
#pragma unroll
          for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kb0 + 32 * t2 + 16 * (r >> 3) + 8 * hsel + (r & 7);
              if (!f8_visible(qrow, key, sk, off, p.wl, p.wr)) sn[t2][r] = mval;
            }
        }
      }
    };
    // consume Q before the loop (one word of each 16-byte load), so that the
    // compiler waits for those loads once instead of inside the steps
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks][0]), "v"(qf[ks][4]));
    f32x16_t sa[NT2], sb[NT2];
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2) sa[t2] = sb[t2] = f32x16_t{};
    if (nb > 0) issue_k(n_lo, s0);
    // Unrolled by two so each call sees fixed stages and score registers.
    // Before each step: K(b_i) and V(b_{i-1}) have landed, and every wave is
    // done with the previous step.
    int i = 0;
    for (; i + 1 <= nb; i += 2) {
      wait_vmem_all();
      __syncthreads();
      step(s0, s1, i, sb, sa);
      wait_vmem_all();
      __syncthreads();
      step(s1, s0, i + 1, sa, sb);
    }
    if (i <= nb) {
      wait_vmem_all();
      __syncthreads();
      step(s0, s1, i, sb, sa);
    }
    m = m_ref;
    l = halves_sum(l_run);
  } else if constexpr (NG == 1) {
    if (n_lo < n_hi) issue(n_lo, s0);
    for (int n = n_lo; n < n_hi; n += 2) {
      wait_vmem_all();
      __syncthreads();
      block(n, s0, s0 + F8TILE, s1);
      if (n + 1 < n_hi) {
        wait_vmem_all();
        __syncthreads();
        block(n + 1, s1, s1 + F8TILE, s0);
      }
    }
  } else {
    const int iters = (n_hi - n_lo + NG - 1) / NG;
    const int nf = n_lo + grp;  // this group's first block
    if (nf < n_hi) issue(nf, s0);
    for (int t = 0; t < iters; t += 2) {
      wait_vmem_all();
      __syncthreads();
      if (nf + NG * t < n_hi) block(nf + NG * t, s0, s0 + F8TILE, s1);
      if (t + 1 < iters) {
        wait_vmem_all();
        __syncthreads();
        if (nf + NG * (t + 1) < n_hi) block(nf + NG * (t + 1), s1, s1 + F8TILE, s0);
      }
    }
  }

  // ---- merge the groups: group g > 0 hands (m, l, O^T) to group 0 through LDS
  // (the stages are free once every wave has passed this barrier).
  if constexpr (NG > 1) {
    static_assert(NG == 2, "two groups");
    __syncthreads();
    float* xo = reinterpret_cast<float*>(smem);                       // [wave][dt][4][lane][4]
    float* xm = reinterpret_cast<float*>(smem) + NW * DT * 16 * 64;   // [wave][lane] m, then l
    if (grp == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4_t w = {o[dt][4 * j], o[dt][4 * j + 1], o[dt][4 * j + 2], o[dt][4 * j + 3]};
          *(f32x4_t*)(xo + (((wave * DT + dt) * 4 + j) * 64 + lane) * 4) = w;
        }
      xm[wave * 64 + lane] = m;
      xm[NW * 64 + wave * 64 + lane] = l;
    }
    __syncthreads();
    if (grp != 0) return;
    const float m1 = xm[wave * 64 + lane], l1 = xm[NW * 64 + wave * 64 + lane];
    const float mt = fmaxf(m, m1);
    const float mu = mt == -__builtin_inff() ? 0.f : mt;
    const float a0 = fast_exp2(m - mu), a1 = fast_exp2(m1 - mu);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4_t w = *(const f32x4_t*)(xo + (((wave * DT + dt) * 4 + j) * 64 + lane) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[dt][4 * j + e] = o[dt][4 * j + e] * a0 + w[e] * a1;
      }
    l = l * a0 + l1 * a1;
    m = mt;
  }

  // ---- O = (O^T)^T v_descale / l as bf16; lane holds head dims 32 dt + 8 J + 4 H + 0..3 of row qrow.
  if (qrow < sq) {
    const float inv = l > 0.f ? p.v_descale / l : 0.f;
    uint16_t* op = p.o + ooff + (int64_t)qrow * p.o_ss + (int64_t)h * p.o_sh;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        u32x2_t w;
        w[0] = Elem<true>::pack2(o[dt][4 * J] * inv, o[dt][4 * J + 1] * inv);
        w[1] = Elem<true>::pack2(o[dt][4 * J + 2] * inv, o[dt][4 * J + 3] * inv);
        *(u32x2_t*)(op + 32 * dt + 8 * J + 4 * hsel) = w;
      }
    if (hsel == 0 && p.lse != nullptr)
      p.lse[lseoff + (int64_t)h * p.lse_sh + qrow] =
          l > 0.f ? (m + fast_log2(l)) * kLn2 : kNegInf;
  }
}

template <int D, bool SOFTCAP>
hipError_t launch_fp8_t(const Fp8Params& p, hipStream_t stream) {
  constexpr int NW = 2;
  const int n_qt = (p.s_q + 32 * NW - 1) / (32 * NW);
  if (n_qt == 0 || p.batch == 0) return hipSuccess;
  const int64_t grid = (int64_t)n_qt * p.h_q * p.batch;
  // Fewer than 1024 tiles leave under two waves per SIMD on 256 CUs: split each
  // tile's keys across two wave groups then (measured 21.9 us against 27.9 at the
  // causal b2 s1024 h16 d128 shape); with more tiles the split only adds the merge
  // (1114 us against 1032 at s16384).
  if (grid < 1024)
    hipLaunchKernelGGL((fp8_prefill_kernel<D, NW, 2, SOFTCAP, false>), dim3((unsigned)grid), dim3(64 * NW * 2), 0,
                       stream, p);
  else if (!SOFTCAP && p.scale_log2 != 0.f)
    hipLaunchKernelGGL((fp8_prefill_kernel<D, NW, 1, false, true>), dim3((unsigned)grid), dim3(64 * NW), 0, stream, p);
  else
    hipLaunchKernelGGL((fp8_prefill_kernel<D, NW, 1, SOFTCAP, false>), dim3((unsigned)grid), dim3(64 * NW), 0, stream,
                       p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Params& p, int head_dim, bool softcap, hipStream_t stream) {
  if (head_dim == 64) return softcap ? launch_fp8_t<64, true>(p, stream) : launch_fp8_t<64, false>(p, stream);
  if (head_dim == 128) return softcap ? launch_fp8_t<128, true>(p, stream) : launch_fp8_t<128, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace exattn
