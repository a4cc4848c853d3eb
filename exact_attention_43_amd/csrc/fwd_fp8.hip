// FP8 forward of exact attention with a bf16 output (Inference Cookbook FAQ
// Q20: FP8 inside, BF16 out, since the normalised result and the V descale
// need more precision than FP8 holds; FAQ Q10 gives FP8 a 1e-2 tolerance).
//
// Inputs Q, K, V are OCP FP8 E4M3 codes with one fp32 descale factor each:
// the real value is code x descale.  S = scale q_descale k_descale (Q K^T) is
// formed on the FP8 MFMA (v_mfma_f32_32x32x16_fp8_fp8: exact products, fp32
// sums), the softmax runs in fp32 with a running max and sum as in the bf16
// forward ("FlashAttention完整说明", section 二.1), and O = P V takes P rounded
// to bf16 against V widened exactly from FP8 to bf16 in LDS (every E4M3 value
// is a bf16 value).  Rounding P to E4M3 instead (3 mantissa bits) would move
// rows that see few keys by several percent, beyond the tolerance.  O is
// scaled by v_descale / l and written as bf16; LSE is the natural log of the
// sum of exp over the row's final scores.
//
// Layout per work group: NW waves x 32 query rows of one query head; a wave's
// lane owns one query row (S^T = K Q^T, Q^T the B operand from registers).
// Key blocks of 64 rows stream by DMA into double-buffered LDS: K as FP8
// (read as A operands), V as FP8 staging, widened by all waves into one bf16
// tile that the PV products read transposed.
#include "device_common.h"
#include "kernels.h"
#include "tiles.h"

namespace exattn {
namespace {

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

// bf16 V tile (rows of 2 D bytes), read only transposed by the PV products
// (4 consecutive rows x 2-4 adjacent chunks per read):
// chunk c of row r at c ^ vswz16(r), 4 consecutive rows differing in bits 2-3
// (d = 128) or bit 2 within a parity (d = 64).
template <int D>
__device__ __forceinline__ int vswz16(int r) {
  if constexpr (D == 64)
    return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  else
    return 4 * (r & 3) + ((r >> 2) & 3);
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

template <int D, int NW>
__global__ void __launch_bounds__(64 * NW) fp8_prefill_kernel(const Fp8Params p) {
  constexpr int BN = kF8Keys;
  constexpr int NT2 = BN / 32;       // 32-key tiles per block
  constexpr int KP = D / 32;         // pairs of 16-wide k-steps over head_dim
  constexpr int DT = D / 32;         // 32-wide head_dim tiles of O^T
  constexpr int F8TILE = BN * D;     // bytes of an FP8 K or V tile
  constexpr int VTILE = BN * D * 2;  // bytes of the bf16 V tile
  constexpr int STAGE = 2 * F8TILE;  // K and V (FP8)
  constexpr int SLICES = F8TILE / 1024;
  static_assert(SLICES % NW == 0, "DMA slices per wave");
  constexpr int ROWS_PER_KB = 1024 / D;
  constexpr int CH = D / 16;         // 16-byte chunks per FP8 row
  static_assert((64 * NW) % BN == 0 && (D / ((64 * NW) / BN)) % 16 == 0, "widening split");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE + VTILE];
  uint8_t* const vb = smem + 2 * STAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hsel = lane >> 5;
  const int l32 = lane & 31;

  const int rows_wg = 32 * NW;
  const int n_qt = (p.s_q + rows_wg - 1) / rows_wg;
  const int units = p.batch * p.h_q;
  const int qt = n_qt - 1 - (int)blockIdx.x / units;  // heaviest (last) tiles first
  const int u = blockIdx.x % units;
  const int b = u / p.h_q, h = u % p.h_q;
  const int hk = h / p.group;
  const int sq = p.s_q, sk = p.s_k, off = sk - sq;
  const int q0 = qt * rows_wg;
  const int q0w = q0 + 32 * wave;
  const int qrow = q0w + l32;

  // ---- key blocks any row of the tile sees.
  const int t1 = min(q0 + rows_wg, sq) - 1;
  int kmin = 0, kmax = sk - 1;
  if (p.wl >= 0) kmin = max(0, q0 + off - p.wl);
  if (p.wr >= 0) kmax = min(kmax, t1 + off + p.wr);
  const int n_lo = kmax >= kmin ? kmin / BN : 0;
  const int n_hi = kmax >= kmin ? kmax / BN + 1 : 0;

  // ---- Q^T as B operand.  Head dims are taken in a fixed order shared with the
  // K reads: k-step pair j, lane half H holds dims 32 j + 16 H .. + 15, its
  // first 8 bytes k-step 2 j and its last 8 bytes k-step 2 j + 1.
  u32x4_t qf[KP];
  {
    const bool in = qrow < sq;
    const uint8_t* qp = p.q + (int64_t)b * p.q_sb + (int64_t)qrow * p.q_ss + (int64_t)h * p.q_sh + 16 * hsel;
#pragma unroll
    for (int j = 0; j < KP; ++j) qf[j] = in ? *(const u32x4_t*)(qp + 32 * j) : u32x4_t{0, 0, 0, 0};
  }

  // ---- DMA of the FP8 K and V tiles: tile row r, chunk c at r * D + 16 * (c ^ f8swz(r)) for K,
  // plain for V.
  const uint8_t* kg = p.k + (int64_t)b * p.k_sb + (int64_t)hk * p.k_sh;
  const uint8_t* vg = p.v + (int64_t)b * p.v_sb + (int64_t)hk * p.v_sh;
  uint32_t kofs[SLICES / NW], vofs[SLICES / NW];
#pragma unroll
  for (int i = 0; i < SLICES / NW; ++i) {
    const int row = (NW * i + wave) * ROWS_PER_KB + lane / CH;
    kofs[i] = (uint32_t)(row * p.k_ss + 16 * ((lane % CH) ^ f8swz<D>(row)));
    vofs[i] = (uint32_t)(row * p.v_ss + 16 * (lane % CH));
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

  // ---- LDS addresses.  K A operand: tile t2 row m = l32 is key 32 t2 + row_key(l32),
  // k-step pair j at chunk 2 j + H.
  const int krow = row_key(l32);
  int kaddr[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) kaddr[j] = krow * D + 16 * ((2 * j + hsel) ^ f8swz<D>(krow));
  // V^T operand of O^T += V^T P^T: rows = head dims, k = 8 consecutive keys per lane half.
  const int gi = lane >> 4, li = lane & 15;
  int tr[2][DT];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int row = 8 * (gi >> 1) + 4 * half + (li >> 2);
      const int dcol = 32 * dt + 16 * (gi & 1) + 4 * (li & 3);
      tr[half][dt] = row * (D * 2) + 16 * ((dcol >> 3) ^ vswz16<D>(row)) + 2 * (dcol & 7);
    }
  // Widening: thread t takes V row t / TPR (TPR threads per row), bytes SEG * (t % TPR) .. + SEG - 1.
  constexpr int TPR = 64 * NW / BN;           // threads per V row
  constexpr int SEG = D / TPR;                // FP8 bytes per thread, a multiple of 16
  const int wrow = tid / TPR, wseg = tid % TPR;

  float m = -__builtin_inff(), l = 0.f;  // running max (log2 domain) and sum
  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16_t{};

  auto block = [&](int n, const uint8_t* __restrict__ kt, const uint8_t* __restrict__ v8,
                   uint8_t* __restrict__ nxt) {
    // S^T = K Q^T on the FP8 MFMA
    f32x16_t s[NT2];
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2) s[t2] = f32x16_t{};
#pragma unroll
    for (int j = 0; j < KP; ++j)
#pragma unroll
      for (int t2 = 0; t2 < NT2; ++t2) {
        const u32x4_t a = *(const u32x4_t*)(kt + kaddr[j] + t2 * 32 * D);
        const long a0 = __builtin_bit_cast(long, u32x2_t{a[0], a[1]});
        const long a1 = __builtin_bit_cast(long, u32x2_t{a[2], a[3]});
        const long b0 = __builtin_bit_cast(long, u32x2_t{qf[j][0], qf[j][1]});
        const long b1 = __builtin_bit_cast(long, u32x2_t{qf[j][2], qf[j][3]});
        s[t2] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a0, b0, s[t2], 0, 0, 0);
        s[t2] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a1, b1, s[t2], 0, 0, 0);
      }
    if (n + 1 < n_hi) issue(n + 1, nxt);
    // widen V: FP8 row-major staging -> bf16 tile
#pragma unroll
    for (int c = 0; c < SEG / 16; ++c) {
      const u32x4_t w = *(const u32x4_t*)(v8 + wrow * D + SEG * wseg + 16 * c);
      u32x4_t lo, hi;
      lo[0] = f8pair_bf16<false>(w[0]), lo[1] = f8pair_bf16<true>(w[0]);
      lo[2] = f8pair_bf16<false>(w[1]), lo[3] = f8pair_bf16<true>(w[1]);
      hi[0] = f8pair_bf16<false>(w[2]), hi[1] = f8pair_bf16<true>(w[2]);
      hi[2] = f8pair_bf16<false>(w[3]), hi[3] = f8pair_bf16<true>(w[3]);
      const int ch = (SEG * wseg + 16 * c) / 8;  // first bf16 chunk of these 16 values
      *(u32x4_t*)(vb + wrow * (D * 2) + 16 * (ch ^ vswz16<D>(wrow))) = lo;
      *(u32x4_t*)(vb + wrow * (D * 2) + 16 * ((ch + 1) ^ vswz16<D>(wrow))) = hi;
    }
    // scores in the log2 domain; register 8c + u of tile t2 is key n BN + 32 t2 + 16 c + 8 H + u
    const int kb0 = n * BN;
    const bool full = q0w + 32 <= sq && kb0 + BN <= sk && (p.wr < 0 || kb0 + BN - 1 <= q0w + off + p.wr) &&
                      (p.wl < 0 || kb0 >= q0w + 31 + off - p.wl);
    float mx = -__builtin_inff();
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[t2][r] * p.scale_log2;
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
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    __syncthreads();  // the bf16 V tile is complete
    // O^T += V^T P^T
#pragma unroll
    for (int t2 = 0; t2 < NT2; ++t2)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int rows = (32 * t2 + 16 * c) * (D * 2);
          const u32x2_t lo = lds_read_tr16(vb + tr[0][dt] + rows), hi = lds_read_tr16(vb + tr[1][dt] + rows);
          u32x4_t a;
          a[0] = lo[0], a[1] = lo[1], a[2] = hi[0], a[3] = hi[1];
          o[dt] = Elem<true>::mfma32x32x16(a, pb[t2][c], o[dt]);
        }
  };

  uint8_t* const s0 = smem;
  uint8_t* const s1 = smem + STAGE;
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

  // ---- O = (O^T)^T v_descale / l as bf16; lane holds head dims 32 dt + 8 J + 4 H + 0..3 of row qrow.
  if (qrow < sq) {
    const float inv = l > 0.f ? p.v_descale / l : 0.f;
    uint16_t* op = p.o + (int64_t)b * p.o_sb + (int64_t)qrow * p.o_ss + (int64_t)h * p.o_sh;
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
      p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + qrow] =
          l > 0.f ? (m + fast_log2(l)) * kLn2 : kNegInf;
  }
}

template <int D>
hipError_t launch_fp8_t(const Fp8Params& p, hipStream_t stream) {
  constexpr int NW = 2;
  const int n_qt = (p.s_q + 32 * NW - 1) / (32 * NW);
  if (n_qt == 0 || p.batch == 0) return hipSuccess;
  hipLaunchKernelGGL((fp8_prefill_kernel<D, NW>), dim3(n_qt * p.h_q * p.batch), dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Params& p, int head_dim, hipStream_t stream) {
  if (head_dim == 64) return launch_fp8_t<64>(p, stream);
  if (head_dim == 128) return launch_fp8_t<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace exattn
