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
// - work group = 4 waves x 32 query rows = 128 rows of one query head;
// - the wave computes S^T = K Q^T with v_mfma_f32_32x32x16 (bf16/f16, fp32
//   accumulate): K is the A operand (read from LDS), Q^T the B operand held in
//   registers for the whole loop.  In the 32x32 accumulator layout every lane
//   then owns ONE query row and 16 keys of it, so the row max and row sum are
//   in-lane, plus one exchange between the two 32-lane halves;
// - the A-operand row -> key assignment is permuted so that each lane's 16
//   scores are 16 consecutive keys; the same registers, rounded to 16-bit, are
//   directly the B operand (P^T) of O^T = V^T P^T, with no data movement;
// - V^T comes from LDS, where the V tile is stored transposed (each thread
//   loads 4 key rows x 8 columns and writes 8 key-contiguous 8-byte pieces);
// - K and V tiles of 64 keys are double-buffered in LDS: the global loads of
//   block n+1 are issued before the MFMAs of block n and written to the other
//   buffer after them, one barrier per block;
// - 16-byte chunks in LDS are XOR-swizzled per row so that the MFMA operand
//   reads of 8 (or 16) lanes fall into distinct banks;
// - scores are kept in the log2 domain: x = s * scale * log2(e), p = 2^(x - m),
//   so the exponential is the hardware 2^x;
// - masks (bottom-right causal, window, sequence tail) are evaluated only on
//   the KV blocks that straddle a boundary; blocks entirely outside every row's
//   window are never visited;
// - query tiles are issued heaviest first (the last tiles of a causal head see
//   the most keys), and the tiles of one head land on one XCD (work group id
//   modulo 8), so their K/V re-reads hit that XCD's L2.
#include "device_common.h"
#include "kernels.h"

namespace exattn {
namespace {

constexpr int kBM = 128;  // query rows per work group
constexpr int kBN = 64;   // keys per KV block
constexpr int kThreads = 256;

// K tile: row `key` is D*2 bytes; 16-byte chunk c lives at chunk c ^ swz(key).
// The swizzle gives the keys that 8 (16) consecutive lanes read in one MFMA
// operand load distinct low 3 (4) bits.
template <int D>
__device__ __forceinline__ int k_off(int key, int chunk) {
  constexpr int kMask = (D / 8 - 1) & 15;
  const int s = (key & 3) | (((key >> 4) & 1) << 2) | (((key >> 2) & 1) << 3);
  return key * (D * 2) + 16 * (chunk ^ (s & kMask));
}

// V^T tile: row d holds the block's 64 keys (8 chunks of 8 keys, 128 bytes);
// chunk kc lives at kc ^ swz(d).
__device__ __forceinline__ int vt_off(int d, int kc) {
  const int s = (d ^ (d >> 3)) & 7;
  return d * (kBN * 2) + 16 * (kc ^ s);
}

template <bool BF16, int D, bool SOFTCAP>
__global__ void __launch_bounds__(kThreads) prefill_kernel(const FwdParams p) {
  using E = Elem<BF16>;
  constexpr int DCH = D / 8;     // 16-byte chunks per row
  constexpr int KS = D / 16;     // k-steps of the 32x32x16 MFMA over head_dim
  constexpr int DT = D / 32;     // 32-wide head_dim tiles of O^T
  constexpr int KTILE = kBN * D * 2;
  constexpr int STAGE = 2 * KTILE;
  constexpr int KLD = kBN * DCH / kThreads;        // K chunks loaded per thread
  constexpr int VUNITS = (kBN / 4) * DCH;          // (4 keys x 8 columns) V pieces
  constexpr int VLD = (VUNITS + kThreads - 1) / kThreads;
  static_assert(KLD >= 1 && kBN * DCH % kThreads == 0, "tile/thread mismatch");

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hsel = lane >> 5;  // which 32-lane half
  const int l32 = lane & 31;

  // ---- tile scheduler: heaviest query tiles first; (batch, head) fastest.
  const int units = p.batch * p.h_q;
  const int bid = blockIdx.x;
  const int qt = p.n_qt - 1 - bid / units;
  const int u = bid % units;
  int b, h;
  if (p.xcd_group) {
    // unit u -> (KV unit, member j): u % 8 selects the XCD and depends only on
    // the KV unit, so the query heads sharing one K/V share one L2.
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

  f32x16_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16_t{};
  float m_run = kNegInf;  // running max of x = score * log2(e)
  float l_run = 0.f;      // this lane's share of the running sum

  // Row of the A operand -> key within a 32-key tile: row 8J + 4H + I is key
  // 16H + 4J + I, so accumulator register r of lane half H is key 16H + r.
  const int sig = ((l32 >> 2) & 1) * 16 + (l32 >> 3) * 4 + (l32 & 3);

  u32x4_t kst[KLD];
  u32x4_t vst[VLD][4];

  auto load_block = [&](int n) {
    const int kb = n * kBN;
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int c = tid + i * kThreads;
      const int key = c / DCH, dc = c % DCH;
      const int gk = kb + key;
      kst[i] = gk < sk ? *(const u32x4_t*)(kg + (int64_t)gk * p.k_ss + 8 * dc)
                       : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int un = tid + i * kThreads;
      if (un < VUNITS) {
        const int kq = un / DCH, dc = un % DCH;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gk = kb + 4 * kq + r;
          vst[i][r] = gk < sk ? *(const u32x4_t*)(vg + (int64_t)gk * p.v_ss + 8 * dc)
                              : u32x4_t{0, 0, 0, 0};
        }
      }
    }
  };

  auto store_block = [&](int stage) {
    uint8_t* ks_ = smem + stage * STAGE;
    uint8_t* vs_ = ks_ + KTILE;
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int c = tid + i * kThreads;
      *(u32x4_t*)(ks_ + k_off<D>(c / DCH, c % DCH)) = kst[i];
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int un = tid + i * kThreads;
      if (un < VUNITS) {
        const int kq = un / DCH, dc = un % DCH;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          *(u32x2_t*)(vs_ + vt_off(8 * dc + t, kq >> 1) + 8 * (kq & 1)) =
              column4(vst[i][0], vst[i][1], vst[i][2], vst[i][3], t);
        }
      }
    }
  };

  if (n_lo < n_hi) {
    load_block(n_lo);
    store_block(0);
  }
  __syncthreads();

  for (int n = n_lo; n < n_hi; ++n) {
    const int stage = (n - n_lo) & 1;
    const bool has_next = n + 1 < n_hi;
    if (has_next) load_block(n + 1);
    const uint8_t* ks_ = smem + stage * STAGE;
    const uint8_t* vs_ = ks_ + KTILE;

    // S^T for the two 32-key tiles of the block.
    f32x16_t s[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      s[t2] = f32x16_t{};
      const int key = 32 * t2 + sig;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t a = *(const u32x4_t*)(ks_ + k_off<D>(key, 2 * ks + hsel));
        s[t2] = E::mfma32x32x16(a, qf[ks], s[t2]);
      }
    }

    // Scores -> log2 domain, softcap, mask.
    const int kb = n * kBN;
    float x[2][16];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (SOFTCAP)
          x[t2][r] = p.cap_out_log2 * tanh_exp2(s[t2][r] * p.cap_in);
        else
          x[t2][r] = s[t2][r] * p.scale_log2;
      }
    const bool need_mask = (kb + kBN > sk) || (p.wr >= 0 && kb + kBN - 1 > q0 + off + p.wr) ||
                           (p.wl >= 0 && kb < q_last + off - p.wl);
    if (need_mask) {
      const int hi = p.wr >= 0 ? min(sk - 1, qrow + off + p.wr) : sk - 1;
      const int lo = p.wl >= 0 ? qrow + off - p.wl : -0x7fffffff;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kidx = kb + 32 * t2 + 16 * hsel + r;
          if (kidx > hi || kidx < lo) x[t2][r] = kNegInf;
        }
    }

    // Online softmax update.
    float mx = x[0][0];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x[t2][r]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float base = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - base);
    float psum = 0.f;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[t2][r] = fast_exp2(x[t2][r] - base);
        psum += x[t2][r];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;

    // P^T fragments: the B operand of MFMA (t2, c) is keys 32 t2 + 16 H + 8 c + 0..7,
    // i.e. this lane's registers 8c .. 8c+7 of tile t2.
    u32x4_t pf[2][2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          pf[t2][c][w] = E::pack2(x[t2][8 * c + 2 * w], x[t2][8 * c + 2 * w + 1]);

    // O^T += V^T P^T.
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 32 * dt + l32;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const u32x4_t a = *(const u32x4_t*)(vs_ + vt_off(d, 4 * t2 + 2 * hsel + c));
          oacc[dt] = E::mfma32x32x16(a, pf[t2][c], oacc[dt]);
        }
    }

    if (has_next) store_block(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2; empty rows: 0 and -inf.
  const float l_tot = l_run + xor32(l_run);
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
      lseg[qrow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
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
