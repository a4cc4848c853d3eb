// KV-cache decode: one query token per sequence against cache_seqlens[b] cached
// keys (Inference Cookbook FAQ Q17), split over the key axis (FAQ Q14's
// num_splits) and merged by log-sum-exp.
//
// Kernel 1 (decode_kernel), one work group per (split, KV head [x group of 16
// query heads], batch entry):
// - the query heads that share the KV head are packed into the columns of a
//   16x16x32 MFMA (S^T = K Q^T), so each K/V byte is read from HBM once for all
//   of them (grouped heads, FAQ Q15);
// - each of the 4 waves walks its own 32-key chunks of the split (chunks
//   w, w+4, ...), so no block-wide barrier is needed in the loop; K goes from
//   global memory straight into MFMA A-operand registers, V through a
//   wave-private LDS area where it is stored transposed for O^T = V^T P^T;
// - the next chunk's K/V loads are issued before the current chunk's math;
// - per query: online softmax in the log2 domain as in the prefill kernel;
// - at the end the 4 waves' (m, l, O) are merged through LDS and the split
//   writes either the final O/LSE (one split) or fp32 partials to the
//   workspace.
// Kernel 2 (combine_kernel): LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s -
// LSE) O_s, the merge of partial softmax results ("FlashAttention完整说明",
// section 二.1); a split with no keys has LSE_s = -inf and weight 0.
#include "device_common.h"
#include "kernels.h"

namespace exattn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kCh = 32;  // keys per wave step

// V^T area of one wave: row d holds the chunk's 32 keys (4 x 16-byte pieces of
// 8 keys); piece kc lives at kc ^ swz(d).
__device__ __forceinline__ int dvt_off(int d, int kc) {
  const int s = ((d >> 1) ^ (d >> 3)) & 3;
  return d * (kCh * 2) + 16 * (kc ^ s);
}

template <int D>
struct DecodeSmem {
  static constexpr int kVt = kWaves * D * kCh * 2;
  static constexpr int kComb = (2 * kWaves * 16 + kWaves * 16 * D) * 4;
  static constexpr int kBytes = kVt > kComb ? kVt : kComb;
};

template <bool BF16, int D, bool SOFTCAP>
__global__ void __launch_bounds__(kThreads) decode_kernel(const DecParams p) {
  using E = Elem<BF16>;
  constexpr int DCH = D / 8;
  constexpr int KS = D / 32;             // k-steps of the 16x16x32 MFMA over head_dim
  constexpr int DT = D / 16;             // 16-wide head_dim tiles of O^T
  constexpr int VLD = (kCh / 4) * DCH / 64;  // (4 keys x 8 columns) V pieces per lane
  static_assert(VLD >= 1, "head_dim too small");

  __shared__ __attribute__((aligned(16))) uint8_t smem[DecodeSmem<D>::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g16 = lane >> 4;
  const int l16 = lane & 15;

  const int split = blockIdx.x;
  const int hk = blockIdx.y / p.n_hg;
  const int hg = blockIdx.y % p.n_hg;
  const int b = blockIdx.z;

  // cache_seqlens[b] is clamped to [0, s_cache] so a bad entry cannot address
  // memory outside the cache.
  const int nk = p.cache_seqlens != nullptr ? min(max(p.cache_seqlens[b], 0), p.s_cache) : p.s_cache;
  // The query sits at position nk - 1; only the left window edge removes keys.
  const int kb = p.wl >= 0 ? max(0, nk - 1 - p.wl) : 0;
  const int nchunks = nk > kb ? (nk - kb + kCh - 1) / kCh : 0;
  const int per = (nchunks + p.n_split - 1) / p.n_split;
  const int c_lo = split * per;
  const int c_hi = min(nchunks, c_lo + per);

  // Query column l16 of the MFMA is query head hk*group + hg*16 + l16.
  const int qj = hg * 16 + l16;
  const bool qvalid = qj < p.group;
  const int hq = hk * p.group + qj;
  u32x4_t qf[KS];
  if (qvalid) {
    const uint16_t* qp = p.q + (int64_t)b * p.q_sb + (int64_t)hq * p.q_sh + 8 * g16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const u32x4_t*)(qp + 32 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = u32x4_t{0, 0, 0, 0};
  }

  const uint16_t* kg = p.k + (int64_t)b * p.k_sb + (int64_t)hk * p.k_sh;
  const uint16_t* vg = p.v + (int64_t)b * p.v_sb + (int64_t)hk * p.v_sh;
  uint8_t* vt = smem + wave * (D * kCh * 2);

  f32x4_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  // A-operand row i of key tile kt is key 8 (i/4) + 4 kt + i%4, so the four
  // accumulator rows a lane group G holds are keys 8G + 4kt + 0..3 and, over
  // both tiles, keys 8G .. 8G+7 in order.
  const int krow = 8 * (l16 >> 2) + (l16 & 3);

  u32x4_t kr[2][KS];
  u32x4_t vr[VLD][4];
  auto load = [&](int c) {
    const int base = kb + c * kCh;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = base + krow + 4 * kt;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kr[kt][ks] = key < nk ? *(const u32x4_t*)(kg + (int64_t)key * p.k_ss + 32 * ks + 8 * g16)
                              : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int un = lane + 64 * i;
      const int kq = un / DCH, dc = un % DCH;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = base + 4 * kq + r;
        vr[i][r] = key < nk ? *(const u32x4_t*)(vg + (int64_t)key * p.v_ss + 8 * dc)
                            : u32x4_t{0, 0, 0, 0};
      }
    }
  };

  int c = c_lo + wave;
  if (c < c_hi) load(c);
  for (; c < c_hi; c += kWaves) {
    u32x4_t kc_[2][KS];
    u32x4_t vc_[VLD][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kc_[kt][ks] = kr[kt][ks];
#pragma unroll
    for (int i = 0; i < VLD; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) vc_[i][r] = vr[i][r];
    if (c + kWaves < c_hi) load(c + kWaves);

    const int base = kb + c * kCh;
    f32x4_t s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s[kt] = E::mfma16x16x32(kc_[kt][ks], qf[ks], s[kt]);
    }

    float x[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (SOFTCAP)
          x[kt][r] = p.cap_out_log2 * tanh_exp2(s[kt][r] * p.cap_in);
        else
          x[kt][r] = s[kt][r] * p.scale_log2;
        const int key = base + 8 * g16 + 4 * kt + r;
        if (key >= nk) x[kt][r] = kNegInf;
      }
    float mx = x[0][0];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, x[kt][r]);
    mx = fmaxf(mx, xor16(mx));
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float bse = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - bse);
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[kt][r] = fast_exp2(x[kt][r] - bse);
        psum += x[kt][r];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;

    // V chunk -> V^T in this wave's LDS area.
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int un = lane + 64 * i;
      const int kq = un / DCH, dc = un % DCH;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        *(u32x2_t*)(vt + dvt_off(8 * dc + t, kq >> 1) + 8 * (kq & 1)) =
            column4(vc_[i][0], vc_[i][1], vc_[i][2], vc_[i][3], t);
    }
    wave_lds_fence();

    // P^T operand: logical k = 8 G + t is key 8 G + t = tile t/4, register t%4.
    u32x4_t pf;
    pf[0] = E::pack2(x[0][0], x[0][1]);
    pf[1] = E::pack2(x[0][2], x[0][3]);
    pf[2] = E::pack2(x[1][0], x[1][1]);
    pf[3] = E::pack2(x[1][2], x[1][3]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const u32x4_t a = *(const u32x4_t*)(vt + dvt_off(16 * dt + l16, g16));
      oacc[dt] = E::mfma16x16x32(a, pf, oacc[dt]);
    }
    wave_lds_fence();
  }

  // ---- merge the four waves through LDS.
  float l_tot = l_run + xor16(l_run);
  l_tot += xor32(l_tot);
  __syncthreads();
  float* cm = reinterpret_cast<float*>(smem);
  float* cl = cm + kWaves * 16;
  float* co = cl + kWaves * 16;  // [wave][query][d]
  if (g16 == 0) {
    cm[wave * 16 + l16] = m_run;
    cl[wave * 16 + l16] = l_tot;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) co[(wave * 16 + l16) * D + 16 * dt + 4 * g16 + r] = oacc[dt][r];
  __syncthreads();

  for (int e = tid; e < 16 * D; e += kThreads) {
    const int j = e / D, d = e % D;
    const int qj2 = hg * 16 + j;
    if (qj2 >= p.group) continue;
    const int h = hk * p.group + qj2;
    float mt = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mt = fmaxf(mt, cm[w * 16 + j]);
    float o = 0.f, lse = kNegInf;
    if (mt != kNegInf) {
      float ws = 0.f, os = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = fast_exp2(cm[w * 16 + j] - mt);
        ws += f * cl[w * 16 + j];
        os += f * co[(w * 16 + j) * D + d];
      }
      o = os / ws;
      lse = (mt + fast_log2(ws)) * kLn2;
    }
    if (p.n_split == 1) {
      const uint32_t packed = E::pack2(o, 0.f);
      p.o[(int64_t)b * p.o_sb + (int64_t)h * p.o_sh + d] = (uint16_t)(packed & 0xffffu);
      if (d == 0 && p.lse != nullptr) p.lse[(int64_t)b * p.h_q + h] = lse;
    } else {
      const int64_t row = ((int64_t)split * p.batch + b) * p.h_q + h;
      p.ws_o[row * D + d] = o;
      if (d == 0) p.ws_lse[row] = lse;
    }
  }
}

template <bool BF16, int D>
__global__ void __launch_bounds__(D) combine_kernel(const DecParams p) {
  using E = Elem<BF16>;
  const int bh = blockIdx.x;
  const int b = bh / p.h_q, h = bh % p.h_q;
  const int d = threadIdx.x;
  const int64_t stride = (int64_t)p.batch * p.h_q;
  const int64_t row0 = (int64_t)b * p.h_q + h;
  float mx = kNegInf;
  for (int s = 0; s < p.n_split; ++s) mx = fmaxf(mx, p.ws_lse[s * stride + row0]);
  float o = 0.f, lse = kNegInf;
  if (mx != kNegInf) {
    float ws = 0.f, acc = 0.f;
    for (int s = 0; s < p.n_split; ++s) {
      const float w = fast_exp2((p.ws_lse[s * stride + row0] - mx) * kLog2e);
      ws += w;
      acc += w * p.ws_o[(s * stride + row0) * D + d];
    }
    o = acc / ws;
    lse = mx + fast_log2(ws) * kLn2;
  }
  const uint32_t packed = E::pack2(o, 0.f);
  p.o[(int64_t)b * p.o_sb + (int64_t)h * p.o_sh + d] = (uint16_t)(packed & 0xffffu);
  if (d == 0 && p.lse != nullptr) p.lse[row0] = lse;
}

template <bool BF16, int D>
hipError_t launch_d(const DecParams& p, bool softcap, hipStream_t stream) {
  const dim3 grid(p.n_split, p.h_kv * p.n_hg, p.batch);
  if (softcap)
    hipLaunchKernelGGL((decode_kernel<BF16, D, true>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_kernel<BF16, D, false>), grid, dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_split == 1) return e;
  hipLaunchKernelGGL((combine_kernel<BF16, D>), dim3(p.batch * p.h_q), dim3(D), 0, stream, p);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_t(const DecParams& p, int head_dim, bool softcap, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<BF16, 64>(p, softcap, stream);
    case 128: return launch_d<BF16, 128>(p, softcap, stream);
    case 256: return launch_d<BF16, 256>(p, softcap, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecParams& p, bool bf16, int head_dim, bool softcap,
                         hipStream_t stream) {
  return bf16 ? launch_t<true>(p, head_dim, softcap, stream)
              : launch_t<false>(p, head_dim, softcap, stream);
}

}  // namespace exattn
