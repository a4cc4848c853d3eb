// KV-cache decode: one query token per sequence against cache_seqlens[b] cached
// keys (Inference Cookbook FAQ Q17), split over the key axis (FAQ Q14's
// num_splits) and merged by log-sum-exp.
//
// Kernel 1 (decode_kernel), one work group per (split, group of hpw adjacent
// KV heads [x group of 16 query heads], batch entry):
// - hpw adjacent KV heads make one 512-byte piece of every key row (2 heads at
//   d = 128), so the work group streams contiguous pieces of the cache rather
//   than 256-byte pieces 2 KiB apart (measured: about 6.0 vs 5.4 TB/s for a
//   plain read of that layout);
// - wave w takes head slot w % hpw and every (4 / hpw)-th 32-key chunk of the
//   split, starting at w / hpw, so no block-wide barrier is needed in the loop;
// - the query heads that share a KV head are packed into the columns of a
//   16x16x32 MFMA (S^T = K Q^T), so each K/V byte is read from HBM once for all
//   of them (grouped heads, FAQ Q15);
// - K goes by DMA (buffer_load ... lds) into a wave-private LDS area, 16 lanes
//   per contiguous 256-byte piece of a key row, XOR-swizzled so the MFMA
//   A-operand reads are free of bank conflicts.  Loading K directly in the
//   A-operand order (16 keys x 64 bytes per instruction) cost about 10% of the
//   read bandwidth (measured);
// - V is loaded into registers (16 lanes per 256-byte row piece) and written
//   to a second wave-private LDS area transposed, for O^T = V^T P^T;
// - the next chunk's V loads are issued before the current chunk's math and
//   its K DMA right after the current chunk's K has been read;
// - per query: online softmax in the log2 domain as in the prefill kernel;
// - at the end the waves of each head merge (m, l, O) through LDS and the
//   split writes either the final O/LSE (one split) or fp32 partials to the
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

// K area of one wave: row `key` (0..31) holds D*2 bytes; 16-byte chunk c is
// stored at c ^ kswz(key).  The 8 lanes of one A-operand read phase read keys
// {b..b+3, b+8..b+11} of one chunk column; the swizzle gives them distinct bank
// groups.
__device__ __forceinline__ int kswz(int key) { return (key & 3) | (((key >> 3) & 1) << 2); }

// Buffer descriptor for the rows kb .. nk-1 of one head (row stride ss
// elements): loads past the last valid element return zeros (per-dword range
// check of raw buffer loads).  Word 3 is the gfx9 default.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* g, int64_t ss, int kb, int nk) {
  const int64_t last = (int64_t)(nk - 1 - kb) * ss + D;
  return __builtin_amdgcn_make_buffer_rsrc((void*)(g + (int64_t)kb * ss), 0, (int)(last * 2), 0x00020000);
}

// 16 bytes per lane from a buffer into LDS at lds + 16 * lane (lds must be
// wave-uniform).  Kept out of lambdas: the host pass of the compiler drops the
// kernel stub when this builtin sits in a lambda body.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, uint8_t* lds, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voffset, 0, 0, 0);
}

template <int D>
struct DecodeSmem {
  static constexpr int kWave = 2 * D * kCh * 2;  // K tile + V^T tile
  static constexpr int kTiles = kWaves * kWave;
  static constexpr int kComb = (2 * kWaves * 16 + kWaves * 16 * D) * 4;
  static constexpr int kBytes = kTiles > kComb ? kTiles : kComb;
};

template <bool BF16, int D, bool SOFTCAP>
__global__ void __launch_bounds__(kThreads) decode_kernel(const DecParams p) {
  using E = Elem<BF16>;
  constexpr int DCH = D / 8;
  constexpr int KS = D / 32;             // k-steps of the 16x16x32 MFMA over head_dim
  constexpr int DT = D / 16;             // 16-wide head_dim tiles of O^T
  constexpr int VLD = (kCh / 4) * DCH / 64;  // (4 keys x 8 columns) V pieces per lane
  constexpr int KI = kCh * D * 2 / 1024;      // K DMA instructions per chunk
  static_assert(VLD >= 1 && KI >= 1 && DCH >= 8, "head_dim too small");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[DecodeSmem<D>::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g16 = lane >> 4;
  const int l16 = lane & 15;

  const int split = blockIdx.x;
  const int hgrp = blockIdx.y / p.n_hg;
  const int hg = blockIdx.y % p.n_hg;
  const int b = blockIdx.z;
  const int hpw = p.hpw;          // 1, 2 or 4: divides the wave count
  const int wph = kWaves / hpw;   // waves per head
  const int slot = wave % hpw;    // head slot of this wave
  const int phase = wave / hpw;   // first chunk of this wave
  const int hk = hgrp * hpw + slot;
  const bool head_ok = hk < p.h_kv;

  // cache_seqlens[b] is clamped to [0, s_cache] so a bad entry cannot address
  // memory outside the cache.
  const int nk = p.cache_seqlens != nullptr ? min(max(p.cache_seqlens[b], 0), p.s_cache) : p.s_cache;
  // The query sits at position nk - 1; only the left window edge removes keys.
  const int kb = p.wl >= 0 ? max(0, nk - 1 - p.wl) : 0;
  const int nchunks = nk > kb ? (nk - kb + kCh - 1) / kCh : 0;
  const int per = (nchunks + p.n_split - 1) / p.n_split;
  const int c_lo = split * per;
  const int c_hi = head_ok ? min(nchunks, c_lo + per) : c_lo;

  // Query column l16 of the MFMA is query head hk*group + hg*16 + l16.
  const int qj = hg * 16 + l16;
  const bool qvalid = head_ok && qj < p.group;
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
  uint8_t* kt_lds = smem + wave * DecodeSmem<D>::kWave;
  uint8_t* vt = kt_lds + D * kCh * 2;

  f32x4_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  // A-operand row i of key tile kt is key 8 (i/4) + 4 kt + i%4, so the four
  // accumulator rows a lane group G holds are keys 8G + 4kt + 0..3 and, over
  // both tiles, keys 8G .. 8G+7 in order.  kswz of these keys does not depend
  // on kt; chunk 4 ks + g16 is stored at 4 (ks ^ s1) + (g16 ^ s0), so two
  // bases cover every ks.
  const int krow = 8 * (l16 >> 2) + (l16 & 3);
  int kaddr[2];
  {
    const int sw = kswz(krow);
#pragma unroll
    for (int j = 0; j < 2; ++j) kaddr[j] = krow * (D * 2) + 64 * (j ^ (sw >> 2)) + 16 * (g16 ^ (sw & 3));
  }
  // K DMA: instruction i, lane l fills LDS bytes i*1024 + 16 l of the K area,
  // i.e. row key, stored chunk pos; it fetches global chunk pos ^ kswz(key).
  uint32_t kofs[KI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int o = i * 1024 + 16 * lane;
    const int key = o / (D * 2), pos = (o % (D * 2)) / 16;
    kofs[i] = (uint32_t)(key * p.k_ss * 2 + 16 * (pos ^ kswz(key)));
  }
  auto issue_k = [&](int c) {
    __amdgpu_buffer_rsrc_t rs = rows_rsrc<D>(kg, p.k_ss, kb + c * kCh, nk);
#pragma unroll
    for (int i = 0; i < KI; ++i) buffer_load_lds16(rs, kt_lds + i * 1024, kofs[i]);
  };

  u32x4_t vr[VLD][4];
  auto load_v = [&](int c) {
    const int base = kb + c * kCh;
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

  int c = c_lo + phase;
  if (c < c_hi) {
    issue_k(c);
    load_v(c);
  }
  for (; c < c_hi; c += wph) {
    // this wave's K DMA and V loads of chunk c have landed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    u32x4_t vc_[VLD][4];
#pragma unroll
    for (int i = 0; i < VLD; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) vc_[i][r] = vr[i][r];
    const bool more = c + wph < c_hi;
    if (more) load_v(c + wph);

    const int base = kb + c * kCh;
    f32x4_t s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t a =
            *(const u32x4_t*)(kt_lds + kaddr[ks & 1] + 128 * (ks >> 1) + kt * 4 * (D * 2));
        s[kt] = E::mfma16x16x32(a, qf[ks], s[kt]);
      }
    }
    // every K read of this chunk has returned: the K area may be refilled
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (more) issue_k(c + wph);

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

  // ---- merge the waves of each head through LDS.
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

  for (int e = tid; e < hpw * 16 * D; e += kThreads) {
    const int sl = e / (16 * D);
    const int j = (e / D) % 16, d = e % D;
    const int hk2 = hgrp * hpw + sl;
    const int qj2 = hg * 16 + j;
    if (hk2 >= p.h_kv || qj2 >= p.group) continue;
    const int h = hk2 * p.group + qj2;
    float mt = kNegInf;
    for (int t = 0; t < wph; ++t) mt = fmaxf(mt, cm[(sl + hpw * t) * 16 + j]);
    float o = 0.f, lse = kNegInf;
    if (mt != kNegInf) {
      float ws = 0.f, os = 0.f;
      for (int t = 0; t < wph; ++t) {
        const int w = sl + hpw * t;
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

// One work group of D threads per (batch, query head); thread d owns column d.
// The splits are taken 16 at a time with all their loads issued together, and
// merged with a running maximum, so a call with up to 16 splits waits for one
// round trip to memory.
template <bool BF16, int D>
__global__ void __launch_bounds__(D) combine_kernel(const DecParams p) {
  using E = Elem<BF16>;
  constexpr int kU = 16;
  const int bh = blockIdx.x;
  const int b = bh / p.h_q, h = bh % p.h_q;
  const int d = threadIdx.x;
  const int64_t stride = (int64_t)p.batch * p.h_q;
  const int64_t row0 = (int64_t)b * p.h_q + h;
  float m = kNegInf, ws = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < p.n_split; s0 += kU) {
    float l[kU], v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool in = s0 + u < p.n_split;
      l[u] = in ? p.ws_lse[(s0 + u) * stride + row0] : kNegInf;
      v[u] = in ? p.ws_o[((s0 + u) * stride + row0) * D + d] : 0.f;
    }
    float mb = l[0];
#pragma unroll
    for (int u = 1; u < kU; ++u) mb = fmaxf(mb, l[u]);
    if (mb > m) {  // move the reference; nothing to rescale while it was -inf
      const float sc = m == kNegInf ? 0.f : fast_exp2((m - mb) * kLog2e);
      ws *= sc;
      acc *= sc;
      m = mb;
    }
    if (m != kNegInf) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float w = fast_exp2((l[u] - m) * kLog2e);  // 0 for an empty split
        ws += w;
        acc += w * v[u];
      }
    }
  }
  float o = 0.f, lse = kNegInf;
  if (m != kNegInf) {
    o = acc / ws;
    lse = m + fast_log2(ws) * kLn2;
  }
  const uint32_t packed = E::pack2(o, 0.f);
  p.o[(int64_t)b * p.o_sb + (int64_t)h * p.o_sh + d] = (uint16_t)(packed & 0xffffu);
  if (d == 0 && p.lse != nullptr) p.lse[row0] = lse;
}

template <bool BF16, int D>
hipError_t launch_d(const DecParams& p, bool softcap, hipStream_t stream) {
  const dim3 grid(p.n_split, ((p.h_kv + p.hpw - 1) / p.hpw) * p.n_hg, p.batch);
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
