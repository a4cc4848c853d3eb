// KV-cache decode: one query token per sequence against cache_seqlens[b] cached
// keys (Inference Cookbook FAQ Q17), split over the key axis (FAQ Q14's
// num_splits) and merged by log-sum-exp.
//
// Kernel 1 (decode_kernel), one work group per (split, group of NH adjacent KV
// heads [x group of 16 query heads], batch entry):
// - NH adjacent KV heads make a contiguous piece of up to 2 KiB of every key
//   row (all 8 heads at d = 128), so the work group streams long contiguous
//   runs of the cache (measured for a plain read of that layout: about 6.1 TB/s
//   for 2 KiB pieces, 5.8 for 512 B, 5.4 for 256 B);
// - each step covers KSTEP keys of all NH heads; K and V go by DMA
//   (buffer_load ... lds, every instruction 1 KiB of consecutive bytes) into
//   one of two LDS stages, so the next step's loads are in flight while the
//   current step is computed.  16-byte chunks are XOR-swizzled per key row so
//   the operand reads below are free of bank conflicts;
// - a wave owns HPWV heads and one 16-key sub-block of each step (WPH waves
//   share a head when NH is small; they merge (m, l, O) through LDS at the end);
// - the query heads that share a KV head are the 16 columns of the MFMAs, so
//   each K/V byte is read from HBM once for all of them (grouped heads, FAQ
//   Q15): S^T = K Q^T with v_mfma_f32_16x16x32 (K rows read from LDS, Q^T in
//   registers); the accumulator of lane (query n, group g) holds keys 4g..4g+3,
//   which rounded to 16 bits is directly the B operand of O^T = V^T P^T with
//   v_mfma_f32_16x16x16, whose V^T operand is one transposing LDS read
//   (ds_read_b64_tr_b16) of V stored in its natural layout;
// - per query: online softmax in the log2 domain (p = 2^(s * scale * log2 e - m));
// - the split writes either the final O/LSE (one split) or fp32 partials to the
//   workspace.
// Kernel 2 (combine_kernel): LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s -
// LSE) O_s, the merge of partial softmax results ("FlashAttention完整说明",
// section 二.1); a split with no keys has LSE_s = -inf and weight 0.  One
// wave per (row, 64 head dims), so the partials are read by many CUs at once.
#include <mutex>
#include <vector>

#include "device_common.h"
#include "kernels.h"

namespace exattn {
namespace {

// Waves per work group for head dim D (one work group per CU: two LDS stages
// of 64 KiB).
template <int D>
struct DecCfg {
  static constexpr int NW = D == 256 ? 4 : 8;
};

// Stored position of 16-byte chunk c of K-tile row `key`: c ^ kswz(key).  A
// ds_read_b128 pass serves 16 lanes, here 16 consecutive keys of one chunk
// column of one head; key rows are whole multiples of 256 bytes apart, so the
// 16 stored chunks must be distinct modulo 16: key & 15 when a head's row has
// 16 chunks or more (d >= 128; key & 7 left keys k and k + 8 in one bank group,
// measured as 28% of the LDS busy cycles being bank conflicts).  At d = 64 a
// head's row has 8 chunks and keeps key & 7.
template <int D>
__device__ __forceinline__ int kswz(int key) { return D >= 128 ? key & 15 : key & 7; }

// Stored position of chunk c of V-tile row `key`: c ^ vswz(key).  A transposing
// read takes 8 bytes from each of 4 consecutive keys x 2 chunks per 16 lanes;
// even offsets keep those 8 chunks apart (and 16 for 8 keys when d >= 128).
template <int D>
__device__ __forceinline__ int vswz(int key) { return D >= 128 ? 2 * (key & 7) : 2 * (key & 3); }

// 16 bytes per lane from a buffer into LDS at lds + 16 * lane (lds
// wave-uniform).  The buffer starts at base and holds `bytes` bytes: raw buffer
// loads past its end return zeros (a per-dword range check), which covers the
// last step's missing rows; word 3 is the gfx9 default.  Issued from inline
// asm so that the compiler does not track it: it cannot tell which ring slot
// a load writes, and tracked, every LDS read after it would wait for all of
// them.  The kernel waits with explicit vmcnt counts before its barriers.
__device__ __forceinline__ void dma16(const uint16_t* base, int64_t bytes, uint8_t* lds, uint32_t voffset) {
  const uint64_t a = (uint64_t)base;
  const u32x4_t rsrc = {(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, (uint32_t)bytes, 0x00020000u};
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voffset), "s"(rsrc)
               : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <bool BF16, int D, bool SOFTCAP, int HPWV, bool PAGED>
__global__ void __launch_bounds__(DecCfg<D>::NW * 64) decode_kernel(const DecParams p) {
  using E = Elem<BF16>;
  constexpr int NW = DecCfg<D>::NW;
  constexpr int KTILE = 16 * NW * HPWV * 2 * D;  // bytes of the K (or V) tile of one step
  constexpr int NSLOT = 5;                       // ring of K / V tiles: a step's two, three in flight
  constexpr int KS = D / 32;                     // k-steps of S^T = K Q^T over head_dim
  constexpr int DT = D / 16;                     // 16-column tiles of O^T
  constexpr int KI = KTILE / (NW * 1024);        // DMA instructions per wave per tile
  constexpr int MERGE = NW * (2 * 64 + DT * 4 * 64) * 4;
  constexpr int SMEM = NSLOT * KTILE > MERGE ? NSLOT * KTILE : MERGE;
  static_assert(KI >= 1 && KTILE % (NW * 1024) == 0, "tile / wave mismatch");
  static_assert(SMEM <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
  prefetch_kernargs<sizeof(DecParams)>();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g16 = lane >> 4;
  const int l16 = lane & 15;

  const int split = blockIdx.x;
  const int hgrp = blockIdx.y / p.n_hg;
  const int hg = blockIdx.y % p.n_hg;
  const int b = blockIdx.z;
  const int NH = p.hpw;                 // adjacent KV heads of the work group (power of two)
  const int WPH = NW * HPWV / NH;       // waves per head slot
  const int KSTEP = 16 * WPH;           // keys per step
  const int R = NH * 2 * D;             // bytes of one key row of the tile
  const int slot = wave / WPH;          // this wave's heads: slot * HPWV ..
  const int sub = wave % WPH;           // this wave's 16-key sub-block of a step
  const int hk0 = hgrp * NH;
  const int nh_valid = min(NH, p.h_kv - hk0);

  // cache_seqlens[b] is clamped to [0, s_cache] so a bad entry cannot address
  // memory outside the cache.
  const int nk = p.cache_seqlens != nullptr ? min(max(p.cache_seqlens[b] + p.seq_add, 0), p.s_cache)
                                            : p.s_cache;
  // Query token t sits at position nk - s_q + t (bottom-right); keys before
  // the first token's left window edge are never needed.  A paged cache starts
  // the steps on a multiple of the step size, so that a step never straddles a
  // page, and masks the keys before kb_w.
  constexpr bool paged = PAGED;  // p.block_table != nullptr
  const int kb_w = p.wl >= 0 ? max(0, nk - p.s_q - p.wl) : 0;
  const int kb = paged ? kb_w - kb_w % KSTEP : kb_w;
  const int nsteps = nk > kb ? (nk - kb + KSTEP - 1) / KSTEP : 0;
  const int per = (nsteps + p.n_split - 1) / p.n_split;
  const int s_lo = split * per;
  const int s_hi = min(nsteps, s_lo + per);

  const uint16_t* kg = p.k + (int64_t)b * p.k_sb + (int64_t)hk0 * p.k_sh;
  const uint16_t* vg = p.v + (int64_t)b * p.v_sb + (int64_t)hk0 * p.v_sh;

  // ---- DMA lane offsets: instruction t of this wave fills tile bytes
  // (wave + NW t) * 1024 + 16 lane = row key, head, stored chunk pos; it fetches
  // global chunk pos ^ swizzle(key).  Loop-invariant (token and head strides
  // are checked on the host).
  uint32_t kofs[KI], vofs[KI];
#pragma unroll
  for (int t = 0; t < KI; ++t) {
    const int o = (wave + NW * t) * 1024 + 16 * lane;
    const int key = o / R, rem = o % R;
    const int head = rem / (2 * D), pos = (rem % (2 * D)) / 16;
    kofs[t] = (uint32_t)((key * p.k_ss + head * p.k_sh) * 2 + 16 * (pos ^ kswz<D>(key)));
    vofs[t] = (uint32_t)((key * p.v_ss + head * p.v_sh) * 2 + 16 * (pos ^ vswz<D>(key)));
  }
  // Page of the cache row `key` (paged cache), clamped to the pool.  The table
  // is read through the constant address space: a scalar load, whose wait is
  // separate from the DMA's (a vector load would need the DMA count drained
  // before its value could move to a scalar register).
  const __attribute__((address_space(4))) int32_t* bt =
      (const __attribute__((address_space(4))) int32_t*)p.block_table;
  auto page_of = [&](int key) {
    const int pg = bt[(int64_t)b * p.bt_stride + key / p.page_size];
    return min(max(pg, 0), p.num_pages - 1);
  };
  // DMA of step st's K (V) tile into the ring slot at dst; pg: its page if
  // paged.  The descriptor covers the step's rows of the work group's heads.
  auto issue_k = [&](int st, uint8_t* dst, int pg) {
    const int kbase = kb + st * KSTEP;
    const int nrows = min(nk - kbase, KSTEP);
    const uint16_t* k0 = kg + (int64_t)kbase * p.k_ss;
    if (paged) k0 = p.k + (int64_t)pg * p.k_sp + (int64_t)(kbase % p.page_size) * p.k_ss + (int64_t)hk0 * p.k_sh;
    const int64_t bytes = ((int64_t)(nrows - 1) * p.k_ss + (int64_t)(nh_valid - 1) * p.k_sh + D) * 2;
#pragma unroll
    for (int t = 0; t < KI; ++t) dma16(k0, bytes, dst + (wave + NW * t) * 1024, kofs[t]);
  };
  auto issue_v = [&](int st, uint8_t* dst, int pg) {
    const int kbase = kb + st * KSTEP;
    const int nrows = min(nk - kbase, KSTEP);
    const uint16_t* v0 = vg + (int64_t)kbase * p.v_ss;
    if (paged) v0 = p.v + (int64_t)pg * p.v_sp + (int64_t)(kbase % p.page_size) * p.v_ss + (int64_t)hk0 * p.v_sh;
    const int64_t bytes = ((int64_t)(nrows - 1) * p.v_ss + (int64_t)(nh_valid - 1) * p.v_sh + D) * 2;
#pragma unroll
    for (int t = 0; t < KI; ++t) dma16(v0, bytes, dst + (wave + NW * t) * 1024, vofs[t]);
  };
  // ring slot of tile i (step s_lo + i / 2, K for even i, V for odd)
  auto slot_of = [&](int i) { return smem + (i % NSLOT) * KTILE; };

  // the first step's DMA goes out before the Q loads (with an append it waits
  // for the new rows, below)
  // (tiles 0-2: K and V of step s_lo and K of step s_lo + 1)
  const bool early = p.seq_add == 0 && s_lo < s_hi;
  auto prologue = [&]() {
    const int pg0 = paged ? page_of(kb + s_lo * KSTEP) : 0;
    issue_k(s_lo, slot_of(0), pg0);
    issue_v(s_lo, slot_of(1), pg0);
    if (s_lo + 1 < s_hi) issue_k(s_lo + 1, slot_of(2), paged ? page_of(kb + (s_lo + 1) * KSTEP) : 0);
  };
  if (early) prologue();

  // ---- Q^T fragments (B operand): lane (query column l16, group g16) holds
  // Q[head][32 ks + 8 g16 .. + 7] of query head hk * group + hg * 16 + l16.
  // query column of this lane: token qt, query head qj of the group
  const int qc = hg * 16 + l16;
  const bool col_valid = qc < p.s_q * p.group;
  const int qt = qc / p.group, qj = qc - qt * p.group;
  u32x4_t qf[HPWV][KS];
  bool hvalid[HPWV];
#pragma unroll
  for (int i = 0; i < HPWV; ++i) {
    const int hh = slot * HPWV + i;
    hvalid[i] = hh < nh_valid;
    const bool qv = hvalid[i] && col_valid;
    const uint16_t* qp =
        p.q + (int64_t)b * p.q_sb + (int64_t)qt * p.q_ss + (int64_t)((hk0 + hh) * p.group + qj) * p.q_sh +
        8 * g16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[i][ks] = qv ? *(const u32x4_t*)(qp + 32 * ks) : u32x4_t{0, 0, 0, 0};
  }
  // Consume Q here: the compiler then waits for these loads before the loop
  // instead of, conservatively, inside every step behind the step's DMA.
#pragma unroll
  for (int i = 0; i < HPWV; ++i)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[i][ks]));

  // ---- this lane's visible keys [k_lo, k_hi] (its token's causal / window band)
  const int qpos = nk - p.s_q + qt;
  const int k_hi = p.wr >= 0 ? min(nk - 1, qpos + p.wr) : nk - 1;
  const int k_lo = p.wl >= 0 ? max(kb_w, qpos - p.wl) : kb_w;

  // ---- loop-invariant LDS operand offsets within a stage.
  const int krow = 16 * sub + l16;                      // K A-operand row (key in the tile)
  const int vkey = 16 * sub + 4 * g16 + (l16 >> 2);     // V row this lane addresses
  const int vd = 4 * (l16 & 3);                         // first of its 4 columns in a 16-column tile
  const int kaddr0 = krow * R;
  const int vaddr0 = vkey * R + 2 * (vd & 7);

  f32x4_t oacc[HPWV][DT];
  float m_run[HPWV], l_run[HPWV];
#pragma unroll
  for (int i = 0; i < HPWV; ++i) {
    m_run[i] = kNegInf;
    l_run[i] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[i][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // One step: compute step st from its K and V tiles (kt, vt).
  auto step = [&](const uint8_t* __restrict__ kt, const uint8_t* __restrict__ vt, int st) {
    const int key0 = kb + st * KSTEP + 16 * sub;  // first key of this wave's sub-block
#pragma unroll
    for (int i = 0; i < HPWV; ++i) {
      if (!hvalid[i]) continue;  // uniform per wave
      const int hoff = (slot * HPWV + i) * 2 * D;
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t a = *(const u32x4_t*)(kt + kaddr0 + hoff + 16 * ((4 * ks + g16) ^ kswz<D>(krow)));
        s = E::mfma16x16x32(a, qf[i][ks], s);
      }
      // lane (query l16, group g16): scores of keys key0 + 4 g16 + r
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (SOFTCAP)
          x[r] = p.cap_out_log2 * tanh_exp2(s[r] * p.cap_in);
        else
          x[r] = s[r] * p.scale_log2;
        const int key = key0 + 4 * g16 + r;
        if (key > k_hi || key < k_lo) x[r] = kNegInf;
      }
      float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mx = fmaxf(mx, xor16(mx));
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run[i], mx);
      const float base = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[i] - base);  // 0 while nothing was seen
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = fast_exp2(x[r] - base);
      l_run[i] = l_run[i] * alpha + ((x[0] + x[1]) + (x[2] + x[3]));
      m_run[i] = m_new;
      u32x2_t pf;
      pf[0] = E::pack2(x[0], x[1]);
      pf[1] = E::pack2(x[2], x[3]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u32x2_t a = lds_read_tr16(vt + vaddr0 + hoff + 16 * ((2 * dt + (vd >> 3)) ^ vswz<D>(vkey)));
        oacc[i][dt] = E::mfma16x16x16(a, pf, oacc[i][dt] * alpha);
      }
    }
  };

  // ---- append (FAQ Q17): the new tokens go to cache rows cache_seqlens[b] + t
  // before they are attended.  Each work group writes the new rows of its own
  // KV heads that fall in its own key range (split 0 also those left of the
  // window), so every row is read only by work groups that wrote it
  // themselves: a wait for the stores and the barrier order them before the
  // DMA.  Work groups for other query heads of the same KV heads write the
  // same bytes.
  if (p.seq_add > 0) {  // uniform
    const int base = p.cache_seqlens[b];
    const int lo = kb + s_lo * KSTEP, hi = kb + s_hi * KSTEP;
    constexpr int CPR = D / 8;  // 16-byte chunks per head row
    const int n = nh_valid * CPR;
    uint16_t* kw = const_cast<uint16_t*>(kg);
    uint16_t* vw = const_cast<uint16_t*>(vg);
    // K / V row `pos` of this work group's first head
    auto row_k = [&](int pos) {
      if (!paged) return kw + (int64_t)pos * p.k_ss;
      return const_cast<uint16_t*>(p.k) + (int64_t)page_of(pos) * p.k_sp +
             (int64_t)(pos % p.page_size) * p.k_ss + (int64_t)hk0 * p.k_sh;
    };
    auto row_v = [&](int pos) {
      if (!paged) return vw + (int64_t)pos * p.v_ss;
      return const_cast<uint16_t*>(p.v) + (int64_t)page_of(pos) * p.v_sp +
             (int64_t)(pos % p.page_size) * p.v_ss + (int64_t)hk0 * p.v_sh;
    };
    for (int idx = tid; idx < p.seq_add * 2 * n; idx += NW * 64) {
      const int t = idx / (2 * n);
      const int c = idx - t * 2 * n;
      const int pos = base + t;
      const bool mine =
          pos >= 0 && pos < p.s_cache && ((pos >= lo && pos < hi) || (split == 0 && pos < kb));
      if (!mine) continue;
      const bool is_v = c >= n;
      const int cc = is_v ? c - n : c;
      const int hh = cc / CPR, j = cc - hh * CPR;
      const int64_t hd = (int64_t)(hk0 + hh);
      const uint16_t* src =
          is_v ? p.v_new + (int64_t)b * p.vn_sb + (int64_t)t * p.vn_ss + hd * p.vn_sh
               : p.k_new + (int64_t)b * p.kn_sb + (int64_t)t * p.kn_ss + hd * p.kn_sh;
      uint16_t* dst = is_v ? row_v(pos) + (int64_t)hh * p.v_sh : row_k(pos) + (int64_t)hh * p.k_sh;
      *(u32x4_t*)(dst + 8 * j) = *(const u32x4_t*)(src + 8 * j);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  if (s_lo < s_hi && !early) prologue();
  // pages of steps st + 1 and st + 2, read ahead by scalar loads
  int pg1 = paged && s_lo + 1 < s_hi ? page_of(kb + (s_lo + 1) * KSTEP) : 0;
  int pg2 = paged && s_lo + 2 < s_hi ? page_of(kb + (s_lo + 2) * KSTEP) : 0;
  for (int st = s_lo; st < s_hi; ++st) {
    // Tiles 2r, 2r + 1 (step st) have landed once only this wave's K load of
    // step st + 1 may still be in flight; after the barrier every wave is done
    // with step st - 1, whose two slots take V of step st + 1 and K of st + 2.
    const int r = st - s_lo;
    if (st + 1 < s_hi)
      wait_vmcnt<KI>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if (st + 1 < s_hi) issue_v(st + 1, slot_of(2 * r + 3), pg1);
    if (st + 2 < s_hi) issue_k(st + 2, slot_of(2 * r + 4), pg2);
    if (paged) {
      pg1 = pg2;
      if (st + 3 < s_hi) pg2 = page_of(kb + (st + 3) * KSTEP);
    }
    step(slot_of(2 * r), slot_of(2 * r + 1), st);
  }

  // ---- row sums over the four lane groups; merge the waves of a head slot.
  float l_tot[HPWV];
#pragma unroll
  for (int i = 0; i < HPWV; ++i) {
    l_tot[i] = l_run[i] + xor16(l_run[i]);
    l_tot[i] += xor32(l_tot[i]);
  }
  if (WPH > 1) {  // HPWV == 1 here
    __syncthreads();  // the stages are free
    float* xm = reinterpret_cast<float*>(smem);  // [wave][lane]
    float* xl = xm + NW * 64;
    float* xo = xl + NW * 64;  // [wave][dt][r][lane]
    xm[wave * 64 + lane] = m_run[0];
    xl[wave * 64 + lane] = l_tot[0];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) xo[((wave * DT + dt) * 4 + r) * 64 + lane] = oacc[0][dt][r];
    __syncthreads();
    if (sub != 0) return;
    float mm = kNegInf;
    for (int w = wave; w < wave + WPH; ++w) mm = fmaxf(mm, xm[w * 64 + lane]);
    const float bm = mm == kNegInf ? 0.f : mm;
    float lt = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[0][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int w = wave; w < wave + WPH; ++w) {
      const float a = fast_exp2(xm[w * 64 + lane] - bm);  // 0 for a wave that saw nothing
      lt += a * xl[w * 64 + lane];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[0][dt][r] += a * xo[((w * DT + dt) * 4 + r) * 64 + lane];
    }
    m_run[0] = mm;
    l_tot[0] = lt;
  }

  // ---- outputs: lane (query l16, group g16) holds O^T[16 dt + 4 g16 + r][l16].
#pragma unroll
  for (int i = 0; i < HPWV; ++i) {
    if (!hvalid[i] || !col_valid) continue;
    const int h = (hk0 + slot * HPWV + i) * p.group + qj;
    const bool empty = !(l_tot[i] > 0.f);
    const float inv = empty ? 0.f : 1.0f / l_tot[i];
    const float lse = empty ? kNegInf : (m_run[i] + fast_log2(l_tot[i])) * kLn2;
    if (p.n_split == 1) {
      uint16_t* op = p.o + (int64_t)b * p.o_sb + (int64_t)qt * p.o_ss + (int64_t)h * p.o_sh + 4 * g16;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        u32x2_t w2;
        w2[0] = E::pack2(oacc[i][dt][0] * inv, oacc[i][dt][1] * inv);
        w2[1] = E::pack2(oacc[i][dt][2] * inv, oacc[i][dt][3] * inv);
        *(u32x2_t*)(op + 16 * dt) = w2;
      }
      if (g16 == 0 && p.lse != nullptr) p.lse[((int64_t)b * p.h_q + h) * p.s_q + qt] = lse;
    } else {
      const int64_t row = (((int64_t)split * p.batch + b) * p.s_q + qt) * p.h_q + h;
      float* wo = p.ws_o + row * D + 4 * g16;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *(f32x4_t*)(wo + 16 * dt) = oacc[i][dt] * inv;
      if (g16 == 0) p.ws_lse[row] = lse;
    }
  }
}


// Thread t of a work group owns 4 columns of one (batch, query head) row: 256
// threads cover 1024 / D rows.  The splits are taken 32 at a time with all
// their loads issued together and merged with a running maximum, so a call
// with up to 32 splits waits for one round trip to memory.
constexpr int kCombineThreads = 64;

// One wave per (row, 64 head dims): lane = (split group sg = lane / 16, column
// quad c = lane % 16).  Split group sg takes splits sg, sg + 4, ...; all its
// loads go out together, the four groups merge by log-sum-exp through two
// lane exchanges, and group 0 writes.  Rows x D/64 work groups, so every CU
// gets some of the 4 MB of partials and each lane waits for one round trip.
template <bool BF16, int D>
__global__ void __launch_bounds__(kCombineThreads) combine_kernel(const DecParams p) {
  using E = Elem<BF16>;
  const int row = blockIdx.x / (D / 64);
  const int cb = blockIdx.x % (D / 64);
  const int lane = threadIdx.x;
  const int sg = lane >> 4;
  const int col = 64 * cb + 4 * (lane & 15);
  const int rows = p.batch * p.s_q * p.h_q;  // (b, token, head)
  const int64_t stride = rows;
  constexpr int kU = 16;  // splits per group per pass
  float m = kNegInf, ws = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < p.n_split; s0 += 4 * kU) {
    float l[kU];
    f32x4_t v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int s = s0 + sg + 4 * u;
      const bool in = s < p.n_split;
      const int64_t r = (int64_t)s * stride + row;
      l[u] = in ? p.ws_lse[r] : kNegInf;
      v[u] = in ? *(const f32x4_t*)(p.ws_o + r * D + col) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    float mb = l[0];
#pragma unroll
    for (int u = 1; u < kU; ++u) mb = fmaxf(mb, l[u]);
    if (mb > m) {
      const float sc = m == kNegInf ? 0.f : fast_exp2((m - mb) * kLog2e);
      ws *= sc;
      acc *= sc;
      m = mb;
    }
    if (m != kNegInf) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float w = fast_exp2((l[u] - m) * kLog2e);
        ws += w;
        acc += w * v[u];
      }
    }
  }
  // merge the four split groups (lanes c, c + 16, c + 32, c + 48)
#pragma unroll
  for (int sh = 16; sh <= 32; sh *= 2) {
    const float m2 = __shfl_xor(m, sh, 64);
    const float w2 = __shfl_xor(ws, sh, 64);
    f32x4_t a2;
#pragma unroll
    for (int e = 0; e < 4; ++e) a2[e] = __shfl_xor(acc[e], sh, 64);
    const float mm = fmaxf(m, m2);
    const float bm = mm == kNegInf ? 0.f : mm;
    const float f1 = fast_exp2((m - bm) * kLog2e), f2 = fast_exp2((m2 - bm) * kLog2e);
    ws = ws * f1 + w2 * f2;
    acc = acc * f1 + a2 * f2;
    m = mm;
  }
  if (sg != 0) return;
  const float inv = m != kNegInf ? 1.0f / ws : 0.f;
  const int h = row % p.h_q, bt = row / p.h_q;
  const int t = bt % p.s_q, b = bt / p.s_q;
  u32x2_t w2;
  w2[0] = E::pack2(acc[0] * inv, acc[1] * inv);
  w2[1] = E::pack2(acc[2] * inv, acc[3] * inv);
  *(u32x2_t*)(p.o + (int64_t)b * p.o_sb + (int64_t)t * p.o_ss + (int64_t)h * p.o_sh + col) = w2;
  if (cb == 0 && lane == 0 && p.lse != nullptr)
    p.lse[((int64_t)b * p.h_q + h) * p.s_q + t] = m != kNegInf ? m + fast_log2(ws) * kLn2 : kNegInf;
}

template <bool BF16, int D, int HPWV>
hipError_t launch_h(const DecParams& p, bool softcap, hipStream_t stream) {
  const dim3 grid(p.n_split, ((p.h_kv + p.hpw - 1) / p.hpw) * p.n_hg, p.batch);
  const dim3 block(DecCfg<D>::NW * 64);
  const bool paged = p.block_table != nullptr;
  if (softcap && paged)
    hipLaunchKernelGGL((decode_kernel<BF16, D, true, HPWV, true>), grid, block, 0, stream, p);
  else if (softcap)
    hipLaunchKernelGGL((decode_kernel<BF16, D, true, HPWV, false>), grid, block, 0, stream, p);
  else if (paged)
    hipLaunchKernelGGL((decode_kernel<BF16, D, false, HPWV, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((decode_kernel<BF16, D, false, HPWV, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_d(const DecParams& p, bool softcap, hipStream_t stream) {
  // a wave owns two heads only when d = 64 and a work group covers 16 heads
  hipError_t e;
  if constexpr (D == 64)
    e = p.hpw == 16 ? launch_h<BF16, D, 2>(p, softcap, stream) : launch_h<BF16, D, 1>(p, softcap, stream);
  else
    e = launch_h<BF16, D, 1>(p, softcap, stream);
  if (e != hipSuccess || p.n_split == 1) return e;
  hipLaunchKernelGGL((combine_kernel<BF16, D>), dim3(p.batch * p.s_q * p.h_q * (D / 64)),
                     dim3(kCombineThreads), 0, stream, p);
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

// Static scratch for the split partials of exattn_decode_noalloc: device memory
// the library holds on every device it runs on, for callers that cannot
// allocate.  In host code `scratch` names a host-side stand-in, not a device
// address: its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device; nullptr = not looked up yet

}  // namespace

hipError_t launch_decode(const DecParams& p, bool bf16, int head_dim, bool softcap,
                         hipStream_t stream) {
  return bf16 ? launch_t<true>(p, head_dim, softcap, stream)
              : launch_t<false>(p, head_dim, softcap, stream);
}

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (g_scratch_ptr[dev] == nullptr) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));  // the current device's copy
    if (e != hipSuccess) return e;
    if (addr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = addr;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace exattn
