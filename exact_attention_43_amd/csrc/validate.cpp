// Host-side argument checks and launch planning (no HIP dependency).
#include "validate.h"

#include <float.h>
#include <math.h>

#include <algorithm>
#include <string>
#include <vector>

namespace exattn {
namespace {

thread_local std::string g_error;

constexpr float kLog2eHost = 1.4426950408889634f;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

bool stride_ok(int64_t s) { return s >= 0 && s % 8 == 0; }

std::string str(int64_t v) { return std::to_string(v); }

// The kernels address one tile of `rows` consecutive tokens (and `heads`
// adjacent heads) with 32-bit byte offsets from the tile's first element
// (DMA lane offsets, buffer-descriptor ranges).  The span from the tile's first
// byte to the end of its last row must stay below 2^31 bytes.
exattn_status check_span(const char* name, int64_t rows, int64_t token_stride, int64_t heads,
                         int64_t head_stride, int64_t head_dim, int64_t elem_bytes) {
  // 128-bit: the strides are only known to be non-negative multiples of 8
  const __int128 span =
      ((__int128)(rows - 1) * token_stride + (__int128)(heads - 1) * head_stride + head_dim) * elem_bytes;
  if (span >= ((__int128)1 << 31))
    return fail(EXATTN_E_UNSUPPORTED,
                std::string(name) + ": a tile of " + str(rows) +
                    " tokens spans 2^31 bytes or more with these strides, beyond the kernels' 32-bit offsets");
  return EXATTN_OK;
}

exattn_status check_common(int32_t dtype, int32_t head_dim, int32_t heads_q, int32_t heads_kv,
                           int32_t batch) {
  if (dtype != EXATTN_F16 && dtype != EXATTN_BF16)
    return fail(EXATTN_E_UNSUPPORTED,
                "dtype " + str(dtype) + " is not supported: inputs must be fp16 or bf16");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(EXATTN_E_UNSUPPORTED,
                "head_dim " + str(head_dim) + " is not supported (64, 128 or 256)");
  if (batch < 0) return fail(EXATTN_E_INVALID, "batch is negative");
  if (heads_q < 1 || heads_kv < 1) return fail(EXATTN_E_INVALID, "heads must be >= 1");
  if (heads_q % heads_kv != 0)
    return fail(EXATTN_E_INVALID, "heads_q (" + str(heads_q) + ") is not a multiple of heads_kv (" +
                                      str(heads_kv) + ")");
  return EXATTN_OK;
}

exattn_status resolve_scales(float softmax_scale, float softcap, int head_dim, float* scale_log2,
                             float* cap_in, float* cap_out_log2, bool* use_cap) {
  // NaN selects the default 1/sqrt(head_dim); every other finite value, 0
  // included (all scores 0: uniform weights over the visible keys), is used as
  // given.
  float scale = softmax_scale;
  if (isnan(scale)) scale = 1.0f / sqrtf((float)head_dim);
  if (!isfinite(scale)) return fail(EXATTN_E_INVALID, "softmax_scale is not finite");
  if (isnan(softcap) || isinf(softcap)) return fail(EXATTN_E_INVALID, "softcap is not finite");
  *use_cap = softcap > 0.0f;
  *scale_log2 = scale * kLog2eHost;
  *cap_in = *use_cap ? scale / softcap : 0.0f;
  *cap_out_log2 = *use_cap ? softcap * kLog2eHost : 0.0f;
  return EXATTN_OK;
}

}  // namespace

// Window edges as the kernels take them: < 0 unbounded, causal forces the
// right edge to 0.  An edge that reaches past every key of every row (left >=
// keys, right >= query rows) bounds nothing and is taken as unbounded: the
// kernels add the edges to row and key positions in 32 bits.
void window_edges(int32_t left, int32_t right, int32_t causal, int64_t rows, int64_t keys, int* wl,
                  int* wr) {
  *wl = left < 0 || left >= keys ? -1 : left;
  *wr = causal ? 0 : (right < 0 || right >= rows ? -1 : right);
}

exattn_status fail(exattn_status st, const std::string& msg) {
  g_error = msg;
  return st;
}

void clear_error() { g_error.clear(); }

const char* last_error() { return g_error.c_str(); }

exattn_status plan_fwd(const exattn_fwd_args* a, int rows_per_tile, FwdPlan* pl) {
  if (a == nullptr || pl == nullptr) return fail(EXATTN_E_INVALID, "args is NULL");
  *pl = FwdPlan{};
  exattn_status st = check_common(a->dtype, a->head_dim, a->heads_q, a->heads_kv, a->batch);
  if (st != EXATTN_OK) return st;
  const bool varlen = a->cu_seqlens_q != nullptr;
  if (varlen != (a->cu_seqlens_k != nullptr))
    return fail(EXATTN_E_INVALID, "cu_seqlens_q and cu_seqlens_k must both be set or both NULL");
  int s_q, s_k;
  if (varlen) {
    if (a->max_seqlen_q < 0 || a->max_seqlen_k < 0)
      return fail(EXATTN_E_INVALID, "max_seqlen_q / max_seqlen_k is negative");
    s_q = a->max_seqlen_q;
    s_k = a->max_seqlen_k;
  } else {
    if (a->seqlen_q < 0 || a->seqlen_k < 0)
      return fail(EXATTN_E_INVALID, "seqlen_q / seqlen_k is negative");
    s_q = a->seqlen_q;
    s_k = a->seqlen_k;
  }
  st = resolve_scales(a->softmax_scale, a->softcap, a->head_dim, &pl->scale_log2, &pl->cap_in,
                      &pl->cap_out_log2, &pl->softcap);
  if (st != EXATTN_OK) return st;
  // The prefill kernel takes its row max on raw scores and scales afterwards,
  // which needs a positive scale: a negative one is applied by negating Q.
  pl->q_sign = 0u;
  if (pl->scale_log2 < 0.0f) {
    pl->q_sign = 0x80008000u;
    pl->scale_log2 = -pl->scale_log2;
    pl->cap_in = -pl->cap_in;
  }
  // It also masks raw scores (-inf) before scaling, and -inf * 0 is NaN: a zero
  // scale is applied as the smallest normal float, whose products with finite
  // scores are so small that every exponential is exactly 1, as for scale 0.
  if (pl->scale_log2 == 0.0f) pl->scale_log2 = FLT_MIN;

  pl->bf16 = a->dtype == EXATTN_BF16;
  pl->head_dim = a->head_dim;
  pl->varlen = varlen;
  pl->s_q = s_q;
  pl->s_k = s_k;
  pl->group = a->heads_q / a->heads_kv;
  window_edges(a->window_left, a->window_right, a->causal, s_q, s_k, &pl->wl, &pl->wr);
  pl->empty = a->batch == 0 || s_q == 0;
  if (pl->empty) return EXATTN_OK;

  if (a->q == nullptr || a->o == nullptr) return fail(EXATTN_E_INVALID, "q or o is NULL");
  if (s_k > 0 && (a->k == nullptr || a->v == nullptr))
    return fail(EXATTN_E_INVALID, "k or v is NULL");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return fail(EXATTN_E_INVALID, "q, k, v and o must be 16-byte aligned");
  const int64_t* strides[4] = {a->q_stride, a->k_stride, a->v_stride, a->o_stride};
  const char* names[4] = {"q", "k", "v", "o"};
  for (int t = 0; t < 4; ++t) {
    for (int i = varlen ? 1 : 0; i < 3; ++i)
      if (!stride_ok(strides[t][i]))
        return fail(EXATTN_E_INVALID, std::string(names[t]) + "_stride[" + str(i) + "] = " +
                                          str(strides[t][i]) +
                                          " must be a non-negative multiple of 8 elements");
  }
  // The kernels address 64 rows of a tile with 32-bit byte offsets from the
  // tile's first row (DMA offsets, buffer descriptor ranges).
  for (int t = 0; t < 3; ++t)
    if (strides[t][1] >= ((int64_t)1 << 24))
      return fail(EXATTN_E_UNSUPPORTED, std::string(names[t]) + "_stride[1] = " + str(strides[t][1]) +
                                            " exceeds the supported token stride (2^24 elements)");
  if (a->lse != nullptr) {
    if ((reinterpret_cast<uintptr_t>(a->lse) & 3u) != 0)
      return fail(EXATTN_E_INVALID, "lse must be 4-byte aligned");
    if (a->lse_stride[1] < 0 || (!varlen && a->lse_stride[0] < 0))
      return fail(EXATTN_E_INVALID, "lse strides must be non-negative");
  }
  if (varlen && a->batch > 0 && (a->cu_seqlens_q == nullptr || a->cu_seqlens_k == nullptr))
    return fail(EXATTN_E_INVALID, "cu_seqlens is NULL");

  // Packed GQA (FAQ Q15): one tile holds the rows of all query heads of a KV
  // head.  Automatic: packed when that takes fewer work groups, i.e. when
  // short query sequences leave most rows of the per-head tiles empty.
  if (a->pack_gqa < -1 || a->pack_gqa > 1)
    return fail(EXATTN_E_INVALID, "pack_gqa must be -1 (automatic), 0 or 1");
  const int64_t g = pl->group;
  const int64_t tiles_plain = (int64_t)a->heads_q * (((int64_t)s_q + rows_per_tile - 1) / rows_per_tile);
  const int64_t tiles_packed = (int64_t)a->heads_kv * (((int64_t)s_q * g + rows_per_tile - 1) / rows_per_tile);
  pl->pack = a->pack_gqa == 1 || (a->pack_gqa == -1 && g > 1 && tiles_packed < tiles_plain);
  const bool pack_fits = (int64_t)s_q * g < ((int64_t)1 << 22);  // the kernel's row division
  if (a->pack_gqa == 1 && !pack_fits)
    return fail(EXATTN_E_UNSUPPORTED, "packed GQA takes seqlen_q x (heads_q / heads_kv) below 2^22");
  pl->pack = pl->pack && pack_fits;
  const int64_t rows = pl->pack ? (int64_t)s_q * g : s_q;
  pl->n_qt = (int)((rows + rows_per_tile - 1) / rows_per_tile);
  const int64_t units = (int64_t)a->batch * (pl->pack ? a->heads_kv : a->heads_q);
  const int64_t grid = units * pl->n_qt;
  if (grid > 0x7fffffffLL) return fail(EXATTN_E_INVALID, "problem too large for one launch");
  pl->grid = (int)grid;
  pl->xcd_group = (!pl->pack && pl->group > 1 && ((int64_t)a->batch * a->heads_kv) % 8 == 0) ? 1 : 0;
  return EXATTN_OK;
}

exattn_status plan_fwd_fp8(const exattn_fwd_args* a, const exattn_fp8_descale* d, Fp8Plan* pl) {
  if (a == nullptr || pl == nullptr) return fail(EXATTN_E_INVALID, "args is NULL");
  *pl = Fp8Plan{};
  if (a->dtype != EXATTN_FP8_E4M3)
    return fail(EXATTN_E_UNSUPPORTED, "exattn_fwd_fp8 takes dtype EXATTN_FP8_E4M3, got " + str(a->dtype));
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(EXATTN_E_UNSUPPORTED, "the FP8 forward provides head_dim 64 and 128");
  if (a->batch < 0) return fail(EXATTN_E_INVALID, "batch is negative");
  if (a->heads_q < 1 || a->heads_kv < 1) return fail(EXATTN_E_INVALID, "heads must be >= 1");
  if (a->heads_q % a->heads_kv != 0) return fail(EXATTN_E_INVALID, "heads_q is not a multiple of heads_kv");
  pl->varlen = a->cu_seqlens_q != nullptr;
  if (pl->varlen != (a->cu_seqlens_k != nullptr))
    return fail(EXATTN_E_INVALID, "cu_seqlens_q and cu_seqlens_k must both be set or both NULL");
  if (pl->varlen) {
    if (a->max_seqlen_q < 0 || a->max_seqlen_k < 0)
      return fail(EXATTN_E_INVALID, "max_seqlen_q / max_seqlen_k is negative");
    pl->s_q = a->max_seqlen_q;
    pl->s_k = a->max_seqlen_k;
  } else {
    if (a->seqlen_q < 0 || a->seqlen_k < 0) return fail(EXATTN_E_INVALID, "seqlen_q / seqlen_k is negative");
    pl->s_q = a->seqlen_q;
    pl->s_k = a->seqlen_k;
  }
  float scale_log2, cap_in, cap_out;
  bool cap;
  exattn_status st = resolve_scales(a->softmax_scale, a->softcap, a->head_dim, &scale_log2, &cap_in, &cap_out, &cap);
  if (st != EXATTN_OK) return st;
  float dq = 1.f, dk = 1.f, dv = 1.f;
  if (d != nullptr) dq = d->q, dk = d->k, dv = d->v;
  if (!isfinite(dq) || !isfinite(dk) || !isfinite(dv))
    return fail(EXATTN_E_INVALID, "descale factors must be finite");
  // the kernel's scores are products of the codes: the descales fold into the scale
  pl->scale_log2 = scale_log2 * dq * dk;
  if (!isfinite(pl->scale_log2)) return fail(EXATTN_E_INVALID, "softmax_scale x descales overflows");
  pl->softcap = cap;
  pl->cap_in = cap_in * dq * dk;
  pl->cap_out_log2 = cap_out;
  if (!isfinite(pl->cap_in)) return fail(EXATTN_E_INVALID, "softmax_scale x descales / softcap overflows");
  pl->v_descale = dv;
  pl->head_dim = a->head_dim;
  pl->group = a->heads_q / a->heads_kv;
  window_edges(a->window_left, a->window_right, a->causal, pl->s_q, pl->s_k, &pl->wl, &pl->wr);
  pl->empty = a->batch == 0 || pl->s_q == 0;
  if (pl->empty) return EXATTN_OK;
  if (a->q == nullptr || a->o == nullptr) return fail(EXATTN_E_INVALID, "q or o is NULL");
  if (pl->s_k > 0 && (a->k == nullptr || a->v == nullptr)) return fail(EXATTN_E_INVALID, "k or v is NULL");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return fail(EXATTN_E_INVALID, "q, k, v and o must be 16-byte aligned");
  const int64_t* s8[3] = {a->q_stride, a->k_stride, a->v_stride};
  for (int t = 0; t < 3; ++t)
    for (int i = 0; i < 3; ++i)
      if (s8[t][i] < 0 || s8[t][i] % 16 != 0)
        return fail(EXATTN_E_INVALID, "FP8 q, k, v strides must be non-negative multiples of 16 elements");
  for (int i = 0; i < 3; ++i)
    if (!stride_ok(a->o_stride[i])) return fail(EXATTN_E_INVALID, "o strides must be non-negative multiples of 8");
  // 64-key K / V tiles (and 64-row Q tiles) of one head, 1 byte per element
  const char* n8[3] = {"q", "k", "v"};
  for (int t = 0; t < 3; ++t) {
    st = check_span(n8[t], 64, s8[t][1], 1, 0, a->head_dim, 1);
    if (st != EXATTN_OK) return st;
  }
  if (a->lse != nullptr) {
    if ((reinterpret_cast<uintptr_t>(a->lse) & 3u) != 0) return fail(EXATTN_E_INVALID, "lse must be 4-byte aligned");
    if (a->lse_stride[0] < 0 || a->lse_stride[1] < 0) return fail(EXATTN_E_INVALID, "lse strides must be non-negative");
  }
  const int64_t grid = (int64_t)a->batch * a->heads_q * (((int64_t)pl->s_q + 63) / 64);
  if (grid > 0x7fffffffLL) return fail(EXATTN_E_INVALID, "problem too large for one launch");
  return EXATTN_OK;
}

int decode_heads_per_group(int head_dim, int heads_kv) {
  int hpw = head_dim <= 64 ? 16 : head_dim <= 128 ? 8 : 4;
  while (hpw > 1 && hpw > heads_kv) hpw >>= 1;
  return hpw;
}

int32_t auto_splits(int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t seqlen_k,
                    int32_t head_dim, int32_t num_cus, int32_t seqlen_q) {
  if (batch <= 0 || seqlen_k <= 0 || heads_kv <= 0 || heads_q <= 0 || num_cus <= 0) return 1;
  const int64_t cols = (int64_t)(heads_q / heads_kv) * (seqlen_q > 1 ? seqlen_q : 1);
  const int64_t hpw = decode_heads_per_group(head_dim, heads_kv);
  const int64_t target_wgs = num_cus;  // one work group (two 64 KiB LDS stages) per compute unit
  // work groups without splitting: batch x KV-head groups x 16-column groups
  // (each factor is at least 1; stop as soon as the product reaches the target)
  const int64_t factors[3] = {batch, ((int64_t)heads_kv + hpw - 1) / hpw, (cols + 15) / 16};
  int64_t units = 1;
  for (const int64_t f : factors) {
    if (f < 1) return 1;
    if (units >= (target_wgs + f - 1) / f) return 1;  // units * f >= target_wgs
    units *= f;
  }
  int64_t splits = (target_wgs + units - 1) / units;
  const int64_t by_len = seqlen_k / 256 > 1 ? seqlen_k / 256 : 1;  // >= 256 keys per split
  if (splits > by_len) splits = by_len;
  if (splits > 256) splits = 256;
  return (int32_t)(splits < 1 ? 1 : splits);
}

void tile_key_blocks(int t, int s_q, int s_k, int wl, int wr, int* lo, int* hi) {
  const int64_t r0 = (int64_t)64 * t, r1 = std::min<int64_t>(r0 + 64, s_q) - 1;
  const int64_t off = (int64_t)s_k - s_q;
  int64_t kmin = 0, kmax = (int64_t)s_k - 1;
  if (wl >= 0) kmin = std::max<int64_t>(0, r0 + off - wl);
  if (wr >= 0) kmax = std::min<int64_t>(kmax, r1 + off + wr);
  *lo = 0;
  *hi = 0;
  if (kmax >= kmin) {
    *lo = (int)(kmin / 32);
    *hi = (int)(kmax / 32 + 1);
  }
}

namespace {
// slot entry s: tile t's key group k of kgn (w visible blocks); keeps the step count
void put_slot(SlotSchedule* out, int s, int t, int k, int kgn, int w) {
  out->slot[s] = (uint32_t)t | ((uint32_t)k << 16) | ((uint32_t)kgn << 19) | (1u << 24);
  out->nb[s] = w > k ? (uint32_t)((w - k + kgn - 1) / kgn) : 0u;
  out->steps = std::max(out->steps, (int)out->nb[s]);
}
}  // namespace

bool build_slot_schedule(const int* w, int n64, int wg_max, SlotSchedule* out) {
  *out = SlotSchedule{};
  if (n64 < 1 || wg_max < 1) return false;
  const int max_wg = std::min(wg_max, kMaxSlots / 4);
  if (n64 > 4 * max_wg) return false;
  std::vector<int> kg(n64);
  auto load = [&](int t) { return (w[t] + kg[t] - 1) / kg[t]; };
  // bins of 4 slots, first fit by decreasing kgn (ties: heavier first); returns
  // the bin count and fills bin / position per tile
  std::vector<int> order(n64), bin(n64), pos(n64);
  auto pack = [&]() {
    for (int t = 0; t < n64; ++t) order[t] = t;
    std::stable_sort(order.begin(), order.end(),
                     [&](int x, int y) { return kg[x] != kg[y] ? kg[x] > kg[y] : w[x] > w[y]; });
    std::vector<int> fill;
    for (int t : order) {
      int b = 0;
      while (b < (int)fill.size() && fill[b] + kg[t] > 4) ++b;
      if (b == (int)fill.size()) fill.push_back(0);
      bin[t] = b;
      pos[t] = fill[b];
      fill[b] += kg[t];
    }
    return (int)fill.size();
  };
  // greedy: give a slot to the tile with the largest per-slot load while the
  // slots last, then shrink the budget until the tiles pack into max_wg groups
  for (int budget = 4 * max_wg; budget >= n64; --budget) {
    for (int t = 0; t < n64; ++t) kg[t] = 1;
    int used = n64;
    while (used < budget) {
      int best = -1;
      for (int t = 0; t < n64; ++t)
        if (kg[t] < 4 && w[t] > kg[t] && (best < 0 || load(t) > load(best))) best = t;
      if (best < 0) break;
      ++kg[best];
      ++used;
    }
    const int n_wg = pack();
    if (n_wg > max_wg) continue;
    out->n_wg = n_wg;
    for (int t = 0; t < n64; ++t)
      for (int k = 0; k < kg[t]; ++k) put_slot(out, 4 * bin[t] + pos[t] + k, t, k, kg[t], w[t]);
    return true;
  }
  return false;
}

exattn_status plan_decode(const exattn_decode_args* a, int num_cus, DecodePlan* pl) {
  if (a == nullptr || pl == nullptr) return fail(EXATTN_E_INVALID, "args is NULL");
  *pl = DecodePlan{};
  exattn_status st = check_common(a->dtype, a->head_dim, a->heads_q, a->heads_kv, a->batch);
  if (st != EXATTN_OK) return st;
  if (a->seqlen_cache < 0) return fail(EXATTN_E_INVALID, "seqlen_cache is negative");
  if (a->num_splits < 0) return fail(EXATTN_E_INVALID, "num_splits is negative");
  st = resolve_scales(a->softmax_scale, a->softcap, a->head_dim, &pl->scale_log2, &pl->cap_in,
                      &pl->cap_out_log2, &pl->softcap);
  if (st != EXATTN_OK) return st;
  pl->bf16 = a->dtype == EXATTN_BF16;
  pl->head_dim = a->head_dim;
  if (a->seqlen_q < 0) return fail(EXATTN_E_INVALID, "seqlen_q is negative");
  pl->s_q = a->seqlen_q > 1 ? a->seqlen_q : 1;
  pl->group = a->heads_q / a->heads_kv;
  // MFMA query columns per KV head: every query token of every query head of
  // the group, in groups of 16 (one work group each)
  const int64_t cols = (int64_t)pl->group * pl->s_q;
  if (cols > 16 * 4096) return fail(EXATTN_E_UNSUPPORTED, "seqlen_q x (heads_q / heads_kv) above 65536");
  pl->n_hg = (int)((cols + 15) / 16);
  pl->hpw = decode_heads_per_group(a->head_dim, a->heads_kv);
  pl->n_hk = (int)(((int64_t)a->heads_kv + pl->hpw - 1) / pl->hpw);
  // keys per batch entry are known on the device only: the left edge is kept
  // (the kernel subtracts it), the right edge is bounded by the query tokens
  window_edges(a->window_left, a->window_right, a->causal, pl->s_q, INT64_MAX, &pl->wl, &pl->wr);
  int64_t ns = a->num_splits == 0
                   ? auto_splits(a->batch, a->heads_q, a->heads_kv, a->seqlen_cache, a->head_dim,
                                 num_cus, pl->s_q)
                   : a->num_splits;
  const int64_t chunks = ((int64_t)a->seqlen_cache + 31) / 32;
  if (ns > chunks) ns = chunks;
  if (ns > 256) ns = 256;
  if (ns < 1) ns = 1;
  pl->n_split = (int)ns;
  pl->empty = a->batch == 0;
  if (pl->n_split > 1) {
    const size_t rows = (size_t)pl->n_split * (size_t)a->batch * (size_t)pl->s_q * (size_t)a->heads_q;
    const size_t o_bytes = rows * (size_t)a->head_dim * 4;
    pl->ws_lse_offset = (o_bytes + 255) & ~(size_t)255;
    pl->ws_bytes = (pl->ws_lse_offset + rows * 4 + 255) & ~(size_t)255;
  }
  if (pl->empty) return EXATTN_OK;

  if (a->q == nullptr || a->o == nullptr) return fail(EXATTN_E_INVALID, "q or o is NULL");
  if (a->seqlen_cache > 0 && (a->k_cache == nullptr || a->v_cache == nullptr))
    return fail(EXATTN_E_INVALID, "k_cache or v_cache is NULL");
  if (!aligned16(a->q) || !aligned16(a->k_cache) || !aligned16(a->v_cache) || !aligned16(a->o))
    return fail(EXATTN_E_INVALID, "q, k_cache, v_cache and o must be 16-byte aligned");
  const int64_t s2[6] = {a->q_stride[0], a->q_stride[1], a->o_stride[0], a->o_stride[1],
                         pl->s_q > 1 ? a->q_token_stride : 0, pl->s_q > 1 ? a->o_token_stride : 0};
  for (int i = 0; i < 6; ++i)
    if (!stride_ok(s2[i]))
      return fail(EXATTN_E_INVALID, "q/o strides must be non-negative multiples of 8 elements");
  for (int i = 0; i < 3; ++i)
    if (!stride_ok(a->k_stride[i]) || !stride_ok(a->v_stride[i]))
      return fail(EXATTN_E_INVALID, "k/v strides must be non-negative multiples of 8 elements");
  if (a->lse != nullptr && (reinterpret_cast<uintptr_t>(a->lse) & 3u) != 0)
    return fail(EXATTN_E_INVALID, "lse must be 4-byte aligned");
  // One step's tile: its keys times the work group's adjacent KV heads.
  const int kstep = decode_keys_per_step(a->head_dim, pl->hpw);
  const int span_heads = a->heads_kv < pl->hpw ? a->heads_kv : pl->hpw;
  st = check_span("k_cache", kstep, a->k_stride[1], span_heads, a->k_stride[2], a->head_dim, 2);
  if (st != EXATTN_OK) return st;
  st = check_span("v_cache", kstep, a->v_stride[1], span_heads, a->v_stride[2], a->head_dim, 2);
  if (st != EXATTN_OK) return st;
  if ((int64_t)pl->n_hk * pl->n_hg > 65535 || a->batch > 65535)
    return fail(EXATTN_E_INVALID, "too many heads or batch entries for one launch");
  return EXATTN_OK;
}

exattn_status check_append(const exattn_decode_args* a, const exattn_kv_new* n) {
  if (n == nullptr) return fail(EXATTN_E_INVALID, "kv_new is NULL");
  if (n->seqlen_new < 0) return fail(EXATTN_E_INVALID, "seqlen_new is negative");
  if (n->seqlen_new == 0 || a->batch == 0) return EXATTN_OK;
  if (a->cache_seqlens == nullptr)
    return fail(EXATTN_E_INVALID, "appending needs cache_seqlens (the rows to write at)");
  if (n->seqlen_new > a->seqlen_cache)
    return fail(EXATTN_E_INVALID, "seqlen_new exceeds seqlen_cache");
  if (n->k_new == nullptr || n->v_new == nullptr) return fail(EXATTN_E_INVALID, "k_new or v_new is NULL");
  if (!aligned16(n->k_new) || !aligned16(n->v_new))
    return fail(EXATTN_E_INVALID, "k_new and v_new must be 16-byte aligned");
  for (int i = 0; i < 3; ++i)
    if (!stride_ok(n->k_new_stride[i]) || !stride_ok(n->v_new_stride[i]))
      return fail(EXATTN_E_INVALID, "k_new/v_new strides must be non-negative multiples of 8 elements");
  return EXATTN_OK;
}

exattn_status plan_bwd(const exattn_bwd_args* a, BwdPlan* pl) {
  if (a == nullptr || pl == nullptr) return fail(EXATTN_E_INVALID, "args is NULL");
  *pl = BwdPlan{};
  exattn_status st = check_common(a->dtype, a->head_dim, a->heads_q, a->heads_kv, a->batch);
  if (st != EXATTN_OK) return st;
  const bool varlen = a->cu_seqlens_q != nullptr;
  if (varlen != (a->cu_seqlens_k != nullptr))
    return fail(EXATTN_E_INVALID, "cu_seqlens_q and cu_seqlens_k must both be set or both NULL");
  // lengths (fixed) or the largest sequence (varlen), which size the grids
  const int32_t s_q = varlen ? a->max_seqlen_q : a->seqlen_q;
  const int32_t s_k = varlen ? a->max_seqlen_k : a->seqlen_k;
  if (s_q < 0 || s_k < 0) return fail(EXATTN_E_INVALID, "seqlen_q / seqlen_k (or their maxima) is negative");
  float scale_log2, cap_in, cap_out;
  bool cap;
  st = resolve_scales(a->softmax_scale, a->softcap, a->head_dim, &scale_log2, &cap_in, &cap_out, &cap);
  if (st != EXATTN_OK) return st;
  pl->softcap = cap;
  pl->cap_in = cap_in;
  pl->cap_out_log2 = cap_out;
  pl->varlen = varlen;
  pl->s_q = s_q;
  pl->s_k = s_k;
  pl->bf16 = a->dtype == EXATTN_BF16;
  pl->head_dim = a->head_dim;
  pl->group = a->heads_q / a->heads_kv;
  pl->scale_log2 = scale_log2;
  pl->scale = scale_log2 / kLog2eHost;
  window_edges(a->window_left, a->window_right, a->causal, s_q, s_k, &pl->wl, &pl->wr);
  const size_t rows = (size_t)a->batch * (size_t)a->heads_q * (size_t)s_q;
  pl->ws_bytes = (rows * 8 + 255) & ~(size_t)255;  // (LSE log2 e, dO . O) per row
  pl->empty = a->batch == 0 || (s_q == 0 && s_k == 0);
  if (pl->empty) return EXATTN_OK;
  const void* ptrs[9] = {a->q, a->k, a->v, a->o, a->dout, a->dq, a->dk, a->dv, a->lse};
  const bool need[9] = {s_q > 0, s_k > 0, s_k > 0, s_q > 0, s_q > 0, s_q > 0, s_k > 0, s_k > 0, s_q > 0};
  for (int i = 0; i < 9; ++i) {
    if (need[i] && ptrs[i] == nullptr)
      return fail(EXATTN_E_INVALID, "q, k, v, o, dout, lse, dq, dk and dv must not be NULL");
    if (i < 8 && ptrs[i] != nullptr && !aligned16(ptrs[i]))
      return fail(EXATTN_E_INVALID, "q, k, v, o, dout, dq, dk and dv must be 16-byte aligned");
  }
  if ((reinterpret_cast<uintptr_t>(a->lse) & 3u) != 0) return fail(EXATTN_E_INVALID, "lse must be 4-byte aligned");
  const int64_t* strides[8] = {a->q_stride, a->k_stride, a->v_stride, a->o_stride,
                               a->dout_stride, a->dq_stride, a->dk_stride, a->dv_stride};
  for (int t = 0; t < 8; ++t)
    for (int i = varlen ? 1 : 0; i < 3; ++i)
      if (!stride_ok(strides[t][i]))
        return fail(EXATTN_E_INVALID, "backward strides must be non-negative multiples of 8 elements");
  if (a->lse_stride[1] < 0 || (!varlen && a->lse_stride[0] < 0))
    return fail(EXATTN_E_INVALID, "lse strides are negative");
  // Q and dO tiles of 32 rows, K and V tiles of up to 128 keys, one head each.
  const char* bn[5] = {"q", "k", "v", "o", "dout"};
  for (int t = 0; t < 5; ++t) {
    st = check_span(bn[t], t == 1 || t == 2 ? 128 : 64, strides[t][1], 1, 0, a->head_dim, 2);
    if (st != EXATTN_OK) return st;
  }
  if (rows > ((size_t)1 << 31) / 2) return fail(EXATTN_E_INVALID, "too many rows for one backward");
  if (a->batch > 65535 || a->heads_q > 65535)
    return fail(EXATTN_E_UNSUPPORTED, "the backward takes at most 65535 batch entries and query heads");
  return EXATTN_OK;
}

int decode_keys_per_step(int head_dim, int hpw) {
  const int nw = head_dim == 256 ? 4 : 8;                 // waves per work group
  const int hpwv = head_dim == 64 && hpw == 16 ? 2 : 1;    // heads per wave
  return 16 * (nw * hpwv / hpw);
}

exattn_status check_paged(const exattn_decode_args* a, const DecodePlan& pl, const exattn_paged_kv* pg) {
  if (pg == nullptr) return fail(EXATTN_E_INVALID, "paged is NULL");
  if (pg->page_size <= 0) return fail(EXATTN_E_INVALID, "page_size must be positive");
  const int kstep = decode_keys_per_step(a->head_dim, pl.hpw);
  if (pg->page_size % kstep != 0)
    return fail(EXATTN_E_UNSUPPORTED, "page_size must be a multiple of " + std::to_string(kstep) +
                                          " for this head_dim and heads_kv");
  if (a->batch == 0 || a->seqlen_cache == 0) return EXATTN_OK;
  if (pg->block_table == nullptr) return fail(EXATTN_E_INVALID, "block_table is NULL");
  if (pg->num_pages <= 0) return fail(EXATTN_E_INVALID, "num_pages must be positive");
  const int64_t need = ((int64_t)a->seqlen_cache + pg->page_size - 1) / pg->page_size;
  if (pg->block_table_stride < need)
    return fail(EXATTN_E_INVALID, "block_table_stride is smaller than ceil(seqlen_cache / page_size)");
  if (!stride_ok(pg->k_page_stride) || !stride_ok(pg->v_page_stride))
    return fail(EXATTN_E_INVALID, "page strides must be non-negative multiples of 8 elements");
  return EXATTN_OK;
}

}  // namespace exattn
