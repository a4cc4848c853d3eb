// Host-only driver of the argument checks and launch planning (validate.cpp),
// built with g++ and the address / undefined-behaviour sanitizers
// (build.build_host_checker) and run by the CPU test suite.  It feeds every
// plan function seeded random arguments drawn around the edges that matter
// (zero, negative, odd and huge sizes and strides, NULL and misaligned
// pointers, NaN / inf scales, sizes near 2^31) and checks the invariants of
// every accepted plan: any signed overflow or out-of-bounds access in the
// checks themselves ends the run with a sanitizer report.
//
//   validate_check [iterations] [seed]
//
// Prints one line of accept / reject counts per function; exits 1 on a broken
// invariant.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <string>

#include "validate.h"

using namespace exattn;

namespace {

uint64_t g_state = 0x9e3779b97f4a7c15ull;

uint64_t next() {  // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 0x2545f4914f6cdd1dull;
}

int pick(int n) { return (int)((next() >> 32) % (uint64_t)n); }  // the high bits: the low ones are weak
bool chance(int percent) { return pick(100) < percent; }

// A size: mostly small valid values, sometimes an edge.
int32_t size_val(int32_t typical_max) {
  static const int32_t edges[] = {0, 1, -1, 2, 7, 63, 64, 65, 127, 128, 129, 4095, 65535, 65536,
                                  (1 << 22) - 1, 1 << 22, 0x7fffffff, (int32_t)0x80000000};
  if (chance(85)) return 1 + pick(typical_max);
  return edges[pick((int)(sizeof edges / sizeof edges[0]))];
}

// A stride in elements: mostly a multiple of 8 from the sizes, sometimes an edge.
int64_t stride_val(int64_t typical) {
  static const int64_t edges[] = {0, 8, -8, 1, 7, 1 << 20, (int64_t)1 << 31, ((int64_t)1 << 31) - 8,
                                  (int64_t)1 << 40, INT64_MAX, INT64_MIN, INT64_MAX - 7};
  if (chance(90)) return typical;
  return edges[pick((int)(sizeof edges / sizeof edges[0]))];
}

const void* ptr_val(bool allow_null = true) {
  if (allow_null && chance(3)) return nullptr;
  if (chance(3)) return reinterpret_cast<const void*>(uintptr_t(0x100008));  // misaligned
  return reinterpret_cast<const void*>(uintptr_t(0x100000) + 256 * pick(1024));
}

float scale_val() {
  static const float edges[] = {0.f, -0.125f, 1e30f, -1e30f, INFINITY, -INFINITY, 1e-30f};
  if (chance(70)) return NAN;
  if (chance(70)) return 0.01f + (float)pick(1000) / 1000.f;
  return edges[pick((int)(sizeof edges / sizeof edges[0]))];
}

float cap_val() {
  static const float edges[] = {-1.f, 1e-20f, 1e30f, INFINITY, NAN};
  if (chance(70)) return 0.f;
  if (chance(80)) return 1.f + (float)pick(100);
  return edges[pick((int)(sizeof edges / sizeof edges[0]))];
}

// a window edge: -1 (unbounded) and sizes, INT32_MIN included
int32_t window_val() {
  const int32_t w = size_val(512);
  return w > INT32_MIN ? w - 1 : w;
}

int32_t head_dim_val() {
  static const int32_t v[] = {64, 128, 256, 64, 128, 256, 0, 32, 96, 512, -64};
  return v[pick((int)(sizeof v / sizeof v[0]))];
}

int32_t dtype_val() { return chance(90) ? pick(2) : (chance(50) ? EXATTN_FP8_E4M3 : 7); }

struct Heads {
  int32_t q, kv;
};
Heads heads_val() {
  const int32_t kv = chance(90) ? 1 + pick(16) : size_val(8);
  const int32_t g = chance(90) ? 1 + pick(8) : size_val(4);
  Heads h{(int32_t)((int64_t)kv * g), kv};
  if (chance(5)) h.q = size_val(64);
  return h;
}

struct Count {
  const char* name;
  long ok = 0, rejected = 0;
};

int g_broken = 0;
void expect(bool cond, const char* what, long it) {
  if (!cond) {
    fprintf(stderr, "iteration %ld: invariant broken: %s\n", it, what);
    ++g_broken;
  }
}

// dense (batch, token, head) strides of an s x h x d tensor, products capped at
// 2^40 so that the driver itself stays free of overflow
int64_t capped(int64_t a, int64_t b) {
  const int64_t cap = (int64_t)1 << 40;
  if (a <= 0 || b <= 0) return a * (b > 0 ? 1 : 0);
  return a > cap / b ? cap : a * b;
}
void fill_dense_strides(int64_t st[3], int32_t s, int32_t h, int32_t d) {
  st[2] = stride_val(d);
  st[1] = stride_val(capped(h, d));
  st[0] = stride_val(capped(capped(s, h), d));
}

// Window edges as planned: an edge inside the rows / keys is kept as given,
// one that reaches past all of them is unbounded (-1), so that row + key
// offset + edge stays within 32 bits in the kernels.
template <class Args>
void window_checks(const Args& a, int64_t s_q, int64_t s_k, int wl, int wr, const char* who, long it) {
  const std::string w = who;
  expect(wl < 0 || wl < s_k, (w + " left edge inside the keys").c_str(), it);
  expect(wr < 0 || wr < std::max<int64_t>(s_q, 1), (w + " right edge inside the rows").c_str(), it);
  if (a.window_left >= 0 && a.window_left < s_k) expect(wl == a.window_left, (w + " left edge kept").c_str(), it);
  if (a.causal) expect(wr == 0, (w + " causal right edge").c_str(), it);
  else if (a.window_right >= 0 && a.window_right < s_q)
    expect(wr == a.window_right, (w + " right edge kept").c_str(), it);
}

void fwd_case(long it, Count& c, Count& c8) {
  exattn_fwd_args a{};
  a.dtype = dtype_val();
  const Heads hd = heads_val();
  a.heads_q = hd.q;
  a.heads_kv = hd.kv;
  a.head_dim = head_dim_val();
  a.batch = chance(90) ? pick(9) : size_val(4);
  a.seqlen_q = chance(90) ? pick(4097) : size_val(1024);
  a.seqlen_k = chance(90) ? pick(4097) : size_val(1024);
  a.q = ptr_val(false);
  a.k = ptr_val(false);
  a.v = ptr_val(false);
  a.o = const_cast<void*>(ptr_val(false));
  a.lse = chance(80) ? (float*)0x200000 : nullptr;
  const bool varlen = chance(25);
  const int32_t d = a.head_dim > 0 && a.head_dim <= 512 ? a.head_dim : 128;
  fill_dense_strides(a.q_stride, a.seqlen_q, a.heads_q > 0 ? a.heads_q : 1, d);
  fill_dense_strides(a.k_stride, a.seqlen_k, a.heads_kv > 0 ? a.heads_kv : 1, d);
  fill_dense_strides(a.v_stride, a.seqlen_k, a.heads_kv > 0 ? a.heads_kv : 1, d);
  fill_dense_strides(a.o_stride, a.seqlen_q, a.heads_q > 0 ? a.heads_q : 1, d);
  a.lse_stride[1] = stride_val(a.seqlen_q);
  a.lse_stride[0] = stride_val((int64_t)a.seqlen_q * (a.heads_q > 0 ? a.heads_q : 1));
  if (varlen) {
    a.cu_seqlens_q = chance(95) ? (const int32_t*)0x300000 : nullptr;
    a.cu_seqlens_k = chance(95) ? (const int32_t*)0x300100 : nullptr;
    a.max_seqlen_q = chance(90) ? pick(4097) : size_val(64);
    a.max_seqlen_k = chance(90) ? pick(4097) : size_val(64);
  }
  a.softmax_scale = scale_val();
  a.softcap = cap_val();
  a.causal = chance(50);
  a.window_left = chance(70) ? -1 : window_val();
  a.window_right = chance(70) ? -1 : window_val();
  a.pack_gqa = chance(90) ? pick(3) - 1 : size_val(4);

  FwdPlan pl{};
  if (plan_fwd(&a, 128 /* the prefill kernel's query tile height */, &pl) == EXATTN_OK) {
    ++c.ok;
    if (!pl.empty) {
      expect(pl.grid >= 1, "fwd grid >= 1", it);
      expect(pl.n_qt >= 1, "fwd n_qt >= 1", it);
      expect(pl.group >= 1 && (int64_t)pl.group * a.heads_kv == a.heads_q, "fwd group", it);
      expect(pl.head_dim == a.head_dim, "fwd head_dim", it);
      expect(isfinite(pl.scale_log2), "fwd scale finite", it);
      expect(!pl.pack || (int64_t)pl.s_q * pl.group < ((int64_t)1 << 22), "fwd pack bound", it);
      const int64_t units = (int64_t)a.batch * (pl.pack ? a.heads_kv : a.heads_q);
      expect(units * pl.n_qt == pl.grid, "fwd grid = units x tiles", it);
      window_checks(a, pl.s_q, pl.s_k, pl.wl, pl.wr, "fwd", it);
    }
  } else {
    ++c.rejected;
    expect(last_error()[0] != '\0', "fwd rejection has a message", it);
  }

  // the same arguments through the FP8 planner
  a.dtype = chance(80) ? EXATTN_FP8_E4M3 : a.dtype;
  exattn_fp8_descale ds{1.f, 1.f, 1.f};
  if (chance(10)) ds.q = chance(50) ? NAN : -1.f;
  Fp8Plan p8{};
  if (plan_fwd_fp8(&a, chance(95) ? &ds : nullptr, &p8) == EXATTN_OK) {
    ++c8.ok;
    if (!p8.empty) {
      expect(p8.group >= 1 && (int64_t)p8.group * a.heads_kv == a.heads_q, "fp8 group", it);
      expect(isfinite(p8.scale_log2) && isfinite(p8.v_descale), "fp8 scales finite", it);
      window_checks(a, p8.s_q, p8.s_k, p8.wl, p8.wr, "fp8", it);
    }
  } else {
    ++c8.rejected;
  }
}

void decode_case(long it, Count& c, Count& capp, Count& cpg) {
  exattn_decode_args a{};
  a.dtype = dtype_val();
  const Heads hd = heads_val();
  a.heads_q = hd.q;
  a.heads_kv = hd.kv;
  a.head_dim = head_dim_val();
  a.batch = chance(90) ? pick(17) : size_val(8);
  a.seqlen_cache = chance(90) ? pick(65537) : size_val(4096);
  a.seqlen_q = chance(80) ? 0 : size_val(16);
  const int32_t d = a.head_dim > 0 && a.head_dim <= 512 ? a.head_dim : 128;
  const int32_t hq = a.heads_q > 0 ? a.heads_q : 1, hkv = a.heads_kv > 0 ? a.heads_kv : 1;
  const int32_t sq = a.seqlen_q > 0 && a.seqlen_q < 4096 ? a.seqlen_q : 1;
  a.q = ptr_val(false);
  a.k_cache = ptr_val(false);
  a.v_cache = ptr_val(false);
  a.o = const_cast<void*>(ptr_val(false));
  a.lse = chance(70) ? (float*)0x200000 : nullptr;
  a.q_stride[1] = stride_val(d);
  a.q_stride[0] = stride_val(capped(capped(sq, hq), d));
  a.o_stride[1] = stride_val(d);
  a.o_stride[0] = stride_val(capped(capped(sq, hq), d));
  a.q_token_stride = stride_val((int64_t)hq * d);
  a.o_token_stride = stride_val((int64_t)hq * d);
  fill_dense_strides(a.k_stride, a.seqlen_cache, hkv, d);
  fill_dense_strides(a.v_stride, a.seqlen_cache, hkv, d);
  a.cache_seqlens = chance(60) ? (const int32_t*)0x300000 : nullptr;
  a.softmax_scale = scale_val();
  a.softcap = cap_val();
  a.causal = chance(50);
  a.window_left = chance(70) ? -1 : window_val();
  a.window_right = chance(80) ? -1 : window_val();
  a.num_splits = chance(70) ? 0 : size_val(64);

  static const int cus[] = {256, 304, 1, 0, -1, 80};
  const int ncu = cus[chance(85) ? 0 : pick(6)];
  DecodePlan pl{};
  if (plan_decode(&a, ncu, &pl) != EXATTN_OK) {
    ++c.rejected;
    return;
  }
  ++c.ok;
  if (!pl.empty) {
    expect(pl.n_split >= 1, "decode n_split >= 1", it);
    expect(a.num_splits <= 0 || pl.n_split <= a.num_splits, "decode n_split <= requested", it);
    expect(pl.n_hg >= 1 && pl.hpw >= 1 && pl.n_hk >= 1, "decode grid factors", it);
    expect((int64_t)pl.n_hk * pl.hpw >= a.heads_kv, "decode head groups cover heads_kv", it);
    expect(pl.s_q >= 1, "decode s_q >= 1", it);
    expect(pl.n_split == 1 || pl.ws_lse_offset <= pl.ws_bytes, "decode workspace layout", it);
  }

  exattn_kv_new n{};
  n.k_new = ptr_val();
  n.v_new = ptr_val();
  n.seqlen_new = chance(80) ? 1 + pick(16) : size_val(8);
  fill_dense_strides(n.k_new_stride, n.seqlen_new, hkv, d);
  fill_dense_strides(n.v_new_stride, n.seqlen_new, hkv, d);
  if (check_append(&a, &n) == EXATTN_OK)
    ++capp.ok;
  else
    ++capp.rejected;

  exattn_paged_kv pg{};
  pg.block_table = chance(95) ? (const int32_t*)0x400000 : nullptr;
  pg.page_size = chance(85) ? 16 << pick(5) : size_val(64);
  pg.num_pages = chance(90) ? 1 + pick(4096) : size_val(64);
  pg.block_table_stride = chance(90) ? 1 + pick(4096) : size_val(64);
  pg.k_page_stride = stride_val(capped(capped(pg.page_size, hkv), d));
  pg.v_page_stride = stride_val(capped(capped(pg.page_size, hkv), d));
  if (check_paged(&a, pl, &pg) == EXATTN_OK)
    ++cpg.ok;
  else
    ++cpg.rejected;
}

void bwd_case(long it, Count& c) {
  exattn_bwd_args a{};
  a.dtype = dtype_val();
  const Heads hd = heads_val();
  a.heads_q = hd.q;
  a.heads_kv = hd.kv;
  a.head_dim = head_dim_val();
  a.batch = chance(90) ? pick(9) : size_val(4);
  a.seqlen_q = chance(90) ? pick(4097) : size_val(1024);
  a.seqlen_k = chance(90) ? pick(4097) : size_val(1024);
  const int32_t d = a.head_dim > 0 && a.head_dim <= 512 ? a.head_dim : 128;
  const int32_t hq = a.heads_q > 0 ? a.heads_q : 1, hkv = a.heads_kv > 0 ? a.heads_kv : 1;
  a.q = ptr_val(false);
  a.k = ptr_val(false);
  a.v = ptr_val(false);
  a.o = ptr_val(false);
  a.dout = ptr_val(false);
  a.lse = chance(97) ? (const float*)0x200000 : nullptr;
  a.dq = const_cast<void*>(ptr_val(false));
  a.dk = const_cast<void*>(ptr_val(false));
  a.dv = const_cast<void*>(ptr_val(false));
  fill_dense_strides(a.q_stride, a.seqlen_q, hq, d);
  fill_dense_strides(a.o_stride, a.seqlen_q, hq, d);
  fill_dense_strides(a.dout_stride, a.seqlen_q, hq, d);
  fill_dense_strides(a.dq_stride, a.seqlen_q, hq, d);
  fill_dense_strides(a.k_stride, a.seqlen_k, hkv, d);
  fill_dense_strides(a.v_stride, a.seqlen_k, hkv, d);
  fill_dense_strides(a.dk_stride, a.seqlen_k, hkv, d);
  fill_dense_strides(a.dv_stride, a.seqlen_k, hkv, d);
  a.lse_stride[1] = stride_val(a.seqlen_q);
  a.lse_stride[0] = stride_val((int64_t)a.seqlen_q * hq);
  if (chance(25)) {
    a.cu_seqlens_q = chance(95) ? (const int32_t*)0x300000 : nullptr;
    a.cu_seqlens_k = chance(95) ? (const int32_t*)0x300100 : nullptr;
    a.max_seqlen_q = chance(90) ? pick(4097) : size_val(64);
    a.max_seqlen_k = chance(90) ? pick(4097) : size_val(64);
  }
  a.softmax_scale = scale_val();
  a.softcap = cap_val();
  a.causal = chance(50);
  a.window_left = chance(70) ? -1 : window_val();
  a.window_right = chance(70) ? -1 : window_val();
  BwdPlan pl{};
  if (plan_bwd(&a, &pl) == EXATTN_OK) {
    ++c.ok;
    if (!pl.empty) {
      expect(pl.group >= 1 && (int64_t)pl.group * a.heads_kv == a.heads_q, "bwd group", it);
      expect(pl.head_dim == 64 || pl.head_dim == 128 || pl.head_dim == 256, "bwd head_dim", it);
      expect(isfinite(pl.scale) && isfinite(pl.scale_log2), "bwd scales finite", it);
      const int64_t sq = a.cu_seqlens_q != nullptr ? a.max_seqlen_q : a.seqlen_q;
      expect(pl.ws_bytes % 256 == 0 && (int64_t)pl.ws_bytes >= 8 * (int64_t)a.batch * a.heads_q * sq,
             "bwd workspace holds 8 bytes per row", it);
      window_checks(a, pl.s_q, pl.s_k, pl.wl, pl.wr, "bwd", it);
    }
  } else {
    ++c.rejected;
  }
}

void splits_case(long it, Count& c) {
  const int32_t b = size_val(16), hq = size_val(64), hkv = size_val(16), sk = size_val(65536);
  const int32_t d = head_dim_val(), cu = chance(90) ? 256 : size_val(512), sq = size_val(8);
  if (b < 1 || hq < 1 || hkv < 1 || sk < 0 || cu < 1 || sq < 1 || d < 1 || hq % hkv != 0) {
    ++c.rejected;  // outside what plan_decode hands over
    return;
  }
  const int32_t s = auto_splits(b, hq, hkv, sk, d, cu, sq);
  expect(s >= 1, "auto_splits >= 1", it);
  ++c.ok;
}

// the invariants the key-split kernel relies on
void check_schedule(const SlotSchedule& sc, const int* w, int n64, int wg_max, long it) {
  expect(sc.n_wg >= 1 && sc.n_wg <= wg_max && sc.n_wg <= kMaxSlots / 4, "schedule work groups", it);
  static int seen[1024];
  for (int t = 0; t < n64; ++t) seen[t] = 0;
  int steps = 0;
  for (int s = 0; s < 4 * sc.n_wg; ++s) {
    const uint32_t e = sc.slot[s];
    if (!(e >> 24)) {
      expect(sc.nb[s] == 0, "an unused slot computes nothing", it);
      continue;
    }
    const int t = (int)(e & 0xffff), k = (int)((e >> 16) & 7), kn = (int)((e >> 19) & 7);
    if (t >= n64 || kn < 1 || kn > 4 || k >= kn) {
      expect(false, "schedule entry out of range", it);
      continue;
    }
    // the tile's slots are consecutive and inside one work group
    const int first = s - k;
    expect(first >= 0 && first / 4 == (first + kn - 1) / 4, "tile slots share one work group", it);
    const int nb = w[t] > k ? (w[t] - k + kn - 1) / kn : 0;
    expect((int)sc.nb[s] == nb, "slot block count", it);
    expect(w[t] == 0 || k < w[t], "every slot of a tile with blocks has one", it);
    ++seen[t];
    steps = std::max(steps, nb);
  }
  for (int t = 0; t < n64; ++t) {
    const uint32_t e0 = [&] {
      for (int s = 0; s < 4 * sc.n_wg; ++s)
        if ((sc.slot[s] >> 24) && (int)(sc.slot[s] & 0xffff) == t && ((sc.slot[s] >> 16) & 7) == 0) return sc.slot[s];
      return 0u;
    }();
    expect(e0 != 0 && seen[t] == (int)((e0 >> 19) & 7), "every tile has its kgn slots", it);
  }
  expect(steps == sc.steps, "schedule steps", it);
}

void slots_case(long it, Count& c) {
  const int n64 = chance(80) ? 1 + pick(64) : size_val(300);
  const int wg_max = chance(80) ? 1 + pick(80) : size_val(100);
  if (n64 < 1 || n64 > 1024) {
    ++c.rejected;
    return;
  }
  static int w[1024];
  for (int t = 0; t < n64; ++t) w[t] = chance(10) ? 0 : pick(chance(50) ? 2 * (t + 1) + 1 : 300);
  SlotSchedule sc;
  if (!build_slot_schedule(w, n64, wg_max, &sc)) {
    ++c.rejected;
    expect(wg_max < 1 || n64 > 4 * std::min(wg_max, kMaxSlots / 4), "schedule refused a fitting case", it);
    return;
  }
  ++c.ok;
  check_schedule(sc, w, n64, wg_max, it);
}

}  // namespace

int main(int argc, char** argv) {
  const long iters = argc > 1 ? atol(argv[1]) : 200000;
  if (argc > 2) {  // splitmix64 of the seed: never the all-zero state xorshift cannot leave
    uint64_t z = strtoull(argv[2], nullptr, 0) + 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    g_state = (z ^ (z >> 31)) | 1u;
  }
  Count fwd{"plan_fwd"}, fp8{"plan_fwd_fp8"}, dec{"plan_decode"}, app{"check_append"}, pg{"check_paged"},
      bwd{"plan_bwd"}, spl{"auto_splits"}, slo{"slot_schedule"};
  for (long it = 0; it < iters; ++it) {
    switch (it % 5) {
      case 0: fwd_case(it, fwd, fp8); break;
      case 1: decode_case(it, dec, app, pg); break;
      case 2: bwd_case(it, bwd); break;
      case 3: slots_case(it, slo); break;
      default: splits_case(it, spl); break;
    }
  }
  for (const Count* c : {&fwd, &fp8, &dec, &app, &pg, &bwd, &spl, &slo})
    printf("%-14s accepted %8ld rejected %8ld\n", c->name, c->ok, c->rejected);
  if (g_broken) printf("%d broken invariants\n", g_broken);
  return g_broken ? 1 : 0;
}
