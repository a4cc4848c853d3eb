// C ABI entry points of libexattn: check, plan, launch.  No allocation, no
// synchronisation, no host read of device memory.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "exattn.h"
#include "kernels.h"
#include "validate.h"

namespace exattn {
namespace {

std::mutex g_mu;
std::vector<int> g_cus;  // per-device compute-unit count, 0 = not queried yet

exattn_status device_cus(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(EXATTN_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_mu);
  if ((int)g_cus.size() <= dev) g_cus.resize(dev + 1, 0);
  if (g_cus[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
      return fail(EXATTN_E_HIP, std::string("hipDeviceGetAttribute: ") + hipGetErrorString(e));
    g_cus[dev] = n > 0 ? n : 1;
  }
  *out = g_cus[dev];
  return EXATTN_OK;
}

// EXATTN_DEBUG, read once per process.
int debug_level() {
  static const int level = [] {
    const char* s = getenv("EXATTN_DEBUG");
    return s ? atoi(s) : 0;
  }();
  return level;
}

// EXATTN_DEBUG=1: print the plan once per distinct launch shape.
void debug_once(const std::string& key, const std::string& text) {
  static std::set<std::string> seen;
  std::lock_guard<std::mutex> lk(g_mu);
  if (seen.insert(key).second) fprintf(stderr, "[exattn] %s\n", text.c_str());
}

// Key-split schedule of a fixed-length masked prefill (one per unit; every
// unit runs the same), remembered for the last shape this thread launched.
bool slot_schedule(int s_q, int s_k, int wl, int wr, int wg_max, SlotSchedule* out) {
  struct Entry {
    int s_q = -1, s_k = -1, wl = 0, wr = 0, wg_max = 0;
    bool ok = false;
    SlotSchedule sch;
  };
  static thread_local Entry last;
  if (last.s_q != s_q || last.s_k != s_k || last.wl != wl || last.wr != wr || last.wg_max != wg_max) {
    const int n64 = (s_q + 63) / 64;
    last.ok = false;
    if (n64 >= 1 && n64 <= kMaxSlots) {
      int w[kMaxSlots];
      for (int t = 0; t < n64; ++t) {
        int lo, hi;
        tile_key_blocks(t, s_q, s_k, wl, wr, &lo, &hi);
        w[t] = hi - lo;
      }
      last.ok = build_slot_schedule(w, n64, wg_max, &last.sch);
    }
    last.s_q = s_q, last.s_k = s_k, last.wl = wl, last.wr = wr, last.wg_max = wg_max;
  }
  if (last.ok) *out = last.sch;
  return last.ok;
}

}  // namespace
}  // namespace exattn

using namespace exattn;

extern "C" {

exattn_status exattn_fwd(const exattn_fwd_args* a, void* stream) {
  try {
    clear_error();
    FwdPlan pl;
    exattn_status st = plan_fwd(a, prefill_rows_per_tile(), &pl);
    if (st != EXATTN_OK || pl.empty) return st;
    FwdParams p{};
    p.q = static_cast<const uint16_t*>(a->q);
    p.k = static_cast<const uint16_t*>(a->k);
    p.v = static_cast<const uint16_t*>(a->v);
    p.o = static_cast<uint16_t*>(a->o);
    p.lse = a->lse;
    p.q_sb = a->q_stride[0], p.q_ss = a->q_stride[1], p.q_sh = a->q_stride[2];
    p.k_sb = a->k_stride[0], p.k_ss = a->k_stride[1], p.k_sh = a->k_stride[2];
    p.v_sb = a->v_stride[0], p.v_ss = a->v_stride[1], p.v_sh = a->v_stride[2];
    p.o_sb = a->o_stride[0], p.o_ss = a->o_stride[1], p.o_sh = a->o_stride[2];
    p.lse_sb = a->lse_stride[0], p.lse_sh = a->lse_stride[1];
    p.cu_q = pl.varlen ? a->cu_seqlens_q : nullptr;
    p.cu_k = pl.varlen ? a->cu_seqlens_k : nullptr;
    p.batch = a->batch;
    p.s_q = pl.s_q;
    p.s_k = pl.s_k;
    p.h_q = a->heads_q;
    p.h_kv = a->heads_kv;
    p.group = pl.group;
    p.n_qt = pl.n_qt;
    p.xcd_group = pl.xcd_group;
    // Launch shape.  With at least two work groups per CU, one-group work
    // groups (two per CU, unsynchronised) are faster; with fewer, two groups
    // split each tile's KV blocks.  When the key range depends on the row
    // (causal or windowed) and the grid is about one work group per CU, the
    // launch lasts as long as its heaviest work group, so light and heavy tiles
    // are paired; with more work groups the dispatch order already balances the
    // CUs and pairing would only idle waves.
    int cus = 1;
    st = device_cus(&cus);
    if (st != EXATTN_OK) return st;
    const int groups = pl.head_dim == 256 || pl.grid >= 2 * cus ? 1 : 2;
    p.pair_tiles = groups == 2 && (pl.wr >= 0 || pl.wl >= 0) && pl.grid <= cus ? 1 : 0;
    p.scale_log2 = pl.scale_log2;
    p.cap_in = pl.cap_in;
    p.cap_out_log2 = pl.cap_out_log2;
    p.wl = pl.wl;
    p.wr = pl.wr;
    p.q_sign = pl.q_sign;
    p.pack = pl.pack ? 1 : 0;
    // Where the paired launch would fill at most half of the CUs at d = 128
    // (fixed lengths, one tile per query head), the key-split kernel runs
    // instead: it spreads the heavy tiles' key blocks over the idle CUs and
    // keeps two busy waves on every SIMD (measured 12-16% faster there).  At
    // about one work group per CU the paired launch measured faster, also
    // against a key-split schedule of the paired launch's size.
    SlotSchedule sch;
    bool slots = false;
    const int64_t units = (int64_t)a->batch * a->heads_q;
    if (p.pair_tiles && 2 * (int64_t)pl.grid <= cus && pl.head_dim == 128 && !pl.varlen && !pl.pack &&
        units <= cus && a->batch <= 65535)
      slots = slot_schedule(pl.s_q, pl.s_k, pl.wl, pl.wr, cus / (int)units, &sch);
    // At d = 256 (not packed) the head-dim-split kernel runs: two waves per
    // SIMD where the general kernel fits one.  With fewer 128-row tiles than
    // CUs it takes 64-row tiles and splits their key blocks between two groups.
    int dsplit = 0;
    if (pl.head_dim == 256 && !pl.pack && a->batch <= 65535) {
      const int64_t n64 = ((int64_t)pl.s_q + 63) / 64;
      dsplit = pl.grid < cus && n64 <= 65535 ? 2 : 1;
      if (dsplit == 2) p.n_qt = (int32_t)n64;
    }
    if (debug_level() >= 1) {
      char buf[256];
      snprintf(buf, sizeof buf,
               "fwd %s d=%d softcap=%d varlen=%d b=%d sq=%d sk=%d hq=%d hkv=%d wl=%d wr=%d grid=%d groups=%d "
               "pair=%d pack=%d slots=%d dsplit=%d",
               pl.bf16 ? "bf16" : "fp16", pl.head_dim, (int)pl.softcap, (int)pl.varlen, a->batch, pl.s_q,
               pl.s_k, a->heads_q, a->heads_kv, pl.wl, pl.wr, pl.grid, groups, p.pair_tiles, p.pack,
               slots ? sch.n_wg : 0, dsplit);
      debug_once(buf, buf);
    }
    hipError_t e;
    if (dsplit) {
      e = launch_prefill_dsplit(p, pl.bf16, dsplit, pl.softcap, static_cast<hipStream_t>(stream));
    } else if (slots) {
      static_assert(sizeof(SlotParams::slot) == 2 * sizeof(SlotSchedule::slot), "slot table");
      SlotParams sp{};
      sp.f = p;
      sp.n_wg = sch.n_wg;
      for (int i = 0; i < 4 * sch.n_wg; ++i) {
        sp.slot[2 * i] = sch.slot[i];
        sp.slot[2 * i + 1] = sch.nb[i];
      }
      e = launch_prefill_slots(sp, pl.bf16, pl.softcap, static_cast<hipStream_t>(stream));
    } else {
      e = launch_prefill(p, pl.bf16, pl.head_dim, pl.softcap, pl.grid, groups, static_cast<hipStream_t>(stream));
    }
    if (e != hipSuccess) return fail(EXATTN_E_HIP, std::string("prefill launch: ") + hipGetErrorString(e));
    return EXATTN_OK;
  } catch (...) {
    return fail(EXATTN_E_HIP, "unexpected host exception");
  }
}

exattn_status exattn_decode_plan(const exattn_decode_args* a, int32_t* num_splits_out,
                                 size_t* workspace_bytes_out) {
  try {
    clear_error();
    DecodePlan pl;
    exattn_status st = plan_decode(a, 1, &pl);  // argument checks need no device
    if (st != EXATTN_OK) return st;
    int cus = 1;
    if (a->num_splits == 0) {
      st = device_cus(&cus);
      if (st != EXATTN_OK) return st;
      st = plan_decode(a, cus, &pl);
      if (st != EXATTN_OK) return st;
    }
    if (num_splits_out) *num_splits_out = pl.n_split;
    if (workspace_bytes_out) *workspace_bytes_out = pl.ws_bytes;
    return EXATTN_OK;
  } catch (...) {
    return fail(EXATTN_E_HIP, "unexpected host exception");
  }
}

}  // extern "C"

namespace {

// The decode behind exattn_decode and exattn_decode_append: kv_new (or NULL)
// is written into the cache first, and the attended length per batch entry is
// cache_seqlens[b] + its seqlen_new.
exattn_status run_decode(const exattn_decode_args* a, const exattn_kv_new* kv_new,
                         const exattn_paged_kv* paged, void* workspace, size_t workspace_bytes,
                         void* stream) {
  try {
    clear_error();
    DecodePlan pl;
    exattn_status st = plan_decode(a, 1, &pl);
    if (st != EXATTN_OK) return st;
    if (kv_new != nullptr) {
      st = check_append(a, kv_new);
      if (st != EXATTN_OK) return st;
    }
    if (paged != nullptr) {
      st = check_paged(a, pl, paged);
      if (st != EXATTN_OK) return st;
    }
    const int32_t s_new = kv_new != nullptr && a->batch > 0 ? kv_new->seqlen_new : 0;
    if (a->num_splits == 0) {
      int cus = 1;
      st = device_cus(&cus);
      if (st != EXATTN_OK) return st;
      st = plan_decode(a, cus, &pl);
      if (st != EXATTN_OK) return st;
    }
    if (pl.empty) return EXATTN_OK;
    if (pl.n_split > 1) {
      if (workspace == nullptr || workspace_bytes < pl.ws_bytes)
        return fail(EXATTN_E_WORKSPACE, "workspace of " + std::to_string(pl.ws_bytes) +
                                            " bytes required, got " +
                                            std::to_string(workspace ? workspace_bytes : 0));
      if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(EXATTN_E_WORKSPACE, "workspace must be 256-byte aligned");
    }
    DecParams p{};
    if (paged != nullptr) {
      p.block_table = paged->block_table;
      p.bt_stride = paged->block_table_stride;
      p.page_size = paged->page_size;
      p.num_pages = paged->num_pages;
      p.k_sp = paged->k_page_stride;
      p.v_sp = paged->v_page_stride;
    }
    p.seq_add = s_new;
    if (s_new > 0) {
      p.k_new = static_cast<const uint16_t*>(kv_new->k_new);
      p.v_new = static_cast<const uint16_t*>(kv_new->v_new);
      p.kn_sb = kv_new->k_new_stride[0], p.kn_ss = kv_new->k_new_stride[1];
      p.kn_sh = kv_new->k_new_stride[2];
      p.vn_sb = kv_new->v_new_stride[0], p.vn_ss = kv_new->v_new_stride[1];
      p.vn_sh = kv_new->v_new_stride[2];
    }
    p.q = static_cast<const uint16_t*>(a->q);
    p.k = static_cast<const uint16_t*>(a->k_cache);
    p.v = static_cast<const uint16_t*>(a->v_cache);
    p.o = static_cast<uint16_t*>(a->o);
    p.lse = a->lse;
    p.q_sb = a->q_stride[0], p.q_sh = a->q_stride[1];
    p.o_sb = a->o_stride[0], p.o_sh = a->o_stride[1];
    p.k_sb = a->k_stride[0], p.k_ss = a->k_stride[1], p.k_sh = a->k_stride[2];
    p.v_sb = a->v_stride[0], p.v_ss = a->v_stride[1], p.v_sh = a->v_stride[2];
    p.cache_seqlens = a->cache_seqlens;
    p.ws_o = pl.n_split > 1 ? static_cast<float*>(workspace) : nullptr;
    p.ws_lse = pl.n_split > 1
                   ? reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.ws_lse_offset)
                   : nullptr;
    p.batch = a->batch;
    p.h_q = a->heads_q;
    p.h_kv = a->heads_kv;
    p.group = pl.group;
    p.s_cache = a->seqlen_cache;
    p.n_split = pl.n_split;
    p.n_hg = pl.n_hg;
    p.hpw = pl.hpw;
    p.scale_log2 = pl.scale_log2;
    p.cap_in = pl.cap_in;
    p.cap_out_log2 = pl.cap_out_log2;
    p.wl = pl.wl;
    p.wr = pl.wr;
    p.s_q = pl.s_q;
    p.q_ss = a->q_token_stride;
    p.o_ss = a->o_token_stride;
    if (debug_level() >= 1) {
      char buf[256];
      snprintf(buf, sizeof buf, "decode %s d=%d softcap=%d b=%d hq=%d hkv=%d cache=%d splits=%d wl=%d",
               pl.bf16 ? "bf16" : "fp16", pl.head_dim, (int)pl.softcap, a->batch, a->heads_q,
               a->heads_kv, a->seqlen_cache, pl.n_split, pl.wl);
      debug_once(buf, buf);
    }
    hipError_t e = launch_decode(p, pl.bf16, pl.head_dim, pl.softcap, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(EXATTN_E_HIP, std::string("decode launch: ") + hipGetErrorString(e));
    return EXATTN_OK;
  } catch (...) {
    return fail(EXATTN_E_HIP, "unexpected host exception");
  }
}

}  // namespace

extern "C" {

exattn_status exattn_fwd_fp8(const exattn_fwd_args* a, const exattn_fp8_descale* d, void* stream) {
  try {
    clear_error();
    Fp8Plan pl;
    exattn_status st = plan_fwd_fp8(a, d, &pl);
    if (st != EXATTN_OK) return st;
    if (pl.empty) return EXATTN_OK;
    Fp8Params p{};
    p.q = static_cast<const uint8_t*>(a->q);
    p.k = static_cast<const uint8_t*>(a->k);
    p.v = static_cast<const uint8_t*>(a->v);
    p.o = static_cast<uint16_t*>(a->o);
    p.lse = a->lse;
    p.q_sb = a->q_stride[0], p.q_ss = a->q_stride[1], p.q_sh = a->q_stride[2];
    p.k_sb = a->k_stride[0], p.k_ss = a->k_stride[1], p.k_sh = a->k_stride[2];
    p.v_sb = a->v_stride[0], p.v_ss = a->v_stride[1], p.v_sh = a->v_stride[2];
    p.o_sb = a->o_stride[0], p.o_ss = a->o_stride[1], p.o_sh = a->o_stride[2];
    p.lse_sb = a->lse_stride[0], p.lse_sh = a->lse_stride[1];
    p.batch = a->batch;
    p.s_q = pl.s_q;
    p.s_k = pl.s_k;
    p.h_q = a->heads_q;
    p.h_kv = a->heads_kv;
    p.group = pl.group;
    p.scale_log2 = pl.scale_log2;
    p.v_descale = pl.v_descale;
    p.wl = pl.wl;
    p.wr = pl.wr;
    p.cap_in = pl.cap_in;
    p.cap_out_log2 = pl.cap_out_log2;
    p.cu_q = pl.varlen ? a->cu_seqlens_q : nullptr;
    p.cu_k = pl.varlen ? a->cu_seqlens_k : nullptr;
    hipError_t e = launch_fwd_fp8(p, pl.head_dim, pl.softcap, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(EXATTN_E_HIP, std::string("fp8 forward launch: ") + hipGetErrorString(e));
    return EXATTN_OK;
  } catch (...) {
    return fail(EXATTN_E_HIP, "unexpected host exception");
  }
}

exattn_status exattn_bwd_plan(const exattn_bwd_args* a, size_t* workspace_bytes_out) {
  try {
    clear_error();
    BwdPlan pl;
    exattn_status st = plan_bwd(a, &pl);
    if (st != EXATTN_OK) return st;
    if (workspace_bytes_out != nullptr) *workspace_bytes_out = pl.ws_bytes;
    return EXATTN_OK;
  } catch (...) {
    return fail(EXATTN_E_HIP, "unexpected host exception");
  }
}

exattn_status exattn_bwd(const exattn_bwd_args* a, void* workspace, size_t workspace_bytes,
                         void* stream) {
  try {
    clear_error();
    BwdPlan pl;
    exattn_status st = plan_bwd(a, &pl);
    if (st != EXATTN_OK) return st;
    if (pl.empty) return EXATTN_OK;
    if (pl.ws_bytes > 0) {
      if (workspace == nullptr || workspace_bytes < pl.ws_bytes)
        return fail(EXATTN_E_WORKSPACE, "workspace of " + std::to_string(pl.ws_bytes) + " bytes required");
      if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(EXATTN_E_WORKSPACE, "workspace must be 256-byte aligned");
    }
    BwdParams p{};
    p.q = static_cast<const uint16_t*>(a->q);
    p.k = static_cast<const uint16_t*>(a->k);
    p.v = static_cast<const uint16_t*>(a->v);
    p.o = static_cast<const uint16_t*>(a->o);
    p.dout = static_cast<const uint16_t*>(a->dout);
    p.lse = a->lse;
    p.dq = static_cast<uint16_t*>(a->dq);
    p.dk = static_cast<uint16_t*>(a->dk);
    p.dv = static_cast<uint16_t*>(a->dv);
    p.ws_stats = static_cast<float*>(workspace);
    p.q_sb = a->q_stride[0], p.q_ss = a->q_stride[1], p.q_sh = a->q_stride[2];
    p.k_sb = a->k_stride[0], p.k_ss = a->k_stride[1], p.k_sh = a->k_stride[2];
    p.v_sb = a->v_stride[0], p.v_ss = a->v_stride[1], p.v_sh = a->v_stride[2];
    p.o_sb = a->o_stride[0], p.o_ss = a->o_stride[1], p.o_sh = a->o_stride[2];
    p.do_sb = a->dout_stride[0], p.do_ss = a->dout_stride[1], p.do_sh = a->dout_stride[2];
    p.dq_sb = a->dq_stride[0], p.dq_ss = a->dq_stride[1], p.dq_sh = a->dq_stride[2];
    p.dk_sb = a->dk_stride[0], p.dk_ss = a->dk_stride[1], p.dk_sh = a->dk_stride[2];
    p.dv_sb = a->dv_stride[0], p.dv_ss = a->dv_stride[1], p.dv_sh = a->dv_stride[2];
    p.lse_sb = a->lse_stride[0], p.lse_sh = a->lse_stride[1];
    p.batch = a->batch;
    p.s_q = pl.s_q;
    p.s_k = pl.s_k;
    p.h_q = a->heads_q;
    p.h_kv = a->heads_kv;
    p.group = pl.group;
    p.scale = pl.scale;
    p.scale_log2 = pl.scale_log2;
    p.cap_in = pl.cap_in;
    p.cap_out_log2 = pl.cap_out_log2;
    p.wl = pl.wl;
    p.wr = pl.wr;
    p.bf16 = pl.bf16 ? 1 : 0;
    p.cu_q = pl.varlen ? a->cu_seqlens_q : nullptr;
    p.cu_k = pl.varlen ? a->cu_seqlens_k : nullptr;
    hipError_t e = launch_bwd(p, pl.head_dim, pl.softcap, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(EXATTN_E_HIP, std::string("backward launch: ") + hipGetErrorString(e));
    return EXATTN_OK;
  } catch (...) {
    return fail(EXATTN_E_HIP, "unexpected host exception");
  }
}

exattn_status exattn_decode(const exattn_decode_args* a, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return run_decode(a, nullptr, nullptr, workspace, workspace_bytes, stream);
}

exattn_status exattn_decode_noalloc(const exattn_decode_args* a, void* stream) {
  try {
    clear_error();
    DecodePlan pl;
    exattn_status st = plan_decode(a, 1, &pl);
    if (st != EXATTN_OK) return st;
    if (a->num_splits == 0) {
      int cus = 1;
      st = device_cus(&cus);
      if (st != EXATTN_OK) return st;
      st = plan_decode(a, cus, &pl);
      if (st != EXATTN_OK) return st;
    }
    if (pl.empty) return EXATTN_OK;
    if (pl.ws_bytes > kDecodeScratchBytes)
      return fail(EXATTN_E_WORKSPACE, "the split partials need " + std::to_string(pl.ws_bytes) +
                                          " bytes, more than the static scratch (" +
                                          std::to_string(kDecodeScratchBytes) +
                                          "): lower num_splits or use exattn_decode");
    void* ptr = nullptr;
    hipError_t e = decode_scratch(&ptr);
    if (e != hipSuccess) return fail(EXATTN_E_HIP, std::string("scratch lookup: ") + hipGetErrorString(e));
    return run_decode(a, nullptr, nullptr, ptr, kDecodeScratchBytes, stream);
  } catch (...) {
    return fail(EXATTN_E_HIP, "unexpected host exception");
  }
}

exattn_status exattn_decode_append(const exattn_decode_args* a, const exattn_kv_new* kv_new,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (kv_new == nullptr) {
    clear_error();
    return fail(EXATTN_E_INVALID, "kv_new is NULL");
  }
  return run_decode(a, kv_new, nullptr, workspace, workspace_bytes, stream);
}

exattn_status exattn_decode_paged(const exattn_decode_args* a, const exattn_paged_kv* paged,
                                  const exattn_kv_new* kv_new, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (paged == nullptr) {
    clear_error();
    return fail(EXATTN_E_INVALID, "paged is NULL");
  }
  return run_decode(a, kv_new, paged, workspace, workspace_bytes, stream);
}

int32_t exattn_decode_auto_splits(int32_t batch, int32_t heads_q, int32_t heads_kv,
                                  int32_t seqlen_k, int32_t head_dim, int32_t num_cus) {
  return auto_splits(batch, heads_q, heads_kv, seqlen_k, head_dim, num_cus);
}

size_t exattn_args_size(int32_t which) {
  return which == 0   ? sizeof(exattn_fwd_args)
         : which == 1 ? sizeof(exattn_decode_args)
         : which == 2 ? sizeof(exattn_kv_new)
         : which == 3 ? sizeof(exattn_paged_kv)
         : which == 4 ? sizeof(exattn_bwd_args)
         : which == 5 ? sizeof(exattn_fp8_descale)
                      : 0;
}

const char* exattn_status_string(int32_t status) {
  switch (status) {
    case EXATTN_OK: return "EXATTN_OK";
    case EXATTN_E_INVALID: return "EXATTN_E_INVALID";
    case EXATTN_E_UNSUPPORTED: return "EXATTN_E_UNSUPPORTED";
    case EXATTN_E_WORKSPACE: return "EXATTN_E_WORKSPACE";
    case EXATTN_E_HIP: return "EXATTN_E_HIP";
    default: return "EXATTN_E_UNKNOWN";
  }
}

const char* exattn_last_error(void) { return last_error(); }

int32_t exattn_abi_version(void) { return EXATTN_ABI_VERSION; }

}  // extern "C"
