// Host-side argument checks and launch planning for the exattn C ABI.
//
// Pure C++ (no HIP): everything here runs before any launch and can be built
// and tested on a machine without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "exattn.h"

namespace exattn {

// Set the calling thread's error text and return `st`.
exattn_status fail(exattn_status st, const std::string& msg);
void clear_error();
const char* last_error();

// Resolved prefill launch: the kernel variant and grid plus the folded scales.
struct FwdPlan {
  bool empty;  // nothing to launch
  bool bf16;
  int head_dim;
  bool softcap;
  bool varlen;
  int s_q, s_k;  // lengths (fixed) or maxima (varlen)
  int group;
  int n_qt;      // query tiles per (batch, head)
  int grid;      // work groups
  int xcd_group;
  float scale_log2, cap_in, cap_out_log2;
  uint32_t q_sign;  // 0x80008000: negative scale, applied by negating Q (scale_log2 holds |scale|)
  int wl, wr;
  bool pack;        // packed GQA: tiles over (position, query head of one KV head)
};

// Check `a` and fill `plan`.  rows_per_tile is the kernel's query tile height.
exattn_status plan_fwd(const exattn_fwd_args* a, int rows_per_tile, FwdPlan* plan);

struct DecodePlan {
  bool empty;
  bool bf16;
  int head_dim;
  bool softcap;
  int group;
  int n_hg;      // groups of 16 query heads per KV head
  int hpw;       // adjacent KV heads per work group (contiguous key-row pieces)
  int n_hk;      // KV-head groups: ceil(heads_kv / hpw)
  int n_split;
  size_t ws_bytes;
  size_t ws_lse_offset;  // byte offset of the LSE partials inside the workspace
  float scale_log2, cap_in, cap_out_log2;
  int wl, wr;   // window edges for the query tokens (wr = 0 for causal); < 0 unbounded
  int s_q;      // query tokens per batch entry (>= 1)
};

// Check `a` and fill `plan` for a device with `num_cus` compute units.
exattn_status plan_decode(const exattn_decode_args* a, int num_cus, DecodePlan* plan);

// Checks the new tokens of exattn_decode_append against the decode arguments
// (which plan_decode has accepted).
exattn_status check_append(const exattn_decode_args* a, const exattn_kv_new* n);

// Checked FP8 forward arguments, resolved for the launch.
struct Fp8Plan {
  bool empty = false;
  bool softcap = false, varlen = false;
  int head_dim = 0, group = 1, wl = -1, wr = -1;
  int s_q = 0, s_k = 0;  // lengths (fixed) or maxima (varlen)
  float scale_log2 = 0.f, v_descale = 1.f;
  float cap_in = 0.f, cap_out_log2 = 0.f;  // softcap: scale x descales / c, and c log2 e
};
exattn_status plan_fwd_fp8(const exattn_fwd_args* a, const exattn_fp8_descale* d, Fp8Plan* pl);

// Checked backward arguments, resolved for the launch.
struct BwdPlan {
  bool bf16 = false;
  bool softcap = false, varlen = false;
  float cap_in = 0.f, cap_out_log2 = 0.f;
  int s_q = 0, s_k = 0;  // lengths, or the largest ones (varlen)
  bool empty = false;  // nothing to compute (batch 0 or no query rows and no keys)
  int head_dim = 0, group = 1, wl = -1, wr = -1;
  float scale = 0.f, scale_log2 = 0.f;
  size_t ws_bytes = 0;
};
exattn_status plan_bwd(const exattn_bwd_args* a, BwdPlan* pl);

// Keys per step of the decode kernel for this head_dim and heads per work
// group: 16 times the waves that share one head slot (the kernel derives the
// same from its wave count and head slots).
int decode_keys_per_step(int head_dim, int hpw);

// Checks a paged-cache description against accepted decode arguments.
exattn_status check_paged(const exattn_decode_args* a, const DecodePlan& pl, const exattn_paged_kv* pg);


// Adjacent KV heads one decode work group covers: enough for a 2 KiB piece of
// every key row (16 at d = 64, 8 at d = 128, 4 at d = 256), rounded down to a
// power of two no larger than heads_kv.
int decode_heads_per_group(int head_dim, int heads_kv);

int32_t auto_splits(int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t seqlen_k,
                    int32_t head_dim, int32_t num_cus, int32_t seqlen_q = 1);

// Key-split prefill schedule (one (batch, head) unit; every unit runs the same).
// A work group has 4 slots of 2 waves; a slot covers one 64-row query tile and
// the key blocks kg, kg + kgn, kg + 2 kgn, ... of that tile's visible range
// (kgn slots per tile, consecutive within one work group, 1 <= kgn <= 4).
constexpr int kMaxSlots = 256;
struct SlotSchedule {
  int n_wg = 0;   // work groups per unit
  int steps = 0;  // the largest per-slot block count
  // per slot: tile (bits 0-15), kg (16-18), kgn (19-21), used (bit 24), and the
  // number of blocks it computes
  uint32_t slot[kMaxSlots] = {};
  uint32_t nb[kMaxSlots] = {};
};
// Visible 32-key blocks [lo, hi) of 64-row query tile t (bottom-right causal /
// window offsets; window edges < 0 unbounded).
void tile_key_blocks(int t, int s_q, int s_k, int wl, int wr, int* lo, int* hi);
// For n64 tiles with w[t] visible blocks each, in at most wg_max work groups
// per unit: the heaviest tiles get the most slots.  Returns false when the
// tiles do not fit.
bool build_slot_schedule(const int* w, int n64, int wg_max, SlotSchedule* out);

}  // namespace exattn
