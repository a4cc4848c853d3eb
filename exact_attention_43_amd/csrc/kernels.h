// Kernel parameter blocks and launcher entry points (internal to libexattn).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace exattn {

// Prefill forward: one work group per (query tile of 128 rows, query head,
// batch entry or sequence).  All strides are in elements.
struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t lse_sb, lse_sh;
  const int32_t* cu_q;  // varlen prefix sums, or nullptr
  const int32_t* cu_k;
  int32_t batch, s_q, s_k;  // s_q / s_k: lengths (fixed) or maxima (varlen)
  int32_t h_q, h_kv, group;
  int32_t n_qt;        // query tiles per (batch, head)
  int32_t xcd_group;   // 1: co-locate the query heads of one KV head on one XCD
  int32_t pair_tiles;  // 1: a two-group work group takes 64-row tiles j and n - 1 - j
  float scale_log2;    // softmax_scale * log2(e)
  float cap_in;        // softmax_scale / softcap
  float cap_out_log2;  // softcap * log2(e)
  int32_t wl, wr;      // window; wr = 0 for causal; < 0 unbounded
  uint32_t q_sign;     // 0x80008000 when the scale is negative: Q is negated, scale_log2 = |.|
  int32_t pack;        // 1: a tile packs the rows of the `group` query heads of one KV head
  int32_t grid3;       // set by the launcher: 1 for a (unit, batch, tile) grid, 0 for a linear one
};

// Split-KV decode: one work group per (split, KV head x query-head group, batch).
struct DecParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int64_t q_sb, q_sh, o_sb, o_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  const int32_t* cache_seqlens;  // or nullptr
  float* ws_o;                   // [split][batch][h_q][D] fp32 partial outputs
  float* ws_lse;                 // [split][batch][h_q] fp32 partial LSE
  int32_t batch, h_q, h_kv, group, s_cache;
  int32_t n_split, n_hg;  // splits; groups of 16 query columns per KV head
  // Several query tokens: query column c of a KV head is token c / group,
  // query head c % group; token t sits at position (keys - s_q + t), bottom-right.
  int32_t s_q;
  int64_t q_ss, o_ss;     // token strides of q and o
  int32_t wr;             // right window edge (0 for causal), < 0 unbounded
  int32_t hpw;            // adjacent KV heads per work group (a power of two)
  float scale_log2, cap_in, cap_out_log2;
  int32_t wl;
  // Append: seq_add new tokens (k_new / v_new, (batch, seq_add, h_kv, d) by
  // the kn_* / vn_* strides) are written to cache rows cache_seqlens[b] + t
  // and attended with the rest: keys per batch entry = cache_seqlens[b] + seq_add.
  int32_t seq_add;
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t kn_sb, kn_ss, kn_sh, vn_sb, vn_ss, vn_sh;
  // Paged cache (block_table != nullptr): k and v point to pools of num_pages
  // pages of page_size tokens (page strides k_sp / v_sp elements; k_ss, k_sh
  // within a page); token j of batch entry b lives in page
  // block_table[b * bt_stride + j / page_size], row j % page_size.
  // page_size is a multiple of the kernel's keys per step.
  const int32_t* block_table;
  int32_t bt_stride, page_size, num_pages;
  int64_t k_sp, v_sp;
};

// FP8 forward (dense layouts): Q, K, V as E4M3 codes (strides in elements =
// bytes), O bf16, LSE fp32 (b, h_q, s_q) or null.  scale_log2 folds the softmax
// scale, both Q and K descales and log2 e; v_descale multiplies O.
struct Fp8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  uint16_t* o;
  float* lse;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t lse_sb, lse_sh;
  int batch, s_q, s_k, h_q, h_kv, group;  // s_q / s_k: lengths (fixed) or maxima (varlen)
  float scale_log2, v_descale;
  int wl, wr;  // window edges, -1 = unbounded (wr = 0 for causal)
  float cap_in, cap_out_log2;  // softcap: scale x descales / c and c log2 e
  const int32_t* cu_q;  // varlen prefix sums (token offsets, batch strides ignored), or nullptr
  const int32_t* cu_k;
};

hipError_t launch_fwd_fp8(const Fp8Params& p, int head_dim, bool softcap, hipStream_t stream);

// Backward (dense layouts): dQ, dK, dV from Q, K, V, O, dO and the forward's LSE.
struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* ws_stats;  // [batch][h_q][s_q][2]: LSE log2 e (+inf for rows without keys), dO_i . O_i
  int64_t q_sb, q_ss, q_sh, k_sb, k_ss, k_sh, v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh, do_sb, do_ss, do_sh;
  int64_t dq_sb, dq_ss, dq_sh, dk_sb, dk_ss, dk_sh, dv_sb, dv_ss, dv_sh;
  int64_t lse_sb, lse_sh;
  int32_t batch, s_q, s_k, h_q, h_kv, group;
  float scale, scale_log2;
  float cap_in, cap_out_log2;  // softcap: scale / c and c log2 e (0 without softcap)
  int32_t wl, wr;  // wr = 0 for causal; < 0 unbounded
  int32_t bf16;
  // Varlen (cu_q != nullptr): sequence b spans rows cu_q[b] .. cu_q[b+1] - 1 of
  // q / o / dout / dq and cu_k[b] .. cu_k[b+1] - 1 of k / v / dk / dv (batch
  // strides ignored); s_q / s_k are the largest lengths.  LSE is (h_q, total_q).
  const int32_t* cu_q;
  const int32_t* cu_k;
};

// Key-split prefill (head_dim 128, fixed lengths): every (batch entry, query
// head) unit runs n_wg work groups, grid (h_q, batch, n_wg); work group w runs
// the 4 slots of slot[8 w .. 8 w + 7], as (entry, block count) pairs.  An entry
// holds a 64-row query tile (bits 0-15), its key group kg (bits 16-18) of kgn
// (bits 19-21) and a used bit (24); key group kg takes the tile's 32-key blocks
// lo + kg, lo + kg + kgn, ...  The kgn slots of a tile sit in one work group at
// consecutive positions, kg 0 first.
struct SlotParams {
  FwdParams f;
  int32_t n_wg, pad[3];
  alignas(32) uint32_t slot[2 * 256];  // starts at byte 256: a work group's 4 pairs are one 32-byte load
};
hipError_t launch_prefill_slots(const SlotParams& sp, bool bf16, bool softcap, hipStream_t stream);

// Head-dim-split prefill at head_dim 256 (not packed): two waves share 32 rows,
// one per half of the head dims.  groups 1: 128-row tiles, all 8 waves on the
// tile's key blocks; groups 2: 64-row tiles, two key groups of 4 waves.  Grid
// (h_q, batch, n_qt) with n_qt counted in tiles of that size.
hipError_t launch_prefill_dsplit(const FwdParams& p, bool bf16, int groups, bool softcap,
                                 hipStream_t stream);

int prefill_rows_per_tile();
// groups: 1 or 2 groups of 4 waves per work group (d = 256 always uses 1).
hipError_t launch_prefill(const FwdParams& p, bool bf16, int head_dim, bool softcap, int grid,
                          int groups, hipStream_t stream);
hipError_t launch_decode(const DecParams& p, bool bf16, int head_dim, bool softcap,
                         hipStream_t stream);

// Bytes of the static scratch array behind exattn_decode_noalloc (one per device).
constexpr size_t kDecodeScratchBytes = size_t(8) << 20;
// Device address of the current device's scratch array (looked up once per device).
hipError_t decode_scratch(void** ptr);
hipError_t launch_bwd(const BwdParams& p, int head_dim, bool softcap, hipStream_t stream);

}  // namespace exattn
