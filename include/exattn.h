/*
 * exattn: exact scaled-dot-product attention forward for AMD MI355X (gfx950).
 *
 * C ABI of libexattn.so.  Plain C types only; device buffers are passed as raw
 * device pointers and the stream as an opaque hipStream_t handle (void *, NULL
 * means the default stream).
 *
 * What is computed (per batch entry / sequence b and query head h, with KV head
 * h / (heads_q / heads_kv)):
 *   S = scale * Q K^T, P = softmax(S), O = P V
 * ("FlashAttention完整说明", section 一, equations (1)-(3)), evaluated tile by
 * tile with an online softmax so that S and P never reach device memory (same
 * page, section 二.1).  The forward keeps only O and the per-row softmax
 * statistics, returned as the natural-log LSE (same page, section 二.2).
 *
 * Masking semantics (Inference Cookbook FAQ):
 *   - causal: aligned to the bottom-right corner, off = seqlen_k - seqlen_q,
 *     key j visible to row i iff j <= i + off (Q6);
 *   - window (left, right): row i sees [i + off - left, i + off + right],
 *     inclusive; a negative bound is unbounded; causal forces right = 0 (Q21);
 *   - softcap c > 0: score -> c * tanh(score / c) after scaling and before
 *     masking (Q22); c <= 0 disables it;
 *   - a row that sees no key gets O = 0 and LSE = -inf.
 * The default scale is 1/sqrt(head_dim) (Q12), selected by softmax_scale = NaN;
 * any finite softmax_scale, 0 and negative values included, is used as given
 * (0 gives every visible key the same weight).
 *
 * Ownership and threading: the caller allocates and owns every buffer.  The
 * library keeps no pointer after a call returns, never allocates or frees
 * device memory, never synchronises and never reads device memory on the host,
 * so a call can be captured into a HIP graph with fixed addresses (Q19).  Its
 * only global state is a per-device cache of the compute-unit count.  Calls on
 * different streams may run concurrently; a call's kernels run in order on the
 * stream it is given.
 *
 * Errors: arguments are checked on the host before anything is launched; on a
 * failed check nothing is launched and the status says why, with detail text
 * from exattn_last_error() (thread-local).  Launch failures return
 * EXATTN_E_HIP.  Device-resident cu_seqlens / cache_seqlens cannot be checked
 * without a host read, so their validity is a precondition (see below).
 */
#ifndef EXATTN_H
#define EXATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EXATTN_ABI_VERSION 4

typedef enum {
  EXATTN_OK = 0,
  EXATTN_E_INVALID = 1,     /* bad argument: null pointer, negative size, head ratio, stride */
  EXATTN_E_UNSUPPORTED = 2, /* valid but not provided: dtype, head_dim */
  EXATTN_E_WORKSPACE = 3,   /* decode workspace missing or too small */
  EXATTN_E_HIP = 4          /* a HIP runtime call or kernel launch failed */
} exattn_status;

/* Storage type of Q, K, V (and O).  exattn_fwd, exattn_decode* and exattn_bwd
 * take fp16 or bf16 ("FlashAttention完整说明", section 八: half-precision types
 * only); EXATTN_FP8_E4M3 is accepted only by exattn_fwd_fp8 (Inference
 * Cookbook FAQ Q20), whose output is bf16.  Accumulation is fp32 throughout. */
typedef enum { EXATTN_F16 = 0, EXATTN_BF16 = 1, EXATTN_FP8_E4M3 = 2 } exattn_dtype;

/*
 * Prefill / general forward: flash_attn_func and its packed and varlen forms
 * (FAQ Q5 layout (batch, seqlen, heads, head_dim); Q7 kv-packed and
 * cross-attention; Q8 varlen; "FlashAttention完整说明" section 六.1 qkv-packed).
 *
 * Tensors are addressed by element strides over (batch, token, head); the
 * head_dim stride must be 1.  Packed layouts are passed as strided views with
 * no copy, e.g. qkv (b, s, 3, h, d) gives q, k, v with token stride 3*h*d and
 * base pointers offset by 0, h*d and 2*h*d elements.
 *
 * Fixed length (cu_seqlens_q == NULL): q (batch, seqlen_q, heads_q, head_dim),
 *   k and v (batch, seqlen_k, heads_kv, head_dim), o like q.
 * Variable length (cu_seqlens_q != NULL, cu_seqlens_k != NULL): sequences are
 *   packed end to end, q (total_q, heads_q, head_dim), k/v (total_k, heads_kv,
 *   head_dim); the batch stride is ignored; sequence b spans tokens
 *   [cu_seqlens_q[b], cu_seqlens_q[b+1]) of q and [cu_seqlens_k[b],
 *   cu_seqlens_k[b+1]) of k/v.  Precondition: both arrays are int32 device
 *   arrays of batch + 1 non-decreasing entries starting at 0, and no sequence
 *   is longer than max_seqlen_q / max_seqlen_k (host values that size the grid).
 *
 * lse: fp32 device buffer, element (b, h, i) at
 *   lse[b * lse_stride[0] + h * lse_stride[1] + i]; for fixed length the usual
 *   layout is (batch, heads_q, seqlen_q); for varlen i is the packed token
 *   index and the batch stride is ignored (layout (heads_q, total_q)).
 *   lse may be NULL when the caller does not want it.
 */
typedef struct {
  int32_t dtype; /* exattn_dtype */
  int32_t batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim;
  const void *q, *k, *v;
  void *o;
  float *lse;
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3]; /* elements: batch, token, head */
  int64_t lse_stride[2];                                       /* elements: batch, head */
  const int32_t *cu_seqlens_q, *cu_seqlens_k;                  /* device int32[batch+1] or NULL */
  int32_t max_seqlen_q, max_seqlen_k;                          /* varlen only */
  float softmax_scale; /* NaN: 1/sqrt(head_dim); any finite value (0 included) as given */
  float softcap;       /* <= 0: off */
  int32_t causal;      /* nonzero: bottom-right causal, forces window_right = 0 */
  int32_t window_left, window_right; /* < 0: unbounded */
  /* Packed GQA (FAQ Q15): 1 = one query tile holds the rows of all
   * heads_q / heads_kv query heads that read one KV head (position-major, head
   * fastest), so short query sequences fill the tiles; 0 = one tile per query
   * head; -1 = automatic (packed when that takes fewer work groups).  The
   * results are the same either way: bitwise equal whenever both launches use
   * the same kernel variant (the variant depends on the grid size), else within
   * rounding (each row then sums its key blocks in another grouping).  Other
   * values: EXATTN_E_INVALID.  exattn_fwd_fp8 ignores it. */
  int32_t pack_gqa;
} exattn_fwd_args;

/* Run the forward.  head_dim must be 64, 128 or 256; heads_q % heads_kv == 0.
 * Sizes of 0 (batch, seqlen_q) launch nothing and return EXATTN_OK; seqlen_k
 * of 0 writes O = 0 and LSE = -inf.  Strides must be non-negative multiples
 * of 8 elements (EXATTN_E_INVALID); a token stride (index 1) of q, k or v of
 * 2^24 elements or more returns EXATTN_E_UNSUPPORTED (the kernels address a
 * 64-row tile with 32-bit byte offsets). */
exattn_status exattn_fwd(const exattn_fwd_args *args, void *stream);

/*
 * KV-cache decode: flash_attn_with_kvcache (FAQ Q17) for one or a few query
 * tokens, split over the key axis into num_splits parts whose partial results
 * are merged by their log-sum-exp (FAQ Q14; the merge is the online-softmax
 * merge of "FlashAttention完整说明" section 二.1).
 *
 * q (batch, seqlen_q, heads_q, head_dim) addressed by q_stride (batch, head)
 * and q_token_stride; o the same by o_stride and o_token_stride; k_cache and
 * v_cache (batch, seqlen_cache, heads_kv, head_dim) by k_stride / v_stride
 * (batch, token, head); lse fp32 (batch, heads_q, seqlen_q) contiguous, or
 * NULL.  The query tokens of all heads_q / heads_kv query heads of a KV head
 * share each key read (up to 16 of them per pass over the keys).
 * cache_seqlens: device int32[batch], the number of valid cache rows per batch
 * entry, or NULL for seqlen_cache.  The caller maintains it (FAQ Q17: the call
 * never advances it).  Precondition: 0 <= cache_seqlens[b] <= seqlen_cache.
 * With one query token it sits at position cache_seqlens[b] - 1
 * (bottom-right), so causal changes nothing and only window_left narrows the
 * keys; with seqlen_q > 1 see the field below.
 * num_splits: 0 = automatic (compute-unit count, KV size per split, length);
 * otherwise the number of key ranges, clamped to [1, 256].
 */
typedef struct {
  int32_t dtype; /* exattn_dtype */
  int32_t batch, heads_q, heads_kv, head_dim, seqlen_cache;
  const void *q, *k_cache, *v_cache;
  void *o;
  float *lse;
  int64_t q_stride[2], o_stride[2];  /* elements: batch, head */
  int64_t k_stride[3], v_stride[3];  /* elements: batch, token, head */
  const int32_t *cache_seqlens;      /* device int32[batch] or NULL */
  float softmax_scale;               /* NaN: 1/sqrt(head_dim); else as given */
  float softcap;                     /* <= 0: off */
  int32_t causal;
  int32_t window_left, window_right; /* < 0: unbounded */
  int32_t num_splits;                /* 0: automatic */
  /* Query tokens per batch entry (0 is taken as 1), e.g. the s_new tokens of
   * an append (FAQ Q17 with causal) or a few speculative tokens.  Token t sits
   * at position len - seqlen_q + t of the len = cache_seqlens[b] (+ seqlen_new)
   * keys, so causal and the window are bottom-right aligned (FAQ Q6, Q21);
   * a token before position 0 sees no key (O = 0, LSE = -inf).  q and o are
   * (batch, seqlen_q, heads_q, head_dim) with these token strides (elements,
   * multiples of 8); lse is (batch, heads_q, seqlen_q) contiguous. */
  int32_t seqlen_q;
  int64_t q_token_stride, o_token_stride;
} exattn_decode_args;

/* Host-only: resolve num_splits and the workspace size (bytes) that
 * exattn_decode needs for these arguments on the current device.  Either
 * output pointer may be NULL. */
exattn_status exattn_decode_plan(const exattn_decode_args *args, int32_t *num_splits_out,
                                 size_t *workspace_bytes_out);

/* Run the decode.  workspace: device buffer of at least the planned size,
 * 256-byte aligned, owned by the caller, used as scratch for the partial
 * results (fp32 O and LSE per split); its contents on entry do not matter.
 * With one split the workspace may be NULL.  Calls that share a workspace
 * must be ordered on one stream. */
exattn_status exattn_decode(const exattn_decode_args *args, void *workspace,
                            size_t workspace_bytes, void *stream);

/* exattn_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the split partials go to a static scratch array of 8 MiB that the library
 * keeps on every device it runs on until the process ends, instead of a caller
 * workspace.  Allocates nothing (no hipMalloc, no hipFree); the first call on a
 * device looks up that device's array.  A plan whose partials need more than
 * 8 MiB (splits x batch x heads_q x (head_dim + 1) x 4 bytes, rounded up)
 * returns EXATTN_E_WORKSPACE with nothing launched: pass a smaller num_splits
 * or use exattn_decode.  All calls on one device share the array and it keeps
 * the last call's contents (nothing in it has to start at zero); calls that
 * overlap on one device race on it, so order them on one stream.  Arguments,
 * results and errors otherwise as exattn_decode. */
exattn_status exattn_decode_noalloc(const exattn_decode_args *args, void *stream);

/*
 * New tokens for exattn_decode_append: flash_attn_with_kvcache called with
 * k=k_new, v=v_new (FAQ Q17).  k_new and v_new are (batch, seqlen_new,
 * heads_kv, head_dim) in the cache's dtype, addressed by k_new_stride /
 * v_new_stride (elements: batch, token, head; last dimension contiguous),
 * 16-byte aligned, strides multiples of 8 elements.
 */
typedef struct {
  const void *k_new, *v_new;
  int32_t seqlen_new;
  int64_t k_new_stride[3], v_new_stride[3];
} exattn_kv_new;

/* KV-cache decode with an append (FAQ Q17): for every batch entry b, new
 * token t is first written to cache row cache_seqlens[b] + t of k_cache and
 * v_cache, then the query attends to the first cache_seqlens[b] + seqlen_new
 * rows exactly as exattn_decode does (the query sits at the last of them).
 * cache_seqlens must not be NULL, and, as in the FAQ, the call does not
 * advance it: the caller adds seqlen_new afterwards.  Precondition:
 * 0 <= cache_seqlens[b] and cache_seqlens[b] + seqlen_new <= seqlen_cache;
 * new rows that would fall outside [0, seqlen_cache) are not written and the
 * attended length is clamped to seqlen_cache, so a violated precondition
 * gives wrong values but no out-of-bounds access.  Cache rows other than the
 * new ones are left unchanged.  workspace as for exattn_decode (the same
 * plan applies: exattn_decode_plan on args).  seqlen_new = 0 is exattn_decode.
 * The rows are written by the decode kernel itself, each by the work groups
 * that read them, before they read them. */
exattn_status exattn_decode_append(const exattn_decode_args *args, const exattn_kv_new *kv_new,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * Paged KV cache (FAQ Q18): k_cache and v_cache of exattn_decode_args point to
 * pools of num_pages pages, each page_size tokens of (heads_kv, head_dim);
 * k_page_stride / v_page_stride are the page strides and k_stride[1..2] /
 * v_stride[1..2] the token and head strides inside a page (k_stride[0] and
 * v_stride[0] are ignored).  Token j of batch entry b lives in page
 * block_table[b * block_table_stride + j / page_size], row j % page_size.
 * block_table: device int32, at least ceil(seqlen_cache / page_size) entries
 * per batch entry; seqlen_cache is the capacity of one sequence.
 * page_size must be a multiple of the decode kernel's keys per step (16 for
 * head_dim 128 with 8 or more KV heads; always satisfied by multiples of 128);
 * other sizes are rejected with EXATTN_E_UNSUPPORTED.  Page indices outside
 * [0, num_pages) are clamped (a precondition violation, memory-safe).
 */
typedef struct {
  const int32_t *block_table;
  int32_t block_table_stride; /* entries per batch entry */
  int32_t page_size, num_pages;
  int64_t k_page_stride, v_page_stride; /* elements */
} exattn_paged_kv;

/* exattn_decode (kv_new NULL) or exattn_decode_append over a paged cache: the
 * same computation, the new rows written into their pages.  The plan and the
 * workspace are those of exattn_decode_plan on args. */
exattn_status exattn_decode_paged(const exattn_decode_args *args, const exattn_paged_kv *paged,
                                  const exattn_kv_new *kv_new, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * Backward of the dense forward: dQ, dK, dV from Q, K,
 * V, the forward's O and LSE, and the upstream gradient dO, recomputing S and
 * P ("FlashAttention完整说明", section 二.2: only O and the softmax statistics
 * are kept).  Same layouts, masks and softcap as exattn_fwd, fixed length or
 * varlen (element strides over batch, token, head; head_dim contiguous); dq
 * like q, dk and dv like k and v; lse as exattn_fwd writes it (fp32, element
 * (b, h, i) at lse[b * lse_stride[0] + h * lse_stride[1] + i]; varlen i is the
 * packed token).  With softcap c the gradient flows through c tanh(s / c)
 * (FAQ Q22), i.e. dS is multiplied by 1 - tanh^2.  A KV head's dK and dV sum
 * over the query heads that read it.  Deterministic (no atomics).
 * head_dim 64, 128 or 256.
 * workspace: batch * heads_q * seqlen_q (varlen: max_seqlen_q) * 8 bytes
 * rounded up to 256 (exattn_bwd_plan), 256-byte aligned, scratch owned by the
 * caller.
 * Errors (nothing launched): EXATTN_E_INVALID for NULL or misaligned pointers,
 * negative sizes or strides that are not non-negative multiples of 8 elements;
 * EXATTN_E_UNSUPPORTED as above; EXATTN_E_WORKSPACE for a missing, short or
 * misaligned workspace; EXATTN_E_HIP when a launch fails.  Empty problems
 * (batch 0, or no rows and no keys) launch nothing and return EXATTN_OK.
 */
typedef struct {
  int32_t dtype; /* exattn_dtype */
  int32_t batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim;
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3], dout_stride[3];
  int64_t dq_stride[3], dk_stride[3], dv_stride[3];
  int64_t lse_stride[2];
  float softmax_scale; /* NaN: 1/sqrt(head_dim); else as given */
  float softcap;       /* <= 0: off; > 0 as in the forward */
  int32_t causal;
  int32_t window_left, window_right;
  /* Varlen (both non-NULL): int32 device arrays of batch + 1 prefix sums as
   * for exattn_fwd; q, o, dout, dq are (total_q, heads_q, head_dim), k, v, dk,
   * dv (total_k, heads_kv, head_dim), the batch strides are ignored, lse is
   * (heads_q, total_q) as exattn_fwd writes it, and max_seqlen_q /
   * max_seqlen_k bound every sequence (they size the grids). */
  const int32_t *cu_seqlens_q, *cu_seqlens_k;
  int32_t max_seqlen_q, max_seqlen_k;
} exattn_bwd_args;

/* Host-only: the workspace size (bytes) exattn_bwd needs for these arguments. */
exattn_status exattn_bwd_plan(const exattn_bwd_args *args, size_t *workspace_bytes_out);

/* Run the backward: three kernels in order on the stream. */
exattn_status exattn_bwd(const exattn_bwd_args *args, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * FP8 forward with a bf16 output (Inference Cookbook FAQ Q20: FP8 inside, BF16
 * out; FAQ Q10 gives FP8 a 1e-2 tolerance).  args as for exattn_fwd with
 * dtype = EXATTN_FP8_E4M3: q, k, v hold OCP FP8 E4M3 codes (1 byte each; the
 * strides count elements, which are bytes here), o is bf16 (b, s_q, h_q, d),
 * lse as for exattn_fwd (or NULL).  The real inputs are code x descale, one
 * fp32 factor per tensor; S = softmax_scale q_descale k_descale (Q K^T) runs
 * on the FP8 MFMA, P V on the bf16 MFMA against V widened exactly from FP8,
 * and O is multiplied by v_descale.  Provided: head_dim 64 and 128 (else
 * EXATTN_E_UNSUPPORTED), fixed lengths or varlen (cu_seqlens as for exattn_fwd),
 * causal and window masks, GQA, softcap (on the scaled real scores, FAQ Q22).
 * Errors as for exattn_fwd; in addition q, k, v strides must be non-negative
 * multiples of 16 elements, o strides multiples of 8, and descale NULL or its
 * factors finite (EXATTN_E_INVALID).  descale NULL means all factors 1.
 */
typedef struct {
  float q, k, v;
} exattn_fp8_descale;

exattn_status exattn_fwd_fp8(const exattn_fwd_args *args, const exattn_fp8_descale *descale, void *stream);

/* The automatic split count, as a pure function (no device query).  One work
 * group covers up to 1024/head_dim adjacent KV heads (16 at d = 64, 8 at
 * d = 128, 4 at d = 256; a power of two no larger than heads_kv) and 16 of
 * their query heads, and one work group runs per compute unit.  The key axis
 * is split so that these units times splits fill num_cus work groups, while
 * each split keeps at least 256 keys (FAQ Q14's rules). */
int32_t exattn_decode_auto_splits(int32_t batch, int32_t heads_q, int32_t heads_kv,
                                  int32_t seqlen_k, int32_t head_dim, int32_t num_cus);

/* sizeof(exattn_fwd_args) for which = 0, sizeof(exattn_decode_args) for which = 1,
 * sizeof(exattn_kv_new) for which = 2, sizeof(exattn_paged_kv) for which = 3,
 * sizeof(exattn_bwd_args) for which = 4, sizeof(exattn_fp8_descale) for which = 5,
 * 0 otherwise: lets a binding check its
 * mirror of the structs. */
size_t exattn_args_size(int32_t which);

const char *exattn_status_string(int32_t status);
const char *exattn_last_error(void);
int32_t exattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXATTN_H */
