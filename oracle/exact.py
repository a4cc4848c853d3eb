"""CPU fp64 oracle for exact scaled-dot-product attention.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The GPU library never calls it and shares no code with it.

What it computes is the plain definition, written out and materialised:
S = scale * Q K^T, P = softmax(S), O = P V ("FlashAttention完整说明", section 一,
equations (1)-(3)).  The tiled method reaches this exactly up to rounding order
(same page, section 二.1; Inference Cookbook FAQ Q10), so there is no tiling,
no online softmax and no reordering here: every query row is scored against
every key, masked, normalised by an ordinary softmax and multiplied with V, in
float64 with numpy (matmul via the installed BLAS).

Semantics, each from the pages, with the readings taken where they are silent:
- layout (batch, seqlen, heads, head_dim) (FAQ Q5);
- default scale 1/sqrt(head_dim) (FAQ Q12);
- softcap c*tanh(s/c) applied to the scaled score before masking (FAQ Q22);
  reading: the scale is applied first and c <= 0 means "off";
- causal mask aligned to the bottom-right corner: with off = s_k - s_q, key j
  is visible to row i iff j <= i + off (FAQ Q6);
- window (left, right): row i sees keys in [i + off - left, i + off + right],
  both ends inclusive, a negative bound meaning unbounded; right = 0 is the
  causal case (FAQ Q21); reading: the same bottom-right offset applies to the
  window when s_q != s_k, and ``causal`` forces right = 0;
- a row with no visible key outputs O = 0 and LSE = -inf (reading of FAQ Q6's
  "no K to attend");
- LSE is the natural log of the sum of exp over the row's visible final scores
  ("FlashAttention完整说明", section 二.2 keeps only O and the softmax
  statistics);
- grouped heads: query head h reads KV head h // (h_q // h_kv) (FAQ Q15);
- variable length: sequences packed end to end and addressed by int32 prefix
  sums cu_seqlens (FAQ Q8); every sequence is attended on its own;
- KV-cache decode: the query attends to the first cache_seqlens[b] cache rows
  (FAQ Q17), with the bottom-right offset s_k - 1; with new tokens k, v the
  rows are first written at cache_seqlens[b] + t and the query attends to
  cache_seqlens[b] + s_new rows (reading: append, then attend, as the FAQ's
  example and its manual cache_seqlens update imply).
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


def _f64(x):
    """Upcast a numpy array or a torch tensor (any float dtype) to a float64 numpy array."""
    if hasattr(x, "detach"):  # torch tensor: fp16/bf16 -> fp32 is exact, fp32 -> fp64 is exact
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def default_scale(head_dim: int) -> float:
    """1/sqrt(d), the default softmax scale (FAQ Q12)."""
    return 1.0 / math.sqrt(head_dim)


def scores(q2, k2, scale):
    """S = scale * Q K^T for one head: (s_q, d) x (s_k, d) -> (s_q, s_k)."""
    return scale * (q2 @ k2.T)


def apply_softcap(s, softcap):
    """c * tanh(s / c) for c > 0, identity otherwise (FAQ Q22)."""
    if softcap is None or softcap <= 0.0:
        return s
    return softcap * np.tanh(s / softcap)


def visible(rows, s_q, s_k, causal, window_left, window_right):
    """Boolean (len(rows), s_k) mask: key j visible from query row i.

    off = s_k - s_q aligns the causal diagonal to the bottom-right (FAQ Q6);
    the window edges use the same offset (FAQ Q21).  Negative window bounds are
    unbounded; causal forces the right bound to 0.
    """
    rows = np.asarray(rows, dtype=np.int64)
    off = s_k - s_q
    wr = 0 if causal else window_right
    j = np.arange(s_k, dtype=np.int64)[None, :]
    i = rows[:, None]
    m = np.ones((rows.size, s_k), dtype=bool)
    if wr >= 0:
        m &= j <= i + off + wr
    if window_left >= 0:
        m &= j >= i + off - window_left
    return m


def softmax_rows(s, mask):
    """Row softmax over the visible entries; rows with nothing visible give P = 0.

    Returns (P, LSE) with LSE = m + ln(sum exp(s - m)) and -inf for empty rows.
    """
    s = np.where(mask, s, NEG_INF)
    any_vis = mask.any(axis=1)
    m = np.where(any_vis, s.max(axis=1, initial=NEG_INF), 0.0)
    e = np.where(mask, np.exp(s - m[:, None]), 0.0)
    ell = e.sum(axis=1)
    p = np.where(any_vis[:, None], e / np.where(ell > 0, ell, 1.0)[:, None], 0.0)
    lse = np.where(any_vis, m + np.log(np.where(ell > 0, ell, 1.0)), NEG_INF)
    return p, lse


def attend_head(q2, k2, v2, *, scale, causal=False, window_left=-1, window_right=-1,
                softcap=0.0, rows=None, return_probs=False):
    """Attention for one (query head, KV head) pair.

    q2 (s_q, d), k2 and v2 (s_k, d) as float64.  ``rows`` restricts the output to
    those query rows (each row depends only on itself), which keeps the
    16384-token shapes affordable.  Returns O (len(rows), d) and LSE (len(rows),)
    and, if asked, P (len(rows), s_k).
    """
    s_q, s_k = q2.shape[0], k2.shape[0]
    if rows is None:
        rows = np.arange(s_q)
    rows = np.asarray(rows, dtype=np.int64)
    if s_k == 0 or rows.size == 0:
        o = np.zeros((rows.size, v2.shape[1]))
        lse = np.full(rows.size, NEG_INF)
        p = np.zeros((rows.size, s_k))
        return (o, lse, p) if return_probs else (o, lse)
    s = scores(q2[rows], k2, scale)
    s = apply_softcap(s, softcap)
    mask = visible(rows, s_q, s_k, causal, window_left, window_right)
    p, lse = softmax_rows(s, mask)
    o = p @ v2
    return (o, lse, p) if return_probs else (o, lse)


def _kv_head(h, h_q, h_kv):
    if h_q % h_kv != 0:
        raise ValueError("heads_q must be a multiple of heads_kv")
    return h // (h_q // h_kv)


def attention(q, k, v, *, softmax_scale=None, causal=False, window_size=(-1, -1),
              softcap=0.0, rows=None, heads=None, return_probs=False):
    """Dense attention.  q (b, s_q, h_q, d); k, v (b, s_k, h_kv, d).

    Returns O (b, s_q, h_q, d) and LSE (b, h_q, s_q) as float64 (and P
    (b, h_q, s_q, s_k) if asked).  With ``rows`` (query indices) and/or ``heads``
    (query head indices) only those entries are computed; the others stay NaN.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    b, s_q, h_q, d = q.shape
    s_k, h_kv = k.shape[1], k.shape[2]
    dv = v.shape[3]
    scale = default_scale(d) if softmax_scale is None else float(softmax_scale)
    row_idx = np.arange(s_q) if rows is None else np.asarray(rows, dtype=np.int64)
    head_idx = range(h_q) if heads is None else heads
    o = np.full((b, s_q, h_q, dv), np.nan)
    lse = np.full((b, h_q, s_q), np.nan)
    p_all = np.zeros((b, h_q, s_q, s_k)) if return_probs else None
    wl, wr = window_size
    for bi in range(b):
        for h in head_idx:
            hk = _kv_head(h, h_q, h_kv)
            res = attend_head(q[bi, :, h, :], k[bi, :, hk, :], v[bi, :, hk, :], scale=scale,
                              causal=causal, window_left=wl, window_right=wr, softcap=softcap,
                              rows=row_idx, return_probs=return_probs)
            o[bi, row_idx, h, :] = res[0]
            lse[bi, h, row_idx] = res[1]
            if return_probs:
                p_all[bi, h][row_idx] = res[2]
    return (o, lse, p_all) if return_probs else (o, lse)


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, *, softmax_scale=None, causal=False,
                     window_size=(-1, -1), softcap=0.0):
    """Packed variable-length attention (FAQ Q8).

    q (total_q, h_q, d); k, v (total_k, h_kv, d); cu_seqlens_* int prefix sums
    of length batch + 1.  Each sequence is attended on its own, with its own
    bottom-right offset.  Returns O (total_q, h_q, d) and LSE (h_q, total_q).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cq = [int(x) for x in np.asarray(cu_seqlens_q).tolist()]
    ck = [int(x) for x in np.asarray(cu_seqlens_k).tolist()]
    total_q, h_q, d = q.shape
    h_kv = k.shape[1]
    scale = default_scale(d) if softmax_scale is None else float(softmax_scale)
    o = np.zeros((total_q, h_q, v.shape[2]))
    lse = np.full((h_q, total_q), NEG_INF)
    wl, wr = window_size
    for bi in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[bi], cq[bi + 1], ck[bi], ck[bi + 1]
        for h in range(h_q):
            hk = _kv_head(h, h_q, h_kv)
            ob, lb = attend_head(q[q0:q1, h, :], k[k0:k1, hk, :], v[k0:k1, hk, :], scale=scale,
                                 causal=causal, window_left=wl, window_right=wr, softcap=softcap)
            o[q0:q1, h, :] = ob
            lse[h, q0:q1] = lb
    return o, lse


def attention_kvcache(q, k_cache, v_cache, cache_seqlens=None, *, softmax_scale=None,
                      causal=False, window_size=(-1, -1), softcap=0.0, heads=None):
    """KV-cache decode (FAQ Q17): q (b, s_q, h_q, d) attends to the first
    cache_seqlens[b] rows of k_cache/v_cache (b, s_cache, h_kv, d).

    ``cache_seqlens`` None means the full cache.  Returns O (b, s_q, h_q, d) and
    LSE (b, h_q, s_q).
    """
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    b = q.shape[0]
    if cache_seqlens is None:
        lens = [kc.shape[1]] * b
    else:
        lens = [int(x) for x in np.asarray(cache_seqlens).tolist()]
    os_, ls_ = [], []
    for bi in range(b):
        n = lens[bi]
        ob, lb = attention(q[bi:bi + 1], kc[bi:bi + 1, :n], vc[bi:bi + 1, :n],
                           softmax_scale=softmax_scale, causal=causal, window_size=window_size,
                           softcap=softcap, heads=heads)
        os_.append(ob)
        ls_.append(lb)
    return np.concatenate(os_, axis=0), np.concatenate(ls_, axis=0)


def attention_backward(q, k, v, do, *, softmax_scale=None, causal=False, window_size=(-1, -1),
                       softcap=0.0):
    """Gradients of the dense forward (same arguments as ``attention``) for the
    upstream gradient dO (b, s_q, h_q, d): returns dQ, dK, dV (float64, shaped
    like q, k, v).

    The backward of "FlashAttention完整说明" section 二.2 recomputes S and P from
    Q, K and the kept statistics; what it computes is the chain rule through
    the definition, written out here per head with P materialised:
    dV = P^T dO; dP = dO V^T; dS = P * (dP - rowsum(P * dP)); through the
    softcap dS_raw = dS * (1 - tanh^2(s_raw / c)); dQ = scale dS_raw K and
    dK = scale dS_raw^T Q.  Masked entries have P = 0 and contribute nothing.
    A KV head's dK and dV sum over the query heads that read it (FAQ Q15).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    b, s_q, h_q, d = q.shape
    s_k, h_kv = k.shape[1], k.shape[2]
    scale = default_scale(d) if softmax_scale is None else float(softmax_scale)
    wl, wr = window_size
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for bi in range(b):
        for h in range(h_q):
            hk = _kv_head(h, h_q, h_kv)
            q2, k2, v2, do2 = q[bi, :, h], k[bi, :, hk], v[bi, :, hk], do[bi, :, h]
            if s_k == 0 or s_q == 0:
                continue
            _, _, p = attend_head(q2, k2, v2, scale=scale, causal=causal, window_left=wl,
                                  window_right=wr, softcap=softcap, return_probs=True)
            dv[bi, :, hk] += p.T @ do2
            dp = do2 @ v2.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            if softcap is not None and softcap > 0.0:
                t = np.tanh(scores(q2, k2, scale) / softcap)
                ds = ds * (1.0 - t * t)
            dq[bi, :, h] = scale * (ds @ k2)
            dk[bi, :, hk] += scale * (ds.T @ q2)
    return dq, dk, dv


def attention_backward_magnitudes(q, k, v, do, *, softmax_scale=None, causal=False,
                                  window_size=(-1, -1), softcap=0.0):
    """The size of the terms each gradient of ``attention_backward`` sums, for
    tolerances: a sum whose terms carry a relative rounding error u is off by
    at most about u times the sum of its terms' absolute values (the classic
    forward error bound of a dot product), however much the terms cancel.
    Written out through the backward's own sums, with every nested sum expanded
    into its terms: dS_ij = P_ij (dP_ij - D_i), and D_i = sum_k dO_ik O_ik is
    itself a sum over O_ik = sum_j' P_ij' V_j'k (the forward's output, which a
    backward takes from the forward with the forward's rounding), so its terms
    are dO_ik P_ij' V_j'k and dS_ij's terms have total size A_ij = P_ij (|dP_ij|
    + sum_k |dO_ik| sum_j' P_ij' |V_j'k|), times the softcap factor
    1 - tanh^2(s_raw / c) when softcap c > 0 (P then from the capped scores).
    The magnitudes returned are scale A |K|, scale A^T |Q| and P^T |dO| (dQ, dK,
    dV), summed over grouped heads like the gradients (the scale enters by its
    absolute value: these are sizes).  Each is >= the matching |gradient|, with
    equality for dV where dO >= 0.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    b, s_q, h_q, d = q.shape
    s_k, h_kv = k.shape[1], k.shape[2]
    scale = default_scale(d) if softmax_scale is None else float(softmax_scale)
    wl, wr = window_size
    mq = np.zeros_like(q)
    mk = np.zeros_like(k)
    mv = np.zeros_like(v)
    if s_k == 0 or s_q == 0:
        return mq, mk, mv
    for bi in range(b):
        for h in range(h_q):
            hk = _kv_head(h, h_q, h_kv)
            q2, k2, v2, do2 = q[bi, :, h], k[bi, :, hk], v[bi, :, hk], do[bi, :, h]
            _, _, p = attend_head(q2, k2, v2, scale=scale, causal=causal, window_left=wl,
                                  window_right=wr, softcap=softcap, return_probs=True)
            dp = do2 @ v2.T
            ov = p @ np.abs(v2)  # sum_j' P_ij' |V_j'k|: the size of O_ik's terms
            a = p * (np.abs(dp) + (np.abs(do2) * ov).sum(axis=1, keepdims=True))
            if softcap is not None and softcap > 0.0:
                t = np.tanh(scores(q2, k2, scale) / softcap)
                a = a * (1.0 - t * t)
            mv[bi, :, hk] += p.T @ np.abs(do2)
            mq[bi, :, h] = abs(scale) * (a @ np.abs(k2))
            mk[bi, :, hk] += abs(scale) * (a.T @ np.abs(q2))
    return mq, mk, mv


def decode_e4m3(codes):
    """Real values of OCP FP8 E4M3 codes (the variant without infinities): sign
    bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
    subnormal, (-1)^s 2^-6 m/8; S.1111.111 is NaN; the largest value is 448.
    Accepts uint8 codes or a torch float8_e4m3fn tensor (its bytes)."""
    x = codes
    if hasattr(x, "detach"):
        import torch
        x = x.detach().cpu().contiguous().view(torch.uint8).numpy()
    c = np.asarray(x).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return sign * val


def attention_fp8(q, k, v, *, q_descale=1.0, k_descale=1.0, v_descale=1.0, softmax_scale=None,
                  causal=False, window_size=(-1, -1), softcap=0.0, rows=None, heads=None):
    """The FP8 forward (FAQ Q20): Q, K, V are E4M3 codes whose real values are
    code x descale (one factor per tensor); the result is exact attention of
    those real values (default scale 1/sqrt(d)), with the same softcap and
    masks as the 16-bit forward (FAQ Q22: the cap on the scaled scores, before
    the mask).  The output precision (bf16) and the internal FP8 products are
    the kernel's business: the reference is the definition in float64."""
    return attention(decode_e4m3(q) * float(q_descale), decode_e4m3(k) * float(k_descale),
                     decode_e4m3(v) * float(v_descale), softmax_scale=softmax_scale, causal=causal,
                     window_size=window_size, softcap=softcap, rows=rows, heads=heads)


def kvcache_append(k_cache, v_cache, cache_seqlens, k_new, v_new):
    """The cache update of flash_attn_with_kvcache(q, k_cache, v_cache, k=k_new,
    v=v_new, cache_seqlens=...) (FAQ Q17): token t of k_new / v_new
    (b, s_new, h_kv, d) becomes cache row cache_seqlens[b] + t.

    Works on copies, in the caches' own storage type (a plain copy of the
    rows, no arithmetic), and returns (k_cache', v_cache').  Rows that would
    land outside the cache are dropped.
    """
    lens = [int(x) for x in np.asarray(cache_seqlens).tolist()]
    kc = k_cache.clone() if hasattr(k_cache, "clone") else np.array(k_cache, copy=True)
    vc = v_cache.clone() if hasattr(v_cache, "clone") else np.array(v_cache, copy=True)
    s_cache, s_new = kc.shape[1], k_new.shape[1]
    for bi, n in enumerate(lens):
        for t in range(s_new):
            if 0 <= n + t < s_cache:
                kc[bi, n + t] = k_new[bi, t]
                vc[bi, n + t] = v_new[bi, t]
    return kc, vc


def attention_kvcache_append(q, k_cache, v_cache, k_new, v_new, cache_seqlens, *, softmax_scale=None,
                             causal=False, window_size=(-1, -1), softcap=0.0, heads=None):
    """Decode with an append (FAQ Q17): the new tokens are written into the
    cache first, then q attends to the first cache_seqlens[b] + s_new rows.

    Returns O, LSE and the updated caches (k_cache', v_cache').
    """
    kc, vc = kvcache_append(k_cache, v_cache, cache_seqlens, k_new, v_new)
    lens = [int(x) + k_new.shape[1] for x in np.asarray(cache_seqlens).tolist()]
    o, lse = attention_kvcache(q, kc, vc, lens, softmax_scale=softmax_scale, causal=causal,
                               window_size=window_size, softcap=softcap, heads=heads)
    return o, lse, kc, vc


def paged_to_contiguous(pool, block_table, seqlen_cache):
    """A paged KV cache (FAQ Q18) as a contiguous one: pool (num_pages,
    page_size, h_kv, d); token j of batch entry b is row j % page_size of page
    block_table[b, j // page_size].  Returns (b, seqlen_cache, h_kv, d) in the
    pool's storage type (a gather of rows, no arithmetic)."""
    bt = np.asarray(block_table)
    page_size = pool.shape[1]
    rows = []
    for bi in range(bt.shape[0]):
        idx = [int(bt[bi, j // page_size]) for j in range(seqlen_cache)]
        off = [j % page_size for j in range(seqlen_cache)]
        rows.append(pool[idx, off])
    if hasattr(pool, "clone"):
        import torch  # the pool's own type; the gather above is torch/numpy agnostic
        return torch.stack(rows, 0)
    return np.stack(rows, 0)


def merge_partials(o_parts, lse_parts):
    """Combine attention results over disjoint key sets by their log-sum-exp.

    The merge of the online softmax ("FlashAttention完整说明", section 二.1):
    LSE = log sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s.  A part with
    LSE_s = -inf has weight 0; if every part is empty the result is O = 0,
    LSE = -inf.  o_parts: (S, ..., d); lse_parts: (S, ...).
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    finite = np.isfinite(m)
    m0 = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m0[None]), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(finite, m0 + np.log(np.where(tot > 0, tot, 1.0)), NEG_INF)
    wn = w / np.where(tot > 0, tot, 1.0)[None]
    o = (wn[..., None] * o_parts).sum(axis=0)
    o = np.where(finite[..., None], o, 0.0)
    return o, lse
