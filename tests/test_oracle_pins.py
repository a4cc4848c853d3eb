"""Pins of the CPU oracle to facts the pages and the mathematics fix.

None of these re-types the oracle's formulas: they use a scalar brute force
written separately, a library routine (PyTorch SDPA on the CPU in float64 with an
explicit mask), closed forms (Q = 0 turns every visible score into 0, so O is
the mean of the visible V rows and LSE = ln(count)), invariants, and the small
fixtures under tests/golden that restate values the pages print.

Every pin is a plain function that raises AssertionError.  ``test_pin`` runs each
against the oracle; ``test_planted_mistake_is_caught`` plants plausible mistakes
in the oracle (on the CPU, by monkeypatching) and checks that some pin fails.
"""
import math

import numpy as np
import pytest
import torch

import golden_io
import oracle
import oracle.exact as OA
from exact_attention_43_amd import workloads

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rng(seed):
    return np.random.default_rng(seed)


def _visible_count(i, s_q, s_k, causal, wl, wr):
    """Number of keys row i may see, counted from the interval ends (no mask matrix)."""
    off = s_k - s_q
    hi = s_k - 1
    if causal:
        wr = 0
    if wr >= 0:
        hi = min(hi, i + off + wr)
    lo = 0
    if wl >= 0:
        lo = max(lo, i + off - wl)
    return max(0, hi - lo + 1), lo, hi


# ----------------------------------------------------------------------------
# brute force: a scalar loop with math.exp / math.fsum, its own mask logic
# ----------------------------------------------------------------------------
def _brute(q, k, v, scale, causal, wl, wr, softcap):
    b, s_q, h_q, d = q.shape
    s_k, h_kv = k.shape[1], k.shape[2]
    g = h_q // h_kv
    o = np.zeros((b, s_q, h_q, v.shape[3]))
    lse = np.zeros((b, h_q, s_q))
    for bi in range(b):
        for h in range(h_q):
            hk = h // g
            for i in range(s_q):
                vis = []
                for j in range(s_k):
                    # bottom-right alignment: row i lines up with key i + (s_k - s_q)
                    diag = i + (s_k - s_q)
                    ok = True
                    right = 0 if causal else wr
                    if right >= 0 and j > diag + right:
                        ok = False
                    if wl >= 0 and j < diag - wl:
                        ok = False
                    if ok:
                        sc = math.fsum(float(q[bi, i, h, t]) * float(k[bi, j, hk, t]) for t in range(d)) * scale
                        if softcap > 0:
                            sc = softcap * math.tanh(sc / softcap)
                        vis.append((j, sc))
                if not vis:
                    lse[bi, h, i] = -math.inf
                    continue
                mx = max(sc for _, sc in vis)
                ws = [(j, math.exp(sc - mx)) for j, sc in vis]
                tot = math.fsum(w for _, w in ws)
                lse[bi, h, i] = mx + math.log(tot)
                for t in range(v.shape[3]):
                    o[bi, i, h, t] = math.fsum(w * float(v[bi, j, hk, t]) for j, w in ws) / tot
    return o, lse


BRUTE_CASES = [
    # s_q, s_k, causal, wl, wr, softcap, h_q, h_kv
    (1, 1, False, -1, -1, 0.0, 2, 2),
    (3, 5, True, -1, -1, 0.0, 2, 1),
    (5, 3, True, -1, -1, 0.0, 2, 2),
    (8, 8, False, 2, 1, 0.0, 2, 2),
    (5, 8, False, 1, -1, 3.0, 2, 1),
    (8, 5, True, 2, -1, 0.5, 2, 2),
    (2, 3, False, -1, 0, 0.0, 2, 2),
]


def pin_bruteforce():
    for n, (s_q, s_k, causal, wl, wr, cap, h_q, h_kv) in enumerate(BRUTE_CASES):
        r = _rng(100 + n)
        d = 4
        q = r.standard_normal((1, s_q, h_q, d)) * 1.5
        k = r.standard_normal((1, s_k, h_kv, d)) * 1.5
        v = r.standard_normal((1, s_k, h_kv, d))
        scale = 0.7
        ob, lb = _brute(q, k, v, scale, causal, wl, wr, cap)
        oo, lo = oracle.attention(q, k, v, softmax_scale=scale, causal=causal, window_size=(wl, wr),
                                  softcap=cap)
        assert np.allclose(oo, ob, atol=1e-12, rtol=1e-12), f"O mismatch in case {n}"
        assert np.array_equal(np.isinf(lo), np.isinf(lb)), f"empty-row mismatch in case {n}"
        fin = np.isfinite(lb)
        assert np.allclose(lo[fin], lb[fin], atol=1e-12, rtol=0), f"LSE mismatch in case {n}"


# ----------------------------------------------------------------------------
# library routine: torch SDPA (CPU, float64) with an explicit bottom-right mask
# ----------------------------------------------------------------------------
def pin_sdpa():
    r = _rng(7)
    for (s_q, s_k, causal, wl, wr) in [(16, 16, True, -1, -1), (8, 24, True, 5, -1),
                                       (24, 8, True, -1, -1), (12, 12, False, 3, 2),
                                       (10, 30, False, -1, -1)]:
        b, h, d = 2, 3, 16
        q = r.standard_normal((b, s_q, h, d))
        k = r.standard_normal((b, s_k, h, d))
        v = r.standard_normal((b, s_k, h, d))
        oo, lo = oracle.attention(q, k, v, causal=causal, window_size=(wl, wr))
        mask = np.zeros((s_q, s_k), dtype=bool)
        for i in range(s_q):
            n, lo_i, hi_i = _visible_count(i, s_q, s_k, causal, wl, wr)
            if n:
                mask[i, lo_i:hi_i + 1] = True
        tq = torch.from_numpy(q).transpose(1, 2)
        tk = torch.from_numpy(k).transpose(1, 2)
        tv = torch.from_numpy(v).transpose(1, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=torch.from_numpy(mask)).transpose(1, 2).numpy()
        rows = mask.any(axis=1)
        assert np.allclose(oo[:, rows], ref[:, rows], atol=1e-12, rtol=1e-12)
        assert np.all(oo[:, ~rows] == 0)


# ----------------------------------------------------------------------------
# invariants and closed forms
# ----------------------------------------------------------------------------
def pin_softmax_rows():
    r = _rng(11)
    q = r.standard_normal((1, 20, 2, 8))
    k = r.standard_normal((1, 12, 2, 8))
    v = r.standard_normal((1, 12, 2, 8))
    _, lse, p = oracle.attention(q, k, v, causal=True, window_size=(4, -1), return_probs=True)
    assert np.all(p >= 0)
    for i in range(20):
        n, lo, hi = _visible_count(i, 20, 12, True, 4, -1)
        row = p[0, :, i, :]
        if n == 0:
            assert np.all(row == 0) and np.all(np.isneginf(lse[0, :, i]))
        else:
            assert np.allclose(row.sum(axis=-1), 1.0, atol=1e-12)
            outside = np.ones(12, dtype=bool)
            outside[lo:hi + 1] = False
            assert np.all(row[:, outside] == 0)


def pin_sk1():
    r = _rng(12)
    q = r.standard_normal((2, 5, 3, 16))
    k = r.standard_normal((2, 1, 3, 16))
    v = r.standard_normal((2, 1, 3, 16))
    o, lse = oracle.attention(q, k, v, softmax_scale=0.3)
    assert np.allclose(o, np.broadcast_to(v, o.shape), atol=1e-14)
    for bi in range(2):
        for h in range(3):
            for i in range(5):
                s00 = 0.3 * math.fsum(q[bi, i, h] * k[bi, 0, h])
                assert abs(lse[bi, h, i] - s00) < 1e-12
    # causal with s_k = 1: only the last query row sees key 0 (bottom-right)
    o, lse = oracle.attention(q, k, v, causal=True)
    assert np.all(o[:, :4] == 0) and np.all(np.isneginf(lse[:, :, :4]))
    assert np.allclose(o[:, 4], v[:, 0], atol=1e-14)


def pin_identical_v_rows():
    r = _rng(13)
    q = r.standard_normal((1, 9, 2, 8)) * 3
    k = r.standard_normal((1, 7, 2, 8)) * 3
    row = r.standard_normal(8)
    v = np.broadcast_to(row, (1, 7, 2, 8)).copy()
    o, _ = oracle.attention(q, k, v, causal=True, window_size=(3, -1))
    for i in range(9):
        n, _, _ = _visible_count(i, 9, 7, True, 3, -1)
        assert np.allclose(o[0, i], row if n else 0.0, atol=1e-13)


COUNT_CASES = [
    # s_q, s_k, causal, wl, wr, h_q, h_kv
    (16, 16, True, -1, -1, 2, 2),
    (128, 64, True, -1, -1, 2, 1),
    (32, 100, True, -1, -1, 4, 2),
    (40, 40, False, 5, 3, 2, 2),
    (40, 60, False, 7, 0, 2, 2),
    (50, 20, False, -1, 4, 2, 2),
    (64, 64, True, 10, -1, 4, 1),
]


def _zero_q_check(s_q, s_k, causal, wl, wr, h_q, h_kv, seed):
    r = _rng(seed)
    d = 8
    q = np.zeros((1, s_q, h_q, d))
    k = r.standard_normal((1, s_k, h_kv, d))
    v = r.standard_normal((1, s_k, h_kv, d))
    o, lse = oracle.attention(q, k, v, causal=causal, window_size=(wl, wr), softcap=30.0)
    g = h_q // h_kv
    for i in range(s_q):
        n, lo, hi = _visible_count(i, s_q, s_k, causal, wl, wr)
        for h in range(h_q):
            if n == 0:
                assert np.all(o[0, i, h] == 0) and np.isneginf(lse[0, h, i])
            else:
                mean = v[0, lo:hi + 1, h // g].sum(axis=0) / n
                assert np.allclose(o[0, i, h], mean, atol=1e-13)
                assert abs(lse[0, h, i] - math.log(n)) < 1e-13


def pin_zero_q_counts():
    for n, c in enumerate(COUNT_CASES):
        _zero_q_check(*c, seed=200 + n)


def pin_bottom_right_causal():
    # s_q = 128 > s_k = 64: rows 0..63 see nothing, row i >= 64 sees i - 63 keys
    q = np.zeros((1, 128, 1, 4))
    k = _rng(3).standard_normal((1, 64, 1, 4))
    v = _rng(4).standard_normal((1, 64, 1, 4))
    o, lse = oracle.attention(q, k, v, causal=True)
    assert np.all(o[0, :64] == 0) and np.all(np.isneginf(lse[0, 0, :64]))
    for i in range(64, 128):
        assert abs(lse[0, 0, i] - math.log(i - 63)) < 1e-13
    # s_q = 512 < s_k = 2048: row i sees i + 1537 keys (the prefix is visible to all rows)
    q = np.zeros((1, 512, 1, 4))
    k = _rng(5).standard_normal((1, 2048, 1, 4))
    v = _rng(6).standard_normal((1, 2048, 1, 4))
    rows = np.array([0, 1, 100, 511])
    o, lse = oracle.attention(q, k, v, causal=True, rows=rows)
    for i in rows:
        assert abs(lse[0, 0, i] - math.log(i + 1537)) < 1e-13
        assert np.allclose(o[0, i, 0], v[0, :i + 1537, 0].mean(axis=0), atol=1e-13)


def pin_window_fixture():
    fx = golden_io.as_dict("faq_q21_window.txt")
    wl, wr, s = int(fx["window_left"][0]), int(fx["window_right"][0]), int(fx["seqlen"][0])
    rows = [list(map(int, r)) for r in fx["row"]]
    idx = np.array([r[0] for r in rows])
    k = _rng(8).standard_normal((1, s, 1, 4))
    v = _rng(9).standard_normal((1, s, 1, 4))
    q = np.zeros((1, s, 1, 4))
    for causal in (False, True):  # right = 0 is causal on its own; causal=True changes nothing
        o, lse = oracle.attention(q, k, v, causal=causal, window_size=(wl, wr), rows=idx)
        for i, lo, hi in rows:
            n = hi - lo + 1
            assert n == min(i, 256) + 1
            assert abs(lse[0, 0, i] - math.log(n)) < 1e-13
            assert np.allclose(o[0, i, 0], v[0, lo:hi + 1, 0].mean(axis=0), atol=1e-13)


def pin_shift_invariance():
    r = _rng(14)
    q = r.standard_normal((1, 12, 2, 16))
    k = r.standard_normal((1, 12, 2, 16))
    v = r.standard_normal((1, 12, 2, 16))
    c = r.standard_normal(16) * 300.0
    o1, l1 = oracle.attention(q, k, v, causal=True)
    o2, l2 = oracle.attention(q, k + c, v, causal=True)
    scale = 1 / 4.0
    assert np.allclose(o1, o2, atol=1e-9)
    shift = scale * np.einsum("bshd,d->bhs", q, c)
    assert np.allclose(l2 - l1, shift, atol=1e-9)


def pin_merge_identity():
    r = _rng(15)
    q = r.standard_normal((2, 6, 4, 16))
    k = r.standard_normal((2, 40, 2, 16))
    v = r.standard_normal((2, 40, 2, 16))
    full_o, full_l = oracle.attention(q, k, v)
    for cuts in ([17], [0, 40], [5, 5, 30], [1, 2, 3, 39]):
        edges = [0] + cuts + [40]
        os_, ls_ = [], []
        for a, b in zip(edges[:-1], edges[1:]):
            o, l = oracle.attention(q, k[:, a:b], v[:, a:b])
            os_.append(o)
            ls_.append(np.moveaxis(l, 1, 2))  # (b, s, h) to line up with o's leading dims
        mo, ml = oracle.merge_partials(os_, ls_)
        assert np.allclose(mo, full_o, atol=1e-12)
        assert np.allclose(np.moveaxis(ml, 2, 1), full_l, atol=1e-12)
    mo, ml = oracle.merge_partials([np.zeros((3, 4)), np.zeros((3, 4))], [np.full(3, -np.inf)] * 2)
    assert np.all(mo == 0) and np.all(np.isneginf(ml))


def pin_gqa_repeat():
    r = _rng(16)
    q = r.standard_normal((2, 10, 8, 8))
    k = r.standard_normal((2, 14, 2, 8))
    v = r.standard_normal((2, 14, 2, 8))
    o1, l1 = oracle.attention(q, k, v, causal=True)
    o2, l2 = oracle.attention(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), causal=True)
    assert np.allclose(o1, o2, atol=1e-14) and np.allclose(l1, l2, atol=1e-14)


def pin_varlen():
    fx = golden_io.as_dict("faq_q8_cu_seqlens.txt")
    lens = [int(x) for x in fx["seqlens"]]
    q, k, v, cu_q, cu_k = workloads.varlen_qkv(lens, lens, 4, 2, 8, seed=17, dtype=torch.float32)
    assert cu_q.tolist() == [int(x) for x in fx["cu_seqlens"]]
    assert cu_q.dtype == torch.int32
    # Q = 0: each row of each sequence averages its own visible keys only
    q = torch.zeros_like(q)
    o, lse = oracle.attention_varlen(q, k, v, cu_q, cu_k, causal=True, window_size=(30, 0))
    vv = v.double().numpy()
    for bi, n_seq in enumerate(lens):
        base = int(cu_q[bi])
        for i in (0, 1, 29, 30, 31, n_seq - 1):
            n, lo, hi = _visible_count(i, n_seq, n_seq, True, 30, 0)
            for h in range(4):
                assert abs(lse[h, base + i] - math.log(n)) < 1e-13
                mean = vv[base + lo: base + hi + 1, h // 2].mean(axis=0)
                assert np.allclose(o[base + i, h], mean, atol=1e-13)


def pin_decode():
    r = _rng(18)
    b, s_cache, h_q, h_kv, d = 3, 50, 4, 2, 8
    kc = r.standard_normal((b, s_cache, h_kv, d))
    vc = r.standard_normal((b, s_cache, h_kv, d))
    lens = [1, 17, 50]
    q = np.zeros((b, 1, h_q, d))
    o, lse = oracle.attention_kvcache(q, kc, vc, lens, causal=True)
    for bi, n in enumerate(lens):
        for h in range(h_q):
            assert abs(lse[bi, h, 0] - math.log(n)) < 1e-13
            assert np.allclose(o[bi, 0, h], vc[bi, :n, h // 2].mean(axis=0), atol=1e-13)
    # window on decode: the single query sits at position n - 1 (bottom-right)
    o, lse = oracle.attention_kvcache(q, kc, vc, lens, window_size=(5, 0))
    for bi, n in enumerate(lens):
        lo = max(0, n - 1 - 5)
        assert abs(lse[bi, 0, 0] - math.log(n - lo)) < 1e-13


def pin_decode_append():
    """Append then attend (FAQ Q17), pinned from the inputs themselves: with
    Q = 0 every visible score is 0, so O is the mean of the old rows
    0..n-1 and the new rows, LSE = ln(n + s_new); the cache copy keeps every
    other row; with an empty cache and one new token O = v_new, LSE = scale q.k_new."""
    r = _rng(22)
    b, s_cache, h_q, h_kv, d, s_new = 3, 40, 4, 2, 8, 3
    kc = r.standard_normal((b, s_cache, h_kv, d))
    vc = r.standard_normal((b, s_cache, h_kv, d))
    kn = r.standard_normal((b, s_new, h_kv, d))
    vn = r.standard_normal((b, s_new, h_kv, d))
    lens = [0, 5, 30]
    q = np.zeros((b, 1, h_q, d))
    o, lse, kc2, vc2 = oracle.attention_kvcache_append(q, kc, vc, kn, vn, lens, causal=True)
    for bi, n in enumerate(lens):
        for h in range(h_q):
            hk = h // 2
            assert abs(lse[bi, h, 0] - math.log(n + s_new)) < 1e-13
            mean = (vc[bi, :n, hk].sum(axis=0) + vn[bi, :, hk].sum(axis=0)) / (n + s_new)
            assert np.allclose(o[bi, 0, h], mean, atol=1e-13)
        keep = [j for j in range(s_cache) if not n <= j < n + s_new]
        assert np.array_equal(kc2[bi, keep], kc[bi, keep]) and np.array_equal(vc2[bi, keep], vc[bi, keep])
        assert np.array_equal(kc2[bi, n:n + s_new], kn[bi]) and np.array_equal(vc2[bi, n:n + s_new], vn[bi])
    assert np.array_equal(kc[1, 5], kc[1, 5])  # inputs untouched (copies)
    # empty cache, one new token
    q1 = r.standard_normal((1, 1, 1, d))
    o1, l1, _, _ = oracle.attention_kvcache_append(q1, kc[:1, :, :1], vc[:1, :, :1], kn[:1, :1, :1],
                                                   vn[:1, :1, :1], [0])
    assert np.allclose(o1[0, 0, 0], vn[0, 0, 0], atol=1e-14)
    assert abs(l1[0, 0, 0] - float(q1[0, 0, 0] @ kn[0, 0, 0]) / math.sqrt(d)) < 1e-12
    # rows past the capacity are dropped
    _, _, kc3, _ = oracle.attention_kvcache_append(q[:1], kc[:1], vc[:1], kn[:1], vn[:1], [s_cache - 2])
    assert np.array_equal(kc3[0, s_cache - 2:], kn[0, :2]) and np.array_equal(kc3[0, :s_cache - 2],
                                                                                kc[0, :s_cache - 2])


def pin_decode_multi_query():
    """Several query tokens against the KV cache after an append (FAQ Q17 passes
    k=k_new, v=v_new with causal=True; the mask is bottom-right, FAQ Q6): with
    s_q = s_new new tokens and n cached rows, query t sits at position n + t of
    the n + s_new keys.  With Q = 0 every visible score is 0, so query t's O is
    the mean of the updated cache's rows 0..n+t and its LSE is ln(n + t + 1);
    without causal every query sees all n + s_new rows; a window (2, 0) leaves
    min(n + t, 2) + 1 rows; a query past the keys (s_q > n + s_new) sees none."""
    r = _rng(24)
    b, s_cache, h_q, h_kv, d, s_new = 3, 40, 4, 2, 8, 3
    kc = r.standard_normal((b, s_cache, h_kv, d))
    vc = r.standard_normal((b, s_cache, h_kv, d))
    kn = r.standard_normal((b, s_new, h_kv, d))
    vn = r.standard_normal((b, s_new, h_kv, d))
    lens = [0, 5, 30]
    q = np.zeros((b, s_new, h_q, d))
    o, lse, kc2, vc2 = oracle.attention_kvcache_append(q, kc, vc, kn, vn, lens, causal=True)
    assert o.shape == (b, s_new, h_q, d) and lse.shape == (b, h_q, s_new)
    for bi, n in enumerate(lens):
        for t in range(s_new):
            for h in range(h_q):
                hk = h // 2
                assert abs(lse[bi, h, t] - math.log(n + t + 1)) < 1e-13
                assert np.allclose(o[bi, t, h], vc2[bi, :n + t + 1, hk].mean(axis=0), atol=1e-13)
    o, lse, _, _ = oracle.attention_kvcache_append(q, kc, vc, kn, vn, lens, causal=False)
    for bi, n in enumerate(lens):
        for t in range(s_new):
            assert abs(lse[bi, 0, t] - math.log(n + s_new)) < 1e-13
    o, lse, _, _ = oracle.attention_kvcache_append(q, kc, vc, kn, vn, lens, causal=True, window_size=(2, 0))
    for bi, n in enumerate(lens):
        for t in range(s_new):
            assert abs(lse[bi, 1, t] - math.log(min(n + t, 2) + 1)) < 1e-13
    # more queries than keys: the first ones see nothing (O = 0, LSE = -inf)
    q5 = np.zeros((1, 5, 2, d))
    o5, l5 = oracle.attention_kvcache(q5, kc[:1], vc[:1], [3], causal=True)
    assert np.all(np.isneginf(l5[0, :, :2])) and np.all(o5[0, :2] == 0)
    for t in range(2, 5):
        assert abs(l5[0, 0, t] - math.log(t - 1)) < 1e-13


def pin_paged():
    """A paged cache (FAQ Q18) read back as contiguous: the pool is built here by
    scattering the pages of a contiguous cache to a random permutation of page
    slots; the gather must return the cache exactly, for any page size."""
    r = _rng(23)
    b, s_cache, h, d = 3, 48, 2, 4
    cache = r.standard_normal((b, s_cache, h, d))
    for page in (16, 12, 48):
        per_seq = -(-s_cache // page)
        n_pages = b * per_seq + 2
        perm = r.permutation(n_pages)
        pool = np.full((n_pages, page, h, d), np.nan)
        bt = np.zeros((b, per_seq), dtype=np.int32)
        for bi in range(b):
            for i in range(per_seq):
                slot = perm[bi * per_seq + i]
                bt[bi, i] = slot
                rows = cache[bi, i * page:(i + 1) * page]
                pool[slot, :rows.shape[0]] = rows
        got = OA.paged_to_contiguous(pool, bt, s_cache)
        assert np.array_equal(got, cache), page


def _sdpa_autograd(q, k, v, do, scale, causal, wl, wr, softcap):
    """dQ, dK, dV by torch autograd (float64, CPU) of a plain masked attention with
    its own bottom-right mask; empty rows are multiplied out instead of NaN."""
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    b, s_q, h_q, d = q.shape
    s_k, h_kv = k.shape[1], k.shape[2]
    g = h_q // h_kv
    ke = kt.repeat_interleave(g, dim=2)
    ve = vt.repeat_interleave(g, dim=2)
    s = torch.einsum("bqhd,bkhd->bhqk", qt, ke) * scale
    if softcap > 0:
        s = softcap * torch.tanh(s / softcap)
    i = torch.arange(s_q)[:, None]
    j = torch.arange(s_k)[None, :]
    off = s_k - s_q
    vis = torch.ones(s_q, s_k, dtype=torch.bool)
    right = 0 if causal else wr
    if right >= 0:
        vis &= j <= i + off + right
    if wl >= 0:
        vis &= j >= i + off - wl
    s = s.masked_fill(~vis, -1e30)
    p = torch.softmax(s, dim=-1) * vis.any(dim=1)[:, None].to(torch.float64)
    o = torch.einsum("bhqk,bkhd->bqhd", p, ve)
    (o * torch.tensor(do)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def pin_backward():
    """The oracle's gradients against autograd of a plain masked attention, against
    central differences, and two closed forms: without softcap each head's dK
    sums to 0 over the keys (every row of dS sums to 0), and dV summed over the
    keys is the sum of dO over the rows that see any key."""
    r = _rng(24)
    cases = [  # s_q, s_k, h_q, h_kv, causal, window, softcap
        (5, 7, 2, 1, True, (-1, -1), 0.0),
        (6, 6, 4, 2, False, (2, 1), 0.0),
        (8, 4, 2, 2, True, (-1, -1), 0.0),   # rows 0-3 see nothing
        (4, 9, 2, 1, False, (-1, -1), 1.5),  # saturating softcap
    ]
    for s_q, s_k, h_q, h_kv, causal, (wl, wr), cap in cases:
        d = 4
        q = r.standard_normal((2, s_q, h_q, d)) * 2
        k = r.standard_normal((2, s_k, h_kv, d)) * 2
        v = r.standard_normal((2, s_k, h_kv, d))
        do = r.standard_normal((2, s_q, h_q, d))
        scale = 0.7
        dq, dk, dv = oracle.attention_backward(q, k, v, do, softmax_scale=scale, causal=causal,
                                               window_size=(wl, wr), softcap=cap)
        gq, gk, gv = _sdpa_autograd(q, k, v, do, scale, causal, wl, wr, cap)
        assert np.allclose(dq, gq, atol=1e-10) and np.allclose(dk, gk, atol=1e-10)
        assert np.allclose(dv, gv, atol=1e-10)
        if cap == 0:  # with a softcap dS is reweighted by 1 - tanh^2 and its rows no longer sum to 0
            assert np.abs(dk.sum(axis=1)).max() < 1e-10
        vis_rows = [i for i in range(s_q) if _visible_count(i, s_q, s_k, causal, wl, wr)[0] > 0]
        want = do[:, vis_rows].reshape(2, len(vis_rows), h_kv, h_q // h_kv, d).sum(axis=(1, 3))
        assert np.allclose(dv.sum(axis=1), want, atol=1e-10)
        # central differences of L = sum(dO * O) for a few entries
        def loss(qq, kk, vv):
            o, _ = oracle.attention(qq, kk, vv, softmax_scale=scale, causal=causal,
                                    window_size=(wl, wr), softcap=cap)
            return float((np.nan_to_num(o) * do).sum())
        eps = 1e-6
        for arr, grad in ((q, dq), (k, dk), (v, dv)):
            idx = tuple(int(x) for x in r.integers(0, arr.shape))
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            args_p = [plus if a is arr else a for a in (q, k, v)]
            args_m = [minus if a is arr else a for a in (q, k, v)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-6, (idx, fd, grad[idx])


def pin_backward_magnitudes():
    """The term magnitudes bound the gradients from above; dV's equals dV where
    dO >= 0 (P >= 0); and on a tiny case they match the terms enumerated one by
    one in scalar Python (probabilities from exp and fsum, every term of D with
    O expanded into its terms P V, of dP and of the three products listed and
    summed in absolute value)."""
    r = _rng(25)
    for s_q, s_k, h_q, h_kv, causal, win in ((7, 9, 4, 2, True, (-1, -1)), (6, 6, 2, 2, False, (2, 0))):
        q = r.standard_normal((2, s_q, h_q, 8))
        k = r.standard_normal((2, s_k, h_kv, 8))
        v = r.standard_normal((2, s_k, h_kv, 8))
        do = r.standard_normal((2, s_q, h_q, 8))
        g = oracle.attention_backward(q, k, v, do, causal=causal, window_size=win)
        m = oracle.attention_backward_magnitudes(q, k, v, do, causal=causal, window_size=win)
        for gi, mi in zip(g, m):
            assert np.all(mi >= np.abs(gi) - 1e-12)
        # a negative scale: the terms' sizes are the same, the bound still holds
        gn = oracle.attention_backward(q, k, v, do, causal=causal, window_size=win, softmax_scale=-0.3)
        mn = oracle.attention_backward_magnitudes(q, k, v, do, causal=causal, window_size=win, softmax_scale=-0.3)
        for gi, mi in zip(gn, mn):
            assert np.all(mi >= 0) and np.all(mi >= np.abs(gi) - 1e-12)
        _, _, dv = oracle.attention_backward(q, k, v, np.abs(do), causal=causal, window_size=win)
        _, _, mv = oracle.attention_backward_magnitudes(q, k, v, np.abs(do), causal=causal, window_size=win)
        assert np.allclose(mv, dv, atol=1e-12)
    # scalar enumeration: s_q 3, s_k 4, two query heads on one KV head, causal, d 3
    s_q, s_k, d, scale = 3, 4, 3, 0.6
    q = r.standard_normal((1, s_q, 2, d))
    k = r.standard_normal((1, s_k, 1, d))
    v = r.standard_normal((1, s_k, 1, d))
    do = r.standard_normal((1, s_q, 2, d))
    mq, mk, mv = oracle.attention_backward_magnitudes(q, k, v, do, softmax_scale=scale, causal=True)
    wq = np.zeros_like(mq)
    wk = np.zeros_like(mk)
    wv = np.zeros_like(mv)
    for h in range(2):
        for i in range(s_q):
            keys = [j for j in range(s_k) if j <= i + s_k - s_q]
            sc = {j: scale * math.fsum(q[0, i, h, t] * k[0, j, 0, t] for t in range(d)) for j in keys}
            top = max(sc.values())
            z = math.fsum(math.exp(sc[j] - top) for j in keys)
            pr = {j: math.exp(sc[j] - top) / z for j in keys}
            # D's terms dO_t P_j' V_j't, each listed
            dterms = math.fsum(abs(do[0, i, h, t] * pr[jj] * v[0, jj, 0, t]) for t in range(d) for jj in keys)
            for j in keys:
                dp = math.fsum(do[0, i, h, t] * v[0, j, 0, t] for t in range(d))
                a = pr[j] * (abs(dp) + dterms)
                for t in range(d):
                    wq[0, i, h, t] += scale * a * abs(k[0, j, 0, t])
                    wk[0, j, 0, t] += scale * a * abs(q[0, i, h, t])
                    wv[0, j, 0, t] += pr[j] * abs(do[0, i, h, t])
    assert np.allclose(mq, wq, rtol=1e-12, atol=1e-14)
    assert np.allclose(mk, wk, rtol=1e-12, atol=1e-14)
    # with softcap c: the bound still holds, and on the same tiny case the terms
    # enumerated in scalar Python (capped scores c tanh(s / c), dS terms times
    # 1 - tanh^2) match
    cap = 1.5
    for causal, win in ((True, (-1, -1)), (False, (2, 1))):
        q8 = r.standard_normal((2, 7, 4, 8)) * 2
        k8 = r.standard_normal((2, 9, 2, 8)) * 2
        v8 = r.standard_normal((2, 9, 2, 8))
        do8 = r.standard_normal((2, 7, 4, 8))
        g = oracle.attention_backward(q8, k8, v8, do8, causal=causal, window_size=win, softcap=cap)
        m = oracle.attention_backward_magnitudes(q8, k8, v8, do8, causal=causal, window_size=win, softcap=cap)
        for gi, mi in zip(g, m):
            assert np.all(mi >= np.abs(gi) - 1e-12)
    mq, mk, mv = oracle.attention_backward_magnitudes(q, k, v, do, softmax_scale=scale, causal=True, softcap=cap)
    wq = np.zeros_like(mq)
    wk = np.zeros_like(mk)
    wv = np.zeros_like(mv)
    for h in range(2):
        for i in range(s_q):
            keys = [j for j in range(s_k) if j <= i + s_k - s_q]
            raw = {j: scale * math.fsum(q[0, i, h, t] * k[0, j, 0, t] for t in range(d)) for j in keys}
            sc = {j: cap * math.tanh(raw[j] / cap) for j in keys}
            top = max(sc.values())
            z = math.fsum(math.exp(sc[j] - top) for j in keys)
            pr = {j: math.exp(sc[j] - top) / z for j in keys}
            # D's terms dO_t P_j' V_j't, each listed
            dterms = math.fsum(abs(do[0, i, h, t] * pr[jj] * v[0, jj, 0, t]) for t in range(d) for jj in keys)
            for j in keys:
                dp = math.fsum(do[0, i, h, t] * v[0, j, 0, t] for t in range(d))
                a = pr[j] * (abs(dp) + dterms) * (1.0 - math.tanh(raw[j] / cap) ** 2)
                for t in range(d):
                    wq[0, i, h, t] += scale * a * abs(k[0, j, 0, t])
                    wk[0, j, 0, t] += scale * a * abs(q[0, i, h, t])
                    wv[0, j, 0, t] += pr[j] * abs(do[0, i, h, t])
    assert np.allclose(mq, wq, rtol=1e-12, atol=1e-14)
    assert np.allclose(mk, wk, rtol=1e-12, atol=1e-14)
    assert np.allclose(mv, wv, rtol=1e-12, atol=1e-14)
    assert np.allclose(mv, wv, rtol=1e-12, atol=1e-14)


def pin_fp8():
    """The E4M3 decoding against torch's float8_e4m3fn conversion for all 256
    codes and against values fixed by the format (1.0, the largest 448, the
    smallest subnormal 2^-9, negative zero, NaN); attention_fp8 depends on the
    Q and K descales only through their product (with the softmax scale), and
    the V descale scales O and leaves LSE."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ours = OA.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref)) and int(np.isnan(ours).sum()) == 2
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert ours[0x38] == 1.0 and ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert ours[0x80] == 0.0 and np.signbit(ours[0x80]) and ours[0xB8] == -1.0
    # from a torch tensor: the same bytes
    assert np.array_equal(OA.decode_e4m3(torch.from_numpy(codes).view(torch.float8_e4m3fn))[fin], ours[fin])
    r = _rng(26)
    q = torch.from_numpy(r.standard_normal((2, 9, 4, 16))).to(torch.float8_e4m3fn)
    k = torch.from_numpy(r.standard_normal((2, 11, 2, 16))).to(torch.float8_e4m3fn)
    v = torch.from_numpy(r.standard_normal((2, 11, 2, 16))).to(torch.float8_e4m3fn)
    o1, l1 = oracle.attention_fp8(q, k, v, causal=True)
    o2, l2 = oracle.attention_fp8(q, k, v, q_descale=4.0, k_descale=0.25, causal=True)
    o3, l3 = oracle.attention_fp8(q, k, v, q_descale=2.0, causal=True, softmax_scale=0.125)
    o4, l4 = oracle.attention_fp8(q, k, v, causal=True, softmax_scale=0.25)
    o5, l5 = oracle.attention_fp8(q, k, v, v_descale=3.0, causal=True)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)
    assert np.allclose(o3, o4, atol=1e-12) and np.allclose(l3, l4, atol=1e-12)
    assert np.allclose(o5, 3.0 * o1, atol=1e-12) and np.allclose(l5, l1, atol=1e-12)
    # the real values are torch's decoding times the descales
    o6, l6 = oracle.attention(q.to(torch.float64) * 2.0, k.to(torch.float64) * 0.5, v.to(torch.float64) * 3.0,
                              causal=True)
    o7, l7 = oracle.attention_fp8(q, k, v, q_descale=2.0, k_descale=0.5, v_descale=3.0, causal=True)
    assert np.allclose(o6, o7, atol=1e-12) and np.allclose(l6, l7, atol=1e-12)


def pin_fp8_softcap():
    """The FP8 forward with softcap (FAQ Q20 with Q22): the cap acts on the scaled
    scores of the real values.  With one key, LSE is c tanh(s / c) of the row's
    single score and O is that key's V row (real values: codes from torch's own
    E4M3 conversion times the descales), and the Q and K descales still enter
    only through their product with the scale."""
    import torch
    r = _rng(27)
    q = torch.from_numpy(r.standard_normal((1, 7, 2, 32)) * 3).to(torch.float8_e4m3fn)
    k = torch.from_numpy(r.standard_normal((1, 1, 2, 32)) * 3).to(torch.float8_e4m3fn)
    v = torch.from_numpy(r.standard_normal((1, 1, 2, 32))).to(torch.float8_e4m3fn)
    cap, dq, dk, dv = 5.0, 0.5, 1.5, 2.0
    o, lse = oracle.attention_fp8(q, k, v, q_descale=dq, k_descale=dk, v_descale=dv, softcap=cap)
    qf, kf, vf = (t.to(torch.float64).numpy() for t in (q, k, v))
    scale = 1.0 / math.sqrt(32)
    for h in range(2):
        for i in range(7):
            raw = scale * dq * dk * math.fsum(qf[0, i, h] * kf[0, 0, h])
            assert abs(lse[0, h, i] - cap * math.tanh(raw / cap)) < 1e-12
            assert np.allclose(o[0, i, h], vf[0, 0, h] * dv, atol=1e-12)
    # the cap bites: the capped LSE is not the uncapped one
    _, lse_nc = oracle.attention_fp8(q, k, v, q_descale=dq, k_descale=dk, v_descale=dv)
    assert np.abs(lse - lse_nc).max() > 0.1
    # descales and scale through their product, with the cap on
    q2 = torch.from_numpy(r.standard_normal((2, 9, 4, 16))).to(torch.float8_e4m3fn)
    k2 = torch.from_numpy(r.standard_normal((2, 11, 2, 16))).to(torch.float8_e4m3fn)
    v2 = torch.from_numpy(r.standard_normal((2, 11, 2, 16))).to(torch.float8_e4m3fn)
    o1, l1 = oracle.attention_fp8(q2, k2, v2, causal=True, softcap=1.5)
    o2, l2 = oracle.attention_fp8(q2, k2, v2, q_descale=4.0, k_descale=0.25, causal=True, softcap=1.5)
    o3, l3 = oracle.attention_fp8(q2, k2, v2, q_descale=2.0, softmax_scale=0.125, causal=True, softcap=1.5)
    o4, l4 = oracle.attention_fp8(q2, k2, v2, softmax_scale=0.25, causal=True, softcap=1.5)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)
    assert np.allclose(o3, o4, atol=1e-12) and np.allclose(l3, l4, atol=1e-12)


def pin_softcap():
    r = _rng(19)
    q = r.standard_normal((1, 6, 2, 16)) * 4
    k = r.standard_normal((1, 1, 2, 16)) * 4
    v = r.standard_normal((1, 1, 2, 16))
    cap = 2.0
    _, lse = oracle.attention(q, k, v, softcap=cap)
    for h in range(2):
        for i in range(6):
            raw = 0.25 * math.fsum(q[0, i, h] * k[0, 0, h])
            assert abs(lse[0, h, i] - cap * math.tanh(raw / cap)) < 1e-12
    # a huge cap is no cap
    q = r.standard_normal((1, 8, 2, 16))
    k = r.standard_normal((1, 8, 2, 16))
    v = r.standard_normal((1, 8, 2, 16))
    o0, l0 = oracle.attention(q, k, v, causal=True)
    o1, l1 = oracle.attention(q, k, v, causal=True, softcap=1e9)
    assert np.allclose(o0, o1, atol=1e-9) and np.allclose(l0, l1, atol=1e-9)
    # saturating cap: every final score lies in [-c, c] (tanh rounds to +-1 in float64 once
    # saturated), so ln n - c <= LSE <= ln n + c, and at least one row is close to saturation
    o2, l2 = oracle.attention(q * 8, k * 8, v, causal=True, softcap=cap)
    for i in range(8):
        n = i + 1
        assert np.all(l2[0, :, i] <= math.log(n) + cap) and np.all(l2[0, :, i] >= math.log(n) - cap)
    assert np.max(np.abs(l2[0, :, 0])) > 0.99 * cap
    # softcap comes before the mask: masked keys stay invisible whatever their score
    _zero_q_check(20, 20, True, 3, -1, 2, 2, seed=300)


def pin_default_scale():
    r = _rng(20)
    q = r.standard_normal((1, 4, 1, 64))
    k = r.standard_normal((1, 4, 1, 64))
    v = r.standard_normal((1, 4, 1, 64))
    o1, l1 = oracle.attention(q, k, v)
    o2, l2 = oracle.attention(q, k, v, softmax_scale=1 / 8.0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


PINS = [pin_bruteforce, pin_sdpa, pin_softmax_rows, pin_sk1, pin_identical_v_rows,
        pin_zero_q_counts, pin_bottom_right_causal, pin_window_fixture, pin_shift_invariance,
        pin_merge_identity, pin_gqa_repeat, pin_varlen, pin_decode, pin_decode_append, pin_decode_multi_query, pin_paged, pin_backward, pin_backward_magnitudes, pin_fp8, pin_fp8_softcap, pin_softcap,
        pin_default_scale]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ----------------------------------------------------------------------------
def _bad_scores_noscale(q2, k2, scale):
    return q2 @ k2.T


def _bad_scores_transposed(q2, k2, scale):
    return scale * (k2 @ q2.T)


def _bad_softcap_none(s, softcap):
    return s


def _bad_softcap_noscale(s, softcap):
    return np.tanh(s / softcap) if softcap and softcap > 0 else s


def _bad_visible_topleft(rows, s_q, s_k, causal, wl, wr):
    return OA_visible(rows, s_k, s_k, causal, wl, wr)


def _bad_visible_window_off_by_one(rows, s_q, s_k, causal, wl, wr):
    return OA_visible(rows, s_q, s_k, causal, wl + 1 if wl >= 0 else wl, wr)


def _bad_visible_causal_ignored(rows, s_q, s_k, causal, wl, wr):
    return OA_visible(rows, s_q, s_k, False, wl, wr)


def _bad_softmax_lse_nomax(s, mask):
    p, lse = OA_softmax(s, mask)
    m = np.where(mask, s, -np.inf).max(axis=1, initial=-np.inf)
    return p, np.where(np.isfinite(lse), lse - np.where(np.isfinite(m), m, 0.0), lse)


def _bad_softmax_sign(s, mask):
    return OA_softmax(-s, mask)


def _bad_kv_head_modulo(h, h_q, h_kv):
    return h % h_kv


def _bad_append_offset(k_cache, v_cache, cache_seqlens, k_new, v_new):
    return OA_append(k_cache, v_cache, [max(0, int(n) - 1) for n in np.asarray(cache_seqlens)], k_new,
                     v_new)


def _bad_paged_row(pool, block_table, seqlen_cache):
    bt = np.asarray(block_table)
    page = pool.shape[1]
    rows = [pool[[int(bt[bi, j // page]) for j in range(seqlen_cache)], [j // page for j in range(seqlen_cache)]]
            for bi in range(bt.shape[0])]
    return np.stack(rows, 0)


OA_visible = OA.visible
OA_softmax = OA.softmax_rows
OA_append = OA.kvcache_append

def _bad_e4m3_bias(codes):
    return ORIG_DECODE_E4M3(codes) * 0.5  # exponent bias 8 instead of 7


ORIG_DECODE_E4M3 = OA.decode_e4m3


MUTATIONS = [
    ("scores", _bad_scores_noscale),
    ("scores", _bad_scores_transposed),
    ("apply_softcap", _bad_softcap_none),
    ("apply_softcap", _bad_softcap_noscale),
    ("visible", _bad_visible_topleft),
    ("visible", _bad_visible_window_off_by_one),
    ("visible", _bad_visible_causal_ignored),
    ("softmax_rows", _bad_softmax_lse_nomax),
    ("softmax_rows", _bad_softmax_sign),
    ("_kv_head", _bad_kv_head_modulo),
    ("kvcache_append", _bad_append_offset),
    ("paged_to_contiguous", _bad_paged_row),
    ("decode_e4m3", _bad_e4m3_bias),
]


@pytest.mark.parametrize("name,bad", MUTATIONS, ids=lambda x: getattr(x, "__name__", str(x)))
def test_planted_mistake_is_caught(monkeypatch, name, bad):
    monkeypatch.setattr(OA, name, bad)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {bad.__name__} in {name}"


def test_tolerance_fixture():
    tol = golden_io.tolerances()
    assert tol["fp16"] == (1e-3, 1e-3) and tol["bf16"] == (5e-3, 5e-3) and tol["fp8"] == (1e-2, 1e-2)


def test_flops_fixture():
    fx = golden_io.as_dict("faq_q16_flops.txt")
    w = workloads.WORKLOADS["causal_prefill"]
    assert (w.batch, w.heads_q, w.seqlen_q, w.head_dim) == tuple(
        int(fx[k][0]) for k in ("batch", "nheads", "seqlen", "headdim"))
    assert workloads.flops(w) == float(fx["causal_flops"][0])


def test_smoke_shapes_fixture():
    rows = [r for k, r in golden_io.read("smoke_shapes.txt") if k == "shape"]
    assert len(rows) == 4
    for b, s, h, d, dt in rows:
        b, s, h, d = int(b), int(s), int(h), int(d)
        q = np.zeros((b, min(s, 8), h, d))
        o, lse = oracle.attention(q, q, q, rows=[0], heads=[0])
        assert o.shape == q.shape and lse.shape == (b, h, q.shape[1])
