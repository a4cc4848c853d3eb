"""GPU parity: the HIP kernels through the C ABI against the CPU fp64 oracle.

Inputs are seeded N(0,1) draws (exact_attention_43_amd.workloads) rounded to
fp16/bf16; the oracle sees exactly the rounded values.  Every configuration the
benchmark names is covered, at full size where the oracle finishes in seconds
and on sampled rows plus size-independent properties otherwise, together with
the extra shapes that make each mask rule bite, ragged tails, empty rows and
sequences, split counts, packed layouts and determinism.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_43_amd as ex
import oracle
from exact_attention_43_amd import workloads as W
from parity import assert_lse_close, assert_o_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    ex.lib()  # the HIP library must load on a GPU machine: no fallback


def _dev(*ts):
    return [t.to(DEV) for t in ts]


def _poison_out(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def _poison_lse(shape):
    return torch.full(shape, 123.0, dtype=torch.float32, device=DEV)


def run_dense(q, k, v, where, **kw):
    """Run attn_func on poisoned outputs and compare everything with the oracle."""
    dq, dk, dv = _dev(q, k, v)
    b, s_q, h_q, d = q.shape
    out = _poison_out(q.shape, q.dtype)
    lse = _poison_lse((b, h_q, s_q))
    ex.attn_func(dq, dk, dv, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, **kw)
    assert_o_close(out, o_ref, q.dtype, where)
    assert_lse_close(lse, l_ref, where)
    return out, lse


# --------------------------------------------------------------------------
# the named workloads
# --------------------------------------------------------------------------
def test_tiny_fp16():
    w = W.WORKLOADS["tiny"]
    q, k, v = W.qkv(1, 64, 64, 4, 4, 64, seed=w.seed, dtype=torch.float16)
    run_dense(q, k, v, "tiny")


def test_causal_prefill_qkvpacked():
    w = W.WORKLOADS["causal_prefill"]
    qkv = W.packed_qkv(w.batch, w.seqlen_q, w.heads_q, w.head_dim, seed=w.seed)
    out, lse = ex.attn_qkvpacked_func(qkv.to(DEV), causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], causal=True)
    assert_o_close(out, o_ref, torch.bfloat16, "causal_prefill")
    assert_lse_close(lse, l_ref, "causal_prefill")


# Paired launches (a light and a heavy 64-row tile per work group, one work
# group per CU) under windows: the tiles' key ranges start above key 0, one
# tile's waves idle while the other's compute, and the idle wave of a group
# pair issues the next block's DMA for both.
@pytest.mark.parametrize("causal,window,dtype", [
    (False, (256, 0), torch.bfloat16),
    (True, (100, -1), torch.float16),
    (False, (128, 64), torch.bfloat16),
    (True, (-1, -1), torch.float16),
], ids=["w256_0", "causal_w100", "w128_64", "causal_f16"])
def test_paired_launch_windows(causal, window, dtype):
    q, k, v = W.qkv(2, 1024, 1024, 16, 16, 128, seed=107, dtype=dtype)
    run_dense(q, k, v, f"paired causal={causal} window={window}", causal=causal, window_size=window)


@pytest.mark.parametrize("name", ["hdim64", "hdim128", "hdim256"])
def test_head_dim_sweep(name):
    w = W.WORKLOADS[name]
    q, k, v = W.qkv(w.batch, w.seqlen_q, w.seqlen_k, w.heads_q, w.heads_kv, w.head_dim, seed=w.seed,
                    dtype=torch.float16)
    out, _ = run_dense(q, k, v, name)
    assert out.shape == q.shape


def test_varlen_gqa_window_softcap():
    w = W.WORKLOADS["varlen_gqa"]
    q, k, v, cu_q, cu_k = W.varlen_qkv(w.seqlens, w.seqlens, w.heads_q, w.heads_kv, w.head_dim,
                                       seed=w.seed)
    dq, dk, dv, dcq, dck = _dev(q, k, v, cu_q, cu_k)
    out = _poison_out(q.shape, q.dtype)
    lse = _poison_lse((w.heads_q, q.shape[0]))
    ex.attn_varlen_func(dq, dk, dv, dcq, dck, max(w.seqlens), max(w.seqlens), causal=True,
                        window_size=w.window, softcap=w.softcap, out=out, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen(q, k, v, cu_q, cu_k, causal=True, window_size=w.window,
                                           softcap=w.softcap)
    assert_o_close(out, o_ref, q.dtype, "varlen")
    assert_lse_close(lse, l_ref, "varlen")


def _dense_grid(b, s_q, h_q):
    """Work groups of a dense prefill launch: one per 128 query rows of a head."""
    return b * h_q * math.ceil(s_q / 128)


def _launch(b, s_q, h_q, h_kv, d, masked, pack=False):
    """The prefill launch the library picks (exattn_api.cpp) for fixed lengths:
    (groups, paired, key-split, head-dim split).  The key-split kernel replaces the
    paired launch at d = 128 without packing when that launch fills at most half of
    the CUs and the schedule fits (at most one unit per CU and 4 slots per work
    group).  At d = 256 without packing the head-dim-split kernel runs, with two key
    groups (64-row tiles) when there are fewer 128-row tiles than CUs."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = b * h_kv * math.ceil(s_q * (h_q // h_kv) / 128) if pack else _dense_grid(b, s_q, h_q)
    if d == 256 and not pack:
        return 0, False, False, 2 if grid < cus else 1
    groups = 1 if d == 256 or grid >= 2 * cus else 2
    paired = groups == 2 and masked and grid <= cus
    units = b * h_q
    slots = (paired and 2 * grid <= cus and d == 128 and not pack and units <= cus and b <= 65535
             and math.ceil(s_q / 64) <= 4 * min(cus // units, 64))
    return groups, paired and not slots, slots, 0


# Every instance of the prefill kernel template, each at a shape that makes the
# library pick it: (dtype, head_dim, softcap on/off, one group / two groups /
# two groups pairing a light and a heavy tile).  Masks, GQA and the sign of the
# scale vary along the way (a negative scale negates Q inside the kernel).
INSTANCE_CASES = []
for _dt in (torch.float16, torch.bfloat16):
    for _d in (64, 128, 256):
        for _cap in (0.0, 30.0):
            for _kind in (("one", "dsplit1", "dsplit2") if _d == 256 else
                          ("one", "two", "paired") + (("slots",) if _d == 128 else ())):
                INSTANCE_CASES.append((_dt, _d, _cap, _kind))


def _instance_shape(d, kind):
    # (b, s_q, s_k, h_q, h_kv, causal, window)
    if kind == "one":
        return (2, 2100, 2100, 16, 4, True, (-1, -1)) if d < 256 else (2, 1100, 1100, 8, 4, True, (-1, -1))
    if kind == "dsplit1":
        return (2, 1100, 1300, 16, 4, True, (-1, -1))
    if kind == "dsplit2":
        return (1, 1000, 1100, 4, 2, False, (-1, -1))
    if kind == "two":
        return (1, 700, 900, 8, 2, False, (-1, -1))
    return (1, 1024, 1024, 4, 2, True, (-1, -1))


@pytest.mark.parametrize("case", INSTANCE_CASES,
                         ids=[f"{'f16' if c[0] == torch.float16 else 'bf16'}-d{c[1]}-cap{int(c[2])}-{c[3]}"
                              for c in INSTANCE_CASES])
def test_prefill_instances(case):
    dt, d, cap, kind = case
    b, sq, sk, hq, hkv, causal, window = _instance_shape(d, kind)
    idx = INSTANCE_CASES.index(case)
    # a negative scale: causal one-group and paired launches at d = 128, and the
    # two-group launches with softcap
    neg = (d == 128 and kind in ("one", "paired", "slots")) or (kind == "two" and cap > 0) or \
        (kind == "dsplit2" and cap > 0)
    scale = -0.7 / math.sqrt(d) if neg else None
    # at d = 128 the paired kernel is reached through packed GQA (dense
    # shapes take the key-split kernel there), and so is the general kernel at
    # d = 256 (dense shapes take the head-dim-split kernel)
    pack = (kind == "paired" and d == 128) or (kind == "one" and d == 256)
    got = _launch(b, sq, hq, hkv, d, causal or window != (-1, -1), pack)
    want = {"one": (1, False, False, 0), "two": (2, False, False, 0), "paired": (2, True, False, 0),
            "slots": (2, False, True, 0), "dsplit1": (0, False, False, 1),
            "dsplit2": (0, False, False, 2)}[kind]
    if kind == "one" and d != 256:
        assert _dense_grid(b, sq, hq) >= 2 * torch.cuda.get_device_properties(0).multi_processor_count
    assert got == want, f"shape picks {got}, not {kind}"
    q, k, v = W.qkv(b, sq, sk, hq, hkv, d, seed=300 + idx, dtype=dt)
    dq, dk, dv = _dev(q, k, v)
    out = _poison_out(q.shape, dt)
    lse = _poison_lse((b, hq, sq))
    ex.attn_func(dq, dk, dv, causal=causal, window_size=window, softcap=cap, softmax_scale=scale,
                 pack_gqa=1 if pack else 0, out=out, lse=lse)
    torch.cuda.synchronize()
    heads = sorted({0, hq // 2 + 1, hq - 1})
    o_ref, l_ref = oracle.attention(q, k, v, causal=causal, window_size=window, softcap=cap,
                                    softmax_scale=scale, heads=heads)
    o_cpu, l_cpu = out.cpu(), lse.cpu()
    assert not torch.isnan(o_cpu).any()
    for h in heads:
        assert_o_close(o_cpu[:, :, h], o_ref[:, :, h], dt, f"{kind} d{d} cap{cap} h{h}")
        assert_lse_close(l_cpu[:, h], l_ref[:, h], f"{kind} d{d} cap{cap} h{h}")


# Key-split launches (fwd_prefill_slots.hip): heavy query tiles are cut into up
# to 4 slots of one work group that take every kgn-th 32-key block and merge at
# the end.  The shapes vary the slot counts (few units: 4 slots per heavy tile;
# many units: few slots per tile), the key ranges (ragged tails, s_q above and
# below s_k, tiles that see no key, windows on either side, no keys at all) and
# the arithmetic (fp16 / bf16, softcap, a negative scale, GQA).
SLOT_CASES = [
    # b, s_q, s_k, h_q, h_kv, dtype, causal, window, softcap, negative scale, seed
    (1, 1000, 1000, 8, 8, torch.bfloat16, True, (-1, -1), 0.0, False, 600),    # ragged last tile
    (2, 700, 300, 4, 2, torch.float16, True, (-1, -1), 0.0, False, 601),       # 400 rows see no key
    (1, 300, 1000, 8, 4, torch.bfloat16, True, (-1, -1), 0.0, True, 602),      # s_q < s_k
    (1, 1024, 1024, 8, 8, torch.float16, False, (100, 50), 0.0, False, 603),   # two-sided window
    (2, 2048, 2048, 4, 4, torch.bfloat16, True, (300, -1), 0.0, False, 604),   # causal + left window
    (1, 4096, 4096, 2, 1, torch.bfloat16, True, (-1, -1), 0.0, False, 605),    # 4 slots on heavy tiles
    (8, 128, 128, 16, 4, torch.float16, True, (-1, -1), 0.0, False, 606),      # two work groups per unit
    (4, 256, 256, 16, 4, torch.bfloat16, True, (20, -1), 0.0, False, 610),     # four per unit, window
    (1, 1536, 1536, 4, 1, torch.bfloat16, True, (-1, -1), 20.0, True, 607),    # softcap, MQA
    (3, 5, 5, 2, 2, torch.float16, True, (-1, -1), 0.0, False, 608),           # one tile, one block
    (1, 100, 0, 2, 2, torch.bfloat16, True, (-1, -1), 0.0, False, 609),        # no keys
]


@pytest.mark.parametrize("case", SLOT_CASES, ids=[f"s{c[-1]}" for c in SLOT_CASES])
def test_prefill_key_split(case):
    """The key-split kernel against the oracle (every row of sampled heads), with
    LSE and without, and bitwise equal over two runs (no atomics)."""
    b, sq, sk, hq, hkv, dt, causal, window, cap, neg, seed = case
    assert _launch(b, sq, hq, hkv, 128, True)[2], "shape does not take the key-split kernel"
    scale = -0.9 / math.sqrt(128) if neg else None
    q, k, v = W.qkv(b, sq, sk, hq, hkv, 128, seed=seed, dtype=dt)
    dq, dk, dv = _dev(q, k, v)
    kw = dict(causal=causal, window_size=window, softcap=cap, softmax_scale=scale, pack_gqa=0)
    out = _poison_out(q.shape, dt)
    lse = _poison_lse((b, hq, sq))
    ex.attn_func(dq, dk, dv, out=out, lse=lse, **kw)
    out2 = _poison_out(q.shape, dt)
    ex.attn_func(dq, dk, dv, out=out2, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    heads = None if b * hq <= 16 else sorted({0, hq // 2 + 1, hq - 1})
    kw.pop("pack_gqa")
    o_ref, l_ref = oracle.attention(q, k, v, heads=heads, **kw)
    o_cpu, l_cpu = out.cpu(), lse.cpu()
    assert not torch.isnan(o_cpu).any()
    for h in (range(hq) if heads is None else heads):
        assert_o_close(o_cpu[:, :, h], o_ref[:, :, h], dt, f"key-split s{seed} h{h}")
        assert_lse_close(l_cpu[:, h], l_ref[:, h], f"key-split s{seed} h{h}")


def test_prefill_key_split_full_table():
    """The key-split schedule at its largest (256 tiles of 64 rows, one per slot of 64
    work groups): b1 s16384 h1 causal, sampled rows at tile and work-group boundaries
    against the oracle."""
    b, sq, hq = 1, 16384, 1
    assert _launch(b, sq, hq, hq, 128, True)[2], "shape does not take the key-split kernel"
    q, k, v = W.qkv(b, sq, sq, hq, hq, 128, seed=611, dtype=torch.bfloat16)
    out, lse = ex.attn_func(*_dev(q, k, v), causal=True)
    torch.cuda.synchronize()
    rows = sorted({0, 1, 63, 64, 255, 256, 4095, 4096, 8191, 8192, 12287, 16320, 16383}
                  | set(np.random.default_rng(611).integers(0, sq, 24).tolist()))
    o_ref, l_ref = oracle.attention(q, k, v, causal=True, rows=rows)
    assert_o_close(out[:, rows].cpu(), o_ref[:, rows], torch.bfloat16, "key-split full table")
    assert_lse_close(lse[:, :, rows].cpu(), l_ref[:, :, rows], "key-split full table")


# Head-dim-split launches at d = 256 (fwd_prefill_dsplit.hip): two waves share 32
# rows, one per half of the head dims, and add their half scores through LDS.  One
# key group (128-row tiles) where there are at least as many tiles as CUs, else two
# (64-row tiles whose key blocks alternate between the groups, merged at the end).
# The shapes vary the launch, masks, GQA, softcap, the sign of the scale, empty
# rows, odd and even block counts per group and ragged tails.
DSPLIT_CASES = [
    # b, s_q, s_k, h_q, h_kv, dtype, causal, window, softcap, scale, seed
    (2, 2048, 2048, 8, 8, torch.bfloat16, False, (-1, -1), 0.0, None, 620),    # one group, plain
    (4, 1024, 1024, 16, 4, torch.bfloat16, True, (200, 0), 0.0, None, 621),    # one group, window, GQA
    (2, 1100, 1300, 16, 16, torch.float16, True, (-1, -1), 30.0, -0.05, 622),  # one group, cap, scale < 0
    (2, 700, 700, 4, 4, torch.float16, False, (64, 64), 0.0, None, 623),       # two groups, two-sided
    (1, 300, 100, 2, 1, torch.bfloat16, True, (-1, -1), 0.0, None, 624),       # rows without keys
    (2, 33, 33, 3, 3, torch.float16, True, (-1, -1), 30.0, None, 625),         # one partial tile
    (1, 64, 5000, 2, 2, torch.bfloat16, False, (-1, -1), 0.0, None, 626),      # 157 blocks: odd split
    (1, 129, 129, 2, 1, torch.bfloat16, False, (0, 0), 0.0, None, 627),        # window of one key
    (1, 500, 2000, 4, 2, torch.bfloat16, False, (-1, 100), 2.0, None, 628),    # right edge, saturating cap
]


@pytest.mark.parametrize("case", DSPLIT_CASES, ids=[f"s{c[-1]}" for c in DSPLIT_CASES])
def test_prefill_dsplit(case):
    b, sq, sk, hq, hkv, dt, causal, window, cap, scale, seed = case
    masked = causal or window != (-1, -1)
    assert _launch(b, sq, hq, hkv, 256, masked)[3], "shape does not take the head-dim-split kernel"
    q, k, v = W.qkv(b, sq, sk, hq, hkv, 256, seed=seed, dtype=dt)
    if cap == 2.0:
        q, k = (q.float() * 4).to(dt), (k.float() * 4).to(dt)
    dq, dk, dv = _dev(q, k, v)
    out = _poison_out(q.shape, dt)
    lse = _poison_lse((b, hq, sq))
    kw = dict(causal=causal, window_size=window, softcap=cap, softmax_scale=scale)
    ex.attn_func(dq, dk, dv, out=out, lse=lse, pack_gqa=0, **kw)
    torch.cuda.synchronize()
    heads = None if b * hq * sq * sk <= (1 << 24) else sorted({0, hq // 2 + 1, hq - 1})
    o_ref, l_ref = oracle.attention(q, k, v, heads=heads, **kw)
    o_cpu, l_cpu = out.cpu(), lse.cpu()
    for h in (range(hq) if heads is None else heads):
        assert_o_close(o_cpu[:, :, h], o_ref[:, :, h], dt, f"dsplit {seed} h{h}")
        assert_lse_close(l_cpu[:, h], l_ref[:, h], f"dsplit {seed} h{h}")


def test_prefill_dsplit_varlen():
    """Varlen at d = 256 through the head-dim-split kernel (unpacked GQA 8 / 2,
    causal): an empty sequence, one of a single row, tails at every tile size."""
    lens_q = [1, 130, 0, 64, 300]
    lens_k = [5, 130, 9, 700, 200]
    q, k, v, cu_q, cu_k = W.varlen_qkv(lens_q, lens_k, 8, 2, 256, seed=629)
    dq, dk, dv, dcq, dck = _dev(q, k, v, cu_q, cu_k)
    out = _poison_out(q.shape, q.dtype)
    lse = _poison_lse((8, q.shape[0]))
    ex.attn_varlen_func(dq, dk, dv, dcq, dck, max(lens_q), max(lens_k), causal=True, pack_gqa=0, out=out,
                        lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen(q, k, v, cu_q, cu_k, causal=True)
    assert_o_close(out, o_ref, q.dtype, "dsplit varlen")
    assert_lse_close(lse, l_ref, "dsplit varlen")


# Packed GQA (FAQ Q15): the rows of all query heads of a KV head share the tiles.
PACK_CASES = [
    # b, s_q, s_k, h_q, h_kv, d, dtype, causal, window, softcap, seed
    (2, 16, 500, 32, 4, 128, torch.bfloat16, True, (-1, -1), 0.0, 400),     # short queries, causal
    (3, 7, 7, 16, 2, 64, torch.float16, True, (-1, -1), 0.0, 401),          # s_q = s_k, tiny
    (1, 100, 1000, 8, 1, 128, torch.bfloat16, False, (300, 20), 20.0, 402),  # window, softcap, MQA
    (2, 33, 33, 12, 3, 256, torch.float16, True, (-1, -1), 0.0, 403),
    (1, 300, 300, 8, 2, 128, torch.float16, True, (64, 0), 0.0, 404),        # tiles of several positions
    (64, 16, 200, 64, 8, 128, torch.bfloat16, True, (-1, -1), 0.0, 405),     # one-group launches both ways
]


@pytest.mark.parametrize("case", PACK_CASES, ids=[f"k{c[-1]}" for c in PACK_CASES])
def test_pack_gqa(case):
    """pack_gqa on against the oracle; off and on bitwise equal when both launches pick the
    same number of wave groups (then every row sums the same key blocks in the same order)."""
    b, sq, sk, hq, hkv, d, dt, causal, window, cap, seed = case
    q, k, v = W.qkv(b, sq, sk, hq, hkv, d, seed=seed, dtype=dt)
    dq, dk, dv = _dev(q, k, v)
    res = {}
    for pack in (True, False):
        out = _poison_out(q.shape, dt)
        lse = _poison_lse((b, hq, sq))
        ex.attn_func(dq, dk, dv, causal=causal, window_size=window, softcap=cap, pack_gqa=pack, out=out,
                     lse=lse)
        res[pack] = (out, lse)
    torch.cuda.synchronize()
    heads = None if b * hq <= 64 else [0, 9, hq - 1]
    o_ref, l_ref = oracle.attention(q, k, v, causal=causal, window_size=window, softcap=cap, heads=heads)
    for pack in (True, False):
        o, l = res[pack][0].cpu(), res[pack][1].cpu()
        if heads is None:
            assert_o_close(o, o_ref, dt, f"pack={pack}")
            assert_lse_close(l, l_ref, f"pack={pack}")
        else:
            for h in heads:
                assert_o_close(o[:, :, h], o_ref[:, :, h], dt, f"pack={pack} h{h}")
                assert_lse_close(l[:, h], l_ref[:, h], f"pack={pack} h{h}")
    masked = causal or window != (-1, -1)
    on, off = _launch(b, sq, hq, hkv, d, masked, True), _launch(b, sq, hq, hkv, d, masked, False)
    if on[0] == off[0] and not on[2] and not off[2] and not on[3] and not off[3]:
        assert torch.equal(res[True][0], res[False][0]) and torch.equal(res[True][1], res[False][1])


@pytest.mark.parametrize("hq,hkv,causal", [(2, 2, False), (4, 1, True)])
def test_prefill_batch_past_grid_y_limit(hq, hkv, causal):
    """More batch entries than a grid's y dimension holds (65535): the prefill indexes a
    linear grid and decodes (batch, head) from the work-group id, plain or with packed GQA
    (4 query heads of one KV head in one tile).  Sampled entries against the oracle."""
    b, sq, sk, d = 65541, 3, 5, 64
    q, k, v = W.qkv(b, sq, sk, hq, hkv, d, seed=215, dtype=torch.float16)
    gq, gk, gv = _dev(q, k, v)
    out = torch.full((b, sq, hq, d), float("nan"), dtype=torch.float16, device="cuda")
    lse = torch.full((b, hq, sq), float("nan"), dtype=torch.float32, device="cuda")
    ex.attn_func(gq, gk, gv, causal=causal, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()
    idx = sorted({0, 1, 2, 65534, 65535, 65536, b - 1} | set(range(40000, 40040)))
    ro, rl = oracle.attention(q[idx], k[idx], v[idx], causal=causal)
    assert_o_close(out[idx].float().cpu(), ro, "fp16", "O")
    assert_lse_close(lse[idx].cpu(), rl, "LSE")



def test_pack_gqa_varlen():
    lens_q = [5, 0, 17, 64, 1]
    lens_k = [40, 3, 17, 300, 1]
    hq, hkv = 16, 4
    q, k, v, cu_q, cu_k = W.varlen_qkv(lens_q, lens_k, hq, hkv, 128, seed=406)
    dq, dk, dv, dcq, dck = _dev(q, k, v, cu_q, cu_k)
    out = _poison_out(q.shape, q.dtype)
    lse = _poison_lse((hq, q.shape[0]))
    ex.attn_varlen_func(dq, dk, dv, dcq, dck, max(lens_q), max(lens_k), causal=True, pack_gqa=True,
                        out=out, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_varlen(q, k, v, cu_q, cu_k, causal=True)
    assert_o_close(out, o_ref, q.dtype, "pack varlen")
    assert_lse_close(lse, l_ref, "pack varlen")


def test_window_edges_past_int32():
    """Window edges that reach past every key (up to 2^31 - 1) bound nothing: every
    entry point gives bitwise what the unbounded window gives (the kernels add
    the edges to positions in 32 bits, so the planner takes such edges as
    unbounded)."""
    big = 2 ** 31 - 1
    q, k, v = W.qkv(1, 300, 200, 4, 2, 128, seed=620, dtype=torch.bfloat16)
    dq, dk, dv = _dev(q, k, v)
    for win, ref in (((big, big), (-1, -1)), ((5, big), (5, -1)), ((big, 7), (-1, 7))):
        o1, l1 = ex.attn_func(dq, dk, dv, window_size=win)
        o2, l2 = ex.attn_func(dq, dk, dv, window_size=ref)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"fwd {win}"
        do = torch.randn_like(o1)
        g1 = ex.attn_backward(do, dq, dk, dv, o1, l1, window_size=win)
        g2 = ex.attn_backward(do, dq, dk, dv, o2, l2, window_size=ref)
        assert all(torch.equal(a, b) for a, b in zip(g1, g2)), f"bwd {win}"
    f8 = [t.to(torch.float8_e4m3fn) for t in (dq, dk, dv)]
    o1, l1 = ex.attn_func_fp8(*f8, window_size=(big, big))
    o2, l2 = ex.attn_func_fp8(*f8, window_size=(-1, -1))
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "fp8"
    kc, vc = _dev(*W.qkv(2, 300, 300, 2, 2, 128, seed=621, dtype=torch.bfloat16)[1:])
    qd = dq[:, :2].expand(2, 2, 4, 128).contiguous()
    kc, vc = kc[:, :, :2].contiguous(), vc[:, :, :2].contiguous()
    o1, l1 = ex.attn_with_kvcache(qd, kc, vc, window_size=(big, big))
    o2, l2 = ex.attn_with_kvcache(qd, kc, vc, window_size=(-1, -1))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "decode"


def test_zero_scale_is_uniform():
    """softmax_scale = 0 is a scale like any other (not the default): every visible key gets
    the same weight, so O is the mean of the visible V rows and LSE = ln(count)."""
    q, k, v = W.qkv(2, 100, 150, 4, 2, 128, seed=407)
    run_dense(q, k, v, "scale 0", causal=True, softmax_scale=0.0)
    qd, kc, vc = W.kvcache(2, 300, 8, 2, 128, seed=408)
    lens = torch.tensor([300, 77], dtype=torch.int32)
    dq, dkc, dvc, dl = _dev(qd, kc, vc, lens)
    out, lse = ex.attn_with_kvcache(dq, dkc, dvc, cache_seqlens=dl, softmax_scale=0.0, num_splits=3)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_kvcache(qd, kc, vc, lens, softmax_scale=0.0)
    assert_o_close(out, o_ref, qd.dtype, "decode scale 0")
    assert_lse_close(lse, l_ref, "decode scale 0")
    np.testing.assert_allclose(lse.cpu().numpy()[:, 0, 0], np.log([300.0, 77.0]), atol=1e-4)


ONE_GROUP_CASES = [
    # dtype, b, s_q, s_k, h_q, h_kv, d, causal, window, softcap
    (torch.bfloat16, 4, 1061, 1061, 16, 4, 128, True, (-1, -1), 0.0),
    (torch.float16, 4, 1061, 1300, 16, 16, 128, False, (100, 20), 0.0),
    (torch.bfloat16, 4, 1061, 1061, 16, 8, 128, False, (-1, -1), 0.0),
    (torch.float16, 4, 1061, 1061, 16, 2, 128, True, (-1, -1), 30.0),
    (torch.bfloat16, 4, 1061, 900, 16, 8, 64, True, (-1, -1), 0.0),
]


@pytest.mark.parametrize("case", ONE_GROUP_CASES, ids=[f"o{i}" for i in range(len(ONE_GROUP_CASES))])
def test_one_group_launches(case):
    """Grids of at least two work groups per CU take 4-wave work groups, and for
    d = 128 without softcap the software-pipelined loop: every mask rule, GQA and
    a ragged tail there, three heads in full against the oracle."""
    dt, b, sq, sk, hq, hkv, d, causal, window, cap = case
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert _dense_grid(b, sq, hq) >= 2 * cus, "shape too small for one-group work groups"
    q, k, v = W.qkv(b, sq, sk, hq, hkv, d, seed=140 + ONE_GROUP_CASES.index(case), dtype=dt)
    dq, dk, dv = _dev(q, k, v)
    out = _poison_out(q.shape, q.dtype)
    lse = _poison_lse((b, hq, sq))
    ex.attn_func(dq, dk, dv, causal=causal, window_size=window, softcap=cap, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    heads = [0, hq // 2 + 1, hq - 1]
    o_ref, l_ref = oracle.attention(q, k, v, causal=causal, window_size=window, softcap=cap,
                                    heads=heads)
    o_cpu, l_cpu = out.cpu(), lse.cpu()
    for h in heads:
        assert_o_close(o_cpu[:, :, h], o_ref[:, :, h], dt, f"one-group h{h}")
        assert_lse_close(l_cpu[:, h], l_ref[:, h], f"one-group h{h}")


def test_one_group_varlen():
    """Varlen with enough sequences for one-group work groups (d = 128, pipelined
    loop), ragged and empty sequences, causal then a window."""
    lens_q = [1100, 37, 640, 1025, 300, 0, 777, 129]
    lens_k = [1100, 50, 640, 1000, 301, 9, 777, 129]
    hq, hkv = 8, 2
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert len(lens_q) * hq * math.ceil(max(lens_q) / 128) >= 2 * cus
    q, k, v, cu_q, cu_k = W.varlen_qkv(lens_q, lens_k, hq, hkv, 128, seed=150)
    dq, dk, dv, dcq, dck = _dev(q, k, v, cu_q, cu_k)
    for causal, window in [(True, (-1, -1)), (False, (70, 5))]:
        out = _poison_out(q.shape, q.dtype)
        lse = _poison_lse((hq, q.shape[0]))
        ex.attn_varlen_func(dq, dk, dv, dcq, dck, max(lens_q), max(lens_k), causal=causal,
                            window_size=window, out=out, lse=lse)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention_varlen(q, k, v, cu_q, cu_k, causal=causal, window_size=window)
        assert_o_close(out, o_ref, q.dtype, f"one-group varlen {causal} {window}")
        assert_lse_close(lse, l_ref, f"one-group varlen {causal} {window}")


def test_cross_attention():
    w = W.WORKLOADS["cross"]
    q, k, v = W.qkv(w.batch, w.seqlen_q, w.seqlen_k, w.heads_q, w.heads_kv, w.head_dim, seed=w.seed)
    run_dense(q, k, v, "cross", causal=False)


def test_long_prefill_sampled():
    """16384-token causal prefill: sampled rows against the oracle, properties everywhere."""
    w = W.WORKLOADS["long_prefill"]
    q, k, v = W.qkv(w.batch, w.seqlen_q, w.seqlen_k, w.heads_q, w.heads_kv, w.head_dim, seed=w.seed)
    dq, dk, dv = _dev(q, k, v)
    out = _poison_out(q.shape, q.dtype)
    lse = _poison_lse((1, w.heads_q, w.seqlen_q))
    ex.attn_func(dq, dk, dv, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any() and torch.isfinite(lse).all()
    # convex combination: |O| never exceeds the largest |V| of its column
    vmax = dv.abs().amax(dim=1, keepdim=True).float()
    assert (out.float().abs() <= vmax * (1 + 1e-2) + 1e-6).all()
    rows = np.array(sorted({0, 1, 63, 64, 127, 128, 129, 4095, 8191, 8192, 12345, 16255, 16256,
                            16382, 16383}))
    heads = [0, 7, 15]
    o_ref, l_ref = oracle.attention(q, k, v, causal=True, rows=rows, heads=heads)
    o_cpu, l_cpu = out.cpu(), lse.cpu()
    for h in heads:
        assert_o_close(o_cpu[:, rows, h], o_ref[:, rows, h], q.dtype, f"long h{h}")
        assert_lse_close(l_cpu[:, h, rows], l_ref[:, h, rows], f"long h{h}")


def test_decode_kvcache():
    w = W.WORKLOADS["decode"]
    q, kc, vc = W.kvcache(w.batch, w.seqlen_k, w.heads_q, w.heads_kv, w.head_dim, seed=w.seed)
    lens = torch.tensor(w.cache_seqlens, dtype=torch.int32)
    dq, dkc, dvc, dl = _dev(q, kc, vc, lens)
    out = _poison_out(q.shape, q.dtype)
    lse = _poison_lse((w.batch, w.heads_q, 1))
    ns, _ = ex.decode_plan(dq[:, 0], dkc, dvc, dl)
    assert ns > 1
    ex.attn_with_kvcache(dq, dkc, dvc, cache_seqlens=dl, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_kvcache(q, kc, vc, lens, causal=True)
    assert_o_close(out, o_ref, q.dtype, "decode")
    assert_lse_close(lse, l_ref, "decode")


APPEND_CASES = [
    # b, s_cache, h_q, h_kv, d, dtype, lens, s_new, window, softcap, splits, seed
    (4, 2048, 32, 8, 128, torch.bfloat16, [0, 5, 1000, 2045], 3, (-1, -1), 0.0, 0, 160),
    (3, 777, 16, 2, 64, torch.float16, [1, 300, 770], 7, (100, -1), 30.0, 0, 161),
    (2, 4096, 8, 8, 256, torch.bfloat16, [4000, 17], 1, (-1, -1), 0.0, 5, 162),
    (2, 1000, 16, 4, 128, torch.float16, [999, 0], 1, (-1, -1), 0.0, 1, 163),
    (2, 500, 8, 2, 128, torch.bfloat16, [10, 200], 7, (3, -1), 0.0, 4, 164),   # new rows left of the window
    (2, 300, 12, 6, 128, torch.float16, [0, 250], 2, (-1, -1), 0.0, 0, 165),   # a partial KV-head group
]


@pytest.mark.parametrize("case", APPEND_CASES, ids=[f"a{c[-1]}" for c in APPEND_CASES])
def test_decode_append(case):
    """k/v appended at cache_seqlens[b] (FAQ Q17), then attended: O and LSE against
    the oracle, the new cache rows bit-exact, every other row untouched, and
    cache_seqlens unchanged."""
    b, s_cache, hq, hkv, d, dt, lens, s_new, window, cap, splits, seed = case
    q, kc, vc = W.kvcache(b, s_cache, hq, hkv, d, seed=seed, dtype=dt)
    kn, vn = W.kv_new(b, s_new, hkv, d, seed=seed + 1000, dtype=dt)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    dq, dkc, dvc, dl = _dev(q, kc, vc, lens_t)
    dkv = torch.stack([kn, vn], dim=2).to(DEV)  # the packed (b, s_new, 2, h_kv, d) draw
    dkn, dvn = dkv[:, :, 0], dkv[:, :, 1]
    assert dkn.stride(1) == 2 * hkv * d  # strided views
    out = _poison_out(q.shape, q.dtype)
    lse = _poison_lse((b, hq, 1))
    ex.attn_with_kvcache(dq, dkc, dvc, k=dkn, v=dvn, cache_seqlens=dl, causal=True, window_size=window,
                         softcap=cap, num_splits=splits, out=out, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref, kc_ref, vc_ref = oracle.attention_kvcache_append(q, kc, vc, kn, vn, lens_t, causal=True,
                                                                   window_size=window, softcap=cap)
    assert_o_close(out, o_ref, dt, "append")
    assert_lse_close(lse, l_ref, "append")
    assert torch.equal(dkc.cpu(), kc_ref) and torch.equal(dvc.cpu(), vc_ref)
    assert torch.equal(dl.cpu(), lens_t)


def test_decode_append_steps():
    """Token-by-token decoding as in FAQ Q17: append one token, attend, then the
    caller advances cache_seqlens; four steps against the oracle."""
    b, s_cache, hq, hkv, d = 3, 600, 16, 4, 128
    q, kc, vc = W.kvcache(b, s_cache, hq, hkv, d, seed=170)
    dkc, dvc = _dev(kc, vc)
    lens = torch.tensor([0, 100, 590], dtype=torch.int32)
    dl = lens.to(DEV)
    kc_ref, vc_ref = kc.clone(), vc.clone()
    for step in range(4):
        kn, vn = W.kv_new(b, 1, hkv, d, seed=171 + step)
        qs = W.kvcache(b, 1, hq, hkv, d, seed=180 + step)[0]
        out, lse = ex.attn_with_kvcache(qs.to(DEV), dkc, dvc, k=kn.to(DEV), v=vn.to(DEV), cache_seqlens=dl,
                                        causal=True)
        torch.cuda.synchronize()
        o_ref, l_ref, kc_ref, vc_ref = oracle.attention_kvcache_append(qs, kc_ref, vc_ref, kn, vn, lens,
                                                                       causal=True)
        assert_o_close(out, o_ref, qs.dtype, f"append step {step}")
        assert_lse_close(lse, l_ref, f"append step {step}")
        dl += 1
        lens += 1
    assert torch.equal(dkc.cpu(), kc_ref) and torch.equal(dvc.cpu(), vc_ref)


MULTI_CASES = [
    # b, s_cache, h_q, h_kv, d, dtype, lens, s_q, s_new, causal, window, softcap, splits, paged, seed
    (4, 2048, 32, 8, 128, torch.bfloat16, [0, 5, 1000, 2040], 4, 4, True, (-1, -1), 0.0, 0, 0, 420),   # 16 columns
    (3, 777, 16, 2, 64, torch.float16, [1, 300, 760], 7, 7, True, (100, -1), 30.0, 0, 0, 421),   # 56 columns
    (2, 4096, 8, 8, 256, torch.bfloat16, [4000, 17], 2, 0, True, (-1, -1), 0.0, 5, 0, 422),
    (2, 1000, 16, 4, 128, torch.float16, [996, 0], 3, 1, True, (-1, -1), 0.0, 1, 0, 423),     # s_q != s_new
    (2, 3000, 32, 8, 128, torch.bfloat16, [3000, 1234], 5, 0, False, (-1, -1), 0.0, 0, 0, 424),  # non-causal
    (3, 1024, 16, 8, 128, torch.bfloat16, [0, 100, 1000], 5, 5, True, (-1, -1), 0.0, 0, 64, 425),  # paged
    (2, 512, 8, 2, 128, torch.bfloat16, [2, 300], 4, 0, True, (7, 0), 0.0, 3, 0, 426),   # tokens before key 0
]


@pytest.mark.parametrize("case", MULTI_CASES, ids=[f"q{c[-1]}" for c in MULTI_CASES])
def test_decode_multi_query(case):
    """Several query tokens against the KV cache (FAQ Q17 with causal, bottom-right per
    FAQ Q6): with an append of s_new tokens, token t sits at position
    cache_seqlens[b] + s_new - s_q + t; O and LSE against the oracle, appended rows
    bit-exact, and the pool untouched elsewhere when paged."""
    b, s_cache, hq, hkv, d, dt, lens, s_q, s_new, causal, window, cap, splits, page, seed = case
    q, kc, vc = W.kvcache(b, s_cache, hq, hkv, d, seed=seed, dtype=dt)
    q = W.qkv(b, s_q, 1, hq, 1, d, seed=seed + 2000, dtype=dt)[0]
    lens_t = torch.tensor(lens, dtype=torch.int32)
    dq, dl = _dev(q, lens_t)
    kw = {}
    if s_new:
        kn, vn = W.kv_new(b, s_new, hkv, d, seed=seed + 1000, dtype=dt)
        kw = dict(k=kn.to(DEV), v=vn.to(DEV))
    if page:
        gen = torch.Generator().manual_seed(seed)
        kp, bt = _to_pages(kc, page, 2, gen)
        vp, _ = _to_pages(vc, page, 2, torch.Generator().manual_seed(seed))
        dkc, dvc, dbt = _dev(kp, vp, bt)
        kw["block_table"] = dbt
    else:
        dkc, dvc = _dev(kc, vc)
    out = _poison_out(q.shape, dt)
    lse = _poison_lse((b, hq, s_q))
    ex.attn_with_kvcache(dq, dkc, dvc, cache_seqlens=dl, causal=causal, window_size=window, softcap=cap,
                         num_splits=splits, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    if s_new:
        o_ref, l_ref, kc_ref, vc_ref = oracle.attention_kvcache_append(q, kc, vc, kn, vn, lens_t, causal=causal,
                                                                       window_size=window, softcap=cap)
        got_k = oracle.paged_to_contiguous(dkc.cpu(), bt, s_cache) if page else dkc.cpu()
        got_v = oracle.paged_to_contiguous(dvc.cpu(), bt, s_cache) if page else dvc.cpu()
        assert torch.equal(got_k, kc_ref) and torch.equal(got_v, vc_ref)
    else:
        o_ref, l_ref = oracle.attention_kvcache(q, kc, vc, lens_t, causal=causal, window_size=window, softcap=cap)
    assert_o_close(out, o_ref, dt, f"multi-query {seed}")
    assert_lse_close(lse, l_ref, f"multi-query {seed}")


def test_decode_multi_query_split_independent():
    """The same multi-token call with 1, 3 and 16 splits agrees with the oracle each time."""
    q, kc, vc = W.kvcache(2, 2000, 16, 4, 128, seed=427)
    q = W.qkv(2, 3, 1, 16, 1, 128, seed=428)[0]
    lens = torch.tensor([2000, 777], dtype=torch.int32)
    dq, dkc, dvc, dl = _dev(q, kc, vc, lens)
    o_ref, l_ref = oracle.attention_kvcache(q, kc, vc, lens, causal=True)
    for ns in (1, 3, 16):
        out, lse = ex.attn_with_kvcache(dq, dkc, dvc, cache_seqlens=dl, causal=True, num_splits=ns)
        torch.cuda.synchronize()
        assert_o_close(out, o_ref, q.dtype, f"splits {ns}")
        assert_lse_close(lse, l_ref, f"splits {ns}")


def _to_pages(cache, page, spare, gen):
    """Scatter a contiguous cache (b, s, h, d) into a pool of pages at a random
    permutation of page slots; returns (pool, block_table)."""
    b, s_cache = cache.shape[:2]
    per_seq = -(-s_cache // page)
    n_pages = b * per_seq + spare
    perm = torch.randperm(n_pages, generator=gen)
    pool = torch.zeros((n_pages, page) + tuple(cache.shape[2:]), dtype=cache.dtype)
    bt = torch.zeros((b, per_seq), dtype=torch.int32)
    for bi in range(b):
        for i in range(per_seq):
            slot = int(perm[bi * per_seq + i])
            bt[bi, i] = slot
            rows = cache[bi, i * page:(i + 1) * page]
            pool[slot, :rows.shape[0]] = rows
    return pool, bt


PAGED_CASES = [
    # b, pages per seq, page, h_q, h_kv, d, dtype, lens, window, softcap, splits, s_new, seed
    (3, 8, 256, 32, 8, 128, torch.bfloat16, [2048, 1, 1000], (-1, -1), 0.0, 0, 0, 190),
    (2, 64, 16, 16, 8, 128, torch.float16, [1024, 77], (-1, -1), 0.0, 6, 0, 191),
    (2, 8, 64, 16, 16, 64, torch.bfloat16, [500, 13], (40, -1), 20.0, 0, 0, 192),
    (2, 4, 128, 8, 4, 256, torch.float16, [512, 300], (-1, -1), 0.0, 3, 0, 193),
    (3, 16, 16, 16, 8, 128, torch.bfloat16, [0, 100, 250], (-1, -1), 0.0, 0, 5, 194),  # append
    (2, 8, 64, 8, 8, 128, torch.bfloat16, [300, 10], (2, -1), 0.0, 2, 7, 195),         # append, window
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=[f"p{c[-1]}" for c in PAGED_CASES])
def test_decode_paged(case):
    """Paged KV cache (FAQ Q18): O and LSE against the oracle on the same cache
    laid out contiguously; without a window and append, bitwise equal to the
    contiguous decode with the same split count; appended rows land in their
    pages and nothing else in the pool changes."""
    b, per_seq, page, hq, hkv, d, dt, lens, window, cap, splits, s_new, seed = case
    s_cache = per_seq * page
    q, kc, vc = W.kvcache(b, s_cache, hq, hkv, d, seed=seed, dtype=dt)
    gen = torch.Generator().manual_seed(seed)
    kpool, bt = _to_pages(kc, page, 3, gen)
    vpool, _ = _to_pages(vc, page, 3, torch.Generator().manual_seed(seed))  # same permutation
    lens_t = torch.tensor(lens, dtype=torch.int32)
    dq, dkp, dvp, dbt, dl = _dev(q, kpool, vpool, bt, lens_t)
    kw = {}
    if s_new:
        kn, vn = W.kv_new(b, s_new, hkv, d, seed=seed + 1000, dtype=dt)
        kw = dict(k=kn.to(DEV), v=vn.to(DEV))
    out = _poison_out(q.shape, q.dtype)
    lse = _poison_lse((b, hq, 1))
    ex.attn_with_kvcache(dq, dkp, dvp, cache_seqlens=dl, causal=True, window_size=window, softcap=cap,
                         num_splits=splits, out=out, lse=lse, block_table=dbt, **kw)
    torch.cuda.synchronize()
    if s_new:
        o_ref, l_ref, kc_ref, vc_ref = oracle.attention_kvcache_append(q, kc, vc, kn, vn, lens_t, causal=True,
                                                                       window_size=window, softcap=cap)
        assert torch.equal(oracle.paged_to_contiguous(dkp.cpu(), bt, s_cache), kc_ref)
        assert torch.equal(oracle.paged_to_contiguous(dvp.cpu(), bt, s_cache), vc_ref)
        used = set(bt.flatten().tolist())
        spare = [i for i in range(kpool.shape[0]) if i not in used]
        assert torch.equal(dkp.cpu()[spare], kpool[spare]) and torch.equal(dvp.cpu()[spare], vpool[spare])
    else:
        o_ref, l_ref = oracle.attention_kvcache(q, kc, vc, lens_t, causal=True, window_size=window, softcap=cap)
    assert_o_close(out, o_ref, dt, "paged")
    assert_lse_close(lse, l_ref, "paged")
    if not s_new and window == (-1, -1):
        dkc, dvc = _dev(kc, vc)
        o2, l2 = ex.attn_with_kvcache(dq, dkc, dvc, cache_seqlens=dl, causal=True, softcap=cap,
                                      num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(out, o2) and torch.equal(lse, l2)


def test_decode_paged_rejects_small_pages():
    """With two KV heads a step covers 64 keys at d = 128: 16-token pages are refused."""
    q, kc, vc = W.kvcache(1, 256, 4, 2, 128, seed=196)
    kpool, bt = _to_pages(kc, 16, 0, torch.Generator().manual_seed(1))
    dq, dkp, dbt = _dev(q, kpool, bt)
    with pytest.raises(NotImplementedError, match="multiple of 64"):
        ex.attn_with_kvcache(dq, dkp, dkp, cache_seqlens=torch.tensor([256], dtype=torch.int32, device=DEV),
                             block_table=dbt)


# Gradient tolerance.  The pages give none for the backward.  The kernels round
# P and dS to the input type before their MFMAs, form D = dO . O from the
# output O rounded to the input type, and round dQ, dK, dV once more.  Each
# gradient element is a sum of terms; rounding each term's factors by a unit
# roundoff u moves the sum by at most about u times the sum of the terms'
# absolute values (the oracle's term magnitudes), whatever the cancellation.
# So per element |g - g_ref| <= 4 u (mag + |g_ref|), u = 2^-8 for bf16 and
# 2^-11 for fp16: one u each for P or dS, D, the output rounding, and one in
# reserve (the forward's own O and LSE errors).  Where mag and g_ref are both
# 0 (a row or key that sees nothing) the gradient must be exactly 0.
GRAD_U = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


def assert_grad_close(g, ref, mag, dtype, where):
    g = g.detach().float().cpu().numpy().astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, f"{where}: shape {g.shape} vs {ref.shape}"
    assert np.isfinite(g).all(), f"{where}: non-finite gradient"
    u = GRAD_U[dtype]
    bound = 4 * u * (np.asarray(mag) + np.abs(ref))
    err = np.abs(g - ref)
    bad = err > bound
    worst = float(np.max(np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), 0.0))) if err.size else 0.0
    print(f"{where}: worst err / bound = {worst:.3f}")
    assert not bad.any(), (f"{where}: {int(bad.sum())} of {bad.size} out of tolerance (max err {err.max():.3e}); "
                           f"first at {np.argwhere(bad)[:3].tolist()}")


BWD_CASES = [
    # b, s_q, s_k, h_q, h_kv, d, dtype, causal, window, seed
    (2, 200, 200, 4, 4, 128, torch.bfloat16, True, (-1, -1), 200),
    (1, 130, 300, 8, 2, 64, torch.float16, False, (-1, -1), 201),
    (2, 257, 100, 4, 1, 128, torch.float16, True, (-1, -1), 202),    # rows without keys
    (1, 300, 300, 2, 2, 128, torch.bfloat16, False, (50, 10), 203),
    (1, 64, 64, 2, 2, 64, torch.bfloat16, False, (-1, -1), 204),
    (1, 1, 513, 4, 2, 128, torch.bfloat16, True, (-1, -1), 205),      # one row
    (1, 77, 40, 4, 2, 64, torch.float16, False, (5, -1), 206),        # left window only
    (2, 1024, 1024, 16, 16, 128, torch.bfloat16, True, (-1, -1), 207),  # the causal training shape
    # d = 128 with a mask bounded on one side: 64-key dK/dV tiles in 4 sets
    (1, 300, 700, 8, 2, 128, torch.bfloat16, False, (120, -1), 215),   # left window only
    (2, 333, 900, 6, 3, 128, torch.float16, True, (-1, -1), 216),      # s_q < s_k, ragged last tile
    # 1024 query tiles and more: the dQ kernel without the key split
    (1, 2048, 2048, 32, 8, 64, torch.bfloat16, True, (-1, -1), 209),
    (1, 1024, 1024, 64, 16, 128, torch.float16, False, (-1, -1), 210),
    # head_dim 256: dK and dV in two head-dim slices, dQ always with the key split
    (2, 200, 200, 4, 2, 256, torch.bfloat16, True, (-1, -1), 211),
    (1, 130, 300, 4, 4, 256, torch.float16, False, (-1, -1), 212),
    (1, 257, 100, 2, 1, 256, torch.bfloat16, True, (-1, -1), 213),    # rows without keys
    (1, 512, 512, 8, 8, 256, torch.float16, False, (100, 20), 214),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[f"g{c[-1]}" for c in BWD_CASES])
def test_backward(case):
    """dQ, dK, dV from the GPU forward's O and LSE against the oracle's gradients;
    two runs bitwise equal (no atomics)."""
    b, sq, sk, hq, hkv, d, dt, causal, window, seed = case
    q, k, v = W.qkv(b, sq, sk, hq, hkv, d, seed=seed, dtype=dt)
    dout = W.qkv(b, sq, 1, hq, 1, d, seed=seed + 1000, dtype=dt)[0]
    dq_, dk_, dv_, ddo = _dev(q, k, v, dout)
    out, lse = ex.attn_func(dq_, dk_, dv_, causal=causal, window_size=window)
    gq, gk, gv = ex.attn_backward(ddo, dq_, dk_, dv_, out, lse, causal=causal, window_size=window)
    gq2, gk2, gv2 = ex.attn_backward(ddo, dq_, dk_, dv_, out, lse, causal=causal, window_size=window)
    torch.cuda.synchronize()
    assert torch.equal(gq, gq2) and torch.equal(gk, gk2) and torch.equal(gv, gv2)
    rq, rk, rv = oracle.attention_backward(q, k, v, dout, causal=causal, window_size=window)
    mq, mk, mv = oracle.attention_backward_magnitudes(q, k, v, dout, causal=causal, window_size=window)
    assert_grad_close(gq, rq, mq, dt, "dq")
    assert_grad_close(gk, rk, mk, dt, "dk")
    assert_grad_close(gv, rv, mv, dt, "dv")


BWD_CAP_CASES = [
    # b, s_q, s_k, h_q, h_kv, d, dtype, causal, window, softcap, scale, seed
    (2, 200, 200, 4, 4, 128, torch.bfloat16, True, (-1, -1), 30.0, None, 230),
    (1, 130, 300, 8, 2, 64, torch.float16, False, (-1, -1), 5.0, None, 231),
    (1, 300, 300, 2, 2, 128, torch.bfloat16, False, (50, 10), 2.0, None, 232),   # saturating cap
    (2, 257, 100, 4, 1, 128, torch.float16, True, (-1, -1), 20.0, -0.09, 233),   # negative scale, empty rows
    (1, 1024, 1024, 16, 16, 128, torch.bfloat16, True, (-1, -1), 50.0, None, 234),
    (1, 200, 200, 4, 2, 256, torch.bfloat16, True, (-1, -1), 30.0, None, 237),
    (1, 150, 150, 2, 2, 256, torch.float16, False, (-1, -1), 2.0, -0.07, 238),  # saturating, negative scale
    (1, 100, 150, 4, 2, 64, torch.bfloat16, True, (-1, -1), 10.0, None, 239),
    # 1024 query tiles and more: the dQ kernel without the key split, with softcap
    (1, 1024, 1024, 64, 16, 128, torch.bfloat16, True, (-1, -1), 30.0, None, 245),
    (1, 2048, 2048, 32, 8, 64, torch.float16, False, (-1, -1), 20.0, None, 246),
]


@pytest.mark.parametrize("case", BWD_CAP_CASES, ids=[f"c{c[-1]}" for c in BWD_CAP_CASES])
def test_backward_softcap(case):
    """The backward through the softcap (FAQ Q22: c tanh(s / c) before the mask) against the
    oracle's gradients, which differentiate through the cap."""
    b, sq, sk, hq, hkv, d, dt, causal, window, cap, scale, seed = case
    q, k, v = W.qkv(b, sq, sk, hq, hkv, d, seed=seed, dtype=dt)
    if cap <= 2.0:
        q, k = (q.float() * 3).to(dt), (k.float() * 3).to(dt)
    dout = W.qkv(b, sq, 1, hq, 1, d, seed=seed + 1000, dtype=dt)[0]
    dq_, dk_, dv_, ddo = _dev(q, k, v, dout)
    kw = dict(causal=causal, window_size=window, softcap=cap, softmax_scale=scale)
    out, lse = ex.attn_func(dq_, dk_, dv_, **kw)
    gq, gk, gv = ex.attn_backward(ddo, dq_, dk_, dv_, out, lse, **kw)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(q, k, v, dout, **kw)
    mq, mk, mv = oracle.attention_backward_magnitudes(q, k, v, dout, **kw)
    assert_grad_close(gq, rq, mq, dt, "dq")
    assert_grad_close(gk, rk, mk, dt, "dk")
    assert_grad_close(gv, rv, mv, dt, "dv")


@pytest.mark.parametrize("causal,window,cap,d", [(True, (-1, -1), 0.0, 128), (False, (40, 7), 0.0, 128),
                                                 (True, (256, 0), 50.0, 128), (True, (-1, -1), 0.0, 256)])
def test_backward_varlen(causal, window, cap, d):
    """Packed sequences (FAQ Q8), ragged and empty ones included: each sequence's gradients
    against the oracle's on that sequence alone."""
    lens_q = [1, 0, 300, 129, 64, 77]
    lens_k = [5, 3, 300, 1, 300, 77]
    hq, hkv = 8, 2
    q, k, v, cu_q, cu_k = W.varlen_qkv(lens_q, lens_k, hq, hkv, d, seed=235)
    dout = W.varlen_qkv(lens_q, [1] * len(lens_q), hq, 1, d, seed=236)[0]
    dq_, dk_, dv_, dcq, dck, ddo = _dev(q, k, v, cu_q, cu_k, dout)
    kw = dict(causal=causal, window_size=window, softcap=cap)
    out, lse = ex.attn_varlen_func(dq_, dk_, dv_, dcq, dck, max(lens_q), max(lens_k), **kw)
    gq = torch.full_like(dq_, float("nan"))
    gk = torch.full_like(dk_, float("nan"))
    gv = torch.full_like(dv_, float("nan"))
    ex.attn_varlen_backward(ddo, dq_, dk_, dv_, out, lse, dcq, dck, max(lens_q), max(lens_k), dq=gq, dk=gk,
                            dv=gv, **kw)
    torch.cuda.synchronize()
    gq, gk, gv = gq.cpu(), gk.cpu(), gv.cpu()
    for i in range(len(lens_q)):
        a, e = int(cu_q[i]), int(cu_q[i + 1])
        ka, ke = int(cu_k[i]), int(cu_k[i + 1])
        qs, ks, vs, ds = q[None, a:e], k[None, ka:ke], v[None, ka:ke], dout[None, a:e]
        rq, rk, rv = oracle.attention_backward(qs, ks, vs, ds, **kw)
        mq, mk, mv = oracle.attention_backward_magnitudes(qs, ks, vs, ds, **kw)
        assert_grad_close(gq[None, a:e], rq, mq, q.dtype, f"seq {i} dq")
        assert_grad_close(gk[None, ka:ke], rk, mk, q.dtype, f"seq {i} dk")
        assert_grad_close(gv[None, ka:ke], rv, mv, q.dtype, f"seq {i} dv")


@pytest.mark.parametrize("s_q,s_k", [(0, 50), (40, 0)])
def test_backward_empty_side(s_q, s_k):
    """No query rows: dK = dV = 0; no keys: dQ = 0 (the buffers start as NaN)."""
    q, k, v = W.qkv(2, s_q, s_k, 4, 2, 128, seed=208, dtype=torch.bfloat16)
    dout = W.qkv(2, s_q, 1, 4, 1, 128, seed=209, dtype=torch.bfloat16)[0]
    dq_, dk_, dv_, ddo = _dev(q, k, v, dout)
    out, lse = ex.attn_func(dq_, dk_, dv_, causal=False)
    gq, gk, gv = (torch.full_like(t, float("nan")) for t in (dq_, dk_, dv_))
    ex.attn_backward(ddo, dq_, dk_, dv_, out, lse, dq=gq, dk=gk, dv=gv)
    torch.cuda.synchronize()
    for t in (gq, gk, gv):
        assert torch.equal(t, torch.zeros_like(t))


FP8_CASES = [
    # b, s_q, s_k, h_q, h_kv, d, causal, window, (q, k, v descale), seed
    (2, 200, 200, 4, 4, 128, True, (-1, -1), (0.5, 2.0, 1.5), 220),
    (1, 130, 300, 8, 2, 64, False, (-1, -1), (1.0, 1.0, 1.0), 221),
    (2, 257, 100, 4, 1, 128, True, (-1, -1), (1.0, 0.25, 4.0), 222),   # rows without keys
    (1, 300, 300, 2, 2, 128, False, (50, 10), (2.0, 2.0, 0.5), 223),
    (1, 1, 513, 4, 2, 64, True, (-1, -1), (1.0, 1.0, 1.0), 224),      # one row
    (2, 1024, 1024, 16, 16, 128, True, (-1, -1), (1.0, 1.0, 1.0), 225),  # the causal prefill shape
    # 1024 tiles and more take the kernel without the key split
    (1, 2048, 2048, 32, 8, 128, True, (-1, -1), (0.5, 1.0, 2.0), 227),
    (1, 2048, 1500, 32, 32, 64, False, (300, 40), (1.0, 1.0, 1.0), 228),
]


def _check_fp8(out, lse, q, k, v, ds, causal, window, cap, where, scale=None):
    """O and LSE of one FP8 call (4-D tensors, one batch entry or more) against the oracle on
    the decoded inputs."""
    dsq, dsk, dsv = ds
    b, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    ro, rl = oracle.attention_fp8(q, k, v, q_descale=dsq, k_descale=dsk, v_descale=dsv, causal=causal,
                                  window_size=window, softcap=cap, softmax_scale=scale)
    # FAQ Q10's FP8 tolerance is for values at the codes' own scale: O is compared after
    # dividing by v_descale (the real V is code x v_descale, so P's rounding moves O by
    # amounts proportional to it).
    assert_o_close(out.float() / dsv, np.nan_to_num(ro) / dsv, "fp8", f"{where} O")
    # LSE: the FP8 MFMA sums its 16 products with a shorter mantissa than fp32 (a probe
    # of 16-term dot products measured errors near 2^-15 of the sum of |products|), and a
    # score takes d / 16 such sums, so a score may move by about (d / 16) 2^-15 of
    # scale * sum_i |q_i k_i|; the LSE moves by at most the largest such move (the softcap
    # c tanh(s / c) has slope at most 1, so it moves no more).  Bound per row:
    # 1e-4 + 2^-11 * scale_eff * max_j sum_i |q_i k_i| (d = 128 gives 2^-12 per sum,
    # times 2 in reserve).
    qa = np.abs(oracle.decode_e4m3(q))
    ka = np.abs(oracle.decode_e4m3(k))
    g = hq // hkv
    mag = np.stack([np.stack([(qa[bi, :, h] @ ka[bi, :, h // g].T).max(axis=1) if sk else np.zeros(sq)
                              for h in range(hq)]) for bi in range(b)])  # (b, h, s_q)
    scale_eff = abs(dsq * dsk) * (abs(scale) if scale is not None else 1.0 / math.sqrt(d))
    lg = lse.detach().cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(lg), np.isneginf(rl)), f"{where} LSE: -inf pattern differs"
    fin = ~np.isneginf(rl)
    bound = 1e-4 + 2.0 ** -11 * scale_eff * mag
    assert not np.isnan(lg).any()
    err = np.zeros_like(rl)
    err[fin] = np.abs(lg[fin] - rl[fin])  # -inf rows already matched exactly above
    assert np.all(err[fin] <= bound[fin]), (f"{where} LSE: max err {err[fin].max():.3e}, "
                                            f"worst err/bound {(err[fin] / bound[fin]).max():.3f}")


@pytest.mark.parametrize("case", FP8_CASES, ids=[f"f{c[-1]}" for c in FP8_CASES])
def test_fp8_forward(case):
    """The FP8 forward (bf16 out) against the oracle on the decoded inputs, FAQ Q10's FP8
    tolerance (1e-2 / 1e-2) on O, 1e-4 on LSE; two runs bitwise equal."""
    b, sq, sk, hq, hkv, d, causal, window, (dsq, dsk, dsv), seed = case
    q, k, v = W.qkv(b, sq, sk, hq, hkv, d, seed=seed, dtype=torch.float8_e4m3fn)
    gq, gk, gv = _dev(q, k, v)
    out, lse = ex.attn_func_fp8(gq, gk, gv, q_descale=dsq, k_descale=dsk, v_descale=dsv, causal=causal,
                                window_size=window)
    out2, lse2 = ex.attn_func_fp8(gq, gk, gv, q_descale=dsq, k_descale=dsk, v_descale=dsv, causal=causal,
                                  window_size=window)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    _check_fp8(out, lse, q, k, v, (dsq, dsk, dsv), causal, window, 0.0, "fp8")


# 1024 tiles and more without softcap take the software-pipelined loop (QK of one
# block beside the exponentials of the one before, a lazy softmax reference),
# unless scale x descales is 0.
FP8_PIPE_CASES = [
    # b, s_q, s_k, h_q, h_kv, d, causal, window, (q, k, v descale), softmax scale, seed
    (1, 2048, 2048, 32, 32, 128, True, (-1, -1), (1.0, 1.0, 1.0), -0.06, 230),   # negative scale
    (1, 4096, 1000, 16, 4, 64, True, (-1, -1), (1.0, 2.0, 1.0), None, 231),      # rows without keys
    (1, 2048, 2048, 32, 32, 128, False, (200, 50), (0.0, 1.0, 1.0), None, 232),  # scale 0: plain loop
    (1, 2048, 2048, 32, 8, 128, False, (-1, -1), (4.0, 4.0, 1.0), None, 233),    # large scores: rescales
]


@pytest.mark.parametrize("case", FP8_PIPE_CASES, ids=[f"f{c[-1]}" for c in FP8_PIPE_CASES])
def test_fp8_pipelined(case):
    b, sq, sk, hq, hkv, d, causal, window, ds, scale, seed = case
    assert b * hq * math.ceil(sq / 64) >= 1024, "shape does not take the one-group kernel"
    q, k, v = W.qkv(b, sq, sk, hq, hkv, d, seed=seed, dtype=torch.float8_e4m3fn)
    gq, gk, gv = _dev(q, k, v)
    out, lse = ex.attn_func_fp8(gq, gk, gv, q_descale=ds[0], k_descale=ds[1], v_descale=ds[2],
                                softmax_scale=scale, causal=causal, window_size=window)
    torch.cuda.synchronize()
    _check_fp8(out, lse, q, k, v, ds, causal, window, 0.0, "fp8 pipelined", scale=scale)


def test_fp8_varlen_pipelined():
    """Varlen FP8 through the pipelined loop (1024 tiles and more over the longest
    sequence): sequences of 1, 3000 and 2500 rows, causal."""
    lens_q = [3000, 1, 2500]
    lens_k = [3000, 40, 2600]
    hq, hkv, d, ds = 16, 4, 128, (0.5, 2.0, 1.5)
    assert len(lens_q) * hq * math.ceil(max(lens_q) / 64) >= 1024
    q, k, v, cu_q, cu_k = W.varlen_qkv(lens_q, lens_k, hq, hkv, d, seed=234, dtype=torch.float8_e4m3fn)
    gq, gk, gv, dcq, dck = _dev(q, k, v, cu_q, cu_k)
    out = torch.full((q.shape[0], hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((hq, q.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
    ex.attn_varlen_func_fp8(gq, gk, gv, dcq, dck, max(lens_q), max(lens_k), q_descale=ds[0], k_descale=ds[1],
                            v_descale=ds[2], causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    for i in range(len(lens_q)):
        a, e = int(cu_q[i]), int(cu_q[i + 1])
        ka, ke = int(cu_k[i]), int(cu_k[i + 1])
        _check_fp8(out[None, a:e], lse[None, :, a:e], q[None, a:e], k[None, ka:ke], v[None, ka:ke], ds, True,
                   (-1, -1), 0.0, f"fp8 varlen pipelined seq {i}")


FP8_CAP_CASES = [
    # b, s_q, s_k, h_q, h_kv, d, causal, window, (q, k, v descale), softcap, seed
    (2, 200, 200, 4, 4, 128, True, (-1, -1), (0.5, 2.0, 1.5), 30.0, 240),
    (1, 130, 300, 8, 2, 64, False, (-1, -1), (1.0, 1.0, 1.0), 5.0, 241),
    (1, 300, 300, 2, 2, 128, False, (50, 10), (2.0, 2.0, 0.5), 2.0, 242),       # saturating
    (1, 2048, 2048, 32, 8, 128, True, (-1, -1), (0.5, 1.0, 2.0), 50.0, 243),  # kernel without the key split
]


@pytest.mark.parametrize("case", FP8_CAP_CASES, ids=[f"f{c[-1]}" for c in FP8_CAP_CASES])
def test_fp8_softcap(case):
    """The FP8 forward with softcap (FAQ Q20 with Q22) against the oracle on the decoded inputs."""
    b, sq, sk, hq, hkv, d, causal, window, ds, cap, seed = case
    q, k, v = W.qkv(b, sq, sk, hq, hkv, d, seed=seed, dtype=torch.float8_e4m3fn)
    gq, gk, gv = _dev(q, k, v)
    out, lse = ex.attn_func_fp8(gq, gk, gv, q_descale=ds[0], k_descale=ds[1], v_descale=ds[2], causal=causal,
                                window_size=window, softcap=cap)
    torch.cuda.synchronize()
    _check_fp8(out, lse, q, k, v, ds, causal, window, cap, "fp8 softcap")


@pytest.mark.parametrize("causal,window,cap", [(True, (-1, -1), 0.0), (False, (40, 7), 0.0), (True, (256, 0), 50.0)])
def test_fp8_varlen(causal, window, cap):
    """The FP8 forward over packed sequences (FAQ Q8), ragged and empty ones included: each
    sequence against the oracle on that sequence alone; rows past the packed total untouched."""
    lens_q = [1, 0, 300, 129, 64, 77]
    lens_k = [5, 3, 300, 1, 300, 77]
    hq, hkv, d, ds = 8, 2, 128, (0.5, 2.0, 1.5)
    q, k, v, cu_q, cu_k = W.varlen_qkv(lens_q, lens_k, hq, hkv, d, seed=244, dtype=torch.float8_e4m3fn)
    gq, gk, gv, dcq, dck = _dev(q, k, v, cu_q, cu_k)
    out = torch.full((q.shape[0], hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((hq, q.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
    ex.attn_varlen_func_fp8(gq, gk, gv, dcq, dck, max(lens_q), max(lens_k), q_descale=ds[0], k_descale=ds[1],
                            v_descale=ds[2], causal=causal, window_size=window, softcap=cap, out=out, lse=lse)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    for i in range(len(lens_q)):
        a, e = int(cu_q[i]), int(cu_q[i + 1])
        ka, ke = int(cu_k[i]), int(cu_k[i + 1])
        _check_fp8(out[None, a:e], lse[None, :, a:e], q[None, a:e], k[None, ka:ke], v[None, ka:ke], ds, causal,
                   window, cap, f"fp8 varlen seq {i}")


def test_fp8_rejects_on_gpu():
    q, k, v = _dev(*W.qkv(1, 64, 64, 2, 2, 128, seed=226, dtype=torch.float8_e4m3fn))
    with pytest.raises(NotImplementedError):
        ex.attn_func_fp8(q[..., :96].contiguous(), k[..., :96].contiguous(), v[..., :96].contiguous())
    with pytest.raises(ValueError):
        ex.attn_func_fp8(q.to(torch.bfloat16), k, v)


# --------------------------------------------------------------------------
# masks, tails and degenerate cases
# --------------------------------------------------------------------------
MASK_CASES = [
    # b, s_q, s_k, h_q, h_kv, d, dtype, causal, window, softcap, seed
    (1, 1024, 1024, 4, 4, 128, torch.bfloat16, True, (256, 0), 0.0, 101),     # window bites
    (2, 128, 64, 4, 2, 128, torch.bfloat16, True, (-1, -1), 0.0, 102),        # s_q > s_k: empty rows
    (1, 512, 2048, 4, 1, 128, torch.bfloat16, True, (-1, -1), 0.0, 103),      # s_q < s_k
    (1, 300, 300, 4, 4, 128, torch.float16, False, (-1, -1), 2.0, 104),       # saturating softcap
    (2, 200, 333, 4, 2, 64, torch.float16, False, (17, 5), 0.0, 105),         # ragged both, 2-sided
    (1, 77, 1000, 2, 1, 256, torch.bfloat16, True, (100, -1), 30.0, 106),
    (3, 129, 129, 6, 2, 128, torch.float16, True, (-1, -1), 0.0, 107),
    (1, 65, 1, 2, 2, 64, torch.bfloat16, False, (-1, -1), 0.0, 108),          # s_k = 1: O = V
    (1, 40, 3000, 2, 2, 256, torch.float16, False, (-1, 0), 0.0, 109),        # right edge only
    (2, 260, 260, 8, 8, 64, torch.bfloat16, True, (0, 0), 0.0, 110),          # window of one key
]


@pytest.mark.parametrize("case", MASK_CASES, ids=[f"m{c[-1]}" for c in MASK_CASES])
def test_masks_and_tails(case):
    b, s_q, s_k, h_q, h_kv, d, dt, causal, window, cap, seed = case
    q, k, v = W.qkv(b, s_q, s_k, h_q, h_kv, d, seed=seed, dtype=dt)
    if cap == 2.0:
        q, k = (q.float() * 4).to(dt), (k.float() * 4).to(dt)
    run_dense(q, k, v, f"mask case {seed}", causal=causal, window_size=window, softcap=cap)


@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (False, (9, 3)), (True, (33, -1))])
def test_zero_q_counts(causal, window):
    """Q = 0: every visible score is 0, so O is the mean of the visible V rows and LSE = ln(count)."""
    s_q, s_k = 150, 230
    _, k, v = W.qkv(2, s_q, s_k, 4, 2, 128, seed=120, dtype=torch.bfloat16)
    q = torch.zeros((2, s_q, 4, 128), dtype=torch.bfloat16)
    run_dense(q, k, v, "zero q", causal=causal, window_size=window, softcap=5.0)


def test_large_shift_stability():
    """Scores of order 1e3 (K + c): the online rescaling must stay finite and exact."""
    q, k, v = W.qkv(1, 256, 256, 2, 2, 128, seed=121, dtype=torch.float32)
    c = torch.randn(128, generator=torch.Generator().manual_seed(5)) * 40
    q = q.to(torch.bfloat16)
    k = (k + c).to(torch.bfloat16)
    v = v.to(torch.bfloat16)
    run_dense(q, k, v, "shift", causal=True)


def test_empty_keys_and_batch():
    q, k, v = W.qkv(2, 70, 0, 4, 4, 64, seed=122, dtype=torch.float16)
    out, lse = ex.attn_func(*_dev(q, torch.zeros((2, 0, 4, 64), dtype=torch.float16),
                                  torch.zeros((2, 0, 4, 64), dtype=torch.float16)))
    torch.cuda.synchronize()
    assert (out == 0).all() and torch.isneginf(lse).all()
    q0 = torch.zeros((0, 16, 4, 64), dtype=torch.float16, device=DEV)
    out0, lse0 = ex.attn_func(q0, q0, q0)
    assert out0.shape == (0, 16, 4, 64) and lse0.shape == (0, 4, 16)


def test_varlen_ragged_and_empty_sequences():
    lens_q = [1, 0, 600, 129, 64]
    lens_k = [5, 3, 600, 1, 300]
    q, k, v, cu_q, cu_k = W.varlen_qkv(lens_q, lens_k, 8, 2, 128, seed=123)
    dq, dk, dv, dcq, dck = _dev(q, k, v, cu_q, cu_k)
    for causal, window, cap in [(True, (-1, -1), 0.0), (False, (40, 7), 0.0), (True, (256, 0), 50.0)]:
        out = _poison_out(q.shape, q.dtype)
        lse = _poison_lse((8, q.shape[0]))
        ex.attn_varlen_func(dq, dk, dv, dcq, dck, max(lens_q), max(lens_k), causal=causal,
                            window_size=window, softcap=cap, out=out, lse=lse)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention_varlen(q, k, v, cu_q, cu_k, causal=causal, window_size=window,
                                               softcap=cap)
        assert_o_close(out, o_ref, q.dtype, f"varlen {causal} {window}")
        assert_lse_close(lse, l_ref, f"varlen {causal} {window}")


def test_packed_layouts_equal_contiguous():
    qkv = W.packed_qkv(2, 200, 4, 128, seed=124)
    d = qkv.to(DEV)
    o1, l1 = ex.attn_qkvpacked_func(d, causal=True)
    o2, l2 = ex.attn_func(d[:, :, 0].contiguous(), d[:, :, 1].contiguous(), d[:, :, 2].contiguous(),
                          causal=True)
    q = d[:, :, 0]
    kv = torch.stack([d[:, :, 1], d[:, :, 2]], dim=2)
    o3, l3 = ex.attn_kvpacked_func(q, kv, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_bitwise_determinism():
    q, k, v = _dev(*W.qkv(2, 700, 900, 8, 2, 128, seed=125))
    a = ex.attn_func(q, k, v, causal=True)
    b = ex.attn_func(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_default_scale_is_inverse_sqrt_d():
    q, k, v = _dev(*W.qkv(1, 100, 100, 2, 2, 64, seed=126, dtype=torch.float16))
    a = ex.attn_func(q, k, v)
    b = ex.attn_func(q, k, v, softmax_scale=1 / 8.0)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# --------------------------------------------------------------------------
# decode: ragged cache lengths, split counts, grouped heads, window, softcap
# --------------------------------------------------------------------------
DECODE_CASES = [
    # b, s_cache, h_q, h_kv, d, dtype, lens, window, softcap, splits, seed
    (6, 16384, 32, 8, 128, torch.bfloat16, [1, 17, 1000, 16384, 0, 4097], (-1, -1), 0.0, 0, 130),
    (2, 3000, 32, 1, 128, torch.bfloat16, [3000, 1234], (-1, -1), 0.0, 0, 131),    # 32 heads per KV head
    (3, 2048, 8, 8, 64, torch.float16, [2048, 100, 1500], (255, 0), 0.0, 3, 132),
    (2, 1024, 16, 4, 256, torch.bfloat16, [1024, 999], (-1, -1), 50.0, 5, 133),
    (1, 33, 4, 2, 128, torch.float16, [33], (-1, -1), 0.0, 1, 134),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"d{c[-1]}" for c in DECODE_CASES])
def test_decode_cases(case):
    b, s_cache, h_q, h_kv, d, dt, lens, window, cap, splits, seed = case
    q, kc, vc = W.kvcache(b, s_cache, h_q, h_kv, d, seed=seed, dtype=dt)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    dq, dkc, dvc, dl = _dev(q, kc, vc, lens_t)
    out = _poison_out(q.shape, dt)
    lse = _poison_lse((b, h_q, 1))
    ex.attn_with_kvcache(dq, dkc, dvc, cache_seqlens=dl, window_size=window, softcap=cap,
                         num_splits=splits, out=out, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_kvcache(q, kc, vc, lens, window_size=window, softcap=cap)
    assert_o_close(out, o_ref, dt, f"decode {seed}")
    assert_lse_close(lse, l_ref, f"decode {seed}")


@pytest.mark.parametrize("splits", [1, 2, 3, 5, 8, 16, 64, 0])
def test_decode_split_sweep(splits):
    q, kc, vc = W.kvcache(2, 4096, 16, 4, 128, seed=135)
    lens = torch.tensor([4096, 2500], dtype=torch.int32)
    dq, dkc, dvc, dl = _dev(q, kc, vc, lens)
    out, lse = ex.attn_with_kvcache(dq, dkc, dvc, cache_seqlens=dl, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_kvcache(q, kc, vc, lens)
    assert_o_close(out, o_ref, torch.bfloat16, f"splits {splits}")
    assert_lse_close(lse, l_ref, f"splits {splits}")


def test_decode_back_to_back_calls_reuse_workspace():
    """Many queued calls on one workspace, with changing split counts: every call equals the
    first call with the same split count bit for bit, and those match the oracle."""
    q, kc, vc = W.kvcache(4, 3000, 32, 8, 128, seed=138)
    lens = torch.tensor([3000, 1, 2047, 0], dtype=torch.int32)
    dq, dkc, dvc, dl = _dev(q, kc, vc, lens)
    ws = torch.zeros(8 << 20, dtype=torch.uint8, device=DEV)
    split_seq = [16, 16, 7, 93, 16, 2, 7, 0, 93, 16] * 3
    outs = []
    for ns in split_seq:
        out, lse = ex.attn_with_kvcache(dq, dkc, dvc, cache_seqlens=dl, num_splits=ns, workspace=ws)
        outs.append((ns, out, lse))
    torch.cuda.synchronize()
    first = {}
    for ns, out, lse in outs:
        if ns not in first:
            first[ns] = (out, lse)
            o_ref, l_ref = oracle.attention_kvcache(q, kc, vc, lens)
            assert_o_close(out, o_ref, torch.bfloat16, f"splits {ns}")
            assert_lse_close(lse, l_ref, f"splits {ns}")
        else:
            assert torch.equal(out, first[ns][0]) and torch.equal(lse, first[ns][1]), ns
    ns, wb = ex.decode_plan(dq[:, 0], dkc, dvc, dl, num_splits=93)
    assert wb <= ws.numel()


def test_decode_matches_prefill_row():
    """s_q = 1 through the prefill kernel and through the decode kernel agree with each other."""
    q, kc, vc = W.kvcache(2, 777, 8, 2, 128, seed=136)
    dq, dkc, dvc = _dev(q, kc, vc)
    o1, l1 = ex.attn_with_kvcache(dq, dkc, dvc, causal=True)
    o2, l2 = ex.attn_func(dq, dkc, dvc, causal=True)
    torch.cuda.synchronize()
    assert_o_close(o1.cpu(), o2.cpu().double().numpy(), torch.bfloat16, "decode vs prefill")
    assert (l1 - l2).abs().max().item() < 1e-4


def test_graph_capture_decode_replays():
    """The decode call captured in a graph (fixed addresses, FAQ Q19) replays correctly."""
    q, kc, vc = W.kvcache(2, 2048, 16, 4, 128, seed=137)
    lens = torch.tensor([2048, 1000], dtype=torch.int32)
    dq, dkc, dvc, dl = _dev(q, kc, vc, lens)
    out = torch.empty_like(dq)
    lse = torch.empty((2, 16, 1), dtype=torch.float32, device=DEV)
    ns, wb = ex.decode_plan(dq[:, 0], dkc, dvc, dl)
    ws = torch.zeros(max(wb, 256), dtype=torch.uint8, device=DEV)
    ex.attn_with_kvcache(dq, dkc, dvc, cache_seqlens=dl, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    eager_o, eager_l = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ex.attn_with_kvcache(dq, dkc, dvc, cache_seqlens=dl, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_o) and torch.equal(lse, eager_l)


@pytest.mark.parametrize("pack", [None, 0], ids=["auto", "unpacked"])
def test_graph_capture_prefill_and_backward(pack):
    """The forward and the backward captured in one graph (fixed addresses, FAQ Q19) replay
    to the eager results, with eager work and synchronisations between the replays (the
    automatic choice packs the GQA heads here; unpacked, the forward is the key-split
    kernel)."""
    q, k, v = W.qkv(2, 300, 300, 8, 2, 128, seed=409)
    dout = W.qkv(2, 300, 1, 8, 1, 128, seed=410)[0]
    dq_, dk_, dv_, ddo = _dev(q, k, v, dout)
    out = torch.empty_like(dq_)
    lse = torch.empty((2, 8, 300), dtype=torch.float32, device=DEV)
    gq, gk, gv = torch.empty_like(dq_), torch.empty_like(dk_), torch.empty_like(dv_)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)

    if pack == 0:
        assert _launch(2, 300, 8, 2, 128, True)[2], "unpacked, the shape takes the key-split kernel"

    def calls():
        ex.attn_func(dq_, dk_, dv_, causal=True, out=out, lse=lse, pack_gqa=pack)
        ex.attn_backward(ddo, dq_, dk_, dv_, out, lse, causal=True, dq=gq, dk=gk, dv=gv, workspace=ws)

    calls()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out, lse, gq, gk, gv)]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            calls()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (out, lse, gq, gk, gv):
            t.fill_(float("nan"))
        junk = (dq_.float() @ dq_.float().transpose(-1, -2)).sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for t, e in zip((out, lse, gq, gk, gv), eager):
            assert torch.equal(t, e), f"replay {rep}"
