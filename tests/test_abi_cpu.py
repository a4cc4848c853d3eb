"""The C ABI on the CPU: the library loads, exports what include/exattn.h
declares, its struct layout matches the binding, and every host-side argument
check fails with the documented status before anything is launched.

No call here reaches a GPU: each one is rejected (or is empty) on the host.
"""
import ctypes as C
import os
import re

import pytest

import exact_attention_43_amd as ex

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "exattn.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ex.library_path()):
        pytest.fail("libexattn.so is not built (run __graft_entry__.build())")
    return ex.lib()


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(exattn_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), f"{n} declared in exattn.h but not exported"


def test_struct_layout_and_version(L):
    assert L.exattn_args_size(0) == C.sizeof(ex.FwdArgs)
    assert L.exattn_args_size(1) == C.sizeof(ex.DecodeArgs)
    assert L.exattn_args_size(2) == C.sizeof(ex.KvNew)
    assert L.exattn_args_size(3) == C.sizeof(ex.PagedKv)
    assert L.exattn_args_size(4) == C.sizeof(ex.BwdArgs)
    assert L.exattn_args_size(5) == C.sizeof(ex.Fp8Descale)
    assert L.exattn_args_size(7) == 0
    assert L.exattn_abi_version() == 4
    assert L.exattn_status_string(0) == b"EXATTN_OK"
    assert L.exattn_status_string(3) == b"EXATTN_E_WORKSPACE"


FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced (rejected on the host)


def _fwd(**kw):
    a = ex.FwdArgs()
    a.dtype, a.batch, a.seqlen_q, a.seqlen_k = 1, 2, 64, 64
    a.heads_q, a.heads_kv, a.head_dim = 4, 4, 128
    a.q = a.k = a.v = a.o = FAKE
    for n in ("q_stride", "k_stride", "v_stride", "o_stride"):
        getattr(a, n)[:] = [64 * 4 * 128, 4 * 128, 128]
    a.lse_stride[:] = [4 * 64, 64]
    a.window_left = a.window_right = -1
    for key, val in kw.items():
        if key.endswith("_stride"):
            getattr(a, key)[:] = val
        else:
            setattr(a, key, val)
    return a


BAD_FWD = [
    ("dtype", dict(dtype=2), ex.EXATTN_E_UNSUPPORTED),
    ("head_dim 96", dict(head_dim=96), ex.EXATTN_E_UNSUPPORTED),
    ("head_dim 60", dict(head_dim=60), ex.EXATTN_E_UNSUPPORTED),
    ("heads ratio", dict(heads_q=6, heads_kv=4), ex.EXATTN_E_INVALID),
    ("heads zero", dict(heads_kv=0), ex.EXATTN_E_INVALID),
    ("negative batch", dict(batch=-1), ex.EXATTN_E_INVALID),
    ("negative seqlen", dict(seqlen_k=-3), ex.EXATTN_E_INVALID),
    ("null q", dict(q=None), ex.EXATTN_E_INVALID),
    ("null v", dict(v=None), ex.EXATTN_E_INVALID),
    ("misaligned k", dict(k=FAKE + 8), ex.EXATTN_E_INVALID),
    ("odd stride", dict(q_stride=[64 * 4 * 128, 4 * 128 + 4, 128]), ex.EXATTN_E_INVALID),
    ("negative stride", dict(o_stride=[-8, 512, 128]), ex.EXATTN_E_INVALID),
    ("token stride past 32-bit tile offsets", dict(k_stride=[1 << 30, 1 << 24, 128]),
     ex.EXATTN_E_UNSUPPORTED),
    ("half varlen", dict(cu_seqlens_q=FAKE), ex.EXATTN_E_INVALID),
    ("inf scale", dict(softmax_scale=float("inf")), ex.EXATTN_E_INVALID),
    ("nan softcap", dict(softcap=float("nan")), ex.EXATTN_E_INVALID),
    ("misaligned lse", dict(lse=FAKE + 2), ex.EXATTN_E_INVALID),
    ("pack_gqa 2", dict(pack_gqa=2), ex.EXATTN_E_INVALID),
    ("pack_gqa -2", dict(pack_gqa=-2), ex.EXATTN_E_INVALID),
]


@pytest.mark.parametrize("name,kw,status", BAD_FWD, ids=[c[0] for c in BAD_FWD])
def test_fwd_rejects(L, name, kw, status):
    st = L.exattn_fwd(C.byref(_fwd(**kw)), None)
    assert st == status, (name, st, L.exattn_last_error())
    assert L.exattn_last_error()  # a reason is given


def test_fwd_empty_is_ok_without_launch(L):
    assert L.exattn_fwd(C.byref(_fwd(batch=0)), None) == ex.EXATTN_OK
    assert L.exattn_fwd(C.byref(_fwd(seqlen_q=0)), None) == ex.EXATTN_OK
    assert L.exattn_fwd(C.byref(_fwd(batch=0, q=None, o=None)), None) == ex.EXATTN_OK


def test_fwd_null_args(L):
    assert L.exattn_fwd(None, None) == ex.EXATTN_E_INVALID


def _dec(**kw):
    a = ex.DecodeArgs()
    a.dtype, a.batch, a.heads_q, a.heads_kv, a.head_dim, a.seqlen_cache = 1, 8, 32, 8, 128, 16384
    a.q = a.k_cache = a.v_cache = a.o = FAKE
    a.q_stride[:] = [32 * 128, 128]
    a.o_stride[:] = [32 * 128, 128]
    a.k_stride[:] = [16384 * 8 * 128, 8 * 128, 128]
    a.v_stride[:] = [16384 * 8 * 128, 8 * 128, 128]
    a.window_left = a.window_right = -1
    a.num_splits = 4
    for key, val in kw.items():
        if key.endswith("_stride") and isinstance(val, list):
            getattr(a, key)[:] = val
        else:
            setattr(a, key, val)
    return a


BAD_DEC = [
    ("dtype", dict(dtype=5), ex.EXATTN_E_UNSUPPORTED),
    ("head_dim", dict(head_dim=80), ex.EXATTN_E_UNSUPPORTED),
    ("heads ratio", dict(heads_q=12, heads_kv=8), ex.EXATTN_E_INVALID),
    ("negative splits", dict(num_splits=-1), ex.EXATTN_E_INVALID),
    ("negative cache", dict(seqlen_cache=-1), ex.EXATTN_E_INVALID),
    ("null cache", dict(k_cache=None), ex.EXATTN_E_INVALID),
    ("odd stride", dict(k_stride=[16384 * 8 * 128, 8 * 128 + 2, 128]), ex.EXATTN_E_INVALID),
    # head-major cache: a step's tile spans 8 adjacent KV heads, 7 head strides of 2^28
    # elements = 3.5 GiB, beyond the kernel's 32-bit offsets
    ("head stride past 32-bit tile offsets", dict(v_stride=[8 << 28, 128, 1 << 28]),
     ex.EXATTN_E_UNSUPPORTED),
    ("token stride past 32-bit tile offsets", dict(k_stride=[1 << 40, 1 << 27, 128]),
     ex.EXATTN_E_UNSUPPORTED),
    ("negative seqlen_q", dict(seqlen_q=-1), ex.EXATTN_E_INVALID),
    ("odd query token stride", dict(seqlen_q=3, q_token_stride=4100), ex.EXATTN_E_INVALID),
    ("too many query columns", dict(seqlen_q=20000), ex.EXATTN_E_UNSUPPORTED),
]


@pytest.mark.parametrize("name,kw,status", BAD_DEC, ids=[c[0] for c in BAD_DEC])
def test_decode_rejects(L, name, kw, status):
    a = _dec(**kw)
    assert L.exattn_decode_plan(C.byref(a), None, None) == status, L.exattn_last_error()
    assert L.exattn_decode(C.byref(a), None, 0, None) == status, L.exattn_last_error()


def _kvn(**kw):
    n = ex.KvNew()
    n.k_new = n.v_new = FAKE
    n.seqlen_new = 2
    n.k_new_stride[:] = [2 * 8 * 128, 8 * 128, 128]
    n.v_new_stride[:] = [2 * 8 * 128, 8 * 128, 128]
    for key, val in kw.items():
        if key.endswith("_stride"):
            getattr(n, key)[:] = val
        else:
            setattr(n, key, val)
    return n


BAD_APPEND = [
    ("no cache_seqlens", dict(), dict(), ex.EXATTN_E_INVALID),
    ("negative seqlen_new", dict(cache_seqlens=FAKE), dict(seqlen_new=-1), ex.EXATTN_E_INVALID),
    ("longer than the cache", dict(cache_seqlens=FAKE, seqlen_cache=1), dict(), ex.EXATTN_E_INVALID),
    ("null k_new", dict(cache_seqlens=FAKE), dict(k_new=None), ex.EXATTN_E_INVALID),
    ("misaligned v_new", dict(cache_seqlens=FAKE), dict(v_new=FAKE + 8), ex.EXATTN_E_INVALID),
    ("odd stride", dict(cache_seqlens=FAKE), dict(k_new_stride=[2048, 1028, 128]), ex.EXATTN_E_INVALID),
    ("bad decode args", dict(cache_seqlens=FAKE, head_dim=80), dict(), ex.EXATTN_E_UNSUPPORTED),
]


@pytest.mark.parametrize("name,dkw,nkw,status", BAD_APPEND, ids=[c[0] for c in BAD_APPEND])
def test_decode_append_rejects(L, name, dkw, nkw, status):
    a, n = _dec(**dkw), _kvn(**nkw)
    assert L.exattn_decode_append(C.byref(a), C.byref(n), C.c_void_p(FAKE), 1 << 30, None) == status, \
        L.exattn_last_error()


def test_decode_append_null_and_empty(L):
    a = _dec(cache_seqlens=FAKE)
    assert L.exattn_decode_append(C.byref(a), None, None, 0, None) == ex.EXATTN_E_INVALID
    # nothing to attend: batch 0 launches nothing, whatever kv_new holds
    assert L.exattn_decode_append(C.byref(_dec(batch=0)), C.byref(_kvn(seqlen_new=3)), None, 0,
                                  None) == ex.EXATTN_OK


def _pg(**kw):
    g = ex.PagedKv()
    g.block_table = FAKE
    g.block_table_stride = 64
    g.page_size, g.num_pages = 256, 1000
    g.k_page_stride = g.v_page_stride = 256 * 8 * 128
    for key, val in kw.items():
        setattr(g, key, val)
    return g


BAD_PAGED = [
    ("zero page size", dict(page_size=0), ex.EXATTN_E_INVALID),
    ("page size not a step multiple", dict(page_size=24), ex.EXATTN_E_UNSUPPORTED),
    ("null block table", dict(block_table=None), ex.EXATTN_E_INVALID),
    ("short block table rows", dict(block_table_stride=63), ex.EXATTN_E_INVALID),
    ("no pages", dict(num_pages=0), ex.EXATTN_E_INVALID),
    ("odd page stride", dict(k_page_stride=256 * 8 * 128 + 4), ex.EXATTN_E_INVALID),
]


@pytest.mark.parametrize("name,kw,status", BAD_PAGED, ids=[c[0] for c in BAD_PAGED])
def test_decode_paged_rejects(L, name, kw, status):
    a = _dec(cache_seqlens=FAKE)  # 16384 tokens per sequence: 64 pages of 256
    assert L.exattn_decode_paged(C.byref(a), C.byref(_pg(**kw)), None, C.c_void_p(FAKE), 1 << 30,
                                 None) == status, L.exattn_last_error()


def test_decode_paged_null(L):
    a = _dec(cache_seqlens=FAKE)
    assert L.exattn_decode_paged(C.byref(a), None, None, None, 0, None) == ex.EXATTN_E_INVALID


def test_decode_workspace_checks(L):
    a = _dec(num_splits=4)
    ns, wb = C.c_int32(0), C.c_size_t(0)
    assert L.exattn_decode_plan(C.byref(a), C.byref(ns), C.byref(wb)) == ex.EXATTN_OK
    assert ns.value == 4
    rows = 4 * 8 * 32
    o_bytes = rows * 128 * 4
    assert wb.value == ((o_bytes + 255) // 256 * 256 + rows * 4 + 255) // 256 * 256
    assert L.exattn_decode(C.byref(a), None, 0, None) == ex.EXATTN_E_WORKSPACE
    assert L.exattn_decode(C.byref(a), C.c_void_p(FAKE), wb.value - 1, None) == ex.EXATTN_E_WORKSPACE
    assert L.exattn_decode(C.byref(a), C.c_void_p(FAKE + 16), wb.value, None) == ex.EXATTN_E_WORKSPACE
    # one split needs no workspace
    a1 = _dec(num_splits=1)
    assert L.exattn_decode_plan(C.byref(a1), C.byref(ns), C.byref(wb)) == ex.EXATTN_OK
    assert ns.value == 1 and wb.value == 0
    # more splits than 32-key chunks are clamped
    a2 = _dec(num_splits=200, seqlen_cache=100)
    assert L.exattn_decode_plan(C.byref(a2), C.byref(ns), C.byref(wb)) == ex.EXATTN_OK
    assert ns.value == 4
    assert L.exattn_decode(C.byref(_dec(batch=0)), None, 0, None) == ex.EXATTN_OK


def _f8(**kw):
    a = _fwd(dtype=ex.EXATTN_FP8_E4M3)
    for n in ("q_stride", "k_stride", "v_stride"):
        getattr(a, n)[:] = [64 * 4 * 128, 4 * 128, 128]
    for key, val in kw.items():
        if key.endswith("_stride"):
            getattr(a, key)[:] = val
        else:
            setattr(a, key, val)
    return a


BAD_FP8 = [
    ("dtype bf16", dict(dtype=1), None, ex.EXATTN_E_UNSUPPORTED),
    ("head_dim 256", dict(head_dim=256), None, ex.EXATTN_E_UNSUPPORTED),
    ("nan softcap", dict(softcap=float("nan")), None, ex.EXATTN_E_INVALID),
    ("varlen half", dict(cu_seqlens_q=FAKE), None, ex.EXATTN_E_INVALID),
    ("varlen negative max", dict(cu_seqlens_q=FAKE, cu_seqlens_k=FAKE, max_seqlen_q=-1), None,
     ex.EXATTN_E_INVALID),
    ("stride not 16", dict(k_stride=[64 * 4 * 128, 4 * 128 + 8, 128]), None, ex.EXATTN_E_INVALID),
    ("odd o stride", dict(o_stride=[64 * 4 * 128, 4 * 128 + 4, 128]), None, ex.EXATTN_E_INVALID),
    ("null q", dict(q=None), None, ex.EXATTN_E_INVALID),
    ("misaligned v", dict(v=FAKE + 8), None, ex.EXATTN_E_INVALID),
    ("heads ratio", dict(heads_q=3), None, ex.EXATTN_E_INVALID),
    ("nan descale", dict(), (1.0, float("nan"), 1.0), ex.EXATTN_E_INVALID),
    ("inf descale", dict(), (1.0, 1.0, float("inf")), ex.EXATTN_E_INVALID),
    ("token stride past 32-bit tile offsets", dict(v_stride=[1 << 40, 1 << 26, 128]), None,
     ex.EXATTN_E_UNSUPPORTED),
]


@pytest.mark.parametrize("name,kw,ds,status", BAD_FP8, ids=[c[0] for c in BAD_FP8])
def test_fp8_rejects(L, name, kw, ds, status):
    d = ex.Fp8Descale(*ds) if ds is not None else None
    st = L.exattn_fwd_fp8(C.byref(_f8(**kw)), C.byref(d) if d is not None else None, None)
    assert st == status, (name, st, L.exattn_last_error())
    assert L.exattn_last_error()


def test_fp8_empty_and_fwd_refuses_fp8(L):
    assert L.exattn_fwd_fp8(C.byref(_f8(batch=0, q=None, o=None)), None, None) == ex.EXATTN_OK
    assert L.exattn_fwd_fp8(C.byref(_f8(seqlen_q=0)), None, None) == ex.EXATTN_OK
    # softcap and packed sequences are provided: with nothing to compute the calls pass every
    # check and launch nothing
    assert L.exattn_fwd_fp8(C.byref(_f8(seqlen_q=0, softcap=30.0)), None, None) == ex.EXATTN_OK
    assert L.exattn_fwd_fp8(C.byref(_f8(cu_seqlens_q=FAKE, cu_seqlens_k=FAKE, max_seqlen_q=0, max_seqlen_k=9)),
                            None, None) == ex.EXATTN_OK
    assert L.exattn_fwd_fp8(None, None, None) == ex.EXATTN_E_INVALID
    assert L.exattn_fwd(C.byref(_f8()), None) == ex.EXATTN_E_UNSUPPORTED  # the 16-bit path takes no FP8


def _bwd(**kw):
    a = ex.BwdArgs()
    a.dtype, a.batch, a.seqlen_q, a.seqlen_k = 1, 2, 64, 96
    a.heads_q, a.heads_kv, a.head_dim = 4, 2, 128
    a.q = a.k = a.v = a.o = a.dout = a.lse = a.dq = a.dk = a.dv = FAKE
    for n in ("q", "o", "dout", "dq"):
        getattr(a, n + "_stride")[:] = [64 * 4 * 128, 4 * 128, 128]
    for n in ("k", "v", "dk", "dv"):
        getattr(a, n + "_stride")[:] = [96 * 2 * 128, 2 * 128, 128]
    a.lse_stride[:] = [4 * 64, 64]
    a.window_left = a.window_right = -1
    for key, val in kw.items():
        if key.endswith("_stride"):
            getattr(a, key)[:] = val
        else:
            setattr(a, key, val)
    return a


BAD_BWD = [
    ("dtype", dict(dtype=3), ex.EXATTN_E_UNSUPPORTED),
    ("head_dim 80", dict(head_dim=80), ex.EXATTN_E_UNSUPPORTED),
    ("heads ratio", dict(heads_q=3), ex.EXATTN_E_INVALID),
    ("half varlen", dict(cu_seqlens_q=FAKE), ex.EXATTN_E_INVALID),
    ("negative max seqlen", dict(cu_seqlens_q=FAKE, cu_seqlens_k=FAKE, max_seqlen_q=-1), ex.EXATTN_E_INVALID),
    ("negative seqlen", dict(seqlen_q=-1), ex.EXATTN_E_INVALID),
    ("null dout", dict(dout=None), ex.EXATTN_E_INVALID),
    ("null dk", dict(dk=None), ex.EXATTN_E_INVALID),
    ("null lse", dict(lse=None), ex.EXATTN_E_INVALID),
    ("misaligned dq", dict(dq=FAKE + 8), ex.EXATTN_E_INVALID),
    ("misaligned lse", dict(lse=FAKE + 2), ex.EXATTN_E_INVALID),
    ("odd stride", dict(dv_stride=[96 * 2 * 128, 2 * 128 + 2, 128]), ex.EXATTN_E_INVALID),
    ("negative lse stride", dict(lse_stride=[-64, 64]), ex.EXATTN_E_INVALID),
    ("inf scale", dict(softmax_scale=float("inf")), ex.EXATTN_E_INVALID),
    ("token stride past 32-bit tile offsets", dict(dout_stride=[1 << 40, 1 << 25, 128]),
     ex.EXATTN_E_UNSUPPORTED),
]


@pytest.mark.parametrize("name,kw,status", BAD_BWD, ids=[c[0] for c in BAD_BWD])
def test_bwd_rejects(L, name, kw, status):
    a = _bwd(**kw)
    assert L.exattn_bwd_plan(C.byref(a), None) == status, (name, L.exattn_last_error())
    assert L.exattn_bwd(C.byref(a), C.c_void_p(FAKE), 1 << 30, None) == status, L.exattn_last_error()
    assert L.exattn_last_error()


def test_bwd_workspace_and_empty(L):
    a = _bwd()
    wb = C.c_size_t(0)
    assert L.exattn_bwd_plan(C.byref(a), C.byref(wb)) == ex.EXATTN_OK
    rows = 2 * 4 * 64
    assert wb.value == (rows * 8 + 255) // 256 * 256
    assert L.exattn_bwd(C.byref(a), None, 0, None) == ex.EXATTN_E_WORKSPACE
    assert L.exattn_bwd(C.byref(a), C.c_void_p(FAKE), wb.value - 1, None) == ex.EXATTN_E_WORKSPACE
    assert L.exattn_bwd(C.byref(a), C.c_void_p(FAKE + 16), wb.value, None) == ex.EXATTN_E_WORKSPACE
    assert L.exattn_bwd(None, None, 0, None) == ex.EXATTN_E_INVALID
    assert L.exattn_bwd_plan(None, None) == ex.EXATTN_E_INVALID
    # nothing to compute: no launch, no pointer needed
    assert L.exattn_bwd(C.byref(_bwd(batch=0, q=None, dq=None)), None, 0, None) == ex.EXATTN_OK
    assert L.exattn_bwd(C.byref(_bwd(seqlen_q=0, seqlen_k=0, q=None, k=None)), None, 0, None) == ex.EXATTN_OK
    # no query rows: no workspace, and q, o, dout, dq, lse may be NULL
    z = _bwd(seqlen_q=0, q=None, o=None, dout=None, dq=None, lse=None)
    assert L.exattn_bwd_plan(C.byref(z), C.byref(wb)) == ex.EXATTN_OK and wb.value == 0


def test_auto_splits_rules(L):
    # FAQ Q14: enough (batch x heads) work -> 1 split; few units -> split toward the CU count;
    # a split never gets fewer than 256 keys.  A work group covers 8 adjacent KV heads at
    # d = 128, 16 at d = 64, 4 at d = 256, and one work group runs per CU.
    assert ex.auto_splits(8, 32, 8, 16384, 128, 256) == 32      # 8 units -> 256 work groups
    assert ex.auto_splits(8, 32, 8, 16384, 64, 256) == 32       # 8 KV heads make one unit too
    assert ex.auto_splits(8, 32, 8, 16384, 256, 256) == 16      # 16 units
    assert ex.auto_splits(256, 32, 8, 16384, 128, 256) == 1     # 256 units already
    assert ex.auto_splits(64, 32, 8, 16384, 128, 256) == 4      # 64 units
    assert ex.auto_splits(1, 32, 8, 16384, 128, 256) == 64      # 1 unit -> capped at length / 256
    assert ex.auto_splits(1, 32, 8, 1024, 128, 256) == 4        # capped by length / 256
    assert ex.auto_splits(1, 32, 8, 100, 128, 256) == 1
    assert ex.auto_splits(1, 8, 8, 0, 128, 256) == 1
    assert ex.auto_splits(2, 64, 1, 1 << 20, 128, 256) == 32    # one KV head, 4 groups of 16 queries
    assert ex.auto_splits(2, 6, 3, 1 << 20, 64, 256) == 64      # 3 KV heads -> 2 per work group


def test_head_major_decode_cache_within_offsets_is_accepted(L):
    """A head-major cache (b, h, s, d) whose 8-head tile stays below 2^31 bytes plans fine."""
    a = _dec(k_stride=[8 * 16384 * 128, 128, 16384 * 128], v_stride=[8 * 16384 * 128, 128, 16384 * 128])
    assert L.exattn_decode_plan(C.byref(a), None, None) == ex.EXATTN_OK, L.exattn_last_error()


def test_fwd_pack_gqa_values_accepted(L):
    for v in (-1, 0, 1):
        assert L.exattn_fwd(C.byref(_fwd(pack_gqa=v, batch=0)), None) == ex.EXATTN_OK


# --------------------------------------------------------------------------
# the binding's own checks of caller-supplied outputs (before any device use)
# --------------------------------------------------------------------------
def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.float16)


def test_binding_rejects_mismatched_out_and_lse():
    import torch
    q = _t(1, 8, 2, 64)
    with pytest.raises(ValueError, match="out must be"):
        ex.attn_func(q, q, q, out=_t(1, 8, 2, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must be"):
        ex.attn_func(q, q, q, out=_t(1, 8, 2, 32))
    with pytest.raises(ValueError, match="contiguous last dimension"):
        ex.attn_func(q, q, q, out=_t(1, 8, 2, 128)[..., ::2])
    with pytest.raises(ValueError, match="lse must be"):
        ex.attn_func(q, q, q, lse=_t(1, 2, 8))  # fp16, not fp32
    with pytest.raises(ValueError, match="lse must be"):
        ex.attn_func(q, q, q, lse=_t(1, 8, 2, dtype=torch.float32))  # (b, s, h) instead of (b, h, s)
    with pytest.raises(ValueError, match="contiguous last dimension"):
        ex.attn_func(q, q, q, lse=_t(1, 2, 16, dtype=torch.float32)[..., ::2])


def test_binding_varlen_checks():
    import torch
    q, k = _t(10, 4, 64), _t(12, 2, 64)
    cu = torch.tensor([0, 10], dtype=torch.int32)
    cuk = torch.tensor([0, 12], dtype=torch.int32)
    with pytest.raises(ValueError, match="shape mismatch"):
        ex.attn_varlen_func(q, k, _t(12, 2, 32), cu, cuk, 10, 12)
    with pytest.raises(ValueError, match="shape mismatch"):
        ex.attn_varlen_func(q, _t(12, 2, 128), _t(12, 2, 128), cu, cuk, 10, 12)
    with pytest.raises(ValueError, match="one dtype"):
        ex.attn_varlen_func(q, k, _t(12, 2, 64, dtype=torch.bfloat16), cu, cuk, 10, 12)
    with pytest.raises(ValueError, match="out must be"):
        ex.attn_varlen_func(q, k, k, cu, cuk, 10, 12, out=_t(10, 4, 32))
    with pytest.raises(ValueError, match="lse must be"):
        ex.attn_varlen_func(q, k, k, cu, cuk, 10, 12, lse=_t(10, 4, dtype=torch.float32))


def test_binding_kvcache_checks():
    import torch
    q, kc = _t(2, 1, 8, 128), _t(2, 100, 2, 128)
    with pytest.raises(ValueError, match="out must be"):
        ex.attn_with_kvcache(q, kc, kc, out=_t(2, 1, 8, 64))
    with pytest.raises(ValueError, match="lse must be contiguous"):
        ex.attn_with_kvcache(q, kc, kc, lse=_t(2, 16, 1, dtype=torch.float32)[:, ::2])
    with pytest.raises(ValueError, match="lse must be"):
        ex.attn_with_kvcache(q, kc, kc, lse=_t(2, 8, dtype=torch.float32))


def test_decode_plan_counts_query_tokens(L):
    """Several query tokens: the workspace holds partials for every (split, batch, token, head)."""
    a = _dec(num_splits=4, seqlen_q=3, q_token_stride=32 * 128, o_token_stride=32 * 128)
    ns, wb = C.c_int32(0), C.c_size_t(0)
    assert L.exattn_decode_plan(C.byref(a), C.byref(ns), C.byref(wb)) == ex.EXATTN_OK, L.exattn_last_error()
    rows = 4 * 8 * 3 * 32
    assert wb.value == ((rows * 128 * 4 + 255) // 256 * 256 + rows * 4 + 255) // 256 * 256
    # 0 query tokens is taken as 1
    a1 = _dec(num_splits=4, seqlen_q=0)
    assert L.exattn_decode_plan(C.byref(a1), C.byref(ns), C.byref(wb)) == ex.EXATTN_OK
    assert wb.value == ((4 * 8 * 32 * 128 * 4 + 255) // 256 * 256 + 4 * 8 * 32 * 4 + 255) // 256 * 256


def test_bwd_accepts_softcap_and_varlen_plans(L):
    """Softcap, packed sequences and head_dim 256 are provided: their plans succeed; the
    varlen workspace is sized by the longest sequence."""
    wb = C.c_size_t(0)
    d256 = _bwd(head_dim=256)
    for name in ("q", "k", "v", "o", "dout", "dq", "dk", "dv"):
        st = getattr(d256, f"{name}_stride")
        st[:] = [st[0] * 2, st[1] * 2, st[2] * 2]
    assert L.exattn_bwd_plan(C.byref(d256), C.byref(wb)) == ex.EXATTN_OK, L.exattn_last_error()
    assert L.exattn_bwd_plan(C.byref(_bwd(softcap=30.0)), C.byref(wb)) == ex.EXATTN_OK, L.exattn_last_error()
    a = _bwd(cu_seqlens_q=FAKE, cu_seqlens_k=FAKE, max_seqlen_q=77, max_seqlen_k=300)
    assert L.exattn_bwd_plan(C.byref(a), C.byref(wb)) == ex.EXATTN_OK, L.exattn_last_error()
    assert wb.value == (2 * 4 * 77 * 8 + 255) // 256 * 256
