"""exattn_decode_noalloc (the decode without a caller workspace, for callers that
cannot allocate) against exattn_decode through the C ABI: two calls in a row on
the shared static scratch, the second smaller, each bitwise equal to the
workspace entry point with the same split count and within the FAQ Q10
tolerances of the oracle."""
import ctypes as C

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
    ex.lib()


def _noalloc(q, kc, vc, lens, num_splits):
    b, _, h_q, d = q.shape
    out = torch.full_like(q, float("nan"))
    lse = torch.full((b, h_q, 1), 123.0, dtype=torch.float32, device=DEV)
    a = ex._decode_args(q[:, 0], kc, vc, out[:, 0], lse, lens, None, False, (-1, -1), 0.0, num_splits)
    st = ex.lib().exattn_decode_noalloc(C.byref(a), C.c_void_p(torch.cuda.current_stream().cuda_stream))
    ex._raise_for(st, "exattn_decode_noalloc")
    return out, lse


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_workspace_decode(order):
    cases = [  # b, s_cache, h_q, h_kv, d, lens, splits, seed
        (8, 16384, 32, 8, 128, [16384] * 8, 0, 500),         # the long-cache decode: 32 splits, 4.2 MB
        (3, 1000, 16, 4, 64, [1000, 1, 517], 3, 501),         # smaller, on the same scratch
    ]
    for b, s_cache, hq, hkv, d, lens, splits, seed in cases:
        q, kc, vc = W.kvcache(b, s_cache, hq, hkv, d, seed=seed)
        lens_t = torch.tensor(lens, dtype=torch.int32)
        dq, dkc, dvc, dl = (t.to(DEV) for t in (q, kc, vc, lens_t))
        ns, wb = ex.decode_plan(dq[:, 0], dkc, dvc, dl, num_splits=splits)
        assert ns > 1 and wb <= 8 << 20
        o_ws, l_ws = ex.attn_with_kvcache(dq, dkc, dvc, cache_seqlens=dl, num_splits=ns)
        o_na, l_na = _noalloc(dq, dkc, dvc, dl, ns)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), f"case {seed}"
        o_ref, l_ref = oracle.attention_kvcache(q, kc, vc, lens_t)
        assert_o_close(o_na, o_ref, q.dtype, f"noalloc {seed}")
        assert_lse_close(l_na, l_ref, f"noalloc {seed}")


def test_noalloc_rejects_plans_beyond_the_scratch():
    q, kc, vc = W.kvcache(16, 2048, 32, 8, 128, seed=502)
    dq, dkc, dvc = (t.to(DEV) for t in (q, kc, vc))
    ns, wb = ex.decode_plan(dq[:, 0], dkc, dvc, num_splits=64)
    assert wb > 8 << 20
    with pytest.raises(ValueError, match="static scratch"):
        _noalloc(dq, dkc, dvc, None, 64)
