"""exact_attention_43_amd: exact attention forward on AMD MI355X (gfx950).

A thin Python binding over the C ABI of ``libexattn.so`` (declared in
``include/exattn.h``).  PyTorch supplies device memory and the current stream;
every step of the attention itself runs in the library's HIP kernels.  There
is no CPU or PyTorch fallback: if the library is not built, or a tensor is not
on a GPU, the call raises.

Entry points, named after the calls the pages show (Inference Cookbook FAQ Q2,
Q7, Q8, Q17; "FlashAttention完整说明" section 六.1), all forward only:

- ``attn_func(q, k, v, ...)``: q (b, s_q, h_q, d), k/v (b, s_k, h_kv, d)
- ``attn_qkvpacked_func(qkv, ...)``: qkv (b, s, 3, h, d)
- ``attn_kvpacked_func(q, kv, ...)``: kv (b, s_k, 2, h_kv, d)
- ``attn_varlen_func(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, ...)``
- ``attn_with_kvcache(q, k_cache, v_cache, cache_seqlens=None, ..., num_splits=0)``

Each returns ``(out, lse)``: out in the layout of q, lse fp32 (b, h_q, s_q)
(varlen: (h_q, total_q); decode: (b, h_q, 1)).
"""
from __future__ import annotations

import ctypes as C
import os
import threading

import torch

__version__ = "0.1.0"

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libexattn.so")

EXATTN_OK, EXATTN_E_INVALID, EXATTN_E_UNSUPPORTED, EXATTN_E_WORKSPACE, EXATTN_E_HIP = range(5)
EXATTN_F16, EXATTN_BF16, EXATTN_FP8_E4M3 = 0, 1, 2


class Fp8Descale(C.Structure):
    """Mirror of exattn_fp8_descale."""
    _fields_ = [("q", C.c_float), ("k", C.c_float), ("v", C.c_float)]


class FwdArgs(C.Structure):
    """Mirror of exattn_fwd_args."""
    _fields_ = [
        ("dtype", C.c_int32), ("batch", C.c_int32), ("seqlen_q", C.c_int32), ("seqlen_k", C.c_int32),
        ("heads_q", C.c_int32), ("heads_kv", C.c_int32), ("head_dim", C.c_int32),
        ("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p), ("o", C.c_void_p),
        ("lse", C.c_void_p),
        ("q_stride", C.c_int64 * 3), ("k_stride", C.c_int64 * 3), ("v_stride", C.c_int64 * 3),
        ("o_stride", C.c_int64 * 3), ("lse_stride", C.c_int64 * 2),
        ("cu_seqlens_q", C.c_void_p), ("cu_seqlens_k", C.c_void_p),
        ("max_seqlen_q", C.c_int32), ("max_seqlen_k", C.c_int32),
        ("softmax_scale", C.c_float), ("softcap", C.c_float),
        ("causal", C.c_int32), ("window_left", C.c_int32), ("window_right", C.c_int32),
        ("pack_gqa", C.c_int32),
    ]


class DecodeArgs(C.Structure):
    """Mirror of exattn_decode_args."""
    _fields_ = [
        ("dtype", C.c_int32), ("batch", C.c_int32), ("heads_q", C.c_int32), ("heads_kv", C.c_int32),
        ("head_dim", C.c_int32), ("seqlen_cache", C.c_int32),
        ("q", C.c_void_p), ("k_cache", C.c_void_p), ("v_cache", C.c_void_p), ("o", C.c_void_p),
        ("lse", C.c_void_p),
        ("q_stride", C.c_int64 * 2), ("o_stride", C.c_int64 * 2),
        ("k_stride", C.c_int64 * 3), ("v_stride", C.c_int64 * 3),
        ("cache_seqlens", C.c_void_p),
        ("softmax_scale", C.c_float), ("softcap", C.c_float),
        ("causal", C.c_int32), ("window_left", C.c_int32), ("window_right", C.c_int32),
        ("num_splits", C.c_int32), ("seqlen_q", C.c_int32),
        ("q_token_stride", C.c_int64), ("o_token_stride", C.c_int64),
    ]


class KvNew(C.Structure):
    """Mirror of exattn_kv_new."""
    _fields_ = [
        ("k_new", C.c_void_p), ("v_new", C.c_void_p), ("seqlen_new", C.c_int32),
        ("k_new_stride", C.c_int64 * 3), ("v_new_stride", C.c_int64 * 3),
    ]


class PagedKv(C.Structure):
    """Mirror of exattn_paged_kv."""
    _fields_ = [
        ("block_table", C.c_void_p), ("block_table_stride", C.c_int32), ("page_size", C.c_int32),
        ("num_pages", C.c_int32), ("k_page_stride", C.c_int64), ("v_page_stride", C.c_int64),
    ]


class BwdArgs(C.Structure):
    """Mirror of exattn_bwd_args."""
    _fields_ = [
        ("dtype", C.c_int32), ("batch", C.c_int32), ("seqlen_q", C.c_int32), ("seqlen_k", C.c_int32),
        ("heads_q", C.c_int32), ("heads_kv", C.c_int32), ("head_dim", C.c_int32),
        ("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p), ("o", C.c_void_p), ("dout", C.c_void_p),
        ("lse", C.c_void_p), ("dq", C.c_void_p), ("dk", C.c_void_p), ("dv", C.c_void_p),
        ("q_stride", C.c_int64 * 3), ("k_stride", C.c_int64 * 3), ("v_stride", C.c_int64 * 3),
        ("o_stride", C.c_int64 * 3), ("dout_stride", C.c_int64 * 3), ("dq_stride", C.c_int64 * 3),
        ("dk_stride", C.c_int64 * 3), ("dv_stride", C.c_int64 * 3), ("lse_stride", C.c_int64 * 2),
        ("softmax_scale", C.c_float), ("softcap", C.c_float), ("causal", C.c_int32),
        ("window_left", C.c_int32), ("window_right", C.c_int32),
        ("cu_seqlens_q", C.c_void_p), ("cu_seqlens_k", C.c_void_p),
        ("max_seqlen_q", C.c_int32), ("max_seqlen_k", C.c_int32),
    ]


_lib_handle = None
_lib_lock = threading.Lock()


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libexattn.so (once).  Raises if it has not been built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    with _lib_lock:
        if _lib_handle is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(
                    f"{_LIB_PATH} is missing: build it with `python -m exact_attention_43_amd.build`")
            L = C.CDLL(_LIB_PATH)
            L.exattn_fwd.argtypes = [C.POINTER(FwdArgs), C.c_void_p]
            L.exattn_fwd.restype = C.c_int
            L.exattn_decode_plan.argtypes = [C.POINTER(DecodeArgs), C.POINTER(C.c_int32),
                                             C.POINTER(C.c_size_t)]
            L.exattn_decode_plan.restype = C.c_int
            L.exattn_decode.argtypes = [C.POINTER(DecodeArgs), C.c_void_p, C.c_size_t, C.c_void_p]
            L.exattn_decode.restype = C.c_int
            L.exattn_decode_noalloc.argtypes = [C.POINTER(DecodeArgs), C.c_void_p]
            L.exattn_decode_noalloc.restype = C.c_int
            L.exattn_decode_append.argtypes = [C.POINTER(DecodeArgs), C.POINTER(KvNew), C.c_void_p,
                                               C.c_size_t, C.c_void_p]
            L.exattn_decode_append.restype = C.c_int
            L.exattn_decode_paged.argtypes = [C.POINTER(DecodeArgs), C.POINTER(PagedKv), C.POINTER(KvNew),
                                              C.c_void_p, C.c_size_t, C.c_void_p]
            L.exattn_decode_paged.restype = C.c_int
            L.exattn_fwd_fp8.argtypes = [C.POINTER(FwdArgs), C.POINTER(Fp8Descale), C.c_void_p]
            L.exattn_fwd_fp8.restype = C.c_int
            L.exattn_bwd_plan.argtypes = [C.POINTER(BwdArgs), C.POINTER(C.c_size_t)]
            L.exattn_bwd_plan.restype = C.c_int
            L.exattn_bwd.argtypes = [C.POINTER(BwdArgs), C.c_void_p, C.c_size_t, C.c_void_p]
            L.exattn_bwd.restype = C.c_int
            L.exattn_decode_auto_splits.argtypes = [C.c_int32] * 6
            L.exattn_decode_auto_splits.restype = C.c_int32
            L.exattn_args_size.argtypes = [C.c_int32]
            L.exattn_args_size.restype = C.c_size_t
            L.exattn_status_string.argtypes = [C.c_int32]
            L.exattn_status_string.restype = C.c_char_p
            L.exattn_last_error.argtypes = []
            L.exattn_last_error.restype = C.c_char_p
            L.exattn_abi_version.argtypes = []
            L.exattn_abi_version.restype = C.c_int32
            if (L.exattn_args_size(0) != C.sizeof(FwdArgs) or L.exattn_args_size(1) != C.sizeof(DecodeArgs)
                    or L.exattn_args_size(2) != C.sizeof(KvNew) or L.exattn_args_size(3) != C.sizeof(PagedKv)
                    or L.exattn_args_size(4) != C.sizeof(BwdArgs)
                    or L.exattn_args_size(5) != C.sizeof(Fp8Descale)):
                raise RuntimeError("libexattn.so struct layout does not match this binding; rebuild it")
            _lib_handle = L
    return _lib_handle


def _raise_for(status: int, what: str):
    if status == EXATTN_OK:
        return
    L = lib()
    msg = f"{what}: {L.exattn_status_string(status).decode()}: {L.exattn_last_error().decode()}"
    if status == EXATTN_E_UNSUPPORTED:
        raise NotImplementedError(msg)
    if status in (EXATTN_E_INVALID, EXATTN_E_WORKSPACE):
        raise ValueError(msg)
    raise RuntimeError(msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return EXATTN_F16
    if t.dtype == torch.bfloat16:
        return EXATTN_BF16
    raise NotImplementedError(f"dtype {t.dtype} is not supported: use float16 or bfloat16")


def _on_gpu(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("exattn tensors must be on a GPU (there is no CPU path)")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def _check_last_dim(*ts):
    for t in ts:
        if t is not None and t.stride(-1) != 1:
            raise ValueError("the head_dim axis must be contiguous (stride 1)")


def _check_dropout(dropout_p):
    if dropout_p not in (0, 0.0, None):
        raise NotImplementedError("dropout is not supported by the forward (dropout_p must be 0)")


def _scale(softmax_scale):
    """None selects the library default 1/sqrt(head_dim) (passed as NaN); any other value as given."""
    return float("nan") if softmax_scale is None else float(softmax_scale)


def _pack(pack_gqa):
    """None: automatic (-1); True / False: on / off."""
    if pack_gqa is None:
        return -1
    return 1 if pack_gqa else 0


def _check_out(out, shape, dtype, what="out"):
    """A caller-supplied output must match what the kernel writes: dtype, shape and a
    contiguous last dimension."""
    if out is None:
        return
    if out.dtype != dtype or tuple(out.shape) != tuple(shape):
        raise ValueError(f"{what} must be {dtype} of shape {tuple(shape)}, got {out.dtype} {tuple(out.shape)}")
    if out.stride(-1) != 1:
        raise ValueError(f"{what} must have a contiguous last dimension")


def _check_lse(lse, shape, contiguous=False):
    if lse is None:
        return
    if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(shape):
        raise ValueError(f"lse must be float32 of shape {tuple(shape)}, got {lse.dtype} {tuple(lse.shape)}")
    if lse.stride(-1) != 1 or (contiguous and not lse.is_contiguous()):
        raise ValueError("lse must be contiguous" if contiguous else "lse must have a contiguous last dimension")


def _window(window_size):
    wl, wr = window_size
    return int(wl), int(wr)


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _fwd_call(q, k, v, out, lse, *, batch, s_q, s_k, h_q, h_kv, d, q_st, k_st, v_st, o_st, lse_st,
              cu_q=None, cu_k=None, max_q=0, max_k=0, softmax_scale=None, causal=False,
              window_size=(-1, -1), softcap=0.0, pack_gqa=None):
    a = FwdArgs()
    a.dtype = _dtype_code(q)
    a.batch, a.seqlen_q, a.seqlen_k = batch, s_q, s_k
    a.heads_q, a.heads_kv, a.head_dim = h_q, h_kv, d
    a.q, a.k, a.v, a.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()
    a.lse = lse.data_ptr() if lse is not None else None
    for name, st in (("q_stride", q_st), ("k_stride", k_st), ("v_stride", v_st), ("o_stride", o_st)):
        getattr(a, name)[:] = list(st)
    a.lse_stride[:] = list(lse_st)
    a.cu_seqlens_q = cu_q.data_ptr() if cu_q is not None else None
    a.cu_seqlens_k = cu_k.data_ptr() if cu_k is not None else None
    a.max_seqlen_q, a.max_seqlen_k = int(max_q), int(max_k)
    a.softmax_scale = _scale(softmax_scale)
    a.softcap = float(softcap or 0.0)
    a.causal = 1 if causal else 0
    a.window_left, a.window_right = _window(window_size)
    a.pack_gqa = _pack(pack_gqa)
    with torch.cuda.device(q.device):
        st = lib().exattn_fwd(C.byref(a), C.c_void_p(_stream(q.device)))
    _raise_for(st, "exattn_fwd")


def attn_func(q, k, v, dropout_p=0.0, softmax_scale=None, causal=False, window_size=(-1, -1),
              softcap=0.0, out=None, lse=None, pack_gqa=None):
    """Dense forward.  q (b, s_q, h_q, d); k, v (b, s_k, h_kv, d); returns (out, lse).

    ``pack_gqa`` (FAQ Q15): None = automatic, True = one tile holds the rows of all
    query heads of a KV head, False = one tile per query head; the result is the same.
    """
    _check_dropout(dropout_p)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D (batch, seqlen, heads, head_dim)")
    b, s_q, h_q, d = q.shape
    s_k, h_kv = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != b or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    _check_out(out, (b, s_q, h_q, d), q.dtype)
    _check_lse(lse, (b, h_q, s_q))
    _on_gpu(q, k, v, out, lse)
    _check_last_dim(q, k, v)
    if out is None:
        out = torch.empty((b, s_q, h_q, d), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((b, h_q, s_q), dtype=torch.float32, device=q.device)
    _fwd_call(q, k, v, out, lse, batch=b, s_q=s_q, s_k=s_k, h_q=h_q, h_kv=h_kv, d=d,
              q_st=q.stride()[:3], k_st=k.stride()[:3], v_st=v.stride()[:3], o_st=out.stride()[:3],
              lse_st=(lse.stride(0), lse.stride(1)), softmax_scale=softmax_scale, causal=causal,
              window_size=window_size, softcap=softcap, pack_gqa=pack_gqa)
    return out, lse


def _fp8_call(q, k, v, out, lse, *, batch, s_q, s_k, h_q, h_kv, d, q_st, k_st, v_st, o_st, lse_st, descales,
              softmax_scale, causal, window_size, softcap, cu_q=None, cu_k=None, max_q=0, max_k=0):
    a = FwdArgs()
    a.dtype = EXATTN_FP8_E4M3
    a.batch, a.seqlen_q, a.seqlen_k, a.heads_q, a.heads_kv, a.head_dim = batch, s_q, s_k, h_q, h_kv, d
    a.q, a.k, a.v, a.o, a.lse = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr()
    a.q_stride[:] = list(q_st)
    a.k_stride[:] = list(k_st)
    a.v_stride[:] = list(v_st)
    a.o_stride[:] = list(o_st)
    a.lse_stride[:] = list(lse_st)
    if cu_q is not None:
        a.cu_seqlens_q, a.cu_seqlens_k = cu_q.data_ptr(), cu_k.data_ptr()
        a.max_seqlen_q, a.max_seqlen_k = int(max_q), int(max_k)
    a.softmax_scale = _scale(softmax_scale)
    a.softcap = float(softcap or 0.0)
    a.causal = 1 if causal else 0
    a.window_left, a.window_right = _window(window_size)
    ds = Fp8Descale(*(float(x) for x in descales))
    with torch.cuda.device(q.device):
        st = lib().exattn_fwd_fp8(C.byref(a), C.byref(ds), C.c_void_p(_stream(q.device)))
    _raise_for(st, "exattn_fwd_fp8")


def attn_func_fp8(q, k, v, q_descale=1.0, k_descale=1.0, v_descale=1.0, softmax_scale=None, causal=False,
                  window_size=(-1, -1), softcap=0.0, out=None, lse=None):
    """FP8 forward with a bf16 output (FAQ Q20).  q (b, s_q, h_q, d), k, v (b, s_k, h_kv, d) as
    torch.float8_e4m3fn; the real inputs are the values times the descale factors.  Returns
    (out bf16 (b, s_q, h_q, d), lse fp32 (b, h_q, s_q)).  head_dim 64 or 128; softcap as for
    attn_func (applied to the scaled real scores)."""
    _on_gpu(q, k, v, out, lse)
    _check_last_dim(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D (batch, seqlen, heads, head_dim)")
    if not (q.dtype == k.dtype == v.dtype == torch.float8_e4m3fn):
        raise ValueError("q, k and v must be torch.float8_e4m3fn")
    b, s_q, h_q, d = q.shape
    s_k, h_kv = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != b or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if out is None:
        out = torch.empty((b, s_q, h_q, d), dtype=torch.bfloat16, device=q.device)
    if out.dtype != torch.bfloat16 or out.shape != (b, s_q, h_q, d):
        raise ValueError("out must be bf16 (batch, seqlen_q, heads_q, head_dim)")
    _check_last_dim(out)
    if lse is None:
        lse = torch.empty((b, h_q, s_q), dtype=torch.float32, device=q.device)
    _check_lse(lse, (b, h_q, s_q))
    _fp8_call(q, k, v, out, lse, batch=b, s_q=s_q, s_k=s_k, h_q=h_q, h_kv=h_kv, d=d, q_st=q.stride()[:3],
              k_st=k.stride()[:3], v_st=v.stride()[:3], o_st=out.stride()[:3],
              lse_st=(lse.stride(0), lse.stride(1)), descales=(q_descale, k_descale, v_descale),
              softmax_scale=softmax_scale, causal=causal, window_size=window_size, softcap=softcap)
    return out, lse


def attn_varlen_func_fp8(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, q_descale=1.0,
                         k_descale=1.0, v_descale=1.0, softmax_scale=None, causal=False, window_size=(-1, -1),
                         softcap=0.0, out=None, lse=None):
    """The FP8 forward over packed sequences (FAQ Q8, Q20): q (total_q, h_q, d), k, v
    (total_k, h_kv, d) as torch.float8_e4m3fn, int32 cu_seqlens.  Returns out bf16
    (total_q, h_q, d) and lse (h_q, total_q)."""
    _on_gpu(q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("varlen q, k, v must be 3-D (total, heads, head_dim)")
    if not (q.dtype == k.dtype == v.dtype == torch.float8_e4m3fn):
        raise ValueError("q, k and v must be torch.float8_e4m3fn")
    if k.shape != v.shape or k.shape[-1] != q.shape[-1]:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    _check_last_dim(q, k, v)
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold batch + 1 entries")
    if not (cu_seqlens_q.is_contiguous() and cu_seqlens_k.is_contiguous()):
        raise ValueError("cu_seqlens must be contiguous")
    total_q, h_q, d = q.shape
    h_kv = k.shape[1]
    if out is None:
        out = torch.empty((total_q, h_q, d), dtype=torch.bfloat16, device=q.device)
    if out.dtype != torch.bfloat16 or out.shape != (total_q, h_q, d):
        raise ValueError("out must be bf16 (total_q, heads_q, head_dim)")
    _check_last_dim(out)
    if lse is None:
        lse = torch.empty((h_q, total_q), dtype=torch.float32, device=q.device)
    _check_lse(lse, (h_q, total_q))
    _fp8_call(q, k, v, out, lse, batch=cu_seqlens_q.numel() - 1, s_q=0, s_k=0, h_q=h_q, h_kv=h_kv, d=d,
              q_st=(0, q.stride(0), q.stride(1)), k_st=(0, k.stride(0), k.stride(1)),
              v_st=(0, v.stride(0), v.stride(1)), o_st=(0, out.stride(0), out.stride(1)),
              lse_st=(0, lse.stride(0)), descales=(q_descale, k_descale, v_descale),
              softmax_scale=softmax_scale, causal=causal, window_size=window_size, softcap=softcap,
              cu_q=cu_seqlens_q, cu_k=cu_seqlens_k, max_q=max_seqlen_q, max_k=max_seqlen_k)
    return out, lse


def attn_qkvpacked_func(qkv, dropout_p=0.0, softmax_scale=None, causal=False, window_size=(-1, -1),
                        softcap=0.0, out=None, lse=None):
    """qkv (b, s, 3, h, d): passed to the kernel as three strided views, no copy."""
    if qkv.dim() != 5 or qkv.shape[2] != 3:
        raise ValueError("qkv must be (batch, seqlen, 3, heads, head_dim)")
    return attn_func(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], dropout_p, softmax_scale, causal,
                     window_size, softcap, out, lse)


def attn_kvpacked_func(q, kv, dropout_p=0.0, softmax_scale=None, causal=False, window_size=(-1, -1),
                       softcap=0.0, out=None, lse=None, pack_gqa=None):
    """kv (b, s_k, 2, h_kv, d) as stacked by torch.stack([k, v], dim=2) (FAQ Q7)."""
    if kv.dim() != 5 or kv.shape[2] != 2:
        raise ValueError("kv must be (batch, seqlen_k, 2, heads_kv, head_dim)")
    return attn_func(q, kv[:, :, 0], kv[:, :, 1], dropout_p, softmax_scale, causal, window_size,
                     softcap, out, lse, pack_gqa)


def attn_varlen_func(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, dropout_p=0.0,
                     softmax_scale=None, causal=False, window_size=(-1, -1), softcap=0.0, out=None,
                     lse=None, pack_gqa=None):
    """Packed sequences (FAQ Q8): q (total_q, h_q, d), k/v (total_k, h_kv, d), int32 cu_seqlens.

    ``max_seqlen_q`` / ``max_seqlen_k`` are host ints bounding every sequence length.
    Returns out (total_q, h_q, d) and lse (h_q, total_q).
    """
    _check_dropout(dropout_p)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("varlen q, k, v must be 3-D (total, heads, head_dim)")
    if k.shape != v.shape or k.shape[-1] != q.shape[-1]:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    _check_out(out, q.shape, q.dtype)
    _check_lse(lse, (q.shape[1], q.shape[0]))
    _on_gpu(q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse)
    _check_last_dim(q, k, v)
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold batch + 1 entries")
    if not (cu_seqlens_q.is_contiguous() and cu_seqlens_k.is_contiguous()):
        raise ValueError("cu_seqlens must be contiguous")
    total_q, h_q, d = q.shape
    h_kv = k.shape[1]
    batch = cu_seqlens_q.numel() - 1
    if out is None:
        out = torch.empty((total_q, h_q, d), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((h_q, total_q), dtype=torch.float32, device=q.device)
    _fwd_call(q, k, v, out, lse, batch=batch, s_q=0, s_k=0, h_q=h_q, h_kv=h_kv, d=d,
              q_st=(0, q.stride(0), q.stride(1)), k_st=(0, k.stride(0), k.stride(1)),
              v_st=(0, v.stride(0), v.stride(1)), o_st=(0, out.stride(0), out.stride(1)),
              lse_st=(0, lse.stride(0)), cu_q=cu_seqlens_q, cu_k=cu_seqlens_k, max_q=max_seqlen_q,
              max_k=max_seqlen_k, softmax_scale=softmax_scale, causal=causal, window_size=window_size,
              softcap=softcap, pack_gqa=pack_gqa)
    return out, lse


_ws_cache = {}
_ws_lock = threading.Lock()


def _workspace(dev, nbytes):
    """A per-(device, stream) scratch buffer for split-KV partials, grown on demand."""
    key = (dev, _stream(dev))
    with _ws_lock:
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
            _ws_cache[key] = buf
    return buf


def _decode_args(q, k_cache, v_cache, out, lse, cache_seqlens, softmax_scale, causal, window_size,
                 softcap, num_splits, block_table=None):
    """q and out are (b, s_q, h_q, d) (or (b, h_q, d) for one token)."""
    if q.dim() == 3:
        q, out = q.unsqueeze(1), out.unsqueeze(1)
    b, s_q, h_q, d = q.shape
    s_cache, h_kv = k_cache.shape[1], k_cache.shape[2]
    if block_table is not None:  # pools of pages: capacity = pages per sequence x page size
        s_cache = block_table.shape[1] * k_cache.shape[1]
    a = DecodeArgs()
    a.dtype = _dtype_code(q)
    a.batch, a.heads_q, a.heads_kv, a.head_dim, a.seqlen_cache = b, h_q, h_kv, d, s_cache
    a.q, a.k_cache, a.v_cache, a.o = q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr()
    a.lse = lse.data_ptr() if lse is not None else None
    a.q_stride[:] = [q.stride(0), q.stride(2)]
    a.o_stride[:] = [out.stride(0), out.stride(2)]
    a.seqlen_q = s_q
    a.q_token_stride, a.o_token_stride = q.stride(1), out.stride(1)
    a.k_stride[:] = list(k_cache.stride()[:3])
    a.v_stride[:] = list(v_cache.stride()[:3])
    if block_table is not None:  # the batch stride is replaced by the page table
        a.k_stride[0] = 0
        a.v_stride[0] = 0
    a.cache_seqlens = cache_seqlens.data_ptr() if cache_seqlens is not None else None
    a.softmax_scale = _scale(softmax_scale)
    a.softcap = float(softcap or 0.0)
    a.causal = 1 if causal else 0
    a.window_left, a.window_right = _window(window_size)
    a.num_splits = int(num_splits)
    return a


def decode_plan(q, k_cache, v_cache, cache_seqlens=None, softmax_scale=None, causal=False,
                window_size=(-1, -1), softcap=0.0, num_splits=0, block_table=None):
    """(num_splits, workspace_bytes) the library would use for this decode call."""
    a = _decode_args(q, k_cache, v_cache, q, None, cache_seqlens, softmax_scale, causal, window_size,
                     softcap, num_splits, block_table)
    ns = C.c_int32(0)
    wb = C.c_size_t(0)
    with torch.cuda.device(q.device):
        st = lib().exattn_decode_plan(C.byref(a), C.byref(ns), C.byref(wb))
    _raise_for(st, "exattn_decode_plan")
    return ns.value, wb.value


def attn_with_kvcache(q, k_cache, v_cache, k=None, v=None, cache_seqlens=None, softmax_scale=None,
                      causal=False, window_size=(-1, -1), softcap=0.0, num_splits=0, out=None, lse=None,
                      workspace=None, block_table=None):
    """KV-cache decode (FAQ Q17) for one or a few query tokens.

    q (b, s_q, h_q, d), token t at position len - s_q + t of the len attended keys
    (bottom-right: with causal, token t sees keys up to that position);
    k_cache, v_cache (b, s_cache, h_kv, d); cache_seqlens an
    int32 GPU tensor (b,), an int, or None for the full cache.  With k, v
    (b, s_new, h_kv, d) the new tokens are first written to cache rows
    cache_seqlens[b] .. cache_seqlens[b] + s_new - 1 (k_cache and v_cache are
    updated in place) and the query attends to cache_seqlens[b] + s_new rows;
    cache_seqlens is required then.  The call never changes cache_seqlens (the
    caller advances it by s_new).  num_splits = 0 picks the split count
    automatically (FAQ Q14).  With block_table (b, pages per sequence) int32 the
    caches are page pools (num_pages, page_size, h_kv, d) (FAQ Q18): token j of
    batch entry b is row j % page_size of page block_table[b, j // page_size].
    """
    if (k is None) != (v is None):
        raise ValueError("pass both k and v to append, or neither")
    if q.dim() != 4 or q.shape[1] < 1:
        raise ValueError("q must be (batch, seqlen_q >= 1, heads_q, head_dim)")
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must be (batch, seqlen_cache, heads_kv, head_dim)")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and the caches must share one dtype")
    _check_out(out, q.shape, q.dtype)
    _check_lse(lse, (q.shape[0], q.shape[2], q.shape[1]), contiguous=True)  # lse[(b * h_q + h) * s_q + t]
    _on_gpu(q, k_cache, v_cache, out, lse, cache_seqlens if torch.is_tensor(cache_seqlens) else None,
            workspace, k, v, block_table)
    pg = None
    if block_table is not None:
        if (block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != q.shape[0]
                or block_table.stride(1) != 1):
            raise ValueError("block_table must be an int32 (batch, pages per sequence) tensor, rows contiguous")
        pg = PagedKv()
        pg.block_table = block_table.data_ptr()
        pg.block_table_stride = block_table.stride(0)
        pg.page_size, pg.num_pages = k_cache.shape[1], k_cache.shape[0]
        pg.k_page_stride, pg.v_page_stride = k_cache.stride(0), v_cache.stride(0)
    _check_last_dim(q, k_cache, v_cache)
    b, s_q, h_q, d = q.shape
    kv = None
    if k is not None:
        if k.dim() != 4 or v.shape != k.shape or k.shape[0] != b or k.shape[2:] != k_cache.shape[2:]:
            raise ValueError("k and v must be (batch, seqlen_new, heads_kv, head_dim) like the cache")
        if k.dtype != q.dtype or v.dtype != q.dtype:
            raise ValueError("k and v must share the cache dtype")
        if cache_seqlens is None:
            raise ValueError("appending k/v needs cache_seqlens")
        _check_last_dim(k, v)
        kv = KvNew()
        kv.k_new, kv.v_new, kv.seqlen_new = k.data_ptr(), v.data_ptr(), k.shape[1]
        kv.k_new_stride[:] = list(k.stride()[:3])
        kv.v_new_stride[:] = list(v.stride()[:3])
    if isinstance(cache_seqlens, int):
        cache_seqlens = torch.full((b,), cache_seqlens, dtype=torch.int32, device=q.device)
    if cache_seqlens is not None:
        if cache_seqlens.dtype != torch.int32 or cache_seqlens.numel() != b or not cache_seqlens.is_contiguous():
            raise ValueError("cache_seqlens must be a contiguous int32 tensor of batch entries")
    if out is None:
        out = torch.empty((b, s_q, h_q, d), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((b, h_q, s_q), dtype=torch.float32, device=q.device)
    a = _decode_args(q, k_cache, v_cache, out, lse, cache_seqlens, softmax_scale, causal,
                     window_size, softcap, num_splits, block_table)
    L = lib()
    with torch.cuda.device(q.device):
        ns = C.c_int32(0)
        wb = C.c_size_t(0)
        st = L.exattn_decode_plan(C.byref(a), C.byref(ns), C.byref(wb))
        _raise_for(st, "exattn_decode_plan")
        ws_ptr, ws_bytes = None, 0
        if wb.value > 0:
            if workspace is None:
                workspace = _workspace(q.device, wb.value)
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        ws = C.c_void_p(ws_ptr) if ws_ptr else None
        strm = C.c_void_p(_stream(q.device))
        if pg is not None:
            st = L.exattn_decode_paged(C.byref(a), C.byref(pg), C.byref(kv) if kv is not None else None, ws,
                                       ws_bytes, strm)
            what = "exattn_decode_paged"
        elif kv is None:
            st, what = L.exattn_decode(C.byref(a), ws, ws_bytes, strm), "exattn_decode"
        else:
            st, what = L.exattn_decode_append(C.byref(a), C.byref(kv), ws, ws_bytes, strm), "exattn_decode_append"
    _raise_for(st, what)
    return out, lse


def _bwd_call(dout, q, k, v, out, lse, dq, dk, dv, workspace, *, batch, s_q, s_k, h_q, h_kv, d, strides,
              lse_st, softmax_scale, causal, window_size, softcap, cu_q=None, cu_k=None, max_q=0, max_k=0):
    a = BwdArgs()
    a.dtype = _dtype_code(q)
    a.batch, a.seqlen_q, a.seqlen_k, a.heads_q, a.heads_kv, a.head_dim = batch, s_q, s_k, h_q, h_kv, d
    a.q, a.k, a.v, a.o, a.dout = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr()
    a.lse = lse.data_ptr()
    a.dq, a.dk, a.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    for name, st in strides.items():
        getattr(a, f"{name}_stride")[:] = list(st)
    a.lse_stride[:] = list(lse_st)
    a.softmax_scale = _scale(softmax_scale)
    a.softcap = float(softcap or 0.0)
    a.causal = 1 if causal else 0
    a.window_left, a.window_right = _window(window_size)
    a.cu_seqlens_q = cu_q.data_ptr() if cu_q is not None else None
    a.cu_seqlens_k = cu_k.data_ptr() if cu_k is not None else None
    a.max_seqlen_q, a.max_seqlen_k = int(max_q), int(max_k)
    L = lib()
    with torch.cuda.device(q.device):
        wb = C.c_size_t(0)
        _raise_for(L.exattn_bwd_plan(C.byref(a), C.byref(wb)), "exattn_bwd_plan")
        ws_ptr, ws_bytes = None, 0
        if wb.value > 0:
            if workspace is None:
                workspace = _workspace(q.device, wb.value)
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        st = L.exattn_bwd(C.byref(a), C.c_void_p(ws_ptr) if ws_ptr else None, ws_bytes,
                          C.c_void_p(_stream(q.device)))
    _raise_for(st, "exattn_bwd")


def attn_backward(dout, q, k, v, out, lse, softmax_scale=None, causal=False, window_size=(-1, -1),
                  softcap=0.0, dq=None, dk=None, dv=None, workspace=None):
    """Gradients of attn_func: (dq, dk, dv) for the upstream gradient dout.

    q, out, dout (b, s_q, h_q, d); k, v (b, s_k, h_kv, d); lse (b, h_q, s_q) fp32
    as attn_func returns it; the same scale, causal, window and softcap as the
    forward call.  A KV head's dk and dv sum over the query heads that read it.
    head_dim 64, 128 or 256.  Deterministic.
    """
    for name, t in (("q", q), ("out", out), ("dout", dout)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be (batch, seqlen, heads, head_dim)")
    if out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("out and dout must have the shape of q")
    if k.dim() != 4 or v.shape != k.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError("k and v must be (batch, seqlen_k, heads_kv, head_dim)")
    if len({q.dtype, k.dtype, v.dtype, out.dtype, dout.dtype}) != 1:
        raise ValueError("q, k, v, out and dout must share one dtype")
    b, s_q, h_q, d = q.shape
    s_k, h_kv = k.shape[1], k.shape[2]
    if lse.dtype != torch.float32 or lse.shape != (b, h_q, s_q):
        raise ValueError("lse must be fp32 (batch, heads_q, seqlen_q)")
    _on_gpu(dout, q, k, v, out, lse, dq, dk, dv, workspace)
    _check_last_dim(dout, q, k, v, out, dq, dk, dv)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("dq, dk and dv must have the shapes of q, k and v")
    if len({q.dtype, dq.dtype, dk.dtype, dv.dtype}) != 1:
        raise ValueError("dq, dk and dv must have the dtype of q")
    strides = {name: t.stride()[:3] for name, t in (("q", q), ("k", k), ("v", v), ("o", out), ("dout", dout),
                                                     ("dq", dq), ("dk", dk), ("dv", dv))}
    _bwd_call(dout, q, k, v, out, lse, dq, dk, dv, workspace, batch=b, s_q=s_q, s_k=s_k, h_q=h_q, h_kv=h_kv,
              d=d, strides=strides, lse_st=(lse.stride(0), lse.stride(1)), softmax_scale=softmax_scale,
              causal=causal, window_size=window_size, softcap=softcap)
    return dq, dk, dv


def attn_varlen_backward(dout, q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                         softmax_scale=None, causal=False, window_size=(-1, -1), softcap=0.0, dq=None, dk=None,
                         dv=None, workspace=None):
    """Gradients of attn_varlen_func (FAQ Q8 packing): q, out, dout (total_q, h_q, d); k, v
    (total_k, h_kv, d); lse (h_q, total_q) as attn_varlen_func returns it.  Returns (dq, dk, dv)."""
    for name, t in (("q", q), ("out", out), ("dout", dout), ("k", k), ("v", v)):
        if t.dim() != 3:
            raise ValueError(f"varlen {name} must be (total, heads, head_dim)")
    if out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("out and dout must have the shape of q")
    if v.shape != k.shape or k.shape[-1] != q.shape[-1]:
        raise ValueError("k and v must be (total_k, heads_kv, head_dim)")
    if len({q.dtype, k.dtype, v.dtype, out.dtype, dout.dtype}) != 1:
        raise ValueError("q, k, v, out and dout must share one dtype")
    total_q, h_q, d = q.shape
    h_kv = k.shape[1]
    if lse.dtype != torch.float32 or lse.shape != (h_q, total_q):
        raise ValueError("lse must be fp32 (heads_q, total_q)")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold batch + 1 entries")
    _on_gpu(dout, q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, dq, dk, dv, workspace)
    _check_last_dim(dout, q, k, v, out, dq, dk, dv)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("dq, dk and dv must have the shapes of q, k and v")
    strides = {name: (0, t.stride(0), t.stride(1)) for name, t in
               (("q", q), ("k", k), ("v", v), ("o", out), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv))}
    _bwd_call(dout, q, k, v, out, lse, dq, dk, dv, workspace, batch=cu_seqlens_q.numel() - 1, s_q=0, s_k=0,
              h_q=h_q, h_kv=h_kv, d=d, strides=strides, lse_st=(0, lse.stride(0)), softmax_scale=softmax_scale,
              causal=causal, window_size=window_size, softcap=softcap, cu_q=cu_seqlens_q, cu_k=cu_seqlens_k,
              max_q=max_seqlen_q, max_k=max_seqlen_k)
    return dq, dk, dv


def auto_splits(batch, heads_q, heads_kv, seqlen_k, head_dim, num_cus):
    """The library's automatic split count for a device with num_cus compute units."""
    return int(lib().exattn_decode_auto_splits(batch, heads_q, heads_kv, seqlen_k, head_dim, num_cus))


__all__ = ["attn_func", "attn_func_fp8", "attn_varlen_func_fp8", "attn_qkvpacked_func", "attn_kvpacked_func", "attn_varlen_func",
           "attn_with_kvcache", "attn_backward", "attn_varlen_backward", "decode_plan", "auto_splits", "lib",
           "library_path"]
