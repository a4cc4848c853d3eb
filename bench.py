#!/usr/bin/env python3
"""Benchmark of the exact-attention forward on one MI355X.

One step is one forward call of the causal prefill workload: packed qkv
(2, 1024, 3, 16, 128) bf16, causal, scale 1/sqrt(128) ("FlashAttention完整说明",
section 六.1).  Inputs are resident in device memory before the timed region.
The FLOP count is the pages' 4*b*h*s_q*s_k*d halved for causal (Inference
Cookbook FAQ Q16).  The KV-cache decode workload (batch 8, 16384 cached
tokens, 32 query / 8 KV heads, d 128, bf16, automatic num_splits) is timed in
the same run and reported as HBM GB/s under "decode", and the backward of the
prefill workload (dQ, dK, dV from O, LSE and dO) as TFLOPS under "backward", the
FP8 forward (E4M3 inputs, bf16 output) of the same shape under "fp8", and every
other forward workload (tiny, the head-dim sweep, varlen + GQA + masks,
cross-attention, the 16k-token causal prefill) at its own shape under "configs".

Prints one JSON line.  Options:
  --gpus N            only 1 is supported (the method runs on one GPU here)
  --steps K --warmup W
  --no-cpu-baseline   skip the CPU oracle timing
  --no-decode         skip the decode measurement
  --no-backward       skip the backward measurement
  --no-fp8            skip the FP8 forward measurement
  --no-configs        skip the other forward workloads
  --only {prefill,decode,backward,fp8,configs,copy}  run one part only (for profiler runs)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_FP8_TFLOPS = 5033.2   # MI355X dense FP8 MFMA: twice the bf16 rate
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
METRIC = "attn fwd TFLOPS (% bf16 MFMA peak) at b2 s1024 h16 d128; decode HBM GB/s"
PREFILL_SOURCES = ["exact_attention_43_amd/csrc/fwd_prefill.hip",
                   "exact_attention_43_amd/csrc/device_common.h",
                   "exact_attention_43_amd/csrc/tiles.h"]
DECODE_SOURCES = ["exact_attention_43_amd/csrc/fwd_decode.hip",
                  "exact_attention_43_amd/csrc/device_common.h"]


def sources_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(name, paths):
    """HBM bytes per launch from a committed counter summary, if it matches the current kernel."""
    fn = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(fn):
        return None
    with open(fn) as f:
        rec = json.load(f)
    if rec.get("kernel_sha") != sources_sha(paths):
        return None
    return rec.get("bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "backward", "fp8", "configs", "copy"], default=None)
    return ap.parse_args()


def prefill_step_fn(ex, qkv, out, lse, causal=True):
    """Build the C-ABI call once; the returned closure only launches."""
    import ctypes as C
    import torch
    b, s, _, h, d = qkv.shape
    a = ex.FwdArgs()
    a.dtype = ex.EXATTN_BF16 if qkv.dtype == torch.bfloat16 else ex.EXATTN_F16
    a.batch, a.seqlen_q, a.seqlen_k, a.heads_q, a.heads_kv, a.head_dim = b, s, s, h, h, d
    es = qkv.element_size()
    base = qkv.data_ptr()
    a.q, a.k, a.v = base, base + h * d * es, base + 2 * h * d * es
    a.o, a.lse = out.data_ptr(), lse.data_ptr()
    st = list(qkv.stride())
    for n in ("q_stride", "k_stride", "v_stride"):
        getattr(a, n)[:] = [st[0], st[1], st[3]]
    a.o_stride[:] = list(out.stride()[:3])
    a.lse_stride[:] = [lse.stride(0), lse.stride(1)]
    a.softmax_scale = float("nan")  # the default 1/sqrt(head_dim)
    a.pack_gqa = -1
    a.softcap = 0.0
    a.causal = 1 if causal else 0
    a.window_left = a.window_right = -1
    L = ex.lib()
    ref = C.byref(a)
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step():
        rc = L.exattn_fwd(ref, stream)
        if rc != 0:
            ex._raise_for(rc, "exattn_fwd")
    return step


def fwd_step_fn(ex, q, k, v, out, lse, *, batch, s_q, s_k, q_st, k_st, v_st, o_st, lse_st, cu_q=None,
                cu_k=None, max_q=0, max_k=0, causal=False, window=(-1, -1), softcap=0.0):
    """exattn_fwd with its argument block built once; the closure only launches."""
    import ctypes as C
    import torch
    a = ex.FwdArgs()
    a.dtype = ex.EXATTN_BF16 if q.dtype == torch.bfloat16 else ex.EXATTN_F16
    a.batch, a.seqlen_q, a.seqlen_k = batch, s_q, s_k
    a.heads_q, a.heads_kv, a.head_dim = q.shape[-2], k.shape[-2], q.shape[-1]
    a.q, a.k, a.v, a.o, a.lse = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr()
    for name, st in (("q_stride", q_st), ("k_stride", k_st), ("v_stride", v_st), ("o_stride", o_st)):
        getattr(a, name)[:] = list(st)
    a.lse_stride[:] = list(lse_st)
    a.cu_seqlens_q = cu_q.data_ptr() if cu_q is not None else None
    a.cu_seqlens_k = cu_k.data_ptr() if cu_k is not None else None
    a.max_seqlen_q, a.max_seqlen_k = max_q, max_k
    a.softmax_scale = float("nan")  # the default 1/sqrt(head_dim)
    a.pack_gqa = -1
    a.softcap = softcap
    a.causal = 1 if causal else 0
    a.window_left, a.window_right = window
    L = ex.lib()
    ref = C.byref(a)
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    keep = (a, q, k, v, out, lse, cu_q, cu_k)

    def step():
        rc = L.exattn_fwd(ref, stream)
        if rc != 0:
            ex._raise_for(rc, "exattn_fwd")
    step.keep = keep
    return step


# The other forward workloads, each timed at its own shape (back-to-back launches,
# inputs resident in HBM) against the bf16/fp16 MFMA peak.
CONFIG_WORKLOADS = ["tiny", "hdim64", "hdim128", "hdim256", "varlen_gqa", "cross", "long_prefill"]


def run_configs(ex, W, args):
    import torch
    res = {}
    for name in CONFIG_WORKLOADS:
        w = W.WORKLOADS[name]
        dt = W.DTYPES[w.dtype]
        if w.kind == "varlen":
            q, k, v, cq, ck = W.varlen_qkv(w.seqlens, w.seqlens, w.heads_q, w.heads_kv, w.head_dim,
                                           seed=w.seed, dtype=dt)
            q, k, v, cq, ck = (t.cuda() for t in (q, k, v, cq, ck))
            out = torch.empty_like(q)
            lse = torch.empty((w.heads_q, q.shape[0]), dtype=torch.float32, device="cuda")
            step = fwd_step_fn(ex, q, k, v, out, lse, batch=len(w.seqlens), s_q=0, s_k=0,
                               q_st=(0, q.stride(0), q.stride(1)), k_st=(0, k.stride(0), k.stride(1)),
                               v_st=(0, v.stride(0), v.stride(1)), o_st=(0, out.stride(0), out.stride(1)),
                               lse_st=(0, lse.stride(0)), cu_q=cq, cu_k=ck, max_q=max(w.seqlens),
                               max_k=max(w.seqlens), causal=w.causal, window=w.window, softcap=w.softcap)
            desc = (f"varlen lengths {list(w.seqlens)}, h_q {w.heads_q} / h_kv {w.heads_kv}, d {w.head_dim}, "
                    f"{w.dtype}, causal, window {tuple(w.window)}, softcap {w.softcap}")
        else:
            q, k, v = W.qkv(w.batch, w.seqlen_q, w.seqlen_k, w.heads_q, w.heads_kv, w.head_dim, seed=w.seed,
                            dtype=dt)
            q, k, v = q.cuda(), k.cuda(), v.cuda()
            out = torch.empty_like(q)
            lse = torch.empty((w.batch, w.heads_q, w.seqlen_q), dtype=torch.float32, device="cuda")
            step = fwd_step_fn(ex, q, k, v, out, lse, batch=w.batch, s_q=w.seqlen_q, s_k=w.seqlen_k,
                               q_st=q.stride()[:3], k_st=k.stride()[:3], v_st=v.stride()[:3],
                               o_st=out.stride()[:3], lse_st=(lse.stride(0), lse.stride(1)), causal=w.causal,
                               window=w.window, softcap=w.softcap)
            desc = (f"b {w.batch}, s_q {w.seqlen_q}, s_k {w.seqlen_k}, h_q {w.heads_q} / h_kv {w.heads_kv}, "
                    f"d {w.head_dim}, {w.dtype}" + (", causal" if w.causal else ", non-causal"))
        fl = W.flops(w)
        reps = 10 if fl > 1e11 else 100
        t = time_steps(step, reps, 5)
        tf = fl / (t["region"] * 1e-3) / 1e12
        res[name] = {"workload": desc, "us_per_call": round(t["region"] * 1e3, 2),
                     "us_per_call_median": round(t["pair_median"] * 1e3, 2), "tflops": round(tf, 2),
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flops": fl,
                     "algorithmic_bytes": W.algorithmic_bytes(w), "calls": reps}
        del step, q, k, v, out, lse
        torch.cuda.empty_cache()
    return res


def time_steps(step, steps, warmup, between=None):
    """Warm up, then time `steps` calls twice on the launching stream.

    Pass 1 launches back to back: wall clock over the region (synchronised on both sides)
    and one HIP event pair around the whole region.  Pass 2 puts an event pair around each
    call, for the median and minimum.  Returns a dict of milliseconds per call."""
    import torch
    for _ in range(warmup):
        if between:
            between()
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        if between:
            between()
        step()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    region_ms = e0.elapsed_time(e1)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        if between:
            between()
        starts[i].record()
        step()
        ends[i].record()
    torch.cuda.synchronize()
    durs = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return {"wall": wall_ms / steps, "region": region_ms / steps, "pair_avg": sum(durs) / len(durs),
            "pair_median": durs[len(durs) // 2], "pair_min": durs[0]}


def cpu_baseline(w, flops_full):
    """The fp64 oracle on the host cores, on the same workload (bounded to ~10-30 s)."""
    import numpy as np  # noqa: F401
    import oracle
    from exact_attention_43_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    qkv = W.packed_qkv(w.batch, w.seqlen_q, w.heads_q, w.head_dim, seed=w.seed)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    heads = list(range(w.heads_q))
    t0 = time.perf_counter()
    passes = 0
    while True:
        oracle.attention(q, k, v, causal=True, heads=heads)
        passes += 1
        el = time.perf_counter() - t0
        if el > 10.0 or passes >= 100:
            break
    sec = el / passes
    return {"value": round(flops_full / sec / 1e12, 6), "unit": "TFLOPS", "cores": int(threads),
            "kind": "oracle",
            "sample": f"full causal_prefill workload (b2 s1024 h16 d128, all 32 heads), "
                      f"{passes} pass(es), {sec:.2f} s per pass, numpy fp64 materialising S and P"}


def run_prefill(ex, W, args):
    import torch
    w = W.WORKLOADS["causal_prefill"]
    qkv = W.packed_qkv(w.batch, w.seqlen_q, w.heads_q, w.head_dim, seed=w.seed).cuda()
    out = torch.empty((w.batch, w.seqlen_q, w.heads_q, w.head_dim), dtype=qkv.dtype, device="cuda")
    lse = torch.empty((w.batch, w.heads_q, w.seqlen_q), dtype=torch.float32, device="cuda")
    step = prefill_step_fn(ex, qkv, out, lse)
    t = time_steps(step, args.steps, args.warmup)
    return w, W.flops(w), t


def run_decode(ex, W, args):
    import torch
    w = W.WORKLOADS["decode"]
    q, kc, vc = W.kvcache(w.batch, w.seqlen_k, w.heads_q, w.heads_kv, w.head_dim, seed=w.seed)
    q, kc, vc = q.cuda(), kc.cuda(), vc.cuda()
    lens = torch.tensor(w.cache_seqlens, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((w.batch, w.heads_q, 1), dtype=torch.float32, device="cuda")
    ns, wb = ex.decode_plan(q[:, 0], kc, vc, lens)
    ws = torch.empty(max(wb, 256), dtype=torch.uint8, device="cuda")
    flush = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")

    def step():
        ex.attn_with_kvcache(q, kc, vc, cache_seqlens=lens, out=out, lse=lse, workspace=ws)

    def between():
        # Reading 1 GiB of other data evicts the KV cache from L2 and the 256 MB MALL.  A write
        # would leave dirty lines in the MALL whose write-back the next kernel's reads pay for.
        torch.amax(flush)

    steps = max(10, min(args.steps, 50))
    t = time_steps(step, steps, max(2, args.warmup // 4), between)
    ms_avg, ms_med, ms_min = t["pair_avg"], t["pair_median"], t["pair_min"]
    nbytes = W.algorithmic_bytes(w)
    gbs = nbytes / (ms_avg * 1e-3) / 1e9
    traffic = measured_traffic("decode_b8_h32x8_d128_cache16384", DECODE_SOURCES)

    # The same step with a one-token append (FAQ Q17): each batch entry's new K/V row is written
    # at cache_seqlens[b] = 16383 and the query attends to all 16384 rows, as above.
    kn, vn = W.kv_new(w.batch, 1, w.heads_kv, w.head_dim, seed=w.seed + 1)
    kn, vn = kn.cuda(), vn.cuda()
    lens_app = lens - 1

    def step_app():
        ex.attn_with_kvcache(q, kc, vc, k=kn, v=vn, cache_seqlens=lens_app, out=out, lse=lse,
                             workspace=ws)

    ta = time_steps(step_app, steps, max(2, args.warmup // 4), between)
    new_bytes = 2 * 2 * kn.numel() * kn.element_size()  # read k_new, v_new and write them into the cache
    gbs_app = (nbytes + new_bytes) / (ta["pair_avg"] * 1e-3) / 1e9
    append = {
        "workload": "the same decode with a one-token k/v append at cache_seqlens = 16383",
        "value": round(gbs_app, 2), "unit": "GB/s", "ms_per_call_avg": round(ta["pair_avg"], 5),
        "ms_per_call_median": round(ta["pair_median"], 5), "ms_per_call_min": round(ta["pair_min"], 5),
        "calls": steps, "algorithmic_bytes": nbytes + new_bytes,
        "frac": round(gbs_app / PEAK_HBM_GBS, 4),
    }
    # The same decode over a paged cache (FAQ Q18): 256-token pages of the same K/V, placed at a
    # seeded random permutation of the pool's page slots.
    page = 256
    per_seq = w.seqlen_k // page
    perm = torch.randperm(w.batch * per_seq, generator=torch.Generator().manual_seed(w.seed + 2))
    bt = perm.to(torch.int32).reshape(w.batch, per_seq).cuda()
    kpool = torch.empty((w.batch * per_seq, page, w.heads_kv, w.head_dim), dtype=kc.dtype, device="cuda")
    vpool = torch.empty_like(kpool)
    kpool[perm.cuda()] = kc.reshape(w.batch * per_seq, page, w.heads_kv, w.head_dim)
    vpool[perm.cuda()] = vc.reshape(w.batch * per_seq, page, w.heads_kv, w.head_dim)

    def step_paged():
        ex.attn_with_kvcache(q, kpool, vpool, cache_seqlens=lens, out=out, lse=lse, workspace=ws,
                             block_table=bt)

    tp = time_steps(step_paged, steps, max(2, args.warmup // 4), between)
    gbs_pg = nbytes / (tp["pair_avg"] * 1e-3) / 1e9
    paged = {
        "workload": "the same decode over a paged cache: 256-token pages in a random pool order",
        "value": round(gbs_pg, 2), "unit": "GB/s", "ms_per_call_avg": round(tp["pair_avg"], 5),
        "ms_per_call_median": round(tp["pair_median"], 5), "ms_per_call_min": round(tp["pair_min"], 5),
        "calls": steps, "algorithmic_bytes": nbytes, "frac": round(gbs_pg / PEAK_HBM_GBS, 4),
    }
    return {
        "workload": "kvcache decode b8 s_q1 cache16384 h_q32 h_kv8 d128 bf16",
        "num_splits": ns, "value": round(gbs, 2), "unit": "GB/s",
        "ms_per_call_avg": round(ms_avg, 5), "ms_per_call_median": round(ms_med, 5),
        "ms_per_call_min": round(ms_min, 5), "calls": steps,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes": nbytes},
        "cache_flush": "1 GiB read of another buffer between calls (outside the event pairs)",
        "append": append,
        "paged": paged,
    }


def run_backward(ex, W, args):
    """The backward of the causal prefill workload: one step is one exattn_bwd call (two
    kernels: dQ with the row statistics, then dK/dV) on resident q, k, v, o, lse and dO."""
    import ctypes as C
    import torch
    w = W.WORKLOADS["causal_prefill"]
    qkv = W.packed_qkv(w.batch, w.seqlen_q, w.heads_q, w.head_dim, seed=w.seed).cuda()
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    out, lse = ex.attn_func(q, k, v, causal=True)
    dout = W.qkv(w.batch, w.seqlen_q, 1, w.heads_q, 1, w.head_dim, seed=w.seed + 7)[0].cuda()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    a = ex.BwdArgs()
    a.dtype = ex.EXATTN_BF16
    a.batch, a.seqlen_q, a.seqlen_k = w.batch, w.seqlen_q, w.seqlen_k
    a.heads_q, a.heads_kv, a.head_dim = w.heads_q, w.heads_kv, w.head_dim
    a.q, a.k, a.v, a.o, a.dout = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr()
    a.lse = lse.data_ptr()
    a.dq, a.dk, a.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", out), ("dout", dout), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        getattr(a, f"{name}_stride")[:] = list(t.stride()[:3])
    a.lse_stride[:] = [lse.stride(0), lse.stride(1)]
    a.softmax_scale = float("nan")  # the default 1/sqrt(head_dim), as in the forward above
    a.causal = 1
    a.window_left = a.window_right = -1
    L = ex.lib()
    wb = C.c_size_t(0)
    ex._raise_for(L.exattn_bwd_plan(C.byref(a), C.byref(wb)), "exattn_bwd_plan")
    ws = torch.empty(max(wb.value, 256), dtype=torch.uint8, device="cuda")
    ref = C.byref(a)
    ws_ptr, ws_bytes = C.c_void_p(ws.data_ptr()), ws.numel()
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step():
        rc = L.exattn_bwd(ref, ws_ptr, ws_bytes, stream)
        if rc != 0:
            ex._raise_for(rc, "exattn_bwd")

    steps = max(10, min(args.steps, 100))
    t = time_steps(step, steps, max(2, args.warmup // 2))
    fl = W.backward_flops(w)
    tflops = fl / (t["region"] * 1e-3) / 1e12
    return {
        "workload": "backward of the causal prefill: q, k, v (2, 1024, 16, 128) bf16 from packed qkv, "
                    "o and lse from the forward, dO synthetic",
        "value": round(tflops, 3), "unit": "TFLOPS", "flops_per_call": fl,
        "ms_per_call_avg": round(t["region"], 6), "ms_per_call_median": round(t["pair_median"], 6),
        "ms_per_call_min": round(t["pair_min"], 6), "calls": steps,
        "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
    }


def fp8_step_fn(ex, W, w):
    """One exattn_fwd_fp8 call on workload w: q, k, v E4M3 codes of the seeded N(0,1) draw of
    its shape, descales 1, bf16 output.  Returns (step, tensors the step uses)."""
    import ctypes as C
    import torch
    q, k, v = (t.cuda() for t in W.qkv(w.batch, w.seqlen_q, w.seqlen_k, w.heads_q, w.heads_kv, w.head_dim,
                                       seed=w.seed, dtype=torch.float8_e4m3fn))
    out = torch.empty((w.batch, w.seqlen_q, w.heads_q, w.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, w.heads_q, w.seqlen_q), dtype=torch.float32, device="cuda")
    a = ex.FwdArgs()
    a.dtype = ex.EXATTN_FP8_E4M3
    a.batch, a.seqlen_q, a.seqlen_k = w.batch, w.seqlen_q, w.seqlen_k
    a.heads_q, a.heads_kv, a.head_dim = w.heads_q, w.heads_kv, w.head_dim
    a.q, a.k, a.v, a.o, a.lse = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr()
    a.q_stride[:] = list(q.stride()[:3])
    a.k_stride[:] = list(k.stride()[:3])
    a.v_stride[:] = list(v.stride()[:3])
    a.o_stride[:] = list(out.stride()[:3])
    a.lse_stride[:] = [lse.stride(0), lse.stride(1)]
    a.causal = 1 if w.causal else 0
    a.window_left = a.window_right = -1
    a.softmax_scale = float("nan")  # the default 1/sqrt(head_dim), as in the 16-bit forward
    a.softcap = 0.0
    ds = ex.Fp8Descale(1.0, 1.0, 1.0)
    L = ex.lib()
    ref, dref = C.byref(a), C.byref(ds)
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step():
        rc = L.exattn_fwd_fp8(ref, dref, stream)
        if rc != 0:
            ex._raise_for(rc, "exattn_fwd_fp8")

    return step, (q, k, v, out, lse, a, ds)


def fp8_timing(ex, W, w, steps, warmup):
    """time_steps of fp8_step_fn's step on workload w.  Returns (result, flops)."""
    step, keep = fp8_step_fn(ex, W, w)
    t = time_steps(step, steps, warmup)
    del step, keep
    return t, W.flops(w)


def bf16_fwd_step_fn(ex, W, w):
    """One exattn_fwd call on fixed-length workload w (its own dtype).  Returns (step, tensors)."""
    import torch
    q, k, v = W.qkv(w.batch, w.seqlen_q, w.seqlen_k, w.heads_q, w.heads_kv, w.head_dim, seed=w.seed,
                    dtype=W.DTYPES[w.dtype])
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    out = torch.empty_like(q)
    lse = torch.empty((w.batch, w.heads_q, w.seqlen_q), dtype=torch.float32, device="cuda")
    step = fwd_step_fn(ex, q, k, v, out, lse, batch=w.batch, s_q=w.seqlen_q, s_k=w.seqlen_k,
                       q_st=q.stride()[:3], k_st=k.stride()[:3], v_st=v.stride()[:3],
                       o_st=out.stride()[:3], lse_st=(lse.stride(0), lse.stride(1)), causal=w.causal,
                       window=w.window, softcap=w.softcap)
    return step, (q, k, v, out, lse)


def interleaved_ms(steps_by_name, rounds=6, calls=3):
    """Median ms per call of each step, timed in alternation (`calls` calls of each per round,
    one event pair around each run of calls), so that every step meets the same clock and
    temperature as the others."""
    import torch
    times = {n: [] for n in steps_by_name}
    for n, f in steps_by_name.items():
        f()
    torch.cuda.synchronize()
    for _ in range(rounds):
        for n, f in steps_by_name.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(calls):
                f()
            e1.record()
            torch.cuda.synchronize()
            times[n].append(e0.elapsed_time(e1) / calls)
    return {n: sorted(v)[len(v) // 2] for n, v in times.items()}


def run_fp8(ex, W, args):
    """The FP8 forward on the causal prefill shape (2, 1024, 16, 128) and on the 16k-token causal
    prefill (1, 16384, 16, 128); one step is one exattn_fwd_fp8 call."""
    import torch
    steps = max(10, min(args.steps, 100))
    t, fl = fp8_timing(ex, W, W.WORKLOADS["causal_prefill"], steps, max(2, args.warmup // 2))
    tflops = fl / (t["region"] * 1e-3) / 1e12
    tl, fll = fp8_timing(ex, W, W.WORKLOADS["long_prefill"], 10, 3)
    torch.cuda.empty_cache()
    tfl = fll / (tl["region"] * 1e-3) / 1e12
    # the same 16k-token causal forward in bf16 and in FP8, alternating, so that the ratio
    # does not depend on which leg ran on a hotter, lower-clocked chip
    f8_step, f8_keep = fp8_step_fn(ex, W, W.WORKLOADS["long_prefill"])
    bf_step, bf_keep = bf16_fwd_step_fn(ex, W, W.WORKLOADS["long_prefill"])
    side = interleaved_ms({"bf16": bf_step, "fp8": f8_step})
    del f8_step, f8_keep, bf_step, bf_keep
    torch.cuda.empty_cache()
    return {
        "workload": "FP8 forward of the causal prefill shape: q, k, v (2, 1024, 16, 128) E4M3, descales 1, "
                    "bf16 out",
        "value": round(tflops, 3), "unit": "TFLOPS", "flops_per_call": fl,
        "ms_per_call_avg": round(t["region"], 6), "ms_per_call_median": round(t["pair_median"], 6),
        "ms_per_call_min": round(t["pair_min"], 6), "calls": steps,
        "frac_of_fp8_peak": round(tflops / PEAK_FP8_TFLOPS, 4),
        "long": {"workload": "FP8 forward, b 1, s 16384, h 16, d 128, causal, E4M3, descales 1, bf16 out",
                 "us_per_call": round(tl["region"] * 1e3, 2), "tflops": round(tfl, 2),
                 "frac_of_fp8_peak": round(tfl / PEAK_FP8_TFLOPS, 4), "calls": 10,
                 "alternating_with_bf16": {"bf16_us_per_call": round(side["bf16"] * 1e3, 2),
                                           "fp8_us_per_call": round(side["fp8"] * 1e3, 2),
                                           "fp8_over_bf16": round(side["fp8"] / side["bf16"], 4),
                                           "method": "6 rounds of 3 bf16 calls then 3 FP8 calls, "
                                                     "medians of the per-round means"}},
        "note": "S on the FP8 MFMA, PV on the bf16 MFMA (P rounded to bf16)",
    }


def run_copy_calibration():
    """A plain device copy of known size, for scaling the HBM byte counters: 7 launches of a
    256 MiB fp32 multiply-by-one (each reads 256 MiB and writes 256 MiB)."""
    import torch
    n = (256 << 20) // 4
    src = torch.full((n,), 3.0, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(7):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n * 4, "copies": 7}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this attention forward is measured on "
              f"one GPU; the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        sys.exit(1)
    import exact_attention_43_amd as ex
    from exact_attention_43_amd import workloads as W
    ex.lib()
    torch.cuda.set_device(0)

    if args.only == "copy":
        run_copy_calibration()
        return
    if args.only == "decode":
        print(json.dumps(run_decode(ex, W, args)))
        return
    if args.only == "backward":
        print(json.dumps(run_backward(ex, W, args)))
        return
    if args.only == "fp8":
        print(json.dumps(run_fp8(ex, W, args)))
        return
    if args.only == "configs":
        print(json.dumps(run_configs(ex, W, args)))
        return

    w, fl, t = run_prefill(ex, W, args)
    if args.only == "prefill":
        print(json.dumps(t))
        return
    ms_step = t["wall"]
    k_avg = t["region"]  # back-to-back launches: the kernel's average duration on the stream
    value = fl / (ms_step * 1e-3) / 1e12
    achieved = fl / (k_avg * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal prefill, packed qkv (2, 1024, 3, 16, 128) bf16, causal, "
                               "scale 1/sqrt(128)",
                   "batch": w.batch, "seqlen": w.seqlen_q, "heads": w.heads_q, "head_dim": w.head_dim,
                   "flops_per_step": fl, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("prefill_causal_b2_s1024_h16_d128", PREFILL_SOURCES),
                     "kernel_ms_avg": round(k_avg, 6),
                     "kernel_ms_median_event_pair": round(t["pair_median"], 6),
                     "kernel_ms_min_event_pair": round(t["pair_min"], 6)},
    }
    if not args.no_decode:
        rec["decode"] = run_decode(ex, W, args)
    if not args.no_backward:
        rec["backward"] = run_backward(ex, W, args)
    if not args.no_fp8:
        rec["fp8"] = run_fp8(ex, W, args)
    if not args.no_configs:
        rec["configs"] = run_configs(ex, W, args)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, fl)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
