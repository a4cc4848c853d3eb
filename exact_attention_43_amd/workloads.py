"""Seeded synthetic inputs and the named workload shapes.

This module is shared by the tests, the benchmark and the smoke check, and it
feeds both the GPU path and the CPU oracle.  It holds no attention arithmetic:
only shapes, seeds and a normal random draw, so that both sides see the same
rounded fp16/bf16 values.

Inputs are i.i.d. N(0, 1) drawn in float32 on the CPU from
``torch.Generator().manual_seed(seed)`` and rounded to the storage dtype
(round-to-nearest-even).  When one call needs several tensors (q, k, v) they are
drawn from one generator in that order.

The shapes follow the workloads the pages describe:
- the tiny (1, 64, 4, 64) fp16 smoke call (Inference Cookbook FAQ, Q2);
- the packed (2, 1024, 3, 16, 128) bf16 causal call ("FlashAttention完整说明",
  section 六.1, native API call);
- the head-dim 64/128/256 smoke tests at batch 2, length 1024 (the Flash-Attention
  2.8.3 RTX 3090 build notes, test code);
- the three packed sequences [100, 200, 150] (FAQ Q8), window (256, 0) (FAQ Q21),
  softcap 50 (FAQ Q22), grouped heads (FAQ Q15), cross-attention (FAQ Q7);
- 16384-token context ("FlashAttention完整说明", section 一, the N = 16384 example)
  and KV-cache decode with split-KV (FAQ Q14, Q17).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


def randn(shape, seed: int | None = None, dtype=torch.bfloat16, generator=None):
    """Draw N(0,1) float32 on the CPU from a seeded generator, then round to ``dtype``."""
    if generator is None:
        generator = torch.Generator().manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=generator, dtype=torch.float32)
    return x.to(dtype)


def qkv(b, s_q, s_k, h_q, h_kv, d, seed, dtype=torch.bfloat16):
    """q (b, s_q, h_q, d), k and v (b, s_k, h_kv, d), drawn in that order from one generator."""
    g = torch.Generator().manual_seed(int(seed))
    q = randn((b, s_q, h_q, d), dtype=dtype, generator=g)
    k = randn((b, s_k, h_kv, d), dtype=dtype, generator=g)
    v = randn((b, s_k, h_kv, d), dtype=dtype, generator=g)
    return q, k, v


def packed_qkv(b, s, h, d, seed, dtype=torch.bfloat16):
    """One (b, s, 3, h, d) tensor drawn in a single call."""
    return randn((b, s, 3, h, d), seed=seed, dtype=dtype)


def varlen_qkv(seqlens_q, seqlens_k, h_q, h_kv, d, seed, dtype=torch.bfloat16):
    """Packed (total, h, d) tensors plus int32 prefix sums of the lengths.

    The prefix sum starts at 0 and has one more entry than there are sequences,
    as in FAQ Q8's ``[0, 100, 300, 450]`` for lengths ``[100, 200, 150]``.
    """
    cu_q = [0]
    for n in seqlens_q:
        cu_q.append(cu_q[-1] + int(n))
    cu_k = [0]
    for n in seqlens_k:
        cu_k.append(cu_k[-1] + int(n))
    g = torch.Generator().manual_seed(int(seed))
    q = randn((cu_q[-1], h_q, d), dtype=dtype, generator=g)
    k = randn((cu_k[-1], h_kv, d), dtype=dtype, generator=g)
    v = randn((cu_k[-1], h_kv, d), dtype=dtype, generator=g)
    return (q, k, v, torch.tensor(cu_q, dtype=torch.int32), torch.tensor(cu_k, dtype=torch.int32))


def kvcache(b, s_cache, h_q, h_kv, d, seed, dtype=torch.bfloat16):
    """q (b, 1, h_q, d), k_cache and v_cache (b, s_cache, h_kv, d), drawn in that order."""
    g = torch.Generator().manual_seed(int(seed))
    q = randn((b, 1, h_q, d), dtype=dtype, generator=g)
    kc = randn((b, s_cache, h_kv, d), dtype=dtype, generator=g)
    vc = randn((b, s_cache, h_kv, d), dtype=dtype, generator=g)
    return q, kc, vc


def kv_new(b, s_new, h_kv, d, seed, dtype=torch.bfloat16):
    """New tokens for a cache append: one (b, s_new, 2, h_kv, d) draw, returned as
    the strided views k_new = [:, :, 0] and v_new = [:, :, 1]."""
    g = torch.Generator().manual_seed(int(seed))
    kv = randn((b, s_new, 2, h_kv, d), dtype=dtype, generator=g)
    return kv[:, :, 0], kv[:, :, 1]


@dataclass(frozen=True)
class Workload:
    """A named attention shape.  ``kind`` is 'dense', 'qkvpacked', 'varlen' or 'decode'."""
    name: str
    kind: str
    batch: int
    seqlen_q: int
    seqlen_k: int
    heads_q: int
    heads_kv: int
    head_dim: int
    dtype: str
    seed: int
    causal: bool = False
    window: tuple = (-1, -1)
    softcap: float = 0.0
    seqlens: tuple = field(default=())
    cache_seqlens: tuple = field(default=())
    num_splits: int = 0


WORKLOADS = {
    "tiny": Workload("tiny", "dense", 1, 64, 64, 4, 4, 64, "fp16", seed=1),
    "causal_prefill": Workload("causal_prefill", "qkvpacked", 2, 1024, 1024, 16, 16, 128, "bf16",
                               seed=2, causal=True),
    "hdim64": Workload("hdim64", "dense", 2, 1024, 1024, 32, 32, 64, "fp16", seed=31),
    "hdim128": Workload("hdim128", "dense", 2, 1024, 1024, 16, 16, 128, "fp16", seed=32),
    "hdim256": Workload("hdim256", "dense", 2, 1024, 1024, 8, 8, 256, "fp16", seed=33),
    "varlen_gqa": Workload("varlen_gqa", "varlen", 3, 200, 200, 32, 8, 128, "bf16", seed=41,
                           causal=True, window=(256, 0), softcap=50.0, seqlens=(100, 200, 150)),
    "cross": Workload("cross", "dense", 2, 512, 2048, 32, 8, 128, "bf16", seed=42),
    "long_prefill": Workload("long_prefill", "dense", 1, 16384, 16384, 16, 16, 128, "bf16",
                             seed=51, causal=True),
    "decode": Workload("decode", "decode", 8, 1, 16384, 32, 8, 128, "bf16", seed=52,
                       cache_seqlens=(16384,) * 8, num_splits=0),
}


def flops(w: Workload) -> float:
    """The pages' FLOP count, 4*b*h*s_q*s_k*d, halved for causal (FAQ Q16).

    Varlen sums per sequence; decode uses the non-causal count over cache_seqlens.
    """
    if w.kind == "varlen":
        tot = sum(4.0 * w.heads_q * n * n * w.head_dim for n in w.seqlens)
        return tot / 2 if w.causal else tot
    if w.kind == "decode":
        return sum(4.0 * w.heads_q * 1 * n * w.head_dim for n in w.cache_seqlens)
    f = 4.0 * w.batch * w.heads_q * w.seqlen_q * w.seqlen_k * w.head_dim
    return f / 2 if w.causal else f


def backward_flops(w: Workload) -> float:
    """FLOPs of the recomputing backward: five products per visible (row, key)
    pair and head (S again, dP = dO V^T, dV, dK and dQ) against the forward's
    two, so 2.5 times ``flops`` (the forward's count extended by the number of
    products; "FlashAttention完整说明", section 二.2 names them)."""
    return 2.5 * flops(w)


def algorithmic_bytes(w: Workload) -> int:
    """Q, K, V read once; O written once (storage dtype); LSE written once (fp32)."""
    e = 2
    d = w.head_dim
    if w.kind == "varlen":
        tq = sum(w.seqlens)
        return e * d * (tq * w.heads_q * 2 + tq * w.heads_kv * 2) + 4 * tq * w.heads_q
    if w.kind == "decode":
        kv = sum(w.cache_seqlens) * w.heads_kv * d * e * 2
        return kv + w.batch * w.heads_q * d * e * 2 + 4 * w.batch * w.heads_q
    qo = w.batch * w.seqlen_q * w.heads_q * d * e * 2
    kv = w.batch * w.seqlen_k * w.heads_kv * d * e * 2
    return qo + kv + 4 * w.batch * w.heads_q * w.seqlen_q
