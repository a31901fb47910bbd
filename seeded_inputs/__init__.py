"""Seeded synthetic inputs for the context-parallel attention workloads.

This module is shared by the oracle tests, the GPU parity tests, ``smoke()`` and
the bench.  It holds the workload shapes and the random draws only: no step of
the attention method (no scores, softmax, masking or merging) lives here, so the
oracle and the HIP path stay independent while consuming identical inputs.

The pages on context parallelism say nothing about inputs: they report
whole-model prefills that need trained weights.  These synthetic workloads stand
in for them at one GPU's share of such a layer, with shapes, chunk counts,
dtypes and seeds fixed in the workload table below: Q, K and V entries i.i.d.
N(0, 1), one seed per workload, rounded to bf16 (round to nearest even) except
the fp32 tiny case.

Stream definition (so that any machine reproduces the same tensors):
each tensor is flattened in [B, S, H, D] order and cut into chunks of
2**24 elements; chunk ``c`` of tensor ``t`` (0 = Q, 1 = K, 2 = V) holds the
first elements of ``numpy.random.Generator(PCG64(SeedSequence(entropy=seed,
spawn_key=(t, c)))).standard_normal(dtype=float32)``.  Chunks are independent
streams, so they can be drawn on several host threads.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK_ELEMS = 1 << 24
TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    """One synthetic workload.  ``Sq``/``Skv`` are per-sequence lengths."""

    name: str
    kind: str  # "prefill" (ring over CP chunks) or "decode" (split-KV)
    B: int
    Hq: int
    Hkv: int
    D: int
    Sq: int
    Skv: int
    n_chunks: int
    dtype: str  # "f32" or "bf16"
    seed: int
    orders: tuple = ("pass_kv",)
    causal: bool = True
    note: str = field(default="", compare=False)

    @property
    def chunk(self) -> int:
        return (self.Skv if self.kind == "decode" else self.Sq) // self.n_chunks

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def q_shape(self):
        return (self.B, self.Sq, self.Hq, self.D)

    def kv_shape(self):
        return (self.B, self.Skv, self.Hkv, self.D)

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs the causal mask leaves visible, per (batch, head)."""
        if self.kind == "decode":
            return self.Skv  # the new token sees the whole cache
        if not self.causal:
            return self.Sq * self.Skv
        assert self.Sq == self.Skv
        return self.Sq * (self.Sq + 1) // 2

    def flops(self) -> float:
        """Unmasked FLOPs: 2*D for Q.K and 2*D for P.V per visible pair and query head."""
        return 4.0 * self.D * self.Hq * self.B * self.visible_pairs()


# The five workloads: a tiny fp32 case, a GQA prefill at one GPU's tensor-parallel
# share of a 405B-shaped layer, a split-KV decode, a 128K-token prefill and a
# 1M-token prefill.  Shapes, chunk counts, dtypes and seeds are fixed here.
WORKLOADS = {
    "tiny_f32_s512_p4": Workload(
        "tiny_f32_s512_p4", "prefill", 1, 1, 1, 64, 512, 512, 4, "f32", 0, ("pass_kv",),
        note="compare with unchunked attention"),
    "gqa16_bf16_s8k_p8": Workload(
        "gqa16_bf16_s8k_p8", "prefill", 1, 16, 1, 128, 8192, 8192, 8, "bf16", 1, ("pass_kv",)),
    "decode_b128_kv32k_p8": Workload(
        "decode_b128_kv32k_p8", "decode", 128, 16, 1, 128, 1, 32768, 8, "bf16", 2, ("splitkv",)),
    "prefill_bf16_s128k_p16": Workload(
        "prefill_bf16_s128k_p16", "prefill", 1, 16, 1, 128, 131072, 131072, 16, "bf16", 3,
        ("pass_kv", "pass_q")),
    "prefill_bf16_s1m_p8": Workload(
        "prefill_bf16_s1m_p8", "prefill", 1, 16, 1, 128, 1048576, 1048576, 8, "bf16", 4,
        ("pass_kv",)),
}
WORKLOAD_ORDER = list(WORKLOADS)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def draw_tensor(seed: int, tensor_id: int, shape, dtype: torch.dtype) -> torch.Tensor:
    """Draw one tensor of the stream described in the module docstring (host memory)."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=dtype)
    n_chunks = (n + CHUNK_ELEMS - 1) // CHUNK_ELEMS

    def fill(c: int) -> None:
        lo = c * CHUNK_ELEMS
        cnt = min(CHUNK_ELEMS, n - lo)
        gen = np.random.Generator(
            np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=(tensor_id, c))))
        vals = torch.from_numpy(gen.standard_normal(cnt, dtype=np.float32))
        out[lo:lo + cnt] = vals.to(dtype)  # bf16: round to nearest even

    if n_chunks <= 1:
        for c in range(n_chunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out.view(*shape)


def make_qkv(w: Workload, dtype: torch.dtype | None = None):
    """Q, K, V host tensors of workload ``w`` in [B, S, H, D] layout."""
    dt = w.torch_dtype if dtype is None else dtype
    q = draw_tensor(w.seed, TENSOR_Q, w.q_shape(), dt)
    k = draw_tensor(w.seed, TENSOR_K, w.kv_shape(), dt)
    v = draw_tensor(w.seed, TENSOR_V, w.kv_shape(), dt)
    return q, k, v


def sampled_rows(w: Workload, n_rows: int = 64) -> np.ndarray:
    """Query positions checked on workloads too large for the full oracle.

    Always includes the first and last token and both sides of every chunk
    boundary; the rest are drawn without replacement from a second stream of
    the workload seed (``SeedSequence(entropy=seed, spawn_key=(3,))``).
    """
    S, C = w.Sq, w.chunk
    fixed = {0, S - 1}
    for c in range(1, w.n_chunks):
        fixed.update((c * C - 1, c * C))
    fixed = sorted(p for p in fixed if 0 <= p < S)
    rest = max(0, n_rows - len(fixed))
    gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=w.seed, spawn_key=(3,))))
    pool = np.setdiff1d(np.arange(S, dtype=np.int64), np.asarray(fixed, dtype=np.int64))
    drawn = gen.choice(pool, size=min(rest, pool.size), replace=False) if rest else np.empty(0, np.int64)
    return np.sort(np.concatenate([np.asarray(fixed, dtype=np.int64), drawn.astype(np.int64)]))
