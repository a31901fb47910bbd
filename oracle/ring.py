"""Ring schedules and ring-attention simulations for the oracle (fp64, CPU).

TEST INFRASTRUCTURE ONLY; see ``oracle/attention.py``.

The pages ("Context Parallelism for Million-Token Contexts") describe two ring
variants over a sequence split across P ranks:

* Pass-KV: rank r keeps its local Q chunk and, at ring step s, holds the K/V
  chunk that started on rank (r - s) mod P (K/V move one rank along the ring
  per step, from rank r-1 to rank r);
* Pass-Q: the same partitioning, but Q chunks travel: at step s rank r holds
  the Q chunk that started on rank (r - s) mod P and attends it against its own
  K/V chunk.

Readings taken where the pages are silent: chunks are contiguous and equal
(chunk c holds tokens [c*C, (c+1)*C)); the ring sends from rank r-1 to rank r;
under a causal mask a (q chunk i, kv chunk j) pair with j > i sees no key and
is skipped; in Pass-Q each partial is handed to the owner of its Q chunk, which
merges in arrival order.
"""
from __future__ import annotations

import torch

from .attention import merge, partial_attention

PASS_KV = "pass_kv"
PASS_Q = "pass_q"


def schedule(P: int, order: str, causal: bool = True):
    """Work items per ring step.

    Returns a list of P steps; step s is a list of ``(rank, q_chunk, kv_chunk)``
    in rank order, with causally empty pairs (kv_chunk > q_chunk) left out.
    """
    steps = []
    for s in range(P):
        items = []
        for r in range(P):
            other = (r - s) % P
            if order == PASS_KV:
                qi, kj = r, other
            elif order == PASS_Q:
                qi, kj = other, r
            else:
                raise ValueError(f"unknown ring order {order!r}")
            if causal and kj > qi:
                continue
            items.append((r, qi, kj))
        steps.append(items)
    return steps


def arrival_order(P: int, order: str, causal: bool = True):
    """For each Q chunk i, the KV chunks of its partials in the order they arrive."""
    arrivals = [[] for _ in range(P)]
    for items in schedule(P, order, causal):
        for _, qi, kj in items:
            arrivals[qi].append(kj)
    return arrivals


def _chunk(x, c: int, C: int):
    return x[:, c * C:(c + 1) * C]


def ring_attention(q, k, v, P: int, order: str = PASS_KV, causal: bool = True, merge_order=None):
    """Simulate the ring on one host: every partial of every step, then per-owner merges.

    ``merge_order`` optionally overrides the arrival order (a list of KV-chunk
    lists per Q chunk); any order gives the same result up to rounding.
    Returns (O [B,S,Hq,D], lse [B,S,Hq]) in float64.
    """
    S = q.shape[1]
    assert S % P == 0 and k.shape[1] == S, "ring needs equal chunks of one sequence"
    C = S // P
    parts = {}
    for items in schedule(P, order, causal):
        for _, qi, kj in items:
            parts[(qi, kj)] = partial_attention(_chunk(q, qi, C), _chunk(k, kj, C), _chunk(v, kj, C),
                                                qi * C, kj * C, causal)
    arrivals = merge_order if merge_order is not None else arrival_order(P, order, causal)
    outs, lses = [], []
    for qi in range(P):
        os_, ls_ = zip(*(parts[(qi, kj)] for kj in arrivals[qi]))
        o, l = merge(list(os_), list(ls_))
        outs.append(o)
        lses.append(l)
    return torch.cat(outs, dim=1), torch.cat(lses, dim=1)


def splitkv_decode(q, k, v, n_chunks: int, causal: bool = True):
    """Split-KV decode: one new query token per sequence against a cached K/V.

    The query sits at position Skv - 1 (it sees every cached key); the cache is
    cut into ``n_chunks`` equal chunks, each giving a partial, merged in chunk
    order.  Returns (O [B,1,Hq,D], lse [B,1,Hq]) in float64.
    """
    Skv = k.shape[1]
    assert q.shape[1] == 1 and Skv % n_chunks == 0
    C = Skv // n_chunks
    parts = [partial_attention(q, _chunk(k, c, C), _chunk(v, c, C), Skv - 1, c * C, causal)
             for c in range(n_chunks)]
    return merge([p[0] for p in parts], [p[1] for p in parts])
