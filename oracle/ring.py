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
(Q chunk i holds Cq = Sq / P queries, K/V chunk j holds Ckv = Skv / P keys at
positions [j Ckv, (j+1) Ckv)); when Q is shorter than K/V (new tokens against a
cached context) the queries are the last Sq positions of the K/V sequence, so
Q chunk i starts at position Skv - Sq + i Cq; the ring sends from rank r-1 to
rank r; under a causal mask a (q chunk, kv chunk) pair whose first key lies
after its last query sees nothing and is skipped; in Pass-Q each partial is
handed to the owner of its Q chunk, which merges in arrival order.

The pages give no rule for choosing between the two variants.  The rule here
counts the bytes each variant moves between ranks (every chunk makes P - 1
hops around the ring; in Pass-Q every partial computed away from its Q chunk's
owner also travels back to it as fp32 O plus fp32 LSE) and takes the smaller,
Pass-KV on a tie.
"""
from __future__ import annotations

import torch

from .attention import merge, partial_attention

PASS_KV = "pass_kv"
PASS_Q = "pass_q"


def _lengths(P: int, q_len, kv_len):
    """Per-chunk lengths and the position of the first query; equal lengths by default."""
    if q_len is None and kv_len is None:
        q_len = kv_len = P  # any equal lengths give the same pairs
    assert q_len is not None and kv_len is not None and q_len <= kv_len
    assert q_len % P == 0 and kv_len % P == 0, "chunks must be equal"
    return q_len // P, kv_len // P, kv_len - q_len


def pair_visible(i: int, j: int, P: int, causal: bool = True, q_len=None, kv_len=None) -> bool:
    """Whether some key of K/V chunk j is visible to some query of Q chunk i."""
    Cq, Ckv, q0 = _lengths(P, q_len, kv_len)
    if not causal:
        return True
    last_query = q0 + (i + 1) * Cq - 1
    first_key = j * Ckv
    return first_key <= last_query


def schedule(P: int, order: str, causal: bool = True, q_len=None, kv_len=None):
    """Work items per ring step.

    Returns a list of P steps; step s is a list of ``(rank, q_chunk, kv_chunk)``
    in rank order, with pairs that see nothing under the causal mask left out.
    ``q_len`` / ``kv_len`` (default: equal) are the sequence lengths of Q and K/V.
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
            if not pair_visible(qi, kj, P, causal, q_len, kv_len):
                continue
            items.append((r, qi, kj))
        steps.append(items)
    return steps


def arrival_order(P: int, order: str, causal: bool = True, q_len=None, kv_len=None):
    """For each Q chunk i, the KV chunks of its partials in the order they arrive."""
    arrivals = [[] for _ in range(P)]
    for items in schedule(P, order, causal, q_len, kv_len):
        for _, qi, kj in items:
            arrivals[qi].append(kj)
    return arrivals


def _chunk(x, c: int, C: int):
    return x[:, c * C:(c + 1) * C]


def ring_attention(q, k, v, P: int, order: str = PASS_KV, causal: bool = True, merge_order=None):
    """Simulate the ring on one host: every partial of every step, then per-owner merges.

    q [B, Sq, Hq, D] holds the last Sq positions of the sequence whose K/V are
    k, v [B, Skv, Hkv, D] (Sq <= Skv; equal lengths are a full prefill).
    ``merge_order`` optionally overrides the arrival order (a list of KV-chunk
    lists per Q chunk); any order gives the same result up to rounding.
    Returns (O [B,Sq,Hq,D], lse [B,Sq,Hq]) in float64.
    """
    Sq, Skv = q.shape[1], k.shape[1]
    Cq, Ckv, q0 = _lengths(P, Sq, Skv)
    parts = {}
    for items in schedule(P, order, causal, Sq, Skv):
        for _, qi, kj in items:
            parts[(qi, kj)] = partial_attention(_chunk(q, qi, Cq), _chunk(k, kj, Ckv), _chunk(v, kj, Ckv),
                                                q0 + qi * Cq, kj * Ckv, causal)
    arrivals = merge_order if merge_order is not None else arrival_order(P, order, causal, Sq, Skv)
    outs, lses = [], []
    for qi in range(P):
        os_, ls_ = zip(*(parts[(qi, kj)] for kj in arrivals[qi]))
        o, l = merge(list(os_), list(ls_))
        outs.append(o)
        lses.append(l)
    return torch.cat(outs, dim=1), torch.cat(lses, dim=1)


def exchange_bytes(P: int, order: str, causal: bool, B: int, q_len: int, kv_len: int, Hq: int, Hkv: int,
                   D: int, elem_bytes: int = 2) -> int:
    """Bytes a P-rank ring moves between ranks, by walking its steps.

    At every step after the first, each rank receives the chunk its neighbour
    held: K and V of one chunk (Pass-KV) or one Q chunk (Pass-Q), ``elem_bytes``
    per element.  In Pass-Q every item computed on a rank other than its Q
    chunk's owner sends its partial back: fp32 O plus fp32 LSE per query row and
    head.
    """
    Cq, Ckv, _ = _lengths(P, q_len, kv_len)
    total = 0
    for s in range(1, P):
        for r in range(P):
            if order == PASS_KV:
                total += 2 * B * Ckv * Hkv * D * elem_bytes
            else:
                total += B * Cq * Hq * D * elem_bytes
    if order == PASS_Q:
        for items in schedule(P, order, causal, q_len, kv_len):
            for r, qi, _ in items:
                if r != qi:
                    total += B * Cq * Hq * (D + 1) * 4
    return total


def select_order(P: int, causal: bool, B: int, q_len: int, kv_len: int, Hq: int, Hkv: int, D: int,
                 elem_bytes: int = 2) -> str:
    """The ring order that moves fewer bytes (Pass-KV on a tie)."""
    kv = exchange_bytes(P, PASS_KV, causal, B, q_len, kv_len, Hq, Hkv, D, elem_bytes)
    qb = exchange_bytes(P, PASS_Q, causal, B, q_len, kv_len, Hq, Hkv, D, elem_bytes)
    return PASS_Q if qb < kv else PASS_KV


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


def cp_decode(q, k_shards, v_shards, lengths):
    """Decode of new query tokens against a KV cache sharded over CP ranks.

    The prefill builds each layer's KV cache and decode reads it ("Why
    Parallelism Defines LLM Serving Cost"); with the cache cut across CP ranks,
    every rank attends the new query against the first ``lengths[r]`` rows of
    its own shard and the per-rank partials are merged (shard order).  The new
    token comes after every cached key, so it sees all of them.
    q [B, 1, Hq, D]; shard r: k_shards[r], v_shards[r] [B, cap_r, Hkv, D].
    Returns (O [B,1,Hq,D], lse [B,1,Hq]) in float64.
    """
    assert q.shape[1] == 1 and len(k_shards) == len(v_shards) == len(lengths) >= 1
    parts = [partial_attention(q, ks[:, :n], vs[:, :n], 0, 0, causal=False)
             for ks, vs, n in zip(k_shards, v_shards, lengths)]
    return merge([p[0] for p in parts], [p[1] for p in parts])
