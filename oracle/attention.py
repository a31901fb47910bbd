"""fp64 CPU oracle for context-parallel causal attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module;
only the tests, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg
call it.  It shares no code with the HIP library.

What it computes is the plain definition of exact softmax attention, written
out in float64 with torch CPU primitives (matmul, max, exp, log, sum).  The
pages (Meta's "Scaling LLM Inference: Innovations in Tensor Parallelism,
Context Parallelism, and Expert Parallelism", and the reader notes on it) fix
only the structure: the sequence is divided among CP ranks, every rank
produces Q, K and V for its own tokens, and either its K/V (Pass-KV) or its Q
(Pass-Q) moves from rank to rank until each query has met the whole context
("Context Parallelism for Million-Token Contexts"; the reader notes' section
"The communication bottleneck across all three axes" adds that the K/V
pieces circulate on a ring and the per-step results combine into the
full-context output).  Where the pages are silent this oracle takes the
plainest reading:

* causal mask with the diagonal included: key position ``kv_offset + j`` is
  visible to query position ``q_offset + i`` iff ``kv_offset + j <= q_offset + i``;
* scale ``1/sqrt(D)``;
* grouped-query heads: query head ``h`` reads KV head ``h // (Hq // Hkv)``;
* LSE is the natural log of the sum of exponentials of the scaled scores;
* a row that sees no key has ``lse = -inf`` and ``O = 0``;
* partial results combine by the exact log-sum-exp merge
  ``O = sum_c exp(lse_c - M) O_c / sum_c exp(lse_c - M)``, ``M = max_c lse_c``.

Inputs are the exact values the GPU consumes (bf16 or fp32), upcast to fp64.
Layout is [B, S, H, D] for Q/K/V/O and [B, S, H] for LSE.
"""
from __future__ import annotations

import math

import torch

F64 = torch.float64
NEG_INF = float("-inf")


def _check(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> tuple[int, int, int, int, int, int]:
    assert q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "expect [B, S, H, D]"
    B, Sq, Hq, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    assert v.shape == k.shape and Bk == B and Dk == D
    assert Hq % Hkv == 0, "query heads must be a multiple of KV heads"
    return B, Sq, Hq, D, Sk, Hkv


def visible_mask(Sq: int, Sk: int, q_offset: int, kv_offset: int, causal: bool) -> torch.Tensor:
    """Boolean [Sq, Sk]: True where key j is visible to query i."""
    if not causal:
        return torch.ones(Sq, Sk, dtype=torch.bool)
    qpos = q_offset + torch.arange(Sq, dtype=torch.int64).unsqueeze(1)
    kpos = kv_offset + torch.arange(Sk, dtype=torch.int64).unsqueeze(0)
    return kpos <= qpos


def partial_attention(q, k, v, q_offset: int = 0, kv_offset: int = 0, causal: bool = True,
                      row_block: int = 4096):
    """Attention of a Q block against one K/V block at global offsets.

    Returns ``(O, lse)``: O [B, Sq, Hq, D] float64 normalised by the block's own
    softmax denominator, lse [B, Sq, Hq] float64.  ``row_block`` bounds the
    memory of the score matrix only; every row is computed independently.
    """
    B, Sq, Hq, D, Sk, Hkv = _check(q, k, v)
    G = Hq // Hkv
    alpha = 1.0 / math.sqrt(D)
    out = torch.zeros(B, Sq, Hq, D, dtype=F64)
    lse = torch.full((B, Sq, Hq), NEG_INF, dtype=F64)
    if Sq == 0 or Sk == 0:
        return out, lse
    for b in range(B):
        for g in range(Hkv):
            kk = k[b, :, g, :].to(F64)  # [Sk, D]
            vv = v[b, :, g, :].to(F64)
            for h in range(g * G, (g + 1) * G):  # the query heads that read KV head g
                for r0 in range(0, Sq, row_block):
                    r1 = min(Sq, r0 + row_block)
                    qq = q[b, r0:r1, h, :].to(F64)  # [R, D]
                    s = alpha * (qq @ kk.T)  # scaled scores [R, Sk]
                    vis = visible_mask(r1 - r0, Sk, q_offset + r0, kv_offset, causal)
                    s = s.masked_fill(~vis, NEG_INF)
                    m = s.max(dim=1, keepdim=True).values  # -inf for rows that see nothing
                    has = torch.isfinite(m).squeeze(1)
                    m_safe = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
                    l = torch.exp(s - m_safe).sum(dim=1, keepdim=True)
                    row_lse = m_safe + torch.log(l)  # log of zero -> -inf for empty rows
                    p = torch.exp(s - torch.where(has.unsqueeze(1), row_lse, torch.zeros_like(row_lse)))
                    o = p @ vv
                    o[~has] = 0.0
                    row_lse[~has] = NEG_INF
                    out[b, r0:r1, h, :] = o
                    lse[b, r0:r1, h] = row_lse.squeeze(1)
    return out, lse


def full_attention(q, k, v, causal: bool = True, row_block: int = 4096):
    """Unchunked attention over the whole sequence (both offsets zero)."""
    return partial_attention(q, k, v, 0, 0, causal, row_block)


def attention_rows(q_rows, k, v, positions, causal: bool = True):
    """Full-context attention for selected query rows.

    ``q_rows`` [B, R, Hq, D] holds the queries at global ``positions`` (length R);
    K/V hold the whole sequence from position 0.  Row ``r`` attends keys
    ``0..positions[r]`` (causal) or all keys.  Returns (O [B,R,Hq,D], lse [B,R,Hq]).
    """
    B, R, Hq, D = q_rows.shape
    k = k.to(F64)  # convert the long K/V once, not once per row
    v = v.to(F64)
    out = torch.zeros(B, R, Hq, D, dtype=F64)
    lse = torch.full((B, R, Hq), NEG_INF, dtype=F64)
    for r, pos in enumerate(list(int(p) for p in positions)):
        kv_len = pos + 1 if causal else k.shape[1]
        o, l = partial_attention(q_rows[:, r:r + 1], k[:, :kv_len], v[:, :kv_len], pos, 0, causal)
        out[:, r] = o[:, 0]
        lse[:, r] = l[:, 0]
    return out, lse


def merge(partials, lses):
    """Exact log-sum-exp merge of partial results, taken in the order given.

    ``partials``: sequence of O tensors [..., D]; ``lses``: matching [...] tensors.
    Returns (O, lse) in float64.  A row whose partials all have lse = -inf
    merges to O = 0, lse = -inf; a partial with lse = -inf contributes nothing.
    """
    assert len(partials) == len(lses) and len(partials) >= 1
    L = torch.stack([x.to(F64) for x in lses])  # [n, ...]
    O = torch.stack([x.to(F64) for x in partials])  # [n, ..., D]
    M = L.max(dim=0).values
    has = torch.isfinite(M)
    M_safe = torch.where(has, M, torch.zeros_like(M))
    w = torch.exp(L - M_safe)  # 0 for -inf partials
    den = w.sum(dim=0)
    num = (w.unsqueeze(-1) * O).sum(dim=0)
    out = torch.where(has.unsqueeze(-1), num / torch.where(has, den, torch.ones_like(den)).unsqueeze(-1),
                      torch.zeros_like(num))
    lse = torch.where(has, M_safe + torch.log(den), torch.full_like(M, NEG_INF))
    return out, lse
