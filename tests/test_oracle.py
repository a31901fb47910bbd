"""Pins for the fp64 oracle, checked against things other than itself.

Each pin is a function of a candidate attention (or merge) implementation, so
the same pins are run against planted mistakes at the bottom of this file to
show that a plausible slip (wrong scale, diagonal dropped, transposed operand,
wrong GQA head, wrong LSE base, dropped merge term) fails at least one of them.
"""
import itertools
import math
import os
import random

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from oracle import PASS_KV, PASS_Q

F64 = torch.float64
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(shape, seed, dtype=F64):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=F64).to(dtype)


# ----------------------------------------------------------------------------
# Independent references
# ----------------------------------------------------------------------------

def brute_partial(q, k, v, q_offset, kv_offset, causal):
    """Pure-Python loops: softmax as exp(score)/sum(exp(score)), no max shift."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    ql, kl, vl = q.tolist(), k.tolist(), v.tolist()
    out = [[[[0.0] * D for _ in range(Hq)] for _ in range(Sq)] for _ in range(B)]
    lse = [[[float("-inf")] * Hq for _ in range(Sq)] for _ in range(B)]
    for b in range(B):
        for i in range(Sq):
            for h in range(Hq):
                g = (h * Hkv) // Hq
                ws = []
                for j in range(Sk):
                    if causal and kv_offset + j > q_offset + i:
                        continue
                    dot = math.fsum(ql[b][i][h][d] * kl[b][j][g][d] for d in range(D))
                    ws.append((math.exp(dot / math.sqrt(D)), j))
                if not ws:
                    continue
                Z = math.fsum(w for w, _ in ws)
                lse[b][i][h] = math.log(Z)
                for d in range(D):
                    out[b][i][h][d] = math.fsum(w * vl[b][j][g][d] for w, j in ws) / Z
    return torch.tensor(out, dtype=F64), torch.tensor(lse, dtype=F64)


def sdpa_reference(q, k, v, q_offset, kv_offset, causal):
    """torch's fp64 scaled_dot_product_attention with an explicit boolean mask (O only)."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    rep = Hq // Hkv
    qt = q.permute(0, 2, 1, 3).contiguous()
    kt = k.repeat_interleave(rep, dim=2).permute(0, 2, 1, 3).contiguous()
    vt = v.repeat_interleave(rep, dim=2).permute(0, 2, 1, 3).contiguous()
    if causal:
        qpos = torch.arange(Sq).unsqueeze(1) + q_offset
        kpos = torch.arange(Sk).unsqueeze(0) + kv_offset
        mask = (kpos <= qpos)
    else:
        mask = torch.ones(Sq, Sk, dtype=torch.bool)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return o.permute(0, 2, 1, 3)


# ----------------------------------------------------------------------------
# Pins, as functions of a candidate partial-attention implementation
# ----------------------------------------------------------------------------

def pin_brute_force(fn):
    cases = [
        # (B, Sq, Sk, Hq, Hkv, D, q_off, kv_off, causal)
        (1, 5, 7, 2, 1, 4, 3, 0, True),
        (2, 4, 4, 4, 2, 8, 0, 0, True),
        (1, 6, 5, 3, 3, 4, 2, 4, True),   # first rows see nothing
        (1, 3, 6, 2, 2, 2, 0, 0, False),
        (1, 4, 4, 2, 1, 4, 0, 8, True),   # whole block masked
    ]
    for n, (B, Sq, Sk, Hq, Hkv, D, qo, ko, causal) in enumerate(cases):
        q, k, v = rand((B, Sq, Hq, D), 10 + n), rand((B, Sk, Hkv, D), 20 + n), rand((B, Sk, Hkv, D), 30 + n)
        o, l = fn(q, k, v, qo, ko, causal)
        bo, bl = brute_partial(q, k, v, qo, ko, causal)
        assert torch.allclose(o, bo, atol=1e-12, rtol=0), f"O mismatch in brute-force case {n}"
        assert torch.equal(torch.isinf(l), torch.isinf(bl)), f"masked rows differ in case {n}"
        fin = torch.isfinite(bl)
        assert torch.allclose(l[fin], bl[fin], atol=1e-12, rtol=0), f"LSE mismatch in case {n}"


def pin_sdpa(fn):
    for n, (Sq, Sk, Hq, Hkv, D, qo, ko, causal) in enumerate([
            (33, 33, 4, 1, 16, 0, 0, True), (17, 40, 8, 2, 32, 23, 0, True), (9, 12, 2, 2, 64, 0, 0, False)]):
        q, k, v = rand((2, Sq, Hq, D), 40 + n), rand((2, Sk, Hkv, D), 50 + n), rand((2, Sk, Hkv, D), 60 + n)
        o, l = fn(q, k, v, qo, ko, causal)
        ref = sdpa_reference(q, k, v, qo, ko, causal)
        assert torch.allclose(o, ref, atol=1e-12, rtol=0), f"SDPA mismatch in case {n}"
        # LSE against torch.logsumexp over the explicitly masked score matrix
        rep = Hq // Hkv
        s = torch.einsum("bihd,bjhd->bhij", q, k.repeat_interleave(rep, dim=2)) / math.sqrt(D)
        if causal:
            vis = (torch.arange(Sk).unsqueeze(0) + ko) <= (torch.arange(Sq).unsqueeze(1) + qo)
            s = s.masked_fill(~vis, float("-inf"))
        ref_l = torch.logsumexp(s, dim=-1).permute(0, 2, 1)
        assert torch.allclose(l, ref_l, atol=1e-12, rtol=0), f"logsumexp mismatch in case {n}"


def pin_zero_query(fn):
    """Q = 0: every visible score is 0, so O is the mean of the visible V rows and lse = ln(count)."""
    Sq, Sk, D = 12, 12, 8
    q = torch.zeros(1, Sq, 2, D, dtype=F64)
    k, v = rand((1, Sk, 1, D), 70), rand((1, Sk, 1, D), 71)
    o, l = fn(q, k, v, 0, 0, True)
    for i in range(Sq):
        cnt = i + 1
        assert abs(l[0, i, 0].item() - math.log(cnt)) < 1e-12, "lse of a zero query must be ln(#visible)"
        mean = v[0, :cnt, 0, :].mean(dim=0)
        assert torch.allclose(o[0, i, 0], mean, atol=1e-12, rtol=0)
        assert torch.allclose(o[0, i, 1], mean, atol=1e-12, rtol=0)


def pin_first_row(fn):
    """Causal row 0 at offset 0 sees key 0 only: O = V0, lse = q0.k0 / sqrt(D)."""
    D = 16
    q, k, v = rand((1, 4, 1, D), 80), rand((1, 4, 1, D), 81), rand((1, 4, 1, D), 82)
    o, l = fn(q, k, v, 0, 0, True)
    assert torch.allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-12, rtol=0)
    expect = float((q[0, 0, 0] * k[0, 0, 0]).sum()) / math.sqrt(D)
    assert abs(l[0, 0, 0].item() - expect) < 1e-12


def pin_golden(fn):
    """Hand-derived 3-token closed form in tests/golden/closed_form_3tok.txt."""
    rows = [list(map(float, ln.split())) for ln in open(os.path.join(GOLDEN, "closed_form_3tok.txt"))
            if ln.strip() and not ln.startswith("#")]
    r2 = math.sqrt(2.0)
    q = torch.tensor([[0.5, 7.0], [r2 * math.log(3.0), 0.0], [0.0, 0.0]], dtype=F64).view(1, 3, 1, 2)
    k = torch.tensor([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]], dtype=F64).view(1, 3, 1, 2)
    v = torch.tensor([[1.0, 0.0], [0.0, 1.0], [2.0, 2.0]], dtype=F64).view(1, 3, 1, 2)
    o, l = fn(q, k, v, 0, 0, True)
    for r, o0, o1, lse in rows:
        r = int(r)
        assert abs(o[0, r, 0, 0].item() - o0) < 1e-12 and abs(o[0, r, 0, 1].item() - o1) < 1e-12
        assert abs(l[0, r, 0].item() - lse) < 1e-12


def pin_peaked(fn):
    """A query aligned with one key far more than the others puts (almost) all weight on it."""
    D = 32
    k = torch.eye(D, dtype=F64)[:8].view(1, 8, 1, D)
    v = rand((1, 8, 1, D), 90)
    q = 40.0 * math.sqrt(D) * torch.eye(D, dtype=F64)[[5]].view(1, 1, 1, D)
    o, _ = fn(q, k, v, 7, 0, True)
    assert torch.allclose(o[0, 0, 0], v[0, 5, 0], atol=1e-12, rtol=0)


def pin_gqa_heads(fn):
    """Query head h must read KV head h // (Hq/Hkv): compare each head with a one-head call."""
    Hq, Hkv, D = 6, 3, 8
    q, k, v = rand((1, 7, Hq, D), 100), rand((1, 7, Hkv, D), 101), rand((1, 7, Hkv, D), 102)
    o, l = fn(q, k, v, 0, 0, True)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        oh, lh = brute_partial(q[:, :, h:h + 1], k[:, :, g:g + 1], v[:, :, g:g + 1], 0, 0, True)
        assert torch.allclose(o[:, :, h:h + 1], oh, atol=1e-12, rtol=0)
        assert torch.allclose(l[:, :, h:h + 1], lh, atol=1e-12, rtol=0)


PARTIAL_PINS = [pin_brute_force, pin_sdpa, pin_zero_query, pin_first_row, pin_golden, pin_peaked,
                pin_gqa_heads]


@pytest.mark.parametrize("pin", PARTIAL_PINS, ids=lambda p: p.__name__)
def test_partial_pins(pin):
    pin(oracle.partial_attention)


# ----------------------------------------------------------------------------
# Invariants of the partial
# ----------------------------------------------------------------------------

def test_empty_rows_and_blocks():
    q, k, v = rand((1, 4, 2, 8), 1), rand((1, 6, 1, 8), 2), rand((1, 6, 1, 8), 3)
    o, l = oracle.partial_attention(q, k, v, 0, 100, True)  # every key in the future
    assert torch.all(torch.isneginf(l)) and torch.all(o == 0)
    o, l = oracle.partial_attention(q[:, :0], k, v, 0, 0, True)
    assert o.shape == (1, 0, 2, 8) and l.shape == (1, 0, 2)


def test_rows_sum_to_one():
    q, k = rand((1, 20, 2, 16), 4), rand((1, 20, 1, 16), 5)
    ones = torch.ones(1, 20, 1, 16, dtype=F64)
    o, l = oracle.partial_attention(q, k, ones, 3, 0, True)
    assert torch.allclose(o, torch.ones_like(o), atol=1e-12, rtol=0)
    # and explicitly: sum_j exp(s_ij - lse_i) == 1
    s = torch.einsum("bihd,bjhd->bhij", q, k.expand(-1, -1, 2, -1)) / 4.0
    vis = oracle.visible_mask(20, 20, 3, 0, True)
    p = torch.exp(s.masked_fill(~vis, float("-inf")) - l.permute(0, 2, 1).unsqueeze(-1))
    assert torch.allclose(p.sum(-1), torch.ones(1, 2, 20, dtype=F64), atol=1e-12, rtol=0)


def test_constant_v_gives_constant_o():
    q, k = rand((1, 16, 4, 8), 6), rand((1, 16, 1, 8), 7)
    v = torch.full((1, 16, 1, 8), -2.5, dtype=F64)
    o, _ = oracle.partial_attention(q, k, v, 0, 0, True)
    assert torch.allclose(o, torch.full_like(o, -2.5), atol=1e-12, rtol=0)


def test_causality_future_perturbation():
    q, k, v = rand((1, 24, 2, 8), 8), rand((1, 24, 1, 8), 9), rand((1, 24, 1, 8), 10)
    o, l = oracle.full_attention(q, k, v)
    for cut in (0, 5, 17, 23):
        k2, v2 = k.clone(), v.clone()
        k2[:, cut + 1:] = rand(k2[:, cut + 1:].shape, 11 + cut)
        v2[:, cut + 1:] = rand(v2[:, cut + 1:].shape, 12 + cut)
        o2, l2 = oracle.full_attention(q, k2, v2)
        assert torch.equal(o[:, :cut + 1], o2[:, :cut + 1]) and torch.equal(l[:, :cut + 1], l2[:, :cut + 1])
        if cut + 1 < 24:
            assert not torch.allclose(o[:, cut + 1:], o2[:, cut + 1:])


def test_attention_rows_match_full():
    q, k, v = rand((1, 40, 3, 8), 13), rand((1, 40, 3, 8), 14), rand((1, 40, 3, 8), 15)
    o, l = oracle.full_attention(q, k, v)
    pos = [0, 7, 19, 39]
    orow, lrow = oracle.attention_rows(q[:, pos], k, v, pos)
    assert torch.allclose(orow, o[:, pos], atol=1e-12, rtol=0)
    assert torch.allclose(lrow, l[:, pos], atol=1e-12, rtol=0)


def test_row_blocking_is_invisible():
    q, k, v = rand((1, 50, 2, 8), 16), rand((1, 50, 1, 8), 17), rand((1, 50, 1, 8), 18)
    o1, l1 = oracle.partial_attention(q, k, v, 0, 0, True, row_block=7)
    o2, l2 = oracle.partial_attention(q, k, v, 0, 0, True, row_block=4096)
    assert torch.allclose(o1, o2, atol=1e-13, rtol=0) and torch.allclose(l1, l2, atol=1e-13, rtol=0)


# ----------------------------------------------------------------------------
# Merge and ring pins
# ----------------------------------------------------------------------------

def _chunk_pieces(q, k, v, bounds, causal=True):
    parts = []
    for lo, hi in bounds:
        parts.append(oracle.partial_attention(q, k[:, lo:hi], v[:, lo:hi], 0, lo, causal))
    return parts


def pin_merge_partition(merge_fn):
    """Merging partials over any partition of the keys equals attention over all keys."""
    q, k, v = rand((1, 30, 2, 8), 200), rand((1, 30, 1, 8), 201), rand((1, 30, 1, 8), 202)
    full_o, full_l = oracle.full_attention(q, k, v)
    rng = random.Random(5)
    for bounds in ([(0, 30)], [(0, 10), (10, 30)], [(0, 3), (3, 4), (4, 29), (29, 30)]):
        parts = _chunk_pieces(q, k, v, bounds)
        rng.shuffle(parts)
        o, l = merge_fn([p[0] for p in parts], [p[1] for p in parts])
        assert torch.allclose(o, full_o, atol=1e-12, rtol=0) and torch.allclose(l, full_l, atol=1e-12, rtol=0)


def pin_merge_masked(merge_fn):
    """A partial with lse = -inf (nothing visible) is the identity; all-masked merges to (0, -inf)."""
    o1, l1 = rand((3, 4), 210), rand((3,), 211)
    z, zl = torch.zeros(3, 4, dtype=F64), torch.full((3,), float("-inf"), dtype=F64)
    o, l = merge_fn([z, o1, z], [zl, l1, zl])
    assert torch.allclose(o, o1, atol=1e-15, rtol=0) and torch.allclose(l, l1, atol=1e-15, rtol=0)
    o, l = merge_fn([z, z], [zl, zl])
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))


def pin_merge_two_point(merge_fn):
    """Two partials with lse a, b: weights e^a : e^b, merged lse = ln(e^a + e^b)."""
    o1 = torch.tensor([[1.0, 0.0]], dtype=F64)
    o2 = torch.tensor([[0.0, 1.0]], dtype=F64)
    a, b = math.log(3.0), 0.0
    o, l = merge_fn([o1, o2], [torch.tensor([a], dtype=F64), torch.tensor([b], dtype=F64)])
    assert torch.allclose(o, torch.tensor([[0.75, 0.25]], dtype=F64), atol=1e-15, rtol=0)
    assert abs(l.item() - math.log(4.0)) < 1e-15


MERGE_PINS = [pin_merge_partition, pin_merge_masked, pin_merge_two_point]


@pytest.mark.parametrize("pin", MERGE_PINS, ids=lambda p: p.__name__)
def test_merge_pins(pin):
    pin(oracle.merge)


def test_merge_extreme_lse_no_overflow():
    o1, o2 = rand((2, 4), 220), rand((2, 4), 221)
    l1 = torch.tensor([1000.0, -1000.0], dtype=F64)
    l2 = torch.tensor([1000.0, -1000.0 + math.log(3.0)], dtype=F64)
    o, l = oracle.merge([o1, o2], [l1, l2])
    assert torch.all(torch.isfinite(o)) and torch.allclose(o[0], 0.5 * (o1[0] + o2[0]), atol=1e-12)
    assert torch.allclose(o[1], 0.25 * o1[1] + 0.75 * o2[1], atol=1e-12)
    assert abs(l[0].item() - (1000.0 + math.log(2.0))) < 1e-12


@settings(max_examples=25, deadline=None)
@given(S=st.sampled_from([8, 12, 24, 30]), D=st.sampled_from([4, 8]), Hkv=st.sampled_from([1, 2]),
       G=st.sampled_from([1, 3]), seed=st.integers(0, 10_000), causal=st.booleans(),
       order=st.sampled_from([PASS_KV, PASS_Q]))
def test_ring_equals_unchunked_every_chunk_count(S, D, Hkv, G, seed, causal, order):
    q = rand((1, S, Hkv * G, D), seed)
    k = rand((1, S, Hkv, D), seed + 1)
    v = rand((1, S, Hkv, D), seed + 2)
    full_o, full_l = oracle.full_attention(q, k, v, causal)
    rng = random.Random(seed)
    for P in [p for p in range(1, S + 1) if S % p == 0]:
        o, l = oracle.ring_attention(q, k, v, P, order, causal)
        assert torch.allclose(o, full_o, atol=1e-12, rtol=0) and torch.allclose(l, full_l, atol=1e-12, rtol=0)
        arr = oracle.arrival_order(P, order, causal)
        shuffled = [rng.sample(a, len(a)) for a in arr]
        o, l = oracle.ring_attention(q, k, v, P, order, causal, merge_order=shuffled)
        assert torch.allclose(o, full_o, atol=1e-12, rtol=0) and torch.allclose(l, full_l, atol=1e-12, rtol=0)


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("order", [PASS_KV, PASS_Q])
def test_schedule_coverage_and_ring_moves(P, order):
    for causal in (True, False):
        steps = oracle.schedule(P, order, causal)
        pairs = [(qi, kj) for items in steps for _, qi, kj in items]
        want = {(i, j) for i in range(P) for j in range(P) if (j <= i or not causal)}
        assert len(pairs) == len(set(pairs)) == len(want) == (P * (P + 1) // 2 if causal else P * P)
        assert set(pairs) == want
        for items in steps:  # a rank does at most one partial per step
            ranks = [r for r, _, _ in items]
            assert len(ranks) == len(set(ranks))
    # without the causal skip, what rank r holds at step s is what rank r-1 held at step s-1
    full = oracle.schedule(P, order, False)
    held = [{r: (qi if order == PASS_Q else kj) for r, qi, kj in items} for items in full]
    local = [{r: (kj if order == PASS_Q else qi) for r, qi, kj in items} for items in full]
    for s in range(1, P):
        for r in range(P):
            assert held[s][r] == held[s - 1][(r - 1) % P]
            assert local[s][r] == local[0][r] == r


def test_arrival_orders():
    P = 6
    kv = oracle.arrival_order(P, PASS_KV)
    pq = oracle.arrival_order(P, PASS_Q)
    for i in range(P):
        assert kv[i] == list(range(i, -1, -1))
        assert pq[i] == [i] + list(range(i))


def test_splitkv_decode_equals_single_query_attention():
    B, Skv, Hq, Hkv, D = 2, 48, 4, 1, 16
    q = rand((B, 1, Hq, D), 300)
    k, v = rand((B, Skv, Hkv, D), 301), rand((B, Skv, Hkv, D), 302)
    ref = sdpa_reference(q, k, v, 0, 0, False)
    for n in (1, 2, 3, 8, 48):
        o, l = oracle.splitkv_decode(q, k, v, n)
        assert torch.allclose(o, ref, atol=1e-12, rtol=0)
        o2, l2 = oracle.partial_attention(q, k, v, Skv - 1, 0, True)
        assert torch.allclose(l, l2, atol=1e-12, rtol=0)


# ----------------------------------------------------------------------------
# Planted mistakes: every one must trip at least one pin
# ----------------------------------------------------------------------------

def _mut_scale(q, k, v, qo, ko, c):       # 1/D instead of 1/sqrt(D)
    return oracle.partial_attention(q / math.sqrt(q.shape[-1]), k, v, qo, ko, c)


def _mut_strict_diag(q, k, v, qo, ko, c):  # causal mask without the diagonal
    return oracle.partial_attention(q, k, v, qo - 1, ko, c)


def _mut_transposed(q, k, v, qo, ko, c):  # K used where V belongs
    return oracle.partial_attention(q, k, k, qo, ko, c)


def _mut_gqa(q, k, v, qo, ko, c):         # head h reads KV head h % Hkv
    Hq, Hkv = q.shape[2], k.shape[2]
    G = Hq // Hkv
    perm = [(h % Hkv) * G + (h // Hkv) for h in range(Hq)]
    o, l = oracle.partial_attention(q[:, :, perm], k, v, qo, ko, c)
    inv = [perm.index(h) for h in range(Hq)]
    return o[:, :, inv], l[:, :, inv]


def _mut_log2(q, k, v, qo, ko, c):        # LSE in base 2
    o, l = oracle.partial_attention(q, k, v, qo, ko, c)
    return o, l / math.log(2.0)


def _mut_unnormalised(q, k, v, qo, ko, c):  # O not divided by the softmax denominator
    o, l = oracle.partial_attention(q, k, v, qo, ko, c)
    return o * torch.exp(torch.nan_to_num(l, neginf=0.0)).unsqueeze(-1), l


def _mut_merge_sign(partials, lses):       # weights e^(M - lse)
    L = torch.stack(lses)
    M = L.max(0).values
    w = torch.exp(M - L)
    o = (w.unsqueeze(-1) * torch.stack(partials)).sum(0) / w.sum(0).unsqueeze(-1)
    return o, M + torch.log(w.sum(0))


def _mut_merge_no_den(partials, lses):     # dropped denominator
    o, l = oracle.merge(partials, lses)
    M = torch.stack(lses).max(0).values
    return o * torch.exp(l - M).unsqueeze(-1), l


def _mut_merge_mean(partials, lses):       # plain average of partials
    return torch.stack(partials).mean(0), torch.stack(lses).max(0).values


def _trips(pins, fn):
    for pin in pins:
        try:
            pin(fn)
        except (AssertionError, RuntimeError, IndexError):
            return True
    return False


@pytest.mark.parametrize("mut", [_mut_scale, _mut_strict_diag, _mut_transposed, _mut_gqa, _mut_log2,
                                 _mut_unnormalised], ids=lambda f: f.__name__)
def test_partial_pins_catch_planted_mistakes(mut):
    assert _trips(PARTIAL_PINS, mut), f"no pin caught {mut.__name__}"


@pytest.mark.parametrize("mut", [_mut_merge_sign, _mut_merge_no_den, _mut_merge_mean],
                         ids=lambda f: f.__name__)
def test_merge_pins_catch_planted_mistakes(mut):
    assert _trips(MERGE_PINS, mut), f"no merge pin caught {mut.__name__}"
