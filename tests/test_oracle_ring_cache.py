"""Pins for the oracle's ring over Q shorter than K/V, its ring-order selection
by exchanged bytes, and its decode over a KV cache sharded across CP ranks.

As in ``test_oracle.py``, every pin compares against something other than the
function itself (pure-Python brute force, torch's fp64 scaled-dot-product
attention, hand-derived byte counts, closed forms), and planted mistakes at the
bottom must each trip at least one pin.
"""
import math
import random

import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from oracle import PASS_KV, PASS_Q
from test_oracle import brute_partial, rand, sdpa_reference

F64 = torch.float64


# ----------------------------------------------------------------------------
# Ring over new tokens against a cached context (Q shorter than K/V)
# ----------------------------------------------------------------------------

def suffix_attention(q, k, v, causal):
    """The result the ring must reach: the last Sq positions attending the whole K/V sequence."""
    return oracle.partial_attention(q, k, v, k.shape[1] - q.shape[1], 0, causal)


def test_suffix_ring_brute_force():
    """Tiny cases against pure-Python loops (no merge, no max shift)."""
    for n, (Sq, Skv, P, Hq, Hkv, D, causal, order) in enumerate([
            (2, 6, 2, 2, 1, 4, True, PASS_KV), (4, 12, 4, 2, 2, 2, True, PASS_Q),
            (3, 9, 3, 3, 1, 4, False, PASS_KV), (6, 6, 3, 2, 1, 2, True, PASS_Q)]):
        q, k, v = rand((1, Sq, Hq, D), 400 + n), rand((1, Skv, Hkv, D), 410 + n), rand((1, Skv, Hkv, D), 420 + n)
        o, l = oracle.ring_attention(q, k, v, P, order, causal)
        bo, bl = brute_partial(q, k, v, Skv - Sq, 0, causal)
        assert torch.allclose(o, bo, atol=1e-12, rtol=0) and torch.allclose(l, bl, atol=1e-12, rtol=0)


@settings(max_examples=25, deadline=None)
@given(Cq=st.sampled_from([1, 2, 3]), ratio=st.sampled_from([1, 2, 3, 5]), P=st.sampled_from([1, 2, 3, 4]),
       G=st.sampled_from([1, 2]), seed=st.integers(0, 10_000), causal=st.booleans(),
       order=st.sampled_from([PASS_KV, PASS_Q]))
def test_suffix_ring_equals_unchunked(Cq, ratio, P, G, seed, causal, order):
    """For any chunk count, both orders and any merge order, the ring reaches the unchunked
    suffix attention (the merge identity), and torch's fp64 SDPA agrees on O."""
    Sq = Cq * P
    Skv = Sq * ratio
    q, k, v = rand((1, Sq, 2 * G, 4), seed), rand((1, Skv, 2, 4), seed + 1), rand((1, Skv, 2, 4), seed + 2)
    ref_o, ref_l = suffix_attention(q, k, v, causal)
    assert torch.allclose(ref_o, sdpa_reference(q, k, v, Skv - Sq, 0, causal), atol=1e-12, rtol=0)
    o, l = oracle.ring_attention(q, k, v, P, order, causal)
    assert torch.allclose(o, ref_o, atol=1e-12, rtol=0) and torch.allclose(l, ref_l, atol=1e-12, rtol=0)
    rng = random.Random(seed)
    arr = oracle.arrival_order(P, order, causal, Sq, Skv)
    o, l = oracle.ring_attention(q, k, v, P, order, causal, merge_order=[rng.sample(a, len(a)) for a in arr])
    assert torch.allclose(o, ref_o, atol=1e-12, rtol=0) and torch.allclose(l, ref_l, atol=1e-12, rtol=0)


@pytest.mark.parametrize("Sq,Skv,P", [(8, 8, 4), (4, 16, 4), (8, 24, 4), (2, 64, 2), (16, 48, 8), (3, 9, 3)])
@pytest.mark.parametrize("order", [PASS_KV, PASS_Q])
def test_suffix_schedule_coverage(Sq, Skv, P, order):
    """Every pair with a visible (query, key) position pair appears exactly once, the rest never;
    visibility decided by brute force over positions."""
    Cq, Ckv, q0 = Sq // P, Skv // P, Skv - Sq
    for causal in (True, False):
        want = set()
        for i in range(P):
            for j in range(P):
                if any((not causal) or kp <= qp for qp in range(q0 + i * Cq, q0 + (i + 1) * Cq)
                       for kp in range(j * Ckv, (j + 1) * Ckv)):
                    want.add((i, j))
        steps = oracle.schedule(P, order, causal, Sq, Skv)
        pairs = [(qi, kj) for items in steps for _, qi, kj in items]
        assert len(pairs) == len(set(pairs)) and set(pairs) == want
        for items in steps:
            assert len({r for r, _, _ in items}) == len(items)
        arr = oracle.arrival_order(P, order, causal, Sq, Skv)
        for i in range(P):
            assert arr[i][0] == i  # every owner first meets its own chunk
            seq = [((i - s) % P) if order == PASS_KV else ((i + s) % P) for s in range(P)]
            assert arr[i] == [j for j in seq if (i, j) in want]


def test_equal_lengths_keep_the_triangle():
    for P in (1, 2, 5, 16):
        for S in (P, 4 * P):
            assert oracle.schedule(P, PASS_KV, True, S, S) == oracle.schedule(P, PASS_KV, True)
            assert oracle.arrival_order(P, PASS_Q, True, S, S) == oracle.arrival_order(P, PASS_Q, True)


# ----------------------------------------------------------------------------
# Exchanged bytes and the order selection
# ----------------------------------------------------------------------------

def _pick(bytes_fn, P, causal, B, ql, kvl, Hq, Hkv, D, e=2):
    kv = bytes_fn(P, PASS_KV, causal, B, ql, kvl, Hq, Hkv, D, e)
    qb = bytes_fn(P, PASS_Q, causal, B, ql, kvl, Hq, Hkv, D, e)
    return PASS_Q if qb < kv else PASS_KV


def pin_bytes_hand_counted(bytes_fn):
    """P = 2, one token per chunk, one head of one element, 2-byte elements, causal.
    Pass-KV: at step 1 each of the 2 ranks receives K and V of one token: 2 x 2 x 2 = 8 bytes.
    Pass-Q: each rank receives one Q element (2 x 2 = 4 bytes); of the step-1 items only rank 0's
    (Q chunk 1 against K/V chunk 0) is visible and it was computed away from Q chunk 1's owner, so
    one partial returns: O and LSE in fp32, (1 + 1) x 4 = 8 bytes; 12 in all."""
    assert bytes_fn(2, PASS_KV, True, 1, 2, 2, 1, 1, 1) == 8
    assert bytes_fn(2, PASS_Q, True, 1, 2, 2, 1, 1, 1) == 12
    # one rank: nothing moves
    assert bytes_fn(1, PASS_KV, True, 1, 8, 8, 4, 1, 8) == 0
    assert bytes_fn(1, PASS_Q, True, 1, 8, 8, 4, 1, 8) == 0
    # without the mask at P = 2 both step-1 items are remote: 4 + 2 x 8 = 20
    assert bytes_fn(2, PASS_Q, False, 1, 2, 2, 1, 1, 1) == 20


def pin_bytes_equal_length_closed_form(bytes_fn):
    """Equal lengths S = P C: Pass-KV moves P (P-1) K/V chunks; Pass-Q moves P (P-1) Q chunks and
    returns every off-diagonal causal pair's partial, P (P+1) / 2 - P of them (P^2 - P unmasked)."""
    B, C, D, e = 2, 3, 8, 2
    for P in (1, 2, 3, 8, 16):
        for Hq, Hkv in ((1, 1), (16, 1), (8, 2), (2, 2)):
            for causal in (True, False):
                kv = P * (P - 1) * 2 * B * C * Hkv * D * e
                remote = (P * (P + 1) // 2 - P) if causal else P * P - P
                qb = P * (P - 1) * B * C * Hq * D * e + remote * B * C * Hq * (D + 1) * 4
                assert bytes_fn(P, PASS_KV, causal, B, P * C, P * C, Hq, Hkv, D, e) == kv
                assert bytes_fn(P, PASS_Q, causal, B, P * C, P * C, Hq, Hkv, D, e) == qb
                # at equal lengths with 2-byte elements Pass-KV never moves more
                assert _pick(bytes_fn, P, causal, B, P * C, P * C, Hq, Hkv, D, e) == PASS_KV


def pin_bytes_long_context(bytes_fn):
    """16 ranks, 16 query heads on 1 KV head, D = 128, bf16.
    Full 128K prefill: Pass-KV moves 240 hops x 4 MiB (K and V of 8192 tokens), Pass-Q at least
    240 hops x 32 MiB of Q: Pass-KV.
    2048 new tokens against a 131072-token cache (K/V length 133120, chunks of 8320 keys and
    128 queries): every pair is visible; Pass-KV moves 240 x 2 x 8320 x 128 x 2 = 1,022,361,600
    bytes, Pass-Q 240 x 128 x 16 x 128 x 2 = 125,829,120 plus 240 returned partials of
    128 x 16 x 129 x 4 = 1,056,768 bytes = 253,624,320: 379,453,440 in all, so Pass-Q."""
    assert _pick(bytes_fn, 16, True, 1, 131072, 131072, 16, 1, 128) == PASS_KV
    assert bytes_fn(16, PASS_KV, True, 1, 2048, 133120, 16, 1, 128) == 1_022_361_600
    assert bytes_fn(16, PASS_Q, True, 1, 2048, 133120, 16, 1, 128) == 379_453_440
    assert _pick(bytes_fn, 16, True, 1, 2048, 133120, 16, 1, 128) == PASS_Q


BYTE_PINS = [pin_bytes_hand_counted, pin_bytes_equal_length_closed_form, pin_bytes_long_context]


@pytest.mark.parametrize("pin", BYTE_PINS, ids=lambda p: p.__name__)
def test_exchange_bytes_pins(pin):
    pin(oracle.exchange_bytes)


def test_select_order_takes_the_smaller():
    for args in ((2, True, 1, 2, 2, 1, 1, 1), (16, True, 1, 131072, 131072, 16, 1, 128),
                 (16, True, 1, 2048, 133120, 16, 1, 128), (4, False, 2, 64, 1024, 32, 8, 64),
                 (8, True, 1, 8, 4096, 4, 4, 128)):
        assert oracle.select_order(*args) == _pick(oracle.exchange_bytes, *args)


# ----------------------------------------------------------------------------
# Decode over a KV cache sharded across CP ranks
# ----------------------------------------------------------------------------

def _shards(k, v, lengths, cap, seed, fill=float("nan")):
    """Cut the key rows into consecutive pieces of the given lengths, each stored in a shard with
    ``cap`` rows whose unused rows hold ``fill``."""
    ks, vs, lo = [], [], 0
    for n in lengths:
        kk = torch.full((k.shape[0], cap, k.shape[2], k.shape[3]), fill, dtype=F64)
        vv = torch.full_like(kk, fill)
        kk[:, :n] = k[:, lo:lo + n]
        vv[:, :n] = v[:, lo:lo + n]
        ks.append(kk)
        vs.append(vv)
        lo += n
    return ks, vs


def pin_cp_decode_sdpa(fn):
    """Per-shard partials merged equal attention over all cached keys (torch fp64 SDPA, no mask)."""
    for n, (lengths, Hq, Hkv) in enumerate([([5, 7, 4], 4, 1), ([1, 9], 6, 2), ([12], 2, 2), ([3, 0, 6, 2], 4, 2)]):
        S = sum(lengths)
        q, k, v = rand((2, 1, Hq, 8), 500 + n), rand((2, S, Hkv, 8), 510 + n), rand((2, S, Hkv, 8), 520 + n)
        ks, vs = _shards(k, v, lengths, max(lengths) + 3, n)
        o, l = fn(q, ks, vs, lengths)
        assert torch.allclose(o, sdpa_reference(q, k, v, 0, 0, False), atol=1e-12, rtol=0)
        s = torch.einsum("bihd,bjhd->bhij", q, k.repeat_interleave(Hq // Hkv, dim=2)) / math.sqrt(8)
        assert torch.allclose(l, torch.logsumexp(s, dim=-1).permute(0, 2, 1), atol=1e-12, rtol=0)


def pin_cp_decode_brute(fn):
    lengths = [2, 3, 1]
    q, k, v = rand((1, 1, 2, 4), 530), rand((1, 6, 1, 4), 531), rand((1, 6, 1, 4), 532)
    ks, vs = _shards(k, v, lengths, 4, 0, fill=1e6)  # unused rows hold huge values: they must stay unread
    o, l = fn(q, ks, vs, lengths)
    bo, bl = brute_partial(q, k, v, 0, 0, False)
    assert torch.allclose(o, bo, atol=1e-12, rtol=0) and torch.allclose(l, bl, atol=1e-12, rtol=0)


def pin_cp_decode_equal_shards_are_splitkv(fn):
    """Shards that are the equal chunks of one cache, full: the split-KV decode of that cache."""
    q, k, v = rand((3, 1, 4, 8), 540), rand((3, 32, 1, 8), 541), rand((3, 32, 1, 8), 542)
    ks = [k[:, c * 8:(c + 1) * 8] for c in range(4)]
    vs = [v[:, c * 8:(c + 1) * 8] for c in range(4)]
    o, l = fn(q, ks, vs, [8] * 4)
    so, sl = oracle.splitkv_decode(q, k, v, 4)
    assert torch.allclose(o, so, atol=1e-12, rtol=0) and torch.allclose(l, sl, atol=1e-12, rtol=0)


CP_DECODE_PINS = [pin_cp_decode_sdpa, pin_cp_decode_brute, pin_cp_decode_equal_shards_are_splitkv]


@pytest.mark.parametrize("pin", CP_DECODE_PINS, ids=lambda p: p.__name__)
def test_cp_decode_pins(pin):
    pin(oracle.cp_decode)


def test_cp_decode_empty_cache_row():
    q = rand((1, 1, 2, 4), 550)
    k = torch.zeros(1, 3, 1, 4, dtype=F64)
    o, l = oracle.cp_decode(q, [k, k], [k, k], [0, 0])
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))


# ----------------------------------------------------------------------------
# Planted mistakes
# ----------------------------------------------------------------------------

def _mut_ring_prefix_queries(q, k, v, P, order, causal, merge_order=None):
    # queries placed at the start of the sequence instead of its end
    Sq = q.shape[1]
    return oracle.ring_attention(q, k[:, :Sq], v[:, :Sq], P, order, causal, merge_order)


def _mut_ring_drop_last_kv_chunk(q, k, v, P, order, causal, merge_order=None):
    # the newest K/V chunk never reaches the merge
    arr = oracle.arrival_order(P, order, causal, q.shape[1], k.shape[1])
    mo = [[j for j in a if j != P - 1] or a[:1] for a in arr] if P > 1 else None
    return oracle.ring_attention(q, k, v, P, order, causal, mo)


@pytest.mark.parametrize("mut", [_mut_ring_prefix_queries, _mut_ring_drop_last_kv_chunk],
                         ids=lambda f: f.__name__)
def test_suffix_ring_pins_catch_planted_mistakes(mut):
    q, k, v = rand((1, 4, 2, 4), 600), rand((1, 16, 1, 4), 601), rand((1, 16, 1, 4), 602)
    ref_o, _ = suffix_attention(q, k, v, True)
    o, _ = mut(q, k, v, 4, PASS_KV, True)
    assert not torch.allclose(o, ref_o, atol=1e-6)


_BYTES = oracle.exchange_bytes


def _mut_bytes_p_hops(P, order, causal, B, ql, kvl, Hq, Hkv, D, e=2):
    # every chunk counted for P hops instead of P - 1
    per_hop = 2 * B * (kvl // P) * Hkv * D * e if order == PASS_KV else B * (ql // P) * Hq * D * e
    return _BYTES(P, order, causal, B, ql, kvl, Hq, Hkv, D, e) + P * per_hop


def _mut_bytes_no_return(P, order, causal, B, ql, kvl, Hq, Hkv, D, e=2):
    # Pass-Q partials never travel back to their owner
    if order == PASS_KV:
        return _BYTES(P, order, causal, B, ql, kvl, Hq, Hkv, D, e)
    return P * (P - 1) * B * (ql // P) * Hq * D * e


def _mut_bytes_swapped_heads(P, order, causal, B, ql, kvl, Hq, Hkv, D, e=2):
    # query and KV head counts swapped
    return _BYTES(P, order, causal, B, ql, kvl, Hkv, Hq, D, e)


def _mut_bytes_all_pairs_return(P, order, causal, B, ql, kvl, Hq, Hkv, D, e=2):
    # the owner's own partial counted as returned too
    extra = P * B * (ql // P) * Hq * (D + 1) * 4 if order == PASS_Q else 0
    return _BYTES(P, order, causal, B, ql, kvl, Hq, Hkv, D, e) + extra


@pytest.mark.parametrize("mut", [_mut_bytes_p_hops, _mut_bytes_no_return, _mut_bytes_swapped_heads,
                                 _mut_bytes_all_pairs_return], ids=lambda f: f.__name__)
def test_byte_pins_catch_planted_mistakes(mut):
    tripped = False
    for pin in BYTE_PINS:
        try:
            pin(mut)
        except AssertionError:
            tripped = True
            break
    assert tripped, f"no byte pin caught {mut.__name__}"


def _mut_cp_decode_full_capacity(q, ks, vs, lengths):
    # reads every row of a shard, not only the valid ones
    return oracle.cp_decode(q, ks, vs, [k.shape[1] for k in ks])


def _mut_cp_decode_first_shard_only(q, ks, vs, lengths):
    return oracle.cp_decode(q, ks[:1], vs[:1], lengths[:1])


def _mut_cp_decode_causal_local(q, ks, vs, lengths):
    # each shard masked as if the query sat at local position 0 of that shard
    parts = [oracle.partial_attention(q, k_[:, :n], v_[:, :n], 0, 0, True) for k_, v_, n in zip(ks, vs, lengths)]
    return oracle.merge([p[0] for p in parts], [p[1] for p in parts])


@pytest.mark.parametrize("mut", [_mut_cp_decode_full_capacity, _mut_cp_decode_first_shard_only,
                                 _mut_cp_decode_causal_local], ids=lambda f: f.__name__)
def test_cp_decode_pins_catch_planted_mistakes(mut):
    tripped = False
    for pin in CP_DECODE_PINS:
        try:
            pin(mut)
        except (AssertionError, RuntimeError, IndexError):
            tripped = True
            break
    assert tripped, f"no cp-decode pin caught {mut.__name__}"
