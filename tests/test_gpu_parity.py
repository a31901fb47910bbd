"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

Every call goes through the C ABI (via the ctypes binding).  Inputs come from
``seeded_inputs``; expected values come from ``oracle`` only.
"""
import math

import pytest
import torch

import oracle
import seeded_inputs as si
from gpu_util import BF16_TOL, F32_TOL, banner, compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def cp():
    import context_attention_cpattn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return m


def draw(seed, shape, dtype, tensor_id=0):
    return si.draw_tensor(seed, tensor_id, shape, dtype)


# (B, Sq, Sk, Hq, Hkv, D, q_offset, kv_offset, causal)
PARTIAL_CASES = [
    (1, 256, 256, 2, 1, 128, 0, 0, True),        # diagonal block, 2 query tiles
    (1, 300, 300, 2, 1, 128, 1000, 1000, True),  # diagonal, ragged (300 = 2*128 + 44)
    (2, 128, 512, 4, 2, 128, 512, 0, True),      # K/V block entirely in the past
    (1, 200, 77, 3, 1, 128, 0, 500, True),       # K/V block entirely in the future: all masked
    (1, 257, 333, 2, 2, 128, 100, 37, True),     # odd offsets straddling the diagonal
    (1, 130, 190, 4, 1, 128, 0, 0, False),       # no mask, ragged both ways
    (1, 256, 256, 2, 1, 64, 0, 0, True),         # D = 64
    (2, 190, 300, 4, 4, 64, 150, 0, True),       # D = 64, GQA off, ragged
    (1, 1, 1000, 16, 1, 128, 999, 0, True),      # one query row (decode-like shape)
    (3, 1, 777, 16, 1, 128, 500, 0, True),       # one row seeing a ragged key prefix (501 keys)
    (2, 1, 300, 8, 2, 128, 10, 50, True),        # one row before the block: all masked
    (2, 1, 300, 40, 1, 128, 0, 0, False),        # one row, 40 heads per KV head (3 head blocks)
    (4, 1, 513, 16, 1, 64, 600, 0, True),        # one row, D = 64
    (1, 64, 0, 2, 1, 128, 0, 0, True),           # empty K/V block
]


@pytest.mark.parametrize("case", PARTIAL_CASES, ids=lambda c: "B{}_Sq{}_Sk{}_H{}-{}_D{}_off{}-{}_c{}".format(*c))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_partial_matches_oracle(cp, case, dtype):
    B, Sq, Sk, Hq, Hkv, D, qo, ko, causal = case
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    seed = 1000 + Sq + 7 * Sk + D
    q = draw(seed, (B, Sq, Hq, D), tdt, 0)
    k = draw(seed, (B, Sk, Hkv, D), tdt, 1)
    v = draw(seed, (B, Sk, Hkv, D), tdt, 2)
    o_ref, l_ref = oracle.partial_attention(q, k, v, qo, ko, causal)
    banner("partial", dtype, case)
    o, l = cp.partial(q.to(DEV), k.to(DEV), v.to(DEV), qo, ko, causal)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL if dtype == "bf16" else F32_TOL, f"partial {dtype} {case}")


@pytest.mark.parametrize("Sq", [200, 1])
def test_partial_strided_views(cp, Sq):
    """Non-contiguous views (head-sliced, padded rows) through the descriptor strides;
    Sq = 1 takes the one-row (decode kernel) route."""
    B, S, H, D = 2, 200, 6, 128
    big_q = draw(77, (B, Sq, H + 2, D), torch.bfloat16, 0)
    big_k = draw(77, (B, S, 3, D), torch.bfloat16, 1)
    big_v = draw(77, (B, S, 3, D), torch.bfloat16, 2)
    q, k, v = big_q[:, :, 1:H + 1], big_k[:, :, 1:3], big_v[:, :, 1:3]
    o_ref, l_ref = oracle.partial_attention(q, k, v, 10, 0, True)
    gq, gk, gv = big_q.to(DEV)[:, :, 1:H + 1], big_k.to(DEV)[:, :, 1:3], big_v.to(DEV)[:, :, 1:3]
    out_big = torch.full((B, Sq, H + 1, D), float("nan"), device=DEV)
    lse_big = torch.full((B, Sq, H + 3), float("nan"), device=DEV)
    banner("partial strided", Sq)
    o, l = cp.partial(gq, gk, gv, 10, 0, True, out=out_big[:, :, :H], lse=lse_big[:, :, 2:2 + H])
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, "partial strided")
    assert torch.isnan(out_big[:, :, H]).all() and torch.isnan(lse_big[:, :, :2]).all()
    assert torch.isnan(lse_big[:, :, 2 + H:]).all()


@pytest.mark.parametrize("n", [1, 2, 5, 64])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_merge_matches_oracle(cp, n, out_dtype):
    B, S, H, D = 2, 37, 3, 128
    parts = [draw(500 + c, (B, S, H, D), torch.float32, 0) for c in range(n)]
    lses = [4.0 * draw(500 + c, (B, S, H), torch.float32, 1) for c in range(n)]
    if n > 1:  # some partials with nothing visible, and one row where every partial is empty
        lses[1][0, :5] = float("-inf")
        for c in range(n):
            lses[c][1, 3, 2] = float("-inf")
    o_ref, l_ref = oracle.merge(parts, lses)
    banner("merge", n, out_dtype)
    o, l = cp.merge([p.to(DEV) for p in parts], [x.to(DEV) for x in lses], out_dtype=out_dtype)
    torch.cuda.synchronize()
    tol = F32_TOL if out_dtype == torch.float32 else BF16_TOL
    compare(o.float(), l, o_ref, l_ref, tol, f"merge n={n} {out_dtype}")


def test_merge_bf16_rounding_is_nearest_even(cp):
    p = draw(9, (1, 16, 2, 64), torch.float32, 0)
    lse = torch.zeros(1, 16, 2)
    o, _ = cp.merge([p.to(DEV)], [lse.to(DEV)], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), p.to(torch.bfloat16))


# ----------------------------------------------------------------------------
# The five workloads
# ----------------------------------------------------------------------------

def test_workload_tiny_f32_unchunked(cp):
    w = si.WORKLOADS["tiny_f32_s512_p4"]
    q, k, v = si.make_qkv(w)
    o_ref, l_ref = oracle.full_attention(q, k, v, causal=True)  # unchunked reference
    banner(w.name, "pass_kv", w.n_chunks)
    o, l = cp.ring_prefill(q.to(DEV), k.to(DEV), v.to(DEV), w.n_chunks, "pass_kv", True)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, w.name + " (workload tolerance)")
    compare(o, l, o_ref, l_ref, F32_TOL, w.name + " (fp32 tolerance)")


def test_workload_tiny_bf16_copy(cp):
    w = si.WORKLOADS["tiny_f32_s512_p4"]
    q, k, v = si.make_qkv(w, torch.bfloat16)
    o_ref, l_ref = oracle.ring_attention(q, k, v, w.n_chunks, oracle.PASS_KV, True)
    for order in ("pass_kv", "pass_q"):
        banner(w.name, "bf16", order)
        o, l = cp.ring_prefill(q.to(DEV), k.to(DEV), v.to(DEV), w.n_chunks, order, True)
        torch.cuda.synchronize()
        compare(o, l, o_ref, l_ref, BF16_TOL, f"{w.name} bf16 {order}")


@pytest.mark.parametrize("P,order,causal", [(1, "pass_kv", True), (3, "pass_q", True), (5, "pass_kv", False),
                                            (6, "pass_q", False), (8, "pass_kv", True),
                                            (64, "pass_kv", True), (64, "pass_q", False)])  # 64: the chunk limit
def test_ring_small_orders(cp, P, order, causal):
    S = 120 * P  # 120-token chunks: one ragged query tile per chunk
    q = draw(31 + P, (1, S, 4, 128), torch.bfloat16, 0)
    k = draw(31 + P, (1, S, 2, 128), torch.bfloat16, 1)
    v = draw(31 + P, (1, S, 2, 128), torch.bfloat16, 2)
    o_ref, l_ref = oracle.full_attention(q, k, v, causal)
    banner("ring", P, order, causal)
    o, l = cp.ring_prefill(q.to(DEV), k.to(DEV), v.to(DEV), P, order, causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, f"ring P={P} {order} causal={causal}")
    o16, _ = cp.ring_prefill(q.to(DEV), k.to(DEV), v.to(DEV), P, order, causal, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16.cpu(), o.cpu().to(torch.bfloat16))


@pytest.mark.parametrize("P,order,causal,C", [(4, "pass_kv", True, 96), (4, "pass_q", True, 96), (3, "pass_kv", False, 96),
                                              (3, "pass_q", False, 96), (9, "pass_kv", True, 96),
                                              (4, "pass_kv", True, 128), (3, "pass_q", False, 192),
                                              (5, "pass_q", True, 320), (6, "pass_kv", True, 64)])
def test_ring_merge_follows_arrival_order(cp, P, order, causal, C):
    """The ring driver's merge equals, bit for bit, merging the same partials in the
    arrival order the oracle's schedule defines (partials via the partial entry point).
    These grids are small, so the driver launches per pair; its per-owner walk, whose
    partials must be the same bits, is checked the same way in the chunk-walk tests."""
    H, D = 2, 128
    S = C * P
    q = draw(61 + P, (1, S, H, D), torch.bfloat16, 0).to(DEV)
    k = draw(61 + P, (1, S, 1, D), torch.bfloat16, 1).to(DEV)
    v = draw(61 + P, (1, S, 1, D), torch.bfloat16, 2).to(DEV)
    banner("ring merge order", P, order, causal)
    o, l = cp.ring_prefill(q, k, v, P, order, causal)
    arrivals = oracle.arrival_order(P, order, causal)
    for i in range(P):
        parts = [cp.partial(q[:, i * C:(i + 1) * C], k[:, j * C:(j + 1) * C], v[:, j * C:(j + 1) * C], i * C, j * C, causal)
                 for j in arrivals[i]]
        om, lm = cp.merge([p_[0] for p_ in parts], [p_[1] for p_ in parts])
        torch.cuda.synchronize()
        assert torch.equal(om, o[:, i * C:(i + 1) * C]), f"owner {i}: O differs"
        assert torch.equal(lm, l[:, i * C:(i + 1) * C]), f"owner {i}: LSE differs"


@pytest.mark.parametrize("P,C,B,H,Hkv,D,order,causal", [(64, 64, 2, 4, 1, 128, "pass_kv", True),
                                                        (8, 64, 2, 32, 2, 128, "pass_q", False),
                                                        (4, 320, 2, 32, 2, 128, "pass_kv", True),
                                                        (3, 4096, 1, 12, 1, 128, "pass_q", True),
                                                        (4, 128, 4, 32, 2, 64, "pass_kv", True)])
def test_ring_prefill_chunk_walk(cp, P, C, B, H, Hkv, D, order, causal):
    """Chunks of a multiple of 64 tokens (up to 16384) on grids of at least two walking
    workgroups per compute unit (on 256 of them): the driver's per-owner walk that writes every
    pair's partial at the chunk boundary and merges them at its end, against the oracle and bit
    for bit against the per-step launches and the merge; 64-token chunks put a boundary after
    every tile, and 64 of them use every segment slot of the merge tail."""
    S = C * P
    walks = P * B * H * ((C + 255) // 256) >= 2 * torch.cuda.get_device_properties(0).multi_processor_count
    q = draw(131 + P, (B, S, H, D), torch.bfloat16, 0)
    k = draw(131 + P, (B, S, Hkv, D), torch.bfloat16, 1)
    v = draw(131 + P, (B, S, Hkv, D), torch.bfloat16, 2)
    o_ref, l_ref = oracle.full_attention(q, k, v, causal)
    banner("ring chunk walk", P, C, B, H, Hkv, D, order, causal, "walks" if walks else "per pair on this device")
    gq, gk, gv = q.to(DEV), k.to(DEV), v.to(DEV)
    o, l = cp.ring_prefill(gq, gk, gv, P, order, causal)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, f"ring chunk walk P={P} C={C} B={B} H={H} Hkv={Hkv} D={D} {order} causal={causal}")
    ws = torch.empty(cp.ring_prefill_workspace_size(gq, P, causal), dtype=torch.uint8, device=DEV)
    for step in range(P):
        cp.ring_step(gq, gk, gv, P, step, ws, order, causal)
    o_s, l_s = torch.empty_like(o), torch.empty_like(l)
    cp.ring_merge(P, ws, o_s, l_s, order, causal)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o) and torch.equal(l_s, l), "ring steps + merge differ from the walk"


@pytest.mark.parametrize("P,order,causal,D,dtype", [(1, "pass_kv", True, 128, "bf16"), (4, "pass_kv", True, 128, "bf16"),
                                                  (4, "pass_q", True, 128, "bf16"), (5, "pass_kv", False, 128, "bf16"),
                                                  (3, "pass_q", False, 64, "bf16"), (6, "pass_kv", True, 64, "bf16"),
                                                  (4, "pass_q", True, 64, "f32"), (3, "pass_kv", False, 128, "f32")])
def test_ring_step_accumulate(cp, P, order, causal, D, dtype):
    """Ring steps that merge each arriving partial into the running (O, LSE): after all steps the
    result is the full attention, and it matches the partials-then-merge driver to fp32 rounding."""
    S = 120 * P
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = draw(91 + P, (2, S, 4, D), tdt, 0)
    k = draw(91 + P, (2, S, 2, D), tdt, 1)
    v = draw(91 + P, (2, S, 2, D), tdt, 2)
    o_ref, l_ref = oracle.full_attention(q, k, v, causal)
    gq, gk, gv = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.full((2, S, 4, D), float("nan"), device=DEV)  # step 0 must write every row
    lse = torch.full((2, S, 4), float("nan"), device=DEV)
    banner("ring accumulate", P, order, causal, D, dtype)
    for step in range(P):
        cp.ring_step_accumulate(gq, gk, gv, P, step, out, lse, order, causal)
    torch.cuda.synchronize()
    compare(out, lse, o_ref, l_ref, BF16_TOL if dtype == "bf16" else F32_TOL,
            f"ring accumulate P={P} {order} causal={causal} D={D} {dtype}")
    o2, l2 = cp.ring_prefill(gq, gk, gv, P, order, causal)
    torch.cuda.synchronize()
    assert (o2 - out).abs().max().item() <= 1e-5 and (l2 - lse).abs().max().item() <= 1e-5


@pytest.mark.parametrize("P,causal,Hkv,D", [(1, True, 1, 128), (4, True, 2, 128), (5, False, 1, 128), (3, True, 1, 64),
                                           (6, True, 4, 64), (64, True, 1, 128), (64, False, 2, 64)])
def test_ring_prefill_fused(cp, P, causal, Hkv, D):
    S = 120 * P  # ragged query tiles inside every chunk
    q = draw(71 + P, (2, S, 4, D), torch.bfloat16, 0)
    k = draw(71 + P, (2, S, Hkv, D), torch.bfloat16, 1)
    v = draw(71 + P, (2, S, Hkv, D), torch.bfloat16, 2)
    o_ref, l_ref = oracle.full_attention(q, k, v, causal)
    banner("ring fused", P, causal, Hkv, D)
    o, l = cp.ring_prefill_fused(q.to(DEV), k.to(DEV), v.to(DEV), P, causal)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, f"ring fused P={P} causal={causal} Hkv={Hkv} D={D}")


def test_ring_prefill_fused_f32_and_no_lse(cp):
    S, P = 300, 3
    q = draw(81, (1, S, 2, 64), torch.float32, 0)
    k = draw(81, (1, S, 1, 64), torch.float32, 1)
    v = draw(81, (1, S, 1, 64), torch.float32, 2)
    o_ref, _ = oracle.ring_attention(q, k, v, P, "pass_kv", True)
    banner("ring fused f32")
    o, l = cp.ring_prefill_fused(q.to(DEV), k.to(DEV), v.to(DEV), P, True, want_lse=False)
    torch.cuda.synchronize()
    assert l is None
    assert (o.double().cpu() - o_ref).abs().max().item() < 1e-4


def test_workload_gqa_8k(cp):
    w = si.WORKLOADS["gqa16_bf16_s8k_p8"]
    q, k, v = si.make_qkv(w)
    banner(w.name, "oracle")
    o_ref, l_ref = oracle.full_attention(q, k, v, causal=True)
    banner(w.name, "pass_kv", w.n_chunks)
    o, l = cp.ring_prefill(q.to(DEV), k.to(DEV), v.to(DEV), w.n_chunks, "pass_kv", True)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, w.name)
    banner(w.name, "ring_prefill_fused", w.n_chunks)
    o, l = cp.ring_prefill_fused(q.to(DEV), k.to(DEV), v.to(DEV), w.n_chunks, True)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, w.name + " fused")


def test_workload_decode_32k(cp):
    w = si.WORKLOADS["decode_b128_kv32k_p8"]
    q, k, v = si.make_qkv(w)
    banner(w.name, "oracle")
    o_ref, l_ref = oracle.splitkv_decode(q, k, v, w.n_chunks)
    gq, gk, gv = q.to(DEV), k.to(DEV), v.to(DEV)
    banner(w.name, "splitkv_decode", w.n_chunks)
    o, l = cp.splitkv_decode(gq, gk, gv, w.n_chunks)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, w.name)
    # the same result through the generic entry points: 8 partials, then a merge
    C = w.chunk
    parts = [cp.partial(gq, gk[:, c * C:(c + 1) * C], gv[:, c * C:(c + 1) * C], w.Skv - 1, c * C, True)
             for c in range(w.n_chunks)]
    o2, l2 = cp.merge([p[0] for p in parts], [p[1] for p in parts])
    torch.cuda.synchronize()
    compare(o2, l2, o_ref, l_ref, BF16_TOL, w.name + " via partial+merge")


def _sampled_check(cp, w, o, l, q, k, v, name):
    rows = si.sampled_rows(w, 64)
    # the oracle runs in groups of rows, reporting each group as it finishes
    parts = []
    for i in range(0, len(rows), 16):
        grp = rows[i:i + 16]
        parts.append(oracle.attention_rows(q[:, grp], k, v, grp, causal=True))
        print(f"[oracle] {name}: rows {i}..{i + len(grp) - 1} of {len(rows)} done", flush=True)
    o_ref = torch.cat([p_[0] for p_ in parts], dim=1)
    l_ref = torch.cat([p_[1] for p_ in parts], dim=1)
    idx = torch.as_tensor(rows, device=o.device)
    compare(o.index_select(1, idx), l.index_select(1, idx), o_ref, l_ref, BF16_TOL, name + " (64 sampled rows)")


@pytest.fixture(scope="module")
def c4(cp):
    """The 128K-token workload through every ring path once: whole ring prefills in both orders, the
    per-step launches bench.py times, the accumulating ring steps and the fused prefill.  Checks
    among the paths run here; the comparisons with the oracle are the tests below."""
    w = si.WORKLOADS["prefill_bf16_s128k_p16"]
    banner(w.name, "drawing inputs")
    q, k, v = si.make_qkv(w)
    gq, gk, gv = q.to(DEV), k.to(DEV), v.to(DEV)
    res = {}
    for order in w.orders:
        banner(w.name, order, w.n_chunks)
        res[order] = cp.ring_prefill(gq, gk, gv, w.n_chunks, order, True)
        torch.cuda.synchronize()
    # the launch configuration bench.py times: one ring_step launch per step, then ring_merge;
    # every pair is computed by the same per-block code, so the result is bit-identical
    banner(w.name, "pass_kv per-step launches")
    ws = torch.empty(cp.ring_prefill_workspace_size(gq, w.n_chunks, True), dtype=torch.uint8, device=DEV)
    o_s = torch.empty_like(res["pass_kv"][0])
    l_s = torch.empty_like(res["pass_kv"][1])
    for step in range(w.n_chunks):
        cp.ring_step(gq, gk, gv, w.n_chunks, step, ws, "pass_kv", True)
    cp.ring_merge(w.n_chunks, ws, o_s, l_s, "pass_kv", True)
    torch.cuda.synchronize()
    assert torch.equal(o_s, res["pass_kv"][0]) and torch.equal(l_s, res["pass_kv"][1])
    del ws, o_s, l_s
    (okv, lkv), (oq, lq) = res["pass_kv"], res["pass_q"]
    d_o = (okv - oq).abs().max().item()
    d_l = (lkv - lq).abs().max().item()
    print(f"[parity] {w.name}: pass_kv vs pass_q max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}", flush=True)
    assert d_o <= 1e-5 and d_l <= 1e-5
    # the accumulating ring steps (each partial merged into the running result by the kernel that
    # computes it), in the order bench.py times them
    banner(w.name, "ring_step_accumulate", w.n_chunks)
    oa = torch.empty_like(okv)
    la = torch.empty_like(lkv)
    for step in range(w.n_chunks):
        cp.ring_step_accumulate(gq, gk, gv, w.n_chunks, step, oa, la, "pass_kv", True)
    torch.cuda.synchronize()
    d_o = (okv - oa).abs().max().item()
    d_l = (lkv - la).abs().max().item()
    print(f"[parity] {w.name}: accumulate vs pass_kv max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}", flush=True)
    assert d_o <= 1e-5 and d_l <= 1e-5
    res["accumulate"] = (oa, la)
    # the fused ring prefill (online merge, one launch).  It and the per-pair path round P to bf16
    # against different running maxima, so they differ by bf16 rounding of P, not by fp32
    # reordering alone: the bar between them is the bf16 tolerance each meets against the oracle.
    banner(w.name, "ring_prefill_fused", w.n_chunks)
    of, lf = cp.ring_prefill_fused(gq, gk, gv, w.n_chunks, True)
    torch.cuda.synchronize()
    d = (okv - of).abs_()
    d_o, m_o = d.max().item(), d.mean().item()
    del d
    d_l = (lkv - lf).abs().max().item()
    print(f"[parity] {w.name}: fused vs pass_kv max|dO|={d_o:.3e} mean|dO|={m_o:.3e} max|dLSE|={d_l:.3e}",
          flush=True)
    assert d_o <= BF16_TOL.max_abs and m_o <= BF16_TOL.mean_abs and d_l <= BF16_TOL.lse_abs
    res["fused"] = (of, lf)
    for name, (o_, l_) in res.items():  # every row: finite output
        assert torch.isfinite(o_).all() and torch.isfinite(l_).all(), name
    del gq, gk, gv
    yield w, q, k, v, res
    del res
    torch.cuda.empty_cache()


C4_PATHS = ["pass_kv", "pass_q", "accumulate", "fused"]


@pytest.mark.parametrize("path", C4_PATHS)
def test_workload_128k_sampled_rows(cp, c4, path):
    """All owners: 64 sampled rows per head (first and last token, both sides of every chunk
    boundary, 30 drawn) against the oracle at full causal context."""
    w, q, k, v, res = c4
    _sampled_check(cp, w, *res[path], q, k, v, f"{w.name} {path}")


# Owner chunks 0 (the first 8192 rows, one pair each) and 15 (the last 8192 rows, which merge all
# 16 pairs and see the longest context) are compared with the oracle at every row and head, in
# parts of 1024 rows so each part's fp64 oracle (~1e12 FLOP at most) finishes in seconds.
C4_PARTS = [(0, r0) for r0 in range(0, 8192, 1024)] + [(15, 15 * 8192 + r0) for r0 in range(0, 8192, 1024)]


@pytest.mark.parametrize("owner,r0", C4_PARTS, ids=lambda x: str(x))
def test_workload_128k_owner_rows(cp, c4, owner, r0):
    import time

    w, q, k, v, res = c4
    r1 = r0 + 1024
    t0 = time.perf_counter()
    banner(w.name, f"oracle rows {r0}..{r1 - 1} (owner {owner})")
    o_ref, l_ref = oracle.partial_attention(q[:, r0:r1], k[:, :r1], v[:, :r1], r0, 0, True, row_block=256)
    print(f"[oracle] {w.name} rows {r0}..{r1 - 1}: {time.perf_counter() - t0:.1f} s", flush=True)
    for path in C4_PATHS:
        o, l = res[path]
        compare(o[:, r0:r1], l[:, r0:r1], o_ref, l_ref, BF16_TOL, f"{w.name} {path} owner {owner} rows {r0}..{r1 - 1}")


# The middle owners (1..14) at every row for two of the 16 heads, one owner per test: with the
# owners 0 and 15 above, every query position of the sequence is compared with the oracle.
C4_MID_HEADS = [0, 11]


@pytest.mark.parametrize("owner", range(1, 15))
def test_workload_128k_middle_owner_rows(cp, c4, owner):
    import time

    w, q, k, v, res = c4
    r0, r1 = owner * 8192, (owner + 1) * 8192
    hs = torch.as_tensor(C4_MID_HEADS)
    t0 = time.perf_counter()
    banner(w.name, f"oracle rows {r0}..{r1 - 1} (owner {owner}), heads {C4_MID_HEADS}")
    o_ref, l_ref = oracle.partial_attention(q[:, r0:r1].index_select(2, hs).contiguous(), k[:, :r1], v[:, :r1], r0, 0,
                                            True, row_block=256)
    print(f"[oracle] {w.name} owner {owner}: {time.perf_counter() - t0:.1f} s", flush=True)
    gh = hs.to(DEV)
    for path in C4_PATHS:
        o, l = res[path]
        compare(o[:, r0:r1].index_select(2, gh), l[:, r0:r1].index_select(2, gh), o_ref, l_ref, BF16_TOL,
                f"{w.name} {path} owner {owner} heads {C4_MID_HEADS}")


@pytest.mark.timeout(900)
def test_workload_1m_sampled(cp):
    w = si.WORKLOADS["prefill_bf16_s1m_p8"]
    banner(w.name, "drawing inputs")
    q, k, v = si.make_qkv(w)
    gq, gk, gv = q.to(DEV), k.to(DEV), v.to(DEV)
    banner(w.name, "pass_kv", w.n_chunks)
    o, l = cp.ring_prefill(gq, gk, gv, w.n_chunks, "pass_kv", True)
    torch.cuda.synchronize()
    banner(w.name, "oracle on sampled rows")
    _sampled_check(cp, w, o, l, q, k, v, w.name)
    # and two blocks of 512 consecutive rows for two heads: across the boundary between chunks 3
    # and 4, and the last rows of the sequence (each row at its full causal context)
    hs = torch.as_tensor([0, 15])
    gh = hs.to(DEV)
    for r0 in (4 * w.chunk - 256, w.Sq - 512):
        r1 = r0 + 512
        banner(w.name, f"oracle rows {r0}..{r1 - 1}, heads 0 and 15")
        o_ref, l_ref = oracle.partial_attention(q[:, r0:r1].index_select(2, hs).contiguous(), k[:, :r1], v[:, :r1],
                                                r0, 0, True, row_block=256)
        compare(o[:, r0:r1].index_select(2, gh), l[:, r0:r1].index_select(2, gh), o_ref, l_ref, BF16_TOL,
                f"{w.name} rows {r0}..{r1 - 1}")
    del o, l, gq, gk, gv
    torch.cuda.empty_cache()
