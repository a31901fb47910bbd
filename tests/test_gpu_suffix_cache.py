"""GPU parity for new tokens against a cached context and for the CP-sharded KV cache.

* Ring attention whose queries are the last Sq positions of a longer K/V
  sequence, in both ring orders and with the order chosen by the library's
  exchanged-bytes rule, through every ring entry point, against the fp64 oracle.
* The prefill's K/V written into per-rank cache shards and new tokens appended
  (byte copies: compared bit for bit with the source rows).
* Decode of new tokens against the sharded cache, per-shard partials merged,
  against the oracle's twin.

Every call goes through the C ABI (ctypes binding); inputs come from
``seeded_inputs``; expected values come from ``oracle`` or, for the copies, from
the source tensors themselves.
"""
import time

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


def suffix_reference(q, k, v, causal):
    return oracle.partial_attention(q, k, v, k.shape[1] - q.shape[1], 0, causal)


# (B, Sq, Skv, P, Hq, Hkv, D, dtype): bf16 with K/V chunks of a multiple of 64 keys (up to 16384)
# takes the per-owner walk when the owners' query tiles number at least two per compute unit (the
# last four cases, on 256 of them; two of those also pack heads), the others one work item per pair
SUFFIX_CASES = [
    (1, 512, 2048, 4, 4, 1, 128, "bf16"),     # 512-key chunks, 128-query chunks
    (2, 300, 12480, 3, 4, 2, 128, "bf16"),    # 4160-key chunks, ragged 100-query chunks
    (1, 200, 4000, 4, 2, 1, 128, "bf16"),     # 1000-key chunks (not a multiple of 64)
    (1, 1024, 1024, 8, 2, 1, 128, "bf16"),    # equal lengths through the same code
    (1, 64, 8192, 16, 8, 1, 128, "bf16"),     # 4 queries per chunk, 512-key chunks
    (2, 192, 960, 3, 4, 2, 64, "bf16"),       # D = 64
    (1, 128, 640, 2, 2, 1, 64, "f32"),        # fp32 vector path
    (1, 96, 1152, 3, 2, 2, 128, "f32"),
    (8, 512, 2048, 4, 16, 1, 128, "bf16"),    # walk, 128-query chunks, two heads to a workgroup
    (12, 300, 3840, 3, 16, 2, 128, "bf16"),   # walk, ragged 100-query chunks, 1280-key chunks
    (8, 64, 8192, 16, 8, 1, 128, "bf16"),     # walk, 4 queries per chunk, four heads to a workgroup
    # walk with queries just shorter than K/V: the first query tiles of owners 0-2 end inside their
    # own chunk (their partial stays in registers for the merge tail) yet store an empty partial
    # for the next chunk, which the owner's later rows see
    (2, 4032, 4096, 4, 16, 1, 128, "bf16"),
]


@pytest.mark.parametrize("case", SUFFIX_CASES, ids=lambda c: "B{}_Sq{}_Skv{}_P{}_H{}-{}_D{}_{}".format(*c))
def test_suffix_ring_prefill(cp, case):
    B, Sq, Skv, P, Hq, Hkv, D, dt = case
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    tol = BF16_TOL if dt == "bf16" else F32_TOL
    seed = 700 + Sq + Skv + D
    q, k, v = draw(seed, (B, Sq, Hq, D), tdt, 0), draw(seed, (B, Skv, Hkv, D), tdt, 1), draw(seed, (B, Skv, Hkv, D), tdt, 2)
    gq, gk, gv = q.to(DEV), k.to(DEV), v.to(DEV)
    for causal in (True, False):
        o_ref, l_ref = suffix_reference(q, k, v, causal)
        outs = {}
        for order in ("pass_kv", "pass_q", "auto"):
            banner("suffix ring", case, order, causal)
            outs[order] = cp.ring_prefill(gq, gk, gv, P, order, causal)
            torch.cuda.synchronize()
            compare(*outs[order], o_ref, l_ref, tol, f"suffix {case} {order} causal={causal}")
        chosen, _, _ = cp.ring_select_order(gq, gk, P, causal)
        assert torch.equal(outs["auto"][0], outs[chosen][0]) and torch.equal(outs["auto"][1], outs[chosen][1])
        d = (outs["pass_kv"][0] - outs["pass_q"][0]).abs().max().item()
        assert d <= (1e-5 if dt == "bf16" else 1e-6)
        # per-step launches + merge equal the whole ring bit for bit (with K/V chunks of a multiple
        # of 64 keys up to 16384 the whole ring walks each owner's keys, writes every pair's partial
        # at the chunk boundaries, empty ones included, and merges them at the end of the walk: the
        # same partials as per-pair launches, merged with the same arithmetic)
        for order in ("pass_kv", "pass_q"):
            banner("suffix ring steps", case, order, causal)
            ws = torch.empty(cp.ring_prefill_workspace_size(gq, P, causal, gk), dtype=torch.uint8, device=DEV)
            o_s = torch.empty(B, Sq, Hq, D, device=DEV)
            l_s = torch.empty(B, Sq, Hq, device=DEV)
            for step in range(P):
                cp.ring_step(gq, gk, gv, P, step, ws, order, causal)
            cp.ring_merge(P, ws, o_s, l_s, order, causal, kv_len=Skv)
            torch.cuda.synchronize()
            assert torch.equal(o_s, outs[order][0]) and torch.equal(l_s, outs[order][1])
        # accumulating steps and the fused walk
        for order in ("pass_kv", "pass_q"):
            banner("suffix accumulate", case, order, causal)
            oa = torch.full((B, Sq, Hq, D), float("nan"), device=DEV)
            la = torch.full((B, Sq, Hq), float("nan"), device=DEV)
            for step in range(P):
                cp.ring_step_accumulate(gq, gk, gv, P, step, oa, la, order, causal)
            torch.cuda.synchronize()
            compare(oa, la, o_ref, l_ref, tol, f"suffix accumulate {case} {order} causal={causal}")
        banner("suffix fused", case, causal)
        of, lf = cp.ring_prefill_fused(gq, gk, gv, P, causal)
        torch.cuda.synchronize()
        compare(of, lf, o_ref, l_ref, tol, f"suffix fused {case} causal={causal}")


def test_suffix_2048_new_tokens_on_128k_context(cp):
    """2048 new tokens against a 131072-token cached context (K/V length 133120), 16 ranks, 16 query
    heads on 1 KV head: every query row of every path against the fp64 oracle.  The selection rule
    picks Pass-Q here (it moves ~0.38 GB against ~1.02 GB for Pass-KV)."""
    B, Sq, Skv, P, Hq, Hkv, D = 1, 2048, 133120, 16, 16, 1, 128
    q = draw(811, (B, Sq, Hq, D), torch.bfloat16, 0)
    k = draw(811, (B, Skv, Hkv, D), torch.bfloat16, 1)
    v = draw(811, (B, Skv, Hkv, D), torch.bfloat16, 2)
    gq, gk, gv = q.to(DEV), k.to(DEV), v.to(DEV)
    order, bkv, bq = cp.ring_select_order(gq, gk, P, True)
    assert order == "pass_q" and bkv == 1_022_361_600 and bq == 379_453_440
    t0 = time.perf_counter()
    banner("2048 on 128K", "oracle")
    o_ref, l_ref = suffix_reference(q, k, v, True)
    print(f"[oracle] 2048 x 133120: {time.perf_counter() - t0:.1f} s", flush=True)
    outs = {}
    for order in ("pass_kv", "pass_q", "auto"):
        banner("2048 on 128K", order)
        outs[order] = cp.ring_prefill(gq, gk, gv, P, order, True)
        torch.cuda.synchronize()
        compare(*outs[order], o_ref, l_ref, BF16_TOL, f"2048 on 128K {order}")
    assert torch.equal(outs["auto"][0], outs["pass_q"][0])
    assert (outs["pass_kv"][0] - outs["pass_q"][0]).abs().max().item() <= 1e-5
    banner("2048 on 128K", "accumulate pass_q")
    oa = torch.empty(B, Sq, Hq, D, device=DEV)
    la = torch.empty(B, Sq, Hq, device=DEV)
    for step in range(P):
        cp.ring_step_accumulate(gq, gk, gv, P, step, oa, la, "auto", True)
    torch.cuda.synchronize()
    compare(oa, la, o_ref, l_ref, BF16_TOL, "2048 on 128K accumulate auto")
    banner("2048 on 128K", "fused")
    of, lf = cp.ring_prefill_fused(gq, gk, gv, P, True)
    torch.cuda.synchronize()
    compare(of, lf, o_ref, l_ref, BF16_TOL, "2048 on 128K fused")


# ----------------------------------------------------------------------------
# KV cache shards
# ----------------------------------------------------------------------------

def nan_shards(n, B, cap, H, D, dtype):
    return [torch.full((B, cap, H, D), float("nan"), dtype=dtype, device=DEV) for _ in range(n)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_kv_cache_write_and_append_are_exact_copies(cp, dtype):
    B, S, H, D, P, cap = 2, 4096, 2, 128, 4, 1100
    k, v = draw(901, (B, S, H, D), dtype, 1).to(DEV), draw(901, (B, S, H, D), dtype, 2).to(DEV)
    ks, vs = nan_shards(P, B, cap, H, D, dtype), nan_shards(P, B, cap, H, D, dtype)
    banner("cache write", dtype)
    cp.kv_cache_write(k, v, P, ks, vs)
    torch.cuda.synchronize()
    C = S // P
    for r in range(P):
        assert torch.equal(ks[r][:, :C], k[:, r * C:(r + 1) * C]) and torch.equal(vs[r][:, :C], v[:, r * C:(r + 1) * C])
        assert torch.isnan(ks[r][:, C:].float()).all() and torch.isnan(vs[r][:, C:].float()).all()
    kn, vn = draw(902, (B, 3, H, D), dtype, 1).to(DEV), draw(902, (B, 3, H, D), dtype, 2).to(DEV)
    banner("cache append", dtype)
    cp.kv_cache_append(kn, vn, ks[2], vs[2], C)
    # a strided source: one token of a wider buffer
    wide = draw(903, (B, 1, H + 1, D), dtype, 1).to(DEV)
    cp.kv_cache_append(wide[:, :, 1:], wide[:, :, :H], ks[3], vs[3], cap - 1)
    torch.cuda.synchronize()
    assert torch.equal(ks[2][:, C:C + 3], kn) and torch.equal(vs[2][:, C:C + 3], vn)
    assert torch.isnan(ks[2][:, C + 3:].float()).all()
    assert torch.equal(ks[3][:, cap - 1:], wide[:, :, 1:]) and torch.equal(vs[3][:, cap - 1:], wide[:, :, :H])


# (B, Hq, Hkv, D, cap, lengths)
CP_DECODE_CASES = [
    (4, 16, 1, 128, 1100, [1024, 1027, 0, 517]),
    (3, 16, 2, 128, 4096, [4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096]),
    (2, 40, 1, 128, 700, [700, 1, 65]),
    (5, 8, 1, 64, 2048, [2000, 33, 1024]),
    (1, 16, 1, 128, 300, [0, 0]),                # no key anywhere: O = 0, LSE = -inf
    (64, 16, 1, 128, 2100, [2048, 2049, 2048, 2050]),
]


@pytest.mark.parametrize("case", CP_DECODE_CASES, ids=lambda c: "B{}_H{}-{}_D{}_cap{}_n{}".format(*c[:5], len(c[5])))
def test_cp_decode_matches_oracle(cp, case):
    B, Hq, Hkv, D, cap, lengths = case
    n = len(lengths)
    q = draw(950, (B, 1, Hq, D), torch.bfloat16, 0)
    ks = [draw(951 + r, (B, cap, Hkv, D), torch.bfloat16, 1) for r in range(n)]
    vs = [draw(951 + r, (B, cap, Hkv, D), torch.bfloat16, 2) for r in range(n)]
    o_ref, l_ref = oracle.cp_decode(q, ks, vs, lengths)
    banner("cp_decode", case)
    o, l = cp.cp_decode(q.to(DEV), [x.to(DEV) for x in ks], [x.to(DEV) for x in vs], lengths)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, f"cp_decode {case}")


def test_prefill_then_decode_new_tokens_over_shards(cp):
    """A 4096-token prefill over 4 CP ranks, its K/V written into the ranks' cache shards, then
    six new tokens decoded one after another: each new token's K/V is appended to a shard (ranks
    in turn) and its query attends the whole cache through per-shard partials, checked against
    the oracle's attention of that token over every key so far in position order."""
    B, S, Hq, Hkv, D, P = 2, 4096, 16, 1, 128, 4
    C, cap = S // P, S // P + 8
    q = draw(960, (B, S, Hq, D), torch.bfloat16, 0)
    k = draw(960, (B, S, Hkv, D), torch.bfloat16, 1)
    v = draw(960, (B, S, Hkv, D), torch.bfloat16, 2)
    gq, gk, gv = q.to(DEV), k.to(DEV), v.to(DEV)
    banner("prefill then decode", "prefill")
    o, l = cp.ring_prefill(gq, gk, gv, P, "pass_kv", True)
    ks, vs = nan_shards(P, B, cap, Hkv, D, torch.bfloat16), nan_shards(P, B, cap, Hkv, D, torch.bfloat16)
    cp.kv_cache_write(gk, gv, P, ks, vs)
    torch.cuda.synchronize()
    rows = [S - 1, S // 2, 0]
    o_ref, l_ref = oracle.attention_rows(q[:, rows], k, v, rows, causal=True)
    compare(o[:, rows], l[:, rows], o_ref, l_ref, BF16_TOL, "prefill rows")
    lens = [C] * P
    k_all, v_all = k, v
    for t in range(6):
        pos = S + t
        qn = draw(970 + t, (B, 1, Hq, D), torch.bfloat16, 0)
        kn = draw(970 + t, (B, 1, Hkv, D), torch.bfloat16, 1)
        vn = draw(970 + t, (B, 1, Hkv, D), torch.bfloat16, 2)
        r = t % P
        banner("prefill then decode", f"token {pos} to shard {r}")
        cp.kv_cache_append(kn.to(DEV), vn.to(DEV), ks[r], vs[r], lens[r])
        lens[r] += 1
        od, ld = cp.cp_decode(qn.to(DEV), ks, vs, lens)
        torch.cuda.synchronize()
        k_all, v_all = torch.cat([k_all, kn], dim=1), torch.cat([v_all, vn], dim=1)
        o_ref, l_ref = oracle.partial_attention(qn, k_all, v_all, pos, 0, True)
        compare(od, ld, o_ref, l_ref, BF16_TOL, f"new token at {pos}")
        # the same through the oracle's twin on host copies of the shards
        o2, l2 = oracle.cp_decode(qn, [x.cpu() for x in ks], [x.cpu() for x in vs], lens)
        compare(od, ld, o2, l2, BF16_TOL, f"new token at {pos} (shard twin)")
