"""GPU properties that hold at any size: determinism, closed forms, causality,
guard bands, and the decode shape checked against its own definition."""
import math

import pytest
import torch

import oracle
import seeded_inputs as si
from gpu_util import BF16_TOL, banner, compare

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def cp():
    import context_attention_cpattn_amd as m
    assert torch.cuda.is_available()
    return m


def qkv(seed, S, Hq, Hkv, D, dtype=torch.bfloat16, B=1):
    return (si.draw_tensor(seed, 0, (B, S, Hq, D), dtype).to(DEV),
            si.draw_tensor(seed, 1, (B, S, Hkv, D), dtype).to(DEV),
            si.draw_tensor(seed, 2, (B, S, Hkv, D), dtype).to(DEV))


def test_bitwise_deterministic(cp):
    q, k, v = qkv(3, 2048, 8, 1, 128)
    banner("determinism ring")
    a = cp.ring_prefill(q, k, v, 4, "pass_kv", True)
    b = cp.ring_prefill(q, k, v, 4, "pass_kv", True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    banner("determinism fused")
    a = cp.ring_prefill_fused(q, k, v, 4, True)
    b = cp.ring_prefill_fused(q, k, v, 4, True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    banner("determinism accumulate")
    runs = []
    for _ in range(2):
        o = torch.empty(1, 2048, 8, 128, device=DEV)
        l = torch.empty(1, 2048, 8, device=DEV)
        for step in range(4):
            cp.ring_step_accumulate(q, k, v, 4, step, o, l, "pass_q", True)
        runs.append((o, l))
    torch.cuda.synchronize()
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])
    qd = si.draw_tensor(4, 0, (8, 1, 16, 128), torch.bfloat16).to(DEV)
    kd = si.draw_tensor(4, 1, (8, 8192, 1, 128), torch.bfloat16).to(DEV)
    vd = si.draw_tensor(4, 2, (8, 8192, 1, 128), torch.bfloat16).to(DEV)
    banner("determinism decode")
    a = cp.splitkv_decode(qd, kd, vd, 4)
    b = cp.splitkv_decode(qd, kd, vd, 4)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_zero_query_closed_form(cp):
    """Q = 0: every visible score is 0, so LSE = ln(#visible) and O is the prefix mean of V."""
    S = 1000
    _, k, v = qkv(5, S, 2, 1, 128)
    q = torch.zeros(1, S, 2, 128, dtype=torch.bfloat16, device=DEV)
    banner("zero query")
    o, l = cp.ring_prefill(q, k, v, 4, "pass_kv", True)
    torch.cuda.synchronize()
    cnt = torch.arange(1, S + 1, dtype=torch.float64)
    assert (l.double().cpu()[0, :, 0] - cnt.log()).abs().max() < 1e-5
    prefix_mean = v.double().cpu()[0, :, 0].cumsum(0) / cnt.unsqueeze(1)
    assert (o.double().cpu()[0, :, 1] - prefix_mean).abs().max() < 1e-5


def test_constant_v_gives_constant_o(cp):
    q, k, _ = qkv(6, 1536, 4, 1, 128)
    v = torch.full((1, 1536, 1, 128), 0.75, dtype=torch.bfloat16, device=DEV)
    banner("constant V")
    o, _ = cp.ring_prefill(q, k, v, 3, "pass_q", True)
    torch.cuda.synchronize()
    assert (o - 0.75).abs().max().item() < 2e-3  # only bf16 rounding of P is left


def test_causality_future_perturbation(cp):
    q, k, v = qkv(7, 1024, 4, 1, 128)
    banner("causality")
    o1, l1 = cp.ring_prefill(q, k, v, 4, "pass_kv", True)
    cut = 517
    k2, v2 = k.clone(), v.clone()
    k2[:, cut + 1:] = -k2[:, cut + 1:] * 3
    v2[:, cut + 1:] = v2[:, cut + 1:] + 5
    o2, l2 = cp.ring_prefill(q, k2, v2, 4, "pass_kv", True)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :cut + 1], o2[:, :cut + 1]) and torch.equal(l1[:, :cut + 1], l2[:, :cut + 1])
    assert not torch.equal(o1[:, cut + 1:], o2[:, cut + 1:])


def test_output_guard_bands(cp):
    """Outputs written through views inside NaN-filled buffers touch only their own elements."""
    B, S, H, D = 1, 640, 4, 128
    q, k, v = qkv(8, S, H, 1, D)
    big = torch.full((B, S + 64, H, D), float("nan"), device=DEV)
    big_l = torch.full((B, S + 64, H), float("nan"), device=DEV)
    banner("guard bands")
    cp.ring_prefill(q, k, v, 5, "pass_kv", True, out=big[:, 32:32 + S], lse=big_l[:, 32:32 + S])
    torch.cuda.synchronize()
    assert torch.isnan(big[:, :32]).all() and torch.isnan(big[:, 32 + S:]).all()
    assert torch.isnan(big_l[:, :32]).all() and torch.isnan(big_l[:, 32 + S:]).all()
    assert torch.isfinite(big[:, 32:32 + S]).all() and torch.isfinite(big_l[:, 32:32 + S]).all()


def test_peaked_rows(cp):
    """A query that matches one key much better than the rest returns (almost exactly) that key's V."""
    S, D = 256, 128
    k = torch.zeros(1, S, 1, D)
    for j in range(S):
        k[0, j, 0, j % D] = 1.0 if j < D else -1.0
    v = si.draw_tensor(9, 2, (1, S, 1, D), torch.float32)
    q = torch.zeros(1, S, 1, D)
    for i in range(S):
        q[0, i, 0, min(i, D - 1) % D] = 64.0  # scaled score 64/sqrt(128) ~ 5.7 above the rest
    qb, kb, vb = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    o_ref, l_ref = oracle.full_attention(qb, kb, vb, True)
    banner("peaked")
    o, l = cp.ring_prefill(qb.to(DEV), kb.to(DEV), vb.to(DEV), 2, "pass_kv", True)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, "peaked rows")


def test_decode_lse_of_zero_query(cp):
    B, Skv = 4, 4096
    q = torch.zeros(B, 1, 16, 128, dtype=torch.bfloat16, device=DEV)
    k = si.draw_tensor(10, 1, (B, Skv, 1, 128), torch.bfloat16).to(DEV)
    v = si.draw_tensor(10, 2, (B, Skv, 1, 128), torch.bfloat16).to(DEV)
    banner("decode zero query")
    o, l = cp.splitkv_decode(q, k, v, 8)
    torch.cuda.synchronize()
    assert (l.double() - math.log(Skv)).abs().max().item() < 1e-5
    mean = v.double().mean(dim=1, keepdim=True).expand(B, 1, 16, 128)
    assert (o.double() - mean).abs().max().item() < 1e-5


@pytest.mark.parametrize("B,Skv,G,Hkv,n,D", [(3, 1000, 16, 1, 4, 128), (2, 4096, 8, 2, 8, 128), (1, 2048, 40, 1, 2, 128),
                                              (5, 96, 16, 1, 3, 128), (2, 8192, 16, 1, 1, 128), (300, 512, 16, 1, 2, 128),
                                              (3, 1000, 16, 1, 4, 64), (2, 4096, 8, 2, 8, 64), (1, 2048, 40, 1, 2, 64)])
def test_decode_shapes(cp, B, Skv, G, Hkv, n, D):
    q = si.draw_tensor(11, 0, (B, 1, G * Hkv, D), torch.bfloat16)
    k = si.draw_tensor(11, 1, (B, Skv, Hkv, D), torch.bfloat16)
    v = si.draw_tensor(11, 2, (B, Skv, Hkv, D), torch.bfloat16)
    o_ref, l_ref = oracle.splitkv_decode(q, k, v, n)
    banner("decode", B, Skv, G, Hkv, n, D)
    o, l = cp.splitkv_decode(q.to(DEV), k.to(DEV), v.to(DEV), n)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, f"decode B{B} Skv{Skv} G{G} Hkv{Hkv} n{n} D{D}")


def test_decode_after_prefill_matches_last_row(cp):
    """The prefill's last token decoded against the same K/V, split into the prefill's CP
    chunks: split-KV decode, the one-row partial and both prefill paths compute one row."""
    S, P, B = 4096, 8, 2
    q, k, v = qkv(21, S, 16, 1, 128, B=B)
    qlast = q[:, S - 1:S]  # strided view: row S-1 of each sequence
    o_ref, l_ref = oracle.attention_rows(qlast.cpu(), k.cpu(), v.cpu(), [S - 1], causal=True)
    banner("prefill then decode", S, P)
    o, l = cp.ring_prefill(q, k, v, P, "pass_kv", True)
    of, lf = cp.ring_prefill_fused(q, k, v, P, True)
    od, ld = cp.splitkv_decode(qlast, k, v, P)
    op, lp = cp.partial(qlast, k, v, S - 1, 0, True)
    torch.cuda.synchronize()
    rows = {"ring_prefill": (o[:, S - 1:S], l[:, S - 1:S]), "fused": (of[:, S - 1:S], lf[:, S - 1:S]),
            "splitkv_decode": (od, ld), "one-row partial": (op, lp)}
    for name, (x, y) in rows.items():
        compare(x, y, o_ref, l_ref, BF16_TOL, f"last row by {name}")
    for name, (x, y) in rows.items():
        d_o = (x - od).abs().max().item()
        d_l = (y - ld).abs().max().item()
        assert d_o <= BF16_TOL.max_abs and d_l <= BF16_TOL.lse_abs, (name, d_o, d_l)


def test_side_stream_buffers_survive_reuse(cp):
    """Calls on a side stream allocate their workspace and outputs on torch's current stream; the
    binding must keep the caching allocator from handing those blocks to work queued on the default
    stream while the side stream's kernels still use them.  Each call is followed at once by large
    allocations filled on the default stream before the side stream is waited for."""
    S, P = 4096, 4
    q, k, v = qkv(31, S, 8, 1, 128)
    qd = si.draw_tensor(32, 0, (16, 1, 16, 128), torch.bfloat16).to(DEV)
    kd = si.draw_tensor(32, 1, (16, 8192, 1, 128), torch.bfloat16).to(DEV)
    vd = si.draw_tensor(32, 2, (16, 8192, 1, 128), torch.bfloat16).to(DEV)
    o_ref, l_ref = oracle.full_attention(q.cpu(), k.cpu(), v.cpu(), True)
    od_ref, ld_ref = oracle.splitkv_decode(qd.cpu(), kd.cpu(), vd.cpu(), 8)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    banner("side stream", "ring_prefill + splitkv_decode")
    o, l = cp.ring_prefill(q, k, v, P, "pass_kv", True, stream=side)
    junk = [torch.full((1 << 26,), 7.0, device=DEV) for _ in range(4)]  # 1 GiB of fills on the default stream
    od, ld = cp.splitkv_decode(qd, kd, vd, 8, stream=side.cuda_stream)  # a raw handle works too
    junk += [torch.full((1 << 26,), -3.0, device=DEV) for _ in range(4)]
    side.synchronize()
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, "ring_prefill on a side stream")
    compare(od, ld, od_ref, ld_ref, BF16_TOL, "splitkv_decode on a side stream")
    del junk


def test_concurrent_streams_bit_identical(cp):
    """Two different problems run at the same time on two streams, their ring steps interleaved,
    give the same bits as each run alone: the library keeps no state between calls that two
    streams could share (only the allocation-free decode's fixed scratch, which this does not use)."""
    qa, ka, va = qkv(41, 4096, 8, 1, 128)          # 4 chunks of 1024: the chunk walk
    qb, kb, vb = qkv(42, 2048, 16, 2, 64)          # 16 chunks of 128: per-pair launches (the whole ring packs heads)
    def run(s1, s2):
        ra = cp.ring_prefill(qa, ka, va, 4, "pass_kv", True, stream=s1)
        oa = torch.full((1, 2048, 16, 64), float("nan"), device=DEV)
        la = torch.full((1, 2048, 16), float("nan"), device=DEV)
        s2.wait_stream(torch.cuda.current_stream())  # the fills above ran on the current stream
        for step in range(16):
            with torch.cuda.stream(s2):
                cp.ring_step_accumulate(qb, kb, vb, 16, step, oa, la, "pass_q", True)
        rf = cp.ring_prefill_fused(qa, ka, va, 4, True, stream=s1)
        rb = cp.ring_prefill(qb, kb, vb, 16, "pass_q", True, stream=s2)
        return ra, (oa, la), rf, rb
    banner("concurrent streams", "alone")
    alone = run(torch.cuda.current_stream(), torch.cuda.current_stream())
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    banner("concurrent streams", "together")
    together = run(s1, s2)
    s1.synchronize()
    s2.synchronize()
    torch.cuda.synchronize()
    for name, x, y in zip(("ring prefill", "accumulating steps", "fused", "ring prefill (packed)"), alone, together):
        assert torch.equal(x[0], y[0]) and torch.equal(x[1], y[1]), f"{name}: results differ between streams"


def test_graph_capture_replays(cp):
    """The ring entry points and the allocation-free decode, given their buffers, issue only kernel
    launches on the caller's stream, so a caller can capture them in a HIP graph: the 4 accumulating
    ring steps, a Pass-Q ring prefill as per-pair launches and the merge, a Pass-KV ring prefill
    sized for the chunk walk (512 walking workgroups), the fused prefill and a decode, captured once
    and replayed three times with eager work between the replays, give the eager bits every time."""
    P = 4
    q, k, v = qkv(51, 4096, 8, 1, 128)
    qd = si.draw_tensor(52, 0, (8, 1, 16, 128), torch.bfloat16).to(DEV)
    kd = si.draw_tensor(52, 1, (8, 4096, 1, 128), torch.bfloat16).to(DEV)
    vd = si.draw_tensor(52, 2, (8, 4096, 1, 128), torch.bfloat16).to(DEV)
    bufs = {name: (torch.empty(1, 4096, 8, 128, device=DEV), torch.empty(1, 4096, 8, device=DEV))
            for name in ("acc", "ring", "fused")}
    qw, kw, vw = qkv(53, 4096, 8, 1, 128, B=4)
    bufs["walk"] = (torch.empty(4, 4096, 8, 128, device=DEV), torch.empty(4, 4096, 8, device=DEV))
    ws_w = torch.empty(cp.ring_prefill_workspace_size(qw, P, True), dtype=torch.uint8, device=DEV)
    dec = (torch.empty(8, 1, 16, 128, device=DEV), torch.empty(8, 1, 16, device=DEV))
    ws = torch.empty(cp.ring_prefill_workspace_size(q, P, True), dtype=torch.uint8, device=DEV)

    def work():
        for step in range(P):
            cp.ring_step_accumulate(q, k, v, P, step, *bufs["acc"], "pass_kv", True)
        cp.ring_prefill(q, k, v, P, "pass_q", True, out=bufs["ring"][0], lse=bufs["ring"][1], workspace=ws)
        cp.ring_prefill(qw, kw, vw, P, "pass_kv", True, out=bufs["walk"][0], lse=bufs["walk"][1], workspace=ws_w)
        cp.ring_prefill_fused(q, k, v, P, True, out=bufs["fused"][0], lse=bufs["fused"][1])
        cp.splitkv_decode_noalloc(qd, kd, vd, 8, *dec)

    banner("graph capture", "eager")
    work()
    torch.cuda.synchronize()
    ref = {name: (o.clone(), l.clone()) for name, (o, l) in bufs.items()}
    ref["decode"] = (dec[0].clone(), dec[1].clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    banner("graph capture", "capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()
    outs = dict(bufs, decode=dec)
    for rep in range(3):
        for o, l in outs.values():  # eager work between the replays
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        torch.cuda.synchronize()
        banner("graph capture", "replay", rep)
        g.replay()
        torch.cuda.synchronize()
        for name, (o, l) in outs.items():
            assert torch.equal(o, ref[name][0]) and torch.equal(l, ref[name][1]), f"replay {rep}: {name} differs"
