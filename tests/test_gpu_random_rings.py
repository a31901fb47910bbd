"""Seeded random ring shapes through every ring entry point, against the fp64 oracle.

Each case draws a ring from a fixed stream: chunk count, Q and K/V chunk lengths
(queries are the last Sq positions of the K/V sequence; K/V chunks a multiple
of 64 tokens in most cases, ragged in the others), batch, query and K/V heads,
head dimension, dtype, mask, ring order, output dtype, whether the LSE is
wanted, and whether q, k and v are strided views of larger tensors.  These
grids are small, so their bf16 rings run as per-pair launches and the merge; a
second stream draws bf16 rings whose batch is sized for two walking query tiles
per compute unit (on 256 of them), so that the per-owner chunk walk with its
merge tail runs (with head packing where the query chunks are short, and with
the owner's own partial kept in registers where it is the last one a tile
computes).  For every case:

* ``ring_prefill`` against ``oracle.partial_attention`` over the whole sequence;
* ``ring_prefill`` equal, bit for bit, to the per-step launches followed by
  ``ring_merge`` (the same partials, merged with the same arithmetic);
* the accumulating ring steps within 1e-5 of ``ring_prefill``;
* ``ring_prefill_fused`` against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from gpu_util import BF16_TOL, F32_TOL, banner, compare

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_CASES = 40


@pytest.fixture(scope="module")
def cp():
    import context_attention_cpattn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return m


def draw_case(i: int) -> dict:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=9001, spawn_key=(i,))))
    P = int(g.choice([1, 2, 3, 4, 5, 8, 16]))
    D = int(g.choice([128, 128, 128, 64]))
    dt = "f32" if g.random() < 0.15 else "bf16"
    walk = g.random() < 0.7  # K/V chunks a multiple of 64
    Cq = int(g.choice([16, 32, 64, 96, 128, 192, 256, 320]))
    ratio = int(g.choice([1, 2, 3, 4]))
    Ckv = Cq * ratio
    if walk:
        Ckv = max(64, (Ckv + 63) // 64 * 64)
    elif Ckv % 64 == 0:
        Ckv += 32
    Cq = min(Cq, Ckv)
    # keep the fp64 oracle quick
    while P * Cq * P * Ckv > 4_000_000 and P > 1:
        P //= 2
    Hkv = int(g.choice([1, 1, 2]))
    G = int(g.choice([1, 2, 4, 8, 16]))
    return dict(P=P, B=int(g.choice([1, 2])), Cq=Cq, Ckv=Ckv, Hkv=Hkv, Hq=Hkv * G, D=D, dt=dt,
                causal=bool(g.random() < 0.75), order=str(g.choice(["pass_kv", "pass_q", "auto"])),
                out_bf16=bool(g.random() < 0.25), want_lse=bool(g.random() < 0.85), strided=bool(g.random() < 0.4))


def tensors(c: dict, seed: int):
    tdt = torch.bfloat16 if c["dt"] == "bf16" else torch.float32
    Sq, Skv = c["P"] * c["Cq"], c["P"] * c["Ckv"]
    extra = 1 if c["strided"] else 0
    qf = si.draw_tensor(seed, 0, (c["B"], Sq, c["Hq"] + extra, c["D"]), tdt)
    kf = si.draw_tensor(seed, 1, (c["B"], Skv, c["Hkv"] + extra, c["D"]), tdt)
    vf = si.draw_tensor(seed, 2, (c["B"], Skv, c["Hkv"] + extra, c["D"]), tdt)
    return qf, kf, vf


N_WALK_CASES = 12


def draw_walk_case(i: int) -> dict:
    """A seeded bf16 ring whose grid takes the chunk walk on 256 compute units."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=9002, spawn_key=(i,))))
    P = int(g.choice([2, 3, 4, 8]))
    Ckv = int(g.choice([64, 128, 192, 256, 384, 512]))
    Cq = int(g.choice([Ckv, Ckv, Ckv - 16, max(16, Ckv // 2)]))  # equal lengths, or queries shorter
    Hkv = int(g.choice([1, 2]))
    Hq = Hkv * int(g.choice([2, 4, 8, 16]))
    B = -(-512 // (P * Hq * ((Cq + 255) // 256)))  # at least 512 walking workgroups
    return dict(P=P, B=B, Cq=Cq, Ckv=Ckv, Hkv=Hkv, Hq=Hq, D=int(g.choice([128, 128, 64])), dt="bf16",
                causal=bool(g.random() < 0.75), order=str(g.choice(["pass_kv", "pass_q", "auto"])),
                out_bf16=bool(g.random() < 0.25), want_lse=bool(g.random() < 0.85), strided=bool(g.random() < 0.4))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_ring(cp, i):
    c = draw_case(i)
    banner("random ring", i, c)
    check_ring(cp, c, 5000 + i, f"random ring {i}")


@pytest.mark.parametrize("i", range(N_WALK_CASES))
def test_random_walk(cp, i):
    c = draw_walk_case(i)
    walks = c["P"] * c["B"] * c["Hq"] * ((c["Cq"] + 255) // 256) >= 2 * torch.cuda.get_device_properties(0).multi_processor_count
    banner("random walk", i, c, "walks" if walks else "per pair on this device")
    check_ring(cp, c, 6000 + i, f"random walk {i}")


def check_ring(cp, c: dict, seed: int, name: str):
    """ring_prefill against the oracle, bit-equal to the per-step launches and the merge; the
    accumulating steps within 1e-5 of it; the fused prefill against the oracle."""
    qf, kf, vf = tensors(c, seed)
    Hq, Hkv = c["Hq"], c["Hkv"]
    q, k, v = qf[:, :, :Hq], kf[:, :, :Hkv], vf[:, :, :Hkv]  # strided views when the case says so
    P, causal, order = c["P"], c["causal"], c["order"]
    Skv = P * c["Ckv"]
    o_ref, l_ref = oracle.partial_attention(q.contiguous(), k.contiguous(), v.contiguous(), Skv - q.shape[1], 0, causal)
    tol = BF16_TOL if c["dt"] == "bf16" else F32_TOL
    gq, gk, gv = (x.to(DEV)[:, :, :h] for x, h in ((qf, Hq), (kf, Hkv), (vf, Hkv)))
    assert gq.is_contiguous() == (not c["strided"])
    out_dtype = torch.bfloat16 if c["out_bf16"] else torch.float32

    o, l = cp.ring_prefill(gq, gk, gv, P, order, causal, out_dtype=out_dtype, want_lse=c["want_lse"])
    torch.cuda.synchronize()
    if c["want_lse"]:
        compare(o.float(), l, o_ref, l_ref, tol if not c["out_bf16"] else BF16_TOL, name)
    else:
        assert l is None
        err = (o.double().cpu() - o_ref).abs().max().item()
        assert err <= (tol.max_abs if not c["out_bf16"] else BF16_TOL.max_abs), f"{name}: max |dO| {err}"

    # the whole ring equals its per-step launches plus the merge, bit for bit
    o32, l32 = cp.ring_prefill(gq, gk, gv, P, order, causal)
    chosen = order if order != "auto" else cp.ring_select_order(gq, gk, P, causal)[0]
    ws = torch.empty(cp.ring_prefill_workspace_size(gq, P, causal, gk), dtype=torch.uint8, device=DEV)
    o_s = torch.empty_like(o32)
    l_s = torch.empty_like(l32)
    for step in range(P):
        cp.ring_step(gq, gk, gv, P, step, ws, chosen, causal)
    cp.ring_merge(P, ws, o_s, l_s, chosen, causal, kv_len=Skv)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o32) and torch.equal(l_s, l32), f"{name}: steps + merge differ from the ring"
    if c["out_bf16"]:
        assert torch.equal(o, o32.to(torch.bfloat16))

    # accumulating ring steps
    oa = torch.full_like(o32, float("nan"))
    la = torch.full_like(l32, float("nan"))
    for step in range(P):
        cp.ring_step_accumulate(gq, gk, gv, P, step, oa, la, chosen, causal)
    torch.cuda.synchronize()
    assert (oa - o32).abs().max().item() <= 1e-5 and (la - l32).abs().max().item() <= 1e-5

    # the fused walk
    of, lf = cp.ring_prefill_fused(gq, gk, gv, P, causal)
    torch.cuda.synchronize()
    compare(of, lf, o_ref, l_ref, tol, f"{name} (fused)")
