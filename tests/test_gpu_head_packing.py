"""Head packing of the bf16 prefill kernel, against the fp64 oracle.

A workgroup of the bf16 kernel holds 256 query rows.  When a query block has at
most 128, 64 or 32 rows and the query heads of a K/V group allow it, the
launcher can give one workgroup 2, 4 or 8 heads of the same K/V head (128, 64
or 32 rows of each), so that every wave has rows; it packs when its estimate
(rounds of workgroups over the compute units, a workgroup with two busy waves
per SIMD counted 1.64 times one with one) favours it.  The shapes below are
sized so that 256 compute units pack them (the banner prints the packing the
launcher picks on the present device), with ragged blocks and both head
dimensions; the ring case also checks that its launches, packed or not,
compute the same bits as the per-step launches and the merge.  Twelve seeded random
calls (query block 2-128 rows, context up to 1200 keys, 2-16 query heads per K/V head,
either head dimension, causal or not) add shapes no fixed case has.
"""
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
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return m


def expected_pack(n_items: int, B: int, Hq: int, Hkv: int, Sq: int) -> int:
    """The launcher's choice of log2(heads per workgroup) for a bf16 launch on this device:
    the packing with the fewest estimated units of rounds x (1.64 with two busy waves per SIMD)."""
    G = Hq // Hkv
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    hp_max = 0
    while hp_max < 3 and Sq <= (256 >> (hp_max + 1)) and G % (2 << hp_max) == 0:
        hp_max += 1
    best, choice = None, 0
    for hpl in range(hp_max + 1):
        rpb = 256 >> hpl
        wgs = n_items * B * (Hq >> hpl) * ((Sq + rpb - 1) // rpb)
        busy = min(8, (1 << hpl) * ((min(Sq, rpb) + 31) // 32))
        est = (wgs + n_cu - 1) // n_cu * (164 if busy > 4 else 100)
        if best is None or est < best:
            best, choice = est, hpl
    return choice


def packs_here() -> bool:
    """Every case below packs heads on a device of at most 256 compute units."""
    return torch.cuda.get_device_properties(0).multi_processor_count <= 256


PARTIAL_CASES = [
    # B, Sq, Skv, Hq, Hkv, D, causal
    (64, 128, 1024, 16, 1, 128, True),   # two heads per workgroup
    (128, 64, 512, 16, 2, 128, True),    # four
    (256, 20, 300, 16, 2, 64, False),    # eight, ragged rows and keys
    (128, 100, 700, 8, 2, 64, True),     # two, 28 idle rows per head
]


@pytest.mark.parametrize("case", PARTIAL_CASES, ids=lambda c: "B%d_Sq%d_Skv%d_H%d-%d_D%d_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "full"))
def test_partial_head_packing(cp, case):
    B, Sq, Skv, Hq, Hkv, D, causal = case
    hpl = expected_pack(1, B, Hq, Hkv, Sq)
    banner("head packing partial", case, "heads per workgroup", 1 << hpl)
    assert hpl > 0 or not packs_here()
    seed = 7100 + Sq + Skv
    q = si.draw_tensor(seed, 0, (B, Sq, Hq, D), torch.bfloat16)
    k = si.draw_tensor(seed, 1, (B, Skv, Hkv, D), torch.bfloat16)
    v = si.draw_tensor(seed, 2, (B, Skv, Hkv, D), torch.bfloat16)
    q_off = Skv - Sq  # the block's queries are the last Sq positions
    o_ref, l_ref = oracle.partial_attention(q, k, v, q_off, 0, causal)
    o, l = cp.partial(q.to(DEV), k.to(DEV), v.to(DEV), q_off, 0, causal)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, f"head packing {case}")


RING_CASES = [
    # B, P, Cq, Hq, Hkv, D
    (32, 4, 64, 16, 1, 128),
    (128, 2, 32, 16, 2, 64),
]


@pytest.mark.parametrize("case", RING_CASES, ids=lambda c: "B%d_P%d_C%d_H%d-%d_D%d" % c)
def test_ring_head_packing(cp, case):
    B, P, Cq, Hq, Hkv, D = case
    S = P * Cq
    hpl = expected_pack(P, B, Hq, Hkv, Cq)
    banner("head packing ring", case, "heads per workgroup (ring prefill walk)", 1 << hpl)
    assert hpl > 0 or not packs_here()
    seed = 7300 + S
    q = si.draw_tensor(seed, 0, (B, S, Hq, D), torch.bfloat16)
    k = si.draw_tensor(seed, 1, (B, S, Hkv, D), torch.bfloat16)
    v = si.draw_tensor(seed, 2, (B, S, Hkv, D), torch.bfloat16)
    o_ref, l_ref = oracle.partial_attention(q, k, v, 0, 0, True)
    gq, gk, gv = q.to(DEV), k.to(DEV), v.to(DEV)

    o, l = cp.ring_prefill(gq, gk, gv, P, "pass_kv", True)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, f"ring head packing {case}")

    ws = torch.empty(cp.ring_prefill_workspace_size(gq, P, True), dtype=torch.uint8, device=DEV)
    for step in range(P):
        cp.ring_step(gq, gk, gv, P, step, ws, "pass_kv", True)
    o_s, l_s = torch.empty_like(o), torch.empty_like(l)
    cp.ring_merge(P, ws, o_s, l_s, "pass_kv", True)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o) and torch.equal(l_s, l), "ring steps + merge differ from the ring prefill"

    oa, la = torch.full_like(o, float("nan")), torch.full_like(l, float("nan"))
    for step in range(P):
        cp.ring_step_accumulate(gq, gk, gv, P, step, oa, la, "pass_kv", True)
    torch.cuda.synchronize()
    assert (oa - o).abs().max().item() <= 1e-5 and (la - l).abs().max().item() <= 1e-5

    of, lf = cp.ring_prefill_fused(gq, gk, gv, P, True)
    torch.cuda.synchronize()
    compare(of, lf, o_ref, l_ref, BF16_TOL, f"fused head packing {case}")


N_RANDOM = 12


def draw_packing_case(i: int) -> dict:
    """A seeded random partial call whose grid is large enough to pack heads on 256 compute units."""
    import numpy as np
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=9100, spawn_key=(i,))))
    G = int(g.choice([2, 4, 8, 16]))
    Hkv = int(g.choice([1, 2]))
    Sq = int(g.integers(2, 129))
    Skv = int(g.integers(Sq, 1200))
    D = int(g.choice([64, 128]))
    causal = bool(g.random() < 0.7)
    q_off = int(g.integers(0, Skv - Sq + 1)) if causal else int(g.integers(0, 4096))
    # enough sequences for 2048 unpacked workgroups: packing wins on 256 compute units
    B = int(max(1, 2048 // (G * Hkv)))
    return dict(B=B, Sq=Sq, Skv=Skv, Hq=G * Hkv, Hkv=Hkv, D=D, causal=causal, q_off=q_off)


@pytest.mark.parametrize("i", range(N_RANDOM))
def test_random_head_packing(cp, i):
    c = draw_packing_case(i)
    hpl = expected_pack(1, c["B"], c["Hq"], c["Hkv"], c["Sq"])
    banner("random head packing", i, c, "heads per workgroup", 1 << hpl)
    seed = 7500 + i
    q = si.draw_tensor(seed, 0, (c["B"], c["Sq"], c["Hq"], c["D"]), torch.bfloat16)
    k = si.draw_tensor(seed, 1, (c["B"], c["Skv"], c["Hkv"], c["D"]), torch.bfloat16)
    v = si.draw_tensor(seed, 2, (c["B"], c["Skv"], c["Hkv"], c["D"]), torch.bfloat16)
    o_ref, l_ref = oracle.partial_attention(q, k, v, c["q_off"], 0, c["causal"])
    o, l = cp.partial(q.to(DEV), k.to(DEV), v.to(DEV), c["q_off"], 0, c["causal"])
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, f"random head packing {i}")
