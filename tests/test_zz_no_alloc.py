"""The allocation-free split-KV decode (fixed device scratch inside the library)
against the workspace entry point it mirrors, through the C ABI.

Two calls in a row, the second with a smaller input: the second call reuses the
scratch the first one left behind, so a stale-partial mistake would show.
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


def inputs(seed, B, Skv, Hq, Hkv, D):
    return (si.draw_tensor(seed, 0, (B, 1, Hq, D), torch.bfloat16),
            si.draw_tensor(seed, 1, (B, Skv, Hkv, D), torch.bfloat16),
            si.draw_tensor(seed, 2, (B, Skv, Hkv, D), torch.bfloat16))


# (B, Skv, Hq, Hkv, D, n_chunks): the decode workload's shape first (8.4 MB of partials), then a
# smaller one with fewer partials per row, then one of D = 64 with GQA groups of 4
CASES = [(128, 32768, 16, 1, 128, 8), (3, 4096, 16, 1, 128, 4), (5, 1000, 8, 2, 64, 2)]


def test_noalloc_matches_workspace_entry_point(cp):
    for case in CASES:
        B, Skv, Hq, Hkv, D, n = case
        q, k, v = inputs(1200 + B, B, Skv, Hq, Hkv, D)
        gq, gk, gv = q.to(DEV), k.to(DEV), v.to(DEV)
        need = cp.splitkv_decode_workspace_size(gq, gk, n)
        assert need <= 64 << 20
        o_ref, l_ref = cp.splitkv_decode(gq, gk, gv, n)
        out = torch.full((B, 1, Hq, D), float("nan"), device=DEV)
        lse = torch.full((B, 1, Hq), float("nan"), device=DEV)
        banner("noalloc decode", case)
        cp.splitkv_decode_noalloc(gq, gk, gv, n, out, lse)
        torch.cuda.synchronize()
        # the same kernels on the same partial layout: bit for bit
        assert torch.equal(out, o_ref) and torch.equal(lse, l_ref), f"noalloc differs from the workspace path {case}"
        if B <= 8:
            oo, ll = oracle.splitkv_decode(q, k, v, n)
            compare(out, lse, oo, ll, BF16_TOL, f"noalloc decode {case}")


def test_noalloc_refuses_more_than_its_scratch(cp):
    # 1024 sequences x 64 heads x 8 chunk partials of 129 floats: ~270 MB, more than 64 MiB holds;
    # refused before any launch
    B, Skv, Hq, n = 1024, 64, 64, 8
    q = torch.zeros(B, 1, Hq, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(B, Skv, 1, 128, dtype=torch.bfloat16, device=DEV)
    out = torch.zeros(B, 1, Hq, 128, device=DEV)
    assert cp.splitkv_decode_workspace_size(q, k, n) > 64 << 20
    with pytest.raises(cp.CpattnError) as ei:
        cp.splitkv_decode_noalloc(q, k, k, n, out)
    assert ei.value.status == cp.ERR_WORKSPACE and "scratch" in ei.value.message
