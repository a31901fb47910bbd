"""Non-contiguous tensors on the ring and decode paths, against the fp64 oracle.

Every entry point takes [B, S, H, D] descriptors with their own batch, token and
head strides (the last axis contiguous).  Here the inputs are head slices of
wider tensors and the outputs are views into wider buffers filled with NaN: the
results must match the oracle, and nothing outside the views may change.  The
shapes reach the chunk walk (enough walking workgroups for it on 256 compute
units), the per-pair launches with the merge kernel (bf16 output), the
accumulating ring steps, the fused prefill, the split-KV decode, the decode
over cache shards, and the cache write and append (bit-exact copies).
"""
import pytest
import torch

import oracle
import seeded_inputs as si
from gpu_util import BF16_TOL, banner, compare

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAN = float("nan")


@pytest.fixture(scope="module")
def cp():
    import context_attention_cpattn_amd as m
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return m


def sliced_inputs(seed, B, S, H, Hkv, D):
    """q, k, v as head slices of tensors two heads wider (CPU copies for the oracle, GPU views)."""
    big = [si.draw_tensor(seed, i, (B, S, h + 2, D), torch.bfloat16) for i, h in enumerate((H, Hkv, Hkv))]
    cpu = [t[:, :, 1:t.shape[2] - 1] for t in big]
    gpu = [t.to(DEV)[:, :, 1:t.shape[2] - 1] for t in big]
    for g in gpu:
        assert not g.is_contiguous()
    return cpu, gpu


def out_views(B, S, H, D, dtype=torch.float32):
    """O as heads [0, H) of a buffer one head wider, LSE as heads [2, 2 + H) of one three wider."""
    ob = torch.full((B, S, H + 1, D), NAN, dtype=dtype, device=DEV)
    lb = torch.full((B, S, H + 3), NAN, device=DEV)
    return ob, lb, ob[:, :, :H], lb[:, :, 2:2 + H]


def guards_intact(ob, lb, H):
    assert torch.isnan(ob[:, :, H]).all(), "the output head past the view was written"
    assert torch.isnan(lb[:, :, :2]).all() and torch.isnan(lb[:, :, 2 + H:]).all(), "LSE outside the view was written"


@pytest.mark.parametrize("order", ["pass_kv", "pass_q"])
def test_ring_prefill_walk_strided(cp, order):
    """Chunk walk (P = 8 chunks of 128 tokens, 4 x 16 heads: 512 walking workgroups)."""
    B, P, C, H, Hkv, D = 4, 8, 128, 16, 2, 128
    S = P * C
    (q, k, v), (gq, gk, gv) = sliced_inputs(8101, B, S, H, Hkv, D)
    o_ref, l_ref = oracle.full_attention(q, k, v, True)
    ob, lb, o, l = out_views(B, S, H, D)
    banner("strided ring prefill walk", order, (B, S, H, Hkv, D, P))
    cp.ring_prefill(gq, gk, gv, P, order, True, out=o, lse=l)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, f"strided ring prefill walk {order}")
    guards_intact(ob, lb, H)


def test_ring_prefill_per_pair_strided_bf16_out(cp):
    """Per-pair launches and the merge kernel (few workgroups), bf16 output view, D = 64."""
    B, P, C, H, Hkv, D = 2, 4, 120, 6, 3, 64
    S = P * C
    (q, k, v), (gq, gk, gv) = sliced_inputs(8102, B, S, H, Hkv, D)
    o_ref, l_ref = oracle.full_attention(q, k, v, True)
    ob, lb, o, l = out_views(B, S, H, D, torch.bfloat16)
    banner("strided ring prefill per pair", (B, S, H, Hkv, D, P))
    cp.ring_prefill(gq, gk, gv, P, "pass_kv", True, out=o, lse=l)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, "strided ring prefill per pair (bf16 out)")
    guards_intact(ob, lb, H)


@pytest.mark.parametrize("order", ["pass_kv", "pass_q"])
def test_ring_accumulate_and_fused_strided(cp, order):
    """Accumulating ring steps into fp32 views, and the fused prefill into views of its own."""
    B, P, C, H, Hkv, D = 2, 4, 200, 8, 1, 128
    S = P * C
    (q, k, v), (gq, gk, gv) = sliced_inputs(8103, B, S, H, Hkv, D)
    o_ref, l_ref = oracle.full_attention(q, k, v, True)
    ob, lb, o, l = out_views(B, S, H, D)
    banner("strided ring accumulate", order, (B, S, H, Hkv, D, P))
    for step in range(P):
        cp.ring_step_accumulate(gq, gk, gv, P, step, o, l, order, True)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, f"strided ring accumulate {order}")
    guards_intact(ob, lb, H)
    fb, flb, fo, fl = out_views(B, S, H, D)
    banner("strided ring fused", (B, S, H, Hkv, D, P))
    cp.ring_prefill_fused(gq, gk, gv, P, True, out=fo, lse=fl)
    torch.cuda.synchronize()
    compare(fo, fl, o_ref, l_ref, BF16_TOL, "strided ring fused")
    guards_intact(fb, flb, H)


def test_splitkv_decode_strided(cp):
    """One new token per sequence (16 query heads on 1 K/V head) against a cache of 4096 tokens in
    4 chunks, all as head slices; output into views."""
    B, Skv, H, Hkv, D, n = 8, 4096, 16, 1, 128, 4
    qb = si.draw_tensor(8104, 0, (B, 1, H + 2, D), torch.bfloat16)
    kb = si.draw_tensor(8104, 1, (B, Skv, Hkv + 2, D), torch.bfloat16)
    vb = si.draw_tensor(8104, 2, (B, Skv, Hkv + 2, D), torch.bfloat16)
    q, k, v = qb[:, :, 1:H + 1], kb[:, :, 1:Hkv + 1], vb[:, :, 1:Hkv + 1]
    o_ref, l_ref = oracle.splitkv_decode(q, k, v, n)
    gq, gk, gv = qb.to(DEV)[:, :, 1:H + 1], kb.to(DEV)[:, :, 1:Hkv + 1], vb.to(DEV)[:, :, 1:Hkv + 1]
    ob, lb, o, l = out_views(B, 1, H, D)
    banner("strided split-KV decode", (B, Skv, H, Hkv, D, n))
    cp.splitkv_decode(gq, gk, gv, n, out=o, lse=l)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, "strided split-KV decode")
    guards_intact(ob, lb, H)


def test_cp_decode_strided_shards(cp):
    """Decode over 3 cache shards that are head slices of wider caches, ragged fill levels."""
    B, cap, H, Hkv, D = 4, 700, 8, 2, 64
    lengths = [700, 333, 64]
    qb = si.draw_tensor(8105, 0, (B, 1, H + 2, D), torch.bfloat16)
    kbs = [si.draw_tensor(8105, 1 + r, (B, cap, Hkv + 1, D), torch.bfloat16) for r in range(3)]
    vbs = [si.draw_tensor(8105, 4 + r, (B, cap, Hkv + 1, D), torch.bfloat16) for r in range(3)]
    q = qb[:, :, 2:]
    ks, vs = [t[:, :, 1:] for t in kbs], [t[:, :, 1:] for t in vbs]
    o_ref, l_ref = oracle.cp_decode(q, ks, vs, lengths)
    gq = qb.to(DEV)[:, :, 2:]
    gks, gvs = [t.to(DEV)[:, :, 1:] for t in kbs], [t.to(DEV)[:, :, 1:] for t in vbs]
    ob, lb, o, l = out_views(B, 1, H, D)
    banner("strided cp decode", (B, cap, H, Hkv, D, lengths))
    cp.cp_decode(gq, gks, gvs, lengths, out=o, lse=l)
    torch.cuda.synchronize()
    compare(o, l, o_ref, l_ref, BF16_TOL, "strided cp decode")
    guards_intact(ob, lb, H)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_kv_cache_write_strided(cp, dtype):
    """K and V as head slices of differently shaped tensors (so their strides differ and they go in
    launches of their own), written into shards that are head slices of wider NaN buffers; then one
    appended token.  A copy: bit-exact against plain slicing, the head outside each view untouched."""
    B, S, H, D, P, cap = 2, 2048, 3, 64, 4, 600
    kb = si.draw_tensor(8106, 0, (B, S, H + 2, D), dtype).to(DEV)
    vb = si.draw_tensor(8106, 1, (B, S, H + 1, D), dtype).to(DEV)
    k, v = kb[:, :, 1:H + 1], vb[:, :, :H]
    assert k.stride() != v.stride()
    kbig = [torch.full((B, cap, H + 1, D), NAN, dtype=dtype, device=DEV) for _ in range(P)]
    vbig = [torch.full((B, cap, H + 1, D), NAN, dtype=dtype, device=DEV) for _ in range(P)]
    ks, vs = [t[:, :, 1:] for t in kbig], [t[:, :, :H] for t in vbig]
    banner("strided cache write", dtype)
    cp.kv_cache_write(k, v, P, ks, vs)
    torch.cuda.synchronize()
    C = S // P
    for r in range(P):
        assert torch.equal(ks[r][:, :C], k[:, r * C:(r + 1) * C]) and torch.equal(vs[r][:, :C], v[:, r * C:(r + 1) * C])
        assert torch.isnan(ks[r][:, C:].float()).all() and torch.isnan(vs[r][:, C:].float()).all()
        assert torch.isnan(kbig[r][:, :, 0].float()).all() and torch.isnan(vbig[r][:, :, H].float()).all()
    new = si.draw_tensor(8107, 0, (B, 1, 2 * H, D), dtype).to(DEV)
    banner("strided cache append", dtype)
    cp.kv_cache_append(new[:, :, :H], new[:, :, H:], ks[1], vs[1], C)
    torch.cuda.synchronize()
    assert torch.equal(ks[1][:, C:C + 1], new[:, :, :H]) and torch.equal(vs[1][:, C:C + 1], new[:, :, H:])
    assert torch.isnan(ks[1][:, C + 1:].float()).all() and torch.isnan(kbig[1][:, :, 0].float()).all()
