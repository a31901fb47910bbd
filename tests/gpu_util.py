"""Shared helpers of the GPU tests: tolerances, comparison, case banners."""
from __future__ import annotations

import sys
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Tol:
    max_abs: float
    mean_abs: float
    lse_abs: float


# bf16 inputs with fp32 accumulation against the fp64 oracle: max |dO| <= 2e-2,
# mean |dO| <= 2e-3, max |dLSE| <= 1e-3.
BF16_TOL = Tol(2e-2, 2e-3, 1e-3)
# fp32 inputs and fp32 arithmetic throughout: a few fp32 ulps of accumulated
# rounding over at most a few thousand terms.
F32_TOL = Tol(1e-4, 1e-5, 1e-4)


def banner(*parts) -> None:
    """Name the case on stdout before a GPU step, so a crash still says which one."""
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def compare(o_gpu, l_gpu, o_ref, l_ref, tol: Tol, name: str = ""):
    """Element-wise comparison of O and LSE; returns the error statistics."""
    o = o_gpu.detach().double().cpu()
    l = l_gpu.detach().double().cpu()
    o_ref = o_ref.double()
    l_ref = l_ref.double()
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    assert l.shape == l_ref.shape, (l.shape, l_ref.shape)
    ref_inf = torch.isneginf(l_ref)
    assert torch.equal(torch.isneginf(l), ref_inf), f"{name}: rows with no visible key differ"
    assert torch.isfinite(o).all(), f"{name}: non-finite output"
    err = (o - o_ref).abs()
    stats = {
        "max_abs": err.max().item() if err.numel() else 0.0,
        "mean_abs": err.mean().item() if err.numel() else 0.0,
        "lse_max_abs": (l[~ref_inf] - l_ref[~ref_inf]).abs().max().item() if (~ref_inf).any() else 0.0,
    }
    if ref_inf.any():
        assert torch.all(o[ref_inf] == 0), f"{name}: masked rows must be exactly zero"
    # Relative RMS error per head: on long rows |O| is small (~sqrt(e/n) for N(0,1) inputs), where the
    # absolute bounds alone would pass a badly wrong result.  Heads whose reference RMS is below 1e-3
    # (empty, masked or degenerate ones) are left to the absolute bounds.
    if o.dim() == 4 and o.numel():
        diff2 = ((o - o_ref) ** 2).sum(dim=(0, 1, 3))
        ref2 = (o_ref ** 2).sum(dim=(0, 1, 3))
        n_h = o.shape[0] * o.shape[1] * o.shape[3]
        big = ref2 / n_h >= 1e-6
        if big.any():
            rel = (diff2[big] / ref2[big]).sqrt()
            stats["head_rel_rms_max"] = rel.max().item()
    print(f"[parity] {name}: " + ", ".join(f"{k}={v:.3e}" for k, v in stats.items()), flush=True)
    assert stats["max_abs"] <= tol.max_abs, f"{name}: max |dO| {stats['max_abs']:.3e} > {tol.max_abs}"
    assert stats["mean_abs"] <= tol.mean_abs, f"{name}: mean |dO| {stats['mean_abs']:.3e} > {tol.mean_abs}"
    assert stats["lse_max_abs"] <= tol.lse_abs, f"{name}: max |dLSE| {stats['lse_max_abs']:.3e} > {tol.lse_abs}"
    if "head_rel_rms_max" in stats:
        assert stats["head_rel_rms_max"] <= 1e-2, f"{name}: per-head relative RMS {stats['head_rel_rms_max']:.3e} > 1e-2"
    return stats
