"""Comparison rules between the GPU step and the oracle's results.

Floating-point outputs: per compared row, max |gpu - ref| / max |ref| must not
exceed the tolerance (elementwise relative error is ill-posed near zero).
Integer decisions: the greedy token must match exactly, except on a row the
oracle records as a near-tie (its fp32 top-1 minus top-2 logit is below
NEAR_TIE); there the GPU may return any token whose oracle logit is within
NEAR_TIE of the maximum. NaN or Inf anywhere fails.
"""
from __future__ import annotations

import math

import torch

NEAR_TIE = 1e-3
TOL = {"f32": 1e-4, "f16": 1e-2, "bf16": 1e-2}


def row_rel_err(gpu: torch.Tensor, ref: torch.Tensor) -> float:
    gpu = gpu.detach().to("cpu", torch.float64).reshape(-1)
    ref = ref.detach().to("cpu", torch.float64).reshape(-1)
    assert torch.isfinite(gpu).all(), "non-finite value in GPU output"
    den = float(ref.abs().max())
    return float((gpu - ref).abs().max()) / (den if den > 0 else 1.0)


def check_rows(gpu_rows, ref_rows, tol: float, what: str) -> float:
    worst = 0.0
    for i, (g, r) in enumerate(zip(gpu_rows, ref_rows)):
        e = row_rel_err(g, r)
        assert e <= tol, f"{what} row {i}: relative error {e:.3e} > {tol:.1e}"
        worst = max(worst, e)
    return worst


def check_argmax(gpu_tok: int, ref_tok: int, ref_logits: torch.Tensor, ref_gap: float, what: str) -> bool:
    """True if exact, False if an allowed near-tie difference; raises otherwise."""
    if gpu_tok == ref_tok:
        return True
    ref = ref_logits.detach().to("cpu", torch.float64).reshape(-1)
    assert ref_gap < NEAR_TIE, f"{what}: argmax {gpu_tok} != oracle {ref_tok} with oracle gap {ref_gap:.3e}"
    assert 0 <= gpu_tok < ref.numel() and float(ref[gpu_tok]) >= float(ref.max()) - NEAR_TIE, \
        f"{what}: near-tie row but token {gpu_tok} is not within {NEAR_TIE} of the maximum"
    return False


def first_divergence_is_near_tie(gpu_argmax: list, ref_argmax: list, ref_gap: list) -> bool:
    for g, r, gap in zip(gpu_argmax, ref_argmax, ref_gap):
        if g != r:
            return not math.isnan(gap) and gap < NEAR_TIE
    return True
