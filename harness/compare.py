"""Comparison rules between the GPU step and the oracle's results.

Floating-point outputs: per compared row, max |gpu - ref| / max |ref| must not
exceed the tolerance (elementwise relative error is ill-posed near zero).
Integer decisions: the greedy token must match exactly, except on a row the
oracle records as a near-tie; there the GPU may return any token whose oracle
logit is within the tie slack of the maximum. The slack of a row is
max(NEAR_TIE, 2 E) where E is that row's largest absolute logit difference
between GPU and oracle: if every GPU logit is within E of the oracle's, the
GPU's argmax t satisfies ref[t] >= ref[top1] - 2E, and nothing weaker can be
promised (the verify pass and the oracle sum in different orders; [KV Cache]
section 08 notes that such a pass matches plain decoding in distribution, not
necessarily bit for bit). A wrong index
or a dropped term moves a logit by far more than 2E. NaN or Inf anywhere
fails.
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


def check_rows(gpu_rows, ref_rows, tol: float, what: str, alt_rows=None) -> float:
    """Every row within tol of the oracle's. With alt_rows (the oracle's fp32 realisation of the same
    rows), a row's bound is max(tol, 2 x the distance between the two oracle realisations): deep
    stacks amplify rounding differences at the storage points, and no correct implementation can be
    held closer to the float64 oracle than a second correct one is."""
    worst = 0.0
    for i, (g, r) in enumerate(zip(gpu_rows, ref_rows)):
        e = row_rel_err(g, r)
        bound = tol if alt_rows is None else max(tol, 2.0 * row_rel_err(alt_rows[i], r))
        assert e <= bound, f"{what} row {i}: relative error {e:.3e} > {bound:.2e}"
        worst = max(worst, e)
    return worst


def tie_slack(gpu_logits: torch.Tensor | None, ref_logits: torch.Tensor) -> float:
    """max(NEAR_TIE, 2 x the row's largest |gpu - oracle| logit difference)."""
    if gpu_logits is None:
        return NEAR_TIE
    g = gpu_logits.detach().to("cpu", torch.float64).reshape(-1)
    r = ref_logits.detach().to("cpu", torch.float64).reshape(-1)
    assert torch.isfinite(g).all(), "non-finite value in GPU logits"
    return max(NEAR_TIE, 2.0 * float((g - r).abs().max()))


def check_argmax(gpu_tok: int, ref_tok: int, ref_logits: torch.Tensor, ref_gap: float, what: str,
                 gpu_logits: torch.Tensor | None = None) -> bool:
    """True if exact, False if an allowed near-tie difference; raises otherwise."""
    if gpu_tok == ref_tok:
        return True
    ref = ref_logits.detach().to("cpu", torch.float64).reshape(-1)
    slack = tie_slack(gpu_logits, ref_logits)
    assert ref_gap < slack, \
        f"{what}: argmax {gpu_tok} != oracle {ref_tok} with oracle gap {ref_gap:.3e} (tie slack {slack:.3e})"
    assert 0 <= gpu_tok < ref.numel() and float(ref[gpu_tok]) >= float(ref.max()) - slack, \
        f"{what}: near-tie row but token {gpu_tok} is not within {slack:.3e} of the maximum"
    return False


def first_divergence_is_near_tie(gpu_argmax: list, ref_argmax: list, ref_gap: list, slack: list | None = None) -> bool:
    slack = slack or [NEAR_TIE] * len(ref_gap)
    for g, r, gap, s in zip(gpu_argmax, ref_argmax, ref_gap, slack):
        if g != r:
            return not math.isnan(gap) and gap < s
    return True


def check_kv8(got, want, what: str, max_frac: float = 0.01) -> int:
    """K/V rows of an 8-bit cache. Both sides round the rotated value once to the format; their
    pre-rounding values differ by fp32-versus-float64 rounding, so an element may land on the
    neighbouring value of the format where the value sits on a rounding boundary. Every element
    must be equal or one value of the format apart, and at most max_frac of them may differ.
    Returns the number of differing elements."""
    import torch

    g, w = got.flatten(), want.flatten()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(g.dtype).double()
    table = torch.unique(codes[torch.isfinite(codes)])  # every finite value of the format, sorted
    gd, wd = g.double(), w.double()
    diff = gd != wd
    n = int(diff.sum())
    if n:
        ig = torch.searchsorted(table, gd[diff])
        iw = torch.searchsorted(table, wd[diff])
        assert bool(((ig - iw).abs() <= 1).all()), f"{what}: an element is more than one value of the format off"
        assert n <= max_frac * g.numel(), f"{what}: {n} of {g.numel()} elements differ"
    return n
