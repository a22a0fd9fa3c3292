"""Comparison rules between the GPU step and the oracle's results.

Floating-point outputs: per compared row, max |gpu - ref| / max |ref| must not
exceed the tolerance (elementwise relative error is ill-posed near zero).
Given the oracle's fp32 realisation of the same rows (``alt``), a row's bound
is max(tol, 2 x the relative distance between the two oracle realisations):
through a deep stack the rounding differences at the storage points compound,
and no correct implementation can be held closer to the float64 oracle than a
second correct one is. For the rows one sequence wrote in one layer, the
distance is taken as the largest over those rows (one depth of compounding, so
one scale; a single row's distance is a noisy sample of it). Both bounds
depend on the oracle alone.

Integer decisions: the greedy token must match exactly, except on a row the
oracle records as a near-tie; there the GPU may return any token whose oracle
logit is within the row's tie slack of the maximum. The slack is
max(NEAR_TIE, 2 E_alt), where E_alt is the row's largest absolute difference
between the oracle's fp32 and float64 realisations (NEAR_TIE alone when no fp32
realisation is given). Two correct implementations that differ only in
rounding order can disagree on a token only where the top-2 gap is of the size
of their logit differences ([KV Cache] section 08: a verify pass matches plain
decoding in distribution, not necessarily bit for bit), and the oracle's own
two realisations measure that size without looking at the GPU. A wrong index,
sign or dropped term moves a logit by far more. NaN or Inf anywhere fails.
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


def check_rows(gpu_rows, ref_rows, tol: float, what: str, alt_rows=None, alt_group: bool = False) -> float:
    """Every row within tol of the oracle's. With alt_rows (the oracle's fp32 realisation of the same
    rows), a row's bound is max(tol, 2 x the distance between the two oracle realisations). With
    alt_group, the rows are one sequence's rows of one layer (or its logit rows), which carry the same
    depth of compounded rounding; the drift scale is then the largest of their fp32-oracle distances
    rather than each row's own single sample of it."""
    worst = 0.0
    alt_err = [row_rel_err(a, r) for a, r in zip(alt_rows, ref_rows)] if alt_rows is not None else None
    for i, (g, r) in enumerate(zip(gpu_rows, ref_rows)):
        e = row_rel_err(g, r)
        if alt_err is None:
            bound = tol
        else:
            bound = max(tol, 2.0 * (max(alt_err) if alt_group else alt_err[i]))
        assert e <= bound, f"{what} row {i}: relative error {e:.3e} > {bound:.2e}"
        worst = max(worst, e)
    return worst


def tie_slack(alt_logits: torch.Tensor | None, ref_logits: torch.Tensor) -> float:
    """max(NEAR_TIE, 2 x the row's largest |fp32 oracle - float64 oracle| logit difference)."""
    if alt_logits is None:
        return NEAR_TIE
    a = alt_logits.detach().to("cpu", torch.float64).reshape(-1)
    r = ref_logits.detach().to("cpu", torch.float64).reshape(-1)
    assert torch.isfinite(a).all(), "non-finite value in the oracle's fp32 logits"
    return max(NEAR_TIE, 2.0 * float((a - r).abs().max()))


def check_argmax(gpu_tok: int, ref_tok: int, ref_logits: torch.Tensor, ref_gap: float, what: str,
                 alt_logits: torch.Tensor | None = None) -> bool:
    """True if exact, False if an allowed near-tie difference; raises otherwise."""
    if gpu_tok == ref_tok:
        return True
    ref = ref_logits.detach().to("cpu", torch.float64).reshape(-1)
    slack = tie_slack(alt_logits, ref_logits)
    assert ref_gap < slack, \
        f"{what}: argmax {gpu_tok} != oracle {ref_tok} with oracle gap {ref_gap:.3e} (tie slack {slack:.3e})"
    assert 0 <= gpu_tok < ref.numel() and float(ref[gpu_tok]) >= float(ref.max()) - slack, \
        f"{what}: near-tie row but token {gpu_tok} is not within {slack:.3e} of the maximum"
    return False


class TieLog:
    """check_argmax over many rows, counting what the near-tie rule let through.

    rows: rows checked; under_slack: rows whose oracle top-2 gap is below their slack (the only rows
    where a difference is allowed); differ: rows whose GPU token differs from the oracle's.
    """

    def __init__(self):
        self.rows = 0
        self.under_slack = 0
        self.differ = 0
        self.max_slack = 0.0

    def check(self, gpu_tok, ref_tok, ref_logits, ref_gap, what, alt_logits=None) -> bool:
        s = tie_slack(alt_logits, ref_logits)
        self.rows += 1
        self.max_slack = max(self.max_slack, s)
        if not math.isnan(ref_gap) and ref_gap < s:
            self.under_slack += 1
        exact = check_argmax(gpu_tok, ref_tok, ref_logits, ref_gap, what, alt_logits)
        self.differ += not exact
        return exact

    def report(self) -> str:
        assert self.differ <= self.under_slack
        return (f"{self.differ} near-tie rows differ (of {self.under_slack} rows under their slack, "
                f"{self.rows} rows, largest slack {self.max_slack:.2e})")


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
