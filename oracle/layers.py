"""Oracle building blocks: plain float64 definitions of each operation in the step.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU path
never calls it, and it shares no code with the GPU path.

Each function is written from the definition the source pages give (or the
textbook definition where the pages name the operation without spelling it
out) and computes in float64 unless told otherwise. Rounding to a storage
type happens only where the caller says the method stores a value.

Page key used in citations:
  [Serving Efficiency]  "Chapter 31 Serving Efficiency: Reuse, Kernels,
                        Speculation, and Batching" (imbrooklyn.dev)
  [Spending the Idle]   "Spending the Idle" (derivingsystems.com)
  [Serving]             "Serving" (pradyotprakash.com, inference-serving)
  [KV Cache]            "Inference at Scale: KV Cache, Prefill, and Decode"
                        (blog.truongducdung.dev)
"""
from __future__ import annotations

import math

import torch

F64 = torch.float64

_STORAGE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def storage_dtype(dt: str) -> torch.dtype:
    return _STORAGE[dt]


def round_to(x: torch.Tensor, dt: str) -> torch.Tensor:
    """Round float64 values to a storage type (round to nearest even) and back to float64.

    This is where the method stores a value in fp32 / fp16 / bf16; everything
    between two such points is carried in float64.
    """
    return x.to(_STORAGE[dt]).to(F64)


# OCP 8-bit floats: (exponent bits, mantissa bits, exponent bias, largest finite magnitude)
FP8_FORMATS = {"e4m3": (4, 3, 7, 448.0), "e5m2": (5, 2, 15, 57344.0)}


def round_fp8(x: torch.Tensor, fmt: str) -> torch.Tensor:
    """Round float64 values to an 8-bit float and return them as float64.

    [KV Cache] section 03 (end): a K/V cache may store K and V in FP8, one byte
    per value, in the e4m3 or e5m2 format. Written from the formats'
    definition: a value in the binade [2^e, 2^(e+1)) is a multiple of
    2^(e - mantissa bits); below the smallest normal binade (e < 1 - bias) the
    spacing stays at the subnormal step 2^(1 - bias - mantissa bits). Rounding
    is to the nearest multiple, ties to even; magnitudes beyond the largest
    finite value saturate to it (the reading taken here: a cache entry stays
    finite).
    """
    _, mb, bias, vmax = FP8_FORMATS[fmt]
    a = x.to(F64).abs().clamp(max=vmax)
    _, ex = torch.frexp(a)  # a = f * 2^ex with f in [0.5, 1), so a lies in [2^(ex-1), 2^ex)
    e = (ex.to(F64) - 1).clamp(min=1 - bias)
    step = torch.exp2(e - mb)
    r = (torch.round(a / step) * step).clamp(max=vmax)  # torch.round: half to even
    return torch.copysign(r, x.to(F64))


def linear(x: torch.Tensor, w: torch.Tensor, cdt: torch.dtype = F64) -> torch.Tensor:
    """y = x W^T for a weight stored row-major as [out][in] (a float64 product by default).

    [KV Cache] section 02 ("Counting FLOPs and counting bytes"): every matrix
    multiply reads the full weight once and uses it for every row passing
    through; the rows share the read. The product itself is the library matmul,
    in the compute type cdt; the result is returned as float64.
    """
    return (x.to(cdt) @ w.to(cdt).T).to(F64)


def rmsnorm(x: torch.Tensor, gain: torch.Tensor, eps: float, cdt: torch.dtype = F64) -> torch.Tensor:
    """Root-mean-square normalisation of the last axis, times a per-feature gain.

    The pages name RMSNorm as a fused step of the decode path without
    writing it out; this is the textbook definition
    y_i = x_i / sqrt(mean_j(x_j^2) + eps) * g_i, computed in cdt.
    """
    x = x.to(cdt)
    ms = (x * x).mean(dim=-1, keepdim=True)
    return (x / torch.sqrt(ms + eps) * gain.to(cdt)).to(F64)


def rope_angles(positions: torch.Tensor, head_dim: int, theta: float) -> torch.Tensor:
    """Rotary angles pos * theta^(-2i/head_dim) for i in [0, head_dim/2), float64.

    The pages name RoPE (fused with RMSNorm on the decode path, and as the
    positional encoding MLA has to carry separately in [KV Cache] section 04)
    without writing it out; this is the rotary definition with base theta.
    """
    half = head_dim // 2
    i = torch.arange(half, dtype=F64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    return positions.to(F64).unsqueeze(-1) * inv_freq


def rope(x: torch.Tensor, positions: torch.Tensor, theta: float, cdt: torch.dtype = F64) -> torch.Tensor:
    """Rotate pairs (x_i, x_{i+d/2}) of each head vector by the angle of its position.

    x: [..., n_heads, head_dim] with the leading axes matching `positions`
    (one position per row). Pairing is "rotate half": feature i is paired with
    feature i + head_dim/2. The angle is float64; cos, sin and the rotation are
    taken in cdt.
    """
    x = x.to(cdt)
    d = x.shape[-1]
    half = d // 2
    ang = rope_angles(positions, d, theta)  # [..., half]
    cos = torch.cos(ang).to(cdt).unsqueeze(-2)  # broadcast over heads
    sin = torch.sin(ang).to(cdt).unsqueeze(-2)
    a, b = x[..., :half], x[..., half:]
    return torch.cat([a * cos - b * sin, b * cos + a * sin], dim=-1).to(F64)


def attention_standard(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: torch.Tensor | None = None,
                       scale: float | None = None) -> torch.Tensor:
    """softmax(q k^T * scale) v with the full score matrix materialised.

    [KV Cache] section 07 ("Online softmax" and the standard attention it is
    compared with): scores for every (query, key) pair are formed, masked
    positions (a later key for a causal query) are set to -inf, and the
    numerically stable softmax takes the row maximum first and then the sum of
    exp(s - max). scale defaults to 1/sqrt(head_dim).

    q: [..., n_q, d]; k, v: [..., n_k, d]; mask: bool [n_q, n_k], True = keep.
    Computes in the dtype of its inputs (the step passes float64; the pages'
    own comparison runs the same function in fp32 and fp64).
    """
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    s = (q @ k.transpose(-1, -2)) * scale
    if mask is not None:
        s = s.masked_fill(~mask, float("-inf"))
    m = s.amax(dim=-1, keepdim=True)
    p = torch.exp(s - m)
    return (p / p.sum(dim=-1, keepdim=True)) @ v


def key_block_stats(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, keep: torch.Tensor | None, scale: float):
    """Softmax statistics of one block of keys, relative to the block's own maximum.

    For every query row: m = the largest scaled score in the block, l = the sum of
    exp(s - m) over the block, o = the sum of exp(s - m) v over the block. A row
    whose keys in the block are all masked has m = -inf and l = o = 0. Computes in
    the dtype of its inputs. These are the per-block sufficient statistics that
    [Serving Efficiency] section 31.4 (Example 31.2) merges instead of normalised
    tile outputs.
    """
    s = (q @ k.transpose(-1, -2)) * scale
    if keep is not None:
        s = s.masked_fill(~keep, float("-inf"))
    m = s.amax(dim=-1)
    live = torch.isfinite(m)
    e = torch.exp(s - torch.where(live, m, torch.zeros_like(m)).unsqueeze(-1))
    e = torch.where(live.unsqueeze(-1), e, torch.zeros_like(e))
    return m, e.sum(dim=-1), e @ v


def attention_blockwise(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block: int,
                        mask: torch.Tensor | None = None, scale: float | None = None) -> torch.Tensor:
    """softmax(q k^T * scale) v computed from blocks of keys, never holding a whole score row.

    [KV Cache] section 07: the online-softmax recurrence keeps a running maximum m and
    a running sum l, shrinking the old sum by exp(m_old - m_new) whenever the maximum
    grows, and FlashAttention applies the same factor to the accumulated output before
    adding a block's part. Applied to whole blocks, the recurrence is the merge of
    per-block statistics: every block's (m_b, l_b, o_b) is brought to the common
    maximum by exp(m_b - max m) and the sums are added (combine_partials), then the
    output is divided by the total sum. Works in the dtype of q (the pages run it in
    fp32 and fp64 to show that both agree to rounding).

    q: [..., n_q, d]; k, v: [..., n_k, d]; mask: bool [n_q, n_k], True = keep.
    """
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    n_k = k.shape[-2]
    stats = [key_block_stats(q, k[..., j0:j0 + block, :], v[..., j0:j0 + block, :],
                             None if mask is None else mask[:, j0:j0 + block], scale)
             for j0 in range(0, n_k, block)]
    maxes = torch.stack([st[0] for st in stats])
    sums = torch.stack([st[1] for st in stats])
    outs = torch.stack([st[2] for st in stats])
    return combine_partials(outs, sums, maxes, cdt=q.dtype)


def combine_partials(nums: torch.Tensor, dens: torch.Tensor, maxes: torch.Tensor | None = None,
                     cdt: torch.dtype = F64) -> torch.Tensor:
    """Merge per-tile softmax statistics into one normalised output.

    [Serving Efficiency] section 31.4, Example 31.2: tiles are combined by
    adding their numerators and their denominators, (sum num) / (sum den), not
    by averaging the tiles' normalised outputs. With running maxima (the
    Flash-Decoding merge of [KV Cache] section 07: each split stores its
    log-sum-exp and the splits are merged with the online-softmax rescaling),
    tile t's numerator and denominator were computed relative to exp(-m_t) and
    are first brought to the common scale exp(-max_t m_t); a tile with
    m_t = -inf (no key) carries weight 0.

    nums: [T, *S, d]; dens: [T, *S]; maxes: [T, *S] or None (S may be empty).
    Computes in cdt (float64 by default) and returns that dtype.
    """
    nums, dens = nums.to(cdt), dens.to(cdt)
    if maxes is not None:
        maxes = maxes.to(cdt)
        mstar = maxes.amax(dim=0, keepdim=True)
        w = torch.where(torch.isfinite(maxes), torch.exp(maxes - mstar), torch.zeros_like(maxes))
        dens = dens * w
        nums = nums * w.reshape(w.shape + (1,) * (nums.dim() - w.dim()))
    den = dens.sum(dim=0)
    return nums.sum(dim=0) / den.reshape(den.shape + (1,) * (nums.dim() - 1 - den.dim()))


def silu(x: torch.Tensor, cdt: torch.dtype = F64) -> torch.Tensor:
    """x * sigmoid(x) = x / (1 + exp(-x)), in cdt (float64 by default)."""
    x = x.to(cdt)
    return x / (1.0 + torch.exp(-x))


def swiglu(gate: torch.Tensor, up: torch.Tensor, cdt: torch.dtype = F64) -> torch.Tensor:
    """Gated feed-forward activation silu(gate) * up (the SwiGLU MLP of a 7B Llama-style model)."""
    return (silu(gate, cdt) * up.to(cdt)).to(F64)


def argmax_lowest(logits: torch.Tensor) -> tuple[int, float]:
    """Greedy token: index of the largest value, the lowest index on exact ties; and the
    gap between the largest and the second-largest value (0 on a tie).

    [KV Cache] section 08: with greedy decoding the verifier compares each
    draft with the target's argmax. The gap is what decides whether a
    reduction-order difference can flip that argmax (section 08's note on
    near-ties between the top two tokens).
    """
    v = logits.to(F64).reshape(-1)
    top = v.max()
    idx = int(torch.nonzero(v == top)[0, 0])
    if v.numel() < 2:
        return idx, float("inf")
    two = torch.topk(v, 2).values
    return idx, float(two[0] - two[1])
