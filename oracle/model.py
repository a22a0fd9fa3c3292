"""Oracle for one batched decode / verify step over contiguous per-sequence K/V.

TEST INFRASTRUCTURE (see oracle/__init__.py): plain, slow and float64.

What the step computes ([KV Cache] section 02 "The two phases of a request",
[Spending the Idle] sections 12.2-12.3, [KV Cache] section 08 "The idea"):
every sequence b brings K_b new tokens. Row i of sequence b sits at position
ctx_b + i, where ctx_b is the number of positions already in that sequence's
K/V cache. Every row computes its own q, k, v; its k and v are appended to the
cache; its attention reads all cached K/V of its own sequence up to and
including its own position (the causal mask, [KV Cache] section 07); old
queries are never needed again ([KV Cache] section 03). Rows of a sequence
are causal among themselves, so a K-row pass is a short prefill ([KV Cache]
section 08: the verify pass over the prefix plus k guesses). All rows of all
sequences go through every weight matrix together ([KV Cache] section 06,
selective batching: weight products batched over all tokens, attention per
sequence).

The block (the pages give the 7B shape as Llama 2 7B, MHA with 32 query and
32 KV heads, [KV Cache] section 03 code sample 2 output): pre-norm RMSNorm,
rotary q/k, softmax attention with scale 1/sqrt(head_dim), output projection
with a residual add, pre-norm RMSNorm, SwiGLU MLP with a residual add; a final
RMSNorm and an untied LM head give fp32 logits for the rows that need them
([KV Cache] section 02 code sample 1 keeps only the rows whose logits are
used).

Storage points (the only places values are rounded):
  * the residual stream is fp32;
  * the inputs of every weight product (normalised activations, the attention
    output, the gated MLP activation) are stored in the model's dtype;
  * q, and the k and v written to the cache, are stored in the model's dtype
    after rotation; with an 8-bit cache ([KV Cache] section 03: e4m3 or e5m2)
    k and v are rounded once, from the rotated value, to that format;
  * logits are fp32 and the argmax is taken on the fp32 values.
Everything between two storage points is float64.

decode_step(..., compute="f32") carries those in-between values in fp32
instead (torch's fp32 CPU kernels: other rounding, other summation order).
It is a second correct realisation of the same storage points, used only to
measure how far two correct implementations drift apart through the layers,
the way [KV Cache] section 07 runs one attention in fp32 and in fp64 and
reads the difference as the size of rounding.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

from .layers import F64, argmax_lowest, attention_standard, linear, rmsnorm, rope, round_fp8, round_to, swiglu


@dataclass
class SeqState:
    """One sequence's contiguous K/V cache and the rows it brings to this step.

    kv: [n_layers][2][capacity][n_kv_heads][head_dim] in the storage dtype;
        positions [0, ctx) hold the cache, and the step writes its rows'
        K/V at positions [ctx, ctx + len(tokens)).
    """

    kv: torch.Tensor
    ctx: int
    tokens: list
    want_logits: bool = True


@dataclass
class StepResult:
    logits: list = field(default_factory=list)   # per row: fp32-valued float64 [vocab] tensor, or None
    argmax: list = field(default_factory=list)   # per row: int, or -1 for rows without logits
    gap: list = field(default_factory=list)      # per row: top1 - top2 of the fp32 logits, or nan


def _w(t: torch.Tensor) -> torch.Tensor:
    return t.to(F64)


def decode_step(dims, weights: dict, seqs: list[SeqState], layer_hook=None, compute: str = "f64") -> StepResult:
    """Run one step for all rows of all sequences; updates each seq.kv in place."""
    cdt = {"f64": F64, "f32": torch.float32}[compute]
    dt = dims.dtype
    kv8 = getattr(dims, "kv_dtype", None)  # "e4m3" / "e5m2" for an 8-bit K/V cache, else None
    H, Hkv, Dh = dims.n_heads, dims.n_kv_heads, dims.head_dim
    group = H // Hkv  # query heads per KV head (1 for MHA)
    rows = [(b, i) for b, s in enumerate(seqs) for i in range(len(s.tokens))]
    M = len(rows)
    res = StepResult()
    if M == 0:
        return res
    pos = torch.tensor([seqs[b].ctx + i for (b, i) in rows], dtype=torch.int64)
    tok = torch.tensor([seqs[b].tokens[i] for (b, i) in rows], dtype=torch.int64)
    for s in seqs:
        assert s.ctx + len(s.tokens) <= s.kv.shape[2], "cache capacity too small"

    # embedding lookup into the fp32 residual stream
    x = round_to(weights["embed"][tok].to(F64), "f32")

    for l in range(dims.n_layers):
        lw = weights["layers"][l]
        # --- attention block ---
        xn = round_to(rmsnorm(x, lw["attn_norm"], dims.eps, cdt), dt)
        q = linear(xn, lw["wq"], cdt).reshape(M, H, Dh)
        k = linear(xn, lw["wk"], cdt).reshape(M, Hkv, Dh)
        v = linear(xn, lw["wv"], cdt).reshape(M, Hkv, Dh)
        q = round_to(rope(q, pos, dims.rope_theta, cdt), dt)
        if kv8:  # an 8-bit cache: k and v go once from the rotated value to the cache's format
            k = round_fp8(rope(k, pos, dims.rope_theta, cdt), kv8)
            v = round_fp8(v, kv8)
        else:
            k = round_to(rope(k, pos, dims.rope_theta, cdt), dt)
            v = round_to(v, dt)
        for r, (b, i) in enumerate(rows):  # append this step's K/V rows to each cache
            p = int(pos[r])
            seqs[b].kv[l, 0, p] = k[r].to(seqs[b].kv.dtype)
            seqs[b].kv[l, 1, p] = v[r].to(seqs[b].kv.dtype)
        o = torch.empty(M, H, Dh, dtype=F64)
        r0 = 0
        for b, s in enumerate(seqs):
            n_rows = len(s.tokens)
            if n_rows == 0:
                continue
            n_keys = s.ctx + n_rows
            K = s.kv[l, 0, :n_keys].to(cdt)  # [n_keys][Hkv][Dh]
            V = s.kv[l, 1, :n_keys].to(cdt)
            # row i (position ctx + i) keeps keys 0..ctx + i
            keep = torch.arange(n_keys).unsqueeze(0) <= (s.ctx + torch.arange(n_rows)).unsqueeze(1)
            for h in range(H):
                kh = K[:, h // group, :]
                vh = V[:, h // group, :]
                o[r0:r0 + n_rows, h, :] = attention_standard(q[r0:r0 + n_rows, h, :].to(cdt), kh, vh, keep,
                                                             1.0 / math.sqrt(Dh))
            r0 += n_rows
        o = round_to(o.reshape(M, H * Dh), dt)
        x = round_to(x + linear(o, lw["wo"], cdt), "f32")
        # --- MLP block ---
        xn2 = round_to(rmsnorm(x, lw["ffn_norm"], dims.eps, cdt), dt)
        hmid = round_to(swiglu(linear(xn2, lw["wg"], cdt), linear(xn2, lw["wu"], cdt), cdt), dt)
        x = round_to(x + linear(hmid, lw["wd"], cdt), "f32")
        if layer_hook is not None:
            layer_hook(l, x)

    want = [r for r, (b, i) in enumerate(rows) if seqs[b].want_logits]
    res.logits = [None] * M
    res.argmax = [-1] * M
    res.gap = [float("nan")] * M
    if want:
        xf = round_to(rmsnorm(x[want], weights["final_norm"], dims.eps, cdt), dt)
        logits = round_to(linear(xf, weights["lm_head"], cdt), "f32")
        for j, r in enumerate(want):
            res.logits[r] = logits[j]
            res.argmax[r], res.gap[r] = argmax_lowest(logits[j])
    return res


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int, bytes_per_value: int) -> int:
    """[KV Cache] section 03 "Bytes per token": 2 (K and V) x layers x KV heads x head_dim x bytes."""
    return 2 * n_layers * n_kv_heads * head_dim * bytes_per_value


def param_count(dims) -> int:
    """Parameters of the decoder: embedding, per-layer norms and projections, final norm, untied head."""
    D, F, V = dims.d_model, dims.ffn, dims.vocab
    q, kv = dims.n_heads * dims.head_dim, dims.n_kv_heads * dims.head_dim
    per_layer = D + q * D + 2 * kv * D + D * q + D + 3 * F * D
    return V * D + dims.n_layers * per_layer + D + V * D


def streamed_weight_bytes(dims) -> int:
    """Bytes of weights one step streams: every per-layer tensor, the final norm and the head.

    The embedding is gathered row by row, not streamed ([Spending the Idle]
    section 12.2: one pass reads the weights once whatever the token count).
    """
    return (param_count(dims) - dims.vocab * dims.d_model) * dims.elem_bytes
