"""Pins for the oracle's whole step on the tiny model (CPU only).

Invariants the pages state (K-row pass == K single steps, batch == independent
runs, exact shared prefix => identical prefix K/V, causality) plus special
weight settings under which the step reduces to library routines
(torch.nn.functional.rms_norm / linear / silu, mean, logistic) or closed forms.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.layers import round_to
from oracle.model import SeqState, decode_step
from synth import workloads as W

SEED = 1001  # tiny workload, weight stream


def seq(dims, content, ctx, tokens, cap=None, want=True, kv_seed=1002):
    cap = cap or ctx + len(tokens)
    kv = torch.zeros(dims.n_layers, 2, cap, dims.n_kv_heads, dims.head_dim, dtype=dims.kv_torch_dtype)
    kv[:, :, :ctx] = W.kv_block(dims, kv_seed, content, 0, ctx)
    return SeqState(kv, ctx, list(tokens), want)


def clone(s):
    return SeqState(s.kv.clone(), s.ctx, list(s.tokens), s.want_logits)


def rel(a, b):
    return float((a - b).abs().max() / b.abs().max())


@pytest.fixture(scope="module", params=["f32", "f16", "bf16"])
def model(request):
    dims = W.TINY.with_dtype(request.param)
    return dims, W.make_weights(dims, SEED, gains="random")


def test_k_row_pass_equals_k_single_steps(model):
    dims, w = model
    toks = W.token_ids(1003, 0, 5, dims.vocab)
    s_all = seq(dims, 0, 17, toks)
    r_all = decode_step(dims, w, [s_all])
    s_one = seq(dims, 0, 17, [], cap=22)
    for i, t in enumerate(toks):
        s_one.tokens = [t]
        r = decode_step(dims, w, [s_one])
        s_one.ctx += 1
        assert rel(r.logits[0], r_all.logits[i]) < 1e-12
        assert r.argmax[0] == r_all.argmax[i]
    assert torch.equal(s_one.kv, s_all.kv)


def test_batch_equals_independent_runs(model):
    dims, w = model
    ctxs = [5, 17, 33, 64]
    toks = W.token_ids(1003, 1, 4, dims.vocab)
    batch = [seq(dims, b, c, [t]) for b, (c, t) in enumerate(zip(ctxs, toks))]
    alone = [clone(s) for s in batch]
    rb = decode_step(dims, w, batch)
    for b, s in enumerate(alone):
        r = decode_step(dims, w, [s])
        assert rel(r.logits[0], rb.logits[b]) < 1e-12
        assert r.argmax[0] == rb.argmax[b]
        assert torch.equal(s.kv, batch[b].kv)


def test_exact_shared_prefix_gives_identical_prefix_kv(model):
    dims, w = model
    prefix = W.token_ids(1003, 2, 20, dims.vocab)
    a = seq(dims, 0, 0, prefix + [1, 2, 3])
    b = seq(dims, 0, 0, prefix + [4, 5, 6, 7])
    decode_step(dims, w, [a, b])
    assert torch.equal(a.kv[:, :, :20], b.kv[:, :, :20])
    assert not torch.equal(a.kv[:, :, 20], b.kv[:, :, 20])


def test_similar_but_not_identical_prefix_differs(model):
    """Same tokens in a different order are not a shared prefix."""
    dims, w = model
    a = seq(dims, 0, 0, [10, 11, 12, 13])
    b = seq(dims, 0, 0, [11, 10, 12, 13])
    decode_step(dims, w, [a, b])
    assert not torch.equal(a.kv[:, :, 0], b.kv[:, :, 0])


def test_causality_within_a_pass(model):
    dims, w = model
    toks = W.token_ids(1003, 3, 5, dims.vocab)
    s1 = seq(dims, 7, 9, toks)
    s2 = seq(dims, 7, 9, toks[:3] + [(toks[3] + 1) % dims.vocab, toks[4]])
    r1 = decode_step(dims, w, [s1])
    r2 = decode_step(dims, w, [s2])
    for i in range(3):
        assert torch.equal(r1.logits[i], r2.logits[i])
    assert not torch.equal(r1.logits[3], r2.logits[3])
    assert torch.equal(s1.kv[:, :, :12], s2.kv[:, :, :12])


def _zero_layers(w, keep=()):
    w = {**w, "layers": [dict(l) for l in w["layers"]]}
    for l in w["layers"]:
        for name in ["wq", "wk", "wv", "wo", "wg", "wu", "wd"]:
            if name not in keep:
                l[name] = torch.zeros_like(l[name])
    return w


def _head(dims, w, x):
    xf = round_to(F.rms_norm(x, (dims.d_model,), weight=w["final_norm"].double(), eps=dims.eps), dims.dtype)
    return round_to(F.linear(xf, w["lm_head"].double()), "f32")


def test_zero_layers_reduce_to_final_norm_and_head(model):
    dims, w = model
    w0 = _zero_layers(w)
    toks = W.token_ids(1003, 4, 3, dims.vocab)
    r = decode_step(dims, w0, [seq(dims, 1, 6, toks)])
    x0 = w["embed"][torch.tensor(toks)].double()
    want = _head(dims, w, x0)
    for i in range(3):
        assert torch.equal(r.logits[i], want[i])


def test_zero_query_gives_uniform_attention_over_the_causal_window():
    """W_q = 0 makes every score 0: the attention output of a row at position p is the
    plain mean of V over positions 0..p, its own freshly written v included.

    Means of stored values often sit exactly on a rounding tie of the storage type,
    where the last bit of the summation order picks the side; so this runs in fp32
    with a 1e-6 gate (a one-ulp flip is 6e-8; a wrong window or a missing own value
    moves the logits by percents)."""
    dims = W.TINY
    w = W.make_weights(dims, SEED, gains="random")
    wz = _zero_layers(w, keep=("wk", "wv", "wo"))
    ctx, toks = 11, W.token_ids(1003, 5, 3, dims.vocab)
    s = seq(dims, 2, ctx, toks)
    cached_v = s.kv[0, 1, :ctx].double().clone()
    r = decode_step(dims, wz, [s])
    lw = w["layers"][0]
    x0 = w["embed"][torch.tensor(toks)].double()
    xn = round_to(F.rms_norm(x0, (dims.d_model,), weight=lw["attn_norm"].double(), eps=dims.eps), dims.dtype)
    v_new = round_to(F.linear(xn, lw["wv"].double()), dims.dtype).reshape(3, dims.n_kv_heads, dims.head_dim)
    allv = torch.cat([cached_v, v_new], dim=0)  # [ctx+3][H][Dh]
    for i in range(3):
        o = round_to(allv[:ctx + i + 1].mean(dim=0).reshape(-1), dims.dtype)
        x1 = round_to(x0[i] + F.linear(o, lw["wo"].double()), "f32")
        want = _head(dims, w, x1.unsqueeze(0))[0]
        assert rel(r.logits[i], want) < 1e-6


def _rotate(x, pos, theta):
    d = x.shape[-1]
    z = x[..., :d // 2] + 1j * x[..., d // 2:]
    z = z * np.exp(1j * pos * theta ** (-2.0 * np.arange(d // 2) / d))
    return np.concatenate([z.real, z.imag], axis=-1)


def test_two_keys_scale_rotary_and_residual(model):
    """ctx = 1: a row at position 1 attends to one cached key and its own key. Per head the
    output is a logistic mix of the two values with scores q.k / sqrt(head_dim)."""
    dims, w = model
    wz = _zero_layers(w, keep=("wq", "wk", "wv", "wo"))
    tok = W.token_ids(1003, 6, 1, dims.vocab)
    s = seq(dims, 3, 1, tok)
    k0 = s.kv[0, 0, 0].double().numpy()
    v0 = s.kv[0, 1, 0].double().numpy()
    r = decode_step(dims, wz, [s])
    lw = w["layers"][0]
    x0 = w["embed"][torch.tensor(tok)].double()
    xn = round_to(F.rms_norm(x0, (dims.d_model,), weight=lw["attn_norm"].double(), eps=dims.eps), dims.dtype)
    H, Dh = dims.n_heads, dims.head_dim
    q = F.linear(xn, lw["wq"].double())[0].reshape(H, Dh).numpy()
    k1 = F.linear(xn, lw["wk"].double())[0].reshape(H, Dh).numpy()
    v1 = round_to(F.linear(xn, lw["wv"].double()), dims.dtype)[0].reshape(H, Dh).numpy()
    q = round_to(torch.tensor(_rotate(q, 1, dims.rope_theta)), dims.dtype).numpy()
    k1 = round_to(torch.tensor(_rotate(k1, 1, dims.rope_theta)), dims.dtype).numpy()
    assert np.array_equal(k1, s.kv[0, 0, 1].double().numpy())
    o = np.empty((H, Dh))
    for h in range(H):
        s0 = float(q[h] @ k0[h]) / math.sqrt(Dh)
        s1 = float(q[h] @ k1[h]) / math.sqrt(Dh)
        a = 1.0 / (1.0 + math.exp(s1 - s0))
        o[h] = a * v0[h] + (1 - a) * v1[h]
    o = round_to(torch.tensor(o.reshape(-1)), dims.dtype)
    x1 = round_to(x0[0] + F.linear(o, lw["wo"].double()), "f32")
    want = _head(dims, w, x1.unsqueeze(0))[0]
    assert rel(r.logits[0], want) < 1e-10


def test_mlp_alone_is_swiglu_with_residual(model):
    dims, w = model
    wz = _zero_layers(w, keep=("wg", "wu", "wd"))
    toks = W.token_ids(1003, 7, 2, dims.vocab)
    r = decode_step(dims, wz, [seq(dims, 4, 3, toks)])
    lw = w["layers"][0]
    x0 = w["embed"][torch.tensor(toks)].double()
    xn = round_to(F.rms_norm(x0, (dims.d_model,), weight=lw["ffn_norm"].double(), eps=dims.eps), dims.dtype)
    hmid = round_to(F.silu(F.linear(xn, lw["wg"].double())) * F.linear(xn, lw["wu"].double()), dims.dtype)
    x1 = round_to(x0 + F.linear(hmid, lw["wd"].double()), "f32")
    want = _head(dims, w, x1)
    for i in range(2):
        assert rel(r.logits[i], want[i]) < 1e-12


def test_up_projection_multiplies_the_gate():
    """With W_u = 0 the MLP adds nothing, whatever W_g and W_d are."""
    dims = W.TINY
    w = W.make_weights(dims, SEED, gains="random")
    wz = _zero_layers(w, keep=("wg", "wd"))
    w0 = _zero_layers(w)
    toks = W.token_ids(1003, 8, 2, dims.vocab)
    a = decode_step(dims, wz, [seq(dims, 4, 3, toks)])
    b = decode_step(dims, w0, [seq(dims, 4, 3, toks)])
    for i in range(2):
        assert torch.equal(a.logits[i], b.logits[i])


def test_grouped_kv_heads_equal_duplicated_full_heads():
    """GQA with 2 KV heads for 4 query heads equals MHA whose K/V heads are the grouped ones duplicated."""
    g = W.ModelDims("tiny-gqa", 256, 4, 2, 64, 1024, 1000, 1, "f32")
    m = W.TINY
    wg_ = W.make_weights(g, SEED, gains="random")
    wm = {**wg_, "layers": [dict(l) for l in wg_["layers"]]}
    dup = torch.tensor([0, 0, 1, 1])
    for name in ("wk", "wv"):
        wm["layers"][0][name] = wg_["layers"][0][name].reshape(2, 64, 256)[dup].reshape(256, 256)
    toks = W.token_ids(1003, 9, 3, 1000)
    sg = seq(g, 5, 12, toks)
    sm = SeqState(sg.kv[:, :, :, dup].clone(), 12, list(toks), True)
    rg = decode_step(g, wg_, [sg])
    rm = decode_step(m, wm, [sm])
    for i in range(3):
        assert rel(rg.logits[i], rm.logits[i]) < 1e-12


def test_fp32_realisation_agrees_to_rounding(model):
    """compute="f32" keeps the storage points and changes only the arithmetic between them: on the
    all-fp32 tiny model the two realisations agree to fp32 rounding, and with fp16 / bf16 storage they
    agree within the storage type's tolerance through one layer; the cache rows they write differ only
    by a rounding step of the storage type."""
    dims, w = model
    a = [seq(dims, b, c, W.token_ids(1003, 40 + b, 2, dims.vocab)) for b, c in enumerate([5, 40])]
    b32 = [clone(s) for s in a]
    r64 = decode_step(dims, w, a)
    r32 = decode_step(dims, w, b32, compute="f32")
    bound = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}[dims.dtype]
    for x, y in zip(r64.logits, r32.logits):
        assert rel(y, x) < bound
        assert rel(y, x) > 0 or dims.dtype != "f32"  # a different summation really happened
    # per cached row (layer, K|V, position): fp32 storage differs by accumulation rounding only; fp16 /
    # bf16 storage by at most one rounding step of the row's largest element
    step = {"f32": 2.0 ** -16, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}[dims.dtype]
    for s64, s32 in zip(a, b32):
        x, y = s64.kv.double(), s32.kv.double()
        d = (x - y).abs().amax(dim=(3, 4))
        assert bool((d <= step * x.abs().amax(dim=(3, 4))).all())


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_cache_holds_the_16_bit_cache_rounded_to_a_neighbour(fmt):
    """[KV Cache] section 03: an 8-bit cache stores the same K and V in one byte each. Every K/V
    element the step writes is one of the two values of the format (decoded from its bit fields)
    that bracket the fp16 cache's element for the same step; the logits move, but only by the
    quantisation."""
    from test_oracle_pins import _fp8_table

    base = W.TINY.with_dtype("f16")
    d8 = base.with_kv(fmt)
    w = W.make_weights(base, SEED, gains="random")
    toks = W.token_ids(1003, 9, 3, base.vocab)
    s16, s8 = seq(base, 3, 20, toks), seq(d8, 3, 20, toks)
    r16, r8 = decode_step(base, w, [s16]), decode_step(d8, w, [s8])
    new16, new8 = s16.kv[:, :, 20:23].double().flatten(), s8.kv[:, :, 20:23].double().flatten()
    vals = torch.tensor(sorted(v for v, _ in _fp8_table(fmt)), dtype=torch.float64)
    i = torch.searchsorted(vals, new16)
    lo = vals[(i - 1).clamp(min=0)]
    hi = vals[i.clamp(max=len(vals) - 1)]
    exact = vals[i.clamp(max=len(vals) - 1)] == new16
    ok = exact & (new8 == new16) | (new8 == lo) | (new8 == hi)
    assert bool(ok.all()), f"{int((~ok).sum())} K/V elements are not a neighbour of the fp16 value"
    assert not torch.equal(new8, new16), "the 8-bit cache rounds"
    for a, b in zip(r8.logits, r16.logits):
        assert 0 < rel(a, b) < 0.2
