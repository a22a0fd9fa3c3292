"""Pins for the oracle's building blocks (CPU only).

Each test ties an oracle function to something other than itself: a value the
pages print, a closed form, a library routine, or an invariant.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import layers as L
from oracle.accept import (accept_greedy, expected_tokens_per_pass, rejection_accept_probs,
                           rejection_output_dist, rejection_residual, rejection_verify, sample_index,
                           softmax_t)
from oracle.model import kv_bytes_per_token, param_count, streamed_weight_bytes
from synth.workloads import LLAMA7B

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- tile merge

def test_example_31_2_tile_statistics():
    g = golden("example_31_2.json")
    w = torch.tensor(g["weights"], dtype=torch.float64)
    v = torch.tensor(g["values"], dtype=torch.float64)
    nums, dens = [], []
    for a, b in g["tiles"]:
        nums.append((w[a:b] * v[a:b]).sum())
        dens.append(w[a:b].sum())
    assert [[float(n), float(d)] for n, d in zip(nums, dens)] == g["tile_numerator_denominator"]
    out = L.combine_partials(torch.stack(nums), torch.stack(dens))
    assert float(out) == g["output"]
    wrong = sum(float(n / d) for n, d in zip(nums, dens)) / len(nums)
    assert wrong == pytest.approx(g["wrong_average_of_tile_outputs"], abs=1e-15)
    assert float(out) != pytest.approx(wrong)


def test_example_31_2_through_attention_with_running_maxima():
    """The same example as attention: scores ln(w), one query, keys split into the page's two tiles."""
    g = golden("example_31_2.json")
    w = torch.tensor(g["weights"], dtype=torch.float64)
    v = torch.tensor(g["values"], dtype=torch.float64).reshape(4, 1)
    q = torch.ones(1, 1, dtype=torch.float64)
    k = torch.log(w).reshape(4, 1)
    assert float(L.attention_standard(q, k, v, scale=1.0)) == pytest.approx(g["output"], abs=1e-15)
    assert float(L.attention_blockwise(q, k, v, block=2, scale=1.0)) == pytest.approx(g["output"], abs=1e-15)
    # per-tile (max, num, den) relative to the tile's own max, merged with rescaling
    nums, dens, maxes = [], [], []
    for a, b in g["tiles"]:
        s = k[a:b, 0]
        m = s.max()
        p = torch.exp(s - m)
        nums.append((p * v[a:b, 0]).sum())
        dens.append(p.sum())
        maxes.append(m)
    out = L.combine_partials(torch.stack(nums), torch.stack(dens), torch.stack(maxes))
    assert float(out) == pytest.approx(g["output"], abs=1e-15)


# ---------------------------------------------------------------- attention

def test_online_and_standard_agree_to_fp32_rounding_as_printed():
    g = golden("online_softmax_fp32.json")
    gen = torch.Generator().manual_seed(0)
    h, n, d = g["shape"]
    q, k, v = (torch.randn(h, n, d, generator=gen) for _ in range(3))
    mask = torch.ones(n, n, dtype=torch.bool).tril()
    ref64 = L.attention_standard(q.double(), k.double(), v.double(), mask)
    std = L.attention_standard(q, k, v, mask)
    onl = L.attention_blockwise(q, k, v, g["block"], mask)
    sdpa = F.scaled_dot_product_attention(q, k, v, is_causal=True)
    errs = {
        "standard_fp32": float((std.double() - ref64).abs().max()),
        "online_fp32": float((onl.double() - ref64).abs().max()),
        "sdpa_fp32": float((sdpa.double() - ref64).abs().max()),
    }
    for name, printed in g["printed_max_abs_err_vs_fp64"].items():
        # same order of magnitude as the printed fp32 errors: within 10x either way
        assert printed / 10 < errs[name] < printed * 10, (name, errs[name])
    assert torch.allclose(onl, std, atol=g["printed_allclose_atol"])
    # in float64 the two orders agree to float64 rounding
    onl64 = L.attention_blockwise(q.double(), k.double(), v.double(), g["block"], mask)
    assert float((onl64 - ref64).abs().max()) < 1e-13


@pytest.mark.parametrize("ctx,rows", [(0, 1), (5, 1), (17, 5), (33, 3)])
def test_attention_matches_library_sdpa_fp64(ctx, rows):
    gen = torch.Generator().manual_seed(ctx * 10 + rows)
    H, d = 3, 16
    n = ctx + rows
    q = torch.randn(H, rows, d, generator=gen, dtype=torch.float64)
    k = torch.randn(H, n, d, generator=gen, dtype=torch.float64)
    v = torch.randn(H, n, d, generator=gen, dtype=torch.float64)
    keep = torch.arange(n).unsqueeze(0) <= (ctx + torch.arange(rows)).unsqueeze(1)
    ours = L.attention_standard(q, k, v, keep)
    lib = F.scaled_dot_product_attention(q, k, v, attn_mask=keep)
    assert torch.allclose(ours, lib, rtol=0, atol=1e-13)


def test_attention_single_key_returns_its_value():
    q = torch.randn(1, 8, dtype=torch.float64) * 100
    k = torch.randn(1, 8, dtype=torch.float64)
    v = torch.randn(1, 8, dtype=torch.float64)
    assert torch.equal(L.attention_standard(q, k, v), v)


def test_attention_equal_scores_give_the_mean():
    n = 7
    q = torch.zeros(1, 4, dtype=torch.float64)
    k = torch.randn(n, 4, dtype=torch.float64)
    v = torch.randn(n, 4, dtype=torch.float64)
    assert torch.allclose(L.attention_standard(q, k, v), v.mean(0, keepdim=True), atol=1e-15)


def test_attention_scale_is_inverse_sqrt_head_dim():
    """Two keys: output = sigmoid(s0 - s1) v0 + sigmoid(s1 - s0) v1 with s = q.k / sqrt(d)."""
    d = 64
    gen = torch.Generator().manual_seed(3)
    q = torch.randn(1, d, generator=gen, dtype=torch.float64)
    k = torch.randn(2, d, generator=gen, dtype=torch.float64)
    v = torch.randn(2, d, generator=gen, dtype=torch.float64)
    s = (k @ q[0]) / 8.0
    a = 1.0 / (1.0 + math.exp(-(float(s[0]) - float(s[1]))))
    want = a * v[0] + (1 - a) * v[1]
    assert torch.allclose(L.attention_standard(q, k, v)[0], want, atol=1e-14)


# ---------------------------------------------------------------- RMSNorm, RoPE, SiLU

def test_rmsnorm_matches_library():
    gen = torch.Generator().manual_seed(1)
    x = torch.randn(5, 96, generator=gen, dtype=torch.float64) * 3
    g = torch.randn(96, generator=gen, dtype=torch.float64)
    ours = L.rmsnorm(x, g, 1e-5)
    lib = F.rms_norm(x, (96,), weight=g, eps=1e-5)
    assert torch.allclose(ours, lib, rtol=1e-14, atol=1e-14)


def test_rmsnorm_constant_vector_closed_form():
    c, eps = -2.5, 1e-5
    x = torch.full((1, 10), c, dtype=torch.float64)
    y = L.rmsnorm(x, torch.ones(10, dtype=torch.float64), eps)
    assert torch.allclose(y, torch.full_like(y, c / math.sqrt(c * c + eps)), atol=1e-15)


def _rope_complex(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotary embedding as complex multiplication: z_i = x_i + 1j x_{i+d/2} times exp(1j pos theta^(-2i/d))."""
    d = x.shape[-1]
    half = d // 2
    z = x[..., :half] + 1j * x[..., half:]
    freq = theta ** (-2.0 * np.arange(half) / d)
    z = z * np.exp(1j * pos * freq)
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("pos", [0, 1, 7, 1023, 4100])
def test_rope_is_complex_rotation(pos):
    gen = torch.Generator().manual_seed(pos)
    x = torch.randn(3, 128, generator=gen, dtype=torch.float64)  # 3 heads
    ours = L.rope(x.unsqueeze(0), torch.tensor([pos]), 10000.0)[0]
    want = _rope_complex(x.numpy(), pos, 10000.0)
    assert np.allclose(ours.numpy(), want, rtol=0, atol=1e-12)
    if pos == 0:
        assert torch.equal(ours, x)


def test_rope_frequency_base_explicit_value():
    # pair i=1 of a 128-wide head at position 1 rotates by 10000^(-2/128)
    x = torch.zeros(1, 1, 128, dtype=torch.float64)
    x[0, 0, 1] = 1.0
    y = L.rope(x, torch.tensor([1]), 10000.0)[0, 0]
    ang = 10000.0 ** (-2.0 / 128)
    assert y[1] == pytest.approx(math.cos(ang), abs=1e-15)
    assert y[65] == pytest.approx(math.sin(ang), abs=1e-15)
    assert float(y.abs().sum() - abs(y[1]) - abs(y[65])) == 0.0


def test_rope_scores_depend_only_on_relative_position():
    gen = torch.Generator().manual_seed(9)
    q = torch.randn(1, 1, 64, generator=gen, dtype=torch.float64)
    k = torch.randn(1, 1, 64, generator=gen, dtype=torch.float64)
    def score(m, n):
        return float((L.rope(q, torch.tensor([m]), 1e4) * L.rope(k, torch.tensor([n]), 1e4)).sum())
    assert score(10, 3) == pytest.approx(score(107, 100), abs=1e-11)
    assert score(500, 20) == pytest.approx(score(480, 0), abs=1e-11)


def test_silu_and_swiglu_match_library():
    x = torch.linspace(-30, 30, 1001, dtype=torch.float64)
    assert torch.allclose(L.silu(x), F.silu(x), rtol=1e-15, atol=1e-300)
    assert L.silu(torch.tensor([0.0], dtype=torch.float64)).item() == 0.0
    u = torch.randn(1001, dtype=torch.float64)
    assert torch.allclose(L.swiglu(x, u), F.silu(x) * u, rtol=1e-15, atol=1e-300)


def test_linear_orientation_matches_library():
    gen = torch.Generator().manual_seed(2)
    x = torch.randn(3, 5, generator=gen, dtype=torch.float64)
    w = torch.randn(7, 5, generator=gen, dtype=torch.float64)  # [out][in]
    assert torch.allclose(L.linear(x, w), F.linear(x, w), atol=1e-14)


def test_round_to_storage_types():
    x = torch.tensor([1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 1.0 + 2 ** -8 + 2 ** -9], dtype=torch.float64)
    # binary16 ties to even: 1+2^-11 -> 1, 1+3*2^-11 -> 1+2^-9; bf16 rounds 1+2^-8+2^-9 (a tie) to even 1+2^-7
    assert L.round_to(x[:2], "f16").tolist() == [1.0, 1.0 + 2 ** -9]
    assert L.round_to(x[2:], "bf16").tolist() == [1.0 + 2 ** -7]


# ---------------------------------------------------------------- argmax

def test_argmax_lowest_index_on_ties_and_gap():
    v = torch.tensor([0.5, 2.0, -1.0, 2.0, 1.75])
    assert L.argmax_lowest(v) == (1, 0.0)
    v = torch.tensor([0.5, 2.0, -1.0, 1.5, 1.75])
    assert L.argmax_lowest(v) == (1, 0.25)


# ---------------------------------------------------------------- acceptance

def _emitted(drafts, g0, row_argmax):
    n, bonus = accept_greedy(drafts, g0, row_argmax)
    return n, list(drafts[:n]) + [bonus]


@pytest.mark.parametrize("K", [1, 2, 3, 4, 5])
def test_greedy_acceptance_brute_force(K):
    """Exhaustive check over drafts, g0 and row argmaxes in {0,1,2}.

    Properties (not the acceptance loop itself): the emitted tokens are exactly
    the target's own greedy continuation g_0..g_n; drafting stops at the first
    draft that differs from the target (or after all K); at least one token is
    always emitted.
    """
    for g0 in range(3):
        for drafts in itertools.product(range(3), repeat=K):
            for am in itertools.product(range(3), repeat=K):
                g = [g0] + list(am)
                n, out = _emitted(list(drafts), g0, list(am))
                assert 0 <= n <= K and len(out) == n + 1
                assert out == g[:n + 1]
                assert n == K or drafts[n] != g[n]


@pytest.mark.parametrize("which", ["spending_the_idle", "kv_cache_section_08"])
def test_expected_tokens_per_pass_printed_values(which):
    g = golden("expected_tokens.json")[which]
    for key, printed in g["printed"].items():
        if which == "spending_the_idle":
            val = expected_tokens_per_pass(g["a"], int(key))
        else:
            val = expected_tokens_per_pass(float(key), g["k"])
        scale = 10 ** g["decimals"]
        shown = math.floor(val * scale) / scale if g["mode"] == "truncate" else round(val, g["decimals"])
        assert shown == pytest.approx(printed, abs=1e-12)


def test_expected_tokens_matches_acceptance_rule_monte_carlo():
    """Drafts that equal the target's greedy token with probability a, i.i.d.: the mean of
    n + 1 from accept_greedy converges to (1 - a^(K+1)) / (1 - a)."""
    rng = np.random.default_rng(5)
    a, K, trials = 0.7, 5, 40000
    total = 0
    for _ in range(trials):
        g = list(rng.integers(0, 1000, K + 1))
        drafts = [g[j] if rng.random() < a else (g[j] + 1) % 1000 for j in range(K)]
        n, _ = accept_greedy(drafts, g[0], g[1:])
        total += n + 1
    mean = total / trials
    want = expected_tokens_per_pass(a, K)
    # variance of n+1 is below K^2/4; 5 sigma
    assert abs(mean - want) < 5 * math.sqrt(K * K / 4 / trials)


@pytest.mark.parametrize("which", ["example_31_3", "exercise_3"])
def test_rejection_sampling_examples(which):
    g = golden("rejection_examples.json")[which]
    p, q = g["p"], g["q"]
    assert rejection_accept_probs(p, q) == pytest.approx(g["accept"], abs=1e-12)
    assert rejection_residual(p, q) == pytest.approx(g["residual"], abs=1e-12)
    assert rejection_output_dist(p, q) == pytest.approx(g["final"], abs=1e-12)
    acc = rejection_accept_probs(p, q)
    assert [qi * ai for qi, ai in zip(q, acc)] == pytest.approx(g["accepted_mass"], abs=1e-12)
    assert 1 - sum(qi * ai for qi, ai in zip(q, acc)) == pytest.approx(g["reject_mass"], abs=1e-12)
    if "wrong_resample_from_p_paris" in g:
        wrong_paris = q[0] * acc[0] + g["reject_mass"] * p[0]
        assert wrong_paris == pytest.approx(g["wrong_resample_from_p_paris"], abs=1e-12)


def test_rejection_output_is_target_for_random_distributions():
    rng = np.random.default_rng(11)
    for _ in range(200):
        p = rng.dirichlet(np.ones(6)).tolist()
        q = rng.dirichlet(np.ones(6) * 0.3).tolist()
        assert rejection_output_dist(p, q) == pytest.approx(p, abs=1e-12)


def _emitted_distribution(p0_logits, row_logits, q_rows, K, N=4000):
    """Distribution of the first emitted token of rejection_verify, with d_1 ~ q_1: the accept test
    is probed on both sides of its threshold (u just below a keeps d_1, u at a rejects it) and the
    replacement draw is integrated over a midpoint grid of N values of v (error <= 1/N per token)."""
    V = len(p0_logits)
    p0 = softmax_t(p0_logits)
    dist = [0.0] * V
    tail = [0.5] * (K - 1)
    for d in range(V):
        w = q_rows[0][d]
        if w == 0:
            continue
        a = min(1.0, p0[d] / w)
        if a > 0:
            n, x, _ = rejection_verify(p0_logits, row_logits, q_rows, [d] + [0] * (K - 1), [a * (1 - 1e-9)] + tail, 0.5)
            assert n >= 1, "u below min(1, p/q) keeps the draft"
            dist[d] += w * a
        if a < 1:
            for iv in range(N):
                n, x, _ = rejection_verify(p0_logits, row_logits, q_rows, [d] + [0] * (K - 1), [a] + tail, (iv + 0.5) / N)
                assert n == 0, "u at min(1, p/q) rejects the draft"
                dist[x] += w * (1 - a) / N
    return dist


@pytest.mark.parametrize("which", ["example_31_3", "exercise_3"])
def test_rejection_verify_reproduces_the_printed_examples(which):
    """The whole procedure (accept test, residual draw) integrated over its random numbers gives
    the printed final distribution: the emitted token follows the target, not the draft."""
    g = golden("rejection_examples.json")[which]
    lp = [math.log(x) for x in g["p"]]
    dist = _emitted_distribution(lp, [[0.0, 0.0]], [g["q"]], 1)
    assert dist == pytest.approx(g["final"], abs=1e-3)


def test_rejection_verify_is_lossless_for_random_distributions():
    """First emitted token ~ p_0 for random p_0, q_1 over 5 tokens, whatever happens after it; the
    token after an accepted d_1 follows p_1; the token after two accepted drafts follows p_2."""
    rng = np.random.default_rng(5)
    for _ in range(4):
        V, K = 5, 2
        p0 = rng.normal(0, 1.5, V).tolist()
        rows = [rng.normal(0, 1.5, V).tolist() for _ in range(K)]
        qs = [rng.dirichlet(np.ones(V) * 0.5).tolist() for _ in range(K)]
        assert _emitted_distribution(p0, rows, qs, K) == pytest.approx(softmax_t(p0), abs=1e-3)
        # with d_1 kept (u_1 = 0), the token after it follows p_1: the same check one position on,
        # feeding p_1's logits as the "previous" distribution of the shifted pass
        assert _emitted_distribution(rows[0], rows[1:], qs[1:], 1) == pytest.approx(softmax_t(rows[0]), abs=1e-3)
        n, _, _ = rejection_verify(p0, rows, qs, [0, 0], [0.0, 0.0], 0.5)
        assert n >= 1 or softmax_t(p0)[0] == 0
        # all drafts kept: the extra token is drawn from p_K by inverse CDF
        ok = [rejection_verify(p0, rows, qs, [0, 0], [0.0, 0.0], (iv + 0.5) / 400) for iv in range(400)]
        if all(n == 2 for n, _, _ in ok):
            emp = np.bincount([x for _, x, _ in ok], minlength=V) / 400
            assert emp.tolist() == pytest.approx(softmax_t(rows[1]), abs=1.0 / 400 + 1e-12)


def test_sample_index_is_the_inverse_cdf():
    rng = np.random.default_rng(9)
    for _ in range(200):
        w = rng.random(17) * (rng.random(17) > 0.3)
        if w.sum() == 0:
            continue
        v = float(rng.random())
        x, margin = sample_index(w.tolist(), v)
        c = np.cumsum(w)
        assert x == int(np.searchsorted(c, v * c[-1], side="right"))
        assert w[x] > 0 and margin >= 0


def test_softmax_t_matches_library_and_temperature_sharpens():
    rng = np.random.default_rng(2)
    z = rng.normal(0, 3, 50)
    for T in (0.5, 1.0, 2.0):
        ref = torch.softmax(torch.tensor(z / T, dtype=torch.float64), 0).tolist()
        assert softmax_t(z.tolist(), T) == pytest.approx(ref, rel=1e-12)
    assert max(softmax_t(z.tolist(), 0.5)) > max(softmax_t(z.tolist(), 2.0))


# ---------------------------------------------------------------- byte accounting

def test_kv_bytes_per_token_printed_table():
    g = golden("kv_bytes.json")
    for m in g["models"]:
        b = kv_bytes_per_token(m["layers"], m["kv_heads"], m["head_dim"], g["bytes_per_value"])
        assert b / 1024 == m["kib_per_token"], m["name"]
        if "gib_at_128k" in m:
            assert round(b * 131072 / 2 ** 30, 2) == m["gib_at_128k"]


def test_7b_parameter_count_matches_printed_weights():
    g = golden("kv_bytes.json")
    n = param_count(LLAMA7B)
    assert n == 6_738_415_616
    assert round(n * 2 / 2 ** 30, 1) == g["llama2_7b_weights_gib_printed"]
    # the per-step weight stream excludes the gathered embedding table
    assert streamed_weight_bytes(LLAMA7B) == (n - 32000 * 4096) * 2 == 13_214_687_232


def test_oracle_package_exports():
    for name in ["decode_step", "accept_greedy", "rmsnorm", "rope", "attention_standard", "PoolModel"]:
        assert hasattr(oracle, name)


def test_rejection_verify_rejects_drafts_that_cannot_have_been_drawn():
    """A draft the draft model gives zero probability, or an id outside the vocabulary, is never kept
    (u = 0 keeps any draft with positive acceptance probability), and the replacement comes from
    norm(max(0, p - q)); where p <= q everywhere there is nothing to correct and the draw is from p itself."""
    lp = [0.0, math.log(2.0), math.log(5.0)]  # p = (1/8, 2/8, 5/8)
    q = [0.5, 0.5, 0.0]
    n, x, _ = rejection_verify(lp, [[0.0] * 3], [q], [2], [0.0], 0.0)
    assert n == 0 and x == 2, "q(d) = 0: rejected; the residual (0, 0, 5/8) puts everything on token 2"
    n, _, _ = rejection_verify(lp, [[0.0] * 3], [q], [0], [0.0], 0.0)
    assert n == 1, "u = 0 keeps a draft with positive acceptance probability"
    for bad in (-1, 3):
        n, x, _ = rejection_verify(lp, [[0.0] * 3], [q], [bad], [0.0], 0.0)
        assert n == 0 and x == 2
    one_hot = [-math.inf, 0.0, -math.inf]  # p = q = (0, 1, 0); draft 0 has q = 0 and is rejected
    n, x, _ = rejection_verify(one_hot, [[0.0] * 3], [[0.0, 1.0, 0.0]], [0], [0.0], 0.9)
    assert n == 0 and x == 1, "p <= q everywhere: the residual is zero, so the draw falls back to p"


def _fp8_table(fmt):
    """Every finite value of an OCP 8-bit float, decoded from its bit fields, with its code's mantissa."""
    eb, mb, bias = {"e4m3": (4, 3, 7), "e5m2": (5, 2, 15)}[fmt]
    vals = []
    for code in range(256):
        sgn, E, M = code >> 7, (code >> mb) & ((1 << eb) - 1), code & ((1 << mb) - 1)
        if fmt == "e4m3" and E == 15 and M == 7:
            continue  # NaN
        if fmt == "e5m2" and E == 31:
            continue  # infinities and NaNs
        mag = (M / 2 ** mb) * 2.0 ** (1 - bias) if E == 0 else (1 + M / 2 ** mb) * 2.0 ** (E - bias)
        vals.append((-mag if sgn else mag, M))
    return vals


@pytest.mark.parametrize("fmt,n_finite,vmax", [("e4m3", 254, 448.0), ("e5m2", 248, 57344.0)])
def test_round_fp8_is_nearest_even_over_the_format(fmt, n_finite, vmax):
    """Brute force over the decoded format: every midpoint between neighbours (a tie: the even
    mantissa wins), points just either side of it, random values across the whole range including
    subnormals, and saturation beyond the largest finite value."""
    from oracle.layers import round_fp8

    table = _fp8_table(fmt)
    assert len(table) == n_finite and max(v for v, _ in table) == vmax
    pos = sorted({(v, m) for v, m in table if v >= 0})
    xs, want = [], []
    for (a, ma), (b, mb_) in zip(pos, pos[1:]):
        mid = (a + b) / 2
        xs += [mid, math.nextafter(mid, 0), math.nextafter(mid, math.inf)]
        want += [a if ma % 2 == 0 else b, a, b]
    rng = np.random.default_rng(8)
    rand = np.exp(rng.uniform(math.log(2.0 ** -20), math.log(vmax), 4000)).astype(np.float32).astype(np.float64)
    vals = np.array([v for v, _ in pos])
    mant = dict(pos)
    for x in rand:
        i = int(np.searchsorted(vals, x))
        lo, hi = vals[max(i - 1, 0)], vals[min(i, len(vals) - 1)]
        xs.append(float(x))
        if x - lo != hi - x:
            want.append(lo if x - lo < hi - x else hi)
        else:
            want.append(lo if mant[float(lo)] % 2 == 0 else hi)
    xs += [vmax * 1.01, vmax * 1e3]
    want += [vmax, vmax]
    x = torch.tensor(xs, dtype=torch.float64)
    got = round_fp8(x, fmt)
    assert torch.equal(got, torch.tensor(want, dtype=torch.float64))
    assert torch.equal(round_fp8(-x, fmt), -got), "rounding is symmetric in the sign"
    # inside the range the library's float8 cast (also nearest-even) agrees on fp32 inputs (it
    # converts a double through fp32 first, so points a hair off a midpoint are left out)
    lib_dt = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[fmt]
    inside = x[(x <= vmax) & (x.to(torch.float32).to(torch.float64) == x)]
    assert len(inside) > 3000
    assert torch.equal(round_fp8(inside, fmt), inside.to(lib_dt).to(torch.float64))
