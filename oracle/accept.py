"""Oracle for the acceptance epilogue of a verify pass.

TEST INFRASTRUCTURE (see oracle/__init__.py).

Reading used throughout (the pages leave the indexing open): a sequence
enters the pass with ctx cached positions and with g0, the target's greedy
token for position ctx, already known from the previous pass. Its K query
rows carry the draft tokens d_1..d_K at positions ctx..ctx+K-1, and row j
(0-based) yields the target's greedy token g_{j+1} for position ctx+j+1.
"""
from __future__ import annotations


def accept_greedy(drafts: list, g0: int, row_argmax: list) -> tuple[int, int]:
    """Greedy verification: accepted-prefix length n in 0..K and the bonus token.

    [Serving Efficiency] section 31.5 and [Spending the Idle] section 12.4:
    under greedy target decoding a draft is kept exactly when it equals the
    target's own greedy choice at that prefix, and checking stops at the first
    draft that does not. [KV Cache] section 08 step 3: the verifier then always
    adds at least one token of the target's own, here the target's greedy token
    at the first unmatched position (or after the last draft if all match).

    drafts[j-1] = d_j is compared with g_{j-1}, where g_j = row_argmax[j-1]
    for j >= 1. Returns (n, g_n).
    """
    K = len(drafts)
    assert len(row_argmax) == K
    g = [g0] + list(row_argmax)
    n = 0
    while n < K and drafts[n] == g[n]:
        n += 1
    return n, g[n]


def expected_tokens_per_pass(a: float, k: int) -> float:
    """1 + a + a^2 + ... + a^k = (1 - a^(k+1)) / (1 - a).

    [Spending the Idle] section 12.4 and [Serving] "Speculative decoding": with
    i.i.d. acceptance probability a, one pass yields the guaranteed target
    token plus the run of accepted drafts.
    """
    if a == 1.0:
        return float(k + 1)
    return (1.0 - a ** (k + 1)) / (1.0 - a)


def rejection_accept_probs(p: list, q: list) -> list:
    """Acceptance probability min(1, p(x)/q(x)) for each candidate x with q(x) > 0.

    [Serving Efficiency] section 31.5 Example 31.3, [Serving] "Why it's
    exactly lossless", [KV Cache] section 08: a stochastic verifier keeps a
    draft x drawn from q with this probability.
    """
    return [min(1.0, pi / qi) if qi > 0 else 0.0 for pi, qi in zip(p, q)]


def rejection_residual(p: list, q: list) -> list:
    """The distribution a rejected draft is resampled from: norm(max(0, p - q))."""
    r = [max(0.0, pi - qi) for pi, qi in zip(p, q)]
    s = sum(r)
    return [ri / s for ri in r] if s > 0 else [0.0 for _ in r]


def rejection_output_dist(p: list, q: list) -> list:
    """Exact output distribution of one accept-or-resample step.

    [KV Cache] section 08 proof: P(x) = q(x) min(1, p/q) + P(reject) norm(max(0, p-q))(x).
    """
    acc = rejection_accept_probs(p, q)
    res = rejection_residual(p, q)
    p_reject = 1.0 - sum(qi * ai for qi, ai in zip(q, acc))
    return [qi * ai + p_reject * ri for qi, ai, ri in zip(q, acc, res)]


def softmax_t(logits, temperature: float = 1.0) -> list:
    """Target distribution of one row: softmax(logits / T), float64, with the maximum subtracted first."""
    import math

    z = [x / temperature for x in logits]
    m = max(z)
    e = [math.exp(x - m) for x in z]
    s = sum(e)
    return [x / s for x in e]


def sample_index(weights: list, v: float) -> tuple[int, float]:
    """Inverse-CDF draw: the smallest x with w(0) + ... + w(x) > v * sum(w), for v in [0, 1).

    Returns (x, margin) where margin is the distance, relative to sum(w), between v * sum(w) and
    the nearer of the two cumulative sums that bracket it (how far the draw is from changing).
    """
    total = sum(weights)
    target = v * total
    c = 0.0
    for x, w in enumerate(weights):
        lo = c
        c += w
        if c > target:
            return x, min(target - lo, c - target) / total if total > 0 else 0.0
    last = max(i for i, w in enumerate(weights) if w > 0) if total > 0 else len(weights) - 1
    return last, 0.0


def rejection_verify(p0_logits, row_logits, q_rows, drafts, u, v, temperature: float = 1.0):
    """Stochastic verification of K drafts of one sequence by modified rejection sampling.

    [Serving Efficiency] section 31.5 (Example 31.3), [Spending the Idle] section 12.4 and
    [Serving] "Lossless": draft d_j, drawn from the draft distribution q_j, is kept with
    probability min(1, p(d_j) / q_j(d_j)) under the target distribution p at its position; at the
    first rejection a replacement is drawn from norm(max(0, p - q_j)) and verification stops; if
    every draft is kept, one more token is drawn from the target distribution after the last
    draft ([KV Cache] section 08: a pass always adds at least one token).

    Target distributions: p_0 = softmax(p0_logits / T) for the position of d_1 (from the previous
    pass), p_j = softmax(row_logits[j - 1] / T) after d_j. u[j - 1] in [0, 1) decides draft j
    (kept when u < min(1, p/q)); v in [0, 1) drives the one inverse-CDF draw. A draft with
    q_j(d_j) = 0 is rejected (it could not have been drawn), and so is an id outside the vocabulary.

    Returns (n_accepted, token, margin): margin is the smallest distance from any decision taken
    to its boundary (|u - a| for the tests made, the draw's bracketing distance for the sample).
    """
    K = len(drafts)
    p = [softmax_t(p0_logits, temperature)] + [softmax_t(r, temperature) for r in row_logits]
    margin = float("inf")
    for j in range(1, K + 1):
        d = drafts[j - 1]
        q = q_rows[j - 1]
        a = rejection_accept_probs([p[j - 1][d]], [q[d]])[0] if 0 <= d < len(q) else 0.0
        margin = min(margin, abs(u[j - 1] - a))
        if not u[j - 1] < a:
            res = [max(0.0, pi - qi) for pi, qi in zip(p[j - 1], q)]
            if sum(res) <= 0.0:
                res = p[j - 1]
            x, mg = sample_index(res, v)
            return j - 1, x, min(margin, mg)
    x, mg = sample_index(p[K], v)
    return K, x, min(margin, mg)
