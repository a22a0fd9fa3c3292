"""verify_sample (stochastic verification by modified rejection sampling) against the oracle.

[Serving Efficiency] section 31.5 (Example 31.3); [Spending the Idle] section
12.4; [Serving] "Lossless"; [KV Cache] section 08.

Parity. The GPU computes the target distributions in fp32, the oracle in
fp64, on the same fp32 logits, draft distributions and uniforms. Every
decision (each accept test u < min(1, p/q), and the one inverse-CDF draw) is
compared exactly unless the oracle finds it within eps of its boundary. The
bound comes from the fp32 error of the GPU's side. A probability carries the
rounding of 1/T and z/T (a common factor: at most 6e-8 |z/T - mean|, under
3e-6 for |z/T| <= 40), of z/T - max and exp (under 3e-6), and of the
normaliser, a sum of at most 32 terms per thread, 64 lanes and 16 waves with
rescales (under 3e-6): under 1e-5 relative in all. The cumulative sum of the
draw adds at most 32 + 16 + 6 roundings (under 4e-6 of the total). So no
decision flips further than eps = 3e-5 from its boundary, plus 1e-5 relative
to the residual's mass when the draw is from norm(max(0, p - q)) (its weights'
absolute errors add up to 1e-5 of p's mass, not of the residual's). Decisions
nearer their boundary must still be valid draws (a token of positive weight
under the distribution the GPU drew from), and at least 85 % of the sequences
of a small-vocabulary case or a peaked full-vocabulary one must compare
exactly. Flat
distributions over 32000 tokens put most draws within fp32 rounding of a
boundary (each token holds about 3e-5 of the mass): there validity and the
distribution test below carry the check.

Distribution. With fixed target and draft distributions and many sequences
whose drafts are drawn from q, the first emitted token must follow p_0 and
the second (after an accepted first draft) p_1: chi-square at the 1e-4
level, seeded.
"""
import math

import numpy as np
import pytest
import torch

from oracle.accept import rejection_verify
import synth
import verify_step_amd as vs

pytestmark = pytest.mark.gpu

EPS_P, EPS_R = 3e-5, 1e-5
SEED = 7100


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _f32(a):
    return np.asarray(a, dtype=np.float32)


def _softmax64(z, T):
    z = np.asarray(z, dtype=np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


class Case:
    """Synthetic inputs of one verify_sample call; all host arrays, fp32 where the GPU reads floats."""

    def __init__(self, seed, B, V, K_lo, K_hi, std=2.0, corr=0.5, T=1.0, bad=False):
        k = synth.key(SEED, seed)
        self.B, self.V, self.T = B, V, T
        self.K = [int(x) for x in synth.uniform_int(synth.key(k, 1), 0, B, K_lo, K_hi + 1)]
        self.q_start = np.concatenate([[0], np.cumsum(self.K)]).astype(np.int32)
        M = self.M = int(self.q_start[-1])
        self.p0 = _f32(synth.normal(synth.key(k, 2), 0, B * V, 0.0, std).numpy().reshape(B, V))
        self.logits = _f32(synth.normal(synth.key(k, 3), 0, M * V, 0.0, std).numpy().reshape(M, V))
        # draft logits: correlated with the target row at the same position for some sequences
        noise = synth.normal(synth.key(k, 4), 0, max(M, 1) * V, 0.0, std).numpy().reshape(max(M, 1), V)[:M]
        mix = synth.uniform(synth.key(k, 5), 0, B)
        self.q = np.zeros((M, V), dtype=np.float32)
        for b in range(B):
            r0 = int(self.q_start[b])
            for j in range(self.K[b]):
                tgt = self.p0[b] if j == 0 else self.logits[r0 + j - 1]
                zq = tgt + 0.25 * noise[r0 + j] if mix[b] < corr else noise[r0 + j]
                self.q[r0 + j] = _f32(_softmax64(zq, T))
        # drafts drawn from q by inverse CDF on their own uniforms
        w = synth.uniform(synth.key(k, 6), 0, max(M, 1))
        cdf = np.cumsum(self.q.astype(np.float64), axis=1)
        self.drafts = np.array([min(int(np.searchsorted(cdf[r], w[r] * cdf[r, -1], side="right")), V - 1)
                                for r in range(M)], dtype=np.int32)
        if bad and M >= 3:  # one draft the drafter gives zero probability, one id outside the vocabulary
            r = int(self.q_start[np.argmax(np.array(self.K) > 0)])
            self.q[r, self.drafts[r]] = 0.0
            self.drafts[min(r + 1, M - 1)] = V + 3
        self.u = _f32(synth.uniform(synth.key(k, 7), 0, max(M, 1))[:M])
        self.v = _f32(synth.uniform(synth.key(k, 8), 0, B))

    def run_gpu(self):
        dev = torch.device("cuda")
        t = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
        self.g = dict(q_start=t(self.q_start, torch.int32), drafts=t(self.drafts, torch.int32), p0=t(self.p0),
                      logits=t(self.logits), q=t(self.q), u=t(self.u), v=t(self.v))
        acc = torch.full((self.B,), -7, dtype=torch.int32, device=dev)
        tok = torch.full((self.B,), -7, dtype=torch.int32, device=dev)
        nb = vs.verify_sample_workspace_bytes(self.B, self.M, self.V)
        ws = torch.empty(max(nb, 8), dtype=torch.uint8, device=dev)
        g = self.g
        vs.verify_sample(self.B, self.M, self.V, g["q_start"], g["drafts"], g["p0"], g["logits"], g["q"], g["u"],
                         g["v"], self.T, acc, tok, ws, nb, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        return acc.cpu().tolist(), tok.cpu().tolist()

    def run_oracle(self, b):
        r0, K = int(self.q_start[b]), self.K[b]
        rows = [self.logits[r0 + j].astype(np.float64).tolist() for j in range(K)]
        qs = [self.q[r0 + j].astype(np.float64).tolist() for j in range(K)]
        return rejection_verify(self.p0[b].astype(np.float64).tolist(), rows, qs,
                                [int(d) for d in self.drafts[r0:r0 + K]], [float(x) for x in self.u[r0:r0 + K]],
                                float(self.v[b]), self.T)

    def eps(self, b, n):
        """Distance from a boundary beyond which no decision can flip: EPS_P, plus EPS_R relative to the
        mass of the residual max(0, p_n - q_{n+1}) when the draw is from that residual (n < K)."""
        r0, K = int(self.q_start[b]), self.K[b]
        if n == K:
            return EPS_P
        p = _softmax64(self.p0[b] if n == 0 else self.logits[r0 + n - 1], self.T)
        R = float(np.maximum(0.0, p - self.q[r0 + n].astype(np.float64)).sum())
        return EPS_P + EPS_R / R if R > 0 else EPS_P

    def valid(self, b, n, x):
        """x has positive weight under the distribution the GPU claims to have drawn from after n kept drafts."""
        r0, K = int(self.q_start[b]), self.K[b]
        if not (0 <= n <= K and 0 <= x < self.V):
            return False
        p = _softmax64(self.p0[b] if n == 0 else self.logits[r0 + n - 1], self.T)
        if n < K:
            res = np.maximum(0.0, p - self.q[r0 + n].astype(np.float64))
            if res.sum() > 0 and res[x] > 0:
                return True
        return p[x] > 0


def _check_case(case, label, min_exact=0.9):
    acc, tok = case.run_gpu()
    exact = 0
    n_acc = 0
    for b in range(case.B):
        n, x, margin = case.run_oracle(b)
        n_acc += n
        if margin > case.eps(b, n):
            assert (acc[b], tok[b]) == (n, x), f"{label} seq {b}: GPU ({acc[b]}, {tok[b]}) vs oracle ({n}, {x}), " \
                                               f"margin {margin:.2e}"
            exact += 1
        else:
            assert case.valid(b, acc[b], tok[b]), f"{label} seq {b}: near-boundary draw ({acc[b]}, {tok[b]}) invalid"
    _say(f"{label}: {exact}/{case.B} decided exactly, {n_acc} drafts kept of {case.M}")
    assert exact >= min_exact * case.B, f"{label}: only {exact} of {case.B} sequences away from a boundary"
    return acc, tok


@pytest.mark.parametrize("V", [50, 1000, 4099])
@pytest.mark.parametrize("T", [1.0, 0.6, 1.7])
def test_verify_sample_matches_oracle_small(V, T):
    case = Case(10 * V + int(10 * T), B=24, V=V, K_lo=0, K_hi=6, std=2.0, T=T, bad=True)
    _check_case(case, f"V={V} T={T}", min_exact=0.85)


@pytest.mark.parametrize("B,K,std", [(8, 5, 4.0), (64, 1, 4.0), (8, 5, 1.0)])
def test_verify_sample_matches_oracle_full_vocab(B, K, std):
    """The 7B vocabulary (32000) at the verify (8 x 5) and batched-decode (64 x 1) shapes."""
    case = Case(1000 + B * 10 + K + int(std), B=B, V=32000, K_lo=K, K_hi=K, std=std, corr=0.6)
    _check_case(case, f"V=32000 B={B} K={K} std={std}", min_exact=0.85 if std >= 4 else 0.0)


def test_verify_sample_vocabulary_past_the_vector_path():
    """A 152064-token vocabulary (more than 16 x 8192): chunks of 32 tokens take the scalar path;
    and a vocabulary that is not a multiple of four (151939) takes unaligned scalar loads."""
    for V in (152064, 151939):
        case = Case(V, B=6, V=V, K_lo=0, K_hi=3, std=4.0, corr=0.6)
        _check_case(case, f"V={V}", min_exact=0.6)


def test_verify_sample_edge_cases():
    # no draft rows at all: every token drawn from p_0
    case = Case(1, B=5, V=300, K_lo=0, K_hi=0)
    assert case.M == 0
    acc, _ = _check_case(case, "M=0", min_exact=0.6)
    assert acc == [0] * 5
    # a single sequence
    _check_case(Case(2, B=1, V=777, K_lo=3, K_hi=3), "B=1")
    # masked tokens (-inf logits) are never drawn; p <= q everywhere falls back to p
    V = 40
    case = Case(3, B=4, V=V, K_lo=2, K_hi=2)
    case.p0[:, ::2] = -np.inf
    case.logits[:, 1::3] = -np.inf
    # sequence 0: one-hot target and draft distributions on token 5, first draft 4 (q = 0): rejected,
    # residual all zero, so the draw falls back to p_0 = one-hot(5)
    case.p0[0] = -np.inf
    case.p0[0, 5] = 0.0
    case.q[0] = 0.0
    case.q[0, 5] = 1.0
    case.drafts[0] = 4
    acc, tok = case.run_gpu()
    for b in range(case.B):
        n, x, margin = case.run_oracle(b)
        if margin > case.eps(b, n):
            assert (acc[b], tok[b]) == (n, x), f"masked seq {b}: GPU ({acc[b]}, {tok[b]}) vs oracle ({n}, {x})"
        p = _softmax64(case.p0[b] if acc[b] == 0 else case.logits[int(case.q_start[b]) + acc[b] - 1], 1.0)
        assert p[tok[b]] > 0, f"masked seq {b}: drew a token of zero target probability"
    assert (acc[0], tok[0]) == (0, 5)
    # the same inputs give the same outputs
    assert case.run_gpu() == (acc, tok)


def test_verify_sample_rejects_bad_arguments():
    dev = torch.device("cuda")
    z = torch.zeros(64, dtype=torch.float32, device=dev)
    i = torch.zeros(4, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    with pytest.raises(vs.VSError, match="temperature"):
        vs.verify_sample(1, 1, 8, i, i, z, z, z, z, z, 0.0, i, i, z, 256, s)
    with pytest.raises(vs.VSError, match="workspace"):
        vs.verify_sample(2, 3, 8, i, i, z, z, z, z, z, 1.0, i, i, z, 39, s)


def test_verify_sample_output_distribution_is_the_target():
    """Many sequences with the same p_0, p_1, p_2, q_1, q_2 and drafts drawn from q: the first emitted
    token follows p_0 and the second, after a kept first draft, follows p_1 (chi-square, 1e-4 level)."""
    from scipy.stats import chi2

    V, K, N = 6, 2, 20000
    k = synth.key(SEED, 99)
    zp = [synth.normal(synth.key(k, j), 0, V, 0.0, 1.0).numpy() for j in range(K + 1)]
    zq = [synth.normal(synth.key(k, 10 + j), 0, V, 0.0, 1.0).numpy() for j in range(K)]
    case = Case(4, B=1, V=V, K_lo=K, K_hi=K)  # shell; replaced below
    case.B, case.M, case.K = N, N * K, [K] * N
    case.q_start = (np.arange(N + 1) * K).astype(np.int32)
    case.p0 = np.tile(_f32(zp[0]), (N, 1))
    case.logits = np.tile(np.stack([_f32(zp[1]), _f32(zp[2])]), (N, 1))
    q = [_f32(_softmax64(zq[j], 1.0)) for j in range(K)]
    case.q = np.tile(np.stack(q), (N, 1))
    w = synth.uniform(synth.key(k, 20), 0, N * K)
    cdf = [np.cumsum(qj.astype(np.float64)) for qj in q]
    case.drafts = np.array([min(int(np.searchsorted(cdf[r % K], w[r] * cdf[r % K][-1], side="right")), V - 1)
                            for r in range(N * K)], dtype=np.int32)
    case.u = _f32(synth.uniform(synth.key(k, 21), 0, N * K))
    case.v = _f32(synth.uniform(synth.key(k, 22), 0, N))
    acc, tok = case.run_gpu()
    first = [int(case.drafts[K * b]) if acc[b] >= 1 else tok[b] for b in range(N)]
    second = [int(case.drafts[K * b + 1]) if acc[b] >= 2 else tok[b] for b in range(N) if acc[b] >= 1]
    for label, got, p in (("first", first, _softmax64(zp[0], 1.0)), ("second", second, _softmax64(zp[1], 1.0))):
        cnt = np.bincount(got, minlength=V).astype(np.float64)
        exp = p * len(got)
        stat = float(((cnt - exp) ** 2 / exp).sum())
        crit = float(chi2.ppf(1 - 1e-4, V - 1))
        _say(f"{label} emitted token over {len(got)} sequences: chi2 {stat:.2f} (critical {crit:.2f})")
        assert stat < crit, f"{label} emitted token does not follow the target: chi2 {stat:.2f} >= {crit:.2f}"
    # and every sequence agrees with the oracle draw for draw, away from boundaries
    for b in range(0, N, 97):
        n, x, margin = case.run_oracle(b)
        if margin > case.eps(b, n):
            assert (acc[b], tok[b]) == (n, x), f"seq {b}"
