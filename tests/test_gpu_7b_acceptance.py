"""Greedy speculative verification on the GPU over 2048 sequence-rounds: the acceptance statistics,
and each verify pass against the single-row steps that built its drafts.

The workload is the 7B fp16 verify shape (8 sequences, context 1024, K = 5 drafts). Each of 256
rounds, for all 8 sequences at once:
  1. one decode step feeds a fresh random token at position 1023; its greedy token is g0;
  2. four more decode steps feed the greedy tokens back (positions 1024..1027), giving the target's
     own greedy chain c_0 = g0, c_1 .. c_4;
  3. drafts d_j = c_{j-1} with probability 0.7 (a seeded uniform below 0.7), else a uniform random
     token ([Spending the Idle] section 12.4: a draft matches the target with probability a);
  4. one verify pass feeds d_1 .. d_5 at positions 1024..1028 with acceptance fused.

Checked:
  * the fused acceptance equals the acceptance rule applied to the pass's own greedy tokens, exactly;
  * a verify row whose drafts so far equal the chain saw the same tokens at the same positions as a
    chain step ([KV Cache] section 08: a K-token verify pass computes what K single steps compute):
    its logits are within the 1e-2 bound of that step's, and its greedy token is the step's, except
    where the step's top-2 gap is below max(1e-3, twice the largest difference between the two rows),
    and such differences stay under 2 % of the compared rows;
  * with independent matches of probability a = 0.7 over k = 5 drafts, P(n >= i) = a^i, so
    E[n] = sum_i a^i = 1.94117, P(n = 5) = a^5 = 0.16807 and E[emitted] = E[n] + 1 = (1 - a^6)/(1 - a)
    = 2.94117 ([Spending the Idle] section 12.4; [KV Cache] section 08, "How many tokens per
    round"): the mean accepted length and the share of fully accepted passes must lie within four
    standard errors of these values over the 2048 sequence-rounds.
"""
import math

import pytest
import torch

import oracle
import synth
import verify_step_amd as vs
from harness import GpuModel, GpuPool, SeqSpec, make_step
from harness.compare import TOL, row_rel_err
from synth import workloads as W

pytestmark = pytest.mark.gpu

SEED_W, SEED_KV, SEED_TOK, SEED_DRAFT, SEED_PAGES = 4101, 4102, 4103, 4105, 4106
B, CTX, K, ROUNDS, ALPHA = 8, 1024, 5, 256, 0.7


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _moments(a, k):
    """E[n], Var[n] and P(n = k) of the accepted length when P(n >= i) = a^i for i <= k."""
    tail = [a ** i for i in range(1, k + 1)]
    mean = sum(tail)
    second = sum((2 * i - 1) * t for i, t in enumerate(tail, start=1))  # E[n^2] = sum P(n >= i)(2i - 1)
    return mean, second - mean * mean, a ** k


def test_7b_greedy_acceptance_statistics_and_k_row_agreement():
    dims = W.LLAMA7B
    _say("7B fp16 acceptance statistics: weights")
    model = GpuModel(dims, seed=SEED_W)
    n_blk = -(-(CTX + K) // 16)
    pool = GpuPool(dims, B * n_blk + 8)
    ids = vs.kv_alloc(pool.handle, pool.num_pages)
    perm = synth.permutation(synth.key(SEED_PAGES), pool.num_pages)
    vs.kv_free(pool.handle, [ids[int(i)] for i in perm])
    rows = []
    for b in range(B):
        r = vs.kv_alloc(pool.handle, -(-(CTX - 1) // 16))
        pool.write(r, 0, W.kv_block(dims, SEED_KV, b, 0, CTX - 1))
        rows.append(vs.kv_append(pool.handle, r, n_blk, CTX - 1, K + 1))
    stream = torch.cuda.current_stream().cuda_stream
    # one-row steps (positions 1023..1027) and the verify pass share the pages; descriptors sized for
    # the furthest position either reaches
    s1 = make_step(model, pool, [SeqSpec(CTX + K - 1, [0]) for _ in range(B)], rows, max_blocks=n_blk)
    sv = make_step(model, pool, [SeqSpec(CTX, [0] * K) for _ in range(B)], rows, max_blocks=n_blk, g0=[0] * B)

    def one_row_step(pos, toks):
        s1.ctx_len.fill_(pos)
        s1.tokens.copy_(torch.tensor(toks, dtype=torch.int32))
        vs.decode_step(s1.desc, s1.block_tables, model.w, s1.out, s1.ws, s1.ws_bytes, stream)
        torch.cuda.synchronize()
        return s1.argmax[:B].cpu().tolist(), s1.logits[:B].cpu().clone()

    n_all, n_checked_rows, n_tie_rows, worst = [], 0, 0, 0.0
    for rnd in range(ROUNDS):
        if rnd % 32 == 0:
            _say(f"7B fp16 acceptance statistics: round {rnd} of {ROUNDS}")
        first = [int(t) for t in synth.uniform_int(synth.key(SEED_TOK, rnd), 0, B, 0, dims.vocab)]
        g0, _ = one_row_step(CTX - 1, first)
        chain, chain_logits = [g0], []
        for i in range(K - 1):  # c_1 .. c_4 from the steps at positions 1024 .. 1027
            c, lg = one_row_step(CTX + i, chain[-1])
            chain.append(c)
            chain_logits.append(lg)
        u = synth.uniform(synth.key(SEED_DRAFT, rnd, 1), 0, B * K).reshape(B, K)
        rnd_tok = synth.uniform_int(synth.key(SEED_DRAFT, rnd, 2), 0, B * K, 0, dims.vocab).reshape(B, K)
        drafts = [[chain[j][b] if u[b, j] < ALPHA else int(rnd_tok[b, j]) for j in range(K)] for b in range(B)]
        sv.tokens.copy_(torch.tensor([t for d in drafts for t in d], dtype=torch.int32))
        sv.g0.copy_(torch.tensor(g0, dtype=torch.int32))
        vs.decode_step(sv.desc, sv.block_tables, model.w, sv.out, sv.ws, sv.ws_bytes, stream)
        torch.cuda.synchronize()
        am = sv.argmax[:B * K].cpu().tolist()
        vlog = sv.logits[:B * K].cpu()
        acc, bon = sv.accept_len.cpu().tolist(), sv.bonus.cpu().tolist()
        for b in range(B):
            a_b = am[K * b:K * b + K]
            assert (acc[b], bon[b]) == oracle.accept_greedy(drafts[b], g0[b], a_b), f"round {rnd} seq {b}"
            n_all.append(acc[b])
            # rows 0..3 whose drafts so far follow the chain saw what chain steps 1..4 saw
            for r in range(K - 1):
                if drafts[b][:r + 1] != [chain[j][b] for j in range(r + 1)]:
                    break
                ref = chain_logits[r][b].double()
                got = vlog[K * b + r].double()
                e = row_rel_err(got, ref)
                worst = max(worst, e)
                assert e <= TOL["f16"], f"round {rnd} seq {b} row {r}: verify row vs single step {e:.2e}"
                n_checked_rows += 1
                if a_b[r] != chain[r + 1][b]:
                    top = torch.topk(ref, 2).values
                    slack = max(1e-3, 2.0 * float((got - ref).abs().max()))
                    assert float(top[0] - top[1]) < slack and float(ref[a_b[r]]) >= float(top[0]) - slack, \
                        f"round {rnd} seq {b} row {r}: verify token {a_b[r]} vs single-step token {chain[r + 1][b]}"
                    n_tie_rows += 1
    pool.close()

    N = len(n_all)
    mean_n = sum(n_all) / N
    p_full = sum(1 for n in n_all if n == K) / N
    e_n, var_n, p5 = _moments(ALPHA, K)
    se_mean, se_p = math.sqrt(var_n / N), math.sqrt(p5 * (1 - p5) / N)
    _say(f"7B fp16 acceptance statistics: {N} sequence-rounds, mean accepted {mean_n:.4f} (closed form "
         f"{e_n:.4f} +- {se_mean:.4f}), P(n = {K}) {p_full:.4f} (closed form {p5:.4f} +- {se_p:.4f}), "
         f"mean emitted {mean_n + 1:.4f}; {n_checked_rows} verify rows compared with single steps, worst "
         f"{worst:.2e}, {n_tie_rows} near-tie token differences")
    assert N == B * ROUNDS >= 2048
    assert abs(mean_n - e_n) <= 4 * se_mean
    assert abs(p_full - p5) <= 4 * se_p
    # the pass and the steps sum in different orders (40-row and 8-row launch shapes), so near-ties can
    # resolve differently; each such row passed the near-tie rule above, and they stay rare
    assert n_tie_rows <= max(2, n_checked_rows // 50)
