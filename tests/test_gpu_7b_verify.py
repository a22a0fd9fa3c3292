"""7B fp16 speculative verify: 8 sequences x 5 drafted rows against the oracle.

The workload ([KV Cache] section 08; [Spending the Idle] section 12.4): 8
sequences with 1023 synthetic cached positions each take one plain decode step
at position 1023 (its greedy token is g0), then one verify pass feeds K = 5
drafted tokens at positions 1024..1028, causal among themselves, with greedy
acceptance fused into the step. The drafts were written by
tests/golden/make_verify_drafts.py from the oracle alone: each is the oracle's
own greedy token with probability 0.7, else a random token.

Checked: the decode step's logits and g0; the verify pass's 40 logit rows,
greedy tokens and gaps, the K/V rows it wrote; accept length and bonus per
sequence against the acceptance rule applied to the oracle's tokens (they may
differ only where the first differing decision is a recorded near-tie), and
against the stored greedy chain. A second verify pass on the same inputs
rewrites the same K/V rows and must reproduce every output bit for bit.
Through 32 layers the bound of a row is the stated tolerance or twice the
distance between the oracle's float64 and fp32 realisations, whichever is
larger; a greedy token may differ only where the oracle's top-2 gap is below
max(1e-3, twice the row's largest difference between those two oracle
realisations).
"""
import json
import os

import pytest
import torch

import oracle
import synth
import verify_step_amd as vs
from harness import GpuModel, GpuPool, SeqSpec, make_step
from harness.compare import NEAR_TIE, TOL, TieLog, check_rows, first_divergence_is_near_tie, tie_slack
from synth import workloads as W

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
SEED_PAGES = 4006


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def test_7b_verify_k5_b8_matches_oracle():
    g = json.load(open(os.path.join(HERE, "golden", "verify_drafts_7b.json")))
    dims = W.LLAMA7B
    B, CTX, K = g["B"], g["ctx"], g["K"]
    seeds = g["seeds"]
    _say("7B fp16 verify B=8 K=5: weights")
    w_cpu = W.make_weights(dims, seeds["weights"])
    model = GpuModel(dims, weights_cpu=w_cpu)
    max_blocks = -(-(CTX + K) // 16)
    pool = GpuPool(dims, B * max_blocks + 16)
    ids = vs.kv_alloc(pool.handle, pool.num_pages)
    perm = synth.permutation(synth.key(SEED_PAGES), pool.num_pages)
    vs.kv_free(pool.handle, [ids[int(i)] for i in perm])

    rows, states = [], []
    for b in range(B):
        kv = W.kv_block(dims, seeds["kv"], b, 0, CTX - 1)
        r = vs.kv_alloc(pool.handle, -(-(CTX - 1) // 16))
        pool.write(r, 0, kv)
        r = vs.kv_append(pool.handle, r, max_blocks, CTX - 1, 1)
        rows.append(r)
        full = torch.zeros(dims.n_layers, 2, CTX + K, dims.n_kv_heads, dims.head_dim, dtype=dims.torch_dtype)
        full[:, :, :CTX - 1] = kv
        states.append(oracle.SeqState(full, CTX - 1, [g["token_at_1023"][b]]))
    states32 = [oracle.SeqState(st.kv.clone(), st.ctx, list(st.tokens)) for st in states]  # fp32 realisation

    # the plain decode step at position 1023
    _say("7B fp16 verify: decode step at position 1023")
    sb = make_step(model, pool, [SeqSpec(CTX - 1, [g["token_at_1023"][b]]) for b in range(B)], rows,
                   max_blocks=max_blocks)
    vs.decode_step(sb.desc, sb.block_tables, model.w, sb.out, sb.ws, sb.ws_bytes,
                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = oracle.decode_step(dims, w_cpu, states)
    alt = oracle.decode_step(dims, w_cpu, states32, compute="f32")
    tol = TOL[dims.dtype]
    am = sb.argmax[:B].cpu().tolist()
    check_rows([sb.logits[b].cpu() for b in range(B)], ref.logits, tol, "decode logits", alt.logits)
    ties = TieLog()
    for b in range(B):
        # float64 sums may round differently on another host; only a recorded near-tie may change g0
        assert ref.argmax[b] == g["g0"][b] or g["g0_gap"][b] < NEAR_TIE, "the oracle must reproduce the stored g0"
        ties.check(am[b], ref.argmax[b], ref.logits[b], ref.gap[b], f"decode seq {b}", alt.logits[b])
    _say(f"7B fp16 verify: decode step: {ties.report()}")

    # the verify pass: drafts at 1024..1028, g0 from the oracle (the drafts were built on it)
    for b in range(B):
        rows[b] = vs.kv_append(pool.handle, rows[b], max_blocks, CTX, K)
        for st in (states[b], states32[b]):
            st.ctx = CTX
            st.tokens = list(g["drafts"][b])
    g0 = list(g["g0"])
    vb = make_step(model, pool, [SeqSpec(CTX, list(g["drafts"][b])) for b in range(B)], rows,
                   max_blocks=max_blocks, g0=g0)
    outs = []
    for rep in range(2):
        _say(f"7B fp16 verify: verify pass {rep}")
        vs.decode_step(vb.desc, vb.block_tables, model.w, vb.out, vb.ws, vb.ws_bytes,
                       torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        outs.append((vb.logits.cpu().clone(), vb.argmax.cpu().clone(), vb.gap.cpu().clone(),
                     vb.accept_len.cpu().clone(), vb.bonus.cpu().clone(),
                     torch.stack([pool.read(rows[b], CTX, CTX + K) for b in range(B)])))
    for a, c in zip(outs[0], outs[1]):
        assert torch.equal(a, c), "a repeated verify pass must reproduce its outputs bit for bit"

    ref = oracle.decode_step(dims, w_cpu, states)
    alt = oracle.decode_step(dims, w_cpu, states32, compute="f32")
    M = B * K
    am = vb.argmax[:M].cpu().tolist()
    worst = check_rows([vb.logits[r].cpu() for r in range(M)], ref.logits, tol, "verify logits", alt.logits)
    e_abs = max(float((vb.logits[r].cpu().double() - ref.logits[r]).abs().max()) for r in range(M))
    _say(f"7B fp16 verify: worst logits row error {worst:.2e} relative, {e_abs:.2e} absolute")
    ties = TieLog()
    for r in range(M):
        ties.check(am[r], ref.argmax[r], ref.logits[r], ref.gap[r], f"verify row {r}", alt.logits[r])
    _say(f"7B fp16 verify: verify rows: {ties.report()}")
    acc = vb.accept_len.cpu().tolist()
    bon = vb.bonus.cpu().tolist()
    n_acc = 0
    for b in range(B):
        rows_b = slice(K * b, K * b + K)
        want = oracle.accept_greedy(g["drafts"][b], g0[b], ref.argmax[rows_b])
        if (acc[b], bon[b]) != want:
            slack = [tie_slack(alt.logits[r], ref.logits[r]) for r in range(K * b, K * b + K)]
            assert first_divergence_is_near_tie(am[rows_b], ref.argmax[rows_b], ref.gap[rows_b], slack), \
                f"seq {b}: accept {(acc[b], bon[b])} vs oracle {want}"
        # the stored chain: the oracle's greedy tokens after d_1..d_4 one step at a time
        chain = [g0[b]] + g["greedy_chain_g1_to_g4"][b]
        lcp = 0
        while lcp < K and g["drafts"][b][lcp] == chain[lcp]:
            lcp += 1
        if min([g["g0_gap"][b]] + g["greedy_chain_gaps"][b]) >= NEAR_TIE:
            assert want[0] == lcp, f"seq {b}: K-row pass and single steps disagree on the accepted length"
            if lcp < K:
                assert want[1] == chain[lcp]
        n_acc += acc[b]
        got = pool.read(rows[b], CTX, CTX + K).double()
        exp = states[b].kv[:, :, CTX:CTX + K].double()
        exp32 = states32[b].kv[:, :, CTX:CTX + K].double()
        for l in range(dims.n_layers):
            for t in range(2):
                check_rows([got[l, t, i] for i in range(K)], [exp[l, t, i] for i in range(K)], tol,
                           f"seq {b} layer {l} {'KV'[t]}", [exp32[l, t, i] for i in range(K)], alt_group=True)
    _say(f"7B fp16 verify: {n_acc} drafts accepted over {B} sequences")
    pool.close()
