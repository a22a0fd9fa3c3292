"""Grouped K/V heads through all 32 layers: a batch of 8B-GQA-width sequences against the oracle.

The shape: Llama 3.1 8B's widths ([KV Cache] section 03 lists it with 32 query heads over 8 K/V heads;
section 04 defines grouped-query attention: each K/V head serves a group of 4 query heads), d_model
4096, head_dim 128, MLP 14336, vocabulary 128256, bf16 weights and K/V, 32 layers. Three steps of
different launch shapes: 16 sequences x 1 row (the 16-feature tile products; grouped heads through the
matrix-core attention), 32 sequences x 1 row (split-K products; 256 (sequence, K/V head) pairs, so the
grouped heads go through the VALU attention's four-head workgroups) and 8 sequences x 5 verify rows with
fused acceptance. The contexts are uniform in 128..4096, with pages scattered through a shuffled pool.

Rows are independent, so two sampled sequences per step are run by the oracle alone: their logits,
greedy tokens and every K/V row they wrote in all 32 layers. The other sequences' pages hold
arbitrary values. Through 32 layers the bound of a row is the stated tolerance or twice the distance
between the oracle's float64 and fp32 realisations, whichever is larger (the distance taken over the
rows of one sequence in one layer, or over its logit rows); a greedy token may differ
only where the oracle's top-2 gap is below max(1e-3, twice the row's largest difference between those
two realisations).
"""
import pytest
import torch

import oracle
import synth
import verify_step_amd as vs
from harness import GpuModel, GpuPool, SeqSpec, make_step
from harness.compare import TOL, TieLog, check_rows
from synth import workloads as W

pytestmark = pytest.mark.gpu

SEED_W, SEED_KV, SEED_TOK, SEED_CTX, SEED_PAGES = 8101, 8102, 8103, 8104, 8106
CTX_LO, CTX_HI, N_SAMPLE = 128, 4096, 2


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def env():
    dims = W.GQA8B.with_dtype("bf16")
    _say("8B-GQA bf16: weights")
    w_cpu = W.make_weights(dims, SEED_W)
    model = GpuModel(dims, weights_cpu=w_cpu)
    max_blocks = -(-(CTX_HI + 5) // 16)
    n_pages = 32 * max_blocks + 16
    pool = GpuPool(dims, n_pages)
    pool.view().normal_()  # pages of unsampled sequences keep arbitrary values
    ids = vs.kv_alloc(pool.handle, n_pages)
    perm = synth.permutation(synth.key(SEED_PAGES), n_pages)
    vs.kv_free(pool.handle, [ids[int(i)] for i in perm])
    torch.cuda.synchronize()
    yield dims, w_cpu, model, pool, max_blocks
    pool.close()


@pytest.mark.parametrize("B,K", [(16, 1), (32, 1), (8, 5)])
def test_8b_gqa_32_layers_sampled(env, B, K):
    dims, w_cpu, model, pool, max_blocks = env
    free0 = vs.kv_num_free(pool.handle)
    ctxs = [int(c) for c in synth.uniform_int(synth.key(SEED_CTX, B, K), 0, B, CTX_LO, CTX_HI + 1)]
    sample = sorted(int(i) for i in synth.permutation(synth.key(SEED_CTX, 100 + B, K), B)[:N_SAMPLE])
    _say(f"8B-GQA bf16 B={B} K={K}: contexts {min(ctxs)}..{max(ctxs)}, sampled {sample}")
    rows, specs, states, states32 = [], [], [], []
    for b in range(B):
        r = vs.kv_alloc(pool.handle, -(-ctxs[b] // 16))
        r = vs.kv_append(pool.handle, r, max_blocks, ctxs[b], K)
        toks = W.token_ids(SEED_TOK, 1000 * K + b, K, dims.vocab)
        rows.append(r)
        specs.append(SeqSpec(ctxs[b], list(toks)))
        if b in sample:
            kv = W.kv_block(dims, SEED_KV, 1000 * K + b, 0, ctxs[b])
            pool.write(r, 0, kv)
            full = torch.zeros(dims.n_layers, 2, ctxs[b] + K, dims.n_kv_heads, dims.head_dim, dtype=dims.torch_dtype)
            full[:, :, :ctxs[b]] = kv
            states.append(oracle.SeqState(full, ctxs[b], list(toks)))
            states32.append(oracle.SeqState(full.clone(), ctxs[b], list(toks)))
    g0 = [int(t) for t in synth.uniform_int(synth.key(SEED_TOK, 7, B), 0, B, 0, dims.vocab)] if K > 1 else None
    sb = make_step(model, pool, specs, rows, max_blocks=max_blocks, g0=g0)
    vs.decode_step(sb.desc, sb.block_tables, model.w, sb.out, sb.ws, sb.ws_bytes,
                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    _say(f"8B-GQA bf16 B={B} K={K}: oracle on the sampled sequences")
    ref = oracle.decode_step(dims, w_cpu, states)
    alt = oracle.decode_step(dims, w_cpu, states32, compute="f32")
    tol = TOL[dims.dtype]
    am = sb.argmax[:B * K].cpu().tolist()
    ties = TieLog()
    worst = 0.0
    for j, b in enumerate(sample):
        worst = max(worst, check_rows([sb.logits[K * b + i].cpu() for i in range(K)], ref.logits[K * j:K * j + K], tol,
                                      f"seq {b} logits", alt.logits[K * j:K * j + K], alt_group=True))
        for i in range(K):
            r, jr = K * b + i, K * j + i
            ties.check(am[r], ref.argmax[jr], ref.logits[jr], ref.gap[jr], f"seq {b} row {i}", alt.logits[jr])
        got = pool.read(rows[b], ctxs[b], ctxs[b] + K).double()
        want = states[j].kv[:, :, ctxs[b]:ctxs[b] + K].double()
        want32 = states32[j].kv[:, :, ctxs[b]:ctxs[b] + K].double()
        for l in range(dims.n_layers):
            for t in range(2):
                check_rows([got[l, t, i] for i in range(K)], [want[l, t, i] for i in range(K)], tol,
                           f"seq {b} layer {l} {'KV'[t]}", [want32[l, t, i] for i in range(K)], alt_group=True)
    if K > 1:  # fused acceptance applies the rule to the step's own greedy tokens
        acc, bon = sb.accept_len.cpu().tolist(), sb.bonus.cpu().tolist()
        for b in range(B):
            assert (acc[b], bon[b]) == oracle.accept_greedy(specs[b].tokens, g0[b], am[K * b:K * b + K])
    _say(f"8B-GQA bf16 B={B} K={K}: worst logits row {worst:.2e}; {ties.report()}")
    for r in rows:
        vs.kv_free(pool.handle, r)
    assert vs.kv_num_free(pool.handle) == free0
