"""7B bf16 continuous batching: B sequences of mixed context decode together, then churn.

The workload: 7B shape, bf16 weights and K/V; a pool of 64 x 257 + 64 pages
(about 138 GB) whose free list is shuffled; B in {1, 8, 32, 64} sequences with
contexts uniform in 128..4096; every sequence decodes one token per step; between
the two steps floor(B/8) sequences chosen at random finish and are replaced by
new ones (B = 1: one replacement with probability 1/8), the survivors append
their greedy token ([Serving] "Continuous batching"; [KV Cache] section 05).

Rows of a step are independent, so parity is checked on a seeded sample of up
to 8 sequences per step (survivors and newcomers alike): their K/V is the
synthetic N(0, 1) of the recipe and the oracle runs them alone. The other
sequences' pages hold arbitrary values, which must not leak into the sampled
rows. Checked: each sampled row's logits, greedy token and gap, and the K/V row
each wrote in every layer. Through 32 layers of bf16 storage the bound of a row
is the stated tolerance or twice the distance between the oracle's float64 and
fp32 realisations, whichever is larger.
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

WL = 3
SEED_W, SEED_KV, SEED_TOK, SEED_CHURN, SEED_PAGES = 3001, 3002, 3003, 3004, 3006
MAX_B, CTX_LO, CTX_HI = 64, 128, 4096
N_PAGES = MAX_B * 257 + 64
MAX_BLOCKS = 257
N_SAMPLE = 8


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def env():
    dims = W.LLAMA7B.with_dtype("bf16")
    _say("7B bf16 batch: weights and a 138 GB pool")
    w_cpu = W.make_weights(dims, SEED_W)
    model = GpuModel(dims, weights_cpu=w_cpu)
    pool = GpuPool(dims, N_PAGES)
    pool.view().normal_()  # pages of unsampled sequences keep arbitrary values
    ids = vs.kv_alloc(pool.handle, N_PAGES)
    perm = synth.permutation(synth.key(SEED_PAGES), N_PAGES)
    vs.kv_free(pool.handle, [ids[int(i)] for i in perm])
    torch.cuda.synchronize()
    yield dims, w_cpu, model, pool
    pool.close()


class Seq:
    def __init__(self, content, ctx, sampled):
        self.content, self.ctx, self.sampled = content, ctx, sampled
        self.row = None
        self.state = None  # oracle state of a sampled sequence
        self.state32 = None  # the oracle's fp32 realisation (its own cache)


def _new_seq(dims, pool, content, ctx, sampled, tok_tag):
    s = Seq(content, ctx, sampled)
    s.row = vs.kv_alloc(pool.handle, -(-ctx // 16))
    s.row = vs.kv_append(pool.handle, s.row, MAX_BLOCKS, ctx, 1)
    tok = W.token_ids(SEED_TOK, tok_tag, 1, dims.vocab)
    if sampled:
        kv = W.kv_block(dims, SEED_KV, content, 0, ctx)
        pool.write(s.row, 0, kv)
        full = torch.zeros(dims.n_layers, 2, ctx + 2, dims.n_kv_heads, dims.head_dim, dtype=dims.torch_dtype)
        full[:, :, :ctx] = kv
        s.state = oracle.SeqState(full, ctx, list(tok))
        s.state32 = oracle.SeqState(full.clone(), ctx, list(tok))
    s.tok = tok
    return s


def _run_and_check(dims, w_cpu, model, pool, seqs, what):
    sb = make_step(model, pool, [SeqSpec(s.ctx, list(s.tok)) for s in seqs], [s.row for s in seqs],
                   max_blocks=MAX_BLOCKS)
    vs.decode_step(sb.desc, sb.block_tables, model.w, sb.out, sb.ws, sb.ws_bytes,
                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    samp = [i for i, s in enumerate(seqs) if s.sampled]
    ref = oracle.decode_step(dims, w_cpu, [seqs[i].state for i in samp])
    alt = oracle.decode_step(dims, w_cpu, [seqs[i].state32 for i in samp], compute="f32")
    tol = TOL[dims.dtype]
    am = sb.argmax[:len(seqs)].cpu().tolist()
    ties = TieLog()
    for j, i in enumerate(samp):
        s = seqs[i]
        check_rows([sb.logits[i].cpu()], [ref.logits[j]], tol, f"{what} seq {i} logits", [alt.logits[j]])
        ties.check(am[i], ref.argmax[j], ref.logits[j], ref.gap[j], f"{what} seq {i}", alt.logits[j])
        got = pool.read(s.row, s.ctx, s.ctx + 1).double()
        want = s.state.kv[:, :, s.ctx:s.ctx + 1].double()
        want32 = s.state32.kv[:, :, s.ctx:s.ctx + 1].double()
        for l in range(dims.n_layers):
            check_rows([got[l, t, 0] for t in range(2)], [want[l, t, 0] for t in range(2)], tol,
                       f"{what} seq {i} layer {l} K/V", [want32[l, t, 0] for t in range(2)], alt_group=True)
    _say(f"{what}: {ties.report()}")
    return am


@pytest.mark.parametrize("B", [1, 8, 32, 64])
def test_7b_bf16_batch_with_churn(env, B):
    dims, w_cpu, model, pool = env
    free0 = vs.kv_num_free(pool.handle)
    ck = synth.key(SEED_CHURN, B)
    ctxs = [int(c) for c in synth.uniform_int(ck, 0, B, CTX_LO, CTX_HI + 1)]
    sample = set(int(i) for i in synth.permutation(synth.key(SEED_CHURN, 100 + B), B)[:N_SAMPLE])
    _say(f"7B bf16 B={B}: contexts {min(ctxs)}..{max(ctxs)}, sampled {sorted(sample)}")
    seqs = [_new_seq(dims, pool, 1000 * B + i, ctxs[i], i in sample, 1000 * B + i) for i in range(B)]
    am = _run_and_check(dims, w_cpu, model, pool, seqs, f"B={B} step 1")

    # churn: floor(B/8) finish (B = 1: with probability 1/8) and new sequences take their places
    n_out = B // 8 if B >= 8 else int(synth.uniform(synth.key(SEED_CHURN, 200 + B), 0, 1)[0] < 1 / 8)
    leaving = [int(i) for i in synth.permutation(synth.key(SEED_CHURN, 300 + B), B)[:n_out]]
    new_ctx = [int(c) for c in synth.uniform_int(synth.key(SEED_CHURN, 400 + B), 0, max(n_out, 1), CTX_LO,
                                                 CTX_HI + 1)]
    for i, s in enumerate(seqs):
        if i in leaving:
            continue
        s.tok = [am[i]]
        s.row = vs.kv_append(pool.handle, s.row, MAX_BLOCKS, s.ctx + 1, 1)
        s.ctx += 1
        if s.sampled:
            for o in (s.state, s.state32):
                o.ctx += 1
                o.tokens = [am[i]]
    for j, i in enumerate(leaving):
        vs.kv_free(pool.handle, seqs[i].row)
        seqs[i] = _new_seq(dims, pool, 1000 * B + 500 + j, new_ctx[j], i in sample, 1000 * B + 500 + j)
    _say(f"7B bf16 B={B}: {n_out} replaced {leaving}")
    _run_and_check(dims, w_cpu, model, pool, seqs, f"B={B} step 2")
    for s in seqs:
        vs.kv_free(pool.handle, s.row)
    assert vs.kv_num_free(pool.handle) == free0
