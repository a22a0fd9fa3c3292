"""7B fp16 mixed step: 64 decode rows on shared prefixes plus a 512-row prompt chunk.

The workload ([KV Cache] section 05 block sharing and prefix caching, section 06
chunked prefill; [Serving] "Chunked prefill"; [Serving Efficiency] section 31.3):
4 prompts of 1024 tokens each sit in 64 pages that the prefix-cache index names
by their chained block hashes; each of 16 sequences per prompt finds its prefix
by a lookup in the index (reference count 17: the 16 sequences plus the index);
each sequence has a private suffix of 16..512 tokens and decodes one token; in
the same step a new 3000-token prompt runs its first 512-position chunk
(positions 0..511, causal within the chunk, no logits). M = 576 rows go through
the tile (MFMA) path.

Checked against the oracle on one sampled decode sequence per prefix and on
the whole chunk: logits, greedy tokens, and every K/V row written (the
chunk's 512 rows in all 32 layers). The shared prefix pages must be untouched.
The step runs twice: with each prompt's 16 sequences named as a prefix group
(their 64 shared pages read once per group and head) and without groups.
Through 32 layers the bound of a row is the stated tolerance or twice the
distance between the oracle's float64 and fp32 realisations, whichever is
larger.
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

SEED_W, SEED_KV, SEED_TOK, SEED_CHURN, SEED_PAGES = 5001, 5002, 5003, 5004, 5006
N_PREFIX, PER_PREFIX, PREFIX, CHUNK = 4, 16, 1024, 512


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def test_7b_shared_prefixes_and_prompt_chunk():
    dims = W.LLAMA7B
    _say("7B fp16 mixed: weights")
    w_cpu = W.make_weights(dims, SEED_W)
    model = GpuModel(dims, weights_cpu=w_cpu)
    B_dec = N_PREFIX * PER_PREFIX
    suffix = [int(s) for s in synth.uniform_int(synth.key(SEED_CHURN, 1), 0, B_dec, 16, 513)]
    max_blocks = -(-(PREFIX + max(suffix) + 1) // 16)
    n_pages = N_PREFIX * PREFIX // 16 + sum(-(-(s + 1) // 16) for s in suffix) + CHUNK // 16 + 64
    pool = GpuPool(dims, n_pages)
    pool.view().normal_()  # pages of unsampled sequences keep arbitrary values
    ids = vs.kv_alloc(pool.handle, n_pages)
    perm = synth.permutation(synth.key(SEED_PAGES), n_pages)
    vs.kv_free(pool.handle, [ids[int(i)] for i in perm])

    # each prompt's prefill leaves its 64 full blocks in the index, which then holds their only reference
    root = vs.kv_prefix_root(f"7B;f16;weights={SEED_W};theta=10000;scope=test".encode())
    prefix_rows, prefix_kv, prefix_tok, prefix_hash = [], [], [], []
    for p in range(N_PREFIX):
        toks = W.token_ids(SEED_TOK, 500 + p, PREFIX, dims.vocab)
        r = vs.kv_alloc(pool.handle, PREFIX // 16)
        kv = W.kv_block(dims, SEED_KV, p, 0, PREFIX)
        pool.write(r, 0, kv)
        h = vs.kv_prefix_chain(root, toks, 16)
        assert vs.kv_prefix_insert(pool.handle, root, h, toks, r) == PREFIX // 16
        vs.kv_free(pool.handle, r)
        prefix_rows.append(r)
        prefix_kv.append(kv)
        prefix_tok.append(toks)
        prefix_hash.append(h)
    sampled = {p * PER_PREFIX + int(synth.uniform_int(synth.key(SEED_CHURN, 2), p, 1, 0, PER_PREFIX)[0])
               for p in range(N_PREFIX)}
    _say(f"7B fp16 mixed: suffixes {min(suffix)}..{max(suffix)}, sampled decode sequences {sorted(sampled)}")

    specs, rows, states, order = [], [], [], []
    for b in range(B_dec):
        p = b // PER_PREFIX
        # the sequence's prompt starts with the shared 1024 tokens: the index hands over their pages
        hit = vs.kv_prefix_lookup(pool.handle, root, vs.kv_prefix_chain(root, prefix_tok[p], 16), prefix_tok[p])
        assert hit == prefix_rows[p], "every full block of the prefix is found"
        ctx = PREFIX + suffix[b]
        r = vs.kv_append(pool.handle, hit, max_blocks, PREFIX, suffix[b] + 1)
        assert r[:PREFIX // 16] == prefix_rows[p], "a page-aligned prefix stays shared"
        tok = W.token_ids(SEED_TOK, b, 1, dims.vocab)
        specs.append(SeqSpec(ctx, tok))
        rows.append(r)
        if b in sampled:
            skv = W.kv_block(dims, SEED_KV, 100 + b, PREFIX, ctx)
            pool.write(r, PREFIX, skv)
            full = torch.zeros(dims.n_layers, 2, ctx + 1, dims.n_kv_heads, dims.head_dim, dtype=dims.torch_dtype)
            full[:, :, :PREFIX] = prefix_kv[p]
            full[:, :, PREFIX:ctx] = skv
            states.append(oracle.SeqState(full, ctx, list(tok)))
            order.append(b)
    for p in range(N_PREFIX):
        assert vs.kv_refcount(pool.handle, prefix_rows[p][0]) == PER_PREFIX + 1
    # the prompt chunk: a new sequence, positions 0..511, no logits
    chunk_tok = W.token_ids(SEED_TOK, 999, CHUNK, dims.vocab)
    crow = vs.kv_append(pool.handle, [], max_blocks, 0, CHUNK)
    specs.append(SeqSpec(0, chunk_tok, want_logits=False))
    rows.append(crow)
    states.append(oracle.SeqState(torch.zeros(dims.n_layers, 2, CHUNK, dims.n_kv_heads, dims.head_dim,
                                              dtype=dims.torch_dtype), 0, list(chunk_tok), want_logits=False))
    order.append(B_dec)

    # each prompt's 16 sequences form a prefix group over its 64 pages; the step runs with the groups
    # (the prefixes read once per group) and without them, the same K/V rows written by both
    groups = [(p * PER_PREFIX, PER_PREFIX, PREFIX // 16) for p in range(N_PREFIX)]
    runs = {}
    for label, g in (("prefix groups", groups), ("no groups", None)):
        _say(f"7B fp16 mixed: GPU step, M = 576, {label}")
        sb = make_step(model, pool, specs, rows, max_blocks=max_blocks, groups=g)
        flags = torch.zeros(1, dtype=torch.int32, device="cuda")
        sb.desc.error_flags = flags.data_ptr()
        vs.decode_step(sb.desc, sb.block_tables, model.w, sb.out, sb.ws, sb.ws_bytes,
                       torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert int(flags.item()) == 0, f"{label}: validation word {int(flags.item())}"
        runs[label] = sb
    _say("7B fp16 mixed: oracle on the sampled sequences and the chunk")
    states32 = [oracle.SeqState(st.kv.clone(), st.ctx, list(st.tokens), st.want_logits) for st in states]
    ref = oracle.decode_step(dims, w_cpu, states)
    alt = oracle.decode_step(dims, w_cpu, states32, compute="f32")
    tol = TOL[dims.dtype]
    ties = TieLog()
    for label, sb in runs.items():
        am = sb.argmax[:B_dec + CHUNK].cpu().tolist()
        for j, b in enumerate(order[:-1]):
            check_rows([sb.logits[b].cpu()], [ref.logits[j]], tol, f"{label}: decode seq {b} logits", [alt.logits[j]])
            ties.check(am[b], ref.argmax[j], ref.logits[j], ref.gap[j], f"{label}: decode seq {b}", alt.logits[j])
        assert all(a == -1 for a in am[B_dec:]), "chunk rows carry no logits"
    for j, b in enumerate(order[:-1]):
        c = specs[b].ctx
        got = pool.read(rows[b], c, c + 1).double()
        want = states[j].kv[:, :, c:c + 1].double()
        want32 = states32[j].kv[:, :, c:c + 1].double()
        err = (got - want).abs().amax(dim=(3, 4)) / want.abs().amax(dim=(3, 4))
        bound = (2 * (want32 - want).abs().amax(dim=(3, 4)) / want.abs().amax(dim=(3, 4))).clamp(min=tol)
        assert bool((err <= bound).all()), f"decode seq {b} K/V rows: worst error / bound {float((err / bound).max()):.3f}"
    got = pool.read(crow, 0, CHUNK).double()  # [layer][2][512][heads][dim]
    want = states[-1].kv.double()
    want32 = states32[-1].kv.double()
    err = (got - want).abs().amax(dim=(3, 4)) / want.abs().amax(dim=(3, 4))
    bound = (2 * (want32 - want).abs().amax(dim=(3, 4)) / want.abs().amax(dim=(3, 4))).clamp(min=tol)
    worst = float(err.max())
    assert bool((err <= bound).all()), \
        f"chunk K/V rows: worst error / bound {float((err / bound).max()):.3f} at {divmod(int((err / bound).argmax()), CHUNK)}"
    _say(f"7B fp16 mixed: chunk K/V worst row error {worst:.2e}; decode rows: {ties.report()}")
    for p in range(N_PREFIX):
        assert torch.equal(pool.read(prefix_rows[p], 0, PREFIX), prefix_kv[p]), "shared prefix pages changed"
    pool.close()
