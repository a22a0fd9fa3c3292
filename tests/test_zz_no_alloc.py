"""decode_step_noalloc against decode_step, through the C ABI.

The allocation-free entry point runs the same step with its workspace in the
library's own per-GPU scratch array. Two calls in a row, the second with a
smaller batch (so the scratch array keeps the first call's contents): at
7B widths with one layer, 8 sequences x 5 verify rows (the split-K tile path
and the largest workspace of the two), then 2 sequences x 1 row (the
row-streaming path). Each call's logits, greedy tokens, top-2 gaps, accepted
lengths, bonus tokens and written K/V rows must equal those of decode_step
with a caller workspace on the same inputs, bit for bit: the kernels and
their launch shapes are the same, only the workspace address differs.
"""
import dataclasses

import pytest
import torch

import synth
import verify_step_amd as vs
from harness import GpuModel, GpuPool, SeqSpec, make_step
from synth import workloads as W

pytestmark = pytest.mark.gpu

SEED_W, SEED_KV, SEED_TOK, SEED_CTX = 7101, 7102, 7103, 7104


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _outputs(sb, pool, rows, ctxs, K):
    M = len(ctxs) * K
    got = [sb.logits[:M].clone(), sb.argmax[:M].clone(), sb.gap[:M].clone()]
    if sb.accept_len is not None:
        got += [sb.accept_len.clone(), sb.bonus.clone()]
    got.append(torch.stack([pool.read(rows[b], ctxs[b], ctxs[b] + K) for b in range(len(ctxs))]))
    return got


def test_noalloc_step_equals_decode_step_on_two_calls():
    dims = dataclasses.replace(W.LLAMA7B, n_layers=1, name="7B-width-1L")
    w_cpu = W.make_weights(dims, SEED_W, gains="random")
    model = GpuModel(dims, weights_cpu=w_cpu)
    stream = torch.cuda.current_stream().cuda_stream
    for B, K in [(8, 5), (2, 1)]:
        _say(f"no-alloc step vs decode_step: 7B widths, 1 layer, fp16, B={B} K={K}")
        ctxs = [int(c) for c in synth.uniform_int(synth.key(SEED_CTX, B, K), 0, B, 1, 2000)]
        max_blocks = -(-(max(ctxs) + K) // 16)
        pool = GpuPool(dims, B * max_blocks + 4)
        rows, specs = [], []
        for b in range(B):
            r = vs.kv_alloc(pool.handle, -(-ctxs[b] // 16))
            pool.write(r, 0, W.kv_block(dims, SEED_KV, 100 * K + b, 0, ctxs[b]))
            rows.append(vs.kv_append(pool.handle, r, max_blocks, ctxs[b], K))
            specs.append(SeqSpec(ctxs[b], W.token_ids(SEED_TOK, 100 * K + b, K, dims.vocab)))
        g0 = [int(t) for t in synth.uniform_int(synth.key(SEED_TOK, 9, B), 0, B, 0, dims.vocab)] if K > 1 else None
        sb = make_step(model, pool, specs, rows, max_blocks=max_blocks, g0=g0)
        assert sb.ws_bytes <= vs.VS_NOALLOC_SCRATCH_BYTES
        vs.decode_step(sb.desc, sb.block_tables, model.w, sb.out, sb.ws, sb.ws_bytes, stream)
        torch.cuda.synchronize()
        want = _outputs(sb, pool, rows, ctxs, K)
        # clear the outputs and the K/V rows the step writes, then the allocation-free call
        sb.logits.fill_(float("nan"))
        sb.argmax.fill_(-7)
        sb.gap.fill_(float("nan"))
        if g0 is not None:
            sb.accept_len.fill_(-7)
            sb.bonus.fill_(-7)
        for b in range(B):
            pool.write(rows[b], ctxs[b], torch.zeros(1, 2, K, dims.n_kv_heads, dims.head_dim, dtype=dims.torch_dtype))
        vs.decode_step_noalloc(sb.desc, sb.block_tables, model.w, sb.out, stream)
        torch.cuda.synchronize()
        got = _outputs(sb, pool, rows, ctxs, K)
        names = ["logits", "argmax", "gap"] + (["accept_len", "bonus"] if g0 is not None else []) + ["K/V rows"]
        for n, a, c in zip(names, want, got):
            assert torch.equal(a.view(torch.uint8) if a.is_floating_point() else a,
                               c.view(torch.uint8) if c.is_floating_point() else c), f"B={B} K={K}: {n} differ"
        _say(f"no-alloc step B={B} K={K}: outputs equal decode_step's bit for bit")
        pool.close()
