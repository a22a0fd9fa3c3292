"""7B fp16 greedy decode at batch 1 against the oracle, in the benchmark's launch configuration.

The workload: 32 layers, d_model 4096, 32 heads x 128, MLP 11008, vocab 32000,
fp16 weights N(0, 0.02), one sequence whose 2048 cached positions (synthetic
N(0, 1) K/V) sit in 16-token pages scattered through the pool. Three greedy
steps: the first eager, the next two replays of a captured HIP graph, with the
host's page bookkeeping (kv_append) between them, exactly as bench.py runs
them; the batch descriptor carries the same context capacity, so the split
plan of the attention kernel is the one the benchmark times. Each step is
checked against the oracle: the logits row, the greedy token, the top-2 gap,
and the K and V rows the step wrote in every layer. Through 32 layers the
bound of a row is the stated tolerance or twice the distance between the
oracle's float64 and fp32 realisations, whichever is larger. The next step's input is
the GPU's token (the oracle is fed the same token).
"""
import pytest
import torch

import bench
import oracle
import synth
import verify_step_amd as vs
from harness import GpuModel, GpuPool, SeqSpec, make_step, model_desc
from harness.compare import TOL, TieLog, check_rows
from synth import workloads as W

pytestmark = pytest.mark.gpu

SEED_W, SEED_KV, SEED_TOK, SEED_PAGES = 2001, 2002, 2003, 2006
CTX0 = 2048
# positions the benchmark's default run reaches (2048 + 16 warm-up + 256 timed + the per-kernel timing
# steps + 1); the descriptor's max_ctx sets the key-split plan, so the test uses the benchmark's value
CAPACITY = CTX0 + 16 + 256 + len(bench.TIMED_KINDS) * bench.ROOFLINE_STEPS + 1


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def check_step(dims, sb, ref, alt, what, ties):
    tol = TOL[dims.dtype]
    am = int(sb.argmax[0])
    gap = float(sb.gap[0])
    check_rows([sb.logits[0].cpu()], [ref.logits[0]], tol, f"{what} logits", [alt.logits[0]])
    exact = ties.check(am, ref.argmax[0], ref.logits[0], ref.gap[0], what, alt.logits[0])
    if exact:
        assert abs(gap - ref.gap[0]) <= tol * float(ref.logits[0].abs().max()), (gap, ref.gap[0])
    return am


def test_7b_decode_b1_graph_replays_match_oracle():
    dims = W.LLAMA7B
    _say("7B fp16 decode B=1 ctx 2048: weights")
    w_cpu = W.make_weights(dims, SEED_W)
    model = GpuModel(dims, weights_cpu=w_cpu)
    n_pages = -(-CAPACITY // 16) + 8
    max_blocks = -(-CAPACITY // 16)
    pool = GpuPool(dims, n_pages)
    ids = vs.kv_alloc(pool.handle, n_pages)
    perm = synth.permutation(synth.key(SEED_PAGES), n_pages)
    vs.kv_free(pool.handle, [ids[int(i)] for i in perm])
    row = vs.kv_alloc(pool.handle, CTX0 // 16)
    assert sorted(row) != row, "pages should be scattered"
    kv0 = W.kv_block(dims, SEED_KV, 0, 0, CTX0)
    pool.write(row, 0, kv0)
    tok0 = W.token_ids(SEED_TOK, 0, 1, dims.vocab)
    row = vs.kv_append(pool.handle, row, max_blocks, CTX0, 1)
    sb = make_step(model, pool, [SeqSpec(CTX0, tok0)], [row], max_blocks=max_blocks)
    sb.desc.max_ctx = CAPACITY
    sb.ws_bytes = vs.decode_step_workspace_bytes(sb.desc, model_desc(dims))
    sb.ws = torch.empty(sb.ws_bytes, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    full = torch.zeros(dims.n_layers, 2, CTX0 + 3, dims.n_kv_heads, dims.head_dim, dtype=dims.torch_dtype)
    full[:, :, :CTX0] = kv0
    st = oracle.SeqState(full, CTX0, list(tok0))
    st32 = oracle.SeqState(full.clone(), CTX0, list(tok0))  # the oracle's fp32 realisation, its own cache

    # the benchmark's device-side loop: tokens are read from the argmax array, ctx_len advances in the step
    sb.argmax[:1].copy_(sb.tokens[:1])
    sb.desc.tokens = sb.argmax.data_ptr()
    sb.desc.ctx_advance = sb.ctx_len.data_ptr()

    def device_step():
        vs.decode_step(sb.desc, sb.block_tables, model.w, sb.out, sb.ws, sb.ws_bytes,
                       torch.cuda.current_stream().cuda_stream)

    state = {"row": row, "len": CTX0}

    def bookkeeping():
        cur = state["len"] + 1
        r = vs.kv_append(pool.handle, state["row"], max_blocks, cur, 1)
        if len(r) != len(state["row"]):
            sb.block_tables[0, len(r) - 1] = r[-1]
        state["row"], state["len"] = r, cur

    graph = None
    ties = TieLog()
    for step in range(3):
        pos = CTX0 + step
        _say(f"7B fp16 decode B=1 step {step} at position {pos} ({'graph replay' if step else 'eager'})")
        if step == 0:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                device_step()
            torch.cuda.current_stream().wait_stream(s)
            bookkeeping()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):  # capture records the step without running it
                device_step()
            torch.cuda.synchronize()
        else:
            graph.replay()
            torch.cuda.synchronize()
        ref = oracle.decode_step(dims, w_cpu, [st])
        alt = oracle.decode_step(dims, w_cpu, [st32], compute="f32")
        am = check_step(dims, sb, ref, alt, f"step {step}", ties)
        got = pool.read(state["row"], pos, pos + 1).double()
        want = st.kv[:, :, pos:pos + 1].double()
        want32 = st32.kv[:, :, pos:pos + 1].double()
        for l in range(dims.n_layers):
            check_rows([got[l, 0, 0], got[l, 1, 0]], [want[l, 0, 0], want[l, 1, 0]], TOL[dims.dtype],
                       f"step {step} layer {l} K/V", [want32[l, 0, 0], want32[l, 1, 0]], alt_group=True)
        assert int(sb.ctx_len[0]) == pos + 1, "the step advances the context length"
        for o in (st, st32):
            o.ctx += 1
            o.tokens = [am]
        if step > 0:
            bookkeeping()
    assert torch.equal(pool.read(state["row"], 0, CTX0), kv0), "the step must not touch cached positions"
    _say(f"7B fp16 decode B=1: {ties.report()}")
    pool.close()
