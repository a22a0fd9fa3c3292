"""GPU parity on the tiny 1-layer decoder: the HIP path through the C ABI against the oracle.

The tiny workload: d_model 256, 4 heads x 64, MLP 1024, vocab 1000, one layer;
weights N(0, 0.02); KV N(0, 1) in 16-token pages drawn at random from a
64-page pool. Every case prints its name before touching the GPU.
"""
import pytest
import torch

import oracle
import synth
import verify_step_amd as vs
from harness import GpuModel, GpuPool, SeqSpec, alloc_rows, make_step, run_step
from harness.compare import TOL, TieLog, check_kv8, check_rows
from synth import workloads as W

pytestmark = pytest.mark.gpu

SEED_W, SEED_KV, SEED_TOK, SEED_PAGES = 1001, 1002, 1003, 1006


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def oracle_step(dims, w_cpu, seqs_o):
    """The oracle's step on seqs_o (their caches updated in place), with the logits of its fp32
    realisation on copies of the same inputs attached as ref.alt (the near-tie slack's measure)."""
    copies = [oracle.SeqState(s.kv.clone(), s.ctx, list(s.tokens), s.want_logits) for s in seqs_o]
    ref = oracle.decode_step(dims, w_cpu, seqs_o)
    ref.alt = oracle.decode_step(dims, w_cpu, copies, compute="f32").logits
    return ref


def run_case(dims, ctxs, rows_per_seq, gains="one", want=None, g0=None, pool_pages=64, contents=None,
             tokens=None):
    """Run one step on the GPU and in the oracle; return (gpu results, oracle results, helpers)."""
    w_cpu = W.make_weights(dims, SEED_W, gains=gains)
    model = GpuModel(dims, weights_cpu=w_cpu)
    pool = GpuPool(dims, pool_pages)
    B = len(ctxs)
    contents = contents or list(range(B))
    if tokens is None:
        tokens = [W.token_ids(SEED_TOK, 100 + b, rows_per_seq[b], dims.vocab) for b in range(B)]
    want = want or [True] * B
    rows = alloc_rows(pool, [c + k for c, k in zip(ctxs, rows_per_seq)], shuffle_key=synth.key(SEED_PAGES))
    seqs_o = []
    for b in range(B):
        kv = W.kv_block(dims, SEED_KV, contents[b], 0, ctxs[b])
        pool.write(rows[b], 0, kv)
        full = torch.zeros(dims.n_layers, 2, ctxs[b] + rows_per_seq[b], dims.n_kv_heads, dims.head_dim,
                           dtype=dims.kv_torch_dtype)
        full[:, :, :ctxs[b]] = kv
        seqs_o.append(oracle.SeqState(full, ctxs[b], list(tokens[b]), want[b]))
    sb = make_step(model, pool, [SeqSpec(c, list(t), wl) for c, t, wl in zip(ctxs, tokens, want)], rows, g0=g0)
    run_step(model, sb)
    torch.cuda.synchronize()
    ref = oracle_step(dims, w_cpu, seqs_o)
    return sb, ref, seqs_o, pool, rows


def check_case(dims, sb, ref, seqs_o, pool, rows, ctxs, rows_per_seq):
    tol = TOL[dims.dtype]
    M = sum(rows_per_seq)
    am = sb.argmax[:M].cpu().tolist()
    gap = sb.gap[:M].cpu()
    lrows = [r for r in range(M) if ref.logits[r] is not None]
    gpu_logits = sb.logits[:len(lrows)].cpu() if lrows else []
    check_rows([gpu_logits[j] for j in range(len(lrows))], [ref.logits[r] for r in lrows], tol, "logits")
    ties = TieLog()
    for j, r in enumerate(lrows):
        ties.check(am[r], ref.argmax[r], ref.logits[r], ref.gap[r], f"row {r}", ref.alt[r])
        if am[r] == ref.argmax[r]:
            assert abs(float(gap[r]) - ref.gap[r]) <= tol * max(1.0, float(ref.logits[r].abs().max())), \
                f"row {r} gap {float(gap[r])} vs {ref.gap[r]}"
    for r in range(M):
        if ref.logits[r] is None:
            assert am[r] == -1
    # the K/V rows this step wrote, read back through the block tables
    for b in range(len(ctxs)):
        got = pool.read(rows[b], ctxs[b], ctxs[b] + rows_per_seq[b]).double()
        want = seqs_o[b].kv[:, :, ctxs[b]:ctxs[b] + rows_per_seq[b]].double()
        if dims.kv_elem_bytes == 1:
            check_kv8(pool.read(rows[b], ctxs[b], ctxs[b] + rows_per_seq[b]),
                      seqs_o[b].kv[:, :, ctxs[b]:ctxs[b] + rows_per_seq[b]], f"kv seq {b}")
        else:
            for l in range(dims.n_layers):
                for t in range(2):
                    for i in range(rows_per_seq[b]):
                        check_rows([got[l, t, i]], [want[l, t, i]], tol, f"kv seq {b} layer {l} {'KV'[t]} row {i}")
        # the cached prefix is untouched
        byte = (lambda t: t.view(torch.uint8)) if dims.kv_elem_bytes == 1 else (lambda t: t)
        assert torch.equal(byte(pool.read(rows[b], 0, ctxs[b])), byte(seqs_o[b].kv[:, :, :ctxs[b]]))
    _say(ties.report())
    return ties


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_tiny_decode_four_sequences(dtype):
    """The tiny workload: B=4, contexts 5, 17, 33, 64, one query token each."""
    _say(f"tiny decode dtype={dtype}")
    dims = W.TINY.with_dtype(dtype)
    ctxs, k = [5, 17, 33, 64], [1, 1, 1, 1]
    sb, ref, so, pool, rows = run_case(dims, ctxs, k)
    check_case(dims, sb, ref, so, pool, rows, ctxs, k)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_tiny_verify_five_rows_random_gains(dtype):
    """K=5 causal rows per sequence (a verify pass) with non-unit norm gains, fused acceptance."""
    _say(f"tiny verify K=5 dtype={dtype}")
    dims = W.TINY.with_dtype(dtype)
    ctxs, k = [0, 15, 16, 47], [5, 5, 5, 5]
    g0 = [7, 8, 9, 10]
    sb, ref, so, pool, rows = run_case(dims, ctxs, k, gains="random", g0=g0)
    check_case(dims, sb, ref, so, pool, rows, ctxs, k)
    acc = sb.accept_len.cpu().tolist()
    bon = sb.bonus.cpu().tolist()
    am = sb.argmax.cpu().tolist()
    toks = sb.tokens.cpu().tolist()
    for b in range(4):
        n, bonus = oracle.accept_greedy(toks[5 * b:5 * b + 5], g0[b], am[5 * b:5 * b + 5])
        assert (acc[b], bon[b]) == (n, bonus)


def test_tiny_verify_accepts_oracle_greedy_drafts():
    """Drafts equal to the oracle's own greedy continuation are accepted in full."""
    _say("tiny verify with oracle-greedy drafts")
    dims = W.TINY.with_dtype("f32")
    ctx = 20
    # oracle greedy continuation: g0 from a one-row step, then g1..g4 by feeding the greedy tokens
    w_cpu = W.make_weights(dims, SEED_W)
    kv = W.kv_block(dims, SEED_KV, 0, 0, ctx)
    full = torch.zeros(1, 2, ctx + 6, 4, 64, dtype=torch.float32)
    full[:, :, :ctx] = kv
    st = oracle.SeqState(full, ctx - 1, [int(W.token_ids(SEED_TOK, 5, 1, 1000)[0])])
    full[:, :, ctx - 1] = 0  # position ctx-1 is recomputed by the step below
    g = [oracle.decode_step(dims, w_cpu, [st]).argmax[0]]
    st.ctx, st.tokens = ctx, [g[0]]
    for _ in range(4):
        g.append(oracle.decode_step(dims, w_cpu, [st]).argmax[0])
        st.ctx += 1
        st.tokens = [g[-1]]
    # the GPU sees positions 0..ctx-1 as cached (the oracle's own K/V) and verifies drafts g0..g4
    model = GpuModel(dims, weights_cpu=w_cpu)
    pool = GpuPool(dims, 16)
    rows = alloc_rows(pool, [ctx + 5])
    pool.write(rows[0], 0, full[:, :, :ctx])
    sb = make_step(model, pool, [SeqSpec(ctx, g[:5])], rows, g0=[g[0]])
    run_step(model, sb)
    torch.cuda.synchronize()
    assert int(sb.accept_len[0]) == 5
    assert sb.argmax[:4].cpu().tolist() == g[1:5]


def test_tiny_grouped_kv_heads():
    """4 query heads over 2 KV heads: each KV page block serves two query heads."""
    _say("tiny GQA 4/2")
    dims = W.ModelDims("tiny-gqa", 256, 4, 2, 64, 1024, 1000, 1, "f16")
    ctxs, k = [3, 40], [2, 3]
    sb, ref, so, pool, rows = run_case(dims, ctxs, k, gains="random")
    check_case(dims, sb, ref, so, pool, rows, ctxs, k)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n_kv,rows", [(4, [1, 1, 1]), (2, [1, 1]), (2, [2, 3, 1]), (2, [5, 5]), (1, [1, 1, 1]),
                                       (1, [2, 1]), (4, [2, 1])])
def test_tiny_grouped_heads_share_kv_loads(dtype, n_kv, rows):
    """8 query heads over 4, 2 or 1 K/V heads: a workgroup takes 2 or 4 query heads of one K/V head
    (up to 4 (row, head) states) for decode and short verify passes; five-row passes keep plain row
    groups."""
    _say(f"tiny GQA 8/{n_kv} rows={rows} dtype={dtype}")
    dims = W.ModelDims(f"tiny-gqa-8x{n_kv}", 512, 8, n_kv, 64, 1024, 1000, 1, dtype)
    ctxs = [37, 0, 70][:len(rows)]
    sb, ref, so, pool, rows_ = run_case(dims, ctxs, rows, gains="random")
    check_case(dims, sb, ref, so, pool, rows_, ctxs, rows)


def test_tiny_grouped_heads_head_dim_128_long_context():
    """Head dim 128, 8 query heads over 1 K/V head, 2 layers, a 900-token context (many pages and
    key splits) and a 3-row pass."""
    _say("tiny GQA 8/1 head_dim 128, 2 layers, ctx 900")
    dims = W.ModelDims("tiny-gqa-8x1-dh128", 1024, 8, 1, 128, 1024, 1000, 2, "bf16")
    ctxs, k = [900, 33], [3, 1]
    sb, ref, so, pool, rows = run_case(dims, ctxs, k, gains="random", pool_pages=128)
    check_case(dims, sb, ref, so, pool, rows, ctxs, k)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("heads,kv_heads,rows", [(2, 2, [1, 1, 1, 1]), (2, 2, [5, 3]), (8, 2, [1, 2])])
def test_tiny_fp8_cache(fmt, dtype, heads, kv_heads, rows):
    """An 8-bit K/V cache ([KV Cache] section 03): the step writes K/V as e4m3 / e5m2 and attention
    reads them back, for decode, verify and grouped heads (head_dim 128)."""
    _say(f"tiny fp8 cache {fmt} dtype={dtype} heads {heads}/{kv_heads} rows={rows}")
    dims = W.ModelDims(f"tiny-dh128-{heads}x{kv_heads}", heads * 128, heads, kv_heads, 128, 1024, 1000, 1,
                       dtype).with_kv(fmt)
    ctxs = [45, 3, 16, 100][:len(rows)]
    sb, ref, so, pool, rows_ = run_case(dims, ctxs, rows, gains="random")
    check_case(dims, sb, ref, so, pool, rows_, ctxs, rows)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiny_prefix_cache_hit_skips_the_shared_prefill(dtype):
    """[KV Cache] section 05 "Prefix caching": request A prefills 40 tokens and indexes its two full
    blocks; request B, equal to A for its first 32 tokens, finds both, takes those pages and runs
    only its last 7 tokens. B's logits and every K/V row of its cache match the oracle running B
    from scratch, its 32-token prefix included."""
    _say(f"tiny prefix cache hit, dtype={dtype}")
    dims = W.TINY.with_dtype(dtype)
    w_cpu = W.make_weights(dims, SEED_W, gains="random")
    model = GpuModel(dims, weights_cpu=w_cpu)
    pool = GpuPool(dims, 16)
    root = vs.kv_prefix_root(f"tiny;{dtype};weights={SEED_W};theta=10000".encode())
    a = W.token_ids(SEED_TOK, 600, 40, dims.vocab)
    b = a[:32] + W.token_ids(SEED_TOK, 601, 7, dims.vocab)
    ra = vs.kv_append(pool.handle, [], 4, 0, 40)
    run_step(model, make_step(model, pool, [SeqSpec(0, a, want_logits=False)], [ra], max_blocks=4))
    torch.cuda.synchronize()
    ha = vs.kv_prefix_chain(root, a, 16)
    assert len(ha) == 2 and vs.kv_prefix_insert(pool.handle, root, ha, a[:32], ra[:2]) == 2
    hb = vs.kv_prefix_chain(root, b, 16)
    assert hb == ha, "the first 32 tokens are equal, so are the names of the two full blocks"
    hit = vs.kv_prefix_lookup(pool.handle, root, hb, b[:32])
    assert hit == ra[:2] and vs.kv_refcount(pool.handle, ra[0]) == 3  # A, the index, B
    rb = vs.kv_append(pool.handle, hit, 4, 32, 7)
    sb = make_step(model, pool, [SeqSpec(32, b[32:])], [rb], max_blocks=4)
    run_step(model, sb)
    torch.cuda.synchronize()
    st = oracle.SeqState(torch.zeros(1, 2, 39, dims.n_kv_heads, dims.head_dim, dtype=dims.kv_torch_dtype), 0, list(b))
    ref = oracle_step(dims, w_cpu, [st])
    tol = TOL[dtype]
    check_rows([sb.logits[i].cpu() for i in range(7)], ref.logits[32:39], tol, "B's logits")
    am = sb.argmax[:7].cpu().tolist()
    ties = TieLog()
    for i in range(7):
        ties.check(am[i], ref.argmax[32 + i], ref.logits[32 + i], ref.gap[32 + i], f"B row {i}", ref.alt[32 + i])
    _say(ties.report())
    got, want = pool.read(rb, 0, 39).double(), st.kv.double()
    check_rows([got[0, t, i] for t in range(2) for i in range(39)], [want[0, t, i] for t in range(2) for i in range(39)],
               tol, "B's K/V (prefix written by A's step)")
    pool.close()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("heads,kv_heads,rows,ctxs", [(2, 2, [5, 16, 20], [100, 0, 37]),
                                                     (8, 2, [1, 5, 2], [300, 17, 0]),
                                                     (8, 1, [3, 1], [64, 250])])
def test_tiny_matrix_core_attention(dtype, heads, kv_heads, rows, ctxs):
    """Head dim 128 with several rows per sequence or grouped heads: attention runs on the matrix
    cores, 16 (row, head) states per workgroup; 20 rows need two row groups, contexts span pages
    and key splits, and a sequence with no cached context attends only within its rows."""
    _say(f"tiny MFMA attention {heads}/{kv_heads} rows={rows} ctxs={ctxs} dtype={dtype}")
    dims = W.ModelDims(f"tiny-dh128-{heads}x{kv_heads}", heads * 128, heads, kv_heads, 128, 1024, 1000, 1, dtype)
    sb, ref, so, pool, rows_ = run_case(dims, ctxs, rows, gains="random")
    check_case(dims, sb, ref, so, pool, rows_, ctxs, rows)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_tiny_prompt_chunk_of_more_than_64_rows(dtype):
    """A 100-row prompt chunk from position 0 beside a decode row and a 5-row verify pass (M = 106):
    steps of more than 64 rows run their products, LM head included, on the LDS-tiled MFMA GEMM."""
    _say(f"tiny 106-row step dtype={dtype}")
    dims = W.TINY.with_dtype(dtype)
    ctxs, k = [0, 30, 7], [100, 1, 5]
    sb, ref, so, pool, rows = run_case(dims, ctxs, k, gains="random")
    check_case(dims, sb, ref, so, pool, rows, ctxs, k)


def test_tiny_rows_without_logits_and_long_context():
    """A long sequence spanning many splits, one sequence without logits, head_dim 128."""
    _say("tiny head_dim 128, long context, no-logit sequence")
    dims = W.ModelDims("tiny-d256-2x128", 256, 2, 2, 128, 512, 1000, 2, "bf16")
    ctxs, k = [1000, 7, 300], [1, 4, 2]
    sb, ref, so, pool, rows = run_case(dims, ctxs, k, want=[True, False, True], pool_pages=128)
    check_case(dims, sb, ref, so, pool, rows, ctxs, k)


@pytest.mark.parametrize("want_any", [True, False])
def test_tiny_edge_cases(want_any):
    """First token of a sequence (no cache), a sequence with no rows this step, a row on the last slot of a
    page, nine rows in one sequence (more than one row group of the attention kernel), and a step without
    any logit row."""
    _say(f"tiny edge cases, logits={want_any}")
    dims = W.TINY.with_dtype("f16")
    ctxs, k = [0, 16, 15, 30, 3], [1, 0, 1, 9, 2]
    want = [want_any, want_any, want_any, want_any, False]
    sb, ref, so, pool, rows = run_case(dims, ctxs, k, gains="random", want=want)
    check_case(dims, sb, ref, so, pool, rows, ctxs, k)


def test_tiny_paged_equals_contiguous_bitwise():
    """The same logical K/V behind two different block tables (ascending pages, shuffled pages) gives
    bit-identical outputs: the page indirection changes addresses only."""
    _say("tiny paged == contiguous")
    dims = W.TINY.with_dtype("f16")
    w_cpu = W.make_weights(dims, SEED_W, gains="random")
    model = GpuModel(dims, weights_cpu=w_cpu)
    ctxs, k = [40, 100, 7], [1, 3, 2]
    outs = []
    for shuffle in (None, synth.key(SEED_PAGES, 9)):
        pool = GpuPool(dims, 64)
        rows = alloc_rows(pool, [c + n for c, n in zip(ctxs, k)], shuffle_key=shuffle)
        if shuffle is None:
            flat = [p for r in rows for p in r]
            assert flat == sorted(flat)
        for b in range(3):
            pool.write(rows[b], 0, W.kv_block(dims, SEED_KV, b, 0, ctxs[b]))
        toks = [W.token_ids(SEED_TOK, 300 + b, k[b], dims.vocab) for b in range(3)]
        sb = make_step(model, pool, [SeqSpec(c, t) for c, t in zip(ctxs, toks)], rows)
        run_step(model, sb)
        torch.cuda.synchronize()
        kv_new = [pool.read(rows[b], ctxs[b], ctxs[b] + k[b]) for b in range(3)]
        outs.append((sb.logits.cpu(), sb.argmax.cpu(), sb.gap.cpu(), kv_new))
        pool.close()
    a, b = outs
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    assert all(torch.equal(x, y) for x, y in zip(a[3], b[3]))


def test_tiny_copy_on_append_of_a_shared_partial_page():
    """Two sequences share a 1000-token prefix (62.5 pages). The first to append gets a private copy of the
    half-filled last page (one page copy enqueued by kv_append); the second then owns the original alone
    and appends in place. Both steps match the oracle run on contiguous caches."""
    _say("tiny copy-on-append")
    dims = W.TINY.with_dtype("f16")
    w_cpu = W.make_weights(dims, SEED_W)
    model = GpuModel(dims, weights_cpu=w_cpu)
    pool = GpuPool(dims, 160)
    ctx = 1000
    pre = vs.kv_alloc(pool.handle, -(-ctx // 16))
    kv = W.kv_block(dims, SEED_KV, 0, 0, ctx)
    pool.write(pre, 0, kv)
    vs.kv_share(pool.handle, pre)
    last = pre[-1]
    assert vs.kv_refcount(pool.handle, last) == 2
    max_blocks = -(-(ctx + 1) // 16)
    free0 = vs.kv_num_free(pool.handle)
    r0 = vs.kv_append(pool.handle, pre, max_blocks, ctx, 1, torch.cuda.current_stream().cuda_stream)
    assert r0[:-1] == pre[:-1] and r0[-1] != last
    assert vs.kv_refcount(pool.handle, last) == 1 and vs.kv_refcount(pool.handle, r0[-1]) == 1
    assert vs.kv_num_free(pool.handle) == free0 - 1
    r1 = vs.kv_append(pool.handle, pre, max_blocks, ctx, 1, torch.cuda.current_stream().cuda_stream)
    assert r1 == pre, "the last holder of a page writes into it without a copy"
    assert vs.kv_num_free(pool.handle) == free0 - 1
    torch.cuda.synchronize()
    # the copy holds the filled slots of the shared page
    assert torch.equal(pool.view()[r0[-1], :, :, :, :ctx % 16], pool.view()[last, :, :, :, :ctx % 16])
    toks = [W.token_ids(SEED_TOK, 400 + b, 1, dims.vocab) for b in range(2)]
    sb = make_step(model, pool, [SeqSpec(ctx, toks[0]), SeqSpec(ctx, toks[1])], [r0, r1])
    run_step(model, sb)
    torch.cuda.synchronize()
    seqs_o = []
    for b in range(2):
        full = torch.zeros(dims.n_layers, 2, ctx + 1, dims.n_kv_heads, dims.head_dim, dtype=dims.torch_dtype)
        full[:, :, :ctx] = kv
        seqs_o.append(oracle.SeqState(full, ctx, list(toks[b])))
    ref = oracle_step(dims, w_cpu, seqs_o)
    check_case(dims, sb, ref, seqs_o, pool, [r0, r1], [ctx, ctx], [1, 1])
    pool.close()


def test_verify_accept_entry_point_against_the_rule():
    """verify_accept on device arrays, every sequence length 0..5 and tokens from {0, 1, 2} so that matches
    are frequent; compared with the acceptance rule of the oracle, exactly."""
    _say("verify_accept entry point")
    gen = torch.Generator().manual_seed(1007)
    B = 257
    K = torch.randint(0, 6, (B,), generator=gen)
    q_start = torch.zeros(B + 1, dtype=torch.int32)
    q_start[1:] = torch.cumsum(K, 0)
    M = int(q_start[-1])
    drafts = torch.randint(0, 3, (M,), generator=gen, dtype=torch.int32)
    argmax = torch.randint(0, 3, (M,), generator=gen, dtype=torch.int32)
    g0 = torch.randint(0, 3, (B,), generator=gen, dtype=torch.int32)
    dev = [t.cuda() for t in (q_start, drafts, g0, argmax)]
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    bon = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    vs.verify_accept(B, *dev, acc, bon, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    acc, bon = acc.cpu().tolist(), bon.cpu().tolist()
    for b in range(B):
        s, e = int(q_start[b]), int(q_start[b + 1])
        want = oracle.accept_greedy(drafts[s:e].tolist(), int(g0[b]), argmax[s:e].tolist())
        assert (acc[b], bon[b]) == want, (b, drafts[s:e].tolist(), int(g0[b]), argmax[s:e].tolist())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiny_long_mlp_rows_stage_in_phases(dtype):
    """An MLP 8192 wide with 4 rows: the down product's input rows (4 x 8192 values) exceed the
    GEMV's LDS budget and are staged in phases, one unit per wave."""
    _say(f"tiny phased down product {dtype}")
    dims = W.ModelDims("tiny-ffn8192", 256, 4, 4, 64, 8192, 1000, 1, dtype)
    ctxs, k = [9, 40], [2, 2]
    sb, ref, so, pool, rows = run_case(dims, ctxs, k, gains="random")
    check_case(dims, sb, ref, so, pool, rows, ctxs, k)


def test_tiny_many_key_splits_use_the_merge_kernel():
    """Few heads and a 3000-token context: more key splits than the output GEMV's prologue merges
    (eight), so the row-streaming path falls back to the standalone merge kernel."""
    _say("tiny 3000-token context, many splits")
    dims = W.TINY.with_dtype("f16")
    ctxs, k = [3000], [1]
    sb, ref, so, pool, rows = run_case(dims, ctxs, k, pool_pages=200)
    check_case(dims, sb, ref, so, pool, rows, ctxs, k)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_tiny_validation_word_flags_bad_inputs(dtype):
    """With desc->error_flags set, the step reports out-of-range inputs instead of only clamping them:
    a token id outside [0, vocab), a block-table entry outside [0, num_pages) among the pages a row
    reads, a negative context length. Valid inputs leave the word at zero; every step completes."""
    _say(f"tiny validation word dtype={dtype}")
    dims = W.TINY.with_dtype(dtype)
    model = GpuModel(dims, weights_cpu=W.make_weights(dims, SEED_W))
    pool = GpuPool(dims, 16)
    rows = alloc_rows(pool, [20, 9])
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step(tokens, bt_patch=None, ctx=(19, 8), ctx_patch=None):
        sb = make_step(model, pool, [SeqSpec(ctx[0], [tokens[0]]), SeqSpec(ctx[1], [tokens[1]])], rows, max_blocks=4)
        if bt_patch is not None:
            sb.block_tables[bt_patch[0], bt_patch[1]] = bt_patch[2]
        if ctx_patch is not None:  # a context length the caller got wrong (the step treats it as 0)
            sb.ctx_len[ctx_patch[0]] = ctx_patch[1]
        flags.zero_()
        sb.desc.error_flags = flags.data_ptr()
        run_step(model, sb)
        torch.cuda.synchronize()
        assert all(0 <= a < dims.vocab for a in sb.argmax[:2].cpu().tolist())
        return int(flags.item())

    assert step([3, 4]) == 0
    assert step([dims.vocab + 5, 4]) == vs.VS_STEP_BAD_TOKEN
    assert step([3, -1]) == vs.VS_STEP_BAD_TOKEN
    assert step([3, 4], bt_patch=(0, 1, pool.num_pages + 3)) == vs.VS_STEP_BAD_PAGE  # row 0 reads page 1
    assert step([3, 4], bt_patch=(1, 2, pool.num_pages + 3)) == 0  # past row 1's pages: never read
    assert step([dims.vocab, 4], bt_patch=(1, 0, -2)) == vs.VS_STEP_BAD_TOKEN | vs.VS_STEP_BAD_PAGE
    assert step([3, 4], ctx_patch=(1, -3)) == vs.VS_STEP_BAD_BATCH
    pool.close()
