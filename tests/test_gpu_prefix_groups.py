"""GPU parity of shared-prefix groups: one-row sequences whose block tables start with the same pages.

[KV Cache] section 05, prefix caching: a prefix's pages are stored once and every sequence that starts
with it holds them in its block table. The step may be told which sequences share which prefix pages
(the batch's prefix groups); attention then reads each group's prefix pages once for all of its
sequences, in the key splits before the sequences' own pages, and merges the two parts as it merges any
key splits ([KV Cache] section 07). The result is the same attention as without groups: every case runs
the step with and without the groups and checks both against the oracle (logits, greedy tokens, the K/V
rows written).

Tiny models with head_dim 128 (the grouped path's shape), fp16 and bf16, plain and grouped K/V heads,
16-bit and 8-bit caches.
A group may span several of the matrix-core kernel's group blocks (16 / HG sequences each), a group
member may fail the check (a block table that differs in the prefix, or two rows), and then it is
attended like any other sequence, with VS_STEP_BAD_BATCH in the validation word.
"""
import pytest
import torch

import oracle
import synth
import verify_step_amd as vs
from harness import GpuModel, GpuPool, SeqSpec, make_step, run_step
from synth import workloads as W
from test_gpu_tiny import SEED_KV, SEED_PAGES, SEED_TOK, SEED_W, check_case, oracle_step

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def run_groups(dims, prefixes, members, groups, flags, pool_pages=256, break_member=None):
    """prefixes: prefix lengths (multiples of 16); members: (prefix index or None, suffix length, rows) per
    sequence; sequences of one prefix share its pages. Runs the step with the given groups and without
    any, each with a cleared validation word; returns both, the oracle's step and what check_case takes."""
    w_cpu = W.make_weights(dims, SEED_W, gains="random")
    model = GpuModel(dims, weights_cpu=w_cpu)
    pool = GpuPool(dims, pool_pages)
    ids = vs.kv_alloc(pool.handle, pool_pages)
    perm = synth.permutation(synth.key(SEED_PAGES), pool_pages)
    vs.kv_free(pool.handle, [ids[int(i)] for i in perm])
    max_ctx = max((prefixes[p] if p is not None else 0) + s + k for p, s, k in members)
    max_blocks = -(-max_ctx // 16) + 1
    pre_rows, pre_kv = [], []
    for i, n in enumerate(prefixes):
        r = vs.kv_alloc(pool.handle, n // 16)
        kv = W.kv_block(dims, SEED_KV, 50 + i, 0, n)
        pool.write(r, 0, kv)
        pre_rows.append(r)
        pre_kv.append(kv)
    specs, rows, seqs_o = [], [], []
    for b, (p, suf, k) in enumerate(members):
        n0 = prefixes[p] if p is not None else 0
        ctx = n0 + suf
        if p is not None:
            vs.kv_share(pool.handle, pre_rows[p])
            r = vs.kv_append(pool.handle, pre_rows[p], max_blocks, n0, suf + k)
        else:
            r = vs.kv_append(pool.handle, [], max_blocks, 0, ctx + k)
        if b == break_member:  # this sequence's first prefix page is a private copy: same values, another page
            own = vs.kv_alloc(pool.handle, 1)[0]
            r = [own] + r[1:]
            pool.write([own], 0, pre_kv[p][:, :, :16])
        kv = torch.zeros(dims.n_layers, 2, ctx + k, dims.n_kv_heads, dims.head_dim, dtype=dims.kv_torch_dtype)
        if p is not None:
            kv[:, :, :n0] = pre_kv[p]
        if ctx > n0:
            skv = W.kv_block(dims, SEED_KV, 100 + b, n0, ctx)
            pool.write(r, n0, skv)
            kv[:, :, n0:ctx] = skv
        tok = W.token_ids(SEED_TOK, 300 + b, k, dims.vocab)
        specs.append(SeqSpec(ctx, list(tok)))
        rows.append(r)
        seqs_o.append(oracle.SeqState(kv, ctx, list(tok)))
    ctxs = [s.ctx for s in specs]
    ks = [len(s.tokens) for s in specs]
    out = {}
    for label, g in (("groups", groups), ("no groups", None)):
        _say(f"  step with {label}")
        sb = make_step(model, pool, specs, rows, max_blocks=max_blocks, groups=g)
        flags.zero_()
        sb.desc.error_flags = flags.data_ptr()
        run_step(model, sb)
        torch.cuda.synchronize()
        out[label] = (sb, int(flags.item()))
    ref = oracle_step(dims, w_cpu, seqs_o)
    run_groups.model = model  # for a caller that runs the step again
    return out, ref, seqs_o, pool, rows, ctxs, ks


CASES = {
    # name: (heads, kv heads, prefixes, members (prefix, suffix, rows), groups (first seq, n, pages))
    # two prefixes; one group of 18 sequences (two group blocks of 16 for HG = 1), one of 3; a loose
    # decode sequence and a 3-row verify pass beside them (the matrix cores take the pass)
    "mha": (2, 2, [48, 160],
            [(0, s, 1) for s in [0, 5, 16, 33, 70, 1, 2, 3, 4, 6, 7, 8, 9, 10, 11, 12, 13, 15]] +
            [(1, 3, 1), (1, 40, 1), (1, 17, 1), (None, 100, 1), (None, 37, 3)],
            [(0, 18, 3), (18, 3, 10)]),
    # 8 query heads over 2 K/V heads: HG = 4, four sequences per group block; one-row sequences only
    "gqa": (8, 2, [64, 32], [(0, s, 1) for s in [0, 9, 30, 61, 2]] + [(1, 5, 1), (1, 0, 1), (None, 70, 1)],
            [(0, 5, 4), (5, 2, 2)]),
    # a group whose prefix is only part of the shared pages (2 of the 3 shared pages)
    "partial": (2, 2, [48], [(0, s, 1) for s in [3, 20, 90]] + [(None, 10, 2)], [(0, 3, 2)]),
    # one-row sequences and plain heads: the VALU kernel takes every sequence's own pages, the group
    # blocks run as a launch of their own
    "mha-decode": (2, 2, [80], [(0, s, 1) for s in [0, 7, 44, 130, 16, 3]] + [(None, 60, 1)], [(0, 6, 5)]),
    # one group on a 640-token prefix (40 pages): the group blocks cut it into several prefix splits
    "long-prefix": (2, 2, [640], [(0, s, 1) for s in [3, 50, 17, 0]] + [(None, 30, 1)], [(0, 4, 40)]),
    # three one-row sequences (the row-streaming GEMV path): the merge kernel combines the grouped rows'
    # splits, where without groups the output product's prologue would
    "gemv": (2, 2, [64], [(0, s, 1) for s in [5, 20, 1]], [(0, 3, 4)]),
    # a 70-row prompt chunk from position 0 beside 12 grouped decode rows: the matrix-core kernel's plain
    # blocks go by its work list (5 row groups of the chunk) instead of 13 sequences x 5 row-group blocks
    "chunk": (2, 2, [32], [(0, s, 1) for s in [0, 3, 9, 17, 30, 1, 2, 4, 5, 6, 7, 8]] + [(None, 0, 70)],
              [(0, 12, 2)]),
}


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("case", list(CASES))
def test_prefix_groups_match_the_oracle(dtype, case):
    heads, kvh, prefixes, members, groups = CASES[case]
    _say(f"prefix groups {case} dtype={dtype}")
    dims = W.ModelDims(f"tiny-dh128-{heads}x{kvh}-2L", heads * 128, heads, kvh, 128, 512, 1000, 2, dtype)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, ref, seqs_o, pool, rows, ctxs, ks = run_groups(dims, prefixes, members, groups, flags)
    for label, (sb, fl) in out.items():
        _say(f"  checking the step with {label}")
        assert fl == 0, f"{label}: validation word {fl}"
        check_case(dims, sb, ref, seqs_o, pool, rows, ctxs, ks)
    pool.close()


@pytest.mark.parametrize("fmt,dtype,case", [("e4m3", "f16", "mha"), ("e5m2", "bf16", "gqa"), ("e4m3", "bf16", "chunk")])
def test_prefix_groups_with_an_8bit_cache(fmt, dtype, case):
    """The same groups over an 8-bit K/V cache ([KV Cache] section 03): the group blocks widen the shared
    prefix pages exactly as the other attention kernels widen their own. One layer, as the other 8-bit
    cache tests: the K/V rows a step writes are then a rounding of the embedding's projections, which the
    check holds to one value of the format (past the first layer they also carry the attention's rounding,
    and an e5m2 element near zero can move by more than one of its steps)."""
    heads, kvh, prefixes, members, groups = CASES[case]
    _say(f"prefix groups {case} dtype={dtype} cache={fmt}")
    dims = W.ModelDims(f"tiny-dh128-{heads}x{kvh}-1L", heads * 128, heads, kvh, 128, 512, 1000, 1, dtype).with_kv(fmt)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, ref, seqs_o, pool, rows, ctxs, ks = run_groups(dims, prefixes, members, groups, flags)
    for label, (sb, fl) in out.items():
        _say(f"  checking the step with {label}")
        assert fl == 0, f"{label}: validation word {fl}"
        check_case(dims, sb, ref, seqs_o, pool, rows, ctxs, ks)
    pool.close()


@pytest.mark.parametrize("bad", ["table", "two rows", "too many pages"])
def test_prefix_group_member_failing_the_check_is_attended_alone(bad):
    """A member whose block table holds another page among the prefix pages (same values), one that brings
    two rows, or a group that claims more pages than its sequences share (the fourth page is each one's
    own, and the first sequence's context does not cover it): the step sets VS_STEP_BAD_BATCH and attends
    such a sequence over its own table, so every result still matches the oracle."""
    _say(f"prefix group member failing the check: {bad}")
    dims = W.ModelDims("tiny-dh128-2x2-2L", 256, 2, 2, 128, 512, 1000, 2, "f16")
    members = [(0, s, 1) for s in [4, 30, 17, 2]] + [(None, 25, 1)]
    groups, brk = [(0, 4, 3)], None
    if bad == "table":
        brk = 2
    elif bad == "two rows":
        members[1] = (0, 30, 2)
    else:
        groups = [(0, 4, 4)]
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, ref, seqs_o, pool, rows, ctxs, ks = run_groups(dims, [48], members, groups, flags, break_member=brk)
    sb, fl = out["groups"]
    assert fl == vs.VS_STEP_BAD_BATCH, f"validation word {fl}"
    check_case(dims, sb, ref, seqs_o, pool, rows, ctxs, ks)
    assert out["no groups"][1] == 0
    check_case(dims, out["no groups"][0], ref, seqs_o, pool, rows, ctxs, ks)
    pool.close()


def test_prefix_groups_graph_replays_match_the_eager_step():
    """The "chunk" case (fp16) captured in a HIP graph after an eager step: the attention of the one-row
    sequences and the matrix-core kernel run on two streams (forked from and joined back into the captured
    one), so the graph holds both branches. Three replays, with other work and a synchronisation between
    them, each give the eager step's logits and greedy tokens bit for bit."""
    _say("prefix groups under graph capture")
    heads, kvh, prefixes, members, groups = CASES["chunk"]
    dims = W.ModelDims(f"tiny-dh128-{heads}x{kvh}-2L", heads * 128, heads, kvh, 128, 512, 1000, 2, "f16")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, ref, seqs_o, pool, rows, ctxs, ks = run_groups(dims, prefixes, members, groups, flags)
    model = run_groups.model
    sb = out["groups"][0]
    check_case(dims, sb, ref, seqs_o, pool, rows, ctxs, ks)
    n_log = int(sb.desc.M_log)
    logits0, am0 = sb.logits[:n_log].clone(), sb.argmax.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_step(model, sb)  # eager once more on the capture's stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(sb.logits[:n_log], logits0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_step(model, sb)
    torch.cuda.synchronize()
    for i in range(3):
        _say(f"  replay {i}")
        sb.logits.fill_(float("nan"))
        sb.argmax.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(sb.logits[:n_log], logits0), f"replay {i}: logits differ from the eager step"
        assert torch.equal(sb.argmax, am0), f"replay {i}: greedy tokens differ"
        junk = torch.randn(1 << 20, device="cuda")  # other work between the replays
        float(junk.square().sum())
    pool.close()


def test_prefix_groups_one_stream_equals_two_streams():
    """decode_step runs the matrix-core kernel and the VALU kernel of a step with groups on two streams;
    decode_step_noalloc keeps every kernel on the caller's stream, one after the other. Same kernels, same
    key splits, so the "chunk" case (fp16) gives the same logits, greedy tokens, gaps and K/V rows bit for
    bit either way."""
    _say("prefix groups: one stream (decode_step_noalloc) against two (decode_step)")
    heads, kvh, prefixes, members, groups = CASES["chunk"]
    dims = W.ModelDims(f"tiny-dh128-{heads}x{kvh}-2L", heads * 128, heads, kvh, 128, 512, 1000, 2, "f16")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, ref, seqs_o, pool, rows, ctxs, ks = run_groups(dims, prefixes, members, groups, flags)
    model = run_groups.model
    sb = out["groups"][0]
    n_log, M = int(sb.desc.M_log), sum(ks)

    def outputs():
        kv = [pool.read(rows[b], ctxs[b], ctxs[b] + ks[b]) for b in range(len(ctxs))]
        return [sb.logits[:n_log].clone(), sb.argmax[:M].clone(), sb.gap[:M].clone()] + kv

    run_step(model, sb)
    torch.cuda.synchronize()
    want = outputs()
    sb.logits.fill_(float("nan"))
    sb.argmax.fill_(-7)
    sb.gap.fill_(float("nan"))
    for b in range(len(ctxs)):
        pool.write(rows[b], ctxs[b], torch.zeros(dims.n_layers, 2, ks[b], kvh, 128, dtype=dims.kv_torch_dtype))
    assert sb.ws_bytes <= vs.VS_NOALLOC_SCRATCH_BYTES
    vs.decode_step_noalloc(sb.desc, sb.block_tables, model.w, sb.out, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = outputs()
    for i, (a, c) in enumerate(zip(want, got)):
        if a.is_floating_point():
            same = torch.equal(a.contiguous().view(torch.uint8), c.contiguous().view(torch.uint8))
        else:
            same = torch.equal(a, c)
        assert same, f"output {i} differs between one and two streams"
    pool.close()
