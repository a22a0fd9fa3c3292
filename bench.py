"""Benchmark: 7B-shaped greedy decode at batch 1 on one MI355X.

Workload: 32 layers, d_model 4096, 32 heads x 128 (MHA), SwiGLU 11008,
vocab 32000, RMSNorm + RoPE, fp16 random-init weights N(0, 0.02) (13.2 GB
streamed per step), one sequence whose 2048-token synthetic context sits in
16-token pages scattered through the pool, K = 1, each step's input token is
the previous step's argmax. One "step" is one decode_step over the whole
path (embedding, 32 layers, LM head, argmax, which also feeds the next
step's token and advances the context length on the device) plus the host's
per-step page bookkeeping (kv_append).

Prints one JSON line. `value` is decode tokens/s over the timed steps;
`roofline` reports the gate/up product (the kernel that streams the most
weight bytes) against the 8 TB/s HBM peak, with its HBM traffic per launch
from the committed counter summary under profiles/ while that summary's
kernel-source digest matches; `cpu_baseline` times the CPU oracle on one
step of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s + achieved HBM TB/s vs peak, 7B-shaped, B=1..64, K=1/5"
HBM_PEAK_GBPS = 8000.0
CTX0 = 2048
ROOFLINE_STEPS = 8
GATEUP_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gateup_gemv_7b_decode_b1_hbm_traffic.md")
CSRC = os.path.join(ROOT, "verify_step_amd", "csrc")
SEED_W, SEED_KV, SEED_TOK, SEED_PAGES = 2001, 2002, 2003, 2006


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles through libamdhip64 (for the per-kernel timer)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.start = (ctypes.c_void_p * n)()
        self.stop = (ctypes.c_void_p * n)()
        for i in range(n):
            for arr in (self.start, self.stop):
                e = ctypes.c_void_p()
                assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
                arr[i] = e
        self.n = n

    def elapsed_ms(self, i, j=None):
        """Launch i's duration; with j, the time from launch i's start to launch j's end (events of one
        device compare across streams)."""
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.start[i], self.stop[i if j is None else j])
        assert rc == 0, rc
        return ms.value

    def start_ms(self, i, j):
        """The time from launch i's start to launch j's start."""
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.start[i], self.start[j])
        assert rc == 0, rc
        return ms.value

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(self.start[i])
            self.hip.hipEventDestroy(self.stop[i])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch every step eagerly instead of replaying a graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with plain device copies of known size (reference dispatches for HBM byte counters)")
    ap.add_argument("--workload", default="decode-b1",
                    choices=["decode-b1"] + sorted(OTHER_WORKLOADS) + sorted(SAMPLE_WORKLOADS),
                    help="decode-b1 is the headline line; the others measure the remaining step shapes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the step runs on one GPU's share of a batch, and --gpus {args.gpus} "
              "(several GPUs) is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import verify_step_amd as vs
    from harness import GpuModel, GpuPool, SeqSpec, make_step
    from synth import workloads as W
    from verify_step_amd import build as vsbuild

    if not os.path.exists(vs.LIB_PATH):
        vsbuild.build()
    vs.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.workload in SAMPLE_WORKLOADS:
        return sample_workload(args)
    if args.workload != "decode-b1":
        return other_workload(args)
    dev = torch.device("cuda:0")
    dims = W.LLAMA7B  # fp16
    K, Wm = args.steps, args.warmup
    total_len = CTX0 + Wm + K + len(TIMED_KINDS) * min(K, ROOFLINE_STEPS) + 1  # every position this run writes

    # ---- weights (generated on the host, one tensor at a time) ----
    t0 = time.time()
    keep_cpu = not args.no_cpu_baseline
    w_cpu = {"layers": [dict() for _ in range(dims.n_layers)]} if keep_cpu else None

    def items():
        for name, layer, t in W.iter_weights(dims, SEED_W):
            if keep_cpu:
                (w_cpu if layer < 0 else w_cpu["layers"][layer])[name] = t
            yield name, layer, t

    model = GpuModel.__new__(GpuModel)
    _load_model(model, dims, items(), dev)
    log(f"weights ready in {time.time() - t0:.1f}s")

    # ---- pool, scattered pages, synthetic 2048-token context ----
    n_pages = -(-total_len // 16) + 8
    pool = GpuPool(dims, n_pages)
    ids = vs.kv_alloc(pool.handle, n_pages)
    perm = synth.permutation(synth.key(SEED_PAGES), n_pages)
    vs.kv_free(pool.handle, [ids[int(i)] for i in perm])
    row = vs.kv_alloc(pool.handle, -(-CTX0 // 16))
    kv0 = W.kv_block(dims, SEED_KV, 0, 0, CTX0)
    pool.write(row, 0, kv0)
    tok0 = W.token_ids(SEED_TOK, 0, 1, dims.vocab)
    max_blocks = -(-total_len // 16)
    row = vs.kv_append(pool.handle, row, max_blocks, CTX0, 1)
    sb = make_step(model, pool, [SeqSpec(CTX0, tok0)], [row], max_blocks=max_blocks, want_logits_tensor=False)
    # the graph is built for the longest context the run reaches
    sb.desc.max_ctx = total_len
    sb.ws_bytes = vs.decode_step_workspace_bytes(sb.desc, __import__("harness").model_desc(dims))
    sb.ws = torch.empty(sb.ws_bytes, dtype=torch.uint8, device=dev)
    # a device-side greedy loop: each step reads its input token from the argmax array the previous
    # step wrote, and advances the context length itself
    sb.argmax[:1].copy_(sb.tokens[:1])
    sb.desc.tokens = sb.argmax.data_ptr()
    sb.desc.ctx_advance = sb.ctx_len.data_ptr()
    bt_host = torch.zeros(max_blocks, dtype=torch.int32).pin_memory()
    bt_host[:len(row)] = torch.tensor(row, dtype=torch.int32)
    sb.block_tables[0].copy_(bt_host)
    torch.cuda.synchronize()
    log(f"context ready: {CTX0} tokens in {len(row)} pages, pool {n_pages} pages")

    state = {"row": row, "len": CTX0}  # host view: positions [0, len) hold K/V after the step

    def device_step():
        vs.decode_step(sb.desc, sb.block_tables, model.w, sb.out, sb.ws, sb.ws_bytes,
                       torch.cuda.current_stream().cuda_stream)

    def host_bookkeeping():
        # the step about to run writes position len + 1's K/V next time; make room for it
        cur = state["len"] + 1
        r = vs.kv_append(pool.handle, state["row"], max_blocks, cur, 1)
        if len(r) != len(state["row"]):
            bt_host[len(r) - 1] = r[-1]
            sb.block_tables[0, len(r) - 1:len(r)].copy_(bt_host[len(r) - 1:len(r)], non_blocking=True)
        state["row"], state["len"] = r, cur

    graph = None
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            device_step()  # one eager step before capture (position 2048)
            host_bookkeeping()
        torch.cuda.current_stream().wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            device_step()
        Wm_left = Wm - 1
    else:
        Wm_left = Wm

    def one():
        if graph is not None:
            graph.replay()
        else:
            device_step()
        host_bookkeeping()

    for _ in range(Wm_left):
        one()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    tw0 = time.perf_counter()
    ev0.record()
    for _ in range(K):
        one()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - tw0
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / K
    log(f"timed {K} steps: {ms_step:.3f} ms/step (wall {wall * 1e3 / K:.3f} ms/step)")

    # ---- per-kernel times from dispatch events: every launch of each kernel kind in n_rf eager steps
    # after the timed window (a graph hides its nodes from events) ----
    n_rf = min(K, ROOFLINE_STEPS)

    def eager():
        device_step()
        host_bookkeeping()

    kt = kernel_times(vs, eager, n_rf, 4 * dims.n_layers)
    gu_launches = kt["gateup"]["launch_us"]
    gu_ms = sum(gu_launches) / len(gu_launches) / 1e3
    gu_bytes = 2 * dims.ffn * dims.d_model * dims.elem_bytes  # W_gate + W_up, read once per launch
    gu_gbps = gu_bytes / (gu_ms * 1e-3) / 1e9
    traffic = measured_traffic(GATEUP_TRAFFIC_PROFILE)
    n_done = len(gu_launches)

    # ---- byte accounting for the whole step ----
    wbytes = streamed_weight_bytes(dims)
    kvpt = 2 * dims.n_layers * dims.n_kv_heads * dims.head_dim * dims.elem_bytes  # K and V of one token
    first = CTX0 + Wm + 1  # keys read by the first timed step
    avg_keys = first + (K - 1) / 2.0
    step_bytes = wbytes + avg_keys * kvpt + kvpt
    result = {
        "metric": METRIC,
        "value": round(1000.0 / ms_step, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "7B-shaped greedy decode, B=1, K=1, fp16 weights+KV, context 2048 grown one token per step, "
                        "16-token pages scattered in the pool",
            "model_shape": dims.name,
            "batch": 1,
            "rows_per_seq": 1,
            "ctx_first_timed_step": first - 1,
            "graph_replay": graph is not None,
        },
        "hbm": {
            "weight_bytes_per_step": wbytes,
            "kv_bytes_per_step_avg": int(avg_keys * kvpt + kvpt),
            "step_TBps": round(step_bytes / (ms_step * 1e-3) / 1e12, 4),
            "step_frac_of_peak": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "wall_ms_per_step": round(wall * 1e3 / K, 4),
        },
        "roofline": {
            "kernel": "gate/up GEMV + SwiGLU (gemv_kernel, EPI_SWIGLU)",
            "bound": "hbm",
            "achieved": round(gu_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gu_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "bytes_per_launch": gu_bytes,
            "avg_launch_us": round(gu_ms * 1e3, 3),
            "launches_timed": n_done,
            "timing": f"dispatch events of every gate/up launch in {n_rf} eager steps after the timed window",
        },
        "weight_stream": weight_stream(dims, kt, n_rf),
        "attention": attention_stream(kt, n_rf, avg_keys * kvpt + kvpt),
    }

    result["stream_ceiling"] = stream_ceiling(vs)
    if args.copy_calibration:
        copy_calibration()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(dims, w_cpu, kv0, tok0)
    print(json.dumps(result), flush=True)


COPY_BYTES = 256 << 20
CEILING_BYTES = 4 << 30


def stream_ceiling(vs):
    """The device's streaming-read rate in the GEMV's load shape (vs_stream_read over 4 GiB, the best of
    20 timed reads after 3 warm-up reads), the practical reference for the weight stream."""
    import torch

    buf = torch.ones(CEILING_BYTES // 2, dtype=torch.float16, device="cuda")
    sink = torch.zeros(512, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        vs.vs_stream_read(buf, CEILING_BYTES, sink, stream)
    best = float("inf")
    for _ in range(20):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        vs.vs_stream_read(buf, CEILING_BYTES, sink, stream)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del buf
    gbps = CEILING_BYTES / (best * 1e-3) / 1e9
    return {"achieved": round(gbps, 1), "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "bytes": CEILING_BYTES, "kernel": "vs_stream_read (1 KB wave loads, nontemporal)"}


def copy_calibration():
    """Three elementwise copies (negation) of 256 MiB of fp32 each: every dispatch reads and writes exactly
    COPY_BYTES, the yardstick for scaling HBM byte counters."""
    import torch

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 x {COPY_BYTES} B read + written")


# ---------------------------------------------------------------- the other step shapes

OTHER_WORKLOADS = {
    # name: (dtype, batch, rows per sequence, context rule, prompt-chunk rows)
    "batch-bf16-b8": ("bf16", 8, 1, "uniform", 0),
    "batch-bf16-b32": ("bf16", 32, 1, "uniform", 0),
    "batch-bf16-b64": ("bf16", 64, 1, "uniform", 0),
    "verify-f16-b8k5": ("f16", 8, 5, "1024", 0),
    "mixed-f16-64+512": ("f16", 64, 1, "prefix", 512),
    # grouped K/V heads (32 query heads over 8 K/V heads, the widths of Llama 3.1 8B)
    "gqa8b-f16-b1": ("f16", 1, 1, "2048", 0),
    "gqa8b-f16-b8k5": ("f16", 8, 5, "1024", 0),
    "gqa8b-bf16-b64": ("bf16", 64, 1, "uniform", 0),
    # 8-bit K/V cache (a name ending in -e4m3 / -e5m2 sets the cache's format)
    "batch-bf16-b64-e4m3": ("bf16", 64, 1, "uniform", 0),
    "gqa8b-bf16-b64-e4m3": ("bf16", 64, 1, "uniform", 0),
    "verify-f16-b8k5-e4m3": ("f16", 8, 5, "1024", 0),
}


def other_workload(args):
    """One step of another shape, repeated: continuous batching of B sequences with contexts uniform in
    128..4096 (bf16), an 8 x 5 verify pass at context 1024, or 64 decode rows on shared 1024-token
    prefixes plus a 512-row prompt chunk; the gqa8b shapes run the grouped-K/V model (32 query heads
    over 8 K/V heads) at batch 1 (context 2048), 8 x 5 verify and batch 64. Every repetition rewrites
    the same K/V rows, so the work per step is fixed. K/V contents are arbitrary normals (timing does
    not depend on them)."""
    import torch

    import synth
    import verify_step_amd as vs
    from harness import GpuModel, GpuPool, SeqSpec, make_step
    from synth import workloads as W

    dt, B, K, ctx_rule, chunk = OTHER_WORKLOADS[args.workload]
    gqa = args.workload.startswith("gqa")
    kv8 = args.workload.rsplit("-", 1)[-1] if args.workload.endswith(("-e4m3", "-e5m2")) else None
    dims = (W.GQA8B if gqa else W.LLAMA7B).with_dtype(dt).with_kv(kv8)
    wl = 6 if gqa else 3 if args.workload.startswith("batch") else 4 if args.workload.startswith("verify") else 5
    t0 = time.time()
    model = GpuModel(dims, seed=1000 * wl + 1)
    log(f"weights ready in {time.time() - t0:.1f}s")
    if ctx_rule == "uniform":
        ctxs = [int(c) for c in synth.uniform_int(synth.key(1000 * wl + 4, B), 0, B, 128, 4097)]
    elif ctx_rule in ("1024", "2048"):
        ctxs = [int(ctx_rule)] * B
    else:
        ctxs = [1024 + int(s) for s in synth.uniform_int(synth.key(1000 * wl + 4, 1), 0, B, 16, 513)]
    max_blocks = -(-(max(ctxs + [chunk]) + K) // 16)
    n_pages = sum(-(-(c + K) // 16) for c in ctxs) + -(-chunk // 16) + 16
    pool = GpuPool(dims, n_pages)
    if kv8:
        pool.mem.fill_(0x30)  # every cached value 0.5 (e4m3) or 0.125 (e5m2): finite, timing-neutral
    else:
        pool.view().normal_()
    ids = vs.kv_alloc(pool.handle, n_pages)
    perm = synth.permutation(synth.key(1000 * wl + 6), n_pages)
    vs.kv_free(pool.handle, [ids[int(i)] for i in perm])
    rows, specs = [], []
    prefix_rows = {}
    root = vs.kv_prefix_root(f"{dims.name};{dt};weights={1000 * wl + 1};theta=10000".encode())
    for b in range(B):
        if ctx_rule == "prefix":  # 4 prefixes of 1024 tokens, each shared by 16 sequences through the index
            p = b // 16
            ptok = W.token_ids(1000 * wl + 3, 500 + p, 1024, dims.vocab)
            hashes = vs.kv_prefix_chain(root, ptok, 16)
            if p not in prefix_rows:  # the prompt's prefill leaves its full blocks in the index
                prefix_rows[p] = vs.kv_alloc(pool.handle, 64)
                vs.kv_prefix_insert(pool.handle, root, hashes, ptok, prefix_rows[p])
                vs.kv_free(pool.handle, prefix_rows[p])
            hit = vs.kv_prefix_lookup(pool.handle, root, hashes, ptok)
            assert hit == prefix_rows[p]
            r = vs.kv_append(pool.handle, hit, max_blocks, 1024, ctxs[b] - 1024 + K)
        else:
            r = vs.kv_alloc(pool.handle, -(-ctxs[b] // 16))
            r = vs.kv_append(pool.handle, r, max_blocks, ctxs[b], K)
        rows.append(r)
        specs.append(SeqSpec(ctxs[b], W.token_ids(1000 * wl + 3, b, K, dims.vocab)))
    if chunk:
        rows.append(vs.kv_append(pool.handle, [], max_blocks, 0, chunk))
        specs.append(SeqSpec(0, W.token_ids(1000 * wl + 3, 999, chunk, dims.vocab), want_logits=False))
    g0 = [0] * len(specs) if K > 1 else None
    # sequences on one shared prefix form a prefix group (the prefix's pages read once for the group)
    groups = [(16 * p, 16, 1024 // 16) for p in range(B // 16)] if ctx_rule == "prefix" else None
    sb = make_step(model, pool, specs, rows, max_blocks=max_blocks, want_logits_tensor=False, g0=g0, groups=groups)
    stream = torch.cuda.current_stream().cuda_stream

    def step():
        vs.decode_step(sb.desc, sb.block_tables, model.w, sb.out, sb.ws, sb.ws_bytes, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    M = sum(len(s.tokens) for s in specs)
    kvpt = 2 * dims.n_layers * dims.n_kv_heads * dims.head_dim * dims.kv_elem_bytes
    kv_read = sum(s.ctx + len(s.tokens) for s in specs) * kvpt  # logical K/V bytes the attention reads
    if groups:  # a prefix group's shared pages are read once for all of its sequences
        kv_read -= sum((n - 1) * pages * 16 for _, n, pages in groups) * kvpt
    step_bytes = streamed_weight_bytes(dims) + kv_read + M * kvpt
    n_rf = min(args.steps, ROOFLINE_STEPS)
    kt = kernel_times(vs, step, n_rf, 8 * dims.n_layers)
    result = {
        "workload": args.workload, "dtype": dt, "batch": B, "rows": M, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "rows_per_s": round(M * 1000.0 / ms, 1),
        "step_bytes": step_bytes, "step_TBps": round(step_bytes / (ms * 1e-3) / 1e12, 4),
        "step_frac_of_hbm_peak": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "contexts": [min(ctxs), max(ctxs)], "prompt_chunk_rows": chunk, "model_shape": dims.name,
        "prefix_groups": [list(g) for g in groups] if groups else None,
        "kv_cache": dims.kv_type,
        "weight_stream": weight_stream(dims, kt, n_rf),
        "attention": attention_stream(kt, n_rf, kv_read + M * kvpt),
    }
    if not args.no_cpu_baseline:
        if kv8:
            result["cpu_baseline"] = {"value": None, "unit": "rows/s", "kind": "oracle",
                                      "sample": "not run: the oracle's 8-bit cache path is timed on the 16-bit shapes"}
        else:
            if chunk:  # two decode rows of the step and the first 16 rows of its prompt chunk
                sample, label = [(ctxs[0], K), (ctxs[1], K), (0, 16)], "2 decode rows + 16 prompt-chunk rows"
            elif K > 1:  # one sequence's verify rows
                sample, label = [(ctxs[0], K)], f"1 sequence x {K} verify rows at context {ctxs[0]}"
            elif B > 1:  # two sequences of the batch
                sample, label = [(ctxs[0], 1), (ctxs[1], 1)], f"2 of the {B} sequences (contexts {ctxs[0]}, {ctxs[1]})"
            else:
                sample, label = [(ctxs[0], 1)], f"1 decode row at context {ctxs[0]}"
            result["cpu_baseline"] = other_cpu_baseline(dims, 1000 * wl + 1, sample, label)
    if args.copy_calibration:
        copy_calibration()
    print(json.dumps(result), flush=True)


def other_cpu_baseline(dims, seed, sample, label):
    """The oracle, as it stands, on a bounded sample of a workload's rows (the whole step would take many
    minutes on the host): the sampled sequences, each with its context and rows, in one oracle step on the
    same weights; reported as rows per second. Cached K/V are zeros (the oracle's time does not depend on
    them)."""
    import torch

    import oracle
    from synth import workloads as W

    log(f"cpu baseline: one oracle step over {label}")
    w_cpu = W.make_weights(dims, seed)
    seqs = []
    for ctx, n in sample:
        kv = torch.zeros(dims.n_layers, 2, ctx + n, dims.n_kv_heads, dims.head_dim, dtype=dims.torch_dtype)
        seqs.append(oracle.SeqState(kv, ctx, [1 + 7 * i for i in range(n)]))
    rows = sum(n for _, n in sample)
    t0 = time.perf_counter()
    oracle.decode_step(dims, w_cpu, seqs)
    dt = time.perf_counter() - t0
    return {"value": round(rows / dt, 5), "unit": "rows/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"{label}, {dims.name} {dims.dtype} (float64 PyTorch CPU oracle): {rows} rows in {dt:.1f} s"}


SAMPLE_WORKLOADS = {
    # name: (sequences, drafts per sequence); the 7B vocabulary, fp32 logits
    "sample-b8k5": (8, 5),
    "sample-b64k1": (64, 1),
}


def sample_workload(args):
    """verify_sample alone on resident inputs: target logits N(0, 4^2) over 32000 tokens (a peaked
    distribution), draft distributions softmax(target logits at the same position + N(0, 1)), drafts
    drawn from them, uniforms u and v. Reports the time per call and each kernel's algorithmic bytes
    against the HBM peak: the statistics kernel reads every target row once; the pick kernel reads,
    per sequence, the target row of the draw and, after a rejection, that draft row (plus a few scalars
    per draft)."""
    import torch

    import synth
    import verify_step_amd as vs

    B, K = SAMPLE_WORKLOADS[args.workload]
    V, M, T = 32000, B * K, 1.0
    dev = torch.device("cuda")
    k = synth.key(9001, B, K)
    p0 = synth.normal(synth.key(k, 1), 0, B * V, 0.0, 4.0).view(B, V).to(dev)
    logits = synth.normal(synth.key(k, 2), 0, M * V, 0.0, 4.0).view(M, V).to(dev)
    noise = synth.normal(synth.key(k, 3), 0, M * V, 0.0, 1.0).view(M, V).to(dev)
    prev = torch.cat([p0.view(B, 1, V), logits.view(B, K, V)[:, :K - 1]], dim=1).reshape(M, V)
    q = torch.softmax((prev + noise).double(), dim=1).float().contiguous()
    w = torch.from_numpy(synth.uniform(synth.key(k, 4), 0, M)).to(dev)
    cdf = torch.cumsum(q.double(), dim=1)
    drafts = torch.searchsorted(cdf, (w * cdf[:, -1]).view(M, 1), right=True).clamp(max=V - 1).view(M).int()
    u = torch.from_numpy(synth.uniform(synth.key(k, 5), 0, M)).float().to(dev)
    v = torch.from_numpy(synth.uniform(synth.key(k, 6), 0, B)).float().to(dev)
    q_start = torch.arange(0, M + 1, K, dtype=torch.int32, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(B, dtype=torch.int32, device=dev)
    nb = vs.verify_sample_workspace_bytes(B, M, V)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    def call():
        vs.verify_sample(B, M, V, q_start, drafts, p0, logits, q, u, v, T, acc, tok, ws, nb, stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        call()
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / args.steps
    n_kept = acc.cpu().tolist()
    rejected = sum(1 for n in n_kept if n < K)
    n_seg = -(-V // 2048)  # 2048-token segments of the statistics kernel, one partial (8 B) each
    stats_bytes = (B + M) * V * 4 + (B + M) * n_seg * 8
    pick_bytes = (B + rejected) * V * 4 + (M + B) * n_seg * 8 + M * 4 * 4 + B * (4 + 2 * 4)
    kern = {}
    for name, nbytes in (("smstats", stats_bytes), ("sample", pick_bytes)):
        n = min(args.steps, 64)
        ev = HipEvents(n)
        vs.vs_time_kernel(vs.VS_KERNEL[name], ev.start, ev.stop, n)
        for _ in range(n):
            call()
        torch.cuda.synchronize()
        done = vs.vs_timed_launches()
        vs.vs_time_kernel(0, None, None, 0)
        d_us = sum(ev.elapsed_ms(i) for i in range(done)) / done * 1e3
        ev.close()
        gbps = nbytes / (d_us * 1e-6) / 1e9
        kern[name] = {"avg_launch_us": round(d_us, 3), "bytes_per_launch": nbytes, "achieved_GBps": round(gbps, 1),
                      "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    result = {
        "workload": args.workload, "sequences": B, "drafts_per_seq": K, "vocab": V, "steps": args.steps,
        "us_per_call": round(us, 3), "accepted": n_kept, "kernels": kern,
        "timing": "call: torch events around the timed calls; kernels: dispatch events of each launch",
    }
    print(json.dumps(result), flush=True)


# kernel kinds timed per step: the weight products (a split-K product's slice reduction counts with it),
# attention and the standalone split merge
TIMED_KINDS = ["gateup", "qkv", "oproj", "down", "lmhead", "attn", "merge"]
PRODUCT_KINDS = ["qkv", "oproj", "gateup", "down", "lmhead"]


def kernel_times(vs, run_step, n_steps, per_step_cap):
    """Dispatch-event durations of every launch of each kind in TIMED_KINDS over n_steps calls of
    run_step (one pass of n_steps per kind)."""
    import torch

    out = {}
    for kind in TIMED_KINDS:
        cap = n_steps * per_step_cap
        ev = HipEvents(cap)
        vs.vs_time_kernel(vs.VS_KERNEL[kind], ev.start, ev.stop, cap)
        for _ in range(n_steps):
            run_step()
        torch.cuda.synchronize()
        n = vs.vs_timed_launches()
        vs.vs_time_kernel(0, None, None, 0)
        assert n < cap, f"{kind}: more launches than the event capacity"
        # each launch's interval from the pass's first start (launches of one kind may overlap on two streams)
        out[kind] = {"launch_us": [ev.elapsed_ms(i) * 1e3 for i in range(n)],
                     "interval_us": [(ev.start_ms(0, i) * 1e3, ev.elapsed_ms(0, i) * 1e3) for i in range(n)]}
        ev.close()
    return out


def weight_stream(dims, kt, n_steps):
    """The weights every step streams once, over the summed time of the product kernels per step (and
    the slice reductions of split-K products), against the HBM peak."""
    per_kind = {k: sum(kt[k]["launch_us"]) / n_steps for k in PRODUCT_KINDS}
    us = sum(per_kind.values())
    wbytes = streamed_weight_bytes(dims)
    gbps = wbytes / (us * 1e-6) / 1e9
    return {"bytes_per_step": wbytes, "product_us_per_step": round(us, 2), "achieved": round(gbps, 1),
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "us_per_step_by_kind": {k: round(v, 2) for k, v in per_kind.items()},
            "timing": f"dispatch events of every product and slice-reduction launch in {n_steps} eager steps"}


def busy_us(intervals):
    """Length of the union of (start, end) intervals: launches that overlap count once."""
    total, cur_s, cur_e = 0.0, None, None
    for a, b in sorted(intervals):
        if cur_e is None or a > cur_e:
            if cur_e is not None:
                total += cur_e - cur_s
            cur_s, cur_e = a, b
        else:
            cur_e = max(cur_e, b)
    return total + (cur_e - cur_s if cur_e is not None else 0.0)


def attention_stream(kt, n_steps, kv_bytes):
    """Logical K/V bytes per step (every cached key and value the step's rows attend to, a prefix group's
    shared pages once, plus the rows written) over the attention and merge kernels' time per step (the
    union of the attention launches' intervals: two that run at once on two streams count once)."""
    us = (busy_us(kt["attn"]["interval_us"]) + sum(kt["merge"]["launch_us"])) / n_steps
    gbps = kv_bytes / (us * 1e-6) / 1e9
    return {"kv_bytes_per_step": int(kv_bytes), "us_per_step": round(us, 2), "achieved": round(gbps, 1),
            "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4)}


def streamed_weight_bytes(dims):
    """Bytes of weights one step streams: every per-layer tensor, the final norm and the LM head (the
    embedding is gathered row by row, not streamed)."""
    D, F, V = dims.d_model, dims.ffn, dims.vocab
    q, kv = dims.n_heads * dims.head_dim, dims.n_kv_heads * dims.head_dim
    per_layer = D + q * D + 2 * kv * D + D * q + D + 3 * F * D
    return (dims.n_layers * per_layer + D + V * D) * dims.elem_bytes


def csrc_digest():
    """sha256 over the kernel sources, so a counter summary can tell whether it still describes them."""
    import hashlib

    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".h", ".hip", ".cpp")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def measured_traffic(path):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None when there is none or its
    kernel sources differ from the ones built here (the counters would describe other code)."""
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("csrc_sha256") != csrc_digest() or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def _load_model(model, dims, items, dev):
    """GpuModel built from a (name, layer, cpu tensor) stream."""
    import torch

    import verify_step_amd as vs
    from harness import model_desc

    model.dims = dims
    model.t = {}
    model.layer_structs = (vs.vs_layer_weights * dims.n_layers)()
    for name, layer, cpu in items:
        d = cpu.to(dev)
        model.t[(name, layer)] = d
        if layer >= 0:
            setattr(model.layer_structs[layer], name, d.data_ptr())
    model.w = vs.vs_weights(model_desc(dims), model.t[("embed", -1)].data_ptr(),
                            model.t[("final_norm", -1)].data_ptr(), model.t[("lm_head", -1)].data_ptr(),
                            ctypes.cast(model.layer_structs, ctypes.POINTER(vs.vs_layer_weights)))
    torch.cuda.synchronize()


def cpu_baseline(dims, w_cpu, kv0, tok0):
    """The oracle, as it stands, on one step of the same workload (B=1, 2048-token context)."""
    import torch

    import oracle

    log("cpu baseline: one oracle step of the same workload")
    full = torch.zeros(dims.n_layers, 2, CTX0 + 1, dims.n_kv_heads, dims.head_dim, dtype=dims.torch_dtype)
    full[:, :, :CTX0] = kv0
    st = oracle.SeqState(full, CTX0, list(tok0))
    t0 = time.perf_counter()
    oracle.decode_step(dims, w_cpu, [st])
    dt = time.perf_counter() - t0
    return {"value": round(1.0 / dt, 5), "unit": "tokens/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"1 decode step, B=1, context {CTX0}, 7B shape fp16 (float64 PyTorch CPU oracle), {dt:.1f} s"}


if __name__ == "__main__":
    main()
