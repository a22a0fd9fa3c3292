"""Host-side set-up around the library for tests and the benchmark.

Puts seeded synthetic inputs (from ``synth``) into device memory, keeps the
ctypes structures that point at them alive, and packs one step's batch
arrays. No part of the step is computed here: the step runs in
libverify_step.so through ``verify_step_amd``. PyTorch supplies device memory
and streams.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, field

import torch

import verify_step_amd as vs
from synth import workloads as W

PAGE = 16


def model_desc(dims: W.ModelDims) -> vs.vs_model_desc:
    return vs.vs_model_desc(dims.d_model, dims.n_heads, dims.n_kv_heads, dims.head_dim, dims.ffn, dims.vocab,
                            dims.n_layers, vs.DTYPE_CODE[dims.dtype], dims.rope_theta, dims.eps)


class GpuModel:
    """Model weights in device memory plus the vs_weights structure that points at them."""

    def __init__(self, dims: W.ModelDims, weights_cpu: dict | None = None, seed: int | None = None,
                 gains: str = "one", device: str = "cuda"):
        self.dims = dims
        self.t: dict = {}
        L = dims.n_layers
        self.layer_structs = (vs.vs_layer_weights * L)()
        if weights_cpu is not None:
            items = [("embed", -1, weights_cpu["embed"]), ("final_norm", -1, weights_cpu["final_norm"]),
                     ("lm_head", -1, weights_cpu["lm_head"])]
            for l in range(L):
                items += [(n, l, weights_cpu["layers"][l][n]) for n in W.LAYER_TENSORS]
        else:
            assert seed is not None
            items = W.iter_weights(dims, seed, gains)
        for name, layer, cpu in items:
            dev = cpu.to(device, non_blocking=False)
            self.t[(name, layer)] = dev
            if layer >= 0:
                setattr(self.layer_structs[layer], name, dev.data_ptr())
        self.w = vs.vs_weights(model_desc(dims), self.t[("embed", -1)].data_ptr(),
                               self.t[("final_norm", -1)].data_ptr(), self.t[("lm_head", -1)].data_ptr(),
                               ctypes.cast(self.layer_structs, ctypes.POINTER(vs.vs_layer_weights)))


class GpuPool:
    """A KV page pool: device memory (a torch tensor) and the library's pool handle."""

    def __init__(self, dims: W.ModelDims, num_pages: int, device: str = "cuda"):
        self.dims = dims
        self.desc = vs.vs_pool_desc(num_pages, PAGE, dims.n_layers, dims.n_kv_heads, dims.head_dim,
                                    vs.DTYPE_CODE[dims.kv_type])
        self.page_bytes = vs.kv_page_bytes(self.desc)
        self.num_pages = num_pages
        self.mem = torch.zeros(num_pages * self.page_bytes, dtype=torch.uint8, device=device)
        self.handle = vs.kv_pool_create(self.desc, self.mem.data_ptr(), self.mem.numel())

    def close(self):
        if self.handle:
            vs.kv_pool_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def view(self, raw: bool = False) -> torch.Tensor:
        """[page][layer][K|V][kv_head][slot][dim] view of the pool in the cache's storage dtype (as
        bytes for an 8-bit cache when raw is set)."""
        d = self.dims
        t = self.mem if raw and d.kv_elem_bytes == 1 else self.mem.view(d.kv_torch_dtype)
        return t.view(self.num_pages, d.n_layers, 2, d.n_kv_heads, PAGE, d.head_dim)

    def write(self, row: list[int], p0: int, kv: torch.Tensor) -> None:
        """Store contiguous K/V [layer][2][n][kv_head][dim] at positions p0.. of a sequence."""
        n = kv.shape[2]
        if n == 0:
            return
        dev = self.mem.device
        pos = torch.arange(p0, p0 + n)
        pages = torch.tensor(row, dtype=torch.int64)[pos // PAGE].to(dev)
        slots = (pos % PAGE).to(dev)
        if self.dims.kv_elem_bytes == 1:  # 8-bit floats move as bytes
            self.view(raw=True)[pages, :, :, :, slots, :] = kv.view(torch.uint8).to(dev).permute(2, 0, 1, 3, 4)
        else:
            self.view()[pages, :, :, :, slots, :] = kv.to(dev).permute(2, 0, 1, 3, 4)

    def read(self, row: list[int], p0: int, p1: int) -> torch.Tensor:
        """Gather positions [p0, p1) of a sequence back to contiguous [layer][2][n][kv_head][dim] (CPU)."""
        dev = self.mem.device
        pos = torch.arange(p0, p1)
        pages = torch.tensor(row, dtype=torch.int64)[pos // PAGE].to(dev)
        slots = (pos % PAGE).to(dev)
        if self.dims.kv_elem_bytes == 1:
            g = self.view(raw=True)[pages, :, :, :, slots, :].permute(1, 2, 0, 3, 4).contiguous().cpu()
            return g.view(self.dims.kv_torch_dtype)
        return self.view()[pages, :, :, :, slots, :].permute(1, 2, 0, 3, 4).cpu()


@dataclass
class SeqSpec:
    ctx: int
    tokens: list
    want_logits: bool = True


@dataclass
class StepBuffers:
    """Device arrays of one step's batch, its outputs and workspace."""

    desc: vs.vs_batch_desc
    out: vs.vs_step_out
    block_tables: torch.Tensor
    q_start: torch.Tensor
    ctx_len: torch.Tensor
    tokens: torch.Tensor
    logit_rows: torch.Tensor
    argmax: torch.Tensor
    gap: torch.Tensor
    logits: torch.Tensor | None
    ws: torch.Tensor
    ws_bytes: int
    g0: torch.Tensor | None = None
    accept_len: torch.Tensor | None = None
    bonus: torch.Tensor | None = None
    keep: list = field(default_factory=list)


def make_step(model: GpuModel, pool: GpuPool, seqs: list[SeqSpec], rows: list[list[int]], max_blocks: int | None = None,
              want_logits_tensor: bool = True, g0: list[int] | None = None, device: str = "cuda",
              groups: list[tuple[int, int, int]] | None = None) -> StepBuffers:
    """One step's device buffers. groups: shared-prefix groups (first sequence, sequences, prefix pages)."""
    d = model.dims
    B = len(seqs)
    q_start = [0]
    for s in seqs:
        q_start.append(q_start[-1] + len(s.tokens))
    M = q_start[-1]
    tokens = [t for s in seqs for t in s.tokens]
    logit_rows = [q_start[b] + i for b, s in enumerate(seqs) if s.want_logits for i in range(len(s.tokens))]
    max_ctx = max(s.ctx + len(s.tokens) for s in seqs)
    need_blocks = -(-max_ctx // PAGE)
    max_blocks = max_blocks or max(need_blocks, max(len(r) for r in rows))
    bt = torch.zeros(B, max_blocks, dtype=torch.int32)
    for b, r in enumerate(rows):
        bt[b, :len(r)] = torch.tensor(r, dtype=torch.int32)
    i32 = dict(dtype=torch.int32, device=device)
    bufs = dict(
        block_tables=bt.to(device),
        q_start=torch.tensor(q_start, **i32),
        ctx_len=torch.tensor([s.ctx for s in seqs], **i32),
        tokens=torch.tensor(tokens, **i32),
        logit_rows=torch.tensor(logit_rows if logit_rows else [0], **i32),
        argmax=torch.full((max(M, 1),), -7, **i32),
        gap=torch.full((max(M, 1),), float("nan"), dtype=torch.float32, device=device),
    )
    logits = (torch.empty(max(len(logit_rows), 1), d.vocab, dtype=torch.float32, device=device)
              if want_logits_tensor else None)
    desc = vs.vs_batch_desc(B, M, len(logit_rows), max(len(s.tokens) for s in seqs), max_ctx, max_blocks,
                            pool.handle, bufs["q_start"].data_ptr(), bufs["ctx_len"].data_ptr(),
                            bufs["tokens"].data_ptr(), bufs["logit_rows"].data_ptr() if logit_rows else None)
    keep = []
    if groups:
        gt = torch.tensor(groups, dtype=torch.int32).t().contiguous().to(device)  # rows: seq0, n, pages
        keep.append(gt)
        desc.n_prefix_groups = len(groups)
        desc.max_group_size = max(g[1] for g in groups)
        desc.max_group_pages = max(g[2] for g in groups)
        desc.group_seq0, desc.group_n, desc.group_pages = gt[0].data_ptr(), gt[1].data_ptr(), gt[2].data_ptr()
    ws_bytes = vs.decode_step_workspace_bytes(desc, model_desc(d))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    extra = {}
    if g0 is not None:
        extra = dict(g0=torch.tensor(g0, **i32), accept_len=torch.full((B,), -7, **i32),
                     bonus=torch.full((B,), -7, **i32))
    out = vs.vs_step_out(logits.data_ptr() if logits is not None else None, bufs["argmax"].data_ptr(),
                         bufs["gap"].data_ptr(),
                         extra["g0"].data_ptr() if extra else None,
                         extra["accept_len"].data_ptr() if extra else None,
                         extra["bonus"].data_ptr() if extra else None)
    return StepBuffers(desc=desc, out=out, logits=logits, ws=ws, ws_bytes=ws_bytes, **bufs, **extra, keep=keep)


def run_step(model: GpuModel, sb: StepBuffers, stream: torch.cuda.Stream | None = None) -> None:
    s = stream or torch.cuda.current_stream()
    vs.decode_step(sb.desc, sb.block_tables, model.w, sb.out, sb.ws, sb.ws_bytes, s.cuda_stream)


def alloc_rows(pool: GpuPool, lengths: list[int], shuffle_key: int | None = None) -> list[list[int]]:
    """Allocate ceil(n / 16) pages for each length. With a shuffle key the pool's free list is
    first permuted (all pages taken, then returned in a seeded order), so ids are scattered."""
    if shuffle_key is not None:
        import synth

        n_free = vs.kv_num_free(pool.handle)
        ids = vs.kv_alloc(pool.handle, n_free)
        perm = synth.permutation(shuffle_key, n_free)
        vs.kv_free(pool.handle, [ids[int(i)] for i in perm])
    return [vs.kv_alloc(pool.handle, -(-n // PAGE)) for n in lengths]
