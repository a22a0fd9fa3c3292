"""Shapes and seeded recipes for the synthetic workloads of the decode/verify step.

Input generation only: model dimensions, random-init weights, synthetic
KV-cache contents and token ids. No part of the step is computed here.

Seeds follow one scheme everywhere: a workload number w uses
seed = 1000 * w + stream, with stream 1 = weights, 2 = KV contents,
3 = token ids, 4 = churn, 5 = drafts, 6 = page shuffles.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import torch

import synth

STREAM_WEIGHTS, STREAM_KV, STREAM_TOKENS, STREAM_CHURN, STREAM_DRAFTS, STREAM_PAGES = 1, 2, 3, 4, 5, 6

_TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
_KV_TDT = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}  # OCP 8-bit floats


@dataclass(frozen=True)
class ModelDims:
    """A Llama-style pre-norm decoder: RMSNorm, rotary attention, SwiGLU MLP, untied head."""

    name: str
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    n_layers: int
    dtype: str  # storage type of weights (and of the KV cache unless kv_dtype says otherwise)
    rope_theta: float = 10000.0
    eps: float = 1e-5
    page_tokens: int = 16
    kv_dtype: str | None = None  # KV cache storage: None (= dtype) or an 8-bit float, "e4m3" / "e5m2"

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TDT[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def kv_type(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def kv_torch_dtype(self) -> torch.dtype:
        return _KV_TDT.get(self.kv_type) or _TDT[self.kv_type]

    @property
    def kv_elem_bytes(self) -> int:
        return 1 if self.kv_type in _KV_TDT else self.elem_bytes

    def with_dtype(self, dtype: str) -> "ModelDims":
        return dataclasses.replace(self, dtype=dtype)

    def with_kv(self, kv_dtype: str | None) -> "ModelDims":
        return dataclasses.replace(self, kv_dtype=kv_dtype, name=f"{self.name}-kv{kv_dtype}" if kv_dtype else self.name)


TINY = ModelDims("tiny-1L-d256-4x64-ffn1024-v1000", 256, 4, 4, 64, 1024, 1000, 1, "f32")
LLAMA7B = ModelDims("7B-MHA-32L-d4096-32x128-ffn11008-v32000", 4096, 32, 32, 128, 11008, 32000, 32, "f16")
# grouped K/V heads at Llama 3.1 8B's widths: 32 query heads over 8 K/V heads of 128, MLP 14336,
# vocabulary 128256 (the block otherwise as above: RMSNorm, rotary with theta 10000, SwiGLU)
GQA8B = ModelDims("8B-GQA-32L-d4096-32q8kv128-ffn14336-v128256", 4096, 32, 8, 128, 14336, 128256, 32, "f16")

# per-layer weight tensors in a fixed order; tags 1..10 name them in the seed scheme
LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "wg", "wu", "wd")
_TAG = {"embed": 0, "attn_norm": 1, "wq": 2, "wk": 3, "wv": 4, "wo": 5, "ffn_norm": 6, "wg": 7, "wu": 8, "wd": 9,
        "final_norm": 10, "lm_head": 11}


def tensor_shape(dims: ModelDims, name: str) -> tuple[int, ...]:
    D, F, V = dims.d_model, dims.ffn, dims.vocab
    q, kv = dims.n_heads * dims.head_dim, dims.n_kv_heads * dims.head_dim
    return {
        "embed": (V, D), "attn_norm": (D,), "wq": (q, D), "wk": (kv, D), "wv": (kv, D), "wo": (D, q),
        "ffn_norm": (D,), "wg": (F, D), "wu": (F, D), "wd": (D, F), "final_norm": (D,), "lm_head": (V, D),
    }[name]


def make_tensor(dims: ModelDims, seed: int, name: str, layer: int = 0, std: float = 0.02,
                gains: str = "one") -> torch.Tensor:
    """One weight tensor: matrices N(0, std); norm gains 1 ("one") or N(1, 0.1) ("random")."""
    shape = tensor_shape(dims, name)
    n = 1
    for s in shape:
        n *= s
    k = synth.key(seed, STREAM_WEIGHTS, layer, _TAG[name])
    if name.endswith("norm"):
        if gains == "one":
            return torch.ones(shape, dtype=dims.torch_dtype)
        return synth.normal(k, 0, n, 1.0, 0.1, dims.dtype).reshape(shape)
    return synth.normal(k, 0, n, 0.0, std, dims.dtype).reshape(shape)


def iter_weights(dims: ModelDims, seed: int, gains: str = "one"):
    """Yield (name, layer, tensor) for every weight, one tensor at a time."""
    yield "embed", -1, make_tensor(dims, seed, "embed", 0xFFFF, gains=gains)
    for l in range(dims.n_layers):
        for name in LAYER_TENSORS:
            yield name, l, make_tensor(dims, seed, name, l, gains=gains)
    yield "final_norm", -1, make_tensor(dims, seed, "final_norm", 0xFFFF, gains=gains)
    yield "lm_head", -1, make_tensor(dims, seed, "lm_head", 0xFFFF, gains=gains)


def make_weights(dims: ModelDims, seed: int, gains: str = "one") -> dict:
    """All weights as CPU tensors in the storage dtype: {"embed", "layers": [..], "final_norm", "lm_head"}."""
    out: dict = {"layers": [dict() for _ in range(dims.n_layers)]}
    for name, layer, t in iter_weights(dims, seed, gains):
        if layer < 0:
            out[name] = t
        else:
            out["layers"][layer][name] = t
    return out


def kv_block(dims: ModelDims, seed: int, content: int, p0: int, p1: int, std: float = 1.0) -> torch.Tensor:
    """Synthetic cached K/V for positions [p0, p1) of one content stream.

    Returns [n_layers][2][p1 - p0][n_kv_heads][head_dim] in the KV cache's storage
    dtype, values N(0, std) read as post-rotary K and V. Element (content, layer,
    k/v, pos, head, dim) is a pure function of the seed, so two sequences that
    share an exact prefix use the same content id and get the same bits. An
    8-bit cache takes the fp32 draws through the library's float8 cast (values
    N(0, 1) stay far inside both formats' range).
    """
    L, H, Dh = dims.n_layers, dims.n_kv_heads, dims.head_dim
    n = p1 - p0
    fp8 = dims.kv_elem_bytes == 1
    out = torch.empty((L, 2, n, H, Dh), dtype=torch.float32 if fp8 else dims.torch_dtype)
    if n <= 0:
        return out.to(dims.kv_torch_dtype)
    for l in range(L):
        for t in range(2):
            k = synth.key(seed, STREAM_KV, content, l, t)
            synth.normal_into(out[l, t].reshape(-1), k, p0 * H * Dh, 0.0, std)
    return out.to(dims.kv_torch_dtype) if fp8 else out


def token_ids(seed: int, tag: int, n: int, vocab: int) -> list[int]:
    """n token ids uniform in [0, vocab) from the token stream, sub-stream `tag`."""
    return [int(t) for t in synth.uniform_int(synth.key(seed, STREAM_TOKENS, tag), 0, n, 0, vocab)]
