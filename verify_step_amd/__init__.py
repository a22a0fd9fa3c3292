"""Python binding of libverify_step.so (the gfx950 decode / verify step).

Argument marshalling only: every function here forwards to the C ABI declared
in include/verify_step.h under the same name, and every step of the decode /
verify path runs in the library's HIP kernels. PyTorch provides device memory
and streams. Importing this module does not need a GPU; calling the step does.
The library must have been built (verify_step_amd.build.build()); there is no
fallback path, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_float, c_int32, c_size_t, c_uint64, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libverify_step.so")

VS_OK, VS_ERR_INVALID, VS_ERR_OOM, VS_ERR_SHAPE, VS_ERR_HIP = 0, -1, -2, -3, -4
VS_F32, VS_F16, VS_BF16, VS_FP8_E4M3, VS_FP8_E5M2 = 0, 1, 2, 3, 4
DTYPE_CODE = {"f32": VS_F32, "f16": VS_F16, "bf16": VS_BF16, "e4m3": VS_FP8_E4M3, "e5m2": VS_FP8_E5M2}

EXPORTS = [
    "vs_last_error", "kv_page_bytes", "kv_pool_create", "kv_pool_destroy", "kv_alloc", "kv_share", "kv_free",
    "kv_append", "kv_num_free", "kv_refcount", "kv_pool_base", "kv_prefix_root", "kv_prefix_chain",
    "kv_prefix_insert", "kv_prefix_lookup", "kv_prefix_evict", "kv_prefix_entries", "decode_step_workspace_bytes",
    "decode_step", "decode_step_noalloc",
    "verify_accept", "verify_sample_workspace_bytes", "verify_sample", "vs_time_kernel", "vs_timed_launches", "vs_stream_read",
]

VS_STEP_BAD_TOKEN, VS_STEP_BAD_PAGE, VS_STEP_BAD_BATCH = 1, 2, 4

VS_KERNEL = {"none": 0, "qkv": 1, "attn": 2, "merge": 3, "oproj": 4, "gateup": 5, "down": 6, "lmhead": 7,
             "smstats": 8, "sample": 9}


class VSError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


class vs_model_desc(Structure):
    _fields_ = [("d_model", c_int32), ("n_heads", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32),
                ("ffn", c_int32), ("vocab", c_int32), ("n_layers", c_int32), ("dtype", c_int32),
                ("rope_theta", c_float), ("eps", c_float)]


class vs_layer_weights(Structure):
    _fields_ = [(n, c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "wg", "wu", "wd")]


class vs_weights(Structure):
    _fields_ = [("dims", vs_model_desc), ("embed", c_void_p), ("final_norm", c_void_p), ("lm_head", c_void_p),
                ("layers", POINTER(vs_layer_weights))]


class vs_pool_desc(Structure):
    _fields_ = [("num_pages", c_int32), ("page_tokens", c_int32), ("n_layers", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("dtype", c_int32)]


class vs_batch_desc(Structure):
    _fields_ = [("B", c_int32), ("M", c_int32), ("M_log", c_int32), ("max_rows", c_int32), ("max_ctx", c_int32),
                ("max_blocks", c_int32), ("pool", c_void_p), ("q_start", c_void_p), ("ctx_len", c_void_p),
                ("tokens", c_void_p), ("logit_rows", c_void_p), ("ctx_advance", c_void_p),
                ("error_flags", c_void_p), ("n_prefix_groups", c_int32), ("max_group_size", c_int32),
                ("max_group_pages", c_int32), ("group_seq0", c_void_p), ("group_n", c_void_p),
                ("group_pages", c_void_p)]


class vs_step_out(Structure):
    _fields_ = [("logits", c_void_p), ("argmax", c_void_p), ("top2_gap", c_void_p), ("g0", c_void_p),
                ("accept_len", c_void_p), ("bonus", c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with verify_step_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        i32p = POINTER(c_int32)
        L.vs_last_error.restype = ctypes.c_char_p
        L.vs_last_error.argtypes = []
        L.kv_page_bytes.restype = c_size_t
        L.kv_page_bytes.argtypes = [POINTER(vs_pool_desc)]
        L.kv_pool_create.restype = c_int32
        L.kv_pool_create.argtypes = [POINTER(vs_pool_desc), c_void_p, c_size_t, POINTER(c_void_p)]
        L.kv_pool_destroy.restype = None
        L.kv_pool_destroy.argtypes = [c_void_p]
        L.kv_alloc.restype = c_int32
        L.kv_alloc.argtypes = [c_void_p, c_int32, i32p]
        L.kv_share.restype = c_int32
        L.kv_share.argtypes = [c_void_p, i32p, c_int32]
        L.kv_free.restype = c_int32
        L.kv_free.argtypes = [c_void_p, i32p, c_int32]
        L.kv_append.restype = c_int32
        L.kv_append.argtypes = [c_void_p, i32p, i32p, c_int32, c_int32, c_int32, c_void_p]
        L.kv_num_free.restype = c_int32
        L.kv_num_free.argtypes = [c_void_p]
        L.kv_refcount.restype = c_int32
        L.kv_refcount.argtypes = [c_void_p, c_int32]
        L.kv_pool_base.restype = c_void_p
        L.kv_pool_base.argtypes = [c_void_p]
        u64p = POINTER(c_uint64)
        L.kv_prefix_root.restype = c_int32
        L.kv_prefix_root.argtypes = [c_void_p, c_size_t, u64p]
        L.kv_prefix_chain.restype = c_int32
        L.kv_prefix_chain.argtypes = [c_uint64, i32p, c_int32, c_int32, u64p]
        L.kv_prefix_insert.restype = c_int32
        L.kv_prefix_insert.argtypes = [c_void_p, c_uint64, u64p, i32p, i32p, c_int32, i32p]
        L.kv_prefix_lookup.restype = c_int32
        L.kv_prefix_lookup.argtypes = [c_void_p, c_uint64, u64p, i32p, c_int32, i32p, i32p]
        L.kv_prefix_evict.restype = c_int32
        L.kv_prefix_evict.argtypes = [c_void_p, c_int32, i32p]
        L.kv_prefix_entries.restype = c_int32
        L.kv_prefix_entries.argtypes = [c_void_p]
        L.decode_step_workspace_bytes.restype = c_int32
        L.decode_step_workspace_bytes.argtypes = [POINTER(vs_batch_desc), POINTER(vs_model_desc), POINTER(c_size_t)]
        L.decode_step.restype = c_int32
        L.decode_step.argtypes = [POINTER(vs_batch_desc), c_void_p, POINTER(vs_weights), POINTER(vs_step_out),
                                  c_void_p, c_size_t, c_void_p]
        L.decode_step_noalloc.restype = c_int32
        L.decode_step_noalloc.argtypes = [POINTER(vs_batch_desc), c_void_p, POINTER(vs_weights),
                                          POINTER(vs_step_out), c_void_p]
        L.verify_accept.restype = c_int32
        L.verify_accept.argtypes = [c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        L.verify_sample_workspace_bytes.restype = c_int32
        L.verify_sample_workspace_bytes.argtypes = [c_int32, c_int32, c_int32, POINTER(c_size_t)]
        L.verify_sample.restype = c_int32
        L.verify_sample.argtypes = [c_int32, c_int32, c_int32] + [c_void_p] * 7 + [c_float, c_void_p, c_void_p,
                                                                                     c_void_p, c_size_t, c_void_p]
        L.vs_time_kernel.restype = c_int32
        L.vs_time_kernel.argtypes = [c_int32, c_void_p, c_void_p, c_int32]
        L.vs_timed_launches.restype = c_int32
        L.vs_timed_launches.argtypes = []
        L.vs_stream_read.restype = c_int32
        L.vs_stream_read.argtypes = [c_void_p, c_size_t, c_void_p, c_void_p]
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != VS_OK:
        raise VSError(status, lib().vs_last_error().decode())


def _ptr(t) -> int | None:
    """Device or host address of a tensor / int / None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _i32_array(values):
    arr = (c_int32 * max(1, len(values)))(*values)
    return arr


def vs_last_error() -> str:
    return lib().vs_last_error().decode()


# ---------------------------------------------------------------- pool

def kv_page_bytes(desc: vs_pool_desc) -> int:
    return int(lib().kv_page_bytes(ctypes.byref(desc)))


def kv_pool_create(desc: vs_pool_desc, dev_base: int, dev_bytes: int) -> int:
    out = c_void_p()
    _check(lib().kv_pool_create(ctypes.byref(desc), c_void_p(dev_base), dev_bytes, ctypes.byref(out)))
    return out.value


def kv_pool_destroy(pool: int) -> None:
    lib().kv_pool_destroy(c_void_p(pool))


def kv_alloc(pool: int, n: int) -> list[int]:
    ids = (c_int32 * max(1, n))()
    _check(lib().kv_alloc(c_void_p(pool), n, ids))
    return list(ids[:n])


def kv_share(pool: int, ids: list[int]) -> None:
    _check(lib().kv_share(c_void_p(pool), _i32_array(ids), len(ids)))


def kv_free(pool: int, ids: list[int]) -> None:
    _check(lib().kv_free(c_void_p(pool), _i32_array(ids), len(ids)))


def kv_append(pool: int, bt_row: list[int], max_blocks: int, cur_len: int, n_new: int, stream: int = 0) -> list[int]:
    """Returns the new block-table row (the input list is not modified)."""
    row = (c_int32 * max_blocks)(*(list(bt_row) + [0] * (max_blocks - len(bt_row))))
    nb = c_int32(len(bt_row))
    _check(lib().kv_append(c_void_p(pool), row, ctypes.byref(nb), max_blocks, cur_len, n_new, c_void_p(stream)))
    return list(row[:nb.value])


def kv_num_free(pool: int) -> int:
    return int(lib().kv_num_free(c_void_p(pool)))


def kv_refcount(pool: int, page: int) -> int:
    return int(lib().kv_refcount(c_void_p(pool), page))


def kv_pool_base(pool: int) -> int:
    return int(lib().kv_pool_base(c_void_p(pool)) or 0)


def kv_prefix_root(key: bytes) -> int:
    out = c_uint64()
    _check(lib().kv_prefix_root(key, len(key), ctypes.byref(out)))
    return int(out.value)


def _u64_array(xs):
    return (c_uint64 * max(1, len(xs)))(*xs)


def kv_prefix_chain(root: int, tokens: list[int], page_tokens: int) -> list[int]:
    n = len(tokens) // page_tokens
    out = (c_uint64 * max(1, n))()
    _check(lib().kv_prefix_chain(root, _i32_array(tokens), len(tokens), page_tokens, out))
    return [int(h) for h in out[:n]]


def kv_prefix_insert(pool: int, root: int, hashes: list[int], tokens: list[int], pages: list[int]) -> int:
    added = c_int32()
    _check(lib().kv_prefix_insert(c_void_p(pool), root, _u64_array(hashes), _i32_array(tokens), _i32_array(pages),
                                  len(hashes), ctypes.byref(added)))
    return int(added.value)


def kv_prefix_lookup(pool: int, root: int, hashes: list[int], tokens: list[int]) -> list[int]:
    """Pages of the longest indexed run of leading blocks (one reference taken on each for the caller)."""
    pages = (c_int32 * max(1, len(hashes)))()
    hit = c_int32()
    _check(lib().kv_prefix_lookup(c_void_p(pool), root, _u64_array(hashes), _i32_array(tokens), len(hashes), pages,
                                  ctypes.byref(hit)))
    return list(pages[:hit.value])


def kv_prefix_evict(pool: int, n_pages: int) -> int:
    freed = c_int32()
    _check(lib().kv_prefix_evict(c_void_p(pool), n_pages, ctypes.byref(freed)))
    return int(freed.value)


def kv_prefix_entries(pool: int) -> int:
    return int(lib().kv_prefix_entries(c_void_p(pool)))


# ---------------------------------------------------------------- step

def decode_step_workspace_bytes(desc: vs_batch_desc, dims: vs_model_desc) -> int:
    n = c_size_t()
    _check(lib().decode_step_workspace_bytes(ctypes.byref(desc), ctypes.byref(dims), ctypes.byref(n)))
    return int(n.value)


def decode_step(desc: vs_batch_desc, block_tables, weights: vs_weights, out: vs_step_out, ws, ws_bytes: int,
                stream: int) -> None:
    _check(lib().decode_step(ctypes.byref(desc), c_void_p(_ptr(block_tables)), ctypes.byref(weights),
                             ctypes.byref(out), c_void_p(_ptr(ws)), ws_bytes, c_void_p(stream)))


VS_NOALLOC_SCRATCH_BYTES = 96 << 20  # the library's per-GPU scratch array (include/verify_step.h)


def decode_step_noalloc(desc: vs_batch_desc, block_tables, weights: vs_weights, out: vs_step_out,
                        stream: int) -> None:
    _check(lib().decode_step_noalloc(ctypes.byref(desc), c_void_p(_ptr(block_tables)), ctypes.byref(weights),
                                     ctypes.byref(out), c_void_p(stream)))


def verify_accept(B: int, q_start, drafts, g0, argmax, accept_len, bonus, stream: int) -> None:
    _check(lib().verify_accept(B, c_void_p(_ptr(q_start)), c_void_p(_ptr(drafts)), c_void_p(_ptr(g0)),
                               c_void_p(_ptr(argmax)), c_void_p(_ptr(accept_len)), c_void_p(_ptr(bonus)),
                               c_void_p(stream)))


def verify_sample_workspace_bytes(B: int, M: int, V: int) -> int:
    n = c_size_t()
    _check(lib().verify_sample_workspace_bytes(B, M, V, ctypes.byref(n)))
    return int(n.value)


def verify_sample(B: int, M: int, V: int, q_start, drafts, p0_logits, logits, q_probs, u, v, temperature: float,
                  accept_len, token, ws, ws_bytes: int, stream: int) -> None:
    _check(lib().verify_sample(B, M, V, *[c_void_p(_ptr(t)) for t in (q_start, drafts, p0_logits, logits, q_probs,
                                                                         u, v)],
                               float(temperature), c_void_p(_ptr(accept_len)), c_void_p(_ptr(token)),
                               c_void_p(_ptr(ws)), ws_bytes, c_void_p(stream)))


# ---------------------------------------------------------------- instrumentation

def vs_time_kernel(kind: int, start_events, stop_events, capacity: int) -> None:
    """start_events / stop_events: ctypes arrays of hipEvent_t (c_void_p) that stay alive while armed."""
    _check(lib().vs_time_kernel(kind, start_events, stop_events, capacity))


def vs_timed_launches() -> int:
    return int(lib().vs_timed_launches())


def vs_stream_read(buf, nbytes: int, sink, stream: int) -> None:
    _check(lib().vs_stream_read(c_void_p(_ptr(buf)), nbytes, c_void_p(_ptr(sink)), c_void_p(stream)))
