"""The C ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments before touching the GPU. No compute calls here."""
import ctypes
import os
import re

import pytest

import verify_step_amd as vs
from verify_step_amd import build as vsbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "verify_step.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(vs.LIB_PATH):
        vsbuild.build()
    return vs.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["kv_alloc", "kv_free", "kv_share", "kv_append", "decode_step", "verify_accept", "verify_sample",
              "decode_step_workspace_bytes", "kv_pool_create", "vs_last_error"]:
        assert n in names
    assert set(names) == set(vs.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def declared_arity():
    """Parameter count of every prototype in the header (a lone `void` counts as none)."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for name, params in re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(([^;{]*?)\)\s*;", text, flags=re.M):
        params = params.strip()
        out[name] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_signatures_match_the_header(L):
    arity = declared_arity()
    assert set(arity) == set(vs.EXPORTS)
    for n, k in arity.items():
        assert len(getattr(L, n).argtypes) == k, f"{n}: binding has {len(getattr(L, n).argtypes)} arguments, header {k}"


def test_binding_has_the_same_names():
    for n in vs.EXPORTS:
        assert callable(getattr(vs, n)), n


def _tiny_desc(**kw):
    d = dict(num_pages=8, page_tokens=16, n_layers=1, n_kv_heads=4, head_dim=64, dtype=vs.VS_F32)
    d.update(kw)
    return vs.vs_pool_desc(*d.values())


def test_pool_create_rejects_bad_geometry(L):
    buf = ctypes.create_string_buffer(64)
    with pytest.raises(vs.VSError) as e:
        vs.kv_pool_create(_tiny_desc(), ctypes.addressof(buf), 64)
    assert e.value.status == vs.VS_ERR_INVALID and "smaller" in str(e.value)
    with pytest.raises(vs.VSError):
        vs.kv_pool_create(_tiny_desc(num_pages=0), ctypes.addressof(buf), 64)
    with pytest.raises(vs.VSError):
        vs.kv_pool_create(_tiny_desc(dtype=7), ctypes.addressof(buf), 64)


def test_page_bytes_formula(L):
    # layers x (K, V) x kv_heads x 16 slots x head_dim x bytes
    assert vs.kv_page_bytes(_tiny_desc()) == 1 * 2 * 4 * 16 * 64 * 4
    assert vs.kv_page_bytes(_tiny_desc(n_layers=32, n_kv_heads=32, head_dim=128, dtype=vs.VS_F16)) == 8 * 2 ** 20


def test_step_rejects_bad_shapes_before_launching(L):
    dims = vs.vs_model_desc(256, 4, 4, 64, 1024, 1000, 1, vs.VS_F32, 10000.0, 1e-5)
    desc = vs.vs_batch_desc(4, 4, 4, 1, 65, 5, None, None, None, None, None)
    assert vs.decode_step_workspace_bytes(desc, dims) > 0
    bad = vs.vs_model_desc(256, 4, 4, 96, 1024, 1000, 1, vs.VS_F32, 10000.0, 1e-5)
    with pytest.raises(vs.VSError) as e:
        vs.decode_step_workspace_bytes(desc, bad)
    assert e.value.status == vs.VS_ERR_SHAPE
    short = vs.vs_batch_desc(4, 4, 4, 1, 100, 5, None, None, None, None, None)  # 5 blocks < 100 positions
    with pytest.raises(vs.VSError):
        vs.decode_step_workspace_bytes(short, dims)
    w = vs.vs_weights(dims, None, None, None, None)
    out = vs.vs_step_out()
    with pytest.raises(vs.VSError) as e:
        vs.decode_step(desc, None, w, out, None, 0, 0)
    assert e.value.status == vs.VS_ERR_INVALID


def test_prefix_groups_checked_on_the_host(L):
    """Shared-prefix groups in the batch descriptor: an fp16 / bf16 model with head_dim 128 plans them (the
    workspace grows by the group bookkeeping) and rejects inconsistent ones with VS_ERR_INVALID before any
    device call; an fp32 model or head_dim 64 ignores them."""
    fake = 4096  # non-null stand-ins for the device arrays (nothing is dereferenced on the host)
    dims = vs.vs_model_desc(256, 2, 2, 128, 512, 1000, 2, vs.VS_F16, 10000.0, 1e-5)

    def desc(n_groups=1, size=4, pages=3, arrays=True, B=5, max_blocks=8):
        d = vs.vs_batch_desc(B, B, B, 1, 100, max_blocks, None, None, None, None, None)
        d.n_prefix_groups, d.max_group_size, d.max_group_pages = n_groups, size, pages
        if arrays:
            d.group_seq0, d.group_n, d.group_pages = fake, fake, fake
        return d

    plain = vs.decode_step_workspace_bytes(desc(n_groups=0), dims)
    assert vs.decode_step_workspace_bytes(desc(), dims) > plain
    for bad in (desc(arrays=False), desc(size=6), desc(n_groups=6), desc(pages=9), desc(size=0), desc(n_groups=-1)):
        with pytest.raises(vs.VSError) as e:
            vs.decode_step_workspace_bytes(bad, dims)
        assert e.value.status == vs.VS_ERR_INVALID
    for other in (vs.vs_model_desc(256, 2, 2, 128, 512, 1000, 2, vs.VS_F32, 10000.0, 1e-5),
                  vs.vs_model_desc(256, 4, 4, 64, 512, 1000, 2, vs.VS_F16, 10000.0, 1e-5)):
        assert vs.decode_step_workspace_bytes(desc(arrays=False, size=6), other) == \
            vs.decode_step_workspace_bytes(desc(n_groups=0), other)


def test_verify_accept_rejects_null(L):
    with pytest.raises(vs.VSError):
        vs.verify_accept(3, None, None, None, None, None, None, 0)
    vs.verify_accept(0, None, None, None, None, None, None, 0)  # nothing to do


def test_noalloc_step_rejects_before_launching(L):
    """decode_step_noalloc checks its arguments and its scratch limit on the host: a null argument is
    VS_ERR_INVALID, and a batch whose workspace exceeds the library's scratch array is VS_ERR_SHAPE,
    both before any device call."""
    dims = vs.vs_model_desc(256, 4, 4, 64, 1024, 1000, 1, vs.VS_F32, 10000.0, 1e-5)
    desc = vs.vs_batch_desc(4, 4, 4, 1, 65, 5, None, None, None, None, None)
    with pytest.raises(vs.VSError) as e:
        vs.decode_step_noalloc(desc, None, vs.vs_weights(dims, None, None, None, None), vs.vs_step_out(), 0)
    assert e.value.status == vs.VS_ERR_INVALID
    # 64 rows of a 32-layer model with a 128256-token vocabulary: the LM head's split-K partial sums
    # alone need more than the scratch array holds
    big = vs.vs_model_desc(4096, 32, 8, 128, 14336, 128256, 32, vs.VS_BF16, 10000.0, 1e-5)
    pdesc = vs.vs_pool_desc(1, 16, 32, 8, 128, vs.VS_BF16)
    nbytes = vs.kv_page_bytes(pdesc)
    buf = ctypes.create_string_buffer(nbytes)
    pool = vs.kv_pool_create(pdesc, ctypes.addressof(buf), nbytes)
    try:
        fake = 4096  # non-null stand-ins: nothing is dereferenced before the size check
        layers = (vs.vs_layer_weights * 32)(*[vs.vs_layer_weights(*([fake] * 9)) for _ in range(32)])
        w = vs.vs_weights(big, fake, fake, fake, ctypes.cast(layers, ctypes.POINTER(vs.vs_layer_weights)))
        bdesc = vs.vs_batch_desc(64, 64, 64, 1, 4100, 257, pool, fake, fake, fake, fake, None)
        need = vs.decode_step_workspace_bytes(bdesc, big)
        assert need > vs.VS_NOALLOC_SCRATCH_BYTES
        out = vs.vs_step_out(fake, fake, None, None, None, None)
        with pytest.raises(vs.VSError) as e:
            vs.decode_step_noalloc(bdesc, fake, w, out, 0)
        assert e.value.status == vs.VS_ERR_SHAPE and "scratch" in str(e.value)
    finally:
        vs.kv_pool_destroy(pool)
