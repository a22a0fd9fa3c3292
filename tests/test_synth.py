"""The seeded input generator: determinism, counter slicing, rounding, distribution (CPU only)."""
import numpy as np
import pytest
import torch

import synth
from synth import workloads as W


def test_key_depends_on_seed_and_tags():
    assert synth.key(1, 2, 3) == synth.key(1, 2, 3)
    assert len({synth.key(1, 2, 3), synth.key(1, 3, 2), synth.key(2, 2, 3), synth.key(1, 2)}) == 4


def test_splitmix64_reference_values():
    # SplitMix64 seeded with 0: the published first outputs of the generator
    k = 0
    assert int(synth.raw(k, 0, 1)[0]) == 0xE220A8397B1DCDAF
    assert int(synth.raw(k, 1, 1)[0]) == 0x6E789E6AA1B965F4


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_counter_slices_agree_with_the_full_stream(dtype):
    k = synth.key(7, 1)
    full = synth.normal(k, 0, 1001, 0.0, 1.0, dtype)
    for a, b in [(0, 1), (1, 2), (3, 500), (499, 1001), (1000, 1001)]:
        part = synth.normal(k, a, b - a, 0.0, 1.0, dtype)
        assert torch.equal(part.view(torch.int16) if dtype != "f32" else part,
                           full[a:b].view(torch.int16) if dtype != "f32" else full[a:b])


def test_half_and_bfloat_rounding_match_library_conversions():
    """The C converters (fp32 -> binary16 / bfloat16, nearest-even) agree bit for bit with
    torch's on values spanning subnormals, normals and overflow."""
    k = synth.key(3)
    for std in [1e-8, 1e-7, 3e-6, 3e-5, 0.02, 1.0, 300.0, 2e4, 7e4]:
        a = synth.normal(k, 0, 20000, 0.0, std, "f32")
        h = synth.normal(k, 0, 20000, 0.0, std, "f16")
        b = synth.normal(k, 0, 20000, 0.0, std, "bf16")
        assert torch.equal(a.to(torch.float16).view(torch.int16), h.view(torch.int16)), std
        assert torch.equal(a.to(torch.bfloat16).view(torch.int16), b.view(torch.int16)), std


def test_normal_moments():
    x = synth.normal(synth.key(11), 0, 400000, 0.0, 0.02, "f32").double()
    assert abs(float(x.mean())) < 5 * 0.02 / np.sqrt(400000)
    assert float(x.std()) == pytest.approx(0.02, rel=0.01)
    # fourth standardised moment of a normal is 3
    z = x / 0.02
    assert float((z ** 4).mean()) == pytest.approx(3.0, rel=0.05)


def test_uniform_int_range_and_balance():
    v = synth.uniform_int(synth.key(5), 0, 100000, 0, 1000)
    assert v.min() >= 0 and v.max() < 1000
    counts = np.bincount(v, minlength=1000)
    assert counts.min() > 40 and counts.max() < 170


def test_permutation_is_a_permutation():
    p = synth.permutation(synth.key(9), 64)
    assert sorted(p.tolist()) == list(range(64))


def test_kv_block_slices_agree():
    dims = W.TINY
    full = W.kv_block(dims, 2001, content=4, p0=0, p1=40)
    part = W.kv_block(dims, 2001, content=4, p0=17, p1=33)
    assert torch.equal(full[:, :, 17:33], part)
    other = W.kv_block(dims, 2001, content=5, p0=17, p1=33)
    assert not torch.equal(other, part)


def test_weights_deterministic_and_shaped():
    a = W.make_weights(W.TINY, 1001)
    b = W.make_weights(W.TINY, 1001)
    assert a["embed"].shape == (1000, 256) and a["lm_head"].shape == (1000, 256)
    assert a["layers"][0]["wq"].shape == (256, 256) and a["layers"][0]["wd"].shape == (256, 1024)
    assert torch.equal(a["layers"][0]["wg"], b["layers"][0]["wg"])
    assert not torch.equal(a["layers"][0]["wg"], a["layers"][0]["wu"])
    assert torch.equal(a["final_norm"], torch.ones(256))
