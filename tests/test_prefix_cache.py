"""Prefix-cache index: oracle pins and the library against the oracle (CPU only).

[KV Cache] section 05 "Prefix caching": every full block is named by a hash of
its own tokens and of its parent block, i.e. of the whole prefix up to it; a
new request that finds a name takes a reference on that block and skips its
prefill. [Serving Efficiency] section 31.3: only an exact prefix from the
first token matches, and the key must also name the computation version (and
stay within the access boundary).
"""
import ctypes
import os
import random

import pytest

from oracle.pool import PoolModel, PrefixIndex, block_hash, fnv1a64, prefix_chain, prefix_root
import verify_step_amd as vs
from verify_step_amd import build as vsbuild

ROOT = prefix_root(b"model=tiny;weights=1001;rope=10000;scope=tenant-a")


# ---------------------------------------------------------------- oracle pins

def test_fnv1a64_published_test_vectors():
    """The FNV authors' published 64-bit FNV-1a values for the empty string, "a" and "foobar"."""
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


@pytest.mark.parametrize("T,shared", [(1, 3), (2, 1), (4, 0)])
def test_chain_shares_exactly_the_common_prefix(T, shared):
    """[Serving Efficiency] section 31.3's requests: A = [10, 11, 12, 13], B = [10, 11, 12, 14] share
    three leading tokens, C = [20, 21] none. With one-token blocks B reuses 3 of A's blocks; with
    two-token blocks only the first full block [10, 11]; with four-token blocks none (the one full
    block differs in its last token)."""
    a, b, c = [10, 11, 12, 13], [10, 11, 12, 14], [20, 21]
    ha, hb, hc = (prefix_chain(ROOT, x, T) for x in (a, b, c))
    assert len(ha) == 4 // T and len(hc) == 2 // T
    n = 0
    while n < min(len(ha), len(hb)) and ha[n] == hb[n]:
        n += 1
    assert n == shared
    assert not set(hc) & set(ha)
    # a block's name covers the whole prefix: the same block tokens after another prefix differ
    assert block_hash(ROOT, [12, 13]) != prefix_chain(ROOT, a, 2)[1]


def test_a_partial_block_has_no_name_and_an_early_change_renames_every_later_block():
    toks = list(range(100, 150))
    h = prefix_chain(ROOT, toks, 16)
    assert len(h) == 3  # 48 of 50 tokens fill three blocks
    moved = prefix_chain(ROOT, [toks[0] + 1] + toks[1:], 16)
    assert all(x != y for x, y in zip(h, moved))


def test_the_version_and_scope_key_separates_caches():
    """Same tokens under another computation version or access scope share nothing."""
    toks = list(range(64))
    other = prefix_root(b"model=tiny;weights=1001;rope=10000;scope=tenant-b")
    assert not set(prefix_chain(ROOT, toks, 16)) & set(prefix_chain(other, toks, 16))
    pool = PoolModel(8, 16)
    idx = PrefixIndex(pool)
    pages = pool.alloc(4)
    idx.insert(ROOT, prefix_chain(ROOT, toks, 16), toks, pages)
    assert idx.lookup(other, prefix_chain(other, toks, 16), toks) == []
    assert len(idx.lookup(ROOT, prefix_chain(ROOT, toks, 16), toks)) == 4


def test_index_references_lookup_and_eviction_by_hand():
    pool = PoolModel(10, 4)
    idx = PrefixIndex(pool)
    a = [1, 2, 3, 4, 5, 6, 7, 8, 9]  # two full blocks and a partial one
    pa = pool.alloc(3)
    ha = prefix_chain(ROOT, a, 4)
    assert idx.insert(ROOT, ha, a, pa[:2]) == 2
    assert [pool.ref[p] for p in pa] == [2, 2, 1]  # the index holds one reference per indexed page
    # B shares the first block only; it takes one reference for itself
    b = [1, 2, 3, 4, 9, 9, 9, 9]
    hb = prefix_chain(ROOT, b, 4)
    got = idx.lookup(ROOT, hb, b)
    assert got == pa[:1] and pool.ref[pa[0]] == 3
    # A finishes and frees its pages: the indexed ones stay allocated, held by the index (and B)
    assert pool.free(pa)
    assert [pool.ref[p] for p in pa] == [2, 1, 0]
    # only entries the index alone holds can go: block 1 of A (block 0 is still B's)
    assert idx.evict(5) == 1 and pool.ref[pa[1]] == 0 and len(idx.entries) == 1
    assert pool.free(got) and idx.evict(5) == 1 and not idx.entries
    # least recently used first; among entries used together, the deeper block first
    c = list(range(20, 32))  # three blocks
    pc = pool.alloc(3)
    hc = prefix_chain(ROOT, c, 4)
    idx.insert(ROOT, hc, c, pc)
    d = list(range(40, 44))
    pd = pool.alloc(1)
    idx.insert(ROOT, prefix_chain(ROOT, d, 4), d, pd)
    pool.free(pc + pd)
    assert idx.evict(2) == 2
    assert sorted(e[2] for e in idx.entries.values()) == sorted([pc[0], pd[0]])  # c's blocks 2, 1 went
    assert idx.lookup(ROOT, hc, c) == pc[:1]  # the trimmed chain still serves its first block


# ---------------------------------------------------------------- the library against the oracle

@pytest.fixture(scope="module")
def L():
    if not os.path.exists(vs.LIB_PATH):
        vsbuild.build()
    return vs.lib()


def test_library_hashes_equal_the_oracle(L):
    rng = random.Random(77)
    for key in (b"", b"v1", bytes(range(256))):
        assert vs.kv_prefix_root(key) == prefix_root(key)
    for T in (1, 4, 16):
        toks = [rng.randrange(-2 ** 31, 2 ** 31) for _ in range(5 * T + 3)]
        assert vs.kv_prefix_chain(ROOT, toks, T) == prefix_chain(ROOT, toks, T)


def test_library_index_matches_the_oracle_on_random_operation_sequences(L):
    """Requests drawn from a few shared prompts arrive, look up their prefix, allocate the rest,
    index their full blocks, and leave; eviction runs when the pool is short. Every lookup, count,
    eviction and reference count must agree with the oracle."""
    T = 4
    rng = random.Random(5150)
    prompts = [[rng.randrange(50) for _ in range(rng.randrange(4, 30))] for _ in range(6)]
    roots = [ROOT, prefix_root(b"another version")]
    for trial in range(8):
        n_pages = 40
        desc = vs.vs_pool_desc(n_pages, T, 1, 1, 64, vs.VS_F32)
        nbytes = n_pages * vs.kv_page_bytes(desc)
        buf = ctypes.create_string_buffer(nbytes)
        h = vs.kv_pool_create(desc, ctypes.addressof(buf), nbytes)
        model = PoolModel(n_pages, T)
        idx = PrefixIndex(model)
        c2o, o2c, live = {}, {}, []  # page id pairing both ways; live sequences (C pages, oracle pages)
        try:
            for step in range(150):
                op = rng.random()
                if op < 0.55 or not live:  # a request arrives
                    root = rng.choice(roots)
                    base = rng.choice(prompts)
                    toks = base[:rng.randrange(len(base) + 1)] + [rng.randrange(50) for _ in range(rng.randrange(6))]
                    hs = vs.kv_prefix_chain(root, toks, T)
                    assert hs == prefix_chain(root, toks, T)
                    hit_c = vs.kv_prefix_lookup(h, root, hs, toks)
                    hit_o = idx.lookup(root, hs, toks)
                    assert [c2o[p] for p in hit_c] == hit_o
                    need = -(-len(toks) // T) - len(hit_c)
                    if need > vs.kv_num_free(h):
                        short = need - vs.kv_num_free(h)
                        assert vs.kv_prefix_evict(h, short) == idx.evict(short)
                    if need > vs.kv_num_free(h):  # still short: give the prefix back
                        vs.kv_free(h, hit_c)
                        assert model.free(hit_o)
                        continue
                    new_c = vs.kv_alloc(h, need)
                    new_o = model.alloc(need)
                    for c, o in zip(new_c, new_o):  # re-pair reused ids on both sides
                        if o in o2c:
                            c2o.pop(o2c.pop(o), None)
                        if c in c2o:
                            o2c.pop(c2o[c], None)
                        c2o[c], o2c[o] = o, c
                    pages_c, pages_o = hit_c + new_c, hit_o + new_o
                    n_full = len(hs)
                    added_c = vs.kv_prefix_insert(h, root, hs, toks[:n_full * T], pages_c[:n_full])
                    added_o = idx.insert(root, hs, toks[:n_full * T], pages_o[:n_full])
                    assert added_c == added_o
                    live.append((pages_c, pages_o))
                elif op < 0.9:  # a request leaves
                    pages_c, pages_o = live.pop(rng.randrange(len(live)))
                    vs.kv_free(h, pages_c)
                    assert model.free(pages_o)
                else:
                    n = rng.randrange(1, 6)
                    assert vs.kv_prefix_evict(h, n) == idx.evict(n)
                assert vs.kv_num_free(h) == model.num_free()
                assert vs.kv_prefix_entries(h) == len(idx.entries)
                for c, o in c2o.items():
                    if model.ref[o] > 0:
                        assert vs.kv_refcount(h, c) == model.ref[o], (trial, step, c, o)
        finally:
            vs.kv_pool_destroy(h)


def test_library_rejects_a_chain_that_is_not_its_tokens(L):
    desc = vs.vs_pool_desc(4, 4, 1, 1, 64, vs.VS_F32)
    nbytes = 4 * vs.kv_page_bytes(desc)
    buf = ctypes.create_string_buffer(nbytes)
    h = vs.kv_pool_create(desc, ctypes.addressof(buf), nbytes)
    try:
        toks = [1, 2, 3, 4]
        pages = vs.kv_alloc(h, 1)
        with pytest.raises(vs.VSError):
            vs.kv_prefix_insert(h, ROOT, [12345], toks, pages)
        with pytest.raises(vs.VSError):  # a page nobody holds
            vs.kv_prefix_insert(h, ROOT, vs.kv_prefix_chain(ROOT, toks, 4), toks, [3])
        assert vs.kv_prefix_entries(h) == 0 and vs.kv_refcount(h, pages[0]) == 1
    finally:
        vs.kv_pool_destroy(h)
