"""The library's page pool against the oracle's pool model, on the CPU.

Random sequences of alloc / share / free / append (and bad calls) run on both
the C pool (kv_* through the C ABI) and oracle.PoolModel ([KV Cache] section
05: block table, reference counts, a new block only when the last is full,
copy-on-write of a shared block). The two may pick different physical ids,
so the test keeps a bijection between them, fixed when pages are handed out,
and compares reference counts, free counts, table lengths and every
accept / reject decision. The pool here sits on a host buffer that no call
touches: forks happen only at page boundaries, where an append never needs a
device copy (copy-on-write is exercised on the GPU).
"""
import ctypes
import os
import random

import pytest

import oracle
import verify_step_amd as vs
from verify_step_amd import build as vsbuild

T = 16


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(vs.LIB_PATH):
        vsbuild.build()
    return vs.lib()


class Pair:
    """The C pool and the oracle model side by side, with the id bijection between them."""

    def __init__(self, n_pages):
        self.desc = vs.vs_pool_desc(n_pages, T, 1, 1, 64, vs.VS_F32)
        nbytes = n_pages * vs.kv_page_bytes(self.desc)
        self.buf = ctypes.create_string_buffer(nbytes)
        self.h = vs.kv_pool_create(self.desc, ctypes.addressof(self.buf), nbytes)
        self.m = oracle.PoolModel(n_pages, T)
        self.c2o = {}
        self.o2c = {}
        self.n = n_pages

    def close(self):
        vs.kv_pool_destroy(self.h)

    def bind(self, c_ids, o_ids):
        assert len(c_ids) == len(o_ids)
        assert len(set(c_ids)) == len(c_ids), "C pool handed out a page twice"
        for c, o in zip(c_ids, o_ids):
            assert 0 <= c < self.n
            assert vs.kv_refcount(self.h, c) == 1
            assert self.m.refcount(o) == 1
            # pages that came back to a free list may be handed out again: drop their old pairing
            if c in self.c2o:
                self.o2c.pop(self.c2o[c], None)
            if o in self.o2c:
                self.c2o.pop(self.o2c[o], None)
            self.c2o[c] = o
            self.o2c[o] = c

    def check(self):
        assert vs.kv_num_free(self.h) == self.m.num_free()
        for c, o in self.c2o.items():
            assert vs.kv_refcount(self.h, c) == self.m.refcount(o), (c, o)


def _status(fn):
    try:
        return 0, fn()
    except vs.VSError as e:
        return e.status, None


def test_random_operation_sequences_match_the_pool_model(L):
    rng = random.Random(4006)
    for trial in range(20):
        P = Pair(rng.choice([8, 24, 64]))
        seqs = []  # (C table, oracle table, length)
        for step in range(300):
            op = rng.random()
            if op < 0.25:  # a new sequence with some context
                n_tok = rng.randint(0, 5 * T)
                n_pg = -(-n_tok // T)
                st, ids = _status(lambda: vs.kv_alloc(P.h, n_pg))
                got = P.m.alloc(n_pg)
                assert (st == 0) == (got is not None), (st, got)
                if st == 0:
                    assert st == 0
                    P.bind(ids, got)
                    seqs.append((ids, got, n_tok))
                else:
                    assert st == vs.VS_ERR_OOM
            elif op < 0.55 and seqs:  # append tokens to a sequence
                i = rng.randrange(len(seqs))
                ct, ot, n_tok = seqs[i]
                n_new = rng.randint(0, 2 * T)
                res = P.m.append(list(ot), n_tok, n_new) if n_tok % T == 0 or P.m.refcount(ot[-1]) == 1 else "cow"
                if res == "cow":
                    continue  # would need a device copy; covered on the GPU
                st, new_ct = _status(lambda: vs.kv_append(P.h, ct, 64, n_tok, n_new))
                assert (st == 0) == (res is not None), (st, res)
                if st == 0:
                    new_ot, copies = res
                    assert copies == []
                    assert new_ct[:len(ct)] == ct and new_ot[:len(ot)] == ot
                    P.bind(new_ct[len(ct):], new_ot[len(ot):])
                    seqs[i] = (new_ct, new_ot, n_tok + n_new)
                else:
                    assert st == vs.VS_ERR_OOM
            elif op < 0.65 and seqs:  # fork a sequence at a page boundary (prefix sharing)
                i = rng.randrange(len(seqs))
                ct, ot, n_tok = seqs[i]
                keep = (n_tok // T) * T
                kp = keep // T
                vs.kv_share(P.h, ct[:kp])
                assert P.m.share(ot[:kp])
                seqs.append((ct[:kp], ot[:kp], keep))
            elif op < 0.85 and seqs:  # a sequence finishes
                i = rng.randrange(len(seqs))
                ct, ot, _ = seqs.pop(i)
                vs.kv_free(P.h, ct)
                assert P.m.free(ot)
            elif op < 0.95:  # bad frees: a page with no reference left, or one dropped too often
                free_c = [c for c in P.c2o if vs.kv_refcount(P.h, c) == 0]
                if free_c:
                    before = [vs.kv_refcount(P.h, c) for c in range(P.n)]
                    st, _ = _status(lambda: vs.kv_free(P.h, [free_c[0]]))
                    assert st == vs.VS_ERR_INVALID
                    assert not P.m.free([P.c2o[free_c[0]]])
                    assert [vs.kv_refcount(P.h, c) for c in range(P.n)] == before
                if seqs:
                    ct, ot, _ = seqs[rng.randrange(len(seqs))]
                    if ct:
                        over = [ct[0]] * (vs.kv_refcount(P.h, ct[0]) + 1)
                        st, _ = _status(lambda: vs.kv_free(P.h, over))
                        assert st == vs.VS_ERR_INVALID
                        assert not P.m.free([ot[0]] * len(over))
            else:  # sharing a free page is refused
                free_c = [c for c in P.c2o if vs.kv_refcount(P.h, c) == 0]
                if free_c:
                    st, _ = _status(lambda: vs.kv_share(P.h, [free_c[0]]))
                    assert st == vs.VS_ERR_INVALID
                    assert not P.m.share([P.c2o[free_c[0]]])
            P.check()
        for ct, ot, _ in seqs:
            vs.kv_free(P.h, ct)
            assert P.m.free(ot)
        P.check()
        assert vs.kv_num_free(P.h) == P.n
        P.close()


def test_append_takes_a_page_only_when_the_last_is_full(L):
    P = Pair(16)
    row = vs.kv_alloc(P.h, 1)
    for cur in range(1, T):  # positions 1..15 fit in the first page
        assert vs.kv_append(P.h, row, 8, cur, 1) == row
    assert vs.kv_num_free(P.h) == 15
    row2 = vs.kv_append(P.h, row, 8, T, 1)  # position 16 opens page 2
    assert len(row2) == 2 and row2[0] == row[0]
    assert vs.kv_num_free(P.h) == 14
    row3 = vs.kv_append(P.h, row2, 8, T + 1, 3 * T)  # positions 17..64: ceil(65 / 16) = 5 pages in all
    assert len(row3) == 5 and row3[:2] == row2 and len(set(row3)) == 5
    assert vs.kv_num_free(P.h) == 11
    P.close()


def test_append_validates_before_changing_anything(L):
    P = Pair(8)
    row = vs.kv_alloc(P.h, 2)
    free0 = vs.kv_num_free(P.h)
    with pytest.raises(vs.VSError) as e:  # table length does not match the length
        vs.kv_append(P.h, row, 8, 40, 1)
    assert e.value.status == vs.VS_ERR_INVALID
    with pytest.raises(vs.VSError) as e:  # the row's capacity is too small
        vs.kv_append(P.h, row, 2, 32, 1)
    assert e.value.status == vs.VS_ERR_SHAPE
    with pytest.raises(vs.VSError) as e:  # more pages than are free
        vs.kv_append(P.h, row, 64, 32, 16 * 7)
    assert e.value.status == vs.VS_ERR_OOM
    with pytest.raises(vs.VSError) as e:  # a table naming a page that is not in use
        vs.kv_append(P.h, [row[0], 7], 8, 32, 1)
    assert e.value.status == vs.VS_ERR_INVALID
    assert vs.kv_num_free(P.h) == free0
    assert [vs.kv_refcount(P.h, p) for p in row] == [1, 1]
    P.close()


def test_alloc_is_all_or_nothing(L):
    P = Pair(8)
    a = vs.kv_alloc(P.h, 5)
    with pytest.raises(vs.VSError) as e:
        vs.kv_alloc(P.h, 4)
    assert e.value.status == vs.VS_ERR_OOM
    assert vs.kv_num_free(P.h) == 3
    b = vs.kv_alloc(P.h, 3)
    assert sorted(a + b) == list(range(8))
    assert vs.kv_refcount(P.h, 8) == -1 and vs.kv_refcount(P.h, -1) == -1
    P.close()
