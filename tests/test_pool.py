"""The library's page pool against the oracle's pool model, on the CPU.

Random sequences of alloc / share / free / append (and bad calls) run on both
the C pool (kv_* through the C ABI) and oracle.PoolModel ([KV Cache] section
05: block table, reference counts, a new block only when the last is full,
copy-on-write of a shared block). The two may pick different physical ids,
so the test keeps a bijection between them, fixed when pages are handed out,
and compares reference counts, free counts, table lengths and every
accept / reject decision. The pool here sits on a host buffer that no call
touches: forks happen only at page boundaries, where an append never needs a
device copy. The library's copy-on-write runs on the GPU (tests/test_gpu_tiny.py);
the oracle's copy-on-write rule is worked by hand in the last test below.
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


def test_pool_model_copy_on_write_of_a_shared_partial_block():
    """The oracle's copy-on-write rule, worked by hand ([KV Cache] section 05, "Block sharing and
    copy-on-write"; [Serving Efficiency] section 31.3): a sequence about to write into a partly filled
    last block that another sequence also references first copies it to a fresh page and writes there;
    a full block is never written again, so it stays shared; a new block is taken only when the last
    one is full. Pages are handed out lowest id first, so every id and count below is fixed."""
    m = oracle.PoolModel(8, T)
    a = m.alloc(2)  # A holds 20 tokens: page 0 full, page 1 with 4 of 16 slots
    assert a == [0, 1]
    assert m.share(a)  # B forks A after 20 tokens
    assert [m.refcount(p) for p in range(8)] == [2, 2, 0, 0, 0, 0, 0, 0]

    # B appends 3 tokens (positions 20..22): its last block is shared and partly filled
    tb, copies = m.append(a, 20, 3)
    assert tb == [0, 2] and copies == [(1, 2)]  # page 1's slots go to page 2, B writes there
    assert [m.refcount(p) for p in range(8)] == [2, 1, 1, 0, 0, 0, 0, 0]

    # A's last block is now its own: no copy; positions 20..32 fill page 1 and open page 3
    ta, copies = m.append(a, 20, 13)
    assert ta == [0, 1, 3] and copies == []
    assert [m.refcount(p) for p in range(8)] == [2, 1, 1, 1, 0, 0, 0, 0]

    # C forks A at the page boundary (16 tokens): the shared block is full, so appending takes a new
    # page and copies nothing; the full block stays shared three ways
    assert m.share([0])
    tc, copies = m.append([0], 16, 5)
    assert tc == [0, 4] and copies == []
    assert [m.refcount(p) for p in range(8)] == [3, 1, 1, 1, 1, 0, 0, 0]

    # appending nothing to a shared partial block copies nothing
    assert m.share([0, 2])  # D forks B after 23 tokens (page 2 holds 7)
    assert m.append([0, 2], 23, 0) == ([0, 2], [])
    assert [m.refcount(p) for p in range(8)] == [4, 1, 2, 1, 1, 0, 0, 0]

    # with no free page the copy cannot be made: the append fails and changes nothing
    assert m.alloc(3) == [5, 6, 7] and m.num_free() == 0
    before = [m.refcount(p) for p in range(8)]
    assert m.append([0, 2], 23, 1) is None
    assert [m.refcount(p) for p in range(8)] == before

    # one page freed: the copy goes there, and B alone holds page 2 again
    assert m.free([7])
    td, copies = m.append([0, 2], 23, 1)
    assert td == [0, 7] and copies == [(2, 7)]
    assert [m.refcount(p) for p in range(8)] == [4, 1, 1, 1, 1, 1, 1, 1]

    # a copy plus further pages in one append: E forks C after 21 tokens and appends 30 (positions
    # 21..50 need ceil(51 / 16) = 4 pages: the copy of page 4 and two new ones, three free pages)
    assert m.free([3, 5, 6])
    assert m.share([0, 4])
    te, copies = m.append([0, 4], 21, 30)
    assert te == [0, 3, 5, 6] and copies == [(4, 3)]
    assert [m.refcount(p) for p in range(8)] == [5, 1, 1, 1, 1, 1, 1, 1]
