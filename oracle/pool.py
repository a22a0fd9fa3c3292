"""Reference model of the paged KV cache's block bookkeeping.

TEST INFRASTRUCTURE (see oracle/__init__.py). A dictionary-and-list model,
slow and obvious, of the rules the pages state for a paged KV cache:

* [KV Cache] section 05 "The block table": the cache is split into blocks of
  a fixed number of token slots (16 by default); each request sees logical
  blocks that a per-request table maps to physical blocks anywhere in memory;
  a new block is taken only once the last block is full.
* [KV Cache] section 05 "Block sharing and copy-on-write": every physical
  block carries a reference count; sharers of a prompt's blocks point at the
  same physical blocks, and a sharer that must write into a shared block first
  copies it and writes into its own copy.
* [Serving Efficiency] section 31.3: an engine can share physical blocks of an
  exact common prefix and copy a block when one branch appends.
* [KV Cache] section 03 "The memory budget of a GPU": the KV region is what is
  left after the weights, carved into fixed-size blocks.
"""
from __future__ import annotations


class PoolModel:
    def __init__(self, num_pages: int, page_tokens: int = 16):
        self.num_pages = num_pages
        self.page_tokens = page_tokens
        self.ref = [0] * num_pages

    # --- queries ---
    def num_free(self) -> int:
        return sum(1 for r in self.ref if r == 0)

    def refcount(self, page: int) -> int:
        return self.ref[page]

    @staticmethod
    def pages_for(n_tokens: int, page_tokens: int = 16) -> int:
        """Blocks a sequence of n tokens occupies: ceil(n / page_tokens)."""
        return -(-n_tokens // page_tokens)

    # --- operations ---
    def alloc(self, n: int) -> list | None:
        """Take n free pages, all or none; each starts with one reference."""
        free = [p for p, r in enumerate(self.ref) if r == 0]
        if len(free) < n:
            return None
        for p in free[:n]:
            self.ref[p] = 1
        return free[:n]

    def share(self, pages: list) -> bool:
        if any(self.ref[p] == 0 for p in pages):
            return False
        for p in pages:
            self.ref[p] += 1
        return True

    def free(self, pages: list) -> bool:
        need = {}
        for p in pages:
            need[p] = need.get(p, 0) + 1
        if any(self.ref[p] < c for p, c in need.items()):
            return False
        for p in pages:
            self.ref[p] -= 1
        return True

    def append(self, table: list, cur_len: int, n_new: int):
        """Make room for positions [cur_len, cur_len + n_new) of a sequence.

        Returns (new_table, copies) where copies lists (src_page, dst_page) block
        copies the caller must perform, or None when the pool is exhausted (state
        unchanged). A partly filled last block that other sequences also reference
        is copied before this sequence writes into it; a full block is never
        written again, so it stays shared.
        """
        T = self.page_tokens
        have = len(table)
        assert have == self.pages_for(cur_len, T), "table does not match the sequence length"
        need_total = self.pages_for(cur_len + n_new, T)
        cow = n_new > 0 and cur_len % T != 0 and self.ref[table[-1]] > 1
        n_alloc = (need_total - have) + (1 if cow else 0)
        got = self.alloc(n_alloc)
        if got is None:
            return None
        table = list(table)
        copies = []
        if cow:
            old = table[-1]
            new = got.pop(0)
            copies.append((old, new))
            self.ref[old] -= 1
            table[-1] = new
        table.extend(got)
        return table, copies
