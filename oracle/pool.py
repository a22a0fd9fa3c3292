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


# ---- prefix caching ([KV Cache] section 05 "Prefix caching"; [Serving Efficiency] section 31.3)

FNV64_OFFSET_BASIS = 0xCBF29CE484222325  # the published 64-bit FNV parameters
FNV64_PRIME = 0x100000001B3


def fnv1a64(data: bytes, h: int = FNV64_OFFSET_BASIS) -> int:
    """64-bit FNV-1a: for each byte, xor it in, then multiply by the prime modulo 2^64."""
    for byte in data:
        h ^= byte
        h = (h * FNV64_PRIME) % (1 << 64)
    return h


def prefix_root(key: bytes) -> int:
    """The chain's root: a hash of the key naming the computation version and access scope
    ([Serving Efficiency] section 31.3: the key must identify token content and computation
    version, and reuse stays inside the allowed access boundary)."""
    return fnv1a64(key)


def block_hash(parent: int, tokens: list) -> int:
    """A full block's name: the parent's hash (8 little-endian bytes) followed by the block's token
    ids (4 little-endian bytes each), so it names the whole prefix up to the block ([KV Cache]
    section 05: each full block is identified by its own content plus its parent block's hash)."""
    data = parent.to_bytes(8, "little") + b"".join((t & 0xFFFFFFFF).to_bytes(4, "little") for t in tokens)
    return fnv1a64(data)


def prefix_chain(root: int, tokens: list, page_tokens: int) -> list:
    """Hashes of the full blocks of a token sequence; a partial last block has none."""
    out, h = [], root
    for i in range(len(tokens) // page_tokens):
        h = block_hash(h, tokens[i * page_tokens:(i + 1) * page_tokens])
        out.append(h)
    return out


class PrefixIndex:
    """The prefix-cache index of a PoolModel: chain hash -> the page holding that full block.

    The index keeps one reference on every indexed page. Inserting names a sequence's leading full
    blocks (a block already named keeps its page). Looking up returns the longest run of leading
    blocks that are named, whose stored tokens and parent also match, and takes a reference on each
    for the caller ([KV Cache] section 05: on a match, bump the reference count and skip that part
    of the prefill). Evicting drops entries only the index still holds, least recently used first;
    among entries last used together the deeper block goes first, so a chain is trimmed from its
    end (the order a radix-tree cache evicts leaves first, [KV Cache] section 05).
    """

    def __init__(self, pool: PoolModel):
        self.pool = pool
        self.entries = {}  # hash -> [parent, tokens, page, depth, last_use]
        self.clock = 0

    def insert(self, root: int, hashes: list, tokens: list, pages: list):
        T = self.pool.page_tokens
        for i, (h, p) in enumerate(zip(hashes, pages)):
            if not (0 <= p < self.pool.num_pages) or self.pool.ref[p] == 0:
                return None
            if block_hash(root if i == 0 else hashes[i - 1], tokens[i * T:(i + 1) * T]) != h:
                return None
        self.clock += 1
        added = 0
        for i, (h, p) in enumerate(zip(hashes, pages)):
            if h in self.entries:
                self.entries[h][4] = self.clock
                continue
            self.entries[h] = [root if i == 0 else hashes[i - 1], list(tokens[i * T:(i + 1) * T]), p, i, self.clock]
            self.pool.ref[p] += 1
            added += 1
        return added

    def lookup(self, root: int, hashes: list, tokens: list) -> list:
        T = self.pool.page_tokens
        self.clock += 1
        hit = []
        for i, h in enumerate(hashes):
            e = self.entries.get(h)
            if e is None or e[0] != (root if i == 0 else hashes[i - 1]) or e[1] != list(tokens[i * T:(i + 1) * T]):
                break
            hit.append(e)
        for e in hit:
            e[4] = self.clock
            self.pool.ref[e[2]] += 1
        return [e[2] for e in hit]

    def evict(self, n_pages: int) -> int:
        cands = sorted((e[4], -e[3], h) for h, e in self.entries.items() if self.pool.ref[e[2]] == 1)
        freed = 0
        for _, _, h in cands[:n_pages]:
            page = self.entries.pop(h)[2]
            self.pool.ref[page] = 0
            freed += 1
        return freed
