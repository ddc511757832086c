"""Oracle model of the host page pool.  Test infrastructure only.

Semantics, from the pages:
  * AstrAI cache.py, PagedCache.alloc / alloc_n / free: a page is free while
    its reference count is zero; ``alloc`` hands out the lowest free page and
    sets its count to one, or fails when none is free; ``alloc_n`` is
    all-or-nothing (a partial grant is rolled back); ``free`` drops one
    reference and the page is free again at zero.
  * libmir-metal paged/mod.rs, PagedStore::snapshot / release: a fork adds one
    reference to every page it shares; release drops one per page.
  * tiny-llm paged_kv.py, BlockAllocator.free: freeing a page that is not in
    use is an error (the AstrAI pool would drive the count negative).
"""
from __future__ import annotations


class PoolError(Exception):
    pass


class PoolModel:
    def __init__(self, n_pages: int):
        self.refs = [0] * n_pages

    def alloc(self) -> int:
        for i, r in enumerate(self.refs):
            if r == 0:
                self.refs[i] = 1
                return i
        return -1

    def alloc_n(self, n: int):
        free = [i for i, r in enumerate(self.refs) if r == 0]
        if n > len(free):
            return None
        got = free[:n]
        for i in got:
            self.refs[i] = 1
        return got

    def retain(self, i: int) -> None:
        if self.refs[i] == 0:
            raise PoolError(f"page {i} is not in use")
        self.refs[i] += 1

    def release(self, i: int) -> None:
        if self.refs[i] == 0:
            raise PoolError(f"page {i} released twice (or never allocated)")
        self.refs[i] -= 1

    def num_free(self) -> int:
        return sum(1 for r in self.refs if r == 0)

    def refcount(self, i: int) -> int:
        return self.refs[i]
