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


_MASK64 = (1 << 64) - 1


def splitmix64(seed: int, n: int) -> list[int]:
    """The first n outputs of SplitMix64 seeded with ``seed`` (Steele, Lea and
    Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014, as
    in Vigna's reference splitmix64.c): the state advances by the golden-ratio
    gamma 0x9e3779b97f4a7c15 per output and each output is the state passed
    through the variant-13 finalizer (xor-shift 30, multiply, xor-shift 27,
    multiply, xor-shift 31)."""
    out, state = [], seed & _MASK64
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        out.append(z ^ (z >> 31))
    return out


class PoolModel:
    """``shuffle_seed`` 0 hands out the lowest free page (AstrAI's rule).
    Otherwise page i is ranked by output i of SplitMix64 seeded with
    ``shuffle_seed`` (ties by page id), and the free page of lowest rank
    goes first: a fresh pool hands out a seeded permutation of its pages.
    This ordering is the build's own choice (the pages name no shuffled
    allocator); what the pages fix is only that any order is allowed."""

    def __init__(self, n_pages: int, shuffle_seed: int = 0):
        self.refs = [0] * n_pages
        if shuffle_seed:
            draws = splitmix64(shuffle_seed, n_pages)
            self.order = sorted(range(n_pages), key=lambda i: (draws[i], i))
        else:
            self.order = list(range(n_pages))

    def alloc(self) -> int:
        for i in self.order:
            if self.refs[i] == 0:
                self.refs[i] = 1
                return i
        return -1

    def alloc_n(self, n: int):
        free = [i for i in self.order if self.refs[i] == 0]
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


class SeqError(Exception):
    pass


class SeqModel:
    """Oracle model of block tables over a PoolModel.  Test infrastructure only.

    Semantics, from the pages:
      * tiny-llm paged_kv.py (module docstring, begin_step): a sequence holds
        ceil(len / page_size) pages in table order and gets a new one when its
        length crosses a page boundary; pages come from the pool, lowest free
        first (AstrAI cache.py PagedCache.alloc).
      * libmir-metal paged/mod.rs PagedStore::snapshot: a fork shares every
        page of its source (one more reference each) and its length.
      * Copy-on-write (implied by sharing a partly filled page; the pages do
        not print it): a write into a page that another sequence also holds
        goes to a fresh page, which first receives a copy of the shared one;
        the writer drops its reference to the shared page.
      * tiny-llm paged_kv.py reserve_step: while the next step's new pages
        exceed the free ones, the sequence admitted last is preempted (its
        pages released, its length 0); victims newest first.
    Appends over a batch are all or nothing and run in sequence order.
    """

    def __init__(self, pool: PoolModel, batch: int, stride: int, page_size: int):
        self.pool, self.batch, self.stride, self.bs = pool, batch, stride, page_size
        self.pages = [[] for _ in range(batch)]
        self.lens = [0] * batch
        self.admitted = [0] * batch  # admission number, 0 = empty
        self.admits = 0
        self.copies: list[tuple[int, int]] = []

    def _admit(self, b: int) -> None:
        if self.lens[b] > 0 and self.admitted[b] == 0:
            self.admits += 1
            self.admitted[b] = self.admits

    def _state(self):
        return ([list(p) for p in self.pages], list(self.lens), list(self.admitted), self.admits,
                list(self.copies), list(self.pool.refs))

    def _restore(self, st) -> None:
        (self.pages, self.lens, self.admitted, self.admits, self.copies, self.pool.refs) = (
            [list(p) for p in st[0]], list(st[1]), list(st[2]), st[3], list(st[4]), list(st[5]))

    def _append_one(self, b: int, n: int) -> None:
        if n < 0:
            raise SeqError("negative append")
        if n == 0:
            return
        pos = self.lens[b]  # the first token written
        if pos % self.bs and self.pool.refcount(self.pages[b][-1]) > 1:
            fresh = self.pool.alloc()
            if fresh < 0:
                raise PoolError("pool exhausted")
            old = self.pages[b][-1]
            self.copies.append((old, fresh))
            self.pages[b][-1] = fresh
            self.pool.release(old)
        need = -(-(pos + n) // self.bs)
        while len(self.pages[b]) < need:
            p = self.pool.alloc()
            if p < 0:
                raise PoolError("pool exhausted")
            self.pages[b].append(p)
        self.lens[b] = pos + n
        self._admit(b)

    def append_all(self, ns) -> None:
        for b in range(self.batch):
            if -(-(self.lens[b] + ns[b]) // self.bs) > self.stride:
                raise SeqError(f"sequence {b} would overflow its table row")
        st = self._state()
        try:
            for b in range(self.batch):
                self._append_one(b, int(ns[b]))
        except (PoolError, SeqError):
            self._restore(st)
            raise

    def append(self, b: int, n: int) -> None:
        ns = [0] * self.batch
        ns[b] = n
        self.append_all(ns)

    def fork(self, dst: int, src: int) -> None:
        if self.pages[dst] or self.lens[dst] or dst == src:
            raise SeqError("fork needs an empty, different destination")
        for p in self.pages[src]:
            self.pool.retain(p)
        self.pages[dst] = list(self.pages[src])
        self.lens[dst] = self.lens[src]
        self._admit(dst)

    def share(self, dst: int, src: int, n_pages: int) -> None:
        if self.pages[dst] or dst == src or n_pages * self.bs > self.lens[src]:
            raise SeqError("share needs an empty destination and full source pages")
        for p in self.pages[src][:n_pages]:
            self.pool.retain(p)
        self.pages[dst] = list(self.pages[src][:n_pages])
        self.lens[dst] = n_pages * self.bs
        self._admit(dst)

    def release(self, b: int) -> None:
        for p in self.pages[b]:
            self.pool.release(p)
        self.pages[b] = []
        self.lens[b] = 0
        self.admitted[b] = 0

    def _pages_needed(self, ns) -> int:
        """Pages the appends would take, found by running them on a copy of
        the state whose pool has room for all of them."""
        trial = SeqModel(PoolModel(len(self.pool.refs)), self.batch, self.stride, self.bs)
        trial.pool.refs = list(self.pool.refs) + [0] * sum(
            -(-int(n) // self.bs) + 1 for n in ns)
        trial.pool.order = list(range(len(trial.pool.refs)))  # the count ignores the order
        trial.pages = [list(p) for p in self.pages]
        trial.lens = list(self.lens)
        before = trial.pool.num_free()
        trial.append_all(ns)
        return before - trial.pool.num_free()

    def reserve(self, ns) -> list[int]:
        ns = [int(x) for x in ns]
        victims = []
        while self._pages_needed(ns) > self.pool.num_free():
            live = [b for b in range(self.batch) if self.lens[b] > 0]
            if not live:
                break
            v = max(live, key=lambda b: self.admitted[b])
            self.release(v)
            ns[v] = 0
            victims.append(v)
        return victims

    def take_copies(self) -> list[tuple[int, int]]:
        out, self.copies = self.copies, []
        return out
