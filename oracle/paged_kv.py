"""Page allocator and page tables of the paged KV cache (oracle; test infrastructure only).

The pages name a paged KV cache (wiki note, *TL;DR* and *Key claims*; GeekNews,
*Serving (SGLang)*), and a rejection makes the next block resume from the rejected
position, so the cache is rolled back to the committed length (wiki note, *Method*).
They give no allocator; page tables must nevertheless be bit-identical between the oracle and
the GPU, so a deterministic one is fixed here:

* a LIFO free stack, stack[0 .. n_free), top at n_free - 1, initialised so that the
  first pops return pages 0, 1, 2, ...;
* a step first reserves, for every live slot in ascending slot order, the pages
  that positions L .. L + q_len - 1 need, popping one page per new logical page in
  ascending logical order;
* after the step's decisions every slot, in ascending slot order, frees the pages
  whose logical index is >= ceil(L'/P) (all of them for a finished slot), pushing
  them in ascending logical order.

Pinned by invariants (no page owned twice, pages in use = sum ceil(len/P),
free + used = pool) and by a hand-worked example in tests/golden.
"""
import numpy as np


def pages_for(length, page_size):
    return -(-int(length) // page_size)


class PagePool:
    def __init__(self, n_pages, page_size):
        self.n_pages = int(n_pages)
        self.P = int(page_size)
        self.stack = list(range(self.n_pages - 1, -1, -1))   # top = last element = page 0
        self.tables = {}                                      # slot -> list of page ids

    @property
    def n_free(self):
        return len(self.stack)

    def table(self, slot):
        return self.tables.setdefault(slot, [])

    def reserve(self, slot, length):
        """Grow slot's table so that it covers `length` tokens."""
        t = self.table(slot)
        need = pages_for(length, self.P) - len(t)
        if need > len(self.stack):
            raise MemoryError("KV page pool exhausted")
        for _ in range(max(0, need)):
            t.append(self.stack.pop())

    def truncate(self, slot, length):
        """Free the slot's pages beyond `length` tokens, ascending logical order."""
        t = self.table(slot)
        keep = pages_for(length, self.P)
        for pg in t[keep:]:
            self.stack.append(pg)
        del t[keep:]

    def check(self, lengths):
        """Invariants: every page is either free or owned by exactly one slot."""
        owned = [p for t in self.tables.values() for p in t]
        assert len(set(owned)) == len(owned), "page owned twice"
        assert not (set(owned) & set(self.stack)), "page both free and owned"
        assert len(owned) + len(self.stack) == self.n_pages, "page lost"
        for slot, n in lengths.items():
            assert len(self.table(slot)) == pages_for(n, self.P)

    def table_array(self, slot, width, fill=-1):
        a = np.full(width, fill, dtype=np.int32)
        t = self.table(slot)
        a[:len(t)] = t
        return a
