"""Pure-Python model of the KV block manager.  TEST INFRASTRUCTURE ONLY.

The pages describe the manager's job, not its API:

* The KV cache is cut into fixed-size blocks that need not be contiguous; a per-
  request block table maps logical blocks to physical ones; a block is taken only
  when needed and all of a request's blocks are returned when it ends -- "vLLM
  explained" (jackchen890311.github.io), PagedAttention section, items 1-4, and the
  table on when KV may be overwritten (released at once without prefix caching);
  "LLM inference optimization" (carlstack.gravito.dev), section 三.1 and section 四
  (blocks released as soon as a request finishes).
* Several logical sequences may point at one physical block, each holder adding one
  to its reference count; a shared block is copied only when a branch first writes
  a different token into it (copy-on-write) -- carlstack page, section 三.2 and the
  block-table panel of Fig. 1 (request 2 shares physical block 7 with request 1).

Where the pages are silent this model takes these readings:

* Free list: a LIFO stack.  ``initial_free_order`` lists the pop order (first
  element is popped first); the default is 0, 1, 2, ...  Freed blocks are pushed in
  logical order, so a sequence's last block is the next one popped.
* Append of ``n`` tokens to a sequence of length ``L``: token positions
  ``L .. L+n-1``.  If ``L % bs != 0`` (the last block is partial) and that block's
  reference count is above one, copy-on-write happens first: pop ``p'``, emit the
  pair ``(p, p')``, drop one reference from ``p``, give ``p'`` one reference and put
  it in the table.  Full blocks are never copied.  Then every position with
  ``pos % bs == 0`` pops a fresh block.  Token ``pos`` gets
  ``slot = table[pos // bs] * bs + pos % bs``.
* All-or-nothing: if the free stack cannot cover every pop an append needs, the
  append raises ``OutOfBlocks`` and nothing changes.
* Fork: the child gets a copy of the parent's table and length; every block gains
  one reference.  Sequence ids are 0, 1, 2, ... and are never reused.
* Free: references are dropped in logical order; each block that reaches zero is
  pushed onto the free stack.
"""


class OutOfBlocks(Exception):
    """The free stack cannot cover an append; the manager is unchanged."""


class BlockManagerModel:
    def __init__(self, num_blocks, block_size, initial_free_order=None):
        if initial_free_order is None:
            initial_free_order = range(num_blocks)
        order = [int(b) for b in initial_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_free_order must be a permutation of the block ids")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.stack = list(reversed(order))      # top of stack = end of the list
        self.refcount = [0] * num_blocks
        self.tables = {}                        # live sequence id -> list of block ids
        self.lengths = {}                       # live sequence id -> token count
        self.next_id = 0

    # -- queries -----------------------------------------------------------------
    def free_stack_top_first(self):
        """Free blocks in the order they would be popped."""
        return list(reversed(self.stack))

    def num_free(self):
        return len(self.stack)

    def table(self, seq):
        return list(self.tables[seq])

    def length(self, seq):
        return self.lengths[seq]

    # -- operations --------------------------------------------------------------
    def seq_new(self):
        seq = self.next_id
        self.next_id += 1
        self.tables[seq] = []
        self.lengths[seq] = 0
        return seq

    def seq_append(self, seq, n):
        """Append ``n`` tokens; returns ``(slots, cow_pairs)``."""
        if seq not in self.tables:
            raise KeyError(seq)
        if n < 0:
            raise ValueError(n)
        bs = self.block_size
        L = self.lengths[seq]
        table = self.tables[seq]
        needs_cow = n > 0 and L % bs != 0 and self.refcount[table[-1]] > 1
        fresh = sum(1 for pos in range(L, L + n) if pos % bs == 0)
        if fresh + int(needs_cow) > len(self.stack):
            raise OutOfBlocks()
        cow_pairs = []
        if needs_cow:
            old = table[-1]
            new = self.stack.pop()
            cow_pairs.append((old, new))
            self.refcount[old] -= 1
            self.refcount[new] = 1
            table[-1] = new
        slots = []
        for pos in range(L, L + n):
            if pos % bs == 0:
                blk = self.stack.pop()
                self.refcount[blk] = 1
                table.append(blk)
            slots.append(table[pos // bs] * bs + pos % bs)
        self.lengths[seq] = L + n
        return slots, cow_pairs

    def seq_fork(self, parent):
        if parent not in self.tables:
            raise KeyError(parent)
        child = self.seq_new()
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for blk in self.tables[child]:
            if blk >= 0:
                self.refcount[blk] += 1
        return child

    def seq_free(self, seq):
        if seq not in self.tables:
            raise KeyError(seq)
        for blk in self.tables[seq]:
            if blk < 0:
                continue
            self.refcount[blk] -= 1
            if self.refcount[blk] == 0:
                self.stack.append(blk)
        del self.tables[seq]
        del self.lengths[seq]

    def seq_release_before(self, seq, token):
        """A sliding window has moved past ``token``: drop this sequence's hold on every
        block whose tokens all come before it ("vLLM explained", table of when KV may be
        overwritten: KV outside a sliding window can be dropped).  The last block is
        always kept (it holds the newest token).  Dropped entries become -1.  Returns the
        number of entries dropped now."""
        if seq not in self.tables or token < 0:
            raise KeyError(seq)
        table = self.tables[seq]
        dropped = 0
        for j in range(len(table) - 1):
            if (j + 1) * self.block_size > token:
                break
            blk = table[j]
            if blk < 0:
                continue
            self.refcount[blk] -= 1
            if self.refcount[blk] == 0:
                self.stack.append(blk)
            table[j] = -1
            dropped += 1
        return dropped

    def export_tables(self, seqs, max_blocks):
        """``(tables, context_lens)``: ``[n][max_blocks]`` padded with -1, and lengths."""
        tables, lens = [], []
        for seq in seqs:
            row = self.tables[seq]
            if len(row) > max_blocks:
                raise ValueError("max_blocks too small")
            tables.append(row + [-1] * (max_blocks - len(row)))
            lens.append(self.lengths[seq])
        return tables, lens

    # -- invariants --------------------------------------------------------------
    def check_invariants(self):
        """Conservation of references and of blocks; raises AssertionError if broken."""
        held = {}
        for row in self.tables.values():
            for blk in row:
                if blk >= 0:
                    held[blk] = held.get(blk, 0) + 1
        for blk in range(self.num_blocks):
            assert self.refcount[blk] == held.get(blk, 0), blk
        free = set(self.stack)
        assert len(free) == len(self.stack), "a block is on the free stack twice"
        assert all(self.refcount[b] == 0 for b in free)
        assert len(free) + sum(1 for r in self.refcount if r > 0) == self.num_blocks
        for seq, row in self.tables.items():
            assert len(row) == -(-self.lengths[seq] // self.block_size)
