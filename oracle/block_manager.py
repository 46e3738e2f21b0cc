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

Automatic prefix caching ("vLLM explained", section on prefix caching): the cache
lives in the same pool; a block is in use (reference count > 0), free and empty, or
free but holding cached content; a request takes empty blocks first and only then
evicts free cached blocks, least recently used first; blocks in use are never evicted.
Readings where the pages are silent:

* A full block's identity is the tuple of its sequence's token ids from the first
  token through the block's last one (this model keys a dict on exactly that tuple).
  Only full blocks are cached.
* A block is registered when an append fills it, if every token of the sequence was
  appended with its id and no block has that identity yet.  An append without ids
  stops registration for the rest of the sequence's life (forks inherit this).
* A new sequence with a prompt takes cached blocks (in use or free) for the prompt's
  leading full blocks while their identities are cached, at most
  ``(len(prompt) - 1) // block_size`` of them.
* A block whose count reaches zero goes to the most-recent end of the LRU list if it
  is cached, else onto the free stack.  With prefix caching on, free and release
  drop references from the last logical block to the first.  Eviction forgets the
  block's identity.

Swap preemption ("vLLM explained", table on when KV may be overwritten: a preempted
request's KV is recomputed later or moved to CPU memory).  Readings:

* A swap space of host blocks, LIFO free stack (0 first), its own reference counts.
* Swapping out a list of sequences gives each distinct device block in their tables
  one host block, in order of first use (sequence order, then logical order), and
  reports (device, host) pairs; tables then name host blocks, and each sequence drops
  its device references as a free would.  Swapping in is the mirror image, taking
  device blocks as an append does; host references are dropped in logical order.
  Both are all-or-nothing.  A swapped-out sequence may only be swapped in or freed.
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
        # prefix caching
        self.caching = False
        self.cache = {}                         # identity tuple -> cached block
        self.identity = {}                      # cached block -> identity tuple
        self.lru = []                           # free cached blocks, next evicted first
        self.tokens = {}                        # live sequence -> token ids, or None
        # swap preemption
        self.host_stack = []                    # top of stack = end of the list
        self.host_refcount = []
        self.swapped = set()

    # -- queries -----------------------------------------------------------------
    def free_stack_top_first(self):
        """Free blocks in the order they would be popped."""
        return list(reversed(self.stack))

    def num_free(self):
        """Blocks an append may take: free and empty plus free and cached."""
        return len(self.stack) + len(self.lru)

    def evictable(self):
        """Free cached blocks in the order they would be evicted."""
        return list(self.lru)

    def block_state(self, blk):
        """0 free and empty, 1 in use, 2 free and cached."""
        if self.refcount[blk] > 0:
            return 1
        return 2 if blk in self.identity else 0

    def table(self, seq):
        return list(self.tables[seq])

    def length(self, seq):
        return self.lengths[seq]

    # -- free lists --------------------------------------------------------------
    def _pop(self):
        if self.stack:
            return self.stack.pop()
        blk = self.lru.pop(0)
        del self.cache[self.identity.pop(blk)]
        return blk

    def _release(self, blk):
        self.refcount[blk] -= 1
        if self.refcount[blk] == 0:
            if blk in self.identity:
                self.lru.append(blk)
            else:
                self.stack.append(blk)

    # -- operations --------------------------------------------------------------
    def enable_prefix_caching(self):
        if self.tables:
            raise ValueError("sequences are live")
        self.caching = True

    def seq_new(self):
        seq = self.next_id
        self.next_id += 1
        self.tables[seq] = []
        self.lengths[seq] = 0
        self.tokens[seq] = []
        return seq

    def set_swap_space(self, host_blocks):
        if self.swapped:
            raise ValueError("sequences are swapped out")
        self.host_refcount = [0] * host_blocks
        self.host_stack = list(reversed(range(host_blocks)))

    def host_free_stack_top_first(self):
        return list(reversed(self.host_stack))

    def _check_resident(self, seq):
        if seq not in self.tables:
            raise KeyError(seq)
        if seq in self.swapped:
            raise ValueError("sequence %d is swapped out" % seq)

    def _release_all(self, row):
        for blk in (reversed(row) if self.caching else row):
            if blk >= 0:
                self._release(blk)

    def seq_swap_out(self, seqs):
        """Move ``seqs`` to host blocks; returns the (device, host) pairs to copy."""
        for i, seq in enumerate(seqs):
            self._check_resident(seq)
            if seq in seqs[:i]:
                raise ValueError("a sequence is listed twice")
        distinct = {b for seq in seqs for b in self.tables[seq] if b >= 0}
        if len(distinct) > len(self.host_stack):
            raise OutOfBlocks()
        to_host, pairs = {}, []
        for seq in seqs:
            row = self.tables[seq]
            device = list(row)
            for j, blk in enumerate(row):
                if blk < 0:
                    continue
                if blk not in to_host:
                    to_host[blk] = self.host_stack.pop()
                    pairs.append((blk, to_host[blk]))
                self.host_refcount[to_host[blk]] += 1
                row[j] = to_host[blk]
            self._release_all(device)
            self.swapped.add(seq)
        return pairs

    def seq_swap_in(self, seqs):
        """Move swapped-out ``seqs`` back to device blocks; returns (host, device) pairs."""
        for i, seq in enumerate(seqs):
            if seq not in self.tables or seq not in self.swapped:
                raise ValueError("sequence %d is not swapped out" % seq)
            if seq in seqs[:i]:
                raise ValueError("a sequence is listed twice")
        distinct = {h for seq in seqs for h in self.tables[seq] if h >= 0}
        if len(distinct) > self.num_free():
            raise OutOfBlocks()
        to_dev, pairs = {}, []
        for seq in seqs:
            row = self.tables[seq]
            host = list(row)
            for j, h in enumerate(row):
                if h < 0:
                    continue
                if h not in to_dev:
                    to_dev[h] = self._pop()
                    pairs.append((h, to_dev[h]))
                self.refcount[to_dev[h]] += 1
                row[j] = to_dev[h]
            for h in host:
                if h >= 0:
                    self.host_refcount[h] -= 1
                    if self.host_refcount[h] == 0:
                        self.host_stack.append(h)
            self.swapped.discard(seq)
        return pairs

    def seq_new_prefix(self, prompt):
        """New sequence sharing the cached blocks of the prompt's leading full blocks;
        returns ``(seq, cached_tokens)``."""
        if not self.caching:
            raise ValueError("prefix caching is off")
        prompt = [int(t) for t in prompt]
        bs = self.block_size
        seq = self.seq_new()
        table = self.tables[seq]
        limit = (len(prompt) - 1) // bs if prompt else 0
        for j in range(limit):
            blk = self.cache.get(tuple(prompt[:(j + 1) * bs]))
            if blk is None:
                break
            if self.refcount[blk] == 0:
                self.lru.remove(blk)
            self.refcount[blk] += 1
            table.append(blk)
        n = len(table) * bs
        self.lengths[seq] = n
        self.tokens[seq] = prompt[:n]
        return seq, n

    def seq_append(self, seq, n, tokens=None):
        """Append ``n`` tokens (ids in ``tokens``, or None); returns ``(slots, cow_pairs)``."""
        self._check_resident(seq)
        if n < 0:
            raise ValueError(n)
        if tokens is not None and len(tokens) != n:
            raise ValueError("one id per token")
        bs = self.block_size
        L = self.lengths[seq]
        table = self.tables[seq]
        needs_cow = n > 0 and L % bs != 0 and self.refcount[table[-1]] > 1
        fresh = sum(1 for pos in range(L, L + n) if pos % bs == 0)
        if fresh + int(needs_cow) > self.num_free():
            raise OutOfBlocks()
        if self.caching and tokens is None and n > 0:
            self.tokens[seq] = None
        known = self.tokens[seq] if self.caching else None
        cow_pairs = []
        if needs_cow:
            old = table[-1]
            new = self._pop()
            cow_pairs.append((old, new))
            self.refcount[old] -= 1
            self.refcount[new] = 1
            table[-1] = new
        slots = []
        for pos in range(L, L + n):
            if pos % bs == 0:
                blk = self._pop()
                self.refcount[blk] = 1
                table.append(blk)
            slots.append(table[pos // bs] * bs + pos % bs)
            if known is not None:
                known.append(int(tokens[pos - L]))
                if (pos + 1) % bs == 0:
                    ident = tuple(known[:pos + 1])
                    if ident not in self.cache:
                        blk = table[pos // bs]
                        self.cache[ident] = blk
                        self.identity[blk] = ident
        self.lengths[seq] = L + n
        return slots, cow_pairs

    def seq_fork(self, parent):
        self._check_resident(parent)
        child = self.seq_new()
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        known = self.tokens[parent]
        self.tokens[child] = None if known is None else list(known)
        for blk in self.tables[child]:
            if blk >= 0:
                self.refcount[blk] += 1
        return child

    def seq_free(self, seq):
        if seq not in self.tables:
            raise KeyError(seq)
        row = self.tables[seq]
        if seq in self.swapped:
            for h in row:
                if h >= 0:
                    self.host_refcount[h] -= 1
                    if self.host_refcount[h] == 0:
                        self.host_stack.append(h)
            self.swapped.discard(seq)
        else:
            self._release_all(row)
        del self.tables[seq]
        del self.lengths[seq]
        del self.tokens[seq]

    def seq_release_before(self, seq, token):
        """A sliding window has moved past ``token``: drop this sequence's hold on every
        block whose tokens all come before it ("vLLM explained", table of when KV may be
        overwritten: KV outside a sliding window can be dropped).  The last block is
        always kept (it holds the newest token).  Dropped entries become -1.  Returns the
        number of entries dropped now."""
        if token < 0:
            raise KeyError(seq)
        self._check_resident(seq)
        table = self.tables[seq]
        whole = [j for j in range(len(table) - 1) if (j + 1) * self.block_size <= token]
        dropped = 0
        for j in (reversed(whole) if self.caching else whole):
            blk = table[j]
            if blk < 0:
                continue
            self._release(blk)
            table[j] = -1
            dropped += 1
        return dropped

    def export_tables(self, seqs, max_blocks):
        """``(tables, context_lens)``: ``[n][max_blocks]`` padded with -1, and lengths."""
        tables, lens = [], []
        for seq in seqs:
            self._check_resident(seq)
            row = self.tables[seq]
            if len(row) > max_blocks:
                raise ValueError("max_blocks too small")
            tables.append(row + [-1] * (max_blocks - len(row)))
            lens.append(self.lengths[seq])
        return tables, lens

    # -- invariants --------------------------------------------------------------
    def check_invariants(self):
        """Conservation of references and of blocks; raises AssertionError if broken."""
        held, host_held = {}, {}
        for seq, row in self.tables.items():
            where = host_held if seq in self.swapped else held
            for blk in row:
                if blk >= 0:
                    where[blk] = where.get(blk, 0) + 1
        for blk in range(self.num_blocks):
            assert self.refcount[blk] == held.get(blk, 0), blk
        for h in range(len(self.host_refcount)):
            assert self.host_refcount[h] == host_held.get(h, 0), h
        hfree = set(self.host_stack)
        assert len(hfree) == len(self.host_stack)
        assert all(self.host_refcount[h] == 0 for h in hfree)
        assert len(hfree) + sum(1 for r in self.host_refcount if r > 0) == len(self.host_refcount)
        free = set(self.stack)
        assert len(free) == len(self.stack), "a block is on the free stack twice"
        assert all(self.refcount[b] == 0 for b in free)
        lru = set(self.lru)
        assert len(lru) == len(self.lru), "a block is on the LRU list twice"
        assert all(self.refcount[b] == 0 and b in self.identity for b in lru)
        assert not (free & lru) and not any(b in self.identity for b in free)
        assert len(free) + len(lru) + sum(1 for r in self.refcount if r > 0) == self.num_blocks
        assert len(self.cache) == len(self.identity)
        for ident, blk in self.cache.items():
            assert self.identity[blk] == ident and len(ident) % self.block_size == 0 and ident
        for seq, row in self.tables.items():
            assert len(row) == -(-self.lengths[seq] // self.block_size)
