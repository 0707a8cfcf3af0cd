"""Oracle: paged KV block allocator with reference counts and copy-on-write.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain Python lists and
dicts; every rule below is written so that an independent implementation can
agree with it bit for bit.

What the pages fix ("PagedAttention: the KV cache was the bottleneck all
along", section "Virtual memory for attention"):
  * the cache is cut into fixed-size blocks of ``bs`` tokens; a per-sequence
    block table maps logical blocks to physical ones;
  * a block is taken from the pool only when a sequence's length reaches
    into it, so only its last block can be partly empty;
  * completions of one prompt share the prompt's blocks and copy a block only
    when they diverge (copy-on-write); beams are forked and discarded.

Readings where the pages are silent:
  * free blocks form a LIFO stack; the block popped first at start-up is
    ``init_order[0]`` (``0, 1, ..., NB-1`` by default);
  * copy-on-write is lazy: ``fork`` copies the table and raises every shared
    block's count; ``append`` into a last block whose count is above one takes
    a fresh block, reports the pair (old, new) for the device copy, drops one
    reference from the old block and points the table at the new one;
  * ``free`` walks the table from the last logical block to the first,
    dropping one reference each and pushing every block that reaches zero;
  * running out of blocks reports ``OOM`` and changes nothing.

Sharing across requests (page "Efficient Memory Management for Large
Language Model Serving with PagedAttention", from the abstract: sharing
within and across requests; "PagedAttention: the KV cache was the
bottleneck all along", section "What is left": prompt-side reuse of blocks,
e.g. one system prompt held once for many users).  Readings:
  * a registry maps caller keys (one per block, naming the whole prefix up
    to that block) to full blocks and holds one reference to each;
  * ``publish`` enters a sequence's first n full blocks; a key already
    present keeps its block;
  * ``create_prefixed`` starts a sequence with the blocks of the longest run
    of present keys, stopping at the first miss, one reference each; its
    length is that many full blocks;
  * ``evict`` walks its keys from last to first, dropping each present
    entry's reference and pushing blocks that reach zero.
"""
from __future__ import annotations


class OutOfBlocks(Exception):
    pass


class Allocator:
    def __init__(self, num_blocks: int, bs: int, init_order=None):
        if num_blocks < 0 or bs < 1:
            raise ValueError("bad allocator shape")
        order = list(range(num_blocks)) if init_order is None else [int(b) for b in init_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("init_order must be a permutation of the pool")
        self.NB = num_blocks
        self.bs = bs
        self.free = list(reversed(order))   # top of the stack is the list's end
        self.ref = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.registry: dict[int, int] = {}    # key -> block

    # -- queries -----------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def refcount(self, b: int) -> int:
        return self.ref[b]

    def seq_len(self, sid: int) -> int:
        return self.lens[sid]

    def table(self, sid: int) -> list[int]:
        return list(self.tables[sid])

    def free_stack(self) -> list[int]:
        """Free blocks in the order they would be handed out."""
        return list(reversed(self.free))

    # -- sequence operations ----------------------------------------------
    def create(self, sid: int) -> None:
        if sid in self.tables:
            raise KeyError(f"sequence {sid} exists")
        self.tables[sid] = []
        self.lens[sid] = 0

    def _pop(self) -> int:
        b = self.free.pop()
        self.ref[b] = 1
        return b

    def append(self, sid: int):
        """Reserve the slot of the sequence's next token.

        Returns ``(slot, cow_src, cow_dst)``; the pair is ``(-1, -1)`` when no
        block has to be copied before the token is written."""
        table = self.tables[sid]
        n = self.lens[sid]
        off = n % self.bs
        cow = (-1, -1)
        if off == 0:                          # last block full (or none yet)
            if not self.free:
                raise OutOfBlocks()
            table.append(self._pop())
        else:
            last = table[-1]
            if self.ref[last] > 1:            # shared: copy before writing
                if not self.free:
                    raise OutOfBlocks()
                new = self._pop()
                self.ref[last] -= 1
                table[-1] = new
                cow = (last, new)
        self.lens[sid] = n + 1
        return table[-1] * self.bs + off, cow[0], cow[1]

    def fork(self, parent: int, child: int) -> None:
        if parent not in self.tables or child in self.tables:
            raise KeyError("bad fork")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def release(self, sid: int) -> None:
        table = self.tables.pop(sid)
        del self.lens[sid]
        for b in reversed(table):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    def build_batch(self, sids, MB: int):
        """Block tables ``[S][MB]`` (padded with -1) and context lengths."""
        tables, lens = [], []
        for sid in sids:
            t = self.tables[sid]
            if len(t) > MB:
                raise ValueError("table wider than MB")
            tables.append(t + [-1] * (MB - len(t)))
            lens.append(self.lens[sid])
        return tables, lens

    # -- sharing across requests ------------------------------------------
    def publish(self, sid: int, keys) -> int:
        keys = [int(k) for k in keys]
        if len(keys) * self.bs > self.lens[sid]:
            raise ValueError("only full blocks can be published")
        added = 0
        for j, k in enumerate(keys):
            if k in self.registry:
                continue
            b = self.tables[sid][j]
            self.registry[k] = b
            self.ref[b] += 1
            added += 1
        return added

    def create_prefixed(self, sid: int, keys) -> int:
        if sid in self.tables:
            raise KeyError(f"sequence {sid} exists")
        blocks = []
        for k in keys:
            if int(k) not in self.registry:
                break
            blocks.append(self.registry[int(k)])
        for b in blocks:
            self.ref[b] += 1
        self.tables[sid] = blocks
        self.lens[sid] = len(blocks) * self.bs
        return len(blocks)

    def evict(self, keys) -> int:
        removed = 0
        for k in reversed([int(k) for k in keys]):
            if k not in self.registry:
                continue
            b = self.registry.pop(k)
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
            removed += 1
        return removed
