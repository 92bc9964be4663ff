"""Pure-Python model of the paged KV block allocator (test infrastructure).

Policy, from the pages (cited by page title and section):

* One preallocated pool of fixed 16-token blocks; a sequence's logical block i
  maps to any physical block ("(2) vLLM Internals ...", 1.1 "The Analogy";
  "My Understanding of vLLM and PagedAttention", "1. Logical Blocks" to
  "3. Block Table").
* The first block taken from the free queue is burned as the null block, an
  ordinary id meaning "no block"; its refcount is not kept ("vLLM: what
  PagedAttention turned into", "The block pool, and the two tricks in it").
  Block tables are padded with it.
* Blocks freed with no content hash go to the front of the free queue and
  are reused first (LIFO) (same section). This model keeps no hashes, so
  every freed block takes that path.
* A request's blocks are handed back tail first, so its last block is the
  first to be reused and its first block the last (same section).
* Identical prefixes share physical blocks by reference counting, and a
  write into a shared block copies it first (copy-on-write) ("(2) vLLM
  Internals ...", 1.2 "Three Direct Wins", items 2 and 3; "vLLM: what
  PagedAttention turned into", "What a block hash actually is").
* Blocks are allocated on demand as tokens arrive and freed when the request
  completes ("My Understanding of vLLM and PagedAttention", "Step 2", "Step 3",
  "Step 5").
* When blocks run out the allocation fails and the caller preempts ("vLLM: what
  PagedAttention turned into", "Preemption, and the path that got deleted");
  here a failed call changes nothing.

Readings where the pages are silent: the initial free queue is 0, 1, ...,
NB-1 unless an explicit order is installed; a batch of freed blocks is placed
at the front in the order it was visited (tail first), so the tail is
reused first; the copy-on-write trigger is an append into a partially filled
last block whose refcount exceeds one; a full shared block is never copied.
"""
from __future__ import annotations

import collections
from typing import Dict, List, Sequence, Tuple

import numpy as np

BLOCK = 16


class OutOfBlocks(Exception):
    pass


class AllocatorModel:
    def __init__(self, num_blocks: int):
        if num_blocks < 2:
            raise ValueError("need the null block plus at least one block")
        self.num_blocks = num_blocks
        self.free: collections.deque = collections.deque(range(num_blocks))
        self.null_block = self.free.popleft()           # id 0
        self.ref = [0] * num_blocks
        self.blocks: Dict[int, List[int]] = {}
        self.length: Dict[int, int] = {}

    # ----------------------------------------------------------------- setup
    def set_free_order(self, order: Sequence[int]) -> None:
        """Install the order in which free blocks are handed out (a
        permutation of 1..NB-1); only while no block is in use."""
        order = [int(x) for x in order]
        if self.blocks or sorted(order) != list(range(1, self.num_blocks)):
            raise ValueError("free order must permute 1..NB-1 while the pool is empty")
        self.free = collections.deque(order)

    # ------------------------------------------------------------- sequences
    def add(self, sid: int) -> None:
        if sid in self.blocks:
            raise KeyError("sequence exists")
        self.blocks[sid] = []
        self.length[sid] = 0

    def _needs(self, sid: int, n: int) -> Tuple[bool, int]:
        """(copy-on-write needed, new blocks needed) to append n tokens."""
        blocks, length = self.blocks[sid], self.length[sid]
        cow = n > 0 and length % BLOCK != 0 and self.ref[blocks[-1]] > 1
        grow = -(-(length + n) // BLOCK) - len(blocks)
        return cow, grow

    def _append(self, sid: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        cow, grow = self._needs(sid, n)
        blocks = self.blocks[sid]
        pairs = []
        if cow:
            old = blocks[-1]
            new = self.free.popleft()
            self.ref[new] = 1
            self.ref[old] -= 1
            blocks[-1] = new
            pairs.append((old, new))
        for _ in range(grow):
            b = self.free.popleft()
            self.ref[b] = 1
            blocks.append(b)
        start = self.length[sid]
        slots = [blocks[p // BLOCK] * BLOCK + p % BLOCK for p in range(start, start + n)]
        self.length[sid] = start + n
        return slots, pairs

    def append(self, sid: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Append n tokens; returns (their slots, copy-on-write pairs)."""
        return self.batch_append([sid], [n])

    def batch_append(self, sids: Sequence[int], ns: Sequence[int]):
        """Append ns[i] tokens to sequence sids[i], in order, all or nothing.
        Returns (slots of every new token in order, copy-on-write pairs)."""
        if len(set(sids)) != len(sids):
            raise ValueError("duplicate sequence in batch")
        total = 0
        for sid, n in zip(sids, ns):
            if sid not in self.blocks:
                raise KeyError("no such sequence")
            if n < 0:
                raise ValueError("negative token count")
            cow, grow = self._needs(sid, n)
            total += grow + int(cow)
        if total > len(self.free):
            raise OutOfBlocks()
        slots: List[int] = []
        pairs: List[Tuple[int, int]] = []
        for sid, n in zip(sids, ns):
            s, p = self._append(sid, n)
            slots += s
            pairs += p
        return slots, pairs

    def fork(self, parent: int, child: int) -> None:
        """Child shares every block of parent (refcount +1 each)."""
        if parent not in self.blocks:
            raise KeyError("no such sequence")
        if child in self.blocks:
            raise KeyError("sequence exists")
        self.blocks[child] = list(self.blocks[parent])
        self.length[child] = self.length[parent]
        for b in self.blocks[child]:
            self.ref[b] += 1

    def free_seq(self, sid: int) -> None:
        """Release a sequence: its blocks are visited tail first; those whose
        refcount drops to zero go to the front of the free queue in that
        order."""
        if sid not in self.blocks:
            raise KeyError("no such sequence")
        released = []
        for b in reversed(self.blocks.pop(sid)):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                released.append(b)
        del self.length[sid]
        self.free.extendleft(reversed(released))

    # ----------------------------------------------------------------- views
    def block_table(self, sids: Sequence[int], max_blocks: int):
        """Dense int32 table [len(sids), max_blocks] padded with the null
        block, and int32 context lengths."""
        table = np.full((len(sids), max_blocks), self.null_block, dtype=np.int32)
        lens = np.zeros(len(sids), dtype=np.int32)
        for i, sid in enumerate(sids):
            b = self.blocks[sid]
            if len(b) > max_blocks:
                raise ValueError("table row too short")
            table[i, :len(b)] = b
            lens[i] = self.length[sid]
        return table, lens

    def num_free(self) -> int:
        return len(self.free)

    def stats(self) -> dict:
        """Pool accounting: blocks in use, free, shared; tokens held; the share
        of the in-use slots holding token state ("vLLM: what PagedAttention
        turned into", "Checking the 96.3%")."""
        filled: Dict[int, int] = {}
        logical = 0
        for sid, blocks in self.blocks.items():
            n = self.length[sid]
            logical += n
            for i, b in enumerate(blocks):
                filled[b] = max(filled.get(b, 0), min(BLOCK, n - BLOCK * i))
        used = sum(1 for r in self.ref if r > 0)
        stored = sum(filled.values())
        return {
            "num_seqs": len(self.blocks),
            "used_blocks": used,
            "free_blocks": len(self.free),
            "shared_blocks": sum(1 for r in self.ref if r > 1),
            "logical_tokens": logical,
            "stored_tokens": stored,
            "utilisation": stored / (BLOCK * used) if used else 0.0,
        }
