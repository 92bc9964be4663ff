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
  are reused first (LIFO); blocks freed with a hash go to the back (FIFO),
  keep their hash and stay reusable until the queue hands them out again,
  which is when they are evicted (lazily) (same section).
* Prefix caching (optional): a full block's hash chains its parent's hash,
  its token ids and extra keys, so it names a prefix ending at the block;
  lookups walk a prompt's full blocks from the start and stop at the first
  miss; the extra key (a tenant salt) enters the first block only ("vLLM:
  what PagedAttention turned into", "What a block hash actually is"). The
  map key is the hash followed by the KV-cache group id, 4 bytes big endian
  ("The block pool, and the two tricks in it").
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
at the front (or, hashed, at the back) in the order it was visited (tail
first), so the tail is reused (or evicted) first; the copy-on-write trigger
is an append into a partially filled last block whose refcount exceeds one; a
full shared block is never copied. The hash is SHA-256 over the parent hash
(32 bytes; for a first block the hash of the fixed string "pkv none hash"),
the 16 token ids as little-endian int32 and the extra key as little-endian
uint64; a block whose key another block already holds stays unhashed; token
ids are recorded per sequence in order and a block is hashed when its
sixteenth id is recorded.
"""
from __future__ import annotations

import collections
import hashlib
import struct
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 16
NONE_HASH = hashlib.sha256(b"pkv none hash").digest()
GROUP_ID = (0).to_bytes(4, "big")


def block_hash(parent: Optional[bytes], tokens: Sequence[int], extra: int = 0) -> bytes:
    """Chained content hash of one full block."""
    msg = (parent if parent is not None else NONE_HASH)
    msg += np.asarray(tokens, dtype="<i4").tobytes() + struct.pack("<Q", int(extra))
    return hashlib.sha256(msg).digest()


def splitmix64(seed: int, n: int) -> List[int]:
    """The first n outputs of SplitMix64 (Steele, Lea and Flood, "Fast
    splittable pseudorandom number generators", OOPSLA 2014) from a 64-bit
    state that starts at seed: each step adds the odd constant
    0x9E3779B97F4A7C15 to the state and returns it mixed by
    z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
    z *= 0x94D049BB133111EB; z ^= z >> 31 (all modulo 2^64)."""
    mask = (1 << 64) - 1
    state = int(seed) & mask
    out = []
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & mask
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
        out.append(z ^ (z >> 31))
    return out


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
        # prefix cache
        self.caching = False
        self.hash: Dict[int, bytes] = {}          # block -> its hash (cached blocks)
        self.parent_of: Dict[int, Optional[bytes]] = {}
        self.cache: Dict[bytes, int] = {}         # hash + group id -> block
        self.chain: Dict[int, dict] = {}          # sequence -> recorded ids state
        self.lookups = 0
        self.hit_blocks = 0

    # ----------------------------------------------------------------- setup
    def set_free_order(self, order: Sequence[int]) -> None:
        """Install the order in which free blocks are handed out (a
        permutation of 1..NB-1); only while no block is in use."""
        order = [int(x) for x in order]
        if self.blocks or sorted(order) != list(range(1, self.num_blocks)):
            raise ValueError("free order must permute 1..NB-1 while the pool is empty")
        self._clear_cache()
        self.free = collections.deque(order)

    def shuffle_free_list(self, seed: int) -> None:
        """Random physical placement from a seed: the ids 1..NB-1, ascending,
        permuted by a Fisher-Yates shuffle (Durstenfeld's form: for i from
        the last index down to 1, swap entry i with entry r mod (i + 1)),
        where r are successive SplitMix64 outputs (Steele, Lea and Flood,
        OOPSLA 2014) of a counter that starts at the seed."""
        draws = splitmix64(seed, max(0, self.num_blocks - 2))
        order = list(range(1, self.num_blocks))
        for k, i in enumerate(range(len(order) - 1, 0, -1)):
            j = draws[k] % (i + 1)
            order[i], order[j] = order[j], order[i]
        self.set_free_order(order)

    def _clear_cache(self) -> None:
        self.hash.clear()
        self.parent_of.clear()
        self.cache.clear()

    def enable_caching(self, enabled: bool = True) -> None:
        if self.blocks:
            raise ValueError("only while no sequence exists")
        self._clear_cache()
        self.caching = bool(enabled)

    def _pop(self) -> int:
        """Take the front block; a cached one is evicted now (lazily)."""
        b = self.free.popleft()
        if b in self.hash:
            key = self.hash.pop(b) + GROUP_ID
            self.parent_of.pop(b)
            if self.cache.get(key) == b:
                del self.cache[key]
        return b

    # ------------------------------------------------------------- sequences
    def add(self, sid: int) -> None:
        if sid in self.blocks:
            raise KeyError("sequence exists")
        self.blocks[sid] = []
        self.length[sid] = 0
        self.chain[sid] = {"recorded": 0, "parent": None, "pending": [], "salt": 0}

    def _walk_cached(self, tokens: Sequence[int], salt: int, max_cached: int):
        """The cached blocks a prompt would attach, in order, and the hash of
        the last one; changes nothing."""
        tokens = [int(t) for t in tokens]
        limit = len(tokens) if max_cached < 0 else min(len(tokens), max_cached)
        full = limit // BLOCK if self.caching else 0
        parent = None
        got: List[int] = []
        for k in range(full):
            h = block_hash(parent, tokens[k * BLOCK:(k + 1) * BLOCK], salt if k == 0 else 0)
            b = self.cache.get(h + GROUP_ID)
            if b is None:
                break
            got.append(b)
            parent = h
        return got, parent

    def lookup_cached(self, tokens: Sequence[int], salt: int = 0, max_cached: int = -1):
        """(tokens add_cached would attach, how many of those blocks it would
        take back out of the free queue); changes nothing."""
        got, _ = self._walk_cached(tokens, salt, max_cached)
        return BLOCK * len(got), sum(1 for b in got if self.ref[b] == 0)

    def add_cached(self, sid: int, tokens: Sequence[int], salt: int = 0, max_cached: int = -1) -> int:
        """New sequence for a prompt: attach the longest run of cached full
        blocks from its start; returns the tokens attached."""
        if sid in self.blocks:
            raise KeyError("sequence exists")
        got, parent = self._walk_cached(tokens, salt, max_cached)
        for b in got:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
        self.blocks[sid] = got
        self.length[sid] = BLOCK * len(got)
        self.chain[sid] = {"recorded": BLOCK * len(got), "parent": parent, "pending": [],
                           "salt": int(salt)}
        self.lookups += 1
        self.hit_blocks += len(got)
        return BLOCK * len(got)

    def record_tokens(self, sid: int, tokens: Sequence[int]) -> None:
        """Ids of the sequence's next tokens; a block whose sixteenth id
        arrives is hashed and, with caching on, enters the map."""
        st = self.chain[sid]
        if st["recorded"] + len(tokens) > self.length[sid]:
            raise ValueError("recording beyond the sequence's length")
        for t in tokens:
            st["pending"].append(int(t))
            st["recorded"] += 1
            if st["recorded"] % BLOCK == 0:
                k = st["recorded"] // BLOCK - 1
                h = block_hash(st["parent"], st["pending"], st["salt"] if k == 0 else 0)
                self._register(self.blocks[sid][k], h, st["parent"])
                st["parent"] = h
                st["pending"] = []

    def _register(self, b: int, h: bytes, parent: Optional[bytes]) -> None:
        if not self.caching or b in self.hash or (h + GROUP_ID) in self.cache:
            return
        self.hash[b] = h
        self.parent_of[b] = parent
        self.cache[h + GROUP_ID] = b

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
            new = self._pop()
            self.ref[new] = 1
            self.ref[old] -= 1
            blocks[-1] = new
            pairs.append((old, new))
        for _ in range(grow):
            b = self._pop()
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
        st = self.chain[parent]
        self.chain[child] = {"recorded": st["recorded"], "parent": st["parent"],
                             "pending": list(st["pending"]), "salt": st["salt"]}
        for b in self.blocks[child]:
            self.ref[b] += 1

    def free_seq(self, sid: int) -> None:
        """Release a sequence: its blocks are visited tail first; those whose
        refcount drops to zero go to the front of the free queue (no hash)
        or to its back (hashed), each pile in visiting order."""
        if sid not in self.blocks:
            raise KeyError("no such sequence")
        front, back = [], []
        for b in reversed(self.blocks.pop(sid)):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                (back if b in self.hash else front).append(b)
        del self.length[sid]
        del self.chain[sid]
        self.free.extendleft(reversed(front))
        self.free.extend(back)

    def block_hash_of(self, b: int) -> Optional[bytes]:
        return self.hash.get(b)

    def cache_stats(self) -> dict:
        return {"cached_blocks": len(self.cache), "lookups": self.lookups,
                "hit_blocks": self.hit_blocks}

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
