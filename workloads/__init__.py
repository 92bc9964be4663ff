"""Seeded synthetic inputs for the paged KV-cache attention path.

This module is shared by the tests, the bench and the oracle-side checks. It
holds only random draws and workload sizes: which sequences exist, how long
they are, which of their tokens are shared, the query/key/value numbers, the
order in which the pool hands out physical blocks, and the pool size. None of
the method's arithmetic lives here: no slot computation, no block table, no
gather, no softmax. Each side (the HIP library and the CPU oracle) turns these
draws into block tables, slots and outputs with its own code.

Value recipe: N(0, 1) float32 from a seeded CPU ``torch.Generator``, then
rounded to bfloat16 (round-to-nearest-even) for the bf16 workloads. Every
random stream is keyed by (workload seed, stream key), so one sequence's
tokens can be regenerated without drawing the others.

The five named workloads follow the shapes the pages' decode and
chunked-prefill discussion implies (one query per sequence in decode, a causal
query chunk over cached plus new tokens in chunked prefill, 16-token blocks,
page 2 "The problem PagedAttention was actually solving"), at the sizes listed
in ``NAMED``.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

BLOCK_SIZE = 16

# Named workloads: name -> (seed, description). The builders below give the
# exact draws.
NAMED = {
    "tiny": (0, "4 decode seqs, ctx {1,7,16,33}, 4 q / 4 kv heads, head_dim 64, fp32, "
                "32-block pool in seeded random order, scale 1/8"),
    "llama": (1, "64 decode seqs, ctx U[128,4096], 32 q / 8 kv heads, head_dim 128, bf16, "
                 "pool 1.5x need, random placement"),
    "long": (2, "8 decode seqs, ctx U[32768,131072], 32 q / 8 kv heads, head_dim 128, bf16, "
                "pool 1.5x need, random placement (split-KV path)"),
    "shared": (3, "128 decode seqs sharing one 2048-token prefix + private suffix U[16,512], "
                  "32 q / 8 kv heads, head_dim 128, bf16"),
    "mixed": (4, "16 decode seqs ctx U[512,8192] + 2 prefill chunks of 512 queries over "
                 "U[0,4096] cached tokens, 32 q / 8 kv heads, head_dim 128, bf16"),
}


@dataclasses.dataclass
class SeqSpec:
    """One sequence of a workload.

    ``segments`` lists (stream key, number of tokens) in logical order; a
    stream key that appears in several sequences denotes tokens whose K/V are
    shared (a common prefix). ``new_tokens`` is how many of the sequence's last
    tokens are written by this step (1 for a decode sequence, the chunk length
    for a prefill chunk); the rest are already cached. ``fork_of`` names the
    earlier sequence whose blocks this one shares (its shared prefix), or None.
    """
    seq_id: int
    segments: List[Tuple[str, int]]
    new_tokens: int
    is_chunk: bool = False
    fork_of: Optional[int] = None
    fork_tokens: int = 0

    @property
    def total(self) -> int:
        return sum(n for _, n in self.segments)

    @property
    def cached(self) -> int:
        return self.total - self.new_tokens


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    dtype: str               # "f32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    num_blocks: int
    seqs: List[SeqSpec]
    free_order: Optional[np.ndarray]   # int32 permutation of 1..num_blocks-1, or None

    # ------------------------------------------------------------------ sizes
    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def decode_seqs(self) -> List[SeqSpec]:
        return [s for s in self.seqs if not s.is_chunk]

    @property
    def chunk_seqs(self) -> List[SeqSpec]:
        return [s for s in self.seqs if s.is_chunk]

    def max_blocks_per_seq(self, extra_tokens: int = 0) -> int:
        return max(1, max(-(-(s.total + extra_tokens) // BLOCK_SIZE) for s in self.seqs))

    # ------------------------------------------------------------------ draws
    def _gen(self, key: str) -> torch.Generator:
        h = hashlib.sha256(f"{self.seed}:{key}".encode()).digest()
        g = torch.Generator()
        g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
        return g

    def segment_kv(self, key: str, n: int) -> Tuple[torch.Tensor, torch.Tensor]:
        """K and V values of one token stream: two CPU tensors [n, Hkv, D]."""
        g = self._gen("kv:" + key)
        shape = (n, self.num_kv_heads, self.head_dim)
        k = torch.randn(shape, generator=g, dtype=torch.float32)
        v = torch.randn(shape, generator=g, dtype=torch.float32)
        return k.to(self.torch_dtype), v.to(self.torch_dtype)

    def seq_kv(self, spec: SeqSpec) -> Tuple[torch.Tensor, torch.Tensor]:
        """All K/V tokens of one sequence in logical order: two [total, Hkv, D]."""
        ks, vs = [], []
        for key, n in spec.segments:
            k, v = self.segment_kv(key, n)
            ks.append(k)
            vs.append(v)
        return torch.cat(ks, 0), torch.cat(vs, 0)

    def seq_q(self, spec: SeqSpec) -> torch.Tensor:
        """Queries of one sequence for this step: [q_len, Hq, D], where q_len is
        the chunk length for a prefill chunk and 1 for a decode sequence (also
        when the decode sequence is empty)."""
        g = self._gen(f"q:{spec.seq_id}")
        n = spec.new_tokens if spec.is_chunk else 1
        q = torch.randn((n, self.num_q_heads, self.head_dim), generator=g, dtype=torch.float32)
        return q.to(self.torch_dtype)

    # ------------------------------------------------------- allocator script
    def setup_ops(self) -> List[tuple]:
        """Allocator calls that place every sequence's cached tokens.

        ("add", sid) creates a sequence; ("fork", parent, child) makes child
        share all of parent's current blocks; ("append", sid, n) appends n
        tokens. A sequence with a shared prefix is forked from its owner right
        after the owner has appended exactly the prefix; afterwards every
        sequence appends the rest of its cached tokens, in sequence order.
        """
        ops: List[tuple] = []
        done: Dict[int, int] = {}
        owners = {s.fork_of for s in self.seqs if s.fork_of is not None}
        for s in self.seqs:
            if s.fork_of is None:
                ops.append(("add", s.seq_id))
                done[s.seq_id] = 0
                if s.seq_id in owners:
                    plen = max(x.fork_tokens for x in self.seqs if x.fork_of == s.seq_id)
                    ops.append(("append", s.seq_id, plen))
                    done[s.seq_id] = plen
        for s in self.seqs:
            if s.fork_of is not None:
                ops.append(("fork", s.fork_of, s.seq_id))
                done[s.seq_id] = s.fork_tokens
        for s in self.seqs:
            rest = s.cached - done[s.seq_id]
            if rest > 0:
                ops.append(("append", s.seq_id, rest))
        return ops

    def step_appends(self) -> Tuple[List[int], List[int]]:
        """The step's batched append: (sequence ids, new tokens per sequence)."""
        ids = [s.seq_id for s in self.seqs if s.new_tokens > 0]
        ns = [s.new_tokens for s in self.seqs if s.new_tokens > 0]
        return ids, ns


def _ints(rng: np.random.Generator, lo: int, hi: int, n: int) -> List[int]:
    """n integers uniform on [lo, hi] inclusive."""
    return [int(x) for x in rng.integers(lo, hi + 1, size=n)]


def _pool_blocks(block_need: int, factor: float) -> int:
    # pool = factor x the blocks the workload occupies, plus the null block
    return int(math.ceil(factor * block_need)) + 1


def _blocks(n: int) -> int:
    return -(-n // BLOCK_SIZE)


def custom(name: str = "custom", seed: int = 0, ctx: Sequence[int] = (1,), *,
           num_q_heads: int = 4, num_kv_heads: int = 4, head_dim: int = 64,
           dtype: str = "f32", scale: Optional[float] = None,
           pool_factor: float = 1.5, num_blocks: Optional[int] = None,
           shuffle: bool = True, shared_prefix: int = 0,
           chunks: Sequence[Tuple[int, int]] = ()) -> Workload:
    """Build a workload from explicit sizes.

    ``ctx`` are the decode sequences' total lengths (current token included).
    ``shared_prefix`` > 0 makes every decode sequence start with the same
    ``shared_prefix`` tokens (held by sequence 0 and forked to the others);
    then ``ctx`` must all exceed it. ``chunks`` are (cached, q_len) pairs of
    prefill-chunk sequences appended after the decode sequences.
    """
    seqs: List[SeqSpec] = []
    sid = 0
    for n in ctx:
        if shared_prefix:
            assert n > shared_prefix
            segs = [("prefix", shared_prefix), (f"s{sid}", n - shared_prefix)]
            fork = 0 if sid > 0 else None
            seqs.append(SeqSpec(sid, segs, 1, fork_of=fork, fork_tokens=shared_prefix if sid else 0))
        else:
            seqs.append(SeqSpec(sid, [(f"s{sid}", n)], 1 if n > 0 else 0))
        sid += 1
    for cached, qlen in chunks:
        seqs.append(SeqSpec(sid, [(f"s{sid}", cached + qlen)], qlen, is_chunk=True))
        sid += 1
    need = 0
    for s in seqs:
        need += _blocks(s.total) - (_blocks(s.fork_tokens) if s.fork_of is not None else 0)
    nb = num_blocks if num_blocks is not None else _pool_blocks(need, pool_factor)
    rng = np.random.default_rng(seed + 7919)
    order = (rng.permutation(np.arange(1, nb, dtype=np.int64)).astype(np.int32)
             if shuffle else None)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return Workload(name, seed, dtype, num_q_heads, num_kv_heads, head_dim, float(scale),
                    nb, seqs, order)


def named(name: str) -> Workload:
    """The five named workloads (see ``NAMED``)."""
    seed = NAMED[name][0]
    rng = np.random.default_rng(seed)
    big = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16")
    if name == "tiny":
        return custom("tiny", seed, [1, 7, 16, 33], num_q_heads=4, num_kv_heads=4, head_dim=64,
                      dtype="f32", scale=1.0 / 8.0, num_blocks=32)
    if name == "llama":
        return custom("llama", seed, _ints(rng, 128, 4096, 64), **big)
    if name == "long":
        return custom("long", seed, _ints(rng, 32768, 131072, 8), **big)
    if name == "shared":
        suffix = _ints(rng, 16, 512, 128)
        return custom("shared", seed, [2048 + x for x in suffix], shared_prefix=2048, **big)
    if name == "mixed":
        dec = _ints(rng, 512, 8192, 16)
        cached = _ints(rng, 0, 4096, 2)
        return custom("mixed", seed, dec, chunks=[(c, 512) for c in cached], **big)
    raise KeyError(name)


def scaled(name: str, divisor: int, seed_offset: int = 100) -> Workload:
    """A smaller workload with the same structure as a named one (for the CPU
    oracle and for quick parity runs): lengths divided by ``divisor``, same
    head counts, head_dim and dtype."""
    base = named(name)
    seed = base.seed + seed_offset
    rng = np.random.default_rng(seed)
    big = dict(num_q_heads=base.num_q_heads, num_kv_heads=base.num_kv_heads,
               head_dim=base.head_dim, dtype=base.dtype)
    if name == "llama":
        return custom("llama/%d" % divisor, seed, _ints(rng, max(1, 128 // divisor), 4096 // divisor, 8), **big)
    if name == "long":
        return custom("long/%d" % divisor, seed, _ints(rng, 32768 // divisor, 131072 // divisor, 2), **big)
    if name == "shared":
        p = max(16, 2048 // divisor)
        suffix = _ints(rng, max(1, 16 // divisor), max(2, 512 // divisor), 6)
        return custom("shared/%d" % divisor, seed, [p + x for x in suffix], shared_prefix=p, **big)
    if name == "mixed":
        dec = _ints(rng, max(1, 512 // divisor), 8192 // divisor, 4)
        cached = _ints(rng, 0, 4096 // divisor, 2)
        return custom("mixed/%d" % divisor, seed, dec,
                      chunks=[(c, max(1, 512 // divisor)) for c in cached], **big)
    raise KeyError(name)


# ------------------------------------------------------------ request streams
@dataclasses.dataclass
class Arrival:
    step: int              # the step before which the request is queued
    req_id: int
    prompt: List[int]      # token ids
    max_new_tokens: int
    extra_key: int = 0


class RequestStream:
    """A seeded stream of requests for scheduler-driven runs.

    Token ids come from a small vocabulary; prompts start with a prefix of
    one of a few shared stems (multiples of 16 tokens, so prefix-cache hits
    occur) and continue with random ids. A token's K and V depend only on
    (token id, position), drawn once per pair from tables, so two requests
    holding the same ids at the same positions hold the same K/V (as a
    causal model would for a shared prefix). Each request's queries are
    drawn per (request, position), and the token it "samples" after
    position p is a seeded draw keyed by (request, p).
    """

    def __init__(self, seed: int, num_requests: int, *, vocab: int = 32, max_pos: int = 320,
                 prompt_range: Tuple[int, int] = (1, 160), new_range: Tuple[int, int] = (1, 40),
                 arrival_span: int = 30, num_q_heads: int = 8, num_kv_heads: int = 2,
                 head_dim: int = 64, dtype: str = "bf16", salted: float = 0.1):
        self.seed = seed
        self.vocab = vocab
        self.max_pos = max_pos
        self.num_q_heads, self.num_kv_heads, self.head_dim = num_q_heads, num_kv_heads, head_dim
        self.dtype = dtype
        self.scale = 1.0 / math.sqrt(head_dim)
        rng = np.random.default_rng(seed)
        stems = [rng.integers(0, vocab, BLOCK_SIZE * int(rng.integers(1, 6))).tolist()
                 for _ in range(3)]
        self.arrivals: List[Arrival] = []
        for r in range(num_requests):
            stem = stems[int(rng.integers(0, len(stems)))]
            keep = BLOCK_SIZE * int(rng.integers(0, len(stem) // BLOCK_SIZE + 1))
            plen = int(rng.integers(prompt_range[0], prompt_range[1] + 1))
            prompt = (stem[:keep] + rng.integers(0, vocab, plen).tolist())[:max(plen, 1)]
            new = int(rng.integers(new_range[0], new_range[1] + 1))
            new = max(1, min(new, max_pos - len(prompt)))
            step = int(rng.integers(0, arrival_span + 1))
            salt = 1 if rng.random() < salted else 0
            self.arrivals.append(Arrival(step, r, prompt, new, salt))
        self.arrivals.sort(key=lambda a: (a.step, a.req_id))
        g = self._gen("kv")
        shape = (vocab, max_pos, num_kv_heads, head_dim)
        self._k = torch.randn(shape, generator=g, dtype=torch.float32).to(self.torch_dtype)
        self._v = torch.randn(shape, generator=g, dtype=torch.float32).to(self.torch_dtype)
        self._q: Dict[int, torch.Tensor] = {}

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def _gen(self, key: str) -> torch.Generator:
        h = hashlib.sha256(f"stream:{self.seed}:{key}".encode()).digest()
        g = torch.Generator()
        g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
        return g

    def kv(self, tokens: Sequence[int], positions: Sequence[int]) -> Tuple[torch.Tensor, torch.Tensor]:
        """K and V of the given (token id, position) pairs: two [n, Hkv, D]."""
        t = torch.as_tensor(list(tokens), dtype=torch.long)
        p = torch.as_tensor(list(positions), dtype=torch.long)
        return self._k[t, p], self._v[t, p]

    def q(self, req_id: int, positions: Sequence[int]) -> torch.Tensor:
        """Queries of request req_id at the given positions: [n, Hq, D]."""
        if req_id not in self._q:
            g = self._gen(f"q:{req_id}")
            self._q[req_id] = torch.randn((self.max_pos, self.num_q_heads, self.head_dim),
                                          generator=g, dtype=torch.float32).to(self.torch_dtype)
        return self._q[req_id][torch.as_tensor(list(positions), dtype=torch.long)]

    def sampled(self, req_id: int, position: int) -> int:
        """The token id request req_id "samples" from its output at position."""
        h = hashlib.sha256(f"stream:{self.seed}:tok:{req_id}:{position}".encode()).digest()
        return int.from_bytes(h[:4], "little") % self.vocab
