"""NumPy float64 reference of the paged KV-cache hot path (test infrastructure).

Storage convention (the pages do not fix a memory layout): a pool is one array
per tensor (K and V) of shape [num_blocks, num_kv_heads, 16, head_dim]; block b,
head h, in-block offset o, dimension d is ``pool[b, h, o, d]``. A pool holds
either float32 values or bfloat16 bit patterns (uint16); ``to_f64`` widens
both exactly.

Slot convention: token position p of a sequence whose logical block p // 16
lives in physical block b is stored at slot ``b * 16 + p % 16``; a negative
slot means "no token" and is never written.
"""
from __future__ import annotations

import numpy as np

BLOCK = 16


# --------------------------------------------------------------------- values
def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact widening to float64 of float32 values or bfloat16 bit patterns.

    A bfloat16 number is the upper 16 bits of a float32, so shifting its bits
    left by 16 gives the float32 with the same value, which float64 holds
    exactly.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError("expected float32 values or uint16 bfloat16 bits, got %s" % x.dtype)


def new_pool(num_blocks: int, num_kv_heads: int, head_dim: int, storage: str,
             fill: float = float("nan")) -> np.ndarray:
    """An empty pool [num_blocks, num_kv_heads, 16, head_dim]; ``storage`` is
    "f32" (float32 values) or "bf16" (uint16 bit patterns). Unwritten entries
    hold ``fill`` (NaN by default, so any read of an unassigned slot shows)."""
    shape = (num_blocks, num_kv_heads, BLOCK, head_dim)
    if storage == "f32":
        return np.full(shape, fill, dtype=np.float32)
    if storage == "bf16":
        bits = np.array([fill], dtype=np.float32).view(np.uint32)[0] >> 16
        return np.full(shape, bits, dtype=np.uint16)
    raise ValueError(storage)


# ------------------------------------------------------------------- the pool
def scatter(pool: np.ndarray, new: np.ndarray, slot_mapping: np.ndarray) -> None:
    """Write each new token's per-head vectors into its slot.

    The KV of a request is logically contiguous but physically stored in
    fixed-size blocks anywhere in one pool, with a table doing the mapping
    ("(2) vLLM Internals ...", section 1.1 "The Analogy"); the worker keeps an
    int64 slot mapping with one entry per scheduled token ("vLLM: what
    PagedAttention turned into", section "The problem PagedAttention was
    actually solving"). Token t goes to block slot // 16, offset slot % 16;
    tokens with a negative slot are skipped. ``new`` is [T, num_kv_heads,
    head_dim] in the pool's storage type. The copy is exact.
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    for t, slot in enumerate(slots.tolist()):
        if slot < 0:
            continue
        pool[slot // BLOCK, :, slot % BLOCK, :] = new[t]


def copy_blocks(pool: np.ndarray, pairs) -> None:
    """Copy-on-write: for each (src, dst) pair, block dst becomes a copy of
    block src ("(2) vLLM Internals ...", section 1.2 "Three Direct Wins",
    item 2; "vLLM: what PagedAttention turned into", section "What a block
    hash actually is", on redirecting a shared tail into a private
    copy-on-write block). Pairs are applied in order."""
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2).tolist():
        pool[dst] = pool[src]


def materialise(pool: np.ndarray, table_row, n: int) -> np.ndarray:
    """A sequence's K (or V) in logical order, float64 [num_kv_heads, n, head_dim].

    Logical block i holds token positions 16*i .. 16*i+15 and the block table
    maps it to a physical block ("My Understanding of vLLM and
    PagedAttention", sections "1. Logical Blocks", "2. Physical Blocks" and
    "3. Block Table"). Concatenating the physical blocks the table names, in
    table order, and keeping the first n tokens restores the logical order.
    """
    nb = -(-n // BLOCK)
    if n == 0:
        return np.zeros((pool.shape[1], 0, pool.shape[3]), dtype=np.float64)
    ids = np.asarray(table_row, dtype=np.int64)[:nb]
    blocks = pool[ids]                                  # [nb, H, 16, D]
    seq = np.transpose(blocks, (1, 0, 2, 3)).reshape(pool.shape[1], nb * BLOCK, pool.shape[3])
    return to_f64(seq[:, :n, :])


# ------------------------------------------------------------------ attention
def _softmax_attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Scaled softmax attention of query rows q [m, D] over keys k [n, D] and
    values v [n, D]: o_r = sum_t p_rt v_t with p_r = softmax(scale * q_r . k_t).
    With n == 0 there is nothing to attend to and the result is zero."""
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    z = scale * (q @ k.T)                               # [m, n]
    z = z - z.max(axis=1, keepdims=True)
    w = np.exp(z)
    return (w @ v) / w.sum(axis=1, keepdims=True)


def decode(q, k_pool, v_pool, block_table, context_lens, scale: float) -> np.ndarray:
    """Decode attention: one query token per sequence over its paged KV.

    q is [S, Hq, D] (float32 values or bf16 bits); block_table is
    [S, max_blocks]; context_lens[s] counts every cached token of sequence s,
    the current one included (its K/V are written before attention). Query
    head h reads KV head h // (Hq / Hkv) (grouped heads, consecutive query
    heads per KV head). Returns float64 [S, Hq, D].

    The kernel the pages describe gathers the scattered KV blocks, restores
    the logical token order and computes attention ("My Understanding of vLLM
    and PagedAttention", sections "3. PagedAttention CUDA Kernel" and "Step 4
    -- Attention Computation"); what it computes is plain scaled softmax
    attention over the sequence's tokens, which this function evaluates
    after materialising the contiguous K/V.
    """
    qf = to_f64(q)
    S, hq, _ = qf.shape
    hkv = k_pool.shape[1]
    group = hq // hkv
    out = np.zeros(qf.shape, dtype=np.float64)
    for s in range(S):
        n = int(context_lens[s])
        ks = materialise(k_pool, block_table[s], n)
        vs = materialise(v_pool, block_table[s], n)
        for g in range(hkv):
            heads = slice(g * group, (g + 1) * group)
            out[s, heads] = _softmax_attend(qf[s, heads], ks[g], vs[g], scale)
    return out


def prefill_chunk(q, cu_q_lens, context_lens, k_pool, v_pool, block_table,
                  scale: float) -> np.ndarray:
    """Chunked-prefill attention: a causal chunk of queries per sequence.

    q is [Tq, Hq, D] holding every chunk's queries back to back; chunk c owns
    rows cu_q_lens[c] .. cu_q_lens[c+1]-1. context_lens[c] is the sequence's
    total KV length including the chunk's own tokens (already written to the
    pool), so the chunk starts at absolute position p0 = context_lens[c] -
    q_len. Query i of the chunk sits at position p0 + i and attends to
    positions 0 .. p0 + i (causal). Long prompts are cut into such chunks and
    interleaved with decode steps ("(2) vLLM Internals ...", section
    "2. Continuous Batching"; "vLLM: what PagedAttention turned into",
    section "The scheduler, and what it has to balance now"). Returns
    float64 [Tq, Hq, D].
    """
    qf = to_f64(q)
    hq = qf.shape[1]
    hkv = k_pool.shape[1]
    group = hq // hkv
    out = np.zeros(qf.shape, dtype=np.float64)
    cu = [int(x) for x in cu_q_lens]
    for c in range(len(cu) - 1):
        lo, hi = cu[c], cu[c + 1]
        qlen = hi - lo
        n = int(context_lens[c])
        p0 = n - qlen
        ks = materialise(k_pool, block_table[c], n)
        vs = materialise(v_pool, block_table[c], n)
        for i in range(qlen):
            visible = p0 + i + 1
            for g in range(hkv):
                heads = slice(g * group, (g + 1) * group)
                out[lo + i, heads] = _softmax_attend(qf[lo + i, heads], ks[g, :visible],
                                                     vs[g, :visible], scale)
    return out


def attend_sequence(q, k, v, positions, scale: float) -> np.ndarray:
    """Attention of one sequence's queries over its own tokens, no paging.

    q is [m, Hq, D]; k and v are [n, Hkv, D], the sequence's tokens in
    logical order; query i sits at positions[i] and attends to tokens
    0 .. positions[i] (causal; decode is the case of one query at the last
    position). This is what the paged kernels must return whatever the
    placement of the blocks, the chunking of the prompt, preemption and
    recompute, or prefix-cache reuse ("(2) vLLM Internals ...", section 1.1
    "The Analogy": paging changes where K/V live, not what attention sees).
    Returns float64 [m, Hq, D].
    """
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    hq, hkv = qf.shape[1], kf.shape[1]
    group = hq // hkv
    out = np.zeros(qf.shape, dtype=np.float64)
    for i, p in enumerate(positions):
        for g in range(hkv):
            heads = slice(g * group, (g + 1) * group)
            out[i, heads] = _softmax_attend(qf[i, heads], kf[:p + 1, g], vf[:p + 1, g], scale)
    return out
