"""Pure-Python scalar brute force of paged attention (test infrastructure).

Written independently of ``oracle.paged``: nested loops over Python floats,
``math.exp``, no NumPy arithmetic, no shared helper. It walks the block table
token by token (position p lives in the table's entry p // 16, offset p % 16:
"My Understanding of vLLM and PagedAttention", sections "1. Logical Blocks"
and "3. Block Table") and evaluates scaled softmax attention by its
definition. Only for tiny inputs.

Pools and queries arrive as nested Python lists (or anything indexable that
yields numbers) already widened to float.
"""
from __future__ import annotations

import math


def _bf16_bits_to_float(bits: int) -> float:
    # a bfloat16 is the top half of a float32: rebuild the float32 by hand
    sign = -1.0 if bits & 0x8000 else 1.0
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0xFF:
        return float("nan") if man else sign * float("inf")
    if exp == 0:
        return sign * man * 2.0 ** (-133)           # subnormal: man/128 * 2^-126
    return sign * (1.0 + man / 128.0) * 2.0 ** (exp - 127)


def widen(x, storage: str):
    """Nested lists of Python floats from a NumPy array of float32 values or
    bfloat16 bit patterns (element by element)."""
    if storage == "f32":
        return x.astype(float).tolist()
    flat = [_bf16_bits_to_float(int(b)) for b in x.reshape(-1).tolist()]

    def build(shape, off):
        if len(shape) == 1:
            return flat[off:off + shape[0]], off + shape[0]
        rows = []
        for _ in range(shape[0]):
            r, off = build(shape[1:], off)
            rows.append(r)
        return rows, off
    return build(list(x.shape), 0)[0]


def _key(pool, table_row, p, h):
    blk = table_row[p // 16]
    return pool[blk][h][p % 16]


def _attend(qv, pool_k, pool_v, table_row, h_kv, visible, scale):
    if visible == 0:
        return [0.0] * len(qv)
    scores = []
    for p in range(visible):
        k = _key(pool_k, table_row, p, h_kv)
        dot = 0.0
        for d in range(len(qv)):
            dot += qv[d] * k[d]
        scores.append(scale * dot)
    top = max(scores)
    weights = [math.exp(z - top) for z in scores]
    total = sum(weights)
    out = [0.0] * len(qv)
    for p in range(visible):
        v = _key(pool_v, table_row, p, h_kv)
        w = weights[p] / total
        for d in range(len(qv)):
            out[d] += w * v[d]
    return out


def decode(q, pool_k, pool_v, table, context_lens, scale):
    """q[s][h][d]; pools[b][h][o][d]; returns out[s][h][d] (lists)."""
    hq = len(q[0])
    hkv = len(pool_k[0])
    group = hq // hkv
    out = []
    for s in range(len(q)):
        row = []
        for h in range(hq):
            row.append(_attend(q[s][h], pool_k, pool_v, table[s], h // group,
                               int(context_lens[s]), scale))
        out.append(row)
    return out


def prefill_chunk(q, cu_q_lens, context_lens, pool_k, pool_v, table, scale):
    """q[t][h][d] with chunks back to back; returns out[t][h][d] (lists)."""
    hq = len(q[0])
    hkv = len(pool_k[0])
    group = hq // hkv
    out = [None] * len(q)
    for c in range(len(cu_q_lens) - 1):
        lo, hi = int(cu_q_lens[c]), int(cu_q_lens[c + 1])
        start = int(context_lens[c]) - (hi - lo)
        for i in range(hi - lo):
            out[lo + i] = [_attend(q[lo + i][h], pool_k, pool_v, table[c], h // group,
                                   start + i + 1, scale) for h in range(hq)]
    return out
