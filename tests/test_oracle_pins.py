"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each ``check_*`` function raises AssertionError when the oracle is wrong; the
``test_*`` wrappers run them, and ``test_planted_mistakes_are_caught`` plants
plausible mistakes in the oracle (on the CPU) and shows that some pin fails
for each.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import allocator as amodel
from oracle import brute, paged

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")
FACTS = json.load(open(GOLDEN))


# --------------------------------------------------------------------- helpers
def _rand_pool(rng, nb, hkv, d, storage):
    x = rng.standard_normal((nb, hkv, 16, d)).astype(np.float32)
    if storage == "f32":
        return x
    # round-to-nearest-even to bf16 bits (plumbing for the test inputs)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _rand_q(rng, shape, storage):
    x = rng.standard_normal(shape).astype(np.float32)
    if storage == "f32":
        return x
    u = x.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _random_tables(rng, nb, lens, maxb):
    """Distinct random physical blocks for each sequence (never block 0)."""
    ids = rng.permutation(np.arange(1, nb))
    table = np.zeros((len(lens), maxb), dtype=np.int32)
    k = 0
    for s, n in enumerate(lens):
        m = -(-n // 16)
        table[s, :m] = ids[k:k + m]
        k += m
    return table


# ----------------------------------------------------------- worked example
def check_block_table_example():
    """Page 3's worked table: logical blocks 0, 1, 2 -> physical 7, 21, 3."""
    ex = FACTS["block_table_example"]
    mapping = ex["logical_to_physical"]
    nb = 32
    a = amodel.AllocatorModel(nb)
    rest = [b for b in range(1, nb) if b not in mapping]
    a.set_free_order(mapping + rest)
    a.add(0)
    slots, pairs = a.append(0, 33)
    table, lens = a.block_table([0], 4)
    assert table[0, :3].tolist() == mapping and table[0, 3] == 0 and lens[0] == 33
    assert pairs == []
    # Hand derivation: the page's 1-based token 18 (0-based position 17) is in
    # "tokens 17-32 -> logical block 1" at offset 1; logical block 1 is
    # physical block 21, so its slot is 21*16 + 1 = 337. Likewise 0-based
    # position 15 (page token 16) is the last slot of physical block 7
    # (7*16 + 15 = 127) and position 32 (page token 33) opens logical block 2
    # = physical block 3 (3*16 = 48).
    assert slots[17] == 337 and slots[15] == 127 and slots[32] == 48 and slots[0] == 112
    # Materialising through the table restores the logical order: fill each
    # slot with its own number and read the sequence back.
    pool = np.full((nb, 1, 16, 1), np.nan, dtype=np.float32)
    for b in range(nb):
        pool[b, 0, :, 0] = np.arange(16) + 16 * b
    seq = paged.materialise(pool, table[0], 33)[0, :, 0]
    expect = list(range(112, 128)) + list(range(336, 352)) + [48]
    assert seq.tolist() == expect


def test_block_table_example():
    check_block_table_example()


# ------------------------------------------------------------ scatter / copy
def check_scatter_roundtrip():
    rng = np.random.default_rng(5)
    nb, hkv, d = 12, 2, 8
    for storage in ("f32", "bf16"):
        pool = paged.new_pool(nb, hkv, d, storage)
        new = _rand_q(rng, (5, hkv, d), storage)
        slots = np.array([17, -1, 33, 190, 16], dtype=np.int64)
        paged.scatter(pool, new, slots)
        for t, s in enumerate(slots):
            if s < 0:
                continue
            assert np.array_equal(pool[s // 16, :, s % 16, :], new[t])
        # slot -1 wrote nothing: exactly 4 token rows are non-NaN
        finite = ~np.isnan(paged.to_f64(pool)).any(axis=3)
        assert finite.sum() == 4 * hkv
        paged.copy_blocks(pool, [(1, 5), (2, 7)])
        assert pool[5].tobytes() == pool[1].tobytes() and pool[7].tobytes() == pool[2].tobytes()


def test_scatter_roundtrip():
    check_scatter_roundtrip()


def check_copy_blocks_direction():
    """Copy-on-write gives the writer a private copy of the shared block
    ("(2) vLLM Internals ...", 1.2 "Three Direct Wins", item 2): after a
    (src, dst) pair, dst holds src's former bytes and src is unchanged. Every
    block starts with distinct finite contents, so a copy run the wrong way
    (or a swap) shows. Pairs apply in order: a chain (a, b), (b, c) carries
    a's bytes on to c."""
    rng = np.random.default_rng(15)
    nb, hkv, d = 9, 2, 8
    for storage in ("f32", "bf16"):
        pool = _rand_pool(rng, nb, hkv, d, storage)
        before = pool.copy()
        assert all(not np.array_equal(before[i], before[j]) for i in range(nb) for j in range(i))
        paged.copy_blocks(pool, [(1, 5), (2, 7), (5, 8)])
        assert pool[5].tobytes() == before[1].tobytes()
        assert pool[7].tobytes() == before[2].tobytes()
        assert pool[8].tobytes() == before[1].tobytes()
        for b in (0, 1, 2, 3, 4, 6):
            assert pool[b].tobytes() == before[b].tobytes()
        pool2 = before.copy()
        paged.copy_blocks(pool2, np.array([[3, 4]], dtype=np.int64))
        assert pool2[4].tobytes() == before[3].tobytes() and pool2[3].tobytes() == before[3].tobytes()


def test_copy_blocks_direction():
    check_copy_blocks_direction()


def check_cow_fork_append_stream():
    """End to end on the CPU: a parent with a partially filled last block is
    forked, both then append into that shared block. The allocator model
    emits a copy-on-write pair for the first writer, the oracle applies it
    with copy_blocks before scattering the step's tokens ("vLLM: what
    PagedAttention turned into", "What a block hash actually is": a shared
    tail is redirected into a private copy-on-write block), and decode over
    the paged pools must equal unpaged attention over each sequence's own
    tokens (attend_sequence). Fresh blocks hold NaN, so a copy that is
    missing or runs the wrong way poisons an output."""
    rng = np.random.default_rng(16)
    hq, hkv, d, nb = 4, 2, 8, 24
    a = amodel.AllocatorModel(nb)
    kp = paged.new_pool(nb, hkv, d, "f32")
    vp = paged.new_pool(nb, hkv, d, "f32")
    toks = {}

    def put(sid, n):
        slots, pairs = a.append(sid, n)
        paged.copy_blocks(kp, pairs)
        paged.copy_blocks(vp, pairs)
        k = rng.standard_normal((n, hkv, d)).astype(np.float32)
        v = rng.standard_normal((n, hkv, d)).astype(np.float32)
        paged.scatter(kp, k, slots)
        paged.scatter(vp, v, slots)
        pk, pv = toks.get(sid, (np.zeros((0, hkv, d), np.float32),) * 2)
        toks[sid] = (np.concatenate([pk, k]), np.concatenate([pv, v]))
        return pairs

    a.add(1)
    assert put(1, 21) == []                    # blocks 1 (full) and 2 (5 tokens)
    a.fork(1, 2)
    toks[2] = (toks[1][0].copy(), toks[1][1].copy())
    a.fork(1, 3)
    toks[3] = (toks[1][0].copy(), toks[1][1].copy())
    pairs = put(2, 3)                          # the child writes into the shared tail first
    assert len(pairs) == 1 and pairs[0][0] == a.blocks[1][1] and pairs[0][1] == a.blocks[2][1]
    assert put(3, 14) != []                    # a second child: its own private copy
    assert put(1, 2) == []                     # the parent is the last holder: in place
    assert put(2, 30) == []
    sids = [1, 2, 3]
    table, lens = a.block_table(sids, 4)
    q = rng.standard_normal((3, hq, d)).astype(np.float32)
    out = paged.decode(q, kp, vp, table, lens, 0.4)
    for i, sid in enumerate(sids):
        k, v = toks[sid]
        ref = paged.attend_sequence(q[i:i + 1], k, v, [k.shape[0] - 1], 0.4)
        assert np.isfinite(out[i]).all()
        assert np.max(np.abs(out[i] - ref[0])) < 1e-12


def test_cow_fork_append_stream():
    check_cow_fork_append_stream()


def test_bf16_widening_exact():
    # 1.0, -2.0, 0.5, max finite, smallest normal, a subnormal, 1 + 2^-7
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x7F7F, 0x0080, 0x0001, 0x3F81], dtype=np.uint16)
    expect = [1.0, -2.0, 0.5, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -126, 2.0 ** -133, 1 + 2 ** -7]
    assert paged.to_f64(bits).tolist() == expect
    assert [brute._bf16_bits_to_float(int(b)) for b in bits] == expect


# ---------------------------------------------------------------- brute force
def check_decode_vs_brute():
    rng = np.random.default_rng(11)
    for storage, hq, hkv, d in (("f32", 4, 2, 8), ("bf16", 6, 3, 4), ("f32", 2, 2, 5)):
        lens = [0, 1, 15, 16, 17, 33]
        nb = 40
        maxb = 4
        kp = _rand_pool(rng, nb, hkv, d, storage)
        vp = _rand_pool(rng, nb, hkv, d, storage)
        table = _random_tables(rng, nb, lens, maxb)
        q = _rand_q(rng, (len(lens), hq, d), storage)
        scale = 0.37
        ref = paged.decode(q, kp, vp, table, lens, scale)
        bq, bk, bv = brute.widen(q, storage), brute.widen(kp, storage), brute.widen(vp, storage)
        out = np.array(brute.decode(bq, bk, bv, table.tolist(), lens, scale))
        assert np.max(np.abs(out - ref)) < 1e-12


def test_decode_vs_brute():
    check_decode_vs_brute()


def check_prefill_vs_brute():
    rng = np.random.default_rng(12)
    for storage, hq, hkv, d in (("f32", 4, 2, 8), ("bf16", 2, 1, 6)):
        # (cached, q_len): start at 0, mid-block start, block-aligned start
        chunks = [(0, 5), (7, 12), (16, 3)]
        lens = [c + q for c, q in chunks]
        cu = np.cumsum([0] + [q for _, q in chunks])
        nb = 30
        kp = _rand_pool(rng, nb, hkv, d, storage)
        vp = _rand_pool(rng, nb, hkv, d, storage)
        table = _random_tables(rng, nb, lens, 3)
        q = _rand_q(rng, (int(cu[-1]), hq, d), storage)
        ref = paged.prefill_chunk(q, cu, lens, kp, vp, table, 0.5)
        out = np.array(brute.prefill_chunk(brute.widen(q, storage), cu, lens, brute.widen(kp, storage),
                                           brute.widen(vp, storage), table.tolist(), 0.5))
        assert np.max(np.abs(out - ref)) < 1e-12


def test_prefill_vs_brute():
    check_prefill_vs_brute()


def check_attend_sequence():
    """Dense causal attention of one sequence against the brute-force
    chunked prefill over the same tokens laid out in a pool, and its closed
    form at position 0 (the output is v_0)."""
    rng = np.random.default_rng(21)
    for hq, hkv, d in ((4, 2, 8), (3, 3, 5)):
        n = 37
        k = rng.standard_normal((n, hkv, d)).astype(np.float32)
        v = rng.standard_normal((n, hkv, d)).astype(np.float32)
        kp, vp, table = _single_seq_pools(k, v)
        pos = [0, 5, 15, 16, 36]
        q = rng.standard_normal((len(pos), hq, d)).astype(np.float32)
        out = paged.attend_sequence(q, k, v, pos, 0.6)
        for i, p in enumerate(pos):
            ref = np.array(brute.prefill_chunk(q[i:i + 1].astype(np.float64).tolist(), [0, 1], [p + 1],
                                               kp.astype(np.float64).tolist(),
                                               vp.astype(np.float64).tolist(), table.tolist(), 0.6))
            assert np.max(np.abs(out[i] - ref[0])) < 1e-12
        group = hq // hkv
        for h in range(hq):
            assert np.array_equal(out[0, h], v[0, h // group].astype(np.float64))


def test_attend_sequence():
    check_attend_sequence()


# --------------------------------------------------------------- closed forms
def _single_seq_pools(k_tokens, v_tokens):
    """Pools holding one sequence's tokens [n, H, D] in blocks 1, 2, ...
    (float32)."""
    n, h, d = k_tokens.shape
    m = -(-n // 16)
    kp = np.full((m + 1, h, 16, d), np.nan, dtype=np.float32)
    vp = np.full((m + 1, h, 16, d), np.nan, dtype=np.float32)
    for p in range(n):
        kp[1 + p // 16, :, p % 16] = k_tokens[p]
        vp[1 + p // 16, :, p % 16] = v_tokens[p]
    table = np.arange(1, m + 1, dtype=np.int32)[None, :]
    return kp, vp, table


def check_two_token_closed_form():
    """q = e0, k0 = e0, k1 = e1, scale s: z = (s, 0), so the output is
    (e^s v0 + v1) / (e^s + 1)."""
    for s in (1.0, 2.0, 0.25):
        k = np.array([[[1.0, 0.0]], [[0.0, 1.0]]], dtype=np.float32)     # [2, 1, 2]
        v = np.array([[[3.0, -1.0]], [[-2.0, 5.0]]], dtype=np.float32)
        kp, vp, table = _single_seq_pools(k, v)
        q = np.array([[[1.0, 0.0]]], dtype=np.float32)
        out = paged.decode(q, kp, vp, table, [2], s)[0, 0]
        w0, w1 = math.exp(s), 1.0
        expect = [(w0 * 3.0 + w1 * -2.0) / (w0 + w1), (w0 * -1.0 + w1 * 5.0) / (w0 + w1)]
        assert np.max(np.abs(out - expect)) < 1e-14


def test_two_token_closed_form():
    check_two_token_closed_form()


def check_single_token_is_value():
    """Context length 1: the softmax weight is exactly 1, so o = v_0."""
    rng = np.random.default_rng(3)
    k = rng.standard_normal((1, 2, 8)).astype(np.float32)
    v = rng.standard_normal((1, 2, 8)).astype(np.float32)
    kp, vp, table = _single_seq_pools(k, v)
    q = rng.standard_normal((1, 4, 8)).astype(np.float32)
    out = paged.decode(q, kp, vp, table, [1], 0.3)
    assert np.array_equal(out[0, :2], np.repeat(v[0, :1].astype(np.float64), 2, 0))
    assert np.array_equal(out[0, 2:], np.repeat(v[0, 1:].astype(np.float64), 2, 0))
    # prefill: the first query of a chunk starting at position 0 sees only itself
    out = paged.prefill_chunk(q, [0, 1], [1], kp, vp, table, 0.3)
    assert np.array_equal(out[0, :2], np.repeat(v[0, :1].astype(np.float64), 2, 0))


def test_single_token_is_value():
    check_single_token_is_value()


def check_uniform_scores_give_mean():
    """Equal keys (or a zero query) make every weight 1/n: o = mean of V."""
    rng = np.random.default_rng(4)
    n = 37
    k = np.repeat(rng.standard_normal((1, 1, 8)).astype(np.float32), n, 0)
    v = rng.standard_normal((n, 1, 8)).astype(np.float32)
    kp, vp, table = _single_seq_pools(k, v)
    q = rng.standard_normal((1, 1, 8)).astype(np.float32)
    out = paged.decode(q, kp, vp, table, [n], 1.0)[0, 0]
    assert np.max(np.abs(out - v[:, 0].astype(np.float64).mean(0))) < 1e-14
    k2 = rng.standard_normal((n, 1, 8)).astype(np.float32)
    kp2, vp2, table2 = _single_seq_pools(k2, v)
    out = paged.decode(np.zeros((1, 1, 8), np.float32), kp2, vp2, table2, [n], 1.0)[0, 0]
    assert np.max(np.abs(out - v[:, 0].astype(np.float64).mean(0))) < 1e-14


def test_uniform_scores_give_mean():
    check_uniform_scores_give_mean()


def check_dominant_key():
    """One key aligned with a large query dominates: o -> v_j."""
    rng = np.random.default_rng(6)
    n, j = 40, 23
    k = (0.01 * rng.standard_normal((n, 1, 8))).astype(np.float32)
    k[j, 0, :] = 1.0
    v = rng.standard_normal((n, 1, 8)).astype(np.float32)
    kp, vp, table = _single_seq_pools(k, v)
    q = np.full((1, 1, 8), 10.0, dtype=np.float32)
    out = paged.decode(q, kp, vp, table, [n], 1.0)[0, 0]
    assert np.max(np.abs(out - v[j, 0])) < 1e-12


def test_dominant_key():
    check_dominant_key()


def check_gqa_mapping():
    """Query head h reads KV head h // (Hq/Hkv): with V of KV head g constant
    g+1, query head h's output is exactly h // G + 1."""
    rng = np.random.default_rng(7)
    hq, hkv, n = 8, 2, 20
    k = rng.standard_normal((n, hkv, 4)).astype(np.float32)
    v = np.zeros((n, hkv, 4), np.float32)
    for g in range(hkv):
        v[:, g, :] = g + 1
    kp, vp, table = _single_seq_pools(k, v)
    q = rng.standard_normal((1, hq, 4)).astype(np.float32)
    out = paged.decode(q, kp, vp, table, [n], 0.5)[0]
    expect = np.array([h // (hq // hkv) + 1 for h in range(hq)], np.float64)
    assert np.max(np.abs(out - expect[:, None])) < 1e-14
    cu = [0, 1]
    outp = paged.prefill_chunk(q, cu, [n], kp, vp, table, 0.5)[0]
    assert np.max(np.abs(outp - expect[:, None])) < 1e-14


def test_gqa_mapping():
    check_gqa_mapping()


# ----------------------------------------------------------------- invariants
def check_placement_and_sharing_invariance():
    """Output depends only on logical content: any physical placement, and a
    shared prefix held once versus copied per sequence, give identical bits."""
    rng = np.random.default_rng(8)
    hq, hkv, d = 4, 2, 8
    prefix, suffixes = 48, [5, 16, 30]
    lens = [prefix + x for x in suffixes]
    pk = rng.standard_normal((prefix, hkv, d)).astype(np.float32)
    pv = rng.standard_normal((prefix, hkv, d)).astype(np.float32)
    seqs = []
    for x in suffixes:
        sk = rng.standard_normal((x, hkv, d)).astype(np.float32)
        sv = rng.standard_normal((x, hkv, d)).astype(np.float32)
        seqs.append((np.concatenate([pk, sk]), np.concatenate([pv, sv])))
    q = rng.standard_normal((3, hq, d)).astype(np.float32)
    nb = 40
    outs = []
    for trial in range(3):
        ids = list(rng.permutation(np.arange(1, nb)))
        kp = paged.new_pool(nb, hkv, d, "f32")
        vp = paged.new_pool(nb, hkv, d, "f32")
        table = np.zeros((3, 6), np.int32)
        shared = trial == 2
        pre = [ids.pop() for _ in range(3)] if shared else None
        for s, (ks, vs) in enumerate(seqs):
            m = -(-lens[s] // 16)
            row = list(pre) + [ids.pop() for _ in range(m - 3)] if shared else [ids.pop() for _ in range(m)]
            table[s, :m] = row
            slots = [row[p // 16] * 16 + p % 16 for p in range(lens[s])]
            paged.scatter(kp, ks, slots)
            paged.scatter(vp, vs, slots)
        outs.append(paged.decode(q, kp, vp, table, lens, 0.35))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_placement_and_sharing_invariance():
    check_placement_and_sharing_invariance()


def check_causal_mask():
    """Query i of a chunk starting at p0 sees positions 0..p0+i: changing
    K/V after p0+i leaves it unchanged, changing position p0+i changes it."""
    rng = np.random.default_rng(9)
    hkv, d, cached, qlen = 1, 8, 19, 9
    n = cached + qlen
    k = rng.standard_normal((n, hkv, d)).astype(np.float32)
    v = rng.standard_normal((n, hkv, d)).astype(np.float32)
    q = rng.standard_normal((qlen, 2, d)).astype(np.float32)
    kp, vp, table = _single_seq_pools(k, v)
    base = paged.prefill_chunk(q, [0, qlen], [n], kp, vp, table, 0.4)
    for i in (0, 4, qlen - 1):
        p = cached + i
        if p + 1 < n:
            k2, v2 = k.copy(), v.copy()
            k2[p + 1:] += 1.0
            v2[p + 1:] -= 3.0
            kp2, vp2, _ = _single_seq_pools(k2, v2)
            out = paged.prefill_chunk(q, [0, qlen], [n], kp2, vp2, table, 0.4)
            assert np.array_equal(out[i], base[i])
        v3 = v.copy()
        v3[p] += 1.0
        kp3, vp3, _ = _single_seq_pools(k, v3)
        out = paged.prefill_chunk(q, [0, qlen], [n], kp3, vp3, table, 0.4)
        assert not np.array_equal(out[i], base[i])


def test_causal_mask():
    check_causal_mask()


def check_prefill_matches_decode_and_splits():
    """A one-query chunk equals decode at the same length, and one chunk
    equals two consecutive half chunks."""
    rng = np.random.default_rng(10)
    hq, hkv, d, n, qlen = 4, 2, 8, 45, 12
    k = rng.standard_normal((n, hkv, d)).astype(np.float32)
    v = rng.standard_normal((n, hkv, d)).astype(np.float32)
    kp, vp, table = _single_seq_pools(k, v)
    q = rng.standard_normal((qlen, hq, d)).astype(np.float32)
    full = paged.prefill_chunk(q, [0, qlen], [n], kp, vp, table, 0.3)
    first = paged.prefill_chunk(q[:5], [0, 5], [n - qlen + 5], kp, vp, table, 0.3)
    second = paged.prefill_chunk(q[5:], [0, qlen - 5], [n], kp, vp, table, 0.3)
    assert np.array_equal(np.concatenate([first, second]), full)
    for i in (0, 7, qlen - 1):
        dec = paged.decode(q[i:i + 1], kp, vp, table, [n - qlen + i + 1], 0.3)
        assert np.array_equal(dec[0], full[i])


def test_prefill_matches_decode_and_splits():
    check_prefill_matches_decode_and_splits()


def test_empty_sequence_gives_zeros():
    kp = paged.new_pool(3, 1, 4, "f32")
    vp = paged.new_pool(3, 1, 4, "f32")
    out = paged.decode(np.ones((1, 2, 4), np.float32), kp, vp, np.zeros((1, 1), np.int32), [0], 1.0)
    assert np.array_equal(out, np.zeros_like(out))


# ----------------------------------------------------------- allocator model
def check_allocator_policy():
    a = amodel.AllocatorModel(10)
    assert a.null_block == 0 and a.num_free() == 9
    a.add(1)
    s1, _ = a.append(1, 20)                   # blocks 1, 2
    a.add(2)
    s2, _ = a.append(2, 40)                   # blocks 3, 4, 5
    assert sorted({x // 16 for x in s1}) == [1, 2] and sorted({x // 16 for x in s2}) == [3, 4, 5]
    a.free_seq(2)                             # visited tail first: 5, 4, 3
    assert list(a.free)[:3] == [5, 4, 3]      # the tail is reused first (LIFO)
    a.add(3)
    s3, _ = a.append(3, 16)
    assert s3[0] // 16 == 5
    # sharing and copy-on-write
    a.fork(1, 4)                              # seq 1 has 20 tokens: block 2 is partial
    assert a.ref[1] == 2 and a.ref[2] == 2
    _, pairs = a.append(4, 1)
    new_tail = a.blocks[4][-1]
    assert pairs == [(2, new_tail)] and a.ref[2] == 1 and a.ref[new_tail] == 1
    # the last sharer appends in place
    _, pairs = a.append(1, 1)
    assert pairs == []
    # full shared blocks are never copied
    a.add(5)
    a.append(5, 32)
    a.fork(5, 6)
    _, pairs = a.append(6, 3)
    assert pairs == []
    # failure leaves the state unchanged
    before = (list(a.free), {k: list(v) for k, v in a.blocks.items()}, dict(a.length), list(a.ref))
    with pytest.raises(amodel.OutOfBlocks):
        a.batch_append([1, 3], [16, 16 * 20])
    assert before == (list(a.free), {k: list(v) for k, v in a.blocks.items()}, dict(a.length), list(a.ref))


def test_allocator_policy():
    check_allocator_policy()


def check_allocator_invariants():
    """Random op streams: block 0 never handed out, refcounts equal table
    references, free + used = NB - 1, waste per sequence within the page's
    bound of 15 tokens."""
    bound = FACTS["waste_bound"]["max_wasted_tokens_per_sequence"]
    rng = np.random.default_rng(13)
    a = amodel.AllocatorModel(64)
    live = []
    nxt = 0
    for _ in range(400):
        op = rng.integers(0, 4)
        try:
            if op == 0 or not live:
                a.add(nxt)
                live.append(nxt)
                nxt += 1
            elif op == 1:
                sid = int(rng.choice(live))
                a.append(sid, int(rng.integers(1, 40)))
            elif op == 2:
                a.fork(int(rng.choice(live)), nxt)
                live.append(nxt)
                nxt += 1
            else:
                sid = int(rng.choice(live))
                a.free_seq(sid)
                live.remove(sid)
        except amodel.OutOfBlocks:
            pass
        refs = {}
        for sid, blocks in a.blocks.items():
            assert 0 not in blocks
            n = a.length[sid]
            assert 0 <= 16 * len(blocks) - n <= bound
            for b in blocks:
                refs[b] = refs.get(b, 0) + 1
        assert all(a.ref[b] == c for b, c in refs.items())
        assert sum(1 for r in a.ref if r > 0) + a.num_free() == 63
        assert 0 not in a.free


def test_allocator_invariants():
    check_allocator_invariants()


def check_utilisation_formula():
    """With the tail waste uniform on 0..15 (mean 7.5) and mean length L, the
    share of in-use slots holding tokens is L / (L + 7.5); page 2 solves it for
    u = 0.963 at L ~ 195."""
    f = FACTS["utilisation_check"]
    rng = np.random.default_rng(14)
    n = 4000
    # lengths 16*m - w with w uniform on 0..15 and mean length 195
    w = rng.integers(0, 16, size=n)
    m = rng.integers(11, 15, size=n)            # mean 16*12.5 - 7.5 = 192.5
    lengths = 16 * m - w
    a = amodel.AllocatorModel(int((16 * m).sum() // 16) + 2)
    for i, L in enumerate(lengths.tolist()):
        a.add(i)
        a.append(i, L)
    st = a.stats()
    L = lengths.mean()
    assert abs(st["utilisation"] - L / (L + f["mean_tail_waste_tokens"])) < 2e-3
    # the page's own number: u at L = 195
    assert abs(f["mean_sequence_tokens"] / (f["mean_sequence_tokens"] + f["mean_tail_waste_tokens"])
               - f["utilisation"]) < 5e-4


def test_utilisation_formula():
    check_utilisation_formula()


# ---------------------------------------------------------- planted mistakes
def _raises(check):
    try:
        check()
    except AssertionError:
        return True
    return False


ALL_CHECKS = [check_block_table_example, check_scatter_roundtrip, check_copy_blocks_direction,
              check_cow_fork_append_stream, check_two_token_closed_form,
              check_single_token_is_value, check_uniform_scores_give_mean, check_dominant_key,
              check_gqa_mapping, check_placement_and_sharing_invariance, check_causal_mask,
              check_prefill_matches_decode_and_splits, check_allocator_policy,
              check_allocator_invariants, check_utilisation_formula, check_attend_sequence]


def _mut_no_scale(q, k, v, scale):
    return _orig_attend(q, k, v, 1.0)


def _mut_softmax_sign(q, k, v, scale):
    return _orig_attend(q, k, v, -scale)


def _mut_no_max_shift(q, k, v, scale):
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]))
    w = np.exp(scale * (q @ k.T))
    return (w @ v) / (w.sum(axis=1, keepdims=True) + 1e-3)


def _mut_transposed_value(q, k, v, scale):
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]))
    z = scale * (q @ k.T)
    w = np.exp(z - z.max(axis=1, keepdims=True))
    return (w @ v[::-1]) / w.sum(axis=1, keepdims=True)


_orig_attend = paged._softmax_attend


def _mut_materialise_reversed(pool, table_row, n):
    nb = -(-n // 16)
    row = list(np.asarray(table_row)[:nb])[::-1] + list(np.asarray(table_row)[nb:])
    return _orig_materialise(pool, np.array(row), n)


def _mut_materialise_offset(pool, table_row, n):
    out = _orig_materialise(pool, table_row, n)
    return np.roll(out, 1, axis=1)


_orig_materialise = paged.materialise


def _mut_gqa_modulo(q, k_pool, v_pool, table, lens, scale):
    qf = paged.to_f64(q)
    S, hq, _ = qf.shape
    hkv = k_pool.shape[1]
    out = np.zeros(qf.shape)
    for s in range(S):
        ks = paged.materialise(k_pool, table[s], int(lens[s]))
        vs = paged.materialise(v_pool, table[s], int(lens[s]))
        for h in range(hq):
            out[s, h] = paged._softmax_attend(qf[s, h:h + 1], ks[h % hkv], vs[h % hkv], scale)[0]
    return out


def _mut_causal_off_by_one(q, cu, lens, kp, vp, table, scale):
    out = _orig_prefill(q, cu, lens, kp, vp, table, scale)
    # shift: query i sees one position fewer
    alt = _orig_prefill(q, cu, [int(x) - 1 for x in lens], kp, vp, table, scale)
    return alt if max(int(x) for x in lens) > 1 else out


_orig_prefill = paged.prefill_chunk


def _mut_sequence_window_short(q, k, v, positions, scale):
    return _orig_sequence(q, k, v, [max(0, p - 1) for p in positions], scale)


_orig_sequence = paged.attend_sequence


def _mut_copy_reversed(pool, pairs):
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2).tolist():
        pool[src] = pool[dst]


class _FifoModel(amodel.AllocatorModel):
    def free_seq(self, sid):
        released = []
        for b in reversed(self.blocks.pop(sid)):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                released.append(b)
        del self.length[sid]
        self.free.extend(released)


class _HeadFirstModel(amodel.AllocatorModel):
    def free_seq(self, sid):
        released = []
        for b in self.blocks.pop(sid):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                released.append(b)
        del self.length[sid]
        self.free.extendleft(reversed(released))


class _NoCowModel(amodel.AllocatorModel):
    def _needs(self, sid, n):
        cow, grow = super()._needs(sid, n)
        return False, grow


class _SlotOffByOne(amodel.AllocatorModel):
    def _append(self, sid, n):
        slots, pairs = super()._append(sid, n)
        return [s + 1 for s in slots], pairs


MUTANTS = {
    "scale dropped": (paged, "_softmax_attend", _mut_no_scale),
    "score sign flipped": (paged, "_softmax_attend", _mut_softmax_sign),
    "unnormalised softmax": (paged, "_softmax_attend", _mut_no_max_shift),
    "values in wrong order": (paged, "_softmax_attend", _mut_transposed_value),
    "table walked backwards": (paged, "materialise", _mut_materialise_reversed),
    "token offset shifted": (paged, "materialise", _mut_materialise_offset),
    "kv head h % Hkv": (paged, "decode", _mut_gqa_modulo),
    "causal window one short": (paged, "prefill_chunk", _mut_causal_off_by_one),
    "sequence window one short": (paged, "attend_sequence", _mut_sequence_window_short),
    "copy-on-write copy reversed": (paged, "copy_blocks", _mut_copy_reversed),
    "FIFO free list": (amodel, "AllocatorModel", _FifoModel),
    "head-first free": (amodel, "AllocatorModel", _HeadFirstModel),
    "no copy-on-write": (amodel, "AllocatorModel", _NoCowModel),
    "slot off by one": (amodel, "AllocatorModel", _SlotOffByOne),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    module, attr, repl = MUTANTS[name]
    monkeypatch.setattr(module, attr, repl)
    caught = [c.__name__ for c in ALL_CHECKS if _raises(c)]
    assert caught, "no pin catches the planted mistake: %s" % name
