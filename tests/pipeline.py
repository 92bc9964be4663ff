"""One step of the hot path, run twice from the same seeded workload:

* ``run_native`` -- through libpkv (C++ allocator, HIP kernels) on the GPU;
* ``run_oracle`` -- through the CPU oracle (Python allocator model, NumPy).

The two share only the workload's random draws; each builds its own block
tables, slots and pools. The step: replay the allocator script that places
every sequence's cached tokens (writing their K/V into the pool), append the
step's new tokens (one per decode sequence, a chunk per prefill sequence),
write their K/V, then run decode attention for the decode sequences and
chunked-prefill attention for the chunks.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np
import torch

import workloads
from oracle import allocator as amodel
from oracle import paged


def to_numpy_storage(t: torch.Tensor) -> np.ndarray:
    """CPU tensor -> the oracle's storage (float32 values or bf16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _positions(w: workloads.Workload):
    """For every append of the setup script: (seq, first position, count)."""
    cur: Dict[int, int] = {}
    out = []
    for op in w.setup_ops():
        if op[0] == "add":
            cur[op[1]] = 0
        elif op[0] == "fork":
            cur[op[2]] = cur[op[1]]
        else:
            out.append((op[1], cur[op[1]], op[2]))
            cur[op[1]] += op[2]
    return out


class KVCache:
    """Per-sequence K/V draws, generated lazily."""

    def __init__(self, w: workloads.Workload):
        self.w = w
        self.specs = {s.seq_id: s for s in w.seqs}
        self._cache = {}

    def get(self, sid: int):
        if sid not in self._cache:
            self._cache[sid] = self.w.seq_kv(self.specs[sid])
        return self._cache[sid]

    def drop(self, sid: int):
        self._cache.pop(sid, None)


def run_native(w: workloads.Workload, device="cuda", keep_pools: bool = True,
               prefill: bool = True, fused_append: bool = False,
               prefill_workspace: bool = True) -> dict:
    """``fused_append``: the decode sequences' new tokens are not scattered
    by reshape_and_cache but written by the decode itself (decode_append);
    the chunks' tokens still go through reshape_and_cache.
    ``prefill_workspace``: the prefill gets the workspace the library asks
    for (position parts when the launch has few row blocks; kept as
    res["prefill_ws"]); False runs it without one."""
    import paged_kv_cache_233_amd as pkv

    dt = w.torch_dtype
    a = pkv.Allocator(w.num_blocks)
    if w.free_order is not None:
        a.set_free_order(w.free_order)
    shape = (w.num_blocks, w.num_kv_heads, 16, w.head_dim)
    kc = torch.full(shape, float("nan"), dtype=dt, device=device)
    vc = torch.full(shape, float("nan"), dtype=dt, device=device)
    kv = KVCache(w)
    script = _positions(w)
    res_pairs = []
    j = 0
    for op in w.setup_ops():
        if op[0] == "add":
            a.add(op[1])
        elif op[0] == "fork":
            a.fork(op[1], op[2])
        else:
            sid, p0, n = script[j]
            slots, pairs = a.append(sid, n)
            if pairs:   # copy-on-write of a shared, partially filled last block
                pkv.copy_blocks(kc, vc, torch.tensor(pairs, dtype=torch.int64, device=device))
                res_pairs.extend(pairs)
            k, v = kv.get(sid)
            pkv.reshape_and_cache(kc, vc, k[p0:p0 + n].to(device), v[p0:p0 + n].to(device),
                                  torch.from_numpy(slots).to(device))
            j += 1
    # the step: new tokens of every sequence, one batched append and scatter
    ids, ns = w.step_appends()
    slots, pairs = a.batch_append(ids, ns)
    if pairs:
        pkv.copy_blocks(kc, vc, torch.tensor(pairs, dtype=torch.int64, device=device))
        res_pairs.extend(pairs)
    ks, vs, keep = [], [], []
    for sid, n in zip(ids, ns):
        k, v = kv.get(sid)
        spec = kv.specs[sid]
        fused = fused_append and not spec.is_chunk
        keep += [not fused] * n
        if not fused:
            ks.append(k[spec.cached:spec.total])
            vs.append(v[spec.cached:spec.total])
    if ks:
        sl = slots[np.array(keep, dtype=bool)]
        pkv.reshape_and_cache(kc, vc, torch.cat(ks).to(device), torch.cat(vs).to(device),
                              torch.from_numpy(np.ascontiguousarray(sl)).to(device))
    res = {"step_slots": slots, "cow_pairs": res_pairs}
    dec = w.decode_seqs
    maxb = w.max_blocks_per_seq()
    if dec:
        sids = [s.seq_id for s in dec]
        table, lens = a.block_table(sids, maxb)
        q = torch.cat([w.seq_q(s) for s in dec]).to(device)
        out = torch.empty_like(q)
        ws = pkv.decode_workspace(len(dec), w.num_q_heads, w.num_kv_heads, w.head_dim, device)
        if fused_append:
            # one new K/V row per decode sequence (zeros for an empty one,
            # which has no position to write)
            k_new = torch.zeros((len(dec), w.num_kv_heads, w.head_dim), dtype=dt)
            v_new = torch.zeros_like(k_new)
            for i, spec in enumerate(dec):
                if spec.new_tokens:
                    k, v = kv.get(spec.seq_id)
                    k_new[i], v_new[i] = k[spec.total - 1], v[spec.total - 1]
            pkv.decode_append(out, q, k_new.to(device), v_new.to(device), kc, vc,
                              torch.from_numpy(table).to(device), torch.from_numpy(lens).to(device),
                              w.scale, ws)
        else:
            pkv.decode(out, q, kc, vc, torch.from_numpy(table).to(device),
                       torch.from_numpy(lens).to(device), w.scale, ws)
        res["decode"] = out
        res["decode_table"] = table
        res["decode_lens"] = lens
    ch = w.chunk_seqs
    if ch and prefill:
        sids = [s.seq_id for s in ch]
        table, lens = a.block_table(sids, maxb)
        qs = [w.seq_q(s) for s in ch]
        cu = np.cumsum([0] + [x.shape[0] for x in qs]).astype(np.int32)
        q = torch.cat(qs).to(device)
        out = torch.empty_like(q)
        qmax = int(max(x.shape[0] for x in qs))
        pws = (pkv.prefill_workspace(len(ch), w.num_q_heads, w.num_kv_heads, w.head_dim, qmax, device)
               if prefill_workspace else None)
        pkv.prefill_chunk(out, q, torch.from_numpy(cu).to(device), torch.from_numpy(lens).to(device),
                          torch.from_numpy(table).to(device), kc, vc, qmax, w.scale, pws)
        res["prefill_ws"] = pws
        res["prefill"] = out
        res["prefill_table"] = table
        res["prefill_lens"] = lens
        res["prefill_cu"] = cu
    torch.cuda.synchronize()
    if keep_pools:
        res["k_cache"], res["v_cache"] = kc, vc
    res["allocator"] = a
    return res


def run_oracle(w: workloads.Workload, decode_sample: Optional[Sequence[int]] = None,
               prefill: bool = True) -> dict:
    """The oracle's step. ``decode_sample`` restricts which decode sequences
    (indices into w.decode_seqs) are attended and written to the pool (the
    rest of the pool keeps its NaN canaries); None means all."""
    storage = w.dtype
    m = amodel.AllocatorModel(w.num_blocks)
    if w.free_order is not None:
        m.set_free_order(w.free_order.tolist())
    dec = w.decode_seqs
    keep = set(s.seq_id for s in w.seqs)
    if decode_sample is not None:
        keep = set(dec[i].seq_id for i in decode_sample) | set(s.seq_id for s in w.chunk_seqs)
        # forked sequences need their owner's shared tokens
        keep |= set(s.fork_of for s in w.seqs if s.seq_id in keep and s.fork_of is not None)
    kp = paged.new_pool(w.num_blocks, w.num_kv_heads, w.head_dim, storage)
    vp = paged.new_pool(w.num_blocks, w.num_kv_heads, w.head_dim, storage)
    kv = KVCache(w)
    script = _positions(w)
    res_pairs = []
    j = 0
    for op in w.setup_ops():
        if op[0] == "add":
            m.add(op[1])
        elif op[0] == "fork":
            m.fork(op[1], op[2])
        else:
            sid, p0, n = script[j]
            slots, pairs = m.append(sid, n)
            paged.copy_blocks(kp, pairs)
            paged.copy_blocks(vp, pairs)
            res_pairs.extend(pairs)
            if sid in keep:
                k, v = kv.get(sid)
                paged.scatter(kp, to_numpy_storage(k[p0:p0 + n]), slots)
                paged.scatter(vp, to_numpy_storage(v[p0:p0 + n]), slots)
            j += 1
    ids, ns = w.step_appends()
    slots, pairs = m.batch_append(ids, ns)
    paged.copy_blocks(kp, pairs)
    paged.copy_blocks(vp, pairs)
    res_pairs.extend(pairs)
    off = 0
    for sid, n in zip(ids, ns):
        if sid in keep:
            spec = kv.specs[sid]
            k, v = kv.get(sid)
            paged.scatter(kp, to_numpy_storage(k[spec.cached:spec.total]), slots[off:off + n])
            paged.scatter(vp, to_numpy_storage(v[spec.cached:spec.total]), slots[off:off + n])
        off += n
    res = {"step_slots": np.array(slots, dtype=np.int64), "k_cache": kp, "v_cache": vp,
           "model": m, "cow_pairs": res_pairs}
    maxb = w.max_blocks_per_seq()
    if dec:
        idx = list(range(len(dec))) if decode_sample is None else list(decode_sample)
        sids = [dec[i].seq_id for i in idx]
        table, lens = m.block_table(sids, maxb)
        q = np.concatenate([to_numpy_storage(w.seq_q(dec[i])) for i in idx])
        res["decode"] = paged.decode(q, kp, vp, table, lens, w.scale)
        res["decode_index"] = idx
        full_table, full_lens = m.block_table([s.seq_id for s in dec], maxb)
        res["decode_table"], res["decode_lens"] = full_table, full_lens
    ch = w.chunk_seqs
    if ch and prefill:
        sids = [s.seq_id for s in ch]
        table, lens = m.block_table(sids, maxb)
        qs = [to_numpy_storage(w.seq_q(s)) for s in ch]
        cu = np.cumsum([0] + [x.shape[0] for x in qs])
        res["prefill"] = paged.prefill_chunk(np.concatenate(qs), cu, lens, kp, vp, table, w.scale)
        res["prefill_table"], res["prefill_lens"] = table, lens
    return res


def assert_close(gpu: torch.Tensor, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    """The parity bar: fp32 max-abs <= 1e-5; bf16 |gpu - ref| <= 2e-2 + 1e-2 |ref|
    elementwise, ref the float64 oracle. Returns error statistics."""
    g = gpu.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), "%s: non-finite output" % what
    err = np.abs(g - ref)
    stats = {"max_abs": float(err.max(initial=0.0)),
             "max_rel": float((err / np.maximum(np.abs(ref), 1e-6)).max(initial=0.0))}
    if dtype == "f32":
        assert stats["max_abs"] <= 1e-5, (what, stats)
    else:
        bad = err > 2e-2 + 1e-2 * np.abs(ref)
        assert not bad.any(), (what, stats, int(bad.sum()))
    return stats
