"""Benchmark of the paged KV-cache decode hot path on one MI355X.

One step = one decode step of one attention layer for the whole batch:
  host   append one token to every sequence (C++ allocator), fill the slot
         mapping, block table and context lengths;
  device reshape_and_cache of the new tokens' K/V and paged decode attention
         (the split-KV kernel, then the kernel that merges the partial
         states of sequences split over several waves).
The headline (value) times the device part with every input resident in
HBM: the allocator plans all steps first and one copy puts their indices on
the device before timing starts. A second leg runs the serving loop as it
would run, the allocator planning each step inside the timed loop and the
indices crossing PCIe every step (staged_step, reported beside it).
Per-kernel times come from HIP events in a separate run of the same planned
steps: event records between the kernels lengthen the step, so the wall
time (value) is taken without them.
Consecutive steps cycle through R copies of the KV pool, as consecutive
layers of a model would, so every step reads its keys and values from HBM
and not from the 256 MB last-level cache.

Workload (default): 64 sequences, context lengths uniform in [128, 4096],
32 query / 8 KV heads, head_dim 128, bf16, blocks of 16 tokens placed at
random in a pool of 1.5x the need (block 0 = null block).

Prints one JSON line (metric: KV-read GB/s over the whole step; decode
tokens/s beside it), with a roofline object for the decode kernels and the
CPU oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA
METRIC = "paged decode attention: KV-read HBM GB/s (% of peak) + tokens/s, 1 GPU"
# the sources the decode kernels are built from (the traffic record names their hash)
DECODE_SRCS = [os.path.join(ROOT, "paged_kv_cache_233_amd", "csrc", f)
               for f in ("decode.hip", "tile_attn.h")]
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_mixed_traffic.json")
PREFILL_SRCS = [os.path.join(ROOT, "paged_kv_cache_233_amd", "csrc", f)
                for f in ("prefill.hip", "tile_attn.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="long", choices=["llama", "long", "shared", "mixed"],
                    help="the headline decode workload (default: long, the largest that fits one GPU)")
    ap.add_argument("--no-side", action="store_true",
                    help="skip the side decode legs (the llama and mixed workloads' decode steps)")
    ap.add_argument("--pools", type=int, default=4, help="KV pool copies cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=64)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-shared", action="store_true",
                    help="skip the leg that times the shared-prefix decode on the shared workload")
    ap.add_argument("--no-staged", action="store_true",
                    help="skip the leg that stages the indices from pinned host memory inside "
                         "each step (PCIe-inclusive)")
    ap.add_argument("--no-mixed", action="store_true",
                    help="skip the leg that times the mixed workload's whole step (one and two streams)")
    ap.add_argument("--no-cache-ops", action="store_true",
                    help="skip the leg that times reshape_and_cache and copy_blocks alone")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the leg that replays the whole step as one HIP graph")
    ap.add_argument("--stage", choices=["kernel", "dma", "mapped"], default="kernel",
                    help="per-step indices to the device: copied by a kernel (pkv_stage_copy), "
                         "copied by the DMA engine (hipMemcpyAsync), or read in place from "
                         "pinned host memory")
    ap.add_argument("--no-stream", action="store_true",
                    help="skip the plain streaming copy/sum measurement reported beside the roofline")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device copy (for counter calibration)")
    ap.add_argument("--shared-probe", action="store_true",
                    help="only run the shared-prefix leg and print its JSON (for profiling it alone)")
    ap.add_argument("--prefill-probe", action="store_true",
                    help="only run the chunked-prefill leg on the mixed chunks and print its JSON (for profiling it alone)")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def copy_probe():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)


def scheduler_leg():
    """Host cost of the step scheduler (C++): a seeded stream of 256 requests
    (prompts U[64, 1024], 32..128 generated tokens each, all queued at once)
    run to completion over a pool of 40% of the blocks they would hold
    together (so preemption happens), token budget 2048, prefix caching on,
    no kernels (the sampled tokens are a fixed function of request and
    position). Reports microseconds per step for schedule + plan copy-out +
    update through the Python binding."""
    import numpy as np

    import paged_kv_cache_233_amd as pkv

    rng = np.random.default_rng(11)
    stems = [rng.integers(0, 32000, 16 * int(rng.integers(2, 20))).astype(np.int32) for _ in range(8)]
    reqs = []
    for r in range(256):
        stem = stems[int(rng.integers(0, len(stems)))]
        plen = int(rng.integers(64, 1025))
        keep = 16 * int(rng.integers(0, len(stem) // 16 + 1))
        prompt = np.concatenate([stem[:keep], rng.integers(0, 32000, plen).astype(np.int32)])[:plen]
        reqs.append((r, prompt, int(rng.integers(32, 129))))
    need = sum(-(-(len(p) + n - 1) // 16) for _, p, n in reqs)
    alloc = pkv.Allocator(int(0.4 * need) + 1)
    alloc.enable_prefix_caching()
    sched = pkv.Scheduler(alloc, 2048)
    for r, p, n in reqs:
        sched.add_request(r, p, n)
    steps = tokens = preempted = 0
    t0 = time.perf_counter()
    while True:
        plan = sched.schedule()
        if len(plan.req_ids) == 0:
            sched.update([])
            if sched.counts() == (0, 0):
                break
            continue
        sampled = ((plan.req_ids[plan.samples] * 7 + (plan.start + plan.num_new)[plan.samples] * 13)
                   % 32000).astype(np.int32)
        sched.update(sampled)
        steps += 1
        tokens += int(plan.num_new.sum())
        preempted += len(plan.preempted)
    el = time.perf_counter() - t0
    r = {"requests": 256, "steps": steps, "tokens_scheduled": tokens, "preemptions": preempted,
         "prefix_hit_blocks": alloc.prefix_cache_stats()["hit_blocks"],
         "us_per_step": round(el / max(steps, 1) * 1e6, 1),
         "what": "host-only scheduler loop (schedule, plan copy-out, update) over a seeded stream; "
                 "pool 40% of the blocks the requests would hold together; budget 2048 tokens"}
    log("scheduler: %d steps, %d tokens, %d preemptions, %.1f us per step"
        % (steps, tokens, preempted, r["us_per_step"]))
    return r


def stream_leg(dev):
    """What plain streaming reaches on this GPU, as the practical ceiling
    beside the decode roofline: the library's streaming-read kernel over
    2 GiB (best of three grid sizes), and a torch device-to-device copy of
    2 GiB (read + written bytes) for comparison; each the median of 10 timed
    runs over four buffers in turn (8 GiB, past the last-level cache)."""
    import numpy as np
    import torch

    import paged_kv_cache_233_amd as pkv

    n = 2 << 30
    bufs = [torch.ones(n // 2, dtype=torch.bfloat16, device=dev) for _ in range(4)]
    dst = torch.empty_like(bufs[0])
    words = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    hip = HipEvents()
    sh = torch.cuda.current_stream().cuda_stream

    def timed(fn):
        out = []
        for r in range(13):
            e0, e1 = hip.create(), hip.create()
            hip.record(e0, sh)
            fn(bufs[r % 4])
            hip.record(e1, sh)
            torch.cuda.synchronize()
            if r >= 3:
                out.append(hip.elapsed_us(e0, e1))
        return float(np.median(out))

    read = {}
    for wg in (1024, 2048, 4096):
        read[wg] = n / timed(lambda b: pkv.stream_read(b, words, wg, stream=sh)) / 1e3
    best = max(read, key=read.get)
    copy_us = timed(lambda b: dst.copy_(b))
    del bufs, dst
    torch.cuda.empty_cache()
    r = {"read_gbs": round(read[best], 1), "read_workgroups": best,
         "torch_copy_gbs": round(2 * n / copy_us / 1e3, 1),
         "what": "pkv_stream_read over 2 GiB (read bytes; best of 1024/2048/4096 workgroups) and "
                 "a torch device-to-device copy of 2 GiB (read + written bytes); median of 10, "
                 "four buffers in turn"}
    log("streaming: read %.1f GB/s (%d workgroups), torch copy %.1f GB/s"
        % (r["read_gbs"], best, r["torch_copy_gbs"]))
    return r


class HipEvents:
    """Timing events on the launch stream, created with
    hipEventDisableSystemFence: recording them does not write back and
    invalidate caches, so they time the commands between them without
    perturbing them (the default events do both)."""

    DISABLE_SYSTEM_FENCE = 0x20000000
    DISABLE_TIMING = 0x2

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventQuery.argtypes = [ctypes.c_void_p]

    def create(self, timing=True):
        e = self.ct.c_void_p()
        flags = self.DISABLE_SYSTEM_FENCE | (0 if timing else self.DISABLE_TIMING)
        rc = self.lib.hipEventCreateWithFlags(self.ct.byref(e), flags)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)
        return e

    def record(self, e, stream):
        rc = self.lib.hipEventRecord(e, stream)
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def sync(self, e):
        self.lib.hipEventSynchronize(e)

    def elapsed_us(self, a, b):
        ms = self.ct.c_float()
        rc = self.lib.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return ms.value * 1e3

    def destroy(self, e):
        self.lib.hipEventDestroy(e)

    def burst_us(self, stream, launch, reps, bursts=5, prime=2):
        """Per-call time of `launch(i)`, the median over `bursts` bursts of
        `reps` calls, each burst between its own pair of events. A burst
        starts on an idle device with `prime` untimed calls queued ahead of
        its first event, so the device never waits on the host inside it. The
        events time the device, idle gaps included: a host stall of tens of
        milliseconds (the process descheduled) spoils the one burst it falls
        in, and the median drops that burst."""
        import statistics

        import torch

        per_call = []
        for _ in range(bursts):
            torch.cuda.synchronize()
            for i in range(prime):
                launch(i)
            e0, e1 = self.create(), self.create()
            self.record(e0, stream)
            for i in range(reps):
                launch(prime + i)
            self.record(e1, stream)
            self.sync(e1)
            per_call.append(self.elapsed_us(e0, e1) / reps)
            self.destroy(e0)
            self.destroy(e1)
        return statistics.median(per_call)


def kernel_source_hash(srcs=None):
    h = hashlib.sha256()
    for f in (srcs or DECODE_SRCS):
        h.update(open(f, "rb").read())
    return h.hexdigest()


def load_traffic(path, srcs=None, key="decode_source_sha256"):
    """HBM bytes per launch from a committed counter record, if it was taken
    on the current source of its kernel; else None."""
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get(key) != kernel_source_hash(srcs):
        return None
    return rec.get("traffic_bytes_per_launch")


SIDE_DECODE = ("llama", "mixed")
WORKLOAD_TEXT = {
    "llama": "llama decode: 64 seqs, ctx U[128,4096] (seeded), 32 q / 8 kv heads, head_dim 128, "
             "bf16, 16-token blocks, random placement, 1.5x pool",
    "long": "long decode (split-KV path): 8 seqs, ctx U[32768,131072] (seeded), 32 q / 8 kv heads, "
            "head_dim 128, bf16, 16-token blocks, random placement, 1.5x pool",
    "mixed": "mixed step's decode part: 16 seqs, ctx U[512,8192] (seeded), 32 q / 8 kv heads, "
             "head_dim 128, bf16, 16-token blocks, random placement, 1.5x pool",
    "shared": "shared decode: 128 seqs sharing one 2048-token prefix + suffix U[16,512], ordinary "
              "decode, 32 q / 8 kv heads, head_dim 128, bf16",
}


class Ctx:
    """Everything one decode workload's legs share (pools, inputs, buffers)."""


def decode_setup(w, args, dev, legs):
    """Allocator, pool copies and step inputs of a workload's decode legs.
    The pool has room for one new token per sequence per step of `legs`
    legs of warm-up + timed steps."""
    import numpy as np
    import torch

    import paged_kv_cache_233_amd as pkv

    c = Ctx()
    c.w = w
    dec = w.decode_seqs
    c.S = S = len(dec)
    extra = legs * (args.warmup + args.steps) + 2
    nb = w.num_blocks + S * (extra // 16 + 2)
    c.maxb = w.max_blocks_per_seq(extra)
    dt = w.torch_dtype
    log("workload %s: %d decode seqs, pool %d blocks, max %d blocks/seq" % (w.name, S, nb, c.maxb))
    c.alloc, kc0, vc0 = build_pool(w, dev, nb)
    c.pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(args.pools - 1)]
    c.sids = np.array([s.seq_id for s in dec], dtype=np.int64)
    c.ones = np.ones(S, dtype=np.int32)
    gen = torch.Generator().manual_seed(1234)
    c.q = torch.randn((S, w.num_q_heads, w.head_dim), generator=gen).to(dt).to(dev)
    c.k_new = torch.randn((S, w.num_kv_heads, w.head_dim), generator=gen).to(dt).to(dev)
    c.v_new = torch.randn((S, w.num_kv_heads, w.head_dim), generator=gen).to(dt).to(dev)
    c.out = torch.empty_like(c.q)
    c.ws = pkv.decode_workspace(S, w.num_q_heads, w.num_kv_heads, w.head_dim, dev)
    # Per-step indices: slots (int64 [S]), then context lengths (int32 [S])
    # and the block table (int32 [S, maxb]), packed in one buffer of int64
    # words.
    n32 = S + S * c.maxb
    c.words = S + (n32 + 1) // 2
    c.kv_bytes_per_token = 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
    c.pairs_buf = np.empty(2 * S, dtype=np.int64)
    return c


def resident_leg(c, args, hip, fused=True):
    """The headline measurement of one workload: the host allocator plans
    every step first (one token appended to each sequence; the slots,
    lengths and block table of step t written into slice t of one pinned
    buffer), one copy puts all slices in HBM, then every planned step
    (warm-up, then timed) runs with its indices resident: the split kernel
    with the new token's cache write folded in (decode_append) and the merge
    kernel, or with ``fused`` False, reshape_and_cache, the plain split
    kernel and the merge kernel. The planned steps run twice with the same
    plans (same slots written, same bytes read): once with HIP events around
    every kernel (per-kernel times; the event records add gaps between the
    kernels), once without (the wall time behind the value)."""
    import numpy as np
    import torch

    import paged_kv_cache_233_amd as pkv

    w, S, maxb = c.w, c.S, c.maxb
    sh = torch.cuda.current_stream().cuda_stream
    total_steps = args.warmup + args.steps
    plan_h = torch.empty((total_steps, c.words), dtype=torch.int64).pin_memory()
    h0 = time.perf_counter()
    ctx_tokens = []
    for t in range(total_steps):
        base = plan_h[t].data_ptr()
        assert c.alloc.batch_append_into(c.sids, c.ones, base, c.pairs_buf) == 0
        c.alloc.fill_block_table_into(c.sids, base + 8 * S + 4 * S, maxb, base + 8 * S)
        ctx_tokens.append(int(plan_h[t, S:].numpy().view(np.int32)[:S].sum()))
    alloc_us = (time.perf_counter() - h0) / total_steps * 1e6
    plan_d = plan_h.to(c.q.device)
    torch.cuda.synchronize()
    ev = [tuple(hip.create() for _ in range(4)) for _ in range(total_steps)]
    launch = []
    for t in range(total_steps):
        x = plan_d[t]
        slots = x[:S]
        lens = x[S:].view(torch.int32)[:S]
        table = x[S:].view(torch.int32)[S:S + S * maxb].view(S, maxb)
        kc, vc = c.pools[t % len(c.pools)]
        if fused:
            launch.append((
                None,
                pkv.decode_append(c.out, c.q, c.k_new, c.v_new, kc, vc, table, lens, w.scale, c.ws,
                                  stream=sh, phase="split", prepare=True),
                pkv.decode_append(c.out, c.q, c.k_new, c.v_new, kc, vc, table, lens, w.scale, c.ws,
                                  stream=sh, phase="merge", prepare=True)))
        else:
            launch.append((
                pkv.reshape_and_cache(kc, vc, c.k_new, c.v_new, slots, stream=sh, prepare=True),
                pkv.decode(c.out, c.q, kc, vc, table, lens, w.scale, c.ws, stream=sh, phase="split",
                           prepare=True),
                pkv.decode(c.out, c.q, kc, vc, table, lens, w.scale, c.ws, stream=sh, phase="merge",
                           prepare=True)))

    def run(events):
        def step(t):
            reshape, split, merge = launch[t]
            if not events:
                if reshape is not None:
                    reshape()
                split()
                merge()
                return
            e0, e1, e2, e3 = ev[t]
            hip.record(e0, sh)
            if reshape is not None:
                reshape()
            hip.record(e1, sh)
            split()                       # decode = split-KV kernel, then merge kernel
            hip.record(e2, sh)
            merge()
            hip.record(e3, sh)

        for t in range(args.warmup):
            step(t)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(args.warmup, total_steps):
            step(t)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    ev_wall = run(True)
    timed = range(args.warmup, total_steps)
    us = {k: np.array([hip.elapsed_us(ev[t][a], ev[t][b]) for t in timed])
          for k, (a, b) in {"reshape": (0, 1), "split": (1, 2), "merge": (2, 3),
                            "decode": (1, 3)}.items()}
    wall = run(False)
    # The split kernel's own duration: the timed steps' split launches again,
    # back to back between one pair of events (an event pair around every
    # launch adds its record overhead to each). Every slot they read was
    # written by the passes above, so they read the same bytes.
    b0, b1 = hip.create(), hip.create()
    hip.record(b0, sh)
    for t in timed:
        launch[t][1]()
    hip.record(b1, sh)
    hip.sync(b1)
    split_b2b_us = hip.elapsed_us(b0, b1) / len(timed)
    del plan_d
    kv_bytes = np.array([ctx_tokens[t] * c.kv_bytes_per_token for t in timed], dtype=np.float64)
    # the split kernel's algorithmic bytes: the K/V it reads, plus with the
    # fused write the new token's K/V read from its buffer and written once
    split_bytes = kv_bytes + (2 * S * c.kv_bytes_per_token if fused else 0)
    r = {"ctx": c, "wall": wall, "ev_wall": ev_wall, "us": us, "kv_bytes": kv_bytes,
         "split_bytes": split_bytes, "fused": fused,
         "alloc_us": alloc_us, "ms_per_step": wall / args.steps * 1e3,
         "split_b2b_us": split_b2b_us,
         "value": float(kv_bytes.sum() / wall / 1e9),
         "achieved": float(split_bytes.mean() / (split_b2b_us * 1e-6) / 1e9),
         "achieved_op": float(kv_bytes.mean() / (us["decode"].mean() * 1e-6) / 1e9)}
    log("%s%s: decode kernels mean %.1f us (min %.1f, median %.1f) = split %.1f + merge %.1f; "
        "reshape_and_cache %.1f us; step %.1f us wall (%.1f with events; indices resident) = "
        "%.1f GB/s (%.1f%% of peak); split kernel %.1f us back to back = %.1f%%; "
        "allocator %.1f us per step on the host"
        % (w.name, " (fused append)" if fused else " (reshape_and_cache + decode)",
           us["decode"].mean(), us["decode"].min(), np.median(us["decode"]),
           us["split"].mean(), us["merge"].mean(), us["reshape"].mean(), r["ms_per_step"] * 1e3,
           ev_wall / args.steps * 1e6, r["value"], 100 * r["value"] / HBM_PEAK_GBS,
           split_b2b_us, 100 * r["achieved"] / HBM_PEAK_GBS, alloc_us))
    return r


def summary(c, r, args):
    """The JSON fields of one workload's resident decode leg."""
    import numpy as np

    w, S, us = c.w, c.S, r["us"]
    rc_us, split_us, merge_us, dec_us = us["reshape"], us["split"], us["merge"], us["decode"]
    kv_bytes = r["kv_bytes"]
    return {
        "config": {"workload": WORKLOAD_TEXT.get(w.name, w.name), "name": w.name,
                   "num_seqs": S,
                   "mean_context_tokens": round(float(kv_bytes.mean() / c.kv_bytes_per_token / S), 1),
                   "kv_bytes_per_step": int(kv_bytes.mean()), "pool_copies_cycled": len(c.pools),
                   "index_staging": "resident: every step's slots, lengths and table copied to "
                                    "HBM before timing",
                   "parallelism": "single GPU"},
        "value_gbs": round(r["value"], 2),
        "ms_per_step": round(r["ms_per_step"], 4),
        "pct_of_hbm_peak": round(100 * r["value"] / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(S * args.steps / r["wall"], 1),
        "step_kernels": ("decode_split_kernel with the new token's cache write (decode_append) "
                         "+ decode_merge_kernel" if r["fused"] else
                         "reshape_and_cache_kernel + decode_split_kernel + decode_merge_kernel"),
        # one layer's kernels only (event times)
        "kernel_tokens_per_s": round(S / (((0 if r["fused"] else rc_us.mean()) + dec_us.mean())
                                          * 1e-6), 1),
        "kernel_us": {"decode_mean": round(float(dec_us.mean()), 2),
                      "decode_median": round(float(np.median(dec_us)), 2),
                      "decode_split_kernel_mean": round(float(split_us.mean()), 2),
                      "decode_split_kernel_back_to_back": round(r["split_b2b_us"], 2),
                      "decode_merge_kernel_mean": round(float(merge_us.mean()), 2),
                      "reshape_and_cache_mean": None if r["fused"] else round(float(rc_us.mean()), 2),
                      "step_with_events": round(r["ev_wall"] / args.steps * 1e6, 2),
                      "allocator_host_us_per_step": round(r["alloc_us"], 2)},
        "roofline": {"bound": "hbm", "achieved": round(r["achieved"], 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(r["achieved"] / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(decode_traffic_file(w.name, r["fused"])),
                     "kernel": "decode_split_kernel (dominant kernel of the decode step%s)"
                               % (", new token's cache write folded in" if r["fused"] else ""),
                     "duration": "mean launch duration of the timed steps' split launches run "
                                 "back to back between one pair of HIP events",
                     "algorithmic_bytes_per_launch": int(r["split_bytes"].mean())},
        "decode_op": {"kernels": "decode_split_kernel + decode_merge_kernel",
                      "achieved_gbs": round(r["achieved_op"], 2),
                      "frac_of_hbm_peak": round(r["achieved_op"] / HBM_PEAK_GBS, 4)},
    }


def decode_traffic_file(name, fused=False):
    return os.path.join(ROOT, "profiles", "decode_%s%s_traffic.json"
                        % (name, "_append" if fused else ""))


def unfused_summary(r, args):
    """The same workload's step with the cache write in its own kernel
    (reshape_and_cache, then the plain split and merge kernels)."""
    us = r["us"]
    return {"ms_per_step": round(r["ms_per_step"], 4), "value_gbs": round(r["value"], 2),
            "pct_of_hbm_peak": round(100 * r["value"] / HBM_PEAK_GBS, 2),
            "kernel_us": {"reshape_and_cache_mean": round(float(us["reshape"].mean()), 2),
                          "decode_split_kernel_mean": round(float(us["split"].mean()), 2),
                          "decode_split_kernel_back_to_back": round(r["split_b2b_us"], 2),
                          "decode_merge_kernel_mean": round(float(us["merge"].mean()), 2)},
            "split_kernel_frac_of_hbm_peak": round(r["achieved"] / HBM_PEAK_GBS, 4),
            "what": "reshape_and_cache_kernel + decode_split_kernel + decode_merge_kernel, "
                    "same plans and pools"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only (the library has no multi-GPU path); "
              "got --gpus %d" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import paged_kv_cache_233_amd as pkv
    import workloads

    if args.copy_probe:
        copy_probe()
        return
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.shared_probe:
        print(json.dumps({"shared_prefix": shared_leg(args, dev)}), flush=True)
        return
    if args.prefill_probe:
        print(json.dumps({"prefill": prefill_leg(args, dev, long_context=False)}), flush=True)
        return
    w = workloads.named(args.config)
    hip = HipEvents()
    sh = torch.cuda.current_stream().cuda_stream
    ctx = decode_setup(w, args, dev, legs=4)        # resident (fused, unfused), staged, graph
    head = resident_leg(ctx, args, hip, fused=True)
    unfused = resident_leg(ctx, args, hip, fused=False)
    S, maxb, words, dt = ctx.S, ctx.maxb, ctx.words, w.torch_dtype
    alloc, pools, sids, ones = ctx.alloc, ctx.pools, ctx.sids, ctx.ones
    q, k_new, v_new, out, ws = ctx.q, ctx.k_new, ctx.v_new, ctx.out, ctx.ws
    pairs_buf, kv_bytes_per_token = ctx.pairs_buf, ctx.kv_bytes_per_token
    total_steps = args.warmup + args.steps
    ms_per_step = head["ms_per_step"]
    value = head["value"]

    # ----------------------------------- staged leg: indices cross PCIe per step
    # The serving loop as it runs: the host allocator plans step t while the
    # GPU runs step t-1, into one of two pinned buffers; the indices reach the
    # device inside the step. "kernel": one copy kernel on the compute stream
    # (starts within a few microseconds); "dma": the same copy through
    # hipMemcpyAsync (the DMA engine, ~20 us to start on this path);
    # "mapped": the kernels read the indices in place (pinned memory is
    # mapped into the device's address space; slower id reads inside the
    # attention kernel). The host refills buffer b only after the last work
    # that read it (step t-2) is done. Reported beside the headline, which
    # excludes the host-to-device copy.
    pinned = [torch.empty(words, dtype=torch.int64).pin_memory() for _ in range(2)]
    released = [hip.create(timing=False), hip.create(timing=False)]
    mapped = args.stage == "mapped"
    stage_mode = args.stage
    stage = pinned if mapped else [torch.empty(words, dtype=torch.int64, device=dev)] * 2
    d_lens = [x[S:].view(torch.int32)[:S] for x in stage]
    d_table = [x[S:].view(torch.int32)[S:S + S * maxb].view(S, maxb) for x in stage]
    # Every call of the step is checked and marshalled once per (staging
    # buffer, pool copy) and replayed as one foreign call per launch: the
    # host must stay ahead of ~110 us of GPU work per step, and the
    # per-call checks of the Python entry points (~10 us each) would not.
    host_lens = [pinned[b].numpy()[S:].view(np.int32)[:S] for b in range(2)]
    append_call = [alloc.batch_append_into(sids, ones, pinned[b].data_ptr(), pairs_buf, prepare=True)
                   for b in range(2)]
    table_call = [alloc.fill_block_table_into(sids, pinned[b].data_ptr() + 8 * S + 4 * S, maxb,
                                              pinned[b].data_ptr() + 8 * S, prepare=True)
                  for b in range(2)]
    copy_call = [pkv.stage_copy(stage[b], pinned[b], stream=sh, prepare=True)
                 if stage_mode == "kernel" else None for b in range(2)]
    slaunch = {}
    for b in range(2):
        for pi, (kc, vc) in enumerate(pools):
            # the headline's kernels: the split kernel with the new
            # token's cache write folded in, then the merge kernel
            slaunch[b, pi] = (
                pkv.decode_append(out, q, k_new, v_new, kc, vc, d_table[b], d_lens[b], w.scale, ws,
                                  stream=sh, phase="split", prepare=True),
                pkv.decode_append(out, q, k_new, v_new, kc, vc, d_table[b], d_lens[b], w.scale, ws,
                                  stream=sh, phase="merge", prepare=True))
    waited = [0.0]
    s_tokens = []

    def sstep(t):
        b = t % 2
        if t >= 2:
            w0 = time.perf_counter()
            hip.sync(released[b])        # the last reader of this pinned buffer is done
            waited[0] += time.perf_counter() - w0
        npairs = append_call[b]()
        assert npairs == 0
        table_call[b]()
        s_tokens.append(int(host_lens[b].sum()))
        if stage_mode == "kernel":
            copy_call[b]()
            hip.record(released[b], sh)
        elif stage_mode == "dma":
            stage[b].copy_(pinned[b], non_blocking=True)
            hip.record(released[b], sh)
        split, merge = slaunch[b, t % len(pools)]
        split()
        merge()
        if mapped:
            hip.record(released[b], sh)

    staged = None
    if not args.no_staged:
        for t in range(args.warmup):
            sstep(t)
        torch.cuda.synchronize()
        host_s = 0.0
        waited[0] = 0.0
        s_tokens.clear()
        s0 = time.perf_counter()
        for t in range(args.warmup, total_steps):
            h0 = time.perf_counter()
            sstep(t)
            host_s += time.perf_counter() - h0
        torch.cuda.synchronize()
        s_wall = time.perf_counter() - s0
        host_us = (host_s - waited[0]) / args.steps * 1e6
        staged = {"ms_per_step": round(s_wall / args.steps * 1e3, 4),
                  "value": round(float(np.sum(s_tokens)) * kv_bytes_per_token / s_wall / 1e9, 2),
                  "unit": "GB/s", "steps": args.steps, "index_staging": stage_mode,
                  "host_us_per_step": round(host_us, 2),
                  "what": "PCIe-inclusive: the host allocator plans each step inside the timed "
                          "loop and the slots, lengths and block table cross from pinned host "
                          "memory to the device every step (%s), then the same two kernels"
                          % stage_mode}
        log("staged step (indices from pinned host memory each step, %s): %.1f us wall, "
            "%.1f GB/s, host work %.1f us per step" % (stage_mode, s_wall / args.steps * 1e6,
                                                       staged["value"], host_us))

    # ------------------------------------------ whole-step graph leg (extra)
    # The same step captured as one HIP graph per (pool copy, staging buffer)
    # and replayed: one launch per step instead of four. Reported beside the
    # eager step; the headline stays the eager run, whose kernels are timed.
    graph = None
    if not args.no_graph and stage_mode != "mapped":
        graphs = []
        for gidx in range(len(pools)):
            gb = gidx % 2
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                if stage_mode == "kernel":
                    pkv.stage_copy(stage[gb], pinned[gb])
                else:
                    stage[gb].copy_(pinned[gb], non_blocking=True)
                kc, vc = pools[gidx]
                pkv.decode_append(out, q, k_new, v_new, kc, vc, d_table[gb], d_lens[gb], w.scale,
                                  ws)
            graphs.append(g)
        torch.cuda.synchronize()
        g_tokens = []

        def gstep(t):
            b = t % 2
            if t >= 2:
                hip.sync(released[b])
            npairs = append_call[b]()
            assert npairs == 0
            table_call[b]()
            g_tokens.append(int(host_lens[b].sum()))
            graphs[t % len(pools)].replay()
            hip.record(released[b], sh)

        base_t = total_steps          # keeps the step parity of the buffers
        for t in range(base_t, base_t + args.warmup):
            gstep(t)
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for t in range(base_t + args.warmup, base_t + args.warmup + args.steps):
            gstep(t)
        torch.cuda.synchronize()
        g_wall = time.perf_counter() - g0
        g_bytes = float(np.sum(g_tokens[args.warmup:])) * kv_bytes_per_token
        graph = {"ms_per_step": round(g_wall / args.steps * 1e3, 4),
                 "value": round(g_bytes / g_wall / 1e9, 2), "unit": "GB/s", "steps": args.steps,
                 "what": "the staged step replayed as one HIP graph per step (index staging, "
                         "split kernel with the cache write, merge kernel captured once per pool "
                         "copy); timed after the eager runs, contexts still growing"}
        log("graph replay: step %.1f us wall, %.1f GB/s" % (g_wall / args.steps * 1e6,
                                                            graph["value"]))

    del ctx, pools, alloc
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    side = {}
    for name in SIDE_DECODE:
        if name != args.config and not args.no_side:
            c2 = decode_setup(workloads.named(name), args, dev, legs=2)
            side[name] = summary(c2, resident_leg(c2, args, hip, fused=True), args)
            side[name]["unfused_step"] = unfused_summary(resident_leg(c2, args, hip, fused=False),
                                                         args)
            del c2
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
    prefill = None if args.no_prefill else prefill_leg(args, dev)
    mixed = None if (args.no_prefill or args.no_mixed) else mixed_leg(args, dev)
    cache_ops = None if args.no_cache_ops else cache_ops_leg(dev)
    shared = None if args.no_shared else shared_leg(args, dev)
    stream = None if args.no_stream else stream_leg(dev)
    scheduler = scheduler_leg()

    # ------------------------------------------------------- CPU oracle leg
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_sample_seqs)

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
    }
    res.update(summary(head["ctx"], head, args))
    res["unfused_step"] = unfused_summary(unfused, args)
    res.update({
        "staged_step": staged,
        "graph_step": graph,
        "prefill": prefill,
        "mixed_step": mixed,
        "cache_ops": cache_ops,
        "shared_prefix": shared,
        "streaming": None if stream is None else dict(
            stream, split_kernel_pct_of_read=round(100 * head["achieved"] / stream["read_gbs"], 1)),
        "scheduler": scheduler,
        "side_decode": side,
        "cpu_baseline": cpu,
    })
    print(json.dumps(res), flush=True)


def build_pool(w, dev, nb, step=False):
    """Allocator and K/V pools of a workload's cached tokens (pool of nb
    blocks, the workload's random placement first); with step=True also the
    step's new tokens. K/V are the workload's seeded values, written through
    reshape_and_cache (copy-on-write pairs through copy_blocks)."""
    import numpy as np
    import torch

    import paged_kv_cache_233_amd as pkv

    alloc = pkv.Allocator(nb)
    order = np.concatenate([w.free_order, np.arange(w.num_blocks, nb, dtype=np.int32)])
    alloc.set_free_order(order)
    shape = (nb, w.num_kv_heads, 16, w.head_dim)
    kc = torch.zeros(shape, dtype=w.torch_dtype, device=dev)
    vc = torch.zeros(shape, dtype=w.torch_dtype, device=dev)
    specs = {s.seq_id: s for s in w.seqs}
    cur = {}
    kvcache = {}
    ops = list(w.setup_ops())
    if step:
        ops += [("append", sid, n) for sid, n in zip(*w.step_appends())]
    for op in ops:
        if op[0] == "add":
            alloc.add(op[1])
            cur[op[1]] = 0
        elif op[0] == "fork":
            alloc.fork(op[1], op[2])
            cur[op[2]] = cur[op[1]]
        else:
            sid, n = op[1], op[2]
            slots, pairs = alloc.append(sid, n)
            if pairs:
                pkv.copy_blocks(kc, vc, torch.tensor(pairs, dtype=torch.int64, device=dev))
            if sid not in kvcache:
                kvcache[sid] = w.seq_kv(specs[sid])
            k, v = kvcache[sid]
            p0 = cur[sid]
            pkv.reshape_and_cache(kc, vc, k[p0:p0 + n].to(dev), v[p0:p0 + n].to(dev),
                                  torch.from_numpy(slots).to(dev))
            cur[sid] = p0 + n
    torch.cuda.synchronize()
    return alloc, kc, vc


def shared_leg(args, dev):
    """The shared workload (128 sequences whose first 2048 tokens are the same
    128 physical blocks) decoded two ways: the ordinary decode (every
    sequence reads the prefix through its table) and the shared-prefix
    decode (the prefix attended once for all sequences as MFMA tiles, then
    each sequence's own blocks). Reports kernel time (median of five timed
    bursts) and GB/s on logical
    bytes (every attended token's K/V once per sequence) and on unique bytes
    (each physical block once)."""
    import numpy as np
    import torch

    import paged_kv_cache_233_amd as pkv
    import workloads

    w = workloads.named("shared")
    dec = w.decode_seqs
    S = len(dec)
    alloc, kc, vc = build_pool(w, dev, w.num_blocks, step=True)
    # consecutive calls cycle through pool copies, as consecutive layers
    # would, so that the private suffixes come from HBM, not from a cache
    # warmed by the previous call (the prefix's reuse within one call stays)
    pools = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(args.pools - 1)]
    sids = [s.seq_id for s in dec]
    maxb = w.max_blocks_per_seq()
    table, lens = alloc.block_table(sids, maxb)
    prefix_blocks = 128
    assert (table[:, :prefix_blocks] == table[0, :prefix_blocks]).all()
    d_table, d_lens = torch.from_numpy(table).to(dev), torch.from_numpy(lens).to(dev)
    gen = torch.Generator().manual_seed(4321)
    q = torch.randn((S, w.num_q_heads, w.head_dim), generator=gen).to(w.torch_dtype).to(dev)
    out = torch.empty_like(q)
    ws = pkv.decode_workspace(S, w.num_q_heads, w.num_kv_heads, w.head_dim, dev)
    wsp = torch.empty(pkv.decode_shared_prefix_workspace_size(S, w.num_q_heads, w.num_kv_heads,
                                                              w.head_dim, prefix_blocks),
                      dtype=torch.uint8, device=dev)
    hip = HipEvents()
    sh = torch.cuda.current_stream().cuda_stream
    reps = max(20, args.steps // 2)

    def timed(fn):
        for r in range(5):
            fn(*pools[r % len(pools)])
        return hip.burst_us(sh, lambda i: fn(*pools[i % len(pools)]), reps)

    plain = timed(lambda kc, vc: pkv.decode(out, q, kc, vc, d_table, d_lens, w.scale, ws))
    shared = timed(lambda kc, vc: pkv.decode_shared_prefix(out, q, kc, vc, d_table, d_lens,
                                                           prefix_blocks, w.scale, wsp))
    per_token = 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
    logical = float(lens.sum()) * per_token
    unique = float(prefix_blocks * 16 + (lens - prefix_blocks * 16).sum()) * per_token
    log("shared prefix: ordinary decode %.1f us, shared-prefix decode %.1f us (x%.2f)"
        % (plain, shared, plain / shared))
    return {"workload": "shared: 128 seqs, one 2048-token prefix held once (128 blocks, refcount 128) "
                        "+ private suffixes U[16,512], 32 q / 8 kv heads, head_dim 128, bf16",
            "logical_kv_bytes": int(logical), "unique_kv_bytes": int(unique),
            "ordinary_decode_us": round(plain, 2), "shared_prefix_decode_us": round(shared, 2),
            "speedup": round(plain / shared, 3),
            "ordinary_logical_gbs": round(logical / plain / 1e3, 1),
            "shared_prefix_logical_gbs": round(logical / shared / 1e3, 1),
            "shared_prefix_unique_gbs": round(unique / shared / 1e3, 1)}


def prefill_leg(args, dev, long_context=True):
    """Chunked prefill on the mixed workload's two 512-query chunks (cached
    prefixes of the seeded lengths), all K/V resident: kernel time (median of
    five timed bursts), tokens/s and MFMA throughput on the algorithmic FLOPs (unmasked query-key pairs
    only: 4 * head_dim * query heads per pair)."""
    import numpy as np
    import torch

    import paged_kv_cache_233_amd as pkv
    import workloads

    w = workloads.named("mixed")
    ch = w.chunk_seqs
    a = pkv.Allocator(w.num_blocks)
    a.set_free_order(w.free_order)
    shape = (w.num_blocks, w.num_kv_heads, 16, w.head_dim)
    kc = torch.zeros(shape, dtype=w.torch_dtype, device=dev)
    vc = torch.zeros_like(kc)
    for spec in ch:
        a.add(spec.seq_id)
        slots, _ = a.append(spec.seq_id, spec.total)
        k, v = w.seq_kv(spec)
        pkv.reshape_and_cache(kc, vc, k.to(dev), v.to(dev), torch.from_numpy(slots).to(dev))
    table, lens = a.block_table([s.seq_id for s in ch], w.max_blocks_per_seq())
    qs = [w.seq_q(s) for s in ch]
    cu = np.cumsum([0] + [x.shape[0] for x in qs]).astype(np.int32)
    q = torch.cat(qs).to(dev)
    out = torch.empty_like(q)
    d_cu, d_lens = torch.from_numpy(cu).to(dev), torch.from_numpy(lens).to(dev)
    d_table = torch.from_numpy(table).to(dev)
    qmax = int(max(x.shape[0] for x in qs))
    for _ in range(5):
        pkv.prefill_chunk(out, q, d_cu, d_lens, d_table, kc, vc, qmax, w.scale)
    reps = max(10, args.steps // 2)
    hip = HipEvents()
    sh = torch.cuda.current_stream().cuda_stream
    # (the library asks for no workspace here: 256 row blocks, one per CU)
    pws = pkv.prefill_workspace(len(ch), w.num_q_heads, w.num_kv_heads, w.head_dim, qmax, dev)
    us = hip.burst_us(sh, lambda i: pkv.prefill_chunk(out, q, d_cu, d_lens, d_table, kc, vc, qmax,
                                                      w.scale, pws), reps)
    pairs = 0
    for spec in ch:
        # queries at positions cached .. total-1 see position+1 keys each
        pairs += sum(range(spec.cached + 1, spec.total + 1))
    flops = 4.0 * w.head_dim * w.num_q_heads * pairs
    tflops = flops / (us * 1e-6) / 1e12
    log("prefill: %d chunks (cached %s, 512 queries each): %.1f us, %.1f TFLOP/s"
        % (len(ch), [s.cached for s in ch], us, tflops))
    return {"workload": "mixed: %d chunks of 512 queries over %s cached tokens, 32 q / 8 kv heads, "
                        "head_dim 128, bf16" % (len(ch), [s.cached for s in ch]),
            "kernel_us": round(us, 2), "query_tokens_per_s": round(int(cu[-1]) / (us * 1e-6), 1),
            "algorithmic_gflop": round(flops / 1e9, 3),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                         "traffic": load_traffic(PREFILL_TRAFFIC_FILE, PREFILL_SRCS,
                                                 "prefill_source_sha256")},
            "long_context": prefill_long_context(args, dev) if long_context else None}


def prefill_long_context(args, dev):
    """One 512-query chunk over 30000 cached tokens (same heads): 128 row
    blocks for 256 CUs, so with the workspace the library asks for each row
    block's positions are cut into two parts (a second kernel folds them).
    Kernel time with and without the workspace (median of five bursts)."""
    import numpy as np
    import torch

    import paged_kv_cache_233_amd as pkv
    import workloads

    w = workloads.custom("prefill long", 11, [], chunks=[(30000, 512)], num_q_heads=32,
                         num_kv_heads=8, head_dim=128, dtype="bf16")
    ch = w.chunk_seqs
    alloc, kc, vc = build_pool(w, dev, w.num_blocks, step=True)
    table, lens = alloc.block_table([s.seq_id for s in ch], w.max_blocks_per_seq())
    q = w.seq_q(ch[0]).to(dev)
    out = torch.empty_like(q)
    a = (torch.tensor([0, q.shape[0]], dtype=torch.int32, device=dev), torch.from_numpy(lens).to(dev),
         torch.from_numpy(table).to(dev))
    qmax = int(q.shape[0])
    ws = pkv.prefill_workspace(1, w.num_q_heads, w.num_kv_heads, w.head_dim, qmax, dev)
    hip = HipEvents()
    sh = torch.cuda.current_stream().cuda_stream
    timed = {}
    for name, wsx in (("no_workspace", None), ("position_parts", ws)):
        for _ in range(3):
            pkv.prefill_chunk(out, q, *a, kc, vc, qmax, w.scale, wsx)
        timed[name] = hip.burst_us(sh, lambda i: pkv.prefill_chunk(out, q, *a, kc, vc, qmax, w.scale, wsx),
                                   max(5, args.steps // 10))
    spec = ch[0]
    flops = 4.0 * w.head_dim * w.num_q_heads * sum(range(spec.cached + 1, spec.total + 1))
    log("prefill, 512 queries over 30000 cached: %.1f us without a workspace, %.1f us with position parts"
        % (timed["no_workspace"], timed["position_parts"]))
    return {"workload": "1 chunk of 512 queries over 30000 cached tokens, 32 q / 8 kv heads, head_dim 128, bf16",
            "algorithmic_gflop": round(flops / 1e9, 3),
            "kernel_us": {k: round(v, 2) for k, v in timed.items()},
            "tflops": {k: round(flops / (v * 1e-6) / 1e12, 1) for k, v in timed.items()},
            "frac_of_bf16_peak": {k: round(flops / (v * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)
                                  for k, v in timed.items()}}


def cache_ops_leg(dev):
    """reshape_and_cache and copy_blocks alone at the llama shapes (8 KV heads,
    head_dim 128, bf16): bursts of 100 back-to-back launches between one pair
    of HIP events (so the events add nothing per launch), pools of 13,000
    blocks. reshape_and_cache: 64 tokens (one decode step) and 1040 tokens
    (the mixed step), random distinct slots. copy_blocks: 64 pairs of
    distinct random blocks. Bytes moved = read + written."""
    import numpy as np
    import torch

    import paged_kv_cache_233_amd as pkv

    nb, hkv, d = 13000, 8, 128
    gen = torch.Generator().manual_seed(77)
    kc = torch.randn((nb, hkv, 16, d), generator=gen).to(torch.bfloat16).to(dev)
    vc = torch.randn((nb, hkv, 16, d), generator=gen).to(torch.bfloat16).to(dev)
    rng = np.random.default_rng(77)
    hip = HipEvents()
    sh = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.create(), hip.create()
    reps = 100

    def burst(call):
        for _ in range(10):
            call()
        torch.cuda.synchronize()
        hip.record(e0, sh)
        for _ in range(reps):
            call()
        hip.record(e1, sh)
        torch.cuda.synchronize()
        return hip.elapsed_us(e0, e1) / reps

    res = {}
    for t in (64, 1040):
        slots = torch.from_numpy(rng.permutation(nb * 16)[:t].astype(np.int64)).to(dev)
        k_new = torch.randn((t, hkv, d), generator=gen).to(torch.bfloat16).to(dev)
        v_new = torch.randn((t, hkv, d), generator=gen).to(torch.bfloat16).to(dev)
        call = pkv.reshape_and_cache(kc, vc, k_new, v_new, slots, stream=sh, prepare=True)
        us = burst(call)
        moved = 2 * 2 * t * hkv * d * 2
        res["reshape_and_cache_%d_tokens" % t] = {"us": round(us, 2),
                                                   "gbs": round(moved / (us * 1e-6) / 1e9, 1)}
    ids = rng.permutation(np.arange(1, nb))[:128]
    pairs = torch.from_numpy(np.stack([ids[:64], ids[64:]], axis=1).astype(np.int64)).to(dev)
    us = burst(pkv.copy_blocks(kc, vc, pairs, stream=sh, prepare=True))
    moved = 2 * 2 * 64 * hkv * 16 * d * 2
    res["copy_blocks_64_pairs"] = {"us": round(us, 2), "gbs": round(moved / (us * 1e-6) / 1e9, 1)}
    log("cache ops: " + ", ".join("%s %.1f us (%.0f GB/s)" % (k, v["us"], v["gbs"])
                                  for k, v in res.items()))
    res["what"] = ("bursts of 100 launches between one pair of HIP events, llama shapes; GB/s on "
                   "bytes read + written")
    return res


def mixed_leg(args, dev):
    """The mixed workload's whole step, all inputs resident: reshape_and_cache
    of its 1040 new tokens (16 decode tokens, two 512-query chunks), then the
    decode of the 16 sequences and the chunked prefill of the two chunks.
    Timed with the two attention calls one after the other on one stream, and
    with the prefill on a second stream beside the decode (they read disjoint
    sequences of the same pools, HBM-bound and MFMA-bound work side by side).
    Pool copies are cycled as in the decode leg."""
    import numpy as np
    import torch

    import paged_kv_cache_233_amd as pkv
    import workloads

    w = workloads.named("mixed")
    dec, ch = w.decode_seqs, w.chunk_seqs
    alloc, kc0, vc0 = build_pool(w, dev, w.num_blocks)
    ids, ns = w.step_appends()
    slots, pairs = alloc.batch_append(ids, ns)
    assert not pairs
    specs = {s.seq_id: s for s in w.seqs}
    ks, vs = [], []
    for sid in ids:
        k, v = w.seq_kv(specs[sid])
        ks.append(k[specs[sid].cached:specs[sid].total])
        vs.append(v[specs[sid].cached:specs[sid].total])
    k_new, v_new = torch.cat(ks).to(dev), torch.cat(vs).to(dev)
    d_slots = torch.from_numpy(slots).to(dev)
    maxb = w.max_blocks_per_seq()
    dt, dl = alloc.block_table([s.seq_id for s in dec], maxb)
    pt, pl = alloc.block_table([s.seq_id for s in ch], maxb)
    d_table, d_lens = torch.from_numpy(dt).to(dev), torch.from_numpy(dl).to(dev)
    p_table, p_lens = torch.from_numpy(pt).to(dev), torch.from_numpy(pl).to(dev)
    qs = [w.seq_q(s) for s in ch]
    cu = np.cumsum([0] + [x.shape[0] for x in qs]).astype(np.int32)
    p_cu = torch.from_numpy(cu).to(dev)
    qmax = int(max(x.shape[0] for x in qs))
    q_dec = torch.cat([w.seq_q(s) for s in dec]).to(dev)
    q_pf = torch.cat(qs).to(dev)
    out_d, out_p = torch.empty_like(q_dec), torch.empty_like(q_pf)
    ws = pkv.decode_workspace(len(dec), w.num_q_heads, w.num_kv_heads, w.head_dim, dev)
    pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(args.pools - 1)]
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()          # default priority
    ready = [torch.cuda.Event() for _ in pools]
    done = [torch.cuda.Event() for _ in pools]

    def step(t, concurrent):
        i = t % len(pools)
        kc, vc = pools[i]
        pkv.reshape_and_cache(kc, vc, k_new, v_new, d_slots, stream=main)
        if concurrent:
            ready[i].record(main)
            side.wait_event(ready[i])
            pkv.prefill_chunk(out_p, q_pf, p_cu, p_lens, p_table, kc, vc, qmax, w.scale,
                              stream=side)
            pkv.decode(out_d, q_dec, kc, vc, d_table, d_lens, w.scale, ws, stream=main)
            done[i].record(side)
            main.wait_event(done[i])
        else:
            pkv.decode(out_d, q_dec, kc, vc, d_table, d_lens, w.scale, ws, stream=main)
            pkv.prefill_chunk(out_p, q_pf, p_cu, p_lens, p_table, kc, vc, qmax, w.scale,
                              stream=main)

    res = {}
    for concurrent in (False, True):
        for t in range(args.warmup):
            step(t, concurrent)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(args.steps):
            step(t, concurrent)
        torch.cuda.synchronize()
        res[concurrent] = (time.perf_counter() - t0) / args.steps * 1e6
    kv = float(dl.sum()) * 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
    ntok = len(dec) + int(cu[-1])
    log("mixed step (reshape_and_cache of %d tokens, decode of %d seqs, prefill of %d chunks): "
        "%.1f us one stream, %.1f us with the prefill on a second stream"
        % (ntok, len(dec), len(ch), res[False], res[True]))
    return {"workload": "mixed: %d decode seqs (ctx U[512,8192]) + %d chunks of 512 queries over %s "
                        "cached tokens; reshape_and_cache of the %d new tokens first"
                        % (len(dec), len(ch), [s.cached for s in ch], ntok),
            "one_stream_us": round(res[False], 2), "two_streams_us": round(res[True], 2),
            "speedup": round(res[False] / res[True], 3),
            "tokens_per_s": round(ntok / (res[True] * 1e-6), 1),
            "decode_kv_bytes": int(kv),
            "what": "the whole step with inputs resident; two_streams: the prefill on a second "
                    "stream (default priority) beside the decode, joined by events"}


def cpu_baseline(w, nseq):
    """The CPU oracle (NumPy float64), timed on host cores over a bounded
    sample of the workload: the first ``nseq`` decode sequences. The oracle's
    own allocator model and scatter build its pool and tables first (not
    timed); the timed part is its decode attention (materialise through the
    block table + float64 softmax attention)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import tests.pipeline as pl
    from oracle import paged

    dec = w.decode_seqs
    sample = list(range(min(nseq, len(dec))))
    t_setup = time.perf_counter()
    with threadpool_limits(limits=1):
        ora = pl.run_oracle(w, decode_sample=sample, prefill=False)
        table = ora["decode_table"][sample]
        lens = ora["decode_lens"][sample]
        q = np.concatenate([pl.to_numpy_storage(w.seq_q(dec[i])) for i in sample])
        log("oracle setup %.1f s" % (time.perf_counter() - t_setup))
        reps = 0
        t0 = time.perf_counter()
        while True:
            paged.decode(q, ora["k_cache"], ora["v_cache"], table, lens, w.scale)
            reps += 1
            el = time.perf_counter() - t0
            # about 10 s of CPU work (bounded in case the host is very slow)
            if el > 10.0 or reps >= 200:
                break
        # The same work spread over host threads: the sequences dealt to the
        # threads by length (longest first, round robin), one BLAS thread
        # each; NumPy's gathers, casts, products and exponentials release
        # the interpreter lock. At most 16 threads, the host share of one GPU.
        nthreads = max(1, min(16, len(os.sched_getaffinity(0))))
        order = sorted(range(len(sample)), key=lambda i: -int(lens[i]))
        parts = [sorted(order[k::nthreads]) for k in range(nthreads)]
        parts = [ix for ix in parts if ix]

        def run_part(ix):        # q is [sequences, Hq, D]
            paged.decode(q[ix], ora["k_cache"], ora["v_cache"], table[ix], lens[ix], w.scale)

        from concurrent.futures import ThreadPoolExecutor
        mreps = 0
        with ThreadPoolExecutor(max_workers=len(parts)) as ex:
            t1 = time.perf_counter()
            while True:
                list(ex.map(run_part, parts))
                mreps += 1
                mel = time.perf_counter() - t1
                if mel > 10.0 or mreps >= 2000:
                    break
    tokens = int(lens.sum())
    kv = float(tokens) * 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
    gbs = kv * reps / el / 1e9
    mgbs = kv * mreps / mel / 1e9
    log("oracle: %d reps over %d seqs in %.2f s -> %.3f GB/s; %d threads: %d reps in %.2f s -> "
        "%.3f GB/s" % (reps, len(sample), el, gbs, len(parts), mreps, mel, mgbs))
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "host_cores": {"cpu_count": os.cpu_count(),
                           "affinity": len(os.sched_getaffinity(0)),
                           "what": "logical CPUs of the host the oracle ran on (os.cpu_count) and "
                                   "those this process may run on (its affinity mask); the oracle "
                                   "used 1 (value) and threads.cores (threads)"},
            "sample": "%d of %d decode sequences of the same workload (%d context tokens), "
                      "materialise + float64 softmax attention, %d repetitions, BLAS limited to "
                      "1 thread" % (len(sample), len(dec), tokens, reps),
            "seconds": round(el, 2), "tokens_per_s": round(len(sample) * reps / el, 2),
            "threads": {"value": round(mgbs, 4), "unit": "GB/s", "cores": len(parts),
                        "repetitions": mreps, "seconds": round(mel, 2),
                        "what": "the same oracle calls over the same sample, the sequences "
                                "dealt to %d host threads (one BLAS thread each)" % len(parts)}}


if __name__ == "__main__":
    main()
