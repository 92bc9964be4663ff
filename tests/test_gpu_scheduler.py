"""Scheduler-driven request streams on the GPU: the C++ scheduler and
allocator plan every step (token budget, chunked prefill, preemption by
recompute, prefix-cache hits); reshape_and_cache, the decode kernel and the
chunked-prefill kernel execute the plans through the C ABI; every output
row is checked against the oracle's attention over the request's own
tokens with no paging (tests/serving.py)."""
import pytest

import workloads
from tests.serving import HipExecutor, run_stream

pytestmark = pytest.mark.gpu

CASES = {
    # name: (seed, requests, pool blocks, budget, threshold, chunked, caching, dtype, Hq, Hkv, D)
    "bf16 d64 g4 tight pool": (11, 24, 40, 96, 0, True, True, "bf16", 8, 2, 64),
    "bf16 d128 g4 threshold": (12, 20, 48, 128, 40, True, True, "bf16", 16, 4, 128),
    "bf16 d128 g8 no chunking": (13, 16, 80, 256, 0, False, True, "bf16", 32, 4, 128),
    "f32 d64 g2 no cache": (14, 16, 36, 64, 0, True, False, "f32", 4, 2, 64),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_stream_on_gpu(name):
    seed, nreq, nb, budget, thr, chunked, caching, dtype, hq, hkv, d = CASES[name]
    print("[gpu] scheduler stream %s" % name, flush=True)
    st = workloads.RequestStream(seed, nreq, prompt_range=(1, 160), new_range=(1, 40), max_pos=240,
                                 dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                 arrival_span=20)
    stats = run_stream(st, HipExecutor, nb, budget, threshold=thr, chunked=chunked, caching=caching,
                       shuffle_seed=seed)
    print("[gpu]   %s" % stats, flush=True)
    assert stats["finished"] == nreq
    if name == "bf16 d64 g4 tight pool":
        assert stats["preempted"] > 0 and stats["chunks"] > 0 and stats["hit_blocks"] > 0
