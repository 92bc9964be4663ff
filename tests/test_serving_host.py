"""Scheduler-driven request streams on the CPU: the C++ scheduler and
allocator plan every step, the oracle's pool scatter and paged attention
execute the plans, and every output is checked against attention over the
request's own tokens with no paging (tests/serving.py). Small pools force
preemption by recompute; shared prompt stems give prefix-cache hits."""
import pytest

import workloads
from tests.serving import OracleExecutor, run_stream

CASES = {
    # name: (stream seed, requests, pool blocks, token budget, threshold, chunked, caching, dtype)
    "chunked, cached, tight pool": (1, 12, 24, 48, 0, True, True, "f32"),
    "threshold, no cache": (2, 10, 22, 64, 20, True, False, "bf16"),
    "no chunking": (3, 10, 40, 128, 0, False, True, "f32"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_stream_through_oracle_executor(name):
    seed, nreq, nb, budget, thr, chunked, caching, dtype = CASES[name]
    st = workloads.RequestStream(seed, nreq, prompt_range=(1, 100), new_range=(1, 24),
                                 max_pos=200, dtype=dtype, num_q_heads=4, num_kv_heads=2,
                                 head_dim=16, arrival_span=10)
    stats = run_stream(st, OracleExecutor, nb, budget, threshold=thr, chunked=chunked,
                       caching=caching, shuffle_seed=seed)
    assert stats["finished"] == nreq
    if name == "chunked, cached, tight pool":
        assert stats["preempted"] > 0 and stats["chunks"] > 0 and stats["hit_blocks"] > 0
