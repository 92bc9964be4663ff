"""The mixed step (decode sequences and prefill chunks of one batch) with its
two attention calls on two streams: decode and prefill read disjoint
sequences of the same pools after one reshape_and_cache, so they may run side
by side. Checked bit for bit against the same calls run one after the other
(whose parity with the oracle the decode and prefill tests establish)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_233_amd as pkv
import workloads
from tests.pipeline import assert_close, run_native, run_oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["mixed/8", "mixed"])
def test_mixed_step_on_two_streams_equals_one(name):
    w = workloads.scaled("mixed", 8) if name == "mixed/8" else workloads.named("mixed")
    print("[gpu] mixed step on two streams: %s" % name, flush=True)
    nat = run_native(w)            # reshape_and_cache, decode, prefill on one stream
    dec, ch = w.decode_seqs, w.chunk_seqs
    dev = torch.device("cuda")
    q_dec = torch.cat([w.seq_q(s) for s in dec]).to(dev)
    q_pf = torch.cat([w.seq_q(s) for s in ch]).to(dev)
    d_table = torch.from_numpy(nat["decode_table"]).to(dev)
    d_lens = torch.from_numpy(nat["decode_lens"]).to(dev)
    p_table = torch.from_numpy(nat["prefill_table"]).to(dev)
    p_lens = torch.from_numpy(nat["prefill_lens"]).to(dev)
    p_cu = torch.from_numpy(nat["prefill_cu"]).to(dev)
    qmax = int(np.diff(nat["prefill_cu"]).max())
    ws = pkv.decode_workspace(len(dec), w.num_q_heads, w.num_kv_heads, w.head_dim, dev)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    for rep in range(3):
        out_d = torch.full_like(q_dec, float("nan"))
        out_p = torch.full_like(q_pf, float("nan"))
        ready = torch.cuda.Event()
        ready.record(main)
        side.wait_event(ready)
        pkv.prefill_chunk(out_p, q_pf, p_cu, p_lens, p_table, nat["k_cache"], nat["v_cache"], qmax,
                          w.scale, nat["prefill_ws"], stream=side)
        pkv.decode(out_d, q_dec, nat["k_cache"], nat["v_cache"], d_table, d_lens, w.scale, ws,
                   stream=main)
        done = torch.cuda.Event()
        done.record(side)
        main.wait_event(done)
        torch.cuda.synchronize()
        assert torch.equal(out_d.view(torch.int16), nat["decode"].view(torch.int16))
        assert torch.equal(out_p.view(torch.int16), nat["prefill"].view(torch.int16))
    if name == "mixed/8":
        ora = run_oracle(w)
        assert_close(out_d, ora["decode"], w.dtype, "mixed/8 decode")
        assert_close(out_p, ora["prefill"], w.dtype, "mixed/8 prefill")
