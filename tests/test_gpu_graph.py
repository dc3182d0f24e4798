"""GPU: a packed step captured into a HIP graph replays exactly.

The library's two step calls enqueue plain kernel launches on the caller's
stream (no allocation, no memset, no synchronisation), so a step can be
captured once and replayed. Every replay, with eager work and
synchronisation between replays, must reproduce the eager output bit for
bit, and the pool must hold exactly what the oracle's scatter writes.
"""
import os

import numpy as np
import pytest
import torch

import paged_kv_attention_packed_amd as P
import workloads
from tests import _harness as H

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("case", ["decode-fp16", "mixed-bf16", "split-bf16", "prefix-bf16"])
def test_graph_replay_matches_eager(case, monkeypatch):
    if case == "decode-fp16":
        st = workloads.config(2)
    elif case == "prefix-bf16":  # shared-prefix pass, merges and the fused scatter
        st = workloads.prefix_groups_step(31, dtype="bf16", num_q_heads=12, num_kv_heads=2, head_dim=128,
                                          verify=True)
    elif case == "mixed-bf16":
        st = workloads.random_step(77, dtype="bf16", num_seqs=8, max_q=80, max_ctx=600)
    else:  # force split-K partials and the merge kernel into the graph
        monkeypatch.setenv("PS_DECODE_SPLIT", "64")
        monkeypatch.setenv("PS_PREFILL_SPLIT", "128")
        st = workloads.random_step(78, dtype="bf16", num_seqs=8, max_q=80, max_ctx=600)
    print(f"[gpu-case] graph {case} {st.summary()}", flush=True)
    pools = H.host_pools(st)
    gk = torch.from_numpy(pools[0]).to(DEV).view(st.dtype)
    gv = torch.from_numpy(pools[1]).to(DEV).view(st.dtype)
    pool = P.make_pool(gk, gv, st.layer)
    step = P.PackedStep(st.q_lens, st.num_computed, st.block_tables, st.num_q_heads, pool, DEV)
    q, k, v = st.q.to(DEV), st.k.to(DEV), st.v.to(DEV)
    eager = torch.full_like(q, float("nan"))
    step.run(q, k, v, pool, eager, st.scale, torch.cuda.current_stream())
    torch.cuda.synchronize()

    out = torch.full_like(q, float("nan"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run(q, k, v, pool, out, st.scale, torch.cuda.current_stream())
    for rep in range(4):
        out.fill_(float("nan"))
        gk.view(torch.int16).add_(0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager step"
    ek, ev = H.oracle_pools_after(st, *pools)
    assert np.array_equal(gk.view(torch.int16).cpu().numpy(), ek)
    assert np.array_equal(gv.view(torch.int16).cpu().numpy(), ev)
