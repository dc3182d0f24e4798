"""GPU: packed steps captured into HIP graphs replay exactly.

The library's two step calls enqueue plain kernel launches on the caller's
stream (no allocation, no memset, no synchronisation), so a step can be
captured once and replayed. Every replay, with eager work and
synchronisation between replays, must reproduce the eager output bit for
bit, and the pool must hold exactly what the oracle's scatter writes.

A fixed-shape plan (PS_PLAN_FIXED_SHAPE) goes further: one captured graph
serves every later step of the same shape class. Each new step's plan is
uploaded into the same metadata buffer and its inputs copied into the same
buffers; the replay then computes that step (PageServe "Next steps": graphs
for decode, to take launch overhead out of small decode batches).
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
def test_graph_replay_matches_eager(case):
    flags, opts = P.PS_PLAN_DEFAULT, None
    if case == "decode-fp16":
        st = workloads.config(2)
    elif case == "prefix-bf16":  # shared-prefix pass, merges and the fused scatter
        st = workloads.prefix_groups_step(31, dtype="bf16", num_q_heads=12, num_kv_heads=2, head_dim=128,
                                          verify=True)
        flags = P.PS_PLAN_SHARED_PREFIX
    elif case == "mixed-bf16":
        st = workloads.random_step(77, dtype="bf16", num_seqs=8, max_q=80, max_ctx=600)
    else:  # force split-K partials and the merge kernel into the graph
        opts = P.plan_options(decode_split_keys=64, prefill_split_keys=128)
        st = workloads.random_step(78, dtype="bf16", num_seqs=8, max_q=80, max_ctx=600)
    print(f"[gpu-case] graph {case} {st.summary()}", flush=True)
    pools = H.host_pools(st)
    gk = torch.from_numpy(pools[0]).to(DEV).view(st.dtype)
    gv = torch.from_numpy(pools[1]).to(DEV).view(st.dtype)
    pool = P.make_pool(gk, gv, st.layer)
    step = P.PackedStep(st.q_lens, st.num_computed, st.block_tables, st.num_q_heads, pool, DEV, flags,
                        options=opts)
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


def _fixed_steps():
    """Decode / verify steps of one shape class (Qwen2.5-0.5B heads, fp16,
    at most 64 sequences of at most 2 query tokens, tables 64 blocks wide)
    with different lengths and sequence counts."""
    steps = []
    for i, (S, nq_max) in enumerate([(64, 1), (41, 2), (57, 2), (9, 1)]):
        rng = np.random.default_rng(900 + i)
        q_lens = rng.integers(1, nq_max, size=S, endpoint=True)
        ctx = rng.integers(16, 1000, size=S, endpoint=True)
        steps.append(workloads.build_step(f"fixed-{i}", 900 + i, "f16", 14, 2, 64, 4096, q_lens.tolist(),
                                          (ctx - q_lens).tolist(), rng=rng, table_width=64))
    return steps


@pytest.mark.parametrize("split", [0, 256])
def test_fixed_shape_graph_serves_later_steps(split):
    # one graph captured on the first step replays every later step of the
    # same shape class: new plan uploaded into the same metadata buffer, new
    # inputs copied into the same buffers, then replay; every step's output
    # is checked against the oracle and against an eager call, and the pool
    # against the oracle's scatter
    from tests.test_gpu_parity import check_out
    steps = _fixed_steps()
    st0 = steps[0]
    opts = dict(max_seqs=64, max_tokens=128, max_query_len=2)
    if split:
        # contexts up to 1000 keys: at most 4 slices per (sequence, KV
        # head), 28 packed rows in at most 2 merge chunks of 16
        opts.update(decode_split_keys=split, max_decode_items=64 * 2 * 4, max_merge_items=64 * 2 * 2,
                    max_workspace_rows=64 * 2 * 28 * 4)
    flags = P.PS_PLAN_FIXED_SHAPE
    options = P.plan_options(**opts)
    T_max, hq, hkv, d = 128, 14, 2, 64
    shape = (1, 4096, 16, hkv, d)
    gk = torch.zeros(shape, dtype=torch.float16, device=DEV)
    gv = torch.zeros(shape, dtype=torch.float16, device=DEV)
    pool = P.make_pool(gk, gv)
    proto = P.ps_pool(0, 0, 1, 4096, 16, hkv, d, P.PS_F16, 0)
    plans = [P.ps_plan_step(st.q_lens, st.num_computed, st.block_tables, hq, proto, flags, options)
             for st in steps]
    sizes = {P.ps_plan_sizes(p) for p in plans}
    assert len(sizes) == 1, sizes
    meta_bytes, ws_bytes = sizes.pop()
    meta = torch.empty(meta_bytes, dtype=torch.uint8, device=DEV)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)
    q = torch.zeros((T_max, hq, d), dtype=torch.float16, device=DEV)
    k = torch.zeros((T_max, hkv, d), dtype=torch.float16, device=DEV)
    v = torch.zeros_like(k)
    out = torch.zeros_like(q)
    stream = torch.cuda.current_stream()

    def load(i):
        st = steps[i]
        pk, pv = H.host_pools(st)
        gk.copy_(torch.from_numpy(pk).view(torch.float16))
        gv.copy_(torch.from_numpy(pv).view(torch.float16))
        T = st.num_tokens
        q.zero_(); k.zero_(); v.zero_()
        q[:T].copy_(st.q)
        k[:T].copy_(st.k)
        v[:T].copy_(st.v)
        P.ps_plan_upload(plans[i], meta, meta_bytes, stream)
        torch.cuda.synchronize()
        return pk, pv

    def call(i, out_):
        st = steps[i]
        a = P.ps_plan_device_arrays(plans[i])
        P.ps_step(q, k, v, a.slot_mapping, pool, a.block_tables, a.block_table_stride, a.query_start_loc,
                  a.num_computed_tokens, a.context_lens, out_, st.num_seqs, st.num_tokens, hq, st.scale,
                  plans[i], ws, ws_bytes, torch.cuda.current_stream())

    load(0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(0, out)
    for i, st in enumerate(steps):
        info = P.ps_plan_get_info(plans[i])
        print(f"[gpu-case] fixed-shape replay step {i}: S={st.num_seqs} T={st.num_tokens} split={split} "
              f"items {info['active_decode_items']}/{info['decode_items']} merges "
              f"{info['active_merge_items']}/{info['merge_items']}", flush=True)
        pk, pv = load(i)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        T = st.num_tokens
        got = out[:T].cpu()
        ek, ev = H.oracle_pools_after(st, pk, pv)
        assert np.array_equal(gk.view(torch.int16).cpu().numpy(), ek), f"step {i}: K pool"
        assert np.array_equal(gv.view(torch.int16).cpu().numpy(), ev), f"step {i}: V pool"
        check_out(st, got)
        # the same step eagerly, from the same starting pool: same bits
        load(i)
        eager = torch.full_like(out, float("nan"))
        call(i, eager)
        torch.cuda.synchronize()
        assert torch.equal(eager[:T].cpu(), got), f"step {i}: replay differs from the eager call"
