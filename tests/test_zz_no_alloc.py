"""GPU: ps_step_no_alloc (the split-K workspace in a static device array)
against ps_step with a caller workspace, through the C ABI.

Two calls in a row on the same GPU, the second with a smaller step that
still uses the workspace: each must give ps_step's output bit for bit (the
same kernels), the oracle's pool bit for bit, and the oracle's attention
within the dtype's tolerance. A plan whose workspace exceeds the static
array is refused before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import paged_kv_attention_packed_amd as P
import workloads
from paged_kv_attention_packed_amd import _binding as B
from tests import _harness as H
from tests.test_gpu_parity import check_out

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _run(st, entry, options, flags=P.PS_PLAN_DEFAULT):
    """One step through `entry` ("step": ps_step with a torch workspace;
    "no_alloc": ps_step_no_alloc) on a fresh device pool; returns
    (out, pool_k bits, pool_v bits, pools before, plan info)."""
    pools = H.host_pools(st)
    gk = torch.from_numpy(pools[0]).to(DEV).view(st.dtype)
    gv = torch.from_numpy(pools[1]).to(DEV).view(st.dtype)
    pool = P.make_pool(gk, gv, st.layer)
    step = P.PackedStep(st.q_lens, st.num_computed, st.block_tables, st.num_q_heads, pool, DEV, flags,
                        options=P.plan_options(**options))
    q, k, v = st.q.to(DEV), st.k.to(DEV), st.v.to(DEV)
    out = torch.full_like(q, float("nan"))
    a = step.arrays
    stream = torch.cuda.current_stream()
    if entry == "step":
        step.step(q, k, v, pool, out, st.scale, stream)
    else:
        P.ps_step_no_alloc(q, k, v, a.slot_mapping, pool, a.block_tables, a.block_table_stride,
                           a.query_start_loc, a.num_computed_tokens, a.context_lens, out, st.num_seqs,
                           st.num_tokens, st.num_q_heads, st.scale, step.plan, stream)
    torch.cuda.synchronize()
    bits = torch.int32 if st.dtype == torch.float32 else torch.int16
    return (out.cpu(), gk.view(bits).cpu().numpy(), gv.view(bits).cpu().numpy(), pools,
            step.info)


def test_no_alloc_step_matches_step_twice_shrinking():
    # a mixed step (decode, verify and prefill rows) with short key splits,
    # then a smaller decode-only one whose partials overwrite part of the
    # first call's: both must match ps_step exactly
    big = workloads.random_step(611, dtype="bf16", num_q_heads=12, num_kv_heads=2, head_dim=128,
                                num_seqs=9, max_q=90, max_ctx=1500)
    small = workloads.build_step("small-decode", 612, "f16", 14, 2, 64, 1024, [1, 1, 2, 1],
                                 [300, 47, 511, 129])
    for st, opts in ((big, dict(decode_split_keys=128, prefill_split_keys=256)),
                     (small, dict(decode_split_keys=64))):
        print(f"[gpu-case] no-alloc {st.name} q_lens={st.q_lens.tolist()} opts={opts}", flush=True)
        ref, rk, rv, _, info = _run(st, "step", opts)
        assert info["workspace_rows"] > 0 and info["merge_items"] > 0
        got, gk, gv, pools, _ = _run(st, "no_alloc", opts)
        assert torch.equal(got, ref), f"{st.name}: ps_step_no_alloc output differs from ps_step"
        assert np.array_equal(gk, rk) and np.array_equal(gv, rv), f"{st.name}: pools differ"
        ek, ev = H.oracle_pools_after(st, *pools)
        assert np.array_equal(gk, ek) and np.array_equal(gv, ev), f"{st.name}: pool differs from the oracle"
        check_out(st, got)


def test_no_alloc_refuses_oversized_workspace():
    # a 2048-token chunk against 30k keys cut into 64-key slices needs far
    # more partials than the static array holds
    st = workloads.build_step("huge-ws", 613, "bf16", 12, 2, 128, 2048, [2048], [30000], values=False)
    pool = P.ps_pool(1 << 20, 1 << 21, 1, st.num_blocks, 16, 2, 128, P.PS_BF16, 0)
    plan = P.ps_plan_step(st.q_lens, st.num_computed, st.block_tables, 12, pool, 0,
                          P.plan_options(prefill_split_keys=64))
    assert P.ps_plan_sizes(plan)[1] > B.PS_STATIC_WORKSPACE_BYTES
    with pytest.raises(P.PsError) as e:
        P.ps_step_no_alloc(1 << 22, 1 << 23, 1 << 24, 1 << 25, pool, 1 << 26, st.block_tables.shape[1],
                           1 << 27, 1 << 28, 1 << 29, 1 << 30, st.num_seqs, st.num_tokens, 12, 0.088, plan)
    assert e.value.status == B.PS_ERR_WORKSPACE_TOO_SMALL


def test_no_alloc_matches_step_on_sweep_cases():
    # twelve of the seeded sweep's steps (routes, plan options, dtypes and
    # head shapes drawn there), back to back on the same static array:
    # ps_step's output bit for bit every time
    from tests.test_gpu_sweep import _cases
    for case in _cases()[::5]:
        i, dt, d, hq, hkv, num_seqs, max_q, max_ctx, flags, opts, _ = case
        st = workloads.random_step(7000 + i, dtype=dt, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                   num_seqs=num_seqs, max_q=max_q, max_ctx=max_ctx)
        print(f"[gpu-case] no-alloc sweep case {i}: {dt} Hq={hq} Hkv={hkv} D={d} flags={flags} opts={opts}",
              flush=True)
        ref, rk, rv, _, _ = _run(st, "step", opts, flags)
        got, gk, gv, pools, _ = _run(st, "no_alloc", opts, flags)
        assert torch.equal(got, ref), f"sweep case {i}: ps_step_no_alloc output differs from ps_step"
        assert np.array_equal(gk, rk) and np.array_equal(gv, rv), f"sweep case {i}: pools differ"
