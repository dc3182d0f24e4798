"""GPU parity of steps whose decode sequences share prefix blocks.

With PS_PLAN_SHARED_PREFIX, sequences whose tables open with the same
blocks are grouped by the planner: attention over the shared prefix runs
once per group, in prefill-kernel items whose query rows are gathered from
every member, and merges with each member's own keys like a key split.
These cases check the result against the oracle (which knows nothing of
groups) with the grouping on and off, across dtypes and head dims, with
verify rows, key splits on both sides, several row ranges per sequence, a
prefill chunk in the step (mixed launch) and the fused scatter.
"""
import numpy as np
import pytest
import torch

import paged_kv_attention_packed_amd as P
import workloads
from tests import _harness as H
from tests.test_gpu_parity import check_out, check_pool, run_on_gpu, _note

pytestmark = pytest.mark.gpu

CASES = [  # dtype, Hq, Hkv, D
    ("f16", 14, 2, 64), ("bf16", 12, 2, 128), ("f32", 4, 2, 64), ("bf16", 8, 8, 64), ("f16", 24, 2, 128),
]


SP = P.PS_PLAN_SHARED_PREFIX


def _info(st, flags=SP, **options):
    pool = P.ps_pool(0, 0, st.num_layers, st.num_blocks, 16, st.num_kv_heads, st.head_dim,
                     {torch.float32: P.PS_F32, torch.float16: P.PS_F16, torch.bfloat16: P.PS_BF16}[st.dtype],
                     st.layer)
    return P.ps_plan_get_info(P.ps_plan_step(st.q_lens, st.num_computed, st.block_tables,
                                             st.num_q_heads, pool, flags,
                                             P.plan_options(**options) if options else None))


@pytest.mark.parametrize("with_prefill", [False, True])
@pytest.mark.parametrize("verify", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefix_groups_match_oracle(case, verify, with_prefill):
    dt, hq, hkv, d = case
    st = workloads.prefix_groups_step(5 + hq + d, dtype=dt, num_q_heads=hq, num_kv_heads=hkv,
                                      head_dim=d, verify=verify, with_prefill=with_prefill)
    info = _info(st)
    _note(f"{st.summary()} verify={verify} prefill={with_prefill} groups={info['prefix_groups']} "
          f"prefix_items={info['prefix_items']} fused={info['step_fused']}")
    assert info["prefix_groups"] >= 1
    pools = H.host_pools(st)
    out, gk, gv = run_on_gpu(st, SP, pools=pools)
    check_pool(st, pools, gk, gv)
    check_out(st, out)


@pytest.mark.parametrize("case", CASES[:3], ids=lambda c: "-".join(map(str, c)))
def test_prefix_groups_with_many_splits(case):
    # short slices on both sides of the prefix boundary: several prefix
    # slices per group and several key splits after it, merged per row
    dt, hq, hkv, d = case
    opts = dict(prefix_slice_keys=64, decode_split_keys=48)
    st = workloads.prefix_groups_step(11 + d, dtype=dt, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                      verify=True)
    info = _info(st, **opts)
    _note(f"{st.summary()} prefix_items={info['prefix_items']} merges={info['merge_items']}")
    assert info["prefix_items"] >= 2 * hkv * 5
    pools = H.host_pools(st)
    out, gk, gv = run_on_gpu(st, SP, pools=pools, **opts)
    check_pool(st, pools, gk, gv)
    check_out(st, out)


@pytest.mark.parametrize("separate", [False, True])
def test_prefix_groups_on_and_off_agree(separate):
    st = workloads.prefix_groups_step(21)
    pools = H.host_pools(st)
    out_on, gk, gv = run_on_gpu(st, SP, pools=pools, separate=separate)
    check_pool(st, pools, gk, gv)
    e_on = check_out(st, out_on)
    assert _info(st, P.PS_PLAN_DEFAULT)["prefix_groups"] == 0
    out_off, _, _ = run_on_gpu(st, pools=pools, separate=separate)
    e_off = check_out(st, out_off)
    diff = (out_on.to(torch.float64) - out_off.to(torch.float64)).abs().max().item()
    _note(f"on/off max diff {diff:.3e} (oracle errors {e_on:.2e} / {e_off:.2e})")
    assert diff <= 2 * 2e-3


def test_config4_groups_whole_batch():
    # 256 decodes behind one 1024-token prefix: one group, prefix pass in
    # prefill-kernel items, the scatter fused into the step's launch
    st = workloads.config(4)
    info = _info(st)
    assert info["prefix_groups"] == 1 and info["step_fused"] == 1 and info["prefix_items"] > 0
    pools = H.host_pools(st)
    out, gk, gv = run_on_gpu(st, SP, pools=pools)
    check_pool(st, pools, gk, gv)
    check_out(st, out)


def test_long_prefix_slices_capped_at_the_item_limit():
    # 61 sequences of 4 verify rows (64 query / 8 KV heads, head_dim 64)
    # behind a 20480-token prefix: with the pass on, the group's 128
    # (KV head, 128-row chunk) pairs would each take one prefix slice by
    # the item-count rule, more keys than a prefill item stages block ids
    # for (16384); the planner cuts every one in two. Every row against
    # the oracle (~10 GB of host memory and ~20 s for the oracle's
    # contiguous K/V).
    S, prefix = 61, 20480
    rng = np.random.default_rng(31)
    nc = (prefix + rng.integers(1, 200, size=S, endpoint=True)).astype(np.int32)
    st = workloads.build_step("long-prefix", 31, "bf16", 64, 8, 64, 4096, [4] * S, nc.tolist(),
                              prefix_tokens=prefix)
    info = _info(st)
    _note(f"{st.summary()} groups={info['prefix_groups']} prefix_items={info['prefix_items']}")
    assert info["prefix_groups"] == 1 and info["prefix_items"] == 2 * 8 * ceil_div(S * 4 * 8, 128)
    pools = H.host_pools(st)
    out, gk, gv = run_on_gpu(st, SP, pools=pools)
    check_pool(st, pools, gk, gv)
    del pools, gk, gv
    check_out(st, out)


def ceil_div(a, b):
    return -(-a // b)
