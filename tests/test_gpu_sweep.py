"""GPU parity over a seeded sweep of shapes and plan choices.

Each case draws a ragged step (decode, verify and prefill sequences), a
data type, head geometry, a kernel route and the plan options (split sizes,
waves per decode item, walk rotation, decode cache policy), and runs it
either through ps_step or through the two separate calls. The pool is
checked bit for bit against the oracle's scatter and the output against
the fp64 oracle within the dtype's tolerance, as in test_gpu_parity.
"""
import numpy as np
import pytest

import paged_kv_attention_packed_amd as P
import workloads
from tests import _harness as H
from tests.test_gpu_parity import check_out, check_pool, run_on_gpu, _note

pytestmark = pytest.mark.gpu

_HEADS = [(4, 2), (12, 2), (14, 2), (8, 8), (16, 1), (32, 4), (6, 1), (28, 4)]
_ROUTES = [P.PS_PLAN_DEFAULT, P.PS_PLAN_ALL_DECODE, P.PS_PLAN_ALL_PREFILL, P.PS_PLAN_SEPARATE_LAUNCHES]


def _cases(n=60, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = ["f32", "f16", "bf16"][rng.integers(3)]
        d = [64, 128][rng.integers(2)]
        hq, hkv = _HEADS[rng.integers(len(_HEADS))]
        num_seqs = int(rng.integers(1, 10))
        max_q = [1, 5, 40, 200][rng.integers(4)]
        max_ctx = [16, 100, 700, 2000][rng.integers(4)]
        if dt == "f32":
            max_ctx = min(max_ctx, 700)   # (keeps the fp32 cases' oracle time small)
        flags = _ROUTES[rng.integers(len(_ROUTES))]
        opts = {}
        if rng.random() < 0.5:
            opts["decode_split_keys"] = 16 * int(rng.integers(1, 64))
        if rng.random() < 0.5:
            opts["prefill_split_keys"] = 64 * int(rng.integers(1, 32))
        waves = [0, 4, 8] + ([16] if d == 64 and dt != "f32" else [])
        opts["decode_waves"] = waves[rng.integers(len(waves))]
        opts["decode_walk_rotation"] = int(rng.integers(3))
        opts["decode_stream_kv"] = int(rng.integers(3))
        separate = bool(rng.integers(2))
        out.append((i, dt, d, hq, hkv, num_seqs, max_q, max_ctx, flags, opts, separate))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}")
def test_sweep_of_shapes_and_plan_options(case):
    i, dt, d, hq, hkv, num_seqs, max_q, max_ctx, flags, opts, separate = case
    st = workloads.random_step(7000 + i, dtype=dt, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                               num_seqs=num_seqs, max_q=max_q, max_ctx=max_ctx)
    _note(f"sweep case {i}: {dt} Hq={hq} Hkv={hkv} D={d} q_lens={st.q_lens.tolist()} "
          f"ctx={(st.num_computed + st.q_lens).tolist()} flags={flags} options={opts} separate={separate}")
    pools = H.host_pools(st)
    out, gk, gv = run_on_gpu(st, flags=flags, pools=pools, separate=separate, **opts)
    check_pool(st, pools, gk, gv)
    check_out(st, out)
