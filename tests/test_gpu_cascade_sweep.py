"""GPU parity of the shared-prefix pass over a seeded sweep of group shapes.

Each case draws one to four groups of decode (or verify) sequences that
share their first blocks, prefix lengths from one block to a few thousand
tokens, sequences that share nothing, sometimes a prefill chunk, and the
pass's options (group thresholds, prefix slice size) with the other plan
options. The result is checked against the oracle, which knows nothing of
groups, and the pool bit for bit against the oracle's scatter.
"""
import numpy as np
import pytest

import paged_kv_attention_packed_amd as P
import workloads
from tests import _harness as H
from tests.test_gpu_parity import check_out, check_pool, run_on_gpu, _note

pytestmark = pytest.mark.gpu

_HEADS = [(14, 2, 64), (12, 2, 128), (4, 2, 64), (8, 8, 64), (24, 2, 128), (6, 1, 128), (16, 2, 64)]


def _case(i, seed=4242):
    rng = np.random.default_rng(seed + 97 * i)
    dt = ["f32", "f16", "bf16"][rng.integers(3)]
    hq, hkv, d = _HEADS[rng.integers(len(_HEADS))]
    g = hq // hkv
    max_q = max(1, 32 // g)                  # decode / verify rows stay on the decode kernel
    q_lens, num_computed, groups = [], [], []
    for _ in range(int(rng.integers(1, 5))):
        members = int(rng.integers(2, 25))
        prefix = 16 * int(rng.integers(1, 130))
        first = len(q_lens)
        for _ in range(members):
            q_lens.append(int(rng.integers(1, max_q + 1)) if rng.random() < 0.3 else 1)
            num_computed.append(prefix + int(rng.integers(0, 300)))
        groups.append((list(range(first, first + members)), prefix))
    for _ in range(int(rng.integers(0, 6))):    # sequences that share nothing
        q_lens.append(1)
        num_computed.append(int(rng.integers(0, 900)))
    if rng.random() < 0.3:                      # a prefill chunk: a mixed launch
        q_lens.append(int(rng.integers(20, 120)))
        num_computed.append(int(rng.integers(0, 400)))
    # packed order: members interleaved with the rest
    S = len(q_lens)
    order = rng.permutation(S)
    inv = np.empty(S, dtype=np.int64)
    inv[order] = np.arange(S)
    q_lens = [q_lens[j] for j in order]
    num_computed = [num_computed[j] for j in order]
    groups = [([int(inv[m]) for m in mem], p) for mem, p in groups]
    opts = {}
    if rng.random() < 0.5:
        opts["prefix_slice_keys"] = 64 * int(rng.integers(1, 40))
    if rng.random() < 0.3:
        opts["decode_split_keys"] = 16 * int(rng.integers(2, 64))
    if rng.random() < 0.3:
        opts["prefix_min_seqs"] = int(rng.integers(2, 12))
    if rng.random() < 0.3:
        opts["prefix_min_keys"] = 16 * int(rng.integers(1, 40))
    opts["decode_walk_rotation"] = int(rng.integers(3))
    separate = bool(rng.integers(2))
    return dict(i=i, dt=dt, hq=hq, hkv=hkv, d=d, q_lens=q_lens, num_computed=num_computed, groups=groups,
                opts=opts, separate=separate)


def _step(c):
    need = sum((n + q + 15) // 16 for n, q in zip(c["num_computed"], c["q_lens"]))
    return workloads.build_step(f"prefix-sweep-{c['i']}", 9000 + c["i"], c["dt"], c["hq"], c["hkv"], c["d"],
                                need + 64, c["q_lens"], c["num_computed"], groups=c["groups"])


@pytest.mark.parametrize("i", range(30), ids=lambda i: f"case{i}")
def test_shared_prefix_sweep(i):
    c = _case(i)
    st = _step(c)
    _note(f"prefix sweep case {i}: {c['dt']} Hq={c['hq']} Hkv={c['hkv']} D={c['d']} S={st.num_seqs} "
          f"groups={[(len(m), p) for m, p in c['groups']]} options={c['opts']} separate={c['separate']}")
    pools = H.host_pools(st)
    out, gk, gv = run_on_gpu(st, P.PS_PLAN_SHARED_PREFIX, pools=pools, separate=c["separate"], **c["opts"])
    check_pool(st, pools, gk, gv)
    check_out(st, out)
