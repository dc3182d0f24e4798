"""CPU: the planner over seeded random steps, valid and not.

Every call either returns a plan or fails with PS_ERR_INVALID_ARGUMENT /
PS_ERR_UNSUPPORTED and a message; nothing crashes and no other status
appears. For every plan, the arrays it hands the kernels are checked
against their definitions: query_start_loc the running sum of the query
lengths, context_lens = num_computed + q_len, positions c + i, and
slot_mapping the page's slot formula (PageServe "03 Paged KV cache");
the accounting splits the sequences and their bytes between the kernels.
"""
import numpy as np
import pytest

import paged_kv_attention_packed_amd as P
from paged_kv_attention_packed_amd import _binding as B

ALLOWED = {B.PS_ERR_INVALID_ARGUMENT, B.PS_ERR_UNSUPPORTED}


def _draw(rng):
    S = int(rng.integers(0, 40))
    hkv = int(rng.choice([1, 2, 8]))
    g = int(rng.choice([1, 2, 6, 7, 16]))
    hq = hkv * g + (1 if rng.random() < 0.05 else 0)            # sometimes not a multiple
    d = int(rng.choice([64, 128, 128, 96 if rng.random() < 0.05 else 64]))
    dt = int(rng.choice([B.PS_F32, B.PS_F16, B.PS_BF16]))
    q_lens = rng.integers(1, 300, size=S)
    q_lens = np.where(rng.random(S) < 0.5, 1, q_lens)
    nc = rng.integers(0, 3000, size=S)
    if S and rng.random() < 0.05:
        q_lens[rng.integers(S)] = int(rng.choice([0, -3]))
    if S and rng.random() < 0.05:
        nc[rng.integers(S)] = -1
    ctx = np.maximum(q_lens, 0) + np.maximum(nc, 0)
    width = max(1, int(max([(c + 15) // 16 for c in ctx], default=1)) + int(rng.integers(0, 3)))
    if rng.random() < 0.05:
        width = max(1, width - 1)                                 # too narrow for someone
    # the pool: mostly large enough for distinct ids (a permutation of it),
    # sometimes too small (then some table names a block twice)
    need = int(sum((c + 15) // 16 for c in ctx))
    nb = max(1, need + int(rng.choice([0, 5, 1000, 70000]))) if rng.random() < 0.9 else int(rng.choice([1, 7, 64]))
    ids = rng.permutation(nb)[:need] if need <= nb else rng.integers(0, nb, size=need)
    bt = np.full((max(S, 1), width), -7, dtype=np.int32)
    off = 0
    for s in range(S):
        n = (int(ctx[s]) + 15) // 16
        bt[s, :min(n, width)] = ids[off:off + min(n, width)]
        off += n
    if S and rng.random() < 0.05:
        bt[rng.integers(S), 0] = nb + int(rng.integers(0, 5))      # outside the pool
    if S and rng.random() < 0.05 and width > 1:
        s = int(rng.integers(S))
        bt[s, 1] = bt[s, 0]                                       # a block twice in one table
    flags = int(rng.choice([0, 1, 2, B.PS_PLAN_SHARED_PREFIX, B.PS_PLAN_SEPARATE_LAUNCHES,
                            3 if rng.random() < 0.1 else 0, 64 if rng.random() < 0.1 else 0]))
    opts = {}
    if rng.random() < 0.3:
        opts["decode_split_keys"] = int(rng.choice([16, 48, 4096, 17 if rng.random() < 0.2 else 256]))
    if rng.random() < 0.3:
        opts["prefill_split_keys"] = int(rng.choice([64, 640, 100 if rng.random() < 0.2 else 128]))
    if rng.random() < 0.3:
        opts["decode_waves"] = int(rng.choice([0, 4, 8, 16, 5 if rng.random() < 0.2 else 4]))
    if rng.random() < 0.2:
        opts["decode_stream_kv"] = int(rng.choice([0, 1, 2, 3 if rng.random() < 0.2 else 0]))
    if rng.random() < 0.2:
        opts["decode_walk_rotation"] = int(rng.choice([0, 1, 2]))
    pool = P.ps_pool(0, 0, 1, nb, 16, hkv, d, dt, 0)
    return q_lens, nc, bt[:S] if S else bt[:0], hq, pool, flags, opts


def _check_plan(plan, q_lens, nc, bt, hq, pool):
    S = len(q_lens)
    T = int(q_lens.sum())
    a = B.ps_plan_host_arrays(plan, S, T)
    qsl = np.concatenate([[0], np.cumsum(q_lens)])
    assert np.array_equal(a["query_start_loc"], qsl)
    assert np.array_equal(a["num_computed_tokens"], nc)
    assert np.array_equal(a["context_lens"], nc + q_lens)
    pos = np.concatenate([np.arange(c, c + n) for c, n in zip(nc, q_lens)]) if S else np.zeros(0, np.int64)
    seq = np.repeat(np.arange(S), q_lens)
    assert np.array_equal(a["positions"], pos)
    assert np.array_equal(a["slot_mapping"], bt[seq, pos // 16] * 16 + pos % 16)
    info = P.ps_plan_get_info(plan)
    assert info["decode_seqs"] + info["prefill_seqs"] == S
    assert info["num_tokens"] == T
    row_kv = 2 * pool.head_dim * (4 if pool.dtype == B.PS_F32 else 2) * pool.num_kv_heads
    assert info["kv_bytes_decode"] + info["kv_bytes_prefill"] == int((nc + q_lens).sum()) * row_kv
    assert 0 < info["kv_bytes_unique"] <= info["kv_bytes_decode"] + info["kv_bytes_prefill"] or S == 0


@pytest.mark.parametrize("chunk", range(4))
def test_planner_fuzz(chunk):
    rng = np.random.default_rng(20261203 + chunk)
    ok = failed = 0
    for _ in range(150):
        q_lens, nc, bt, hq, pool, flags, opts = _draw(rng)
        try:
            plan = P.ps_plan_step(q_lens, nc, bt, hq, pool, flags, P.plan_options(**opts) if opts else None)
        except B.PsError as e:
            assert e.status in ALLOWED, (e.status, str(e))
            assert str(e).split(": ", 1)[-1], "an error without a message"
            failed += 1
            continue
        _check_plan(plan, np.asarray(q_lens, np.int64), np.asarray(nc, np.int64), bt, hq, pool)
        ok += 1
    # both outcomes occur in every chunk
    assert ok >= 30 and failed >= 5, (ok, failed)
