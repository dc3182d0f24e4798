"""GPU: fixed-shape plans over more shape classes, one captured graph each.

For each class (dtype, heads, head dim, the most query tokens a sequence
brings, waves per decode item, key split), four steps of different
sequence counts, query lengths and contexts are planned with the class's
capacities. One graph captured on the first step replays every step after
its plan and inputs are loaded into the same buffers; each replay is
checked against the oracle (output) and the oracle's scatter (pool), and
against an eager call of the same step (bit for bit).
"""
import numpy as np
import pytest
import torch

import paged_kv_attention_packed_amd as P
import workloads
from tests import _harness as H
from tests.test_gpu_parity import check_out

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

_DT = {"f32": (torch.float32, P.PS_F32, torch.int32), "f16": (torch.float16, P.PS_F16, torch.int16),
       "bf16": (torch.bfloat16, P.PS_BF16, torch.int16)}

CLASSES = [  # dtype, Hq, Hkv, D, max_query_len, decode_waves, decode_split_keys
    ("bf16", 12, 2, 128, 2, 0, 0),
    ("bf16", 12, 2, 128, 5, 4, 512),
    ("f32", 4, 2, 64, 4, 8, 0),
    ("f16", 16, 1, 64, 1, 16, 0),
    ("f16", 16, 1, 64, 2, 0, 0),
    ("bf16", 8, 8, 64, 3, 8, 128),
    ("f16", 14, 2, 64, 1, 4, 256),
]
MAX_SEQS, WIDTH, NB = 48, 64, 4096


def _steps(cls, ci):
    dt, hq, hkv, d, mql = cls[:5]
    steps = []
    for i, S in enumerate([MAX_SEQS, 29, 41, 5]):
        rng = np.random.default_rng(1300 + 10 * ci + i)
        q_lens = rng.integers(1, mql, size=S, endpoint=True)
        ctx = rng.integers(1, WIDTH * 16, size=S, endpoint=True)
        ctx = np.maximum(ctx, q_lens)
        steps.append(workloads.build_step(f"fixed-sweep-{ci}-{i}", 1300 + 10 * ci + i, dt, hq, hkv, d, NB,
                                          q_lens.tolist(), (ctx - q_lens).tolist(), rng=rng, table_width=WIDTH))
    return steps


@pytest.mark.parametrize("ci", range(len(CLASSES)), ids=lambda i: "-".join(map(str, CLASSES[i])))
def test_fixed_shape_classes_replay(ci):
    cls = CLASSES[ci]
    dt, hq, hkv, d, mql, waves, split = cls
    tdt, pdt, bits = _DT[dt]
    steps = _steps(cls, ci)
    opts = dict(max_seqs=MAX_SEQS, max_tokens=MAX_SEQS * mql, max_query_len=mql, decode_waves=waves)
    if split:
        nsplit = -(-WIDTH * 16 // split)
        opts.update(decode_split_keys=split, max_decode_items=MAX_SEQS * hkv * nsplit,
                    max_merge_items=MAX_SEQS * hkv * 4, max_workspace_rows=MAX_SEQS * hkv * 32 * nsplit)
    options = P.plan_options(**opts)
    shape = (1, NB, 16, hkv, d)
    gk = torch.zeros(shape, dtype=tdt, device=DEV)
    gv = torch.zeros(shape, dtype=tdt, device=DEV)
    pool = P.make_pool(gk, gv)
    proto = P.ps_pool(0, 0, 1, NB, 16, hkv, d, pdt, 0)
    plans = [P.ps_plan_step(st.q_lens, st.num_computed, st.block_tables, hq, proto, P.PS_PLAN_FIXED_SHAPE, options)
             for st in steps]
    sizes = {P.ps_plan_sizes(p) for p in plans}
    assert len(sizes) == 1, sizes
    meta_bytes, ws_bytes = sizes.pop()
    meta = torch.empty(meta_bytes, dtype=torch.uint8, device=DEV)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)
    T_max = MAX_SEQS * mql
    q = torch.zeros((T_max, hq, d), dtype=tdt, device=DEV)
    k = torch.zeros((T_max, hkv, d), dtype=tdt, device=DEV)
    v = torch.zeros_like(k)
    out = torch.zeros_like(q)

    def load(i):
        st = steps[i]
        pk, pv = H.host_pools(st)
        gk.copy_(torch.from_numpy(pk).view(tdt))
        gv.copy_(torch.from_numpy(pv).view(tdt))
        T = st.num_tokens
        q.zero_(); k.zero_(); v.zero_()
        q[:T].copy_(st.q)
        k[:T].copy_(st.k)
        v[:T].copy_(st.v)
        P.ps_plan_upload(plans[i], meta, meta_bytes, torch.cuda.current_stream())
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
        print(f"[gpu-case] fixed class {cls} step {i}: S={st.num_seqs} T={st.num_tokens} items "
              f"{info['active_decode_items']}/{info['decode_items']} merges "
              f"{info['active_merge_items']}/{info['merge_items']} waves {info['decode_waves']} "
              f"row tiles {info['decode_row_tiles']}", flush=True)
        pk, pv = load(i)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        T = st.num_tokens
        got = out[:T].cpu()
        ek, ev = H.oracle_pools_after(st, pk, pv)
        assert np.array_equal(gk.view(bits).cpu().numpy(), ek), f"step {i}: K pool"
        assert np.array_equal(gv.view(bits).cpu().numpy(), ev), f"step {i}: V pool"
        check_out(st, got)
        load(i)
        eager = torch.full_like(out, float("nan"))
        call(i, eager)
        torch.cuda.synchronize()
        assert torch.equal(eager[:T].cpu(), got), f"step {i}: replay differs from the eager call"
