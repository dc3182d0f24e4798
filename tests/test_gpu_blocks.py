"""GPU: ps_copy_blocks against the oracle's block copy, bit for bit.

Covers copy-on-write inside one device pool, swap out to a pinned host
pool and swap back in to different device blocks (the round trip must be
lossless), every layer, and ids outside a pool (skipped by the kernel)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_packed_amd as P
import workloads
from tests import _harness as H

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _ids(a):
    return torch.tensor(np.asarray(a, dtype=np.int32), device=DEV)


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f16", 64), ("f32", 64)])
def test_copy_on_write_and_swap_round_trip(dt, d):
    st = workloads.random_step(41 + d, dtype=dt, num_q_heads=4, num_kv_heads=2, head_dim=d,
                               num_seqs=6, max_q=10, max_ctx=200, num_layers=3, layer=2)
    print(f"[gpu-case] blocks {dt} D={d} {st.summary()}", flush=True)
    pk, pv = H.host_pools(st)
    ib = torch.int32 if dt == "f32" else torch.int16
    gk = torch.from_numpy(pk).to(DEV).view(st.dtype)
    gv = torch.from_numpy(pv).to(DEV).view(st.dtype)
    dev_pool = P.make_pool(gk, gv)
    used = np.unique(st.block_tables[st.block_tables >= 0])
    free = np.setdiff1d(np.arange(st.num_blocks), used)
    rng = np.random.default_rng(d)

    # copy-on-write: duplicate some used blocks into free ones (same pool)
    src = rng.choice(used, size=min(9, len(used)), replace=False)
    dst = rng.choice(free, size=len(src), replace=False)
    P.ps_copy_blocks(dev_pool, dev_pool, _ids(src), _ids(dst), len(src))
    torch.cuda.synchronize()
    ek, ev = pk.copy(), pv.copy()
    oracle.copy_blocks(ek, ev, ek, ev, src, dst)
    assert np.array_equal(gk.view(ib).cpu().numpy(), ek)
    assert np.array_equal(gv.view(ib).cpu().numpy(), ev)

    # swap out every used block to a pinned host pool, clobber them on the
    # device, swap them back in to their own ids: lossless
    host_shape = (st.num_layers, len(used), 16, st.num_kv_heads, d)
    hk = torch.zeros(host_shape, dtype=st.dtype, pin_memory=True)
    hv = torch.zeros(host_shape, dtype=st.dtype, pin_memory=True)
    host_pool = P.make_pool(hk, hv)
    P.ps_copy_blocks(dev_pool, host_pool, _ids(used), _ids(np.arange(len(used))), len(used))
    torch.cuda.synchronize()
    hek, hev = np.zeros(host_shape, dtype=ek.dtype), np.zeros(host_shape, dtype=ek.dtype)
    oracle.copy_blocks(ek, ev, hek, hev, used, np.arange(len(used)))
    assert np.array_equal(hk.view(ib).numpy(), hek)
    assert np.array_equal(hv.view(ib).numpy(), hev)
    gk.view(ib)[:, torch.from_numpy(used).to(DEV)] = 0
    gv.view(ib)[:, torch.from_numpy(used).to(DEV)] = 0
    P.ps_copy_blocks(host_pool, dev_pool, _ids(np.arange(len(used))), _ids(used), len(used))
    torch.cuda.synchronize()
    assert np.array_equal(gk.view(ib).cpu().numpy(), ek)
    assert np.array_equal(gv.view(ib).cpu().numpy(), ev)


def test_out_of_range_ids_are_skipped():
    shape = (2, 8, 16, 2, 64)
    gk = torch.arange(np.prod(shape), dtype=torch.int32, device=DEV).view(shape).to(torch.int16).view(torch.float16)
    gv = gk.clone()
    pool = P.make_pool(gk, gv)
    before = gk.clone()
    P.ps_copy_blocks(pool, pool, _ids([-1, 0, 8, 3]), _ids([1, 99, 2, 5]), 4)
    torch.cuda.synchronize()
    # only the in-range pair (3 -> 5) moved
    exp = before.clone()
    exp[:, 5] = before[:, 3]
    assert torch.equal(gk.view(torch.int16), exp.view(torch.int16))
