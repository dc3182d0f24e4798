"""GPU: ps_rope_reshape_and_cache against the oracle's rotary embedding.

The kernel forms each angle and its cos / sin in fp64, rotates in fp32 and
rounds to the storage dtype, so against the oracle's exact fp64 rotation an
element may differ by half an ulp of the dtype (the final rounding) plus
the fp32 arithmetic: rounding cos and sin to fp32 and two fp32 products and
a sum, each within 2^-24 relative of |x_j| + |x_{j+D/2}|. The bound used
is 0.5 ulp_dtype(|ref|) + 8 * 2^-24 * (|x_j| + |x_{j+D/2}|).

Covered: ragged mixed steps (positions from the plan), every dtype, D 64
and 128, theta 1e4 and 1e6, in-place q, k-only calls, slots outside the
pool (skipped), positions up to 2^31 - 1, and a whole step (rotary
scatter then attention) against the oracle's attention over its own
rotation rounded to the storage dtype.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_packed_amd as P
import workloads
from tests import _harness as H
from tests.test_gpu_parity import check_out

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
MANT = {torch.float32: 23, torch.float16: 10, torch.bfloat16: 7}
MIN_EXP = {torch.float32: -126, torch.float16: -14, torch.bfloat16: -126}
INT = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16}


def _note(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _bound(ref, x, dtype):
    """Per-element error bound of the kernel's rotation (see the module doc)."""
    e = np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** MIN_EXP[dtype])))
    ulp = 2.0 ** (e - MANT[dtype])
    if dtype == torch.float32:
        ulp = 0.0 * ulp
    half = x.shape[-1] // 2
    pair = np.abs(x[..., :half]) + np.abs(x[..., half:])
    return 0.5 * ulp + 8 * 2.0 ** -24 * np.concatenate([pair, pair], axis=-1)


def _check_rot(got, x, positions, theta, dtype, what):
    ref = oracle.rope(H.f64(x), positions, theta)
    g = got.to(torch.float64).numpy()
    err = np.abs(g - ref)
    bound = _bound(ref, H.f64(x), dtype)
    worst = float((err / bound).max()) if err.size else 0.0
    _note(f"{what}: max_abs={err.max() if err.size else 0:.3e} worst err/bound={worst:.3f}")
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    assert np.all(err <= bound), f"{what}: error above the rounding bound"


def _written(st, slots):
    """Boolean mask over one layer's flat slots that the step writes."""
    m = np.zeros(st.num_blocks * 16, dtype=bool)
    s = slots[(slots >= 0) & (slots < st.num_blocks * 16)]
    m[s] = True
    return m


def _run(st, theta, in_place=False, num_q_heads=None, slots=None, positions=None):
    pk, pv = H.host_pools(st)
    gk = torch.from_numpy(pk).to(DEV).view(st.dtype)
    gv = torch.from_numpy(pv).to(DEV).view(st.dtype)
    pool = P.make_pool(gk, gv, st.layer)
    step = P.PackedStep(st.q_lens, st.num_computed, st.block_tables, st.num_q_heads, pool, DEV)
    host = P.ps_plan_host_arrays(step.plan, st.num_seqs, st.num_tokens)
    slots = host["slot_mapping"] if slots is None else np.asarray(slots, dtype=np.int32)
    positions = host["positions"] if positions is None else np.asarray(positions, dtype=np.int32)
    hq = st.num_q_heads if num_q_heads is None else num_q_heads
    q, k, v = st.q.to(DEV), st.k.to(DEV), st.v.to(DEV)
    q_out = q if in_place else torch.full_like(q, float("nan"))
    d_slots = torch.from_numpy(slots).to(DEV)
    d_pos = torch.from_numpy(positions).to(DEV)
    P.ps_rope_reshape_and_cache(q, q_out, k, v, d_pos, d_slots, st.num_tokens, hq, theta, pool,
                                torch.cuda.current_stream())
    torch.cuda.synchronize()
    it = INT[st.dtype]
    return (q_out.cpu(), gk.view(it).cpu().numpy(), gv.view(it).cpu().numpy(), pk, pv, slots, positions)


def _check_pools(st, gk, gv, pk, pv, slots, positions, theta):
    L, NB, bs, hkv, d = H.pool_shape(st)
    # V: the oracle's plain scatter, bit for bit (valid slots only)
    ok = (slots >= 0) & (slots < NB * 16)
    ev = pv.copy().reshape(L, NB * 16, hkv, d)
    ev[st.layer, slots[ok]] = H.bits(st.v)[ok]
    assert np.array_equal(gv.reshape(ev.shape), ev), "V pool differs from the oracle's scatter"
    # K: untouched slots keep their bits, written slots hold the rotated k
    gk2 = gk.reshape(L, NB * 16, hkv, d)
    pk2 = pk.reshape(L, NB * 16, hkv, d)
    w = _written(st, slots)
    keep = np.ones((L, NB * 16), dtype=bool)
    keep[st.layer, w] = False
    assert np.array_equal(gk2[keep], pk2[keep]), "K pool changed outside the written slots"
    got = torch.from_numpy(gk2[st.layer, slots[ok]].copy()).view(st.dtype)
    _check_rot(got, st.k[torch.from_numpy(np.nonzero(ok)[0])], positions[ok], theta, st.dtype, "pool K")


# the last two have more than 512 units (16-byte chunk pairs and v words)
# per token: a token then takes a workgroup of its own
CASES = [("f32", 4, 2, 64), ("f32", 2, 1, 128), ("f16", 14, 2, 64), ("f16", 12, 2, 128),
         ("bf16", 12, 2, 128), ("bf16", 32, 4, 64), ("bf16", 7, 1, 128),
         ("bf16", 64, 8, 128), ("f32", 28, 4, 128)]


@pytest.mark.parametrize("theta", [1e4, 1e6])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_rope_scatter_random_steps(case, theta):
    dt, hq, hkv, d = case
    st = workloads.random_step(hq * 7 + d, dtype=dt, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                               num_seqs=9, max_q=70, max_ctx=3000, num_layers=2, layer=1)
    _note(f"rope {case} theta={theta:g} q_lens={st.q_lens.tolist()}")
    q_out, gk, gv, pk, pv, slots, pos = _run(st, theta)
    _check_rot(q_out, st.q, pos, theta, st.dtype, "q_out")
    _check_pools(st, gk, gv, pk, pv, slots, pos, theta)


def test_rope_in_place_and_k_only():
    st = workloads.random_step(3, dtype="bf16", num_q_heads=12, num_kv_heads=2, head_dim=128,
                               num_seqs=5, max_q=40, max_ctx=500)
    q_out, gk, gv, pk, pv, slots, pos = _run(st, 1e6, in_place=True)
    _check_rot(q_out, st.q, pos, 1e6, st.dtype, "q in place")
    _check_pools(st, gk, gv, pk, pv, slots, pos, 1e6)
    # num_q_heads = 0: q is neither read nor written
    q_out, gk, gv, pk, pv, slots, pos = _run(st, 1e6, num_q_heads=0)
    assert torch.isnan(q_out.float()).all()
    _check_pools(st, gk, gv, pk, pv, slots, pos, 1e6)


def test_rope_slots_outside_the_pool_are_skipped():
    st = workloads.random_step(4, dtype="f16", num_q_heads=8, num_kv_heads=2, head_dim=64,
                               num_seqs=4, max_q=30, max_ctx=100)
    geom = P.ps_pool(0, 0, st.num_layers, st.num_blocks, 16, st.num_kv_heads, st.head_dim, P.PS_F16,
                     st.layer)
    plan = P.ps_plan_step(st.q_lens, st.num_computed, st.block_tables, st.num_q_heads, geom)
    slots = P.ps_plan_host_arrays(plan, st.num_seqs, st.num_tokens)["slot_mapping"].copy()
    slots[::3] = -1
    slots[1::7] = st.num_blocks * 16
    q_out, gk, gv, pk, pv, slots, pos = _run(st, 1e4, slots=slots)
    _check_rot(q_out, st.q, pos, 1e4, st.dtype, "q_out")
    _check_pools(st, gk, gv, pk, pv, slots, pos, 1e4)


def test_rope_large_positions():
    # explicit positions far beyond the step's own, up to 2^31 - 1: fp64
    # angles keep the rotation within the rounding bound
    st = workloads.random_step(6, dtype="bf16", num_q_heads=12, num_kv_heads=2, head_dim=128,
                               num_seqs=6, max_q=40, max_ctx=200)
    rng = np.random.default_rng(6)
    pos = rng.integers(0, 2 ** 31 - 1, st.num_tokens, endpoint=True).astype(np.int32)
    pos[:4] = [0, 2 ** 31 - 1, 1 << 20, 1000000]
    for theta in (1e4, 1e6):
        q_out, gk, gv, pk, pv, slots, p2 = _run(st, theta, positions=pos)
        _check_rot(q_out, st.q, p2, theta, st.dtype, f"q_out theta={theta:g}")
        _check_pools(st, gk, gv, pk, pv, slots, p2, theta)


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f16", 64), ("f32", 128)])
def test_step_with_rope_matches_oracle_attention(dt, d):
    # the whole step: rotary scatter (q rotated in place), then attention.
    # The oracle rotates q and k itself (fp64), rounds them to the storage
    # dtype as the pool and q hold them, and attends.
    st = workloads.random_step(11 + d, dtype=dt, num_q_heads=8, num_kv_heads=2, head_dim=d,
                               num_seqs=7, max_q=60, max_ctx=400)
    _note(f"step+rope {dt} D={d} q_lens={st.q_lens.tolist()}")
    pk, pv = H.host_pools(st)
    gk = torch.from_numpy(pk).to(DEV).view(st.dtype)
    gv = torch.from_numpy(pv).to(DEV).view(st.dtype)
    pool = P.make_pool(gk, gv, st.layer)
    step = P.PackedStep(st.q_lens, st.num_computed, st.block_tables, st.num_q_heads, pool, DEV)
    q, k, v = st.q.to(DEV), st.k.to(DEV), st.v.to(DEV)
    out = torch.full_like(q, float("nan"))
    step.run(q, k, v, pool, out, st.scale, torch.cuda.current_stream(), rope_theta=1e6)
    torch.cuda.synchronize()
    pos = P.ps_plan_host_arrays(step.plan, st.num_seqs, st.num_tokens)["positions"]
    rq = torch.from_numpy(oracle.rope(H.f64(st.q), pos, 1e6)).to(st.dtype)
    rk = torch.from_numpy(oracle.rope(H.f64(st.k), pos, 1e6)).to(st.dtype)
    st_rot = dataclasses.replace(st, q=rq, k=rk)
    check_out(st_rot, out.cpu())
