"""Pins for the CPU oracle: checks against what the pages and the
mathematics fix, independent of the oracle's own code.

 * the slot formula and the pages' block-table example (golden fixture);
 * the pages' memory-accounting example (golden fixture);
 * a library routine (torch scaled_dot_product_attention, fp64, GQA) on
   contiguous full prefills, where the step reduces to textbook causal
   attention;
 * closed forms: one visible key, equal keys, a dominant key;
 * invariances the pages state: chunked prefill equals full prefill,
   a 1 + k verify equals k + 1 successive decodes, physical block
   placement and prefix sharing do not change what a sequence reads;
 * a second formulation (full-matrix numpy) on tiny inputs;
 * rotary embedding: the transformers Qwen2 rotary routine at small
   positions, the two-dimensional case (a plane rotation by the position),
   pair-norm preservation, scores that depend on relative position only,
   and additive composition of rotations.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import brute
import workloads
from tests import _harness as H

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# slot formula and pool


def test_slot_matches_block_table_example():
    g = _golden("tinyserve_block_tables.json")
    for case in g["cases"]:
        table = g["sequences"][case["seq"]]["block_table"]
        s = oracle.slot(table, case["pos"], g["block_size"])
        assert s == case["slot"], case
        assert s // g["block_size"] == case["block"], case
        assert s % g["block_size"] == case["pos"] % g["block_size"]


def test_example_shared_prefix_block_lands_in_one_place():
    # both sequences' first 16 positions address the same 16 slots (block 7)
    g = _golden("tinyserve_block_tables.json")
    a = [oracle.slot(g["sequences"]["A"]["block_table"], p) for p in range(16)]
    b = [oracle.slot(g["sequences"]["B"]["block_table"], p) for p in range(16)]
    assert a == b == list(range(7 * 16, 8 * 16))
    tails = {oracle.slot(g["sequences"][s]["block_table"], 18) for s in "AB"}
    assert len(tails) == 2  # private tails stay apart


def test_memory_accounting_example():
    g = _golden("tinyserve_memory_accounting.json")
    per_block = oracle.kv_bytes_per_block(g["num_layers"], g["block_size"], g["num_kv_heads"],
                                          g["head_dim"], g["dtype_bytes"])
    assert per_block == g["bytes_per_block"] == 384 * 1024
    assert per_block * g["pool_blocks"] == g["pool_bytes"] == 768 * 1024 * 1024
    assert g["pool_blocks"] * g["block_size"] == g["pool_token_slots"]


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_configs_waste_at_most_15_slots_per_sequence(idx):
    # PageServe "03 Paged KV cache", Memory efficiency: <= 15 empty slots / seq
    st = workloads.config(idx, values=False)
    ctx = st.num_computed.astype(np.int64) + st.q_lens
    nblk = (st.block_tables >= 0).sum(axis=1)
    empty = nblk * 16 - ctx
    assert empty.min() >= 0 and empty.max() <= 15


def test_scatter_then_gather_returns_logical_kv_and_leaves_rest_untouched():
    st = workloads.random_step(11, dtype="bf16", num_q_heads=4, num_kv_heads=2, head_dim=64,
                               num_seqs=5, max_q=20, max_ctx=70, num_layers=3, layer=1)
    pk, pv = H.host_pools(st)
    pk2, pv2 = H.oracle_pools_after(st, pk, pv)
    kb, vb = H.bits(st.k), H.bits(st.v)
    kcb, vcb = H.bits(st.k_ctx), H.bits(st.v_ctx)
    touched = np.zeros(pk.shape[:3], dtype=bool)
    t0 = c0 = 0
    for s in range(st.num_seqs):
        n, c = int(st.q_lens[s]), int(st.num_computed[s])
        gk, gv = oracle.gather(pk2, pv2, st.layer, st.block_tables[s], c + n)
        np.testing.assert_array_equal(gk, np.concatenate([kcb[c0:c0 + c], kb[t0:t0 + n]]))
        np.testing.assert_array_equal(gv, np.concatenate([vcb[c0:c0 + c], vb[t0:t0 + n]]))
        for p in range(c + n):
            sl = oracle.slot(st.block_tables[s], p)
            touched[st.layer, sl // 16, sl % 16] = True
        t0 += n
        c0 += c
    # every other slot, in every layer, still holds the poison pattern
    nan = H.NAN_BITS[st.dtype][1]
    assert np.all(pk2[~touched] == nan) and np.all(pv2[~touched] == nan)
    assert np.all(pk2[0] == nan) and np.all(pk2[2] == nan)


def test_block_placement_does_not_change_gathered_kv():
    # same lengths and values, two different physical permutations
    a = workloads.random_step(21, dtype="f16", num_q_heads=2, num_kv_heads=1, head_dim=64,
                              num_seqs=4, max_q=9, max_ctx=60)
    b = workloads.build_step("b", 99, "f16", 2, 1, 64, a.num_blocks, a.q_lens, a.num_computed,
                             values=False)
    b.k_ctx, b.v_ctx, b.k, b.v, b.q = a.k_ctx, a.v_ctx, a.k, a.v, a.q
    assert not np.array_equal(a.block_tables, b.block_tables)
    pa = H.oracle_pools_after(a, *H.host_pools(a))
    pb = H.oracle_pools_after(b, *H.host_pools(b))
    for s in range(a.num_seqs):
        n = int(a.q_lens[s] + a.num_computed[s])
        ga = oracle.gather(*pa, a.layer, a.block_tables[s], n)
        gb = oracle.gather(*pb, b.layer, b.block_tables[s], n)
        np.testing.assert_array_equal(ga[0], gb[0])
        np.testing.assert_array_equal(ga[1], gb[1])


def test_shared_prefix_blocks_serve_every_sequence():
    st = workloads.build_step("share", 5, "bf16", 4, 2, 64, 64, [1, 1, 1], [40, 52, 33],
                              prefix_tokens=32)
    pk, pv = H.oracle_pools_after(st, *H.host_pools(st))
    kcb, kb = H.bits(st.k_ctx), H.bits(st.k)
    c0 = 0
    for s in range(3):
        c = int(st.num_computed[s])
        gk, _ = oracle.gather(pk, pv, 0, st.block_tables[s], c + 1)
        np.testing.assert_array_equal(gk, np.concatenate([kcb[c0:c0 + c], kb[s:s + 1]]))
        c0 += c
    assert np.all(st.block_tables[:, :2] == st.block_tables[0, :2])


# --------------------------------------------------------------------------
# attention


def _sdpa_full_prefill(q, k, v, scale):
    # q [n, Hq, D], k/v [n, Hkv, D] -> textbook causal GQA attention (fp64)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None].contiguous()
    vt = torch.from_numpy(v).permute(1, 0, 2)[None].contiguous()
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hq,hkv,d", [(2, 1, 64), (6, 2, 128), (7, 1, 64), (4, 4, 32)])
def test_full_prefill_matches_library_sdpa(hq, hkv, d):
    # sequences with no cached context: the step is plain causal attention
    rng = np.random.default_rng(hq * 100 + d)
    lens = [1, 7, 23, 40]
    st = workloads.build_step("full", 3, "f32", hq, hkv, d, 64, lens, [0] * len(lens), rng=rng)
    out = H.oracle_out(st)
    t0 = 0
    for n in lens:
        ref = _sdpa_full_prefill(H.f64(st.q)[t0:t0 + n], H.f64(st.k)[t0:t0 + n],
                                 H.f64(st.v)[t0:t0 + n], st.scale)
        np.testing.assert_allclose(out[t0:t0 + n], ref, rtol=0, atol=1e-12)
        t0 += n


def test_chunked_prefill_equals_full_prefill():
    # PageServe "01 Scheduler loop / System architecture": a prefill chunk and
    # a full prefill are the same operation over the uncomputed tokens
    rng = np.random.default_rng(7)
    ctx, hq, hkv, d = 45, 6, 2, 64
    K = rng.standard_normal((ctx, hkv, d))
    V = rng.standard_normal((ctx, hkv, d))
    Q = rng.standard_normal((ctx, hq, d))
    scale = 1 / math.sqrt(d)
    full = oracle.attention(Q, K[:0], V[:0], K, V, [ctx], [0], scale)
    ref = _sdpa_full_prefill(Q, K, V, scale)
    np.testing.assert_allclose(full, ref, atol=1e-12, rtol=0)
    for c in [1, 16, 17, 31, 44]:
        chunk = oracle.attention(Q[c:], K[:c], V[:c], K[c:], V[c:], [ctx - c], [c], scale)
        np.testing.assert_array_equal(chunk, full[c:])
    # a split into three chunks packed as three "sequences" of one step is
    # not the same thing: each packed sequence only sees its own context
    two = oracle.attention(np.concatenate([Q[10:20], Q[10:20]]), np.concatenate([K[:10], K[:10]]),
                           np.concatenate([V[:10], V[:10]]), np.concatenate([K[10:20], K[10:20]]),
                           np.concatenate([V[10:20], V[10:20]]), [10, 10], [10, 10], scale)
    np.testing.assert_array_equal(two[:10], full[10:20])
    np.testing.assert_array_equal(two[10:], full[10:20])


def test_verify_rows_equal_successive_decodes():
    # tinyserve README "How it works": 1 + k verify rows in one pass under a
    # stepped causal mask score what k + 1 successive decodes would
    rng = np.random.default_rng(8)
    c, k, hq, hkv, d = 37, 4, 6, 2, 128
    K = rng.standard_normal((c + k + 1, hkv, d))
    V = rng.standard_normal((c + k + 1, hkv, d))
    Q = rng.standard_normal((k + 1, hq, d))
    scale = 1 / math.sqrt(d)
    verify = oracle.attention(Q, K[:c], V[:c], K[c:], V[c:], [k + 1], [c], scale)
    for i in range(k + 1):
        dec = oracle.attention(Q[i:i + 1], K[:c + i], V[:c + i], K[c + i:c + i + 1],
                               V[c + i:c + i + 1], [1], [c + i], scale)
        np.testing.assert_array_equal(dec[0], verify[i])


def test_single_visible_key_returns_its_value_exactly():
    rng = np.random.default_rng(9)
    Q = rng.standard_normal((3, 4, 64))
    K = rng.standard_normal((3, 2, 64))
    V = rng.standard_normal((3, 2, 64))
    out = oracle.attention(Q, K[:0], V[:0], K, V, [3], [0], 0.125)
    # row 0 (position 0) sees only key 0; head h reads kv head h // 2
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], V[0, h // 2])


def test_equal_keys_average_values():
    rng = np.random.default_rng(10)
    c = 12
    K = np.repeat(rng.standard_normal((1, 1, 64)), c + 1, axis=0)
    V = rng.standard_normal((c + 1, 1, 64))
    Q = rng.standard_normal((1, 3, 64))
    out = oracle.attention(Q, K[:c], V[:c], K[c:], V[c:], [1], [c], 0.3)
    for h in range(3):
        np.testing.assert_allclose(out[0, h], V[:, 0].mean(axis=0), atol=1e-14, rtol=0)


def test_dominant_key_selects_its_value():
    # a huge scale makes the softmax a hard argmax over the visible keys;
    # the key picked must be the largest-score one (not the smallest)
    rng = np.random.default_rng(12)
    n, c, d = 1, 20, 32
    K = rng.standard_normal((c + n, 1, d))
    V = rng.standard_normal((c + n, 1, d))
    Q = rng.standard_normal((n, 2, d))
    out = oracle.attention(Q, K[:c], V[:c], K[c:], V[c:], [n], [c], 1e4)
    for h in range(2):
        scores = K[:, 0] @ Q[0, h]
        np.testing.assert_allclose(out[0, h], V[int(np.argmax(scores)), 0], atol=1e-12, rtol=0)
        assert not np.allclose(out[0, h], V[int(np.argmin(scores)), 0])


def test_large_logits_stay_finite():
    rng = np.random.default_rng(13)
    K = rng.standard_normal((50, 1, 64)) * 30
    V = rng.standard_normal((50, 1, 64))
    Q = rng.standard_normal((2, 2, 64)) * 30
    out = oracle.attention(Q, K[:48], V[:48], K[48:], V[48:], [2], [48], 1.0)
    assert np.all(np.isfinite(out))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_loop_oracle_matches_full_matrix_form(seed):
    st = workloads.random_step(seed, dtype="f32", num_q_heads=6, num_kv_heads=2, head_dim=32,
                               num_seqs=5, max_q=12, max_ctx=40)
    out = H.oracle_out(st)
    ref = brute.attention(H.f64(st.q), H.f64(st.k_ctx), H.f64(st.v_ctx), H.f64(st.k),
                          H.f64(st.v), st.q_lens, st.num_computed, st.scale)
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)


def test_row_selection_computes_only_selected_rows():
    st = workloads.random_step(4, dtype="f16", num_q_heads=4, num_kv_heads=2, head_dim=64,
                               num_seqs=3, max_q=6, max_ctx=30)
    full = H.oracle_out(st)
    sel = H.sample_rows(st, 3)
    part = H.oracle_out(st, row_sel=sel)
    np.testing.assert_array_equal(part[sel], full[sel])
    assert np.all(np.isnan(part[~sel]))


def test_config1_matches_full_matrix_form():
    st = workloads.config(1)
    out = H.oracle_out(st)
    ref = brute.attention(H.f64(st.q), H.f64(st.k_ctx), H.f64(st.v_ctx), H.f64(st.k),
                          H.f64(st.v), st.q_lens, st.num_computed, st.scale)
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)
    # the 8-token chunk at num_computed 0: its first row sees one key
    t_first_chunk = 4
    for h in range(2):
        np.testing.assert_array_equal(out[t_first_chunk, h], H.f64(st.v)[t_first_chunk, 0])


# --------------------------------------------------------------------------
# block copy (copy-on-write, swap out / in)


def _pools_with_context(seed, layers=2):
    st = workloads.random_step(seed, dtype="bf16", num_q_heads=4, num_kv_heads=2, head_dim=64,
                               num_seqs=4, max_q=8, max_ctx=60, num_layers=layers, layer=layers - 1)
    return st, H.host_pools(st)


def test_swap_round_trip_is_lossless():
    # tinyserve README "Correctness & testing": swap round-trip losslessness
    st, (pk, pv) = _pools_with_context(31)
    used = np.unique(st.block_tables[st.block_tables >= 0])
    host_k = np.zeros((pk.shape[0], len(used)) + pk.shape[2:], dtype=pk.dtype)
    host_v = np.zeros_like(host_k)
    oracle.copy_blocks(pk, pv, host_k, host_v, used, np.arange(len(used)))
    back_k = np.full_like(pk, 7)
    back_v = np.full_like(pv, 7)
    oracle.copy_blocks(host_k, host_v, back_k, back_v, np.arange(len(used)), used)
    np.testing.assert_array_equal(back_k[:, used], pk[:, used])
    np.testing.assert_array_equal(back_v[:, used], pv[:, used])
    rest = np.setdiff1d(np.arange(pk.shape[1]), used)
    assert np.all(back_k[:, rest] == 7) and np.all(back_v[:, rest] == 7)


def test_copy_on_write_duplicate_serves_the_same_tokens():
    # tinyserve README "How it works": a write into a shared block first
    # copies it; the copy must read back exactly as the original
    st, (pk, pv) = _pools_with_context(32)
    s = int(np.argmax(st.num_computed))
    n = int(st.num_computed[s])
    row = st.block_tables[s].copy()
    free = np.setdiff1d(np.arange(pk.shape[1]), st.block_tables[st.block_tables >= 0])
    last = (n - 1) // 16
    before_k, before_v = pk.copy(), pv.copy()
    oracle.copy_blocks(pk, pv, pk, pv, [row[last]], [free[0]])
    new_row = row.copy()
    new_row[last] = free[0]
    for layer in range(pk.shape[0]):
        a = oracle.gather(pk, pv, layer, row, n)
        b = oracle.gather(pk, pv, layer, new_row, n)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])
    # only the destination block changed
    diff = np.any(pk != before_k, axis=(0, 2, 3, 4)) | np.any(pv != before_v, axis=(0, 2, 3, 4))
    assert set(np.nonzero(diff)[0].tolist()) <= {int(free[0])}


# --------------------------------------------------------------------------
# rotary position embedding (tinyserve README "Highlights": the Qwen2 forward
# applies rotary embeddings; PageServe "01 Scheduler loop": explicit
# position_ids per packed token)


@pytest.mark.parametrize("d,theta", [(64, 1e4), (128, 1e6)])
def test_rope_matches_transformers_qwen2(d, theta):
    # library routine: the Qwen2 rotary embedding of the transformers
    # package. It forms its angles and cos/sin in fp32, so positions stay
    # small (< 64) and the tolerance covers fp32 angle rounding
    # (64 * 2^-24 * |x| per element).
    transformers = pytest.importorskip("transformers")
    from transformers.models.qwen2.modeling_qwen2 import Qwen2RotaryEmbedding, apply_rotary_pos_emb
    cfg = transformers.Qwen2Config(hidden_size=d * 4, num_attention_heads=4, num_key_value_heads=2,
                                   rope_theta=theta)
    rot = Qwen2RotaryEmbedding(config=cfg)
    rng = np.random.default_rng(7)
    T = 48
    pos = rng.integers(0, 64, T)
    x = rng.standard_normal((T, 3, d))
    xt = torch.from_numpy(x).permute(1, 0, 2)[None]  # [1, H, T, D]
    cos, sin = rot(xt, torch.from_numpy(pos)[None])
    ref, _ = apply_rotary_pos_emb(xt, xt, cos, sin)
    ref = ref[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(oracle.rope(x, pos, theta), ref, rtol=0, atol=5e-5)


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(1).standard_normal((5, 4, 64))
    assert np.array_equal(oracle.rope(x, np.zeros(5, np.int32), 1e6), x)


def test_rope_two_dims_is_a_plane_rotation_by_the_position():
    # D = 2: one pair, frequency theta^0 = 1, so the angle is the position
    # itself: multiply x0 + i x1 by e^{i pos}
    rng = np.random.default_rng(2)
    x = rng.standard_normal((9, 1, 2))
    pos = np.array([0, 1, 2, 3, 7, 100, 12345, 10**6, 2**30], np.int32)
    z = (x[:, 0, 0] + 1j * x[:, 0, 1]) * np.exp(1j * pos.astype(np.float64))
    got = oracle.rope(x, pos, 10.0)
    np.testing.assert_allclose(got[:, 0, 0], z.real, rtol=0, atol=1e-9)
    np.testing.assert_allclose(got[:, 0, 1], z.imag, rtol=0, atol=1e-9)


def test_rope_preserves_every_pair_norm():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 3, 128))
    pos = rng.integers(0, 1 << 20, 16)
    y = oracle.rope(x, pos, 1e6)
    h = 64
    np.testing.assert_allclose(y[..., :h] ** 2 + y[..., h:] ** 2, x[..., :h] ** 2 + x[..., h:] ** 2,
                               rtol=1e-12, atol=1e-12)


def test_rope_scores_depend_only_on_relative_position():
    # <R(m) q, R(n) k> is a function of m - n alone
    rng = np.random.default_rng(4)
    for d, theta in [(64, 1e4), (128, 1e6)]:
        q = rng.standard_normal((1, 1, d))
        k = rng.standard_normal((1, 1, d))
        for m, n, delta in [(5, 2, 11), (0, 0, 1000), (300, 17, 4096), (9, 40, 77777)]:
            a = np.sum(oracle.rope(q, [m], theta) * oracle.rope(k, [n], theta))
            b = np.sum(oracle.rope(q, [m + delta], theta) * oracle.rope(k, [n + delta], theta))
            assert abs(a - b) <= 1e-9 * (1 + abs(a)), (d, m, n, delta)
        # and the relative offset matters (the rotation is not trivial)
        a = np.sum(oracle.rope(q, [3], theta) * oracle.rope(k, [0], theta))
        b = np.sum(oracle.rope(q, [4], theta) * oracle.rope(k, [0], theta))
        assert abs(a - b) > 1e-3


def test_rope_rotations_compose_additively():
    # turning by position a and then by position b equals turning by a + b
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 2, 64))
    a = np.array([0, 1, 31, 500, 4096, 70000], np.int32)
    b = np.array([3, 0, 33, 12, 4095, 1], np.int32)
    np.testing.assert_allclose(oracle.rope(oracle.rope(x, a, 1e4), b, 1e4), oracle.rope(x, a + b, 1e4),
                               rtol=0, atol=1e-9)
