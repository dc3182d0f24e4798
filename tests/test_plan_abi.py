"""Host-side checks of the C ABI: exported symbols, the planner's packed
metadata against the oracle's slot formula, validation errors, and the
step's algorithmic byte / FLOP accounting. No GPU needed: nothing here
launches a kernel or touches device memory."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import paged_kv_attention_packed_amd as P
from paged_kv_attention_packed_amd import _binding as B
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DT = {"f32": P.PS_F32, "f16": P.PS_F16, "bf16": P.PS_BF16}


def _pool(st, layer=None):
    return P.ps_pool(0, 0, st.num_layers, st.num_blocks, 16, st.num_kv_heads, st.head_dim,
                     DT[st.dtype_name], st.layer if layer is None else layer)


def _plan(st, flags=0, **options):
    opts = P.plan_options(**options) if options else None
    return P.ps_plan_step(st.q_lens, st.num_computed, st.block_tables, st.num_q_heads, _pool(st), flags, opts)


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "ps.h")).read()
    declared = set(re.findall(r"\b(ps_[a-z_]+)\s*\(", header))
    assert declared == set(B.EXPORTED), declared ^ set(B.EXPORTED)
    for name in declared:
        assert hasattr(B.lib, name), name
    assert P.ps_abi_version() == int(re.search(r"#define PS_ABI_VERSION (\d+)", header).group(1))


def test_one_hip_runtime_whatever_the_import_order():
    # imported before torch, the package must still leave a single HIP
    # runtime in the process (torch's), or the library's calls would not
    # see the device torch allocates on
    import subprocess
    import sys
    code = ("import paged_kv_attention_packed_amd, torch\n"
            "maps = open('/proc/self/maps').read()\n"
            "print(len({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))\n")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip().splitlines()[-1] == "1", res.stdout


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_planner_arrays_match_oracle_slot_formula(idx):
    st = workloads.config(idx, values=False)
    plan = _plan(st)
    h = P.ps_plan_host_arrays(plan, st.num_seqs, st.num_tokens)
    ql, nc = st.q_lens.astype(np.int64), st.num_computed.astype(np.int64)
    np.testing.assert_array_equal(h["query_start_loc"], np.concatenate([[0], np.cumsum(ql)]))
    np.testing.assert_array_equal(h["num_computed_tokens"], nc)
    np.testing.assert_array_equal(h["context_lens"], nc + ql)
    np.testing.assert_array_equal(h["block_tables"], st.block_tables)
    expect, positions = [], []
    for s in range(st.num_seqs):
        for i in range(int(ql[s])):
            expect.append(oracle.slot(st.block_tables[s], int(nc[s]) + i))
            positions.append(int(nc[s]) + i)
    np.testing.assert_array_equal(h["slot_mapping"], np.array(expect, dtype=np.int32))
    # explicit position of each packed token (PageServe "01 Scheduler loop", Pack)
    np.testing.assert_array_equal(h["positions"], np.array(positions, dtype=np.int32))
    assert len(set(expect)) == len(expect)


def test_planner_slots_match_page_example():
    # tinyserve README "How it works": seq A (19 tokens) [7, 2]; a step that
    # appends A's tokens 16..18 writes slots 32, 33, 34 (block 2)
    pool = P.ps_pool(0, 0, 1, 8, 16, 1, 64, P.PS_F16, 0)
    plan = P.ps_plan_step([3], [16], np.array([[7, 2]]), 2, pool)
    h = P.ps_plan_host_arrays(plan, 1, 3)
    assert h["slot_mapping"].tolist() == [32, 33, 34]


def test_algorithmic_accounting():
    st = workloads.config(4, values=False)
    info = P.ps_plan_get_info(_plan(st))
    ctx = st.num_computed.astype(np.int64) + st.q_lens
    row = 2 * st.head_dim * 2 * st.num_kv_heads           # K+V bytes per token, all KV heads (bf16)
    assert info["kv_bytes_decode"] == int(ctx.sum()) * row
    assert info["kv_bytes_prefill"] == 0
    # unique: the 1024 shared prefix tokens count once
    assert info["kv_bytes_unique"] == int((ctx - 1024).sum() + 1024) * row
    T = st.num_tokens
    assert info["q_bytes"] == T * st.num_q_heads * st.head_dim * 2
    assert info["scatter_bytes"] == 2 * 2 * T * st.num_kv_heads * st.head_dim * 2 + 4 * T
    assert info["flops_decode"] == pytest.approx(4 * st.head_dim * st.num_q_heads * float(ctx.sum()))
    # a prefill chunk's flops: every row sees c + i + 1 keys
    st5 = workloads.config(5, values=False)
    i5 = P.ps_plan_get_info(_plan(st5))
    n, c = 2048, 30000
    assert i5["flops_prefill"] == pytest.approx(4 * 128 * 12 * (n * c + n * (n + 1) / 2))
    assert i5["kv_bytes_decode"] == 2 ** 30


def test_forced_paths_cover_every_sequence():
    st = workloads.config(3, values=False)
    dec = P.ps_plan_get_info(_plan(st, P.PS_PLAN_ALL_DECODE))
    pre = P.ps_plan_get_info(_plan(st, P.PS_PLAN_ALL_PREFILL))
    assert dec["prefill_seqs"] == 0 and dec["decode_seqs"] == st.num_seqs and dec["prefill_items"] == 0
    assert pre["decode_seqs"] == 0 and pre["prefill_seqs"] == st.num_seqs and pre["decode_items"] == 0
    dflt = P.ps_plan_get_info(_plan(st))
    assert dflt["decode_seqs"] == 128 and dflt["prefill_seqs"] == 4


def test_empty_step():
    pool = P.ps_pool(0, 0, 1, 4, 16, 2, 128, P.PS_BF16, 0)
    plan = P.ps_plan_step(np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros((0, 1), np.int32), 12, pool)
    info = P.ps_plan_get_info(plan)
    assert info["num_tokens"] == 0 and info["decode_items"] == 0 and info["prefill_items"] == 0
    assert P.ps_plan_sizes(plan)[1] == 0


def _expect_error(status, fn, *args, match=None, **kwargs):
    with pytest.raises(P.PsError) as e:
        fn(*args, **kwargs)
    assert e.value.status == status
    if match:
        assert re.search(match, str(e.value)), str(e.value)


def test_validation_errors():
    pool = P.ps_pool(0, 0, 1, 8, 16, 2, 64, P.PS_F16, 0)
    bt = np.array([[0, 1], [2, 3]], dtype=np.int32)
    INV, UNS = B.PS_ERR_INVALID_ARGUMENT, B.PS_ERR_UNSUPPORTED
    _expect_error(INV, P.ps_plan_step, [1, 0], [3, 3], bt, 4, pool, match="q_lens")
    _expect_error(INV, P.ps_plan_step, [1, 1], [-1, 3], bt, 4, pool, match="num_computed")
    _expect_error(INV, P.ps_plan_step, [1, 1], [3, 40], bt, 4, pool, match="table width")
    _expect_error(INV, P.ps_plan_step, [1, 1], [3, 3], np.array([[0, 1], [9, 3]]), 4, pool, match="outside")
    # (the same in a full block, which the scan takes on its own path, and
    # a negative id)
    _expect_error(INV, P.ps_plan_step, [1, 1], [20, 3], np.array([[9, 1], [2, 3]]), 4, pool, match="outside")
    _expect_error(INV, P.ps_plan_step, [1, 1], [20, 3], np.array([[-1, 1], [2, 3]]), 4, pool, match="outside")
    _expect_error(INV, P.ps_plan_step, [1, 1], [3, 20], np.array([[0, 1], [2, 2]]), 4, pool, match="twice")
    # sequence 1 appends into block 0, which sequence 0 also reads
    _expect_error(INV, P.ps_plan_step, [1, 1], [20, 3], np.array([[0, 1], [0, 3]]), 4, pool, match="share")
    _expect_error(INV, P.ps_plan_step, [1, 1], [3, 3], bt, 5, pool, match="multiple")
    _expect_error(INV, P.ps_plan_step, [1, 1], [3, 3], bt, 4, pool, 7, match="flags")
    for field, val, st in [("head_dim", 96, UNS), ("block_size", 32, UNS), ("dtype", 7, UNS),
                           ("layer", 1, INV), ("num_kv_heads", 0, INV)]:
        bad = P.ps_pool(0, 0, 1, 8, 16, 2, 64, P.PS_F16, 0)
        setattr(bad, field, val)
        _expect_error(st, P.ps_plan_step, [1, 1], [3, 3], bt, 4, bad)
    # a valid plan with reads of a shared block is fine
    P.ps_plan_step([1, 1], [20, 20], np.array([[0, 1], [0, 3]]), 4, pool)
    # limits: slots (num_blocks * 16) and a block's bytes must fit int32
    big = P.ps_pool(0, 0, 1, (1 << 27), 16, 2, 64, P.PS_F16, 0)
    _expect_error(UNS, P.ps_plan_step, [1, 1], [3, 3], bt, 4, big, match="slots")
    wide = P.ps_pool(0, 0, 1, 8, 16, 1 << 18, 128, P.PS_F32, 0)
    _expect_error(UNS, P.ps_plan_step, [1, 1], [3, 3], bt, 1 << 18, wide, match="block exceeds")
    _expect_error(UNS, P.ps_reshape_and_cache, 1, 1, 1, 4, wide, match="block exceeds")
    _expect_error(UNS, P.ps_copy_blocks, wide, wide, 1, 1, 1, match="block exceeds")


def test_attention_argument_errors_return_before_any_launch():
    st = workloads.config(5, values=False)
    plan = _plan(st)
    pool = _pool(st)
    meta, ws = P.ps_plan_sizes(plan)
    assert ws > 0
    args = dict(q=1 << 20, pool=pool, block_tables=1 << 20, block_table_stride=st.block_tables.shape[1],
                query_start_loc=1 << 20, num_computed_tokens=1 << 20, context_lens=1 << 20,
                out=1 << 20, num_seqs=st.num_seqs, num_tokens=st.num_tokens,
                num_q_heads=st.num_q_heads, scale=0.125, plan=plan, workspace=1 << 20,
                workspace_bytes=ws)
    INV = B.PS_ERR_INVALID_ARGUMENT

    def call(**kw):
        a = dict(args)
        a.update(kw)
        P.ps_paged_attention(**a)

    _expect_error(INV, call, num_tokens=st.num_tokens + 1, match="differ")
    _expect_error(INV, call, num_q_heads=7, match="differ")
    _expect_error(INV, call, block_table_stride=3, match="stride")
    _expect_error(B.PS_ERR_WORKSPACE_TOO_SMALL, call, workspace_bytes=ws - 1)
    _expect_error(INV, call, scale=0.0, match="scale")
    _expect_error(INV, call, scale=float("nan"), match="scale")
    # everything consistent, but the plan was never uploaded
    _expect_error(INV, call, match="uploaded")
    bad = _pool(st)
    bad.head_dim = 64
    _expect_error(INV, call, pool=bad, match="geometry")


def test_scatter_argument_errors():
    pool = P.ps_pool(0, 0, 1, 8, 16, 2, 64, P.PS_F16, 0)
    _expect_error(B.PS_ERR_INVALID_ARGUMENT, P.ps_reshape_and_cache, 1, 1, 1, -1, pool)
    _expect_error(B.PS_ERR_INVALID_ARGUMENT, P.ps_reshape_and_cache, 0, 1, 1, 4, pool)
    bad = P.ps_pool(0, 0, 1, 8, 8, 2, 64, P.PS_F16, 0)
    _expect_error(B.PS_ERR_UNSUPPORTED, P.ps_reshape_and_cache, 1, 1, 1, 4, bad)
    # zero tokens is a no-op even with NULL pointers
    P.ps_reshape_and_cache(0, 0, 0, 0, pool)


def test_rope_scatter_argument_errors():
    pool = P.ps_pool(1 << 20, 1 << 21, 1, 8, 16, 2, 64, P.PS_F16, 0)
    INV, UNS = B.PS_ERR_INVALID_ARGUMENT, B.PS_ERR_UNSUPPORTED
    args = dict(q=1 << 22, q_out=1 << 23, k=1 << 24, v=1 << 25, positions=1 << 26,
                slot_mapping=1 << 27, num_tokens=4, num_q_heads=4, rope_theta=1e6, pool=pool)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        P.ps_rope_reshape_and_cache(**a)

    _expect_error(INV, call, num_tokens=-1, match="num_tokens")
    _expect_error(INV, call, num_q_heads=-1, match="num_q_heads")
    for theta in (0.0, -1.0, float("nan"), float("inf")):
        _expect_error(INV, call, rope_theta=theta, match="rope_theta")
    _expect_error(INV, call, positions=0, match="NULL")
    _expect_error(INV, call, k=0, match="NULL")
    _expect_error(INV, call, q=0, match="q or q_out")
    # 4 tokens x 4 heads x 64 x 2 bytes = 2048 bytes: q_out 1 KiB past q overlaps it
    _expect_error(INV, call, q_out=(1 << 22) + 1024, match="overlap")
    bad = P.ps_pool(1 << 20, 1 << 21, 1, 8, 16, 2, 96, P.PS_F16, 0)
    _expect_error(UNS, call, pool=bad, match="head_dim")
    bad = P.ps_pool(1 << 20, 1 << 21, 1, 8, 16, 2, 64, P.PS_F16, 1)
    _expect_error(INV, call, pool=bad, match="layer")
    # zero tokens is a no-op even with NULL pointers
    P.ps_rope_reshape_and_cache(0, 0, 0, 0, 0, 0, 0, 4, 1e4, pool)


def test_spec_verify_argument_errors():
    INV, UNS, WS = B.PS_ERR_INVALID_ARGUMENT, B.PS_ERR_UNSUPPORTED, B.PS_ERR_WORKSPACE_TOO_SMALL
    V, S = 151936, 32
    ws = P.ps_spec_verify_workspace_bytes(S, V)
    # 38 chunks of 4096 entries: one u64 sum each, then two int32 per sequence
    assert ws == 256 * -(-(S * 38 * 8) // 256) + 256 * -(-(S * 8) // 256)
    assert P.ps_spec_verify_workspace_bytes(0, V) == 0
    args = dict(target_probs=1 << 22, draft_probs=1 << 23, draft_tokens=1 << 24, draft_start=1 << 25,
                accept_uniforms=1 << 26, sample_uniforms=1 << 27, num_seqs=S, total_drafts=128,
                vocab_size=V, num_accepted=1 << 28, next_token=1 << 29, workspace=1 << 30,
                workspace_bytes=ws)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        P.ps_spec_verify(**a)

    _expect_error(INV, call, num_seqs=-1, match="num_seqs")
    _expect_error(INV, call, total_drafts=-1, match="total_drafts")
    _expect_error(UNS, call, vocab_size=0, match="vocab_size")
    _expect_error(UNS, call, vocab_size=(1 << 23) + 1, match="vocab_size")
    _expect_error(WS, call, workspace_bytes=ws - 1)
    _expect_error(INV, call, workspace=(1 << 30) + 4, match="aligned")
    _expect_error(INV, call, target_probs=0, match="NULL")
    _expect_error(INV, call, draft_tokens=0, match="NULL")
    # no drafts: the draft arrays may be NULL (the call is then plain sampling); zero sequences is a no-op
    P.ps_spec_verify(0, 0, 0, 0, 0, 0, 0, 0, V, 0, 0, 0, 0)


def test_split_plan_depends_only_on_logical_lengths():
    a = workloads.config(3, values=False)
    b = workloads.build_step("b", 77, "f16", 12, 2, 128, a.num_blocks, a.q_lens, a.num_computed,
                             values=False)
    pa, pb = _plan(a), _plan(b)
    ia, ib = P.ps_plan_get_info(pa), P.ps_plan_get_info(pb)
    for key in ("decode_items", "prefill_items", "merge_items"):
        assert ia[key] == ib[key]
    assert P.ps_plan_sizes(pa)[1] == P.ps_plan_sizes(pb)[1]


def test_shared_prefix_groups():
    # two groups (10 sequences sharing 320 tokens, 9 sharing 512) among
    # sequences that share nothing, one of which shares only one block
    st = workloads.prefix_groups_step(3, values=False)
    g, hkv = st.num_q_heads // st.num_kv_heads, st.num_kv_heads
    SP = P.PS_PLAN_SHARED_PREFIX
    # the pass is opt-in: by default physical sharing changes nothing
    off = P.ps_plan_get_info(_plan(st))
    assert off["prefix_groups"] == off["prefix_items"] == off["prefill_items"] == 0
    assert off["decode_items"] == 24 * hkv and off["step_fused"] == 1

    info = P.ps_plan_get_info(_plan(st, SP))
    assert info["prefix_groups"] == 2
    assert info["prefill_items"] == info["prefix_items"] > 0
    assert info["step_fused"] == 1
    # one prefix pass per (group, KV head, chunk of <= 128 gathered rows, key slice)
    assert info["prefix_items"] % hkv == 0
    assert info["prefix_items"] >= hkv * (-(-10 * g // 128) + -(-9 * g // 128))
    # every grouped sequence merges its own keys with the prefix pass
    assert info["merge_items"] >= 19 * hkv
    kinds = P.ps_plan_sequence_kernels(_plan(st, SP), st.num_seqs)
    assert (kinds == 2).sum() == 19 and (kinds == 0).sum() == st.num_seqs - 19

    assert P.ps_plan_get_info(_plan(st, SP, prefix_min_seqs=10))["prefix_groups"] == 1   # group B has 9
    assert P.ps_plan_get_info(_plan(st, SP, prefix_min_seqs=11))["prefix_groups"] == 0   # the outlier stays out of A
    assert P.ps_plan_get_info(_plan(st, SP, prefix_min_keys=336))["prefix_groups"] == 1  # group A shares 320

    for flags in (P.PS_PLAN_ALL_DECODE, P.PS_PLAN_ALL_PREFILL):
        assert P.ps_plan_get_info(_plan(st, flags | SP))["prefix_groups"] == 0
    # a chunk in the step: the scatter is no longer fused
    wp = workloads.prefix_groups_step(3, with_prefill=True, values=False)
    iw = P.ps_plan_get_info(_plan(wp, SP))
    assert iw["prefix_groups"] == 2 and iw["step_fused"] == 0
    assert iw["prefill_items"] > iw["prefix_items"]


def test_long_shared_prefix_slices_fit_a_prefill_item():
    # 256 sequences of 64 query / 8 KV heads sharing a 20480-token prefix:
    # each (KV head, 128-row chunk) gets one prefix slice by the item-count
    # rule, but no prefill item may span more keys than it stages block
    # ids for (16384), so every chunk takes two slices of 10240
    S, prefix = 256, 20480
    nc = np.full(S, prefix + 37, dtype=np.int32)
    st = workloads.build_step("long-prefix", 5, "bf16", 64, 8, 128, 8192, [1] * S, nc.tolist(),
                              prefix_tokens=prefix, values=False)
    info = P.ps_plan_get_info(_plan(st, P.PS_PLAN_SHARED_PREFIX))
    chunks = 8 * (S * 8 // 128)
    assert info["prefix_groups"] == 1
    assert info["prefix_items"] == 2 * chunks
    # an explicit slice length above the limit is refused
    _expect_error(B.PS_ERR_INVALID_ARGUMENT, _plan, st, P.PS_PLAN_SHARED_PREFIX, prefix_slice_keys=20480,
                  match="prefix_slice_keys")


def test_options_are_validated_and_recorded(monkeypatch):
    st = workloads.config(3, values=False)
    INV = B.PS_ERR_INVALID_ARGUMENT
    for kw in (dict(decode_split_keys=24), dict(decode_split_keys=32768), dict(prefill_split_keys=100),
               dict(decode_waves=6), dict(prefix_min_seqs=1)):
        _expect_error(INV, _plan, st, **kw)
    _expect_error(INV, _plan, st, decode_waves=16, match="head_dim 64")
    info = P.ps_plan_get_info(_plan(st, decode_split_keys=512, prefill_split_keys=256))
    assert info["decode_split_keys"] == 512 and info["prefill_split_keys"] == 256
    assert info["merge_items"] > 0 and info["workspace_rows"] > 0
    dflt = P.ps_plan_get_info(_plan(st))
    assert dflt["mixed_launch"] == 1
    assert P.ps_plan_get_info(_plan(st, P.PS_PLAN_SEPARATE_LAUNCHES))["mixed_launch"] == 0
    # nothing in the environment changes a plan
    for name in ("PS_DECODE_SPLIT", "PS_PREFILL_SPLIT", "PS_CASCADE", "PS_DECODE_WAVES", "PS_MIXED"):
        monkeypatch.setenv(name, "64")
    again = P.ps_plan_get_info(_plan(st))
    for key in ("decode_items", "prefill_items", "merge_items", "decode_split_keys", "prefill_split_keys",
                "decode_waves", "mixed_launch", "prefix_groups"):
        assert again[key] == dflt[key], key


def test_decode_stream_choice():
    """Decode K/V loads stream (non-temporal) only for steps that read every
    block once and more decode K/V than the 256 MiB last-level cache; the
    option forces either policy, and fixed-shape plans keep cached loads."""
    INV = B.PS_ERR_INVALID_ARGUMENT
    c3, c4, c5 = (workloads.config(i, values=False) for i in (3, 4, 5))
    _expect_error(INV, _plan, c3, decode_stream_kv=3)
    _expect_error(INV, _plan, c3, decode_stream_kv=-1)
    info5 = P.ps_plan_get_info(_plan(c5))
    assert info5["kv_bytes_decode"] > (256 << 20) and info5["kv_bytes_unique"] == (
        info5["kv_bytes_decode"] + info5["kv_bytes_prefill"])
    assert info5["decode_stream_kv"] == 1
    # small step (its K/V fit the cache): cached
    assert P.ps_plan_get_info(_plan(c3))["kv_bytes_decode"] < (256 << 20)
    assert P.ps_plan_get_info(_plan(c3))["decode_stream_kv"] == 0
    # shared prefix blocks are read again within the step: cached
    assert P.ps_plan_get_info(_plan(c4))["kv_bytes_unique"] < P.ps_plan_get_info(_plan(c4))["kv_bytes_decode"]
    assert P.ps_plan_get_info(_plan(c4))["decode_stream_kv"] == 0
    # forced either way
    assert P.ps_plan_get_info(_plan(c3, decode_stream_kv=1))["decode_stream_kv"] == 1
    assert P.ps_plan_get_info(_plan(c5, decode_stream_kv=2))["decode_stream_kv"] == 0
    # the choice changes nothing else in the plan
    a, b = P.ps_plan_get_info(_plan(c5)), P.ps_plan_get_info(_plan(c5, decode_stream_kv=2))
    for key in ("decode_items", "prefill_items", "merge_items", "decode_split_keys", "prefill_split_keys",
                "decode_waves", "mixed_launch", "workspace_rows"):
        assert a[key] == b[key], key
    # a long unshared decode step in a fixed shape stays cached
    long_ctx = workloads.build_step("fixed-long", 1, "bf16", 12, 2, 128, 80000, [1] * 32, [32767] * 32,
                                    values=False)
    fx = P.ps_plan_get_info(_plan(long_ctx, P.PS_PLAN_FIXED_SHAPE, max_seqs=32, max_tokens=32, max_query_len=1,
                                  max_decode_items=1024, max_merge_items=4096, max_workspace_rows=1 << 16))
    assert fx["kv_bytes_decode"] > (256 << 20) and fx["decode_stream_kv"] == 0


def test_walk_rotation_choice():
    # walk rotation: the planner's choice is on from 512 decode items up
    # (a function of the step's logical shape), off for fixed shapes; the
    # option forces it either way
    INV = B.PS_ERR_INVALID_ARGUMENT
    c2, c4, c5 = (workloads.config(i, values=False) for i in (2, 4, 5))
    _expect_error(INV, _plan, c2, decode_walk_rotation=3)
    assert P.ps_plan_get_info(_plan(c2))["decode_walk_rotation"] == 0      # 128 items
    assert P.ps_plan_get_info(_plan(c4))["decode_walk_rotation"] == 1      # 512 items
    assert P.ps_plan_get_info(_plan(c5))["decode_walk_rotation"] == 1
    assert P.ps_plan_get_info(_plan(c4, decode_walk_rotation=2))["decode_walk_rotation"] == 0
    assert P.ps_plan_get_info(_plan(c2, decode_walk_rotation=1))["decode_walk_rotation"] == 1
    # the same logical step with the prefix blocks shared or private: the
    # same choice
    priv = workloads.build_step("c4-private", 4, "bf16", 12, 2, 128, 32768, c4.q_lens.tolist(),
                                c4.num_computed.tolist(), values=False)
    assert P.ps_plan_get_info(_plan(priv))["decode_walk_rotation"] == 1


def test_sequence_kernels():
    st = workloads.config(3, values=False)
    kinds = P.ps_plan_sequence_kernels(_plan(st), st.num_seqs)
    g = st.num_q_heads // st.num_kv_heads
    np.testing.assert_array_equal(kinds, np.where(g * st.q_lens > 32, 1, 0))
    assert (P.ps_plan_sequence_kernels(_plan(st, P.PS_PLAN_ALL_PREFILL), st.num_seqs) == 1).all()


def _fixed(**kw):
    base = dict(max_seqs=64, max_tokens=64, max_query_len=1)
    base.update(kw)
    return base


def test_fixed_shape_layout_depends_only_on_capacities():
    # two decode steps of different lengths and sequence counts planned to
    # one fixed shape: same metadata and workspace sizes, same launch
    # counts, and idle items pad the work lists
    c2 = workloads.config(2, values=False)
    a = workloads.build_step("c2-width64", 12, "f16", 14, 2, 64, 4096, c2.q_lens, c2.num_computed,
                             table_width=64, values=False)
    b = workloads.build_step("c2-next", 13, "f16", 14, 2, 64, 4096, [1] * 50,
                             np.random.default_rng(3).integers(15, 700, 50).tolist(),
                             table_width=64, values=False)
    F = P.PS_PLAN_FIXED_SHAPE
    pa = _plan(a, F, **_fixed())
    pb = _plan(b, F, **_fixed())
    assert P.ps_plan_sizes(pa) == P.ps_plan_sizes(pb)
    ia, ib = P.ps_plan_get_info(pa), P.ps_plan_get_info(pb)
    for key in ("decode_items", "merge_items", "decode_row_tiles", "decode_waves", "workspace_rows"):
        assert ia[key] == ib[key], key
    assert ia["decode_items"] == 128 and ia["active_decode_items"] == 128
    assert ib["active_decode_items"] == 100 and ib["step_fused"] == 1
    # too many sequences, too long a query, a prefill route: refused
    INV = B.PS_ERR_INVALID_ARGUMENT
    _expect_error(INV, _plan, a, F, **_fixed(max_seqs=63), match="exceeds")
    _expect_error(INV, _plan, a, F, **_fixed(max_query_len=5), match="rows")
    _expect_error(INV, _plan, a, F | P.PS_PLAN_ALL_PREFILL, **_fixed(), match="FIXED")
    _expect_error(INV, _plan, a, F | P.PS_PLAN_SHARED_PREFIX, **_fixed(), match="FIXED")
    # key splits need merge capacity
    _expect_error(INV, _plan, a, F, **_fixed(decode_split_keys=64), match="fixed shape holds")
    ok = P.ps_plan_get_info(_plan(a, F, **_fixed(decode_split_keys=64, max_decode_items=2048,
                                                  max_merge_items=1024, max_workspace_rows=16384)))
    assert ok["merge_items"] == 1024 and 0 < ok["active_merge_items"] <= 1024


def _c5_like_tables(num_blocks, seed=0):
    rng = np.random.default_rng(seed)
    q_lens = np.array([5] * 32 + [2048], dtype=np.int32)
    nc = np.array([32763] * 32 + [30000], dtype=np.int32)
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = np.full((33, 2048), -1, dtype=np.int32)
    off = 0
    for s in range(33):
        nb = -(-(int(nc[s]) + int(q_lens[s])) // 16)
        bt[s, :nb] = perm[off:off + nb]
        off += nb
    return q_lens, nc, bt


def test_planner_cost_follows_the_step_not_the_pool():
    # the same C5-shaped step (67k table entries) over pools of 100k and of
    # 1M blocks: the plans agree, and the larger pool does not make the
    # planner walk or clear pool-sized state
    times = {}
    for nb in (100_000, 1_000_000):
        q_lens, nc, bt = _c5_like_tables(nb)
        pool = P.ps_pool(0, 0, 1, nb, 16, 2, 128, P.PS_BF16, 0)
        best, info = float("inf"), None
        for _ in range(5):
            plan = P.ps_plan_step(q_lens, nc, bt, 12, pool)
            info = P.ps_plan_get_info(plan)
            best = min(best, info["plan_us"])
        times[nb] = best
        assert info["kv_bytes_unique"] == info["kv_bytes_decode"] + info["kv_bytes_prefill"]
        # validation still sees every entry: a duplicate near the top of the pool
        bt2 = bt.copy()
        bt2[7, 100] = bt2[7, 3]
        _expect_error(B.PS_ERR_INVALID_ARGUMENT, P.ps_plan_step, q_lens, nc, bt2, 12, pool, match="twice")
        bt2 = bt.copy()
        bt2[32, 1999] = bt2[4, 10]   # the chunk appends into a block another table reads
        _expect_error(B.PS_ERR_INVALID_ARGUMENT, P.ps_plan_step, q_lens, nc, bt2, 12, pool, match="share")
    # generous bound (shared CI hosts are noisy): a pool-sized pass would be
    # 10x; the step-sized work is a small constant factor at most
    assert times[1_000_000] < 6 * times[100_000] + 2000, times
