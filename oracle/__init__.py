"""CPU fp64 oracle for one packed paged-attention step.

TEST INFRASTRUCTURE ONLY: the tests, the graft entry's smoke check and the
benchmark's CPU-baseline leg may import this package; the GPU library and
its Python binding never do. It shares no code with the GPU path.

The arithmetic lives in ``oracle.c`` (plain C loops, fp64, built by gcc);
this module only marshals numpy arrays into it. ``brute.py`` holds a
second, full-matrix numpy formulation used on tiny inputs.

Passages followed (see ``oracle.c`` for the per-function mapping):
PageServe "01 Scheduler loop" (Pack / Execute, System architecture),
"03 Paged KV cache" (slot formula, scatter, attend through the table),
"06 Development history" phase 7 (pool [layers, blocks, 16, H, D]) and
phase 8 (one packed [1, T] pass); tinyserve README "How it works" (two
K/V slabs, block tables, stepped causal mask for verify rows) and
"Highlights" (grouped-query attention, rotary embeddings of the Qwen2
forward pass), tinyserve README "How it works" (rejection-sampling
verification of speculative drafts).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f64p = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_slot.restype = ctypes.c_int64
    lib.oracle_slot.argtypes = [_i32p, ctypes.c_int64, ctypes.c_int32]
    lib.oracle_store_tokens.restype = None
    lib.oracle_store_tokens.argtypes = [
        _u8p, _u8p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        _i32p, ctypes.c_int64, ctypes.c_int64, _u8p, _u8p]
    lib.oracle_reshape_and_cache.restype = None
    lib.oracle_reshape_and_cache.argtypes = [
        _u8p, _u8p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        _u8p, _u8p, _i32p, _i32p, _i32p, ctypes.c_int32, ctypes.c_int32]
    lib.oracle_gather.restype = None
    lib.oracle_gather.argtypes = [
        _u8p, _u8p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        _i32p, ctypes.c_int64, _u8p, _u8p]
    lib.oracle_attention.restype = None
    lib.oracle_attention.argtypes = [
        _f64p, _f64p, _f64p, _f64p, _f64p, _i32p, _i32p, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
        _u8p, _f64p]
    lib.oracle_copy_blocks.restype = None
    lib.oracle_copy_blocks.argtypes = [_u8p, _u8p, _u8p, _u8p, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int64, _i32p, _i32p, ctypes.c_int32]
    lib.oracle_rope.restype = None
    lib.oracle_rope.argtypes = [_f64p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _i32p,
                                ctypes.c_double, _f64p]
    _f32p = ctypes.POINTER(ctypes.c_float)
    lib.oracle_spec_verify.restype = None
    lib.oracle_spec_verify.argtypes = [_f32p, _f32p, _i32p, _i32p, _f64p, _f64p, ctypes.c_int32,
                                       ctypes.c_int32, _i32p, _i32p]
    lib.oracle_num_threads.restype = ctypes.c_int32
    lib.oracle_num_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def slot(block_table_row, pos: int, block_size: int = 16) -> int:
    """Flat slot of logical position ``pos`` (PageServe "03 Paged KV cache")."""
    bt = _i32(block_table_row)
    return int(_load().oracle_slot(_ptr(bt, ctypes.c_int32), int(pos), int(block_size)))


def _pool_geometry(pool_k: np.ndarray):
    assert pool_k.ndim == 5, "pool is [layers, blocks, block_size, Hkv, D]"
    L, NB, bs, hkv, d = pool_k.shape
    return L, NB, bs, hkv, d, pool_k.dtype.itemsize


def store_tokens(pool_k, pool_v, layer, block_table_row, pos0, k_rows, v_rows):
    """Write ``len(k_rows)`` consecutive positions of one sequence into the pools."""
    L, NB, bs, hkv, d, elt = _pool_geometry(pool_k)
    assert pool_v.shape == pool_k.shape and pool_v.dtype == pool_k.dtype
    k_rows = np.ascontiguousarray(k_rows)
    v_rows = np.ascontiguousarray(v_rows)
    assert k_rows.dtype.itemsize == elt and k_rows.shape[1:] == (hkv, d)
    assert v_rows.shape == k_rows.shape
    bt = _i32(block_table_row)
    n = k_rows.shape[0]
    if n == 0:
        return
    _load().oracle_store_tokens(
        pool_k.view(np.uint8).ctypes.data_as(_u8p), pool_v.view(np.uint8).ctypes.data_as(_u8p),
        layer, NB, bs, hkv, d, elt, _ptr(bt, ctypes.c_int32), int(pos0), int(n),
        k_rows.view(np.uint8).ctypes.data_as(_u8p), v_rows.view(np.uint8).ctypes.data_as(_u8p))


def reshape_and_cache(pool_k, pool_v, layer, k, v, q_lens, num_computed, block_tables):
    """The step's scatter: new token i of sequence s goes to position num_computed[s] + i."""
    L, NB, bs, hkv, d, elt = _pool_geometry(pool_k)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    bt = _i32(block_tables)
    ql = _i32(q_lens)
    nc = _i32(num_computed)
    assert k.shape[0] == int(ql.sum()) and k.shape[1:] == (hkv, d) and k.dtype.itemsize == elt
    _load().oracle_reshape_and_cache(
        pool_k.view(np.uint8).ctypes.data_as(_u8p), pool_v.view(np.uint8).ctypes.data_as(_u8p),
        layer, NB, bs, hkv, d, elt,
        k.view(np.uint8).ctypes.data_as(_u8p), v.view(np.uint8).ctypes.data_as(_u8p),
        _ptr(ql, ctypes.c_int32), _ptr(nc, ctypes.c_int32), _ptr(bt, ctypes.c_int32),
        bt.shape[1], len(ql))


def gather(pool_k, pool_v, layer, block_table_row, n):
    """Read positions [0, n) of one sequence back out of the pools."""
    L, NB, bs, hkv, d, elt = _pool_geometry(pool_k)
    bt = _i32(block_table_row)
    k_rows = np.empty((n, hkv, d), dtype=pool_k.dtype)
    v_rows = np.empty((n, hkv, d), dtype=pool_k.dtype)
    if n:
        _load().oracle_gather(
            pool_k.view(np.uint8).ctypes.data_as(_u8p), pool_v.view(np.uint8).ctypes.data_as(_u8p),
            layer, NB, bs, hkv, d, elt, _ptr(bt, ctypes.c_int32), int(n),
            k_rows.view(np.uint8).ctypes.data_as(_u8p), v_rows.view(np.uint8).ctypes.data_as(_u8p))
    return k_rows, v_rows


def attention(q, kctx, vctx, knew, vnew, q_lens, num_computed, scale, row_sel=None):
    """Causal GQA attention of a packed step over contiguous per-sequence K/V (fp64).

    q [T, Hq, D]; kctx/vctx [sum c_s, Hkv, D]; knew/vnew [T, Hkv, D]; all
    float64. ``row_sel`` is an optional boolean [T, Hq] mask of rows to
    compute; unselected output rows are NaN.
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    kctx = np.ascontiguousarray(kctx, dtype=np.float64)
    vctx = np.ascontiguousarray(vctx, dtype=np.float64)
    knew = np.ascontiguousarray(knew, dtype=np.float64)
    vnew = np.ascontiguousarray(vnew, dtype=np.float64)
    ql = _i32(q_lens)
    nc = _i32(num_computed)
    T, hq, d = q.shape
    hkv = knew.shape[1]
    assert T == int(ql.sum()) and knew.shape == (T, hkv, d) and vnew.shape == knew.shape
    assert kctx.shape == (int(nc.sum()), hkv, d) and vctx.shape == kctx.shape
    assert hq % hkv == 0
    out = np.full((T, hq, d), np.nan, dtype=np.float64)
    sel = None
    if row_sel is not None:
        sel = np.ascontiguousarray(np.asarray(row_sel, dtype=bool).reshape(T, hq).astype(np.uint8))
    if T == 0:
        return out
    # zero-length arrays still need a valid pointer
    kc = kctx if kctx.size else np.zeros(1)
    vc = vctx if vctx.size else np.zeros(1)
    _load().oracle_attention(
        _ptr(q, ctypes.c_double), _ptr(kc, ctypes.c_double), _ptr(vc, ctypes.c_double),
        _ptr(knew, ctypes.c_double), _ptr(vnew, ctypes.c_double),
        _ptr(ql, ctypes.c_int32), _ptr(nc, ctypes.c_int32), len(ql),
        hq, hkv, d, float(scale),
        sel.ctypes.data_as(_u8p) if sel is not None else None,
        _ptr(out, ctypes.c_double))
    return out


def kv_bytes_per_block(num_layers: int, block_size: int, num_kv_heads: int,
                       head_dim: int, elt_bytes: int) -> int:
    """K+V bytes one block holds across all layers (tinyserve README,
    "Memory accounting": 2 x layers x block_size x kv heads x head_dim x dtype)."""
    return 2 * num_layers * block_size * num_kv_heads * head_dim * elt_bytes


def copy_blocks(src_k, src_v, dst_k, dst_v, src_ids, dst_ids):
    """Copy whole blocks (every layer, K and V) between pools of one layout."""
    L, NBs, bs, hkv, d, elt = _pool_geometry(src_k)
    L2, NBd, bs2, hkv2, d2, elt2 = _pool_geometry(dst_k)
    assert (L, bs, hkv, d, elt) == (L2, bs2, hkv2, d2, elt2)
    si, di = _i32(src_ids), _i32(dst_ids)
    assert si.shape == di.shape
    _load().oracle_copy_blocks(
        src_k.view(np.uint8).ctypes.data_as(_u8p), src_v.view(np.uint8).ctypes.data_as(_u8p),
        dst_k.view(np.uint8).ctypes.data_as(_u8p), dst_v.view(np.uint8).ctypes.data_as(_u8p),
        L, NBs, NBd, bs * hkv * d * elt, _ptr(si, ctypes.c_int32), _ptr(di, ctypes.c_int32), len(si))


def rope(x, positions, theta: float):
    """Rotary embedding of ``x`` [T, H, D] at per-row ``positions`` [T] (fp64).

    Pair (x[j], x[j + D/2]) turns by positions[t] * theta^(-2j/D) (the
    Qwen2 rotation; tinyserve README "Highlights").
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    assert x.ndim == 3 and x.shape[2] % 2 == 0
    T, H, D = x.shape
    pos = _i32(positions)
    assert pos.shape == (T,)
    out = np.empty_like(x)
    if T:
        _load().oracle_rope(_ptr(x, ctypes.c_double), T, H, D, _ptr(pos, ctypes.c_int32),
                            float(theta), _ptr(out, ctypes.c_double))
    return out


def spec_verify(target_probs, draft_probs, draft_tokens, draft_start, accept_u, sample_u):
    """Rejection-sampling verification of speculative rounds (see oracle.c).

    target_probs [total_drafts + S, V] fp32, draft_probs [total_drafts, V]
    fp32, draft_tokens [total_drafts], draft_start [S + 1] (exclusive prefix
    sum of the per-sequence draft counts), accept_u [total_drafts] and
    sample_u [S] fp64 uniforms. Returns (num_accepted [S], next_token [S]).
    """
    tp = np.ascontiguousarray(target_probs, dtype=np.float32)
    dp = np.ascontiguousarray(draft_probs, dtype=np.float32)
    dt = _i32(draft_tokens)
    ds = _i32(draft_start)
    au = np.ascontiguousarray(accept_u, dtype=np.float64)
    su = np.ascontiguousarray(sample_u, dtype=np.float64)
    S = len(ds) - 1
    V = tp.shape[1]
    assert tp.ndim == 2 and (dp.size == 0 or dp.shape[1] == V)
    assert len(su) == S
    na = np.empty(S, dtype=np.int32)
    nt = np.empty(S, dtype=np.int32)
    if S == 0:
        return na, nt
    # zero-length arrays still need a valid pointer
    dp = dp if dp.size else np.zeros((1, V), np.float32)
    dt = dt if dt.size else np.zeros(1, np.int32)
    au = au if au.size else np.zeros(1)
    _load().oracle_spec_verify(_ptr(tp, ctypes.c_float), _ptr(dp, ctypes.c_float), _ptr(dt, ctypes.c_int32),
                               _ptr(ds, ctypes.c_int32), _ptr(au, ctypes.c_double),
                               _ptr(su, ctypes.c_double), S, V, _ptr(na, ctypes.c_int32),
                               _ptr(nt, ctypes.c_int32))
    return na, nt
