"""ctypes binding of ``libps.so`` (the C ABI declared in ``include/ps.h``).

Argument marshalling only: every step of the packed attention path runs in
the library's HIP kernels and host planner. Function names match the C
entry points. torch tensors provide device memory and streams; their data
pointers are handed to the library as plain addresses.

The library is required: importing this module fails loudly when
``libps.so`` is missing (build it with ``paged_kv_attention_packed_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libps.so")

PS_OK = 0
PS_ERR_INVALID_ARGUMENT = 1
PS_ERR_UNSUPPORTED = 2
PS_ERR_WORKSPACE_TOO_SMALL = 3
PS_ERR_HIP = 4
PS_ERR_HOST_MEMORY = 5

PS_F32, PS_F16, PS_BF16 = 0, 1, 2
PS_PLAN_DEFAULT, PS_PLAN_ALL_DECODE, PS_PLAN_ALL_PREFILL = 0, 1, 2
PS_PLAN_SHARED_PREFIX, PS_PLAN_SEPARATE_LAUNCHES, PS_PLAN_FIXED_SHAPE = 4, 8, 16

EXPORTED = [
    "ps_plan_step", "ps_plan_sizes", "ps_plan_upload", "ps_plan_device_arrays",
    "ps_plan_host_arrays", "ps_plan_get_info", "ps_plan_sequence_kernels", "ps_plan_destroy",
    "ps_reshape_and_cache",
    "ps_paged_attention", "ps_step", "ps_step_no_alloc", "ps_copy_blocks", "ps_rope_reshape_and_cache", "ps_spec_verify",
    "ps_spec_verify_workspace_bytes", "ps_status_string", "ps_last_error_message", "ps_abi_version",
]


class ps_pool(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("num_layers", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("layer", ctypes.c_int32)]


class ps_step_arrays(ctypes.Structure):
    _fields_ = [("slot_mapping", ctypes.c_void_p), ("block_tables", ctypes.c_void_p),
                ("block_table_stride", ctypes.c_int32), ("query_start_loc", ctypes.c_void_p),
                ("num_computed_tokens", ctypes.c_void_p), ("context_lens", ctypes.c_void_p),
                ("positions", ctypes.c_void_p)]


class ps_plan_options(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "decode_split_keys", "prefill_split_keys", "decode_waves", "prefix_min_seqs",
        "prefix_min_keys", "prefix_slice_keys", "max_seqs", "max_tokens", "max_query_len",
        "max_decode_items", "max_merge_items", "max_workspace_rows", "decode_walk_rotation",
        "decode_stream_kv")] + [
        ("reserved", ctypes.c_int32 * 2)]


def plan_options(**kw) -> ps_plan_options:
    """ps_plan_options with the named fields set (the rest 0 = planner's choice)."""
    o = ps_plan_options()
    for k, v in kw.items():
        if k not in dict(ps_plan_options._fields_) or k == "reserved":
            raise TypeError(f"unknown plan option {k}")
        setattr(o, k, int(v))
    return o


class ps_plan_info(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_tokens", "num_q_heads", "num_kv_heads", "head_dim", "dtype",
        "decode_seqs", "prefill_seqs", "decode_items", "prefill_items", "merge_items",
        "decode_row_tiles")] + [(n, ctypes.c_int64) for n in (
        "kv_bytes_decode", "kv_bytes_prefill", "kv_bytes_unique", "q_bytes", "out_bytes",
        "scatter_bytes", "table_bytes")] + [("flops_decode", ctypes.c_double),
                                            ("flops_prefill", ctypes.c_double)] + [
        (n, ctypes.c_int32) for n in ("prefix_groups", "prefix_items", "step_fused", "flags",
                                      "decode_split_keys", "prefill_split_keys", "decode_waves",
                                      "mixed_launch", "active_decode_items", "active_merge_items",
                                      "decode_walk_rotation", "decode_stream_kv")] + [
        ("workspace_rows", ctypes.c_int64), ("plan_us", ctypes.c_double)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class PsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_attention_packed_amd.build`")

# torch first: its HIP runtime (a copy of libamdhip64 that its own libraries
# load by file name) is then the one libps.so binds to, by soname. Opened
# the other way round, the process would hold two HIP runtimes, and the
# library's calls would not see the device torch allocates on.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)
_i32p = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t

lib.ps_plan_step.restype = ctypes.c_int32
lib.ps_plan_step.argtypes = [_i32p, _i32p, ctypes.c_int32, _i32p, ctypes.c_int32, ctypes.c_int32,
                             ctypes.POINTER(ps_pool), ctypes.c_uint32, ctypes.POINTER(ps_plan_options),
                             ctypes.POINTER(_vp)]
lib.ps_plan_sizes.restype = ctypes.c_int32
lib.ps_plan_sizes.argtypes = [_vp, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]
lib.ps_plan_upload.restype = ctypes.c_int32
lib.ps_plan_upload.argtypes = [_vp, _vp, _sz, _vp]
lib.ps_plan_device_arrays.restype = ctypes.c_int32
lib.ps_plan_device_arrays.argtypes = [_vp, ctypes.POINTER(ps_step_arrays)]
lib.ps_plan_host_arrays.restype = ctypes.c_int32
lib.ps_plan_host_arrays.argtypes = [_vp, ctypes.POINTER(ps_step_arrays)]
lib.ps_plan_get_info.restype = ctypes.c_int32
lib.ps_plan_get_info.argtypes = [_vp, ctypes.POINTER(ps_plan_info)]
lib.ps_plan_sequence_kernels.restype = ctypes.c_int32
lib.ps_plan_sequence_kernels.argtypes = [_vp, _i32p, ctypes.c_int32]
lib.ps_plan_destroy.restype = None
lib.ps_plan_destroy.argtypes = [_vp]
lib.ps_reshape_and_cache.restype = ctypes.c_int32
lib.ps_reshape_and_cache.argtypes = [_vp, _vp, _vp, ctypes.c_int32, ctypes.POINTER(ps_pool), _vp]
lib.ps_paged_attention.restype = ctypes.c_int32
lib.ps_paged_attention.argtypes = [_vp, ctypes.POINTER(ps_pool), _vp, ctypes.c_int32, _vp, _vp, _vp,
                                   _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_float, _vp, _vp, _sz, _vp]
lib.ps_step.restype = ctypes.c_int32
lib.ps_step.argtypes = [_vp, _vp, _vp, _vp, ctypes.POINTER(ps_pool), _vp, ctypes.c_int32, _vp, _vp, _vp, _vp,
                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _vp, _vp, _sz, _vp]
lib.ps_step_no_alloc.restype = ctypes.c_int32
lib.ps_step_no_alloc.argtypes = [_vp, _vp, _vp, _vp, ctypes.POINTER(ps_pool), _vp, ctypes.c_int32, _vp, _vp, _vp,
                                 _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _vp, _vp]
lib.ps_copy_blocks.restype = ctypes.c_int32
lib.ps_copy_blocks.argtypes = [ctypes.POINTER(ps_pool), ctypes.POINTER(ps_pool), _vp, _vp, ctypes.c_int32, _vp]
lib.ps_rope_reshape_and_cache.restype = ctypes.c_int32
lib.ps_rope_reshape_and_cache.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_double, ctypes.POINTER(ps_pool), _vp]
lib.ps_spec_verify_workspace_bytes.restype = ctypes.c_size_t
lib.ps_spec_verify_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
lib.ps_spec_verify.restype = ctypes.c_int32
lib.ps_spec_verify.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                               _vp, _vp, _vp, _sz, _vp]
lib.ps_status_string.restype = ctypes.c_char_p
lib.ps_status_string.argtypes = [ctypes.c_int32]
lib.ps_last_error_message.restype = ctypes.c_char_p
lib.ps_last_error_message.argtypes = []
lib.ps_abi_version.restype = ctypes.c_int32
lib.ps_abi_version.argtypes = []


def status_string(status: int) -> str:
    return lib.ps_status_string(status).decode()


def _check(status: int):
    if status != PS_OK:
        raise PsError(status, lib.ps_last_error_message().decode())


def _ptr(x) -> Optional[int]:
    """Device or host address of a torch tensor / numpy array / int."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return x.ctypes.data


def _stream(stream) -> Optional[int]:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dtype_code(torch_dtype) -> int:
    import torch
    return {torch.float32: PS_F32, torch.float16: PS_F16, torch.bfloat16: PS_BF16}[torch_dtype]


def make_pool(k, v, layer: int = 0) -> ps_pool:
    """ps_pool over two [layers, blocks, 16, Hkv, D] tensors."""
    assert k.shape == v.shape and k.dim() == 5 and k.is_contiguous() and v.is_contiguous()
    L, NB, bs, hkv, d = k.shape
    return ps_pool(_ptr(k), _ptr(v), L, NB, bs, hkv, d, dtype_code(k.dtype), layer)


class Plan:
    """Owns a ps_plan*; destroyed with the object."""

    def __init__(self, handle: int):
        self.handle = handle
        self._lib = lib   # (module globals may be gone when the last plans die at exit)

    def __del__(self):
        if getattr(self, "handle", None) and getattr(self, "_lib", None) is not None:
            self._lib.ps_plan_destroy(self.handle)
            self.handle = None


def ps_plan_step(q_lens, num_computed_tokens, block_tables, num_q_heads: int, pool: ps_pool,
                 flags: int = PS_PLAN_DEFAULT, options: Optional[ps_plan_options] = None) -> Plan:
    ql = np.ascontiguousarray(q_lens, dtype=np.int32)
    nc = np.ascontiguousarray(num_computed_tokens, dtype=np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    if bt.ndim == 1:
        bt = bt.reshape(len(ql), -1) if len(ql) else bt.reshape(0, 1)
    stride = bt.shape[1] if bt.ndim == 2 and bt.shape[1] > 0 else 1
    out = _vp()
    _check(lib.ps_plan_step(ql.ctypes.data_as(_i32p), nc.ctypes.data_as(_i32p), len(ql),
                            bt.ctypes.data_as(_i32p), stride, num_q_heads,
                            ctypes.byref(pool), flags, ctypes.byref(options) if options is not None else None,
                            ctypes.byref(out)))
    return Plan(out.value)


def ps_plan_sizes(plan: Plan):
    m, w = _sz(), _sz()
    _check(lib.ps_plan_sizes(plan.handle, ctypes.byref(m), ctypes.byref(w)))
    return m.value, w.value


def ps_plan_upload(plan: Plan, metadata_dev, metadata_bytes: int, stream=None):
    _check(lib.ps_plan_upload(plan.handle, _ptr(metadata_dev), metadata_bytes, _stream(stream)))


def ps_plan_device_arrays(plan: Plan) -> ps_step_arrays:
    a = ps_step_arrays()
    _check(lib.ps_plan_device_arrays(plan.handle, ctypes.byref(a)))
    return a


def ps_plan_host_arrays(plan: Plan, num_seqs: int, num_tokens: int) -> dict:
    """Host copies of the plan's index arrays, as numpy views."""
    a = ps_step_arrays()
    _check(lib.ps_plan_host_arrays(plan.handle, ctypes.byref(a)))

    def view(addr, n):
        if n == 0:
            return np.zeros(0, dtype=np.int32)
        return np.ctypeslib.as_array(ctypes.cast(addr, _i32p), shape=(n,)).copy()

    return {"slot_mapping": view(a.slot_mapping, num_tokens),
            "block_tables": view(a.block_tables, num_seqs * a.block_table_stride).reshape(
                num_seqs, a.block_table_stride),
            "query_start_loc": view(a.query_start_loc, num_seqs + 1),
            "num_computed_tokens": view(a.num_computed_tokens, num_seqs),
            "context_lens": view(a.context_lens, num_seqs),
            "positions": view(a.positions, num_tokens)}


def ps_plan_get_info(plan: Plan) -> dict:
    info = ps_plan_info()
    _check(lib.ps_plan_get_info(plan.handle, ctypes.byref(info)))
    return info.as_dict()


def ps_plan_sequence_kernels(plan: Plan, num_seqs: int) -> np.ndarray:
    """Per sequence: 0 decode kernel, 1 prefill kernel, 2 decode after a shared prefix."""
    kinds = np.zeros(max(num_seqs, 1), dtype=np.int32)
    _check(lib.ps_plan_sequence_kernels(plan.handle, kinds.ctypes.data_as(_i32p), num_seqs))
    return kinds[:num_seqs]


def ps_reshape_and_cache(k, v, slot_mapping, num_tokens: int, pool: ps_pool, stream=None):
    _check(lib.ps_reshape_and_cache(_ptr(k), _ptr(v), _ptr(slot_mapping), num_tokens,
                                    ctypes.byref(pool), _stream(stream)))


def ps_paged_attention(q, pool: ps_pool, block_tables, block_table_stride: int, query_start_loc,
                       num_computed_tokens, context_lens, out, num_seqs: int, num_tokens: int,
                       num_q_heads: int, scale: float, plan: Plan, workspace, workspace_bytes: int,
                       stream=None):
    _check(lib.ps_paged_attention(_ptr(q), ctypes.byref(pool), _ptr(block_tables), block_table_stride,
                                  _ptr(query_start_loc), _ptr(num_computed_tokens), _ptr(context_lens),
                                  _ptr(out), num_seqs, num_tokens, num_q_heads, scale, plan.handle,
                                  _ptr(workspace), workspace_bytes, _stream(stream)))


def ps_step(q, k, v, slot_mapping, pool: ps_pool, block_tables, block_table_stride: int, query_start_loc,
            num_computed_tokens, context_lens, out, num_seqs: int, num_tokens: int, num_q_heads: int,
            scale: float, plan: Plan, workspace, workspace_bytes: int, stream=None):
    _check(lib.ps_step(_ptr(q), _ptr(k), _ptr(v), _ptr(slot_mapping), ctypes.byref(pool), _ptr(block_tables),
                       block_table_stride, _ptr(query_start_loc), _ptr(num_computed_tokens),
                       _ptr(context_lens), _ptr(out), num_seqs, num_tokens, num_q_heads, scale, plan.handle,
                       _ptr(workspace), workspace_bytes, _stream(stream)))


PS_STATIC_WORKSPACE_BYTES = 128 << 20


def ps_step_no_alloc(q, k, v, slot_mapping, pool: ps_pool, block_tables, block_table_stride: int,
                     query_start_loc, num_computed_tokens, context_lens, out, num_seqs: int, num_tokens: int,
                     num_q_heads: int, scale: float, plan: Plan, stream=None):
    _check(lib.ps_step_no_alloc(_ptr(q), _ptr(k), _ptr(v), _ptr(slot_mapping), ctypes.byref(pool),
                                _ptr(block_tables), block_table_stride, _ptr(query_start_loc),
                                _ptr(num_computed_tokens), _ptr(context_lens), _ptr(out), num_seqs, num_tokens,
                                num_q_heads, scale, plan.handle, _stream(stream)))


def ps_copy_blocks(src: ps_pool, dst: ps_pool, src_blocks, dst_blocks, num_pairs: int, stream=None):
    _check(lib.ps_copy_blocks(ctypes.byref(src), ctypes.byref(dst), _ptr(src_blocks), _ptr(dst_blocks),
                              num_pairs, _stream(stream)))


def ps_rope_reshape_and_cache(q, q_out, k, v, positions, slot_mapping, num_tokens: int,
                              num_q_heads: int, rope_theta: float, pool: ps_pool, stream=None):
    _check(lib.ps_rope_reshape_and_cache(_ptr(q), _ptr(q_out), _ptr(k), _ptr(v), _ptr(positions),
                                         _ptr(slot_mapping), num_tokens, num_q_heads, float(rope_theta),
                                         ctypes.byref(pool), _stream(stream)))


def ps_spec_verify_workspace_bytes(num_seqs: int, vocab_size: int) -> int:
    return lib.ps_spec_verify_workspace_bytes(num_seqs, vocab_size)


def ps_spec_verify(target_probs, draft_probs, draft_tokens, draft_start, accept_uniforms,
                   sample_uniforms, num_seqs: int, total_drafts: int, vocab_size: int, num_accepted,
                   next_token, workspace, workspace_bytes: int, stream=None):
    _check(lib.ps_spec_verify(_ptr(target_probs), _ptr(draft_probs), _ptr(draft_tokens), _ptr(draft_start),
                              _ptr(accept_uniforms), _ptr(sample_uniforms), num_seqs, total_drafts,
                              vocab_size, _ptr(num_accepted), _ptr(next_token), _ptr(workspace),
                              workspace_bytes, _stream(stream)))


def ps_abi_version() -> int:
    return lib.ps_abi_version()
