"""Packed paged-attention step for AMD Instinct MI355X (gfx950).

The work is done by ``libps.so`` (hand-written HIP kernels plus a C++ host
planner behind the C ABI in ``include/ps.h``); this package is its Python
binding plus a small helper that runs one step with torch-allocated device
buffers.
"""
from ._binding import (  # noqa: F401
    PS_BF16, PS_F16, PS_F32, PS_PLAN_ALL_DECODE, PS_PLAN_ALL_PREFILL, PS_PLAN_DEFAULT,
    PS_PLAN_FIXED_SHAPE, PS_PLAN_SEPARATE_LAUNCHES, PS_PLAN_SHARED_PREFIX, Plan, PsError, make_pool,
    plan_options, ps_abi_version, ps_copy_blocks, ps_paged_attention, ps_plan_device_arrays,
    ps_plan_get_info, ps_plan_host_arrays, ps_plan_sequence_kernels, ps_plan_sizes, ps_plan_step,
    ps_plan_upload, ps_pool, ps_reshape_and_cache, ps_rope_reshape_and_cache, ps_spec_verify,
    ps_spec_verify_workspace_bytes, ps_step, ps_step_no_alloc, status_string)
from .step import PackedStep  # noqa: F401
