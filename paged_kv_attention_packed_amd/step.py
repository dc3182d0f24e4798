"""One packed step with torch-allocated device buffers (marshalling only).

Builds the plan on the host (libps's planner), uploads its metadata into a
torch uint8 buffer, allocates the split-K workspace, and forwards the two
step calls to the library on a given stream.
"""
from __future__ import annotations

import torch

from . import _binding as B


class PackedStep:
    def __init__(self, q_lens, num_computed_tokens, block_tables, num_q_heads: int,
                 pool: B.ps_pool, device, flags: int = B.PS_PLAN_DEFAULT, stream=None, options=None):
        self.num_seqs = len(q_lens)
        self.num_tokens = int(sum(int(x) for x in q_lens))
        self.num_q_heads = num_q_heads
        self.plan = B.ps_plan_step(q_lens, num_computed_tokens, block_tables, num_q_heads, pool, flags,
                                   options)
        self.meta_bytes, self.ws_bytes = B.ps_plan_sizes(self.plan)
        self.meta = torch.empty(self.meta_bytes, dtype=torch.uint8, device=device)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        B.ps_plan_upload(self.plan, self.meta, self.meta_bytes, stream)
        self.arrays = B.ps_plan_device_arrays(self.plan)
        self.info = B.ps_plan_get_info(self.plan)

    def reshape_and_cache(self, k, v, pool: B.ps_pool, stream=None):
        B.ps_reshape_and_cache(k, v, self.arrays.slot_mapping, self.num_tokens, pool, stream)

    def rope_reshape_and_cache(self, q, q_out, k, v, pool: B.ps_pool, rope_theta: float, stream=None):
        """Rotate q (into q_out) and k at the plan's positions, then cache k and v."""
        a = self.arrays
        B.ps_rope_reshape_and_cache(q, q_out, k, v, a.positions, a.slot_mapping, self.num_tokens,
                                    self.num_q_heads, rope_theta, pool, stream)

    def attention(self, q, pool: B.ps_pool, out, scale: float, stream=None):
        a = self.arrays
        B.ps_paged_attention(q, pool, a.block_tables, a.block_table_stride, a.query_start_loc,
                             a.num_computed_tokens, a.context_lens, out, self.num_seqs,
                             self.num_tokens, self.num_q_heads, scale, self.plan, self.ws,
                             self.ws_bytes, stream)

    def step(self, q, k, v, pool: B.ps_pool, out, scale: float, stream=None):
        """Scatter and attention through ps_step (fused when the plan allows)."""
        a = self.arrays
        B.ps_step(q, k, v, a.slot_mapping, pool, a.block_tables, a.block_table_stride, a.query_start_loc,
                  a.num_computed_tokens, a.context_lens, out, self.num_seqs, self.num_tokens,
                  self.num_q_heads, scale, self.plan, self.ws, self.ws_bytes, stream)

    def run(self, q, k, v, pool: B.ps_pool, out, scale: float, stream=None, rope_theta=None,
            separate=False):
        """The whole step: scatter this step's K/V, then attend (ps_step, or
        the two calls with ``separate``). With ``rope_theta`` q and k arrive
        unrotated: q is rotated in place and k on its way into the pool."""
        if rope_theta is not None:
            self.rope_reshape_and_cache(q, q, k, v, pool, rope_theta, stream)
            self.attention(q, pool, out, scale, stream)
        elif separate:
            self.reshape_and_cache(k, v, pool, stream)
            self.attention(q, pool, out, scale, stream)
        else:
            self.step(q, k, v, pool, out, scale, stream)
