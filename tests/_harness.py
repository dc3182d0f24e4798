"""Test-side helpers: host pools, oracle calls on a workloads.Step.

Only test code imports this. It calls the oracle for setup and for
expected values; nothing here calls the GPU library.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

# bit patterns of a quiet NaN in each storage dtype, used to poison every
# pool slot that no sequence owns
NAN_BITS = {torch.float32: (np.int32, 0x7FC00000),
            torch.float16: (np.int16, 0x7E00),
            torch.bfloat16: (np.int16, 0x7FC0)}


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a CPU tensor as a same-width integer numpy array."""
    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.view(torch.int16).numpy()


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of the rounded storage values to float64."""
    return t.to(torch.float64).numpy()


def pool_shape(step):
    return (step.num_layers, step.num_blocks, step.block_size, step.num_kv_heads, step.head_dim)


def host_pools(step, poison: bool = True):
    """K and V pools holding every sequence's cached context (positions
    0..c_s-1 written through its block table); all other slots NaN."""
    np_dtype, nan = NAN_BITS[step.dtype]
    fill = nan if poison else 0
    pk = np.full(pool_shape(step), fill, dtype=np_dtype)
    pv = np.full(pool_shape(step), fill, dtype=np_dtype)
    kc, vc = bits(step.k_ctx), bits(step.v_ctx)
    c0 = 0
    for s in range(step.num_seqs):
        c = int(step.num_computed[s])
        oracle.store_tokens(pk, pv, step.layer, step.block_tables[s], 0, kc[c0:c0 + c], vc[c0:c0 + c])
        c0 += c
    return pk, pv


def oracle_pools_after(step, pk, pv):
    """Pools after the step's scatter, by the oracle."""
    pk2, pv2 = pk.copy(), pv.copy()
    oracle.reshape_and_cache(pk2, pv2, step.layer, bits(step.k), bits(step.v),
                             step.q_lens, step.num_computed, step.block_tables)
    return pk2, pv2


def oracle_out(step, row_sel=None) -> np.ndarray:
    """fp64 attention output of the step by the oracle ([T, Hq, D])."""
    return oracle.attention(f64(step.q), f64(step.k_ctx), f64(step.v_ctx), f64(step.k),
                            f64(step.v), step.q_lens, step.num_computed, step.scale,
                            row_sel=row_sel)


def sample_rows(step, n_random: int, seed: int = 0) -> np.ndarray:
    """Boolean [T, Hq] selection: first and last token of every sequence in
    every head, plus ``n_random`` random (token, head) rows."""
    T, H = step.num_tokens, step.num_q_heads
    sel = np.zeros((T, H), dtype=bool)
    t0 = 0
    for n in step.q_lens.tolist():
        sel[t0, :] = True
        sel[t0 + n - 1, :] = True
        t0 += n
    rng = np.random.default_rng(1000 + seed)
    sel[rng.integers(0, T, n_random), rng.integers(0, H, n_random)] = True
    return sel


# Measured error margins of every output check in this process (tests
# append; conftest writes them out at the end of the session).
MARGINS = []


def record_margin(name, dtype, rows, max_abs, tol, max_rel, rtol):
    MARGINS.append({"case": name, "dtype": dtype, "rows": rows, "max_abs": max_abs, "tol": tol,
                    "abs_margin": tol / max_abs if max_abs > 0 else None, "max_row_rel_l2": max_rel,
                    "rtol": rtol, "rel_margin": rtol / max_rel if max_rel > 0 else None})
