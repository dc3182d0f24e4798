"""Full-matrix numpy formulation of the step's attention, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``). A second reading of
the same definition as ``oracle.c``: for each sequence build the whole
[n_s, ctx_s] score matrix per head, mask keys past each query's position
(PageServe "01 Scheduler loop / System architecture": query token i of a
sequence with c cached tokens sits at position c + i; tinyserve README "How
it works": stepped causal mask), softmax along keys, multiply by V.
"""
from __future__ import annotations

import numpy as np


def attention(q, kctx, vctx, knew, vnew, q_lens, num_computed, scale):
    q = np.asarray(q, dtype=np.float64)
    T, hq, d = q.shape
    hkv = knew.shape[1]
    g = hq // hkv
    out = np.empty_like(q)
    t0 = 0
    c0 = 0
    for n, c in zip(np.asarray(q_lens).tolist(), np.asarray(num_computed).tolist()):
        K = np.concatenate([kctx[c0:c0 + c], knew[t0:t0 + n]], axis=0).astype(np.float64)
        V = np.concatenate([vctx[c0:c0 + c], vnew[t0:t0 + n]], axis=0).astype(np.float64)
        ctx = c + n
        pos = c + np.arange(n)[:, None]                # [n, 1] query positions
        visible = np.arange(ctx)[None, :] <= pos       # [n, ctx]
        for h in range(hq):
            j = h // g
            Z = scale * (q[t0:t0 + n, h, :] @ K[:, j, :].T)
            Z = np.where(visible, Z, -np.inf)
            Z = Z - Z.max(axis=1, keepdims=True)
            W = np.exp(Z)
            W = W / W.sum(axis=1, keepdims=True)
            out[t0:t0 + n, h, :] = W @ V[:, j, :]
        t0 += n
        c0 += c
    return out
