"""Seeded synthetic inputs for one packed paged-attention step.

This module only draws inputs: sequence lengths, block tables and N(0,1)
values. It holds none of the step's arithmetic (no slots, no positions, no
attention), so both the GPU path and the CPU oracle can consume what it
makes without sharing any of the method.

Recipe (shared by tests and the benchmark):
  * one ``numpy.random.default_rng(seed)`` (PCG64) per step;
  * draw order: lengths, then one permutation of the pool's block ids,
    then cached-context K and V, then the step's new K and V, then Q;
  * values are standard normal drawn in float32 and rounded
    (round-to-nearest-even, by torch's CPU cast) to the step's dtype;
  * integer lengths are uniform on inclusive ranges;
  * sequence s needs ceil((c_s + n_s) / 16) blocks; block tables take
    consecutive slices of the permutation, so physical placement is
    random (tinyserve README "How it works": a sequence never owns a
    contiguous cache region);
  * with a shared prefix, the first ``prefix_blocks`` ids of the
    permutation open every table and the prefix tokens have the same
    values in every sequence (PageServe "03 Paged KV cache": full blocks
    are shared between requests with a common prefix);
  * padding entries of a block table are -1;
  * packed token order is the sequence order given (the five named
    configurations list decodes before prefill chunks, as tinyserve's
    step orders decodes first, then chunked-prefill admissions).

The five named configurations are Qwen2.5-shaped steps (see ``CONFIGS``).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

BLOCK_SIZE = 16

_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Step:
    """One packed step's inputs (all host memory)."""
    name: str
    seed: int
    dtype: torch.dtype
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    num_layers: int
    layer: int
    block_size: int
    q_lens: np.ndarray          # int32 [S]   new tokens per sequence this step
    num_computed: np.ndarray    # int32 [S]   tokens whose K/V are already in the pool
    block_tables: np.ndarray    # int32 [S, max_blocks], -1 padded
    prefix_blocks: int          # blocks shared by every table (0: none)
    k_ctx: Optional[torch.Tensor]  # [sum c_s, Hkv, D] cached context K, sequence after sequence
    v_ctx: Optional[torch.Tensor]
    k: Optional[torch.Tensor]      # [T, Hkv, D] this step's K
    v: Optional[torch.Tensor]
    q: Optional[torch.Tensor]      # [T, Hq, D]
    scale: float

    @property
    def num_seqs(self) -> int:
        return int(len(self.q_lens))

    @property
    def num_tokens(self) -> int:
        return int(self.q_lens.sum())

    @property
    def dtype_name(self) -> str:
        return {v: k for k, v in _DTYPES.items()}[self.dtype]

    def summary(self) -> dict:
        return {"name": self.name, "dtype": self.dtype_name, "Hq": self.num_q_heads,
                "Hkv": self.num_kv_heads, "D": self.head_dim, "S": self.num_seqs,
                "T": self.num_tokens, "num_blocks": self.num_blocks,
                "num_layers": self.num_layers, "layer": self.layer}


def _normal(rng: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    t = torch.from_numpy(a)
    return t if dtype == torch.float32 else t.to(dtype)


def build_step(name: str, seed: int, dtype, num_q_heads: int, num_kv_heads: int,
               head_dim: int, num_blocks: int, q_lens: Sequence[int],
               num_computed: Sequence[int], *, rng: Optional[np.random.Generator] = None,
               prefix_tokens: int = 0, num_layers: int = 1, layer: int = 0,
               scale: Optional[float] = None, values: bool = True,
               table_width: Optional[int] = None,
               groups: Optional[Sequence[Tuple[Sequence[int], int]]] = None) -> Step:
    """Draw block tables and values for the given lengths.

    ``rng`` continues a generator that already drew the lengths; when None a
    fresh one is seeded with ``seed``. ``prefix_tokens`` (a multiple of 16)
    gives every sequence the same first blocks and the same values there.
    ``groups`` instead lists (members, prefix_tokens) pairs: the members of
    a pair share their first prefix_tokens / 16 blocks and the values there
    (disjoint member lists; sequences in no pair share nothing).
    """
    if groups is not None:
        return _build_grouped(name, seed, dtype, num_q_heads, num_kv_heads, head_dim, num_blocks,
                              q_lens, num_computed, groups, rng=rng, num_layers=num_layers,
                              layer=layer, scale=scale, values=values)
    if isinstance(dtype, str):
        dtype = _DTYPES[dtype]
    if rng is None:
        rng = np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    num_computed = np.asarray(num_computed, dtype=np.int32)
    assert q_lens.shape == num_computed.shape
    S = len(q_lens)
    ctx = (num_computed.astype(np.int64) + q_lens)
    assert prefix_tokens % BLOCK_SIZE == 0
    prefix_blocks = prefix_tokens // BLOCK_SIZE
    assert np.all(num_computed >= prefix_tokens), "prefix must lie in the cached context"

    # blocks each sequence needs, and the permutation they are sliced from
    nblk = [(int(c) + BLOCK_SIZE - 1) // BLOCK_SIZE for c in ctx]
    width = max(nblk) if S else 1
    if table_width is not None:
        assert table_width >= width
        width = table_width
    perm = rng.permutation(num_blocks).astype(np.int32)
    need = prefix_blocks + sum(b - prefix_blocks for b in nblk)
    assert need <= num_blocks, f"{name}: needs {need} blocks, pool has {num_blocks}"
    tables = np.full((S, max(width, 1)), -1, dtype=np.int32)
    off = prefix_blocks
    for s in range(S):
        tables[s, :prefix_blocks] = perm[:prefix_blocks]
        own = nblk[s] - prefix_blocks
        tables[s, prefix_blocks:nblk[s]] = perm[off:off + own]
        off += own

    k_ctx = v_ctx = k = v = q = None
    T = int(q_lens.sum())
    if values:
        if prefix_tokens:
            pk = _normal(rng, (prefix_tokens, num_kv_heads, head_dim), dtype)
            pv = _normal(rng, (prefix_tokens, num_kv_heads, head_dim), dtype)
            ks, vs = [], []
            for s in range(S):
                rest = int(num_computed[s]) - prefix_tokens
                ks.append(torch.cat([pk, _normal(rng, (rest, num_kv_heads, head_dim), dtype)]))
                vs.append(torch.cat([pv, _normal(rng, (rest, num_kv_heads, head_dim), dtype)]))
            k_ctx = torch.cat(ks) if ks else pk[:0]
            v_ctx = torch.cat(vs) if vs else pv[:0]
        else:
            nctx = int(num_computed.sum())
            k_ctx = _normal(rng, (nctx, num_kv_heads, head_dim), dtype)
            v_ctx = _normal(rng, (nctx, num_kv_heads, head_dim), dtype)
        k = _normal(rng, (T, num_kv_heads, head_dim), dtype)
        v = _normal(rng, (T, num_kv_heads, head_dim), dtype)
        q = _normal(rng, (T, num_q_heads, head_dim), dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return Step(name=name, seed=seed, dtype=dtype, num_q_heads=num_q_heads,
                num_kv_heads=num_kv_heads, head_dim=head_dim, num_blocks=num_blocks,
                num_layers=num_layers, layer=layer, block_size=BLOCK_SIZE,
                q_lens=q_lens, num_computed=num_computed, block_tables=tables,
                prefix_blocks=prefix_blocks, k_ctx=k_ctx, v_ctx=v_ctx, k=k, v=v, q=q,
                scale=float(scale))


def _build_grouped(name, seed, dtype, num_q_heads, num_kv_heads, head_dim, num_blocks, q_lens,
                   num_computed, groups, *, rng=None, num_layers=1, layer=0, scale=None,
                   values=True) -> Step:
    """build_step with several shared-prefix groups (see its ``groups``)."""
    if isinstance(dtype, str):
        dtype = _DTYPES[dtype]
    if rng is None:
        rng = np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    num_computed = np.asarray(num_computed, dtype=np.int32)
    S = len(q_lens)
    ctx = num_computed.astype(np.int64) + q_lens
    nblk = [(int(c) + BLOCK_SIZE - 1) // BLOCK_SIZE for c in ctx]
    group_of = [-1] * S
    for gi, (members, ptok) in enumerate(groups):
        assert ptok % BLOCK_SIZE == 0
        for m in members:
            assert group_of[m] < 0, "a sequence in two groups"
            assert num_computed[m] >= ptok, "prefix must lie in the cached context"
            group_of[m] = gi
    perm = rng.permutation(num_blocks).astype(np.int32)
    off = 0
    gblocks = []
    for members, ptok in groups:
        gblocks.append(perm[off:off + ptok // BLOCK_SIZE])
        off += ptok // BLOCK_SIZE
    tables = np.full((S, max(max(nblk) if S else 1, 1)), -1, dtype=np.int32)
    for s in range(S):
        pb = len(gblocks[group_of[s]]) if group_of[s] >= 0 else 0
        if pb:
            tables[s, :pb] = gblocks[group_of[s]]
        own = nblk[s] - pb
        tables[s, pb:nblk[s]] = perm[off:off + own]
        off += own
    assert off <= num_blocks, f"{name}: needs {off} blocks, pool has {num_blocks}"
    k_ctx = v_ctx = k = v = q = None
    T = int(q_lens.sum())
    if values:
        gk = [_normal(rng, (ptok, num_kv_heads, head_dim), dtype) for _, ptok in groups]
        gv = [_normal(rng, (ptok, num_kv_heads, head_dim), dtype) for _, ptok in groups]
        ks, vs = [], []
        for s in range(S):
            gi = group_of[s]
            ptok = groups[gi][1] if gi >= 0 else 0
            rest = int(num_computed[s]) - ptok
            pk = gk[gi] if gi >= 0 else _normal(rng, (0, num_kv_heads, head_dim), dtype)
            pv = gv[gi] if gi >= 0 else _normal(rng, (0, num_kv_heads, head_dim), dtype)
            ks.append(torch.cat([pk, _normal(rng, (rest, num_kv_heads, head_dim), dtype)]))
            vs.append(torch.cat([pv, _normal(rng, (rest, num_kv_heads, head_dim), dtype)]))
        k_ctx = torch.cat(ks)
        v_ctx = torch.cat(vs)
        k = _normal(rng, (T, num_kv_heads, head_dim), dtype)
        v = _normal(rng, (T, num_kv_heads, head_dim), dtype)
        q = _normal(rng, (T, num_q_heads, head_dim), dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return Step(name=name, seed=seed, dtype=dtype, num_q_heads=num_q_heads,
                num_kv_heads=num_kv_heads, head_dim=head_dim, num_blocks=num_blocks,
                num_layers=num_layers, layer=layer, block_size=BLOCK_SIZE,
                q_lens=q_lens, num_computed=num_computed, block_tables=tables,
                prefix_blocks=0, k_ctx=k_ctx, v_ctx=v_ctx, k=k, v=v, q=q, scale=float(scale))


def prefix_groups_step(seed: int, dtype="f16", num_q_heads: int = 14, num_kv_heads: int = 2,
                       head_dim: int = 64, verify: bool = False, with_prefill: bool = False,
                       values: bool = True) -> Step:
    """A decode step with two shared-prefix groups among other sequences.

    Group A: 10 sequences sharing 320 tokens (20 blocks); group B: 9
    sharing 512 tokens, some of them with nothing cached past the prefix.
    Four sequences share nothing, and one more shares only group A's first
    block (too little to join it). ``verify`` gives group B 2-5 query
    tokens per sequence; ``with_prefill`` adds a 40-token chunk. Sequences
    of the groups are interleaved with the others in the packed order.
    """
    rng = np.random.default_rng(seed)
    a_n = 1 + (rng.integers(0, 3, size=10) if verify else np.zeros(10, dtype=np.int64))
    a_c = 320 + rng.integers(0, 100, size=10, endpoint=True)
    b_n = rng.integers(2, 5, size=9, endpoint=True) if verify else np.ones(9, dtype=np.int64)
    b_c = 512 + np.where(np.arange(9) % 3 == 0, 0, rng.integers(1, 64, size=9, endpoint=True))
    l_n = np.ones(5, dtype=np.int64)
    l_c = rng.integers(10, 300, size=5, endpoint=True)
    l_c[4] = 400   # the outlier
    q_lens = list(a_n) + list(b_n) + list(l_n)
    num_computed = list(a_c) + list(b_c) + list(l_c)
    if with_prefill:
        q_lens.append(40)
        num_computed.append(30)
    S = len(q_lens)
    order = rng.permutation(S)                      # packed position of each sequence
    inv = np.empty(S, dtype=np.int64)
    inv[order] = np.arange(S)
    q_lens = [int(q_lens[i]) for i in order]
    num_computed = [int(num_computed[i]) for i in order]
    groups = [([int(inv[i]) for i in range(10)], 320), ([int(inv[i]) for i in range(10, 19)], 512)]
    st = build_step("prefix-groups", seed, dtype, num_q_heads, num_kv_heads, head_dim, 512,
                    q_lens, num_computed, rng=rng, values=values, groups=groups)
    # the outlier takes group A's first block, and its values
    o, a0 = int(inv[23]), groups[0][0][0]
    st.block_tables[o, 0] = st.block_tables[a0, 0]
    if values:
        offs = np.concatenate([[0], np.cumsum(st.num_computed.astype(np.int64))])
        for t in (st.k_ctx, st.v_ctx):
            t[offs[o]:offs[o] + BLOCK_SIZE] = t[offs[a0]:offs[a0] + BLOCK_SIZE]
    return st


# ---------------------------------------------------------------------------
# The five named configurations.

def _c1(values=True):
    # tiny fp32: 4 decodes at context 5, 17, 33, 50 and one 8-token prefill
    # chunk at num_computed 0; 2 Q heads / 1 KV head, D 64, pool of 64 blocks
    ctx = [5, 17, 33, 50]
    q_lens = [1, 1, 1, 1, 8]
    num_computed = [c - 1 for c in ctx] + [0]
    return build_step("C1-tiny-fp32", 1, "f32", 2, 1, 64, 64, q_lens, num_computed,
                      values=values)


def _c2(values=True):
    # Qwen2.5-0.5B-shaped decode step: 64 sequences, context U[16, 512]
    rng = np.random.default_rng(2)
    ctx = rng.integers(16, 512, size=64, endpoint=True)
    return build_step("C2-qwen0.5b-decode-fp16", 2, "f16", 14, 2, 64, 4096,
                      [1] * 64, (ctx - 1).tolist(), rng=rng, values=values)


def _c3(values=True):
    # Qwen2.5-1.5B-shaped mixed step: 128 decodes at context U[100, 2048]
    # plus 4 prefill chunks of 512 at num_computed U[0, 1024]
    rng = np.random.default_rng(3)
    dctx = rng.integers(100, 2048, size=128, endpoint=True)
    pc = rng.integers(0, 1024, size=4, endpoint=True)
    q_lens = [1] * 128 + [512] * 4
    num_computed = (dctx - 1).tolist() + pc.tolist()
    return build_step("C3-qwen1.5b-mixed-fp16", 3, "f16", 12, 2, 128, 32768,
                      q_lens, num_computed, rng=rng, values=values)


def _c4(values=True):
    # prefix sharing: 256 decodes whose first 1024 tokens (64 blocks) are the
    # same physical blocks, then a private suffix of U[64, 512] tokens; the
    # query is the last suffix token
    rng = np.random.default_rng(4)
    suffix = rng.integers(64, 512, size=256, endpoint=True)
    ctx = 1024 + suffix
    return build_step("C4-prefix-share-bf16", 4, "bf16", 12, 2, 128, 8192,
                      [1] * 256, (ctx - 1).tolist(), rng=rng, prefix_tokens=1024,
                      values=values)


def _c5(values=True):
    # long-context speculative verify: 32 sequences at context 32768 with
    # 1 + 4 causal query tokens each, plus one 2048-token prefill chunk at
    # position 30000
    rng = np.random.default_rng(5)
    q_lens = [5] * 32 + [2048]
    num_computed = [32768 - 5] * 32 + [30000]
    return build_step("C5-longctx-verify-bf16", 5, "bf16", 12, 2, 128, 80000,
                      q_lens, num_computed, rng=rng, values=values)


CONFIGS = {1: _c1, 2: _c2, 3: _c3, 4: _c4, 5: _c5}


def config(idx: int, values: bool = True) -> Step:
    """Named configuration ``idx`` in 1..5, seeded with ``idx``."""
    return CONFIGS[idx](values=values)


def random_step(seed: int, dtype="f16", num_q_heads=12, num_kv_heads=2, head_dim=128,
                num_seqs=6, max_q=40, max_ctx=300, num_blocks=None, num_layers=1,
                layer=0, values=True) -> Step:
    """A small ragged step with mixed decode / verify / prefill sequences."""
    rng = np.random.default_rng(seed)
    q_lens = rng.integers(1, max_q, size=num_seqs, endpoint=True)
    # a third of the sequences decode (1 token), a third verify (5 tokens)
    kind = rng.integers(0, 3, size=num_seqs, endpoint=False)
    q_lens = np.where(kind == 0, 1, np.where(kind == 1, np.minimum(5, max_q), q_lens))
    num_computed = rng.integers(0, max_ctx, size=num_seqs, endpoint=True)
    need = sum((int(c) + int(n) + 15) // 16 for c, n in zip(num_computed, q_lens))
    if num_blocks is None:
        num_blocks = 2 * need + 8
    return build_step(f"random-{seed}", seed, dtype, num_q_heads, num_kv_heads, head_dim,
                      num_blocks, q_lens.tolist(), num_computed.tolist(), rng=rng,
                      num_layers=num_layers, layer=layer, values=values)


# --------------------------------------------------------------------------
# Speculative verify rounds: the distributions a verify pass hands to the
# rejection sampler. Input synthesis only (target and draft distributions,
# draft tokens drawn by the proposer, uniforms); the acceptance test and
# the residual / bonus draws are not here.

QWEN25_VOCAB = 151936


@dataclasses.dataclass
class SpecRound:
    """One batch of verify rounds (all host memory)."""
    name: str
    vocab: int
    target_probs: np.ndarray   # float32 [total_drafts + S, V]: rows p_0..p_k of each sequence
    draft_probs: np.ndarray    # float32 [total_drafts, V]: rows q_0..q_{k-1}
    draft_tokens: np.ndarray   # int32 [total_drafts]
    draft_start: np.ndarray    # int32 [S + 1], exclusive prefix sum of the draft counts
    accept_u: np.ndarray       # float64 [total_drafts], uniforms in [0, 1)
    sample_u: np.ndarray       # float64 [S]

    @property
    def num_seqs(self) -> int:
        return len(self.draft_start) - 1

    @property
    def total_drafts(self) -> int:
        return int(self.draft_start[-1])


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def spec_round(name: str, seed: int, num_drafts: Sequence[int], vocab: int, logit_scale: float = 6.0,
               draft_noise: float = 1.5, proposer: str = "draft", copy_rate: float = 0.9) -> SpecRound:
    """Seeded verify rounds.

    Recipe: one PCG64 generator; per sequence, in order: k + 1 target
    logit rows z ~ N(0, logit_scale^2) (fp64), then the draft rows, then
    the drafts. Target rows are softmax(z) rounded to fp32 (peaked like a
    language model's next-token distribution: the top token typically
    holds tens of percent). Proposer "draft" (a small draft model):
    q_i = softmax(z_i + N(0, draft_noise^2)) and d_i is drawn from q_i.
    Proposer "ngram" (prompt lookup, deterministic): q_i is one-hot at
    d_i, which is the target's top token with probability copy_rate and
    a uniform random token otherwise. Uniforms come last: one per draft,
    then one per sequence.
    """
    rng = np.random.default_rng(seed)
    ks = [int(k) for k in num_drafts]
    S, total = len(ks), int(sum(ks))
    tp = np.empty((total + S, vocab), np.float32)
    dp = np.zeros((total, vocab), np.float32)
    dt = np.empty(total, np.int32)
    starts = np.zeros(S + 1, np.int32)
    starts[1:] = np.cumsum(ks)
    for s, k in enumerate(ks):
        z = rng.standard_normal((k + 1, vocab)) * logit_scale
        tp[starts[s] + s: starts[s] + s + k + 1] = _softmax_rows(z).astype(np.float32)
        for i in range(k):
            row = starts[s] + i
            if proposer == "draft":
                q = _softmax_rows(z[i] + rng.standard_normal(vocab) * draft_noise)
                dp[row] = q.astype(np.float32)
                c = np.cumsum(dp[row].astype(np.float64))
                dt[row] = min(int(np.searchsorted(c, rng.random() * c[-1], side="right")), vocab - 1)
            else:
                top = int(np.argmax(z[i]))
                dt[row] = top if rng.random() < copy_rate else int(rng.integers(0, vocab))
                dp[row, dt[row]] = 1.0
    au = rng.random(total)
    su = rng.random(S)
    return SpecRound(name, vocab, tp, dp, dt, starts, au, su)


def spec_config(idx: int, proposer: str = "draft") -> SpecRound:
    """The verify rows of named step ``idx``: every sequence scheduled with
    1 + k tokens (k >= 1) is one round of k drafts over the Qwen2.5
    vocabulary."""
    st = config(idx, values=False)
    ks = [int(n) - 1 for n in st.q_lens if 2 <= int(n) <= 9]
    return spec_round(f"{st.name}-verify-{proposer}", 1000 + idx, ks, QWEN25_VOCAB, proposer=proposer)
