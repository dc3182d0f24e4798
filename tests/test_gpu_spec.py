"""GPU: ps_spec_verify against the oracle's rejection sampler, exactly.

Acceptance decisions are fp64 products compared with fp32 probabilities
and draws are exact integer inverse-CDF lookups, so the number of kept
drafts and the next token must equal the oracle's for every sequence.

Covered: draft-model and n-gram proposers over the Qwen2.5 vocabulary and
small / ragged vocabularies (vector and scalar loads, several chunks and
a ragged last chunk), ragged draft counts including 0 and more than one
wave (k = 70), the greedy special case, malformed sequences, degenerate
uniforms, a misaligned row base, workspace reuse, the verify rows of the
long-context step, and the pages' statistical test of the sampler run
through the HIP path.
"""
import numpy as np
import pytest
import torch
from scipy import stats

import oracle
import paged_kv_attention_packed_amd as P
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _note(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run_gpu(r, target=None, ws=None):
    """Run the library on a SpecRound; returns (num_accepted, next_token) on the host."""
    S, V = r.num_seqs, r.vocab
    tp = _dev(r.target_probs) if target is None else target
    dp = _dev(r.draft_probs) if r.total_drafts else None
    dt = _dev(r.draft_tokens) if r.total_drafts else None
    au = _dev(r.accept_u) if r.total_drafts else None
    na = torch.full((S,), -7, dtype=torch.int32, device=DEV)
    nt = torch.full((S,), -7, dtype=torch.int32, device=DEV)
    need = P.ps_spec_verify_workspace_bytes(S, V)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
    P.ps_spec_verify(tp, dp, dt, _dev(r.draft_start), au, _dev(r.sample_u), S, r.total_drafts, V,
                     na, nt, ws, ws.numel(), torch.cuda.current_stream())
    torch.cuda.synchronize()
    return na.cpu().numpy(), nt.cpu().numpy()


def check(r, **kw):
    na, nt = run_gpu(r, **kw)
    ena, ent = oracle.spec_verify(r.target_probs, r.draft_probs, r.draft_tokens, r.draft_start,
                                  r.accept_u, r.sample_u)
    _note(f"{r.name}: S={r.num_seqs} V={r.vocab} drafts={r.total_drafts} "
          f"kept={int(ena[ena >= 0].sum())} mismatches={int((na != ena).sum() + (nt != ent).sum())}")
    np.testing.assert_array_equal(na, ena)
    np.testing.assert_array_equal(nt, ent)
    return na, nt


@pytest.mark.parametrize("proposer", ["draft", "ngram"])
@pytest.mark.parametrize("vocab", [7, 1000, 4097, 12288, workloads.QWEN25_VOCAB])
def test_random_rounds_match_oracle(vocab, proposer):
    rng = np.random.default_rng(vocab)
    ks = rng.integers(0, 9, 24)
    r = workloads.spec_round(f"rounds-{proposer}", vocab % 1000 + 17, ks, vocab, proposer=proposer)
    check(r)


def test_long_context_step_verify_rows():
    for proposer in ("draft", "ngram"):
        check(workloads.spec_config(5, proposer))


def test_more_drafts_than_a_wave():
    r = workloads.spec_round("k70", 3, [70, 0, 65, 1], 300, logit_scale=1.0, draft_noise=0.05)
    check(r)
    # one-hot rows and copied drafts: sequence 0 keeps 66 drafts (its first
    # rejection sits in the second group of 64), sequence 2 keeps all 65
    g = workloads.spec_round("k70-greedy", 4, [70, 0, 65, 1], 300, proposer="ngram", copy_rate=1.0)
    top = g.target_probs.argmax(axis=1)
    g.target_probs[:] = 0
    g.target_probs[np.arange(len(top)), top] = 1
    bad = (g.draft_tokens[66] + 1) % 300
    g.draft_tokens[66] = bad
    g.draft_probs[66] = 0
    g.draft_probs[66, bad] = 1
    na, nt = check(g)
    assert na[0] == 66 and na[2] == 65


def test_greedy_special_case():
    rng = np.random.default_rng(8)
    V, S = 5000, 64
    ks = rng.integers(0, 6, S)
    r = workloads.spec_round("greedy", 9, ks, V, proposer="ngram", copy_rate=0.8)
    # one-hot target rows at their top token: verification is greedy
    top = r.target_probs.argmax(axis=1)
    r.target_probs[:] = 0
    r.target_probs[np.arange(len(top)), top] = 1
    na, nt = check(r)
    for s in range(S):
        d0, k = int(r.draft_start[s]), int(ks[s])
        match = 0
        while match < k and r.draft_tokens[d0 + match] == top[d0 + s + match]:
            match += 1
        assert na[s] == match and nt[s] == top[d0 + s + match]


def test_malformed_sequences_and_degenerate_uniforms():
    r = workloads.spec_round("bad", 4, [2, 3, 1, 0, 2, 2], 2000)
    r.draft_tokens[r.draft_start[1] + 1] = 2000          # token out of range
    r.draft_tokens[r.draft_start[4]] = -3
    r.sample_u[:] = [0.0, 1.0, float("nan"), -1.0, 2.0, 1 - 2 ** -53]
    r.accept_u[0] = float("nan")
    na, nt = check(r)
    assert na[1] == nt[1] == -1 and na[4] == nt[4] == -1
    # draft_start out of order for one sequence
    r2 = workloads.spec_round("bad-starts", 5, [1, 2, 1], 600)
    r2.draft_start[:] = [0, 2, 1, 4]
    na, nt = check(r2)
    assert na[1] == nt[1] == -1


def test_misaligned_rows_take_the_scalar_path():
    r = workloads.spec_round("misaligned", 6, [3, 0, 2], 4096)
    buf = torch.empty(r.target_probs.size + 1, dtype=torch.float32, device=DEV)
    view = buf[1:].view(r.target_probs.shape)          # 4-byte offset from a 256-byte allocation
    view.copy_(torch.from_numpy(r.target_probs))
    na, nt = run_gpu(r, target=view)
    ena, ent = oracle.spec_verify(r.target_probs, r.draft_probs, r.draft_tokens, r.draft_start,
                                  r.accept_u, r.sample_u)
    np.testing.assert_array_equal(na, ena)
    np.testing.assert_array_equal(nt, ent)


def test_workspace_reuse_across_calls():
    ws = torch.empty(P.ps_spec_verify_workspace_bytes(40, 9000), dtype=torch.uint8, device=DEV)
    check(workloads.spec_round("reuse-a", 10, [4] * 40, 9000), ws=ws)
    check(workloads.spec_round("reuse-b", 11, [1, 0, 2], 500), ws=ws)


def test_statistical_law_through_the_gpu():
    # the pages' statistical test of the sampler, run on the HIP path:
    # 100k independent rounds over fixed rows; the first emitted token
    # follows p_0 and, after an accepted first draft, the second follows p_1
    rng = np.random.default_rng(12)
    V, k, N = 8, 3, 100_000
    P_ = np.stack([rng.dirichlet(np.full(V, 0.7)) for _ in range(k + 1)]).astype(np.float32)
    Q_ = np.stack([rng.dirichlet(np.full(V, 0.7)) for _ in range(k)]).astype(np.float32)
    cdf = np.cumsum(Q_.astype(np.float64), axis=1)
    d = np.stack([np.minimum(np.searchsorted(cdf[i], rng.random(N) * cdf[i, -1], side="right"), V - 1)
                  for i in range(k)], axis=1).astype(np.int32)
    r = workloads.SpecRound("statistical", V, np.tile(P_, (N, 1)), np.tile(Q_, (N, 1)), d.reshape(-1),
                            (np.arange(N + 1) * k).astype(np.int32), rng.random(N * k), rng.random(N))
    na, nt = check(r)
    law = P_.astype(np.float64) / P_.astype(np.float64).sum(axis=1, keepdims=True)
    x0 = np.where(na >= 1, d[:, 0], nt)
    p0 = stats.chisquare(np.bincount(x0, minlength=V), law[0] * N).pvalue
    one = na >= 1
    x1 = np.where(na[one] >= 2, d[one, 1], nt[one])
    p1 = stats.chisquare(np.bincount(x1, minlength=V), law[1] * one.sum()).pvalue
    _note(f"chi-square p-values: first token {p0:.3f}, second token {p1:.3f}")
    assert p0 > 1e-3 and p1 > 1e-3


@pytest.mark.parametrize("vocab", [300, workloads.QWEN25_VOCAB])
def test_residual_without_mass_draws_from_target(vocab):
    # target rows p_i = q_i / 2 (not normalised): a rejection happens about
    # half the time, and its residual max(p - q, 0) is zero everywhere, so
    # the draw comes from p_j by the whole-row path
    r = workloads.spec_round("no-residual", 21, [3, 2, 4, 1, 0, 2], vocab)
    for s in range(r.num_seqs):
        d0, k = int(r.draft_start[s]), int(r.draft_start[s + 1] - r.draft_start[s])
        for i in range(k):
            r.target_probs[d0 + s + i] = r.draft_probs[d0 + i] * np.float32(0.5)
    na, nt = check(r)
    ks = np.diff(r.draft_start)
    assert (na < ks).sum() >= 2       # some rejections took the fallback
