#!/usr/bin/env python3
"""Throughput of one packed paged-attention step on one MI355X.

A step is the whole hot path over one batch of synthetic input: scatter
this step's K/V into the block pool (ps_reshape_and_cache), then causal
GQA attention of every packed query token through the block tables
(ps_paged_attention: split-K decode/verify kernel, prefill-chunk kernel,
split-K merge). The host planner's metadata is built and uploaded once
before timing (inputs resident in HBM); its host cost is reported as
``host_plan_us``.

Default workload: the long-context speculative-verify step (32 sequences
at context 32768 with 5 causal query tokens each, plus one 2048-token
prefill chunk at position 30000; 12 Q / 2 KV heads, D 128, bf16), the
largest of the five named steps and the one that carries both the HBM
target (verify rows) and the MFMA target (the chunk). ``--config N``
picks another. Sub-lines time the prefill chunks alone (MFMA fraction)
and the decode / verify rows alone (HBM fraction) over the same pools.

The pool is replicated so that consecutive timed steps touch different
copies and the working set exceeds the 256 MB Infinity Cache plus L2:
every step reads its K/V from HBM, as a real step would.

Steps are timed replaying HIP graphs that captured them (the library's
calls are plain kernel launches on the caller's stream, so a step can be
captured); ``--eager`` times individual launches instead.

Prints one JSON line on stdout; details go to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA, TFLOP/s
FP32_PEAK_TFLOPS = 157.3       # MI355X dense fp32 matrix, TFLOP/s
LLC_BYTES = 256 << 20          # Infinity Cache
ROTATE_TARGET = 1 << 30        # bytes touched between reuses of one pool copy


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--shared-prefix", action="store_true",
                    help="plan with PS_PLAN_SHARED_PREFIX (attention over blocks shared by several "
                         "tables runs once; output bits then depend on the sharing)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured FETCH/WRITE bytes per attention launch (from rocprofv3 --pmc)")
    ap.add_argument("--eager", action="store_true",
                    help="time steps as individual launches instead of replaying them from a "
                         "captured HIP graph")
    ap.add_argument("--op", default="step",
                    choices=["step", "copy-blocks", "swap-blocks", "rope-cache", "spec-verify", "fixed-graph"],
                    help="step: the packed step (default); copy-blocks: copy-on-write block copies "
                         "in one device pool; swap-blocks: blocks out to a pinned host pool and back; "
                         "rope-cache: rotary embedding of the step's q and k fused with the KV scatter; "
                         "spec-verify: rejection sampling over the step's verify rows (use --config 5); "
                         "fixed-graph: one captured graph of a fixed-shape decode plan replayed over "
                         "steps of different lengths, against eager launches (use --config 2)")
    ap.add_argument("--proposer", default="draft", choices=["draft", "ngram"],
                    help="spec-verify: draft-model or n-gram proposer distributions")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB (3 times): the "
                         "reference kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_attention_packed_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def fill_context(P, step, pool, dev, stream):
    """Write every sequence's cached context into the pool with the
    library's own scatter (as the earlier steps that computed it would)."""
    import numpy as np
    import torch
    kc, vc = step.k_ctx, step.v_ctx
    offs = np.concatenate([[0], np.cumsum(step.num_computed.astype(np.int64))])
    groups = []
    if step.prefix_blocks:
        # the shared prefix is written once, by the first sequence; the
        # others only write their private part
        P_tok = step.prefix_blocks * 16
        groups.append(([0], [0], [int(step.num_computed[0])]))
        rest = list(range(1, step.num_seqs))
        groups.append((rest, [P_tok] * len(rest), [int(step.num_computed[s]) - P_tok for s in rest]))
    else:
        seqs = [s for s in range(step.num_seqs) if step.num_computed[s] > 0]
        groups.append((seqs, [0] * len(seqs), [int(step.num_computed[s]) for s in seqs]))
    for seqs, starts, lens in groups:
        sel = [(s, a, n) for s, a, n in zip(seqs, starts, lens) if n > 0]
        if not sel:
            continue
        rows = np.concatenate([np.arange(offs[s] + a, offs[s] + a + n) for s, a, n in sel])
        idx = torch.from_numpy(rows)
        kk = kc[idx].to(dev)
        vv = vc[idx].to(dev)
        ps = P.PackedStep([n for _, _, n in sel], [a for _, a, _ in sel],
                          step.block_tables[[s for s, _, _ in sel]], step.num_q_heads, pool, dev,
                          stream=stream)
        ps.reshape_and_cache(kk, vv, pool, stream)
        torch.cuda.synchronize()
        del ps, kk, vv


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(step, seconds):
    """The fp64 oracle (scatter + attention of the whole step) on host cores.

    A step whose attention takes the oracle longer than ``seconds`` is
    sampled: the scatter runs whole, attention runs on a uniform random
    sample of (token, head) rows sized to take about ``seconds``, and the
    rate is that of the whole step extrapolated from the sample's time per
    row."""
    import numpy as np
    import torch
    import oracle

    def bits(t):
        t = t.contiguous()
        return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).numpy()

    shape = (step.num_layers, step.num_blocks, 16, step.num_kv_heads, step.head_dim)
    pk = np.zeros(shape, dtype=bits(step.k).dtype)
    pv = np.zeros_like(pk)
    kcb, vcb = bits(step.k_ctx), bits(step.v_ctx)
    c0 = 0
    for s in range(step.num_seqs):  # cached context, as the GPU pool holds it
        c = int(step.num_computed[s])
        oracle.store_tokens(pk, pv, step.layer, step.block_tables[s], 0, kcb[c0:c0 + c], vcb[c0:c0 + c])
        c0 += c
    q, kc, vc, k, v = (t.to(torch.float64).numpy() for t in (step.q, step.k_ctx, step.v_ctx, step.k, step.v))
    kb, vb = bits(step.k), bits(step.v)
    T, H = step.num_tokens, step.num_q_heads
    rows = T * H
    rng = np.random.default_rng(12345)

    def attend(n_rows):
        sel = None
        if n_rows < rows:
            sel = np.zeros(rows, dtype=bool)
            sel[rng.choice(rows, size=n_rows, replace=False)] = True
            sel = sel.reshape(T, H)
        t0 = time.perf_counter()
        oracle.attention(q, kc, vc, k, v, step.q_lens, step.num_computed, step.scale, row_sel=sel)
        return time.perf_counter() - t0

    t0 = time.perf_counter()
    oracle.reshape_and_cache(pk, pv, step.layer, kb, vb, step.q_lens, step.num_computed, step.block_tables)
    t_scatter = time.perf_counter() - t0
    # calibrate on a small sample, then size the timed one
    n0 = max(1, min(rows, 4 * oracle.num_threads()))
    per_row = attend(n0) / n0
    n = int(min(rows, max(n0, seconds / max(per_row, 1e-9))))
    if n >= rows:
        reps, t_attn = 0, 0.0
        while True:
            t_attn += attend(rows)
            reps += 1
            if t_attn >= seconds or reps >= 10000:
                break
        t_step = t_scatter + t_attn / reps
        sample = f"{reps} full steps of {step.name} (scatter + attention, fp64) in {t_attn:.1f} s"
    else:
        t_attn = attend(n)
        t_step = t_scatter + t_attn * rows / n
        sample = (f"{step.name}: scatter of all {T} tokens ({t_scatter * 1e3:.1f} ms) + attention on a "
                  f"uniform sample of {n} of {rows} (token, head) rows in {t_attn:.1f} s, scaled to the "
                  f"whole step ({t_step:.1f} s)")
    return {"value": round(T / t_step, 3), "unit": "query tok/s",
            "cores": oracle.num_threads(), "kind": "oracle", "cpu": cpu_model(), "sample": sample}


def bench_blocks(args):
    """ps_copy_blocks throughput: copy-on-write inside the device pool, or
    swap out to / in from a pinned host pool, on the chosen workload's pool."""
    import numpy as np
    import torch
    import paged_kv_attention_packed_amd as P
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    step = workloads.config(args.config, values=False)
    shape = (step.num_layers, step.num_blocks, 16, step.num_kv_heads, step.head_dim)
    pk = torch.randn(shape, device=dev).to(step.dtype)
    pv = torch.randn(shape, device=dev).to(step.dtype)
    pool = P.make_pool(pk, pv)
    rng = np.random.default_rng(args.config)
    npairs = min(4096, step.num_blocks // 2)
    perm = rng.permutation(step.num_blocks).astype(np.int32)
    block_bytes = 16 * step.num_kv_heads * step.head_dim * pk.element_size() * step.num_layers
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e-3

    if args.op == "copy-blocks":
        src = torch.from_numpy(perm[:npairs]).to(dev)
        dst = torch.from_numpy(perm[npairs:2 * npairs]).to(dev)
        t = timed(lambda: P.ps_copy_blocks(pool, pool, src, dst, npairs, stream), args.steps)
        moved = 2 * 2 * npairs * block_bytes  # K and V, read and written
        result = {"metric": "copy-on-write block copy HBM GB/s, 1 MI355X", "value": round(moved / t / 1e9, 1),
                  "unit": "GB/s", "us_per_launch": round(t * 1e6, 2),
                  "roofline": {"bound": "hbm", "achieved": round(moved / t / 1e9, 1), "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": round(moved / t / 1e9 / HBM_PEAK_GBS, 4),
                               "traffic": None}}
    else:
        hshape = (step.num_layers, npairs, 16, step.num_kv_heads, step.head_dim)
        hk = torch.empty(hshape, dtype=step.dtype, pin_memory=True)
        hv = torch.empty(hshape, dtype=step.dtype, pin_memory=True)
        host = P.make_pool(hk, hv)
        blocks = torch.from_numpy(perm[:npairs]).to(dev)
        slots = torch.arange(npairs, dtype=torch.int32, device=dev)
        t_out = timed(lambda: P.ps_copy_blocks(pool, host, blocks, slots, npairs, stream), args.steps)
        t_in = timed(lambda: P.ps_copy_blocks(host, pool, slots, blocks, npairs, stream), args.steps)
        one_way = 2 * npairs * block_bytes
        # the runtime's own copy of the same bytes, contiguous, for reference
        flat_d = torch.empty(one_way, dtype=torch.uint8, device=dev)
        flat_h = torch.empty(one_way, dtype=torch.uint8, pin_memory=True)
        t_ref = timed(lambda: flat_h.copy_(flat_d, non_blocking=True), args.steps)
        result = {"metric": "swap out / in block copy GB/s over the host link, 1 MI355X",
                  "value": round(one_way / t_out / 1e9, 2), "unit": "GB/s (swap out)",
                  "swap_in_gbs": round(one_way / t_in / 1e9, 2),
                  "contiguous_d2h_memcpy_gbs": round(one_way / t_ref / 1e9, 2),
                  "us_per_launch": {"out": round(t_out * 1e6, 1), "in": round(t_in * 1e6, 1)}}
    result.update({"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
                   "dtype": step.dtype_name, "data": "synthetic",
                   "config": {"workload": step.name, "op": args.op, "pairs": npairs,
                              "block_bytes_all_layers_kv": 2 * block_bytes}})
    print(json.dumps(result), flush=True)


def bench_rope(args):
    """ps_rope_reshape_and_cache throughput on the chosen workload's new tokens:
    q rotated into q_out, k rotated into the pool, v copied into the pool.
    Input sets and slot placements rotate so that the working set between
    reuses exceeds the Infinity Cache."""
    import numpy as np
    import torch
    import paged_kv_attention_packed_amd as P
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    step = workloads.config(args.config, values=False)
    T, hq, hkv, d = step.num_tokens, step.num_q_heads, step.num_kv_heads, step.head_dim
    shape = (step.num_layers, step.num_blocks, 16, hkv, d)
    pk = torch.zeros(shape, dtype=step.dtype, device=dev)
    pv = torch.zeros(shape, dtype=step.dtype, device=dev)
    pool = P.make_pool(pk, pv, step.layer)
    ps = P.PackedStep(step.q_lens, step.num_computed, step.block_tables, hq, pool, dev, stream=stream)
    host = P.ps_plan_host_arrays(ps.plan, step.num_seqs, T)
    elt = pk.element_size()
    moved = T * (2 * hq * d * elt + 4 * hkv * d * elt + 8)   # q in/out, k and v in/out, position + slot
    nrot = min(1024, max(1, math.ceil(ROTATE_TARGET / moved)))
    rng = np.random.default_rng(args.config)
    g = torch.Generator(device=dev).manual_seed(args.config)
    sets = []
    for r in range(nrot):
        perm = rng.permutation(step.num_blocks).astype(np.int64)
        sl = host["slot_mapping"].astype(np.int64)
        slots = (perm[sl // 16] * 16 + sl % 16).astype(np.int32)
        sets.append((torch.randn((T, hq, d), generator=g, device=dev).to(step.dtype),
                     torch.empty((T, hq, d), dtype=step.dtype, device=dev),
                     torch.randn((T, hkv, d), generator=g, device=dev).to(step.dtype),
                     torch.randn((T, hkv, d), generator=g, device=dev).to(step.dtype),
                     torch.from_numpy(host["positions"]).to(dev), torch.from_numpy(slots).to(dev)))
    theta = 1e6

    def launch(i):
        q, qo, k, v, pos, sl = sets[i % nrot]
        P.ps_rope_reshape_and_cache(q, qo, k, v, pos, sl, T, hq, theta, pool, stream)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        launch(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / args.steps * 1e-3
    gbs = moved / t / 1e9
    result = {"metric": "rotary embedding + KV scatter HBM GB/s, 1 MI355X", "value": round(gbs, 1),
              "unit": "GB/s", "us_per_launch": round(t * 1e6, 2),
              "tokens_per_s": round(T / t, 1),
              "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
              "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
              "dtype": step.dtype_name, "data": "synthetic",
              "config": {"workload": step.name, "op": args.op, "tokens": T, "rope_theta": theta,
                         "bytes_per_launch": moved, "input_sets": nrot}}
    print(json.dumps(result), flush=True)


def bench_spec(args):
    """ps_spec_verify throughput on the verify rows of the chosen step: one
    round per sequence scheduled with 1 + k tokens, over the Qwen2.5
    vocabulary. Copies of the probability rows rotate so that the rows a
    call reads come from HBM."""
    import numpy as np
    import torch
    import oracle  # expected outputs only: checked once after timing
    import paged_kv_attention_packed_amd as P
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    r = workloads.spec_config(args.config, args.proposer)
    S, V, K = r.num_seqs, r.vocab, r.total_drafts
    if S == 0:
        print(f"config {args.config} has no verify rows", file=sys.stderr)
        sys.exit(2)
    ena, ent = oracle.spec_verify(r.target_probs, r.draft_probs, r.draft_tokens, r.draft_start,
                                  r.accept_u, r.sample_u)
    ks = np.diff(r.draft_start)
    rows_read = int(np.where(ena < ks, 2, 1).sum())          # rejection: p_j and q_j; else p_k
    moved = rows_read * V * 4
    per_copy = r.target_probs.nbytes + r.draft_probs.nbytes
    nrot = max(1, min(64, math.ceil(ROTATE_TARGET / moved)))
    tp0, dp0 = torch.from_numpy(r.target_probs).to(dev), torch.from_numpy(r.draft_probs).to(dev)
    copies = [(tp0, dp0)] + [(tp0.clone(), dp0.clone()) for _ in range(nrot - 1)]
    dt, ds = torch.from_numpy(r.draft_tokens).to(dev), torch.from_numpy(r.draft_start).to(dev)
    au, su = torch.from_numpy(r.accept_u).to(dev), torch.from_numpy(r.sample_u).to(dev)
    na = torch.empty(S, dtype=torch.int32, device=dev)
    nt = torch.empty(S, dtype=torch.int32, device=dev)
    wsb = P.ps_spec_verify_workspace_bytes(S, V)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def launch(i):
        tp, dp = copies[i % nrot]
        P.ps_spec_verify(tp, dp, dt, ds, au, su, S, K, V, na, nt, ws, wsb, stream)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        launch(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / args.steps * 1e-3
    ok = bool((na.cpu().numpy() == ena).all() and (nt.cpu().numpy() == ent).all())
    gbs = moved / t / 1e9
    result = {"metric": "speculative verify (rejection sampling) HBM GB/s, 1 MI355X", "value": round(gbs, 1),
              "unit": "GB/s", "us_per_call": round(t * 1e6, 2), "rounds_per_s": round(S / t, 1),
              "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
              "matches_oracle": ok,
              "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
              "dtype": "f32", "data": "synthetic",
              "config": {"workload": r.name, "op": args.op, "rounds": S, "drafts": K, "vocab": V,
                         "drafts_kept": int(ena.sum()), "rows_read": rows_read,
                         "bytes_per_call": moved, "input_copies": nrot,
                         "input_bytes_per_copy": per_copy}}
    print(json.dumps(result), flush=True)


def time_calls(fn, n, warmup, stream):
    """Average seconds per call of fn(i) over n calls on ``stream`` (HIP
    events recorded on the stream the kernels are launched on)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e-3


def sub_step(P, step, seqs, flags, pool0, dev, stream, q):
    """The step's sequences `seqs` planned on their own: (PackedStep, q rows, out)."""
    import numpy as np
    import torch
    qsl = np.concatenate([[0], np.cumsum(step.q_lens)])
    rows = torch.cat([torch.arange(int(qsl[s]), int(qsl[s + 1])) for s in seqs]).to(dev)
    q_sub = q.index_select(0, rows).contiguous()
    ps = P.PackedStep(step.q_lens[seqs], step.num_computed[seqs], step.block_tables[seqs],
                      step.num_q_heads, pool0, dev, flags, stream=stream)
    return ps, q_sub, torch.empty_like(q_sub)


def bench_fixed_graph(args):
    """NEXT-1 across steps: a fixed-shape decode plan (PS_PLAN_FIXED_SHAPE)
    serving a whole model step, every layer of it, from one captured HIP
    graph. Each step's plan is uploaded into the same metadata buffer, then
    either the graph is replayed once or the layers' ps_step calls are
    launched one by one; wall-clock time per step on the host, synchronised
    at the end of every step as a serving loop would, includes the launch
    overhead that the graph removes."""
    import numpy as np
    import torch
    import paged_kv_attention_packed_amd as P
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    base = workloads.config(args.config, values=False)
    hq, hkv, d, dt = base.num_q_heads, base.num_kv_heads, base.head_dim, base.dtype
    layers = 24   # Qwen2.5-0.5B's layer count
    S_max = base.num_seqs
    max_ctx = int((base.num_computed + base.q_lens).max())
    width = -(-max_ctx // 16)
    n_steps = 8
    steps = []
    for i in range(n_steps):   # same distribution as the named step, new lengths each step
        rng = np.random.default_rng(4000 + i)
        ctx = rng.integers(16, max_ctx, size=S_max, endpoint=True)
        steps.append(workloads.build_step(f"{base.name}-step{i}", 4000 + i, base.dtype_name, hq, hkv, d,
                                          base.num_blocks, [1] * S_max, (ctx - 1).tolist(), rng=rng,
                                          table_width=width, values=False))
    opts = P.plan_options(max_seqs=S_max, max_tokens=S_max, max_query_len=1)
    proto = P.ps_pool(0, 0, layers, base.num_blocks, 16, hkv, d, P._binding.dtype_code(dt), 0)
    shape = (layers, base.num_blocks, 16, hkv, d)
    pk = torch.randn(shape, device=dev).to(dt)
    pv = torch.randn(shape, device=dev).to(dt)
    pools = [P.make_pool(pk, pv, layer) for layer in range(layers)]
    fixed = [P.ps_plan_step(st.q_lens, st.num_computed, st.block_tables, hq, proto, P.PS_PLAN_FIXED_SHAPE, opts)
             for st in steps]
    meta_bytes, ws_bytes = P.ps_plan_sizes(fixed[0])
    meta = torch.empty(meta_bytes, dtype=torch.uint8, device=dev)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    q = torch.randn((layers, S_max, hq, d), device=dev).to(dt)
    k = torch.randn((layers, S_max, hkv, d), device=dev).to(dt)
    v = torch.randn((layers, S_max, hkv, d), device=dev).to(dt)
    out = torch.empty_like(q)

    def layers_once(plan, st, cs):
        a = P.ps_plan_device_arrays(plan)
        for layer in range(layers):
            P.ps_step(q[layer], k[layer], v[layer], a.slot_mapping, pools[layer], a.block_tables,
                      a.block_table_stride, a.query_start_loc, a.num_computed_tokens, a.context_lens, out[layer],
                      st.num_seqs, st.num_tokens, hq, base.scale, plan, ws, ws_bytes, cs)

    P.ps_plan_upload(fixed[0], meta, meta_bytes, stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layers_once(fixed[0], steps[0], torch.cuda.current_stream())
    reps = max(1, args.steps // n_steps)

    def serve(use_graph):
        t = 0.0
        for i, st in enumerate(steps):
            for r in range(reps + 2):
                t0 = time.perf_counter()
                P.ps_plan_upload(fixed[i], meta, meta_bytes, stream)
                if use_graph:
                    g.replay()
                else:
                    layers_once(fixed[i], st, stream)
                torch.cuda.synchronize()
                if r >= 2:
                    t += time.perf_counter() - t0
        return t / (n_steps * reps)

    serve(True)
    t_graph = serve(True)
    t_eager = serve(False)
    # GPU time of the graph alone, back to back
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    gpu_us = e0.elapsed_time(e1) / reps * 1e3
    plan_us = float(np.mean([P.ps_plan_get_info(p)["plan_us"] for p in fixed]))
    result = {"metric": "fixed-shape decode step, all layers: HIP-graph replay vs eager launches, wall clock, 1 MI355X",
              "value": round(t_graph * 1e6, 2), "unit": "us per step (graph replay, host-synchronised)",
              "higher_is_better": False, "eager_us": round(t_eager * 1e6, 2),
              "graph_vs_eager": round(t_graph / t_eager, 4), "graph_gpu_us_back_to_back": round(gpu_us, 2),
              "host_plan_us": round(plan_us, 1),
              "n_gpus": 1, "steps": reps * n_steps, "warmup": 2 * n_steps, "dtype": base.dtype_name,
              "data": "synthetic",
              "config": {"workload": f"{base.name}: {n_steps} steps of {S_max} decodes, context U[16, {max_ctx}], "
                                     f"{layers} layers", "op": args.op, "layers": layers, "max_seqs": S_max,
                         "decode_items": P.ps_plan_get_info(fixed[0])["decode_items"]}}
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    if args.op == "rope-cache":
        bench_rope(args)
        return
    if args.op == "spec-verify":
        bench_spec(args)
        return
    if args.op == "fixed-graph":
        bench_fixed_graph(args)
        return
    if args.op != "step":
        bench_blocks(args)
        return
    import numpy as np
    import torch
    import paged_kv_attention_packed_amd as P
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    step = workloads.config(args.config)
    flags = P.PS_PLAN_SHARED_PREFIX if args.shared_prefix else P.PS_PLAN_DEFAULT
    log(f"workload {step.summary()} flags {flags}")

    # ---- plan (host): the planner's own clock, and the Python call
    proto = P.ps_pool(0, 0, step.num_layers, step.num_blocks, 16, step.num_kv_heads,
                      step.head_dim, P._binding.dtype_code(step.dtype), step.layer)
    nplan = 20
    plan_us = []
    t0 = time.perf_counter()
    for _ in range(nplan):
        pl = P.ps_plan_step(step.q_lens, step.num_computed, step.block_tables, step.num_q_heads, proto, flags)
        plan_us.append(P.ps_plan_get_info(pl)["plan_us"])
        del pl
    host_call_us = (time.perf_counter() - t0) / nplan * 1e6

    # ---- pools: one filled copy, replicated
    shape = (step.num_layers, step.num_blocks, 16, step.num_kv_heads, step.head_dim)
    pk0 = torch.zeros(shape, dtype=step.dtype, device=dev)
    pv0 = torch.zeros(shape, dtype=step.dtype, device=dev)
    pool0 = P.make_pool(pk0, pv0, step.layer)
    fill_context(P, step, pool0, dev, stream)

    ps = P.PackedStep(step.q_lens, step.num_computed, step.block_tables, step.num_q_heads, pool0,
                      dev, flags, stream=stream)
    info = ps.info
    kinds = P.ps_plan_sequence_kernels(ps.plan, step.num_seqs)
    kv_bytes = info["kv_bytes_decode"] + info["kv_bytes_prefill"]
    touched = info["kv_bytes_unique"] + info["q_bytes"] + info["out_bytes"] + info["scatter_bytes"]
    pool_bytes = 2 * pk0.numel() * pk0.element_size()
    nrot = max(1, math.ceil(ROTATE_TARGET / max(touched, 1)))
    free = torch.cuda.mem_get_info()[0]
    nrot = int(max(1, min(nrot, (free * 0.6) // pool_bytes)))
    pools, tensors = [], []
    for i in range(nrot):
        if i == 0:
            k_, v_ = pk0, pv0
        else:
            k_, v_ = pk0.clone(), pv0.clone()
        tensors.append((k_, v_))
        pools.append(P.make_pool(k_, v_, step.layer))
    q = step.q.to(dev)
    k = step.k.to(dev)
    v = step.v.to(dev)
    outs = [torch.empty_like(q) for _ in range(min(nrot, 8))]
    torch.cuda.synchronize()
    log(f"pool copies {nrot} x {pool_bytes / 2**20:.1f} MiB; touched/step {touched / 1e6:.2f} MB; "
        f"plan {info}")

    def one_step(i):
        ps.run(q, k, v, pools[i % nrot], outs[i % len(outs)], step.scale, stream)

    # ---- warmup, then the timed steps
    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.eager:
        e0.record(stream)
        for i in range(args.steps):
            one_step(i)
        e1.record(stream)
        torch.cuda.synchronize()
    else:
        # the steps, one per pool copy, captured once into HIP graphs: a
        # block of nrot steps and a tail, replayed to give exactly K steps
        def capture(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cs = torch.cuda.current_stream()
                for i in range(n):
                    ps.run(q, k, v, pools[i % nrot], outs[i % len(outs)], step.scale, cs)
            return g
        block = min(nrot, args.steps)
        g_block = capture(block)
        tail = args.steps % block
        g_tail = capture(tail) if tail else None
        for _ in range(2):  # replay warmup
            g_block.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0.record(stream)
        for _ in range(args.steps // block):
            g_block.replay()
        if g_tail is not None:
            g_tail.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # ---- the calls alone, eager, same rotation
    ms_attn = 1e3 * time_calls(lambda i: ps.attention(q, pools[i % nrot], outs[i % len(outs)], step.scale, stream),
                               args.steps, args.warmup, stream)
    ms_scatter = 1e3 * time_calls(lambda i: ps.reshape_and_cache(k, v, pools[i % nrot], stream),
                                  args.steps, 0, stream)
    # when the planner fuses the scatter into the attention launch (every
    # non-prefix item on the decode kernel), ps_step is that one launch
    # (plus the split-K merge)
    fused = info["step_fused"] == 1
    ms_call = 1e3 * time_calls(lambda i: ps.step(q, k, v, pools[i % nrot], outs[i % len(outs)], step.scale, stream),
                               args.steps, 0, stream)

    # ---- each kind of sequence alone, planned on its own (the step's other
    # sequences left out), its attention call timed over the same pools:
    # the prefill chunks against the MFMA peak, the decode / verify rows
    # against HBM
    peak_mfma = MFMA_PEAK_TFLOPS if step.dtype_name != "f32" else FP32_PEAK_TFLOPS
    prefill_alone = decode_alone = None
    pre = [s for s in range(step.num_seqs) if kinds[s] == 1]
    dec = [s for s in range(step.num_seqs) if kinds[s] != 1]
    if pre and dec:
        ps_pre, q_pre, out_pre = sub_step(P, step, pre, flags, pool0, dev, stream, q)
        ms_pre = 1e3 * time_calls(lambda i: ps_pre.attention(q_pre, pools[i % nrot], out_pre, step.scale, stream),
                                  args.steps, args.warmup, stream)
        pflops = ps_pre.info["flops_prefill"]
        tf_pre = pflops / (ms_pre * 1e-3) / 1e12
        prefill_alone = {"call": "ps_paged_attention over the prefill sequences alone (prefill kernel + merge)",
                         "sequences": len(pre), "prefill_items": ps_pre.info["prefill_items"],
                         "merge_items": ps_pre.info["merge_items"], "us": round(ms_pre * 1e3, 3),
                         "gflop": round(pflops / 1e9, 3), "bound": "mfma", "achieved": round(tf_pre, 1),
                         "peak": peak_mfma, "unit": "TFLOP/s", "frac": round(tf_pre / peak_mfma, 4)}
        ps_dec, q_dec, out_dec = sub_step(P, step, dec, flags, pool0, dev, stream, q)
        ms_dec = 1e3 * time_calls(lambda i: ps_dec.attention(q_dec, pools[i % nrot], out_dec, step.scale, stream),
                                  args.steps, args.warmup, stream)
        di = ps_dec.info
        dbytes = di["kv_bytes_unique"] + di["q_bytes"] + di["out_bytes"] + di["table_bytes"]
        gbs_dec = dbytes / (ms_dec * 1e-3) / 1e9
        decode_alone = {"call": "ps_paged_attention over the decode / verify sequences alone (decode kernel + merge)",
                        "sequences": len(dec), "decode_items": di["decode_items"], "merge_items": di["merge_items"],
                        "us": round(ms_dec * 1e3, 3), "algorithmic_bytes": dbytes,
                        "kv_bytes_unique": di["kv_bytes_unique"], "bound": "hbm", "achieved": round(gbs_dec, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs_dec / HBM_PEAK_GBS, 4)}

    T = step.num_tokens
    tok_s = T / (ms_step * 1e-3)
    # algorithmic bytes of one attention call: each visible K/V row once per
    # (sequence, KV head) -- physical blocks once when tables share them --
    # plus q read, out write and block-table reads
    attn_bytes = info["kv_bytes_unique"] + info["q_bytes"] + info["out_bytes"] + info["table_bytes"]
    if fused:   # the dominant launch is the fused step: its bytes include the scatter's
        dom_bytes, ms_dom, dom_call = attn_bytes + info["scatter_bytes"], ms_call, "ps_step (scatter fused)"
    else:
        dom_bytes, ms_dom, dom_call = attn_bytes, ms_attn, "ps_paged_attention"
    achieved = dom_bytes / (ms_dom * 1e-3) / 1e9
    # measured HBM bytes per attention launch, valid only for the kernel
    # sources the counters were taken with
    traffic = None
    if os.path.exists(args.traffic):
        try:
            with open(args.traffic) as f:
                tr = json.load(f).get(step.name + ("+shared-prefix" if args.shared_prefix else ""))
            if tr and tr.get("kernel_source_digest") == kernel_source_digest():
                traffic = tr["bytes_per_launch"]
        except (OSError, ValueError, KeyError):
            traffic = None
    flops = info["flops_decode"] + info["flops_prefill"]
    nd, npf = info["decode_items"], info["prefill_items"]
    npx = info["prefix_items"]
    pre_note = f"{npf} prefill items, {npx} of them shared-prefix" if npx else f"{npf} prefill items"
    if info["mixed_launch"]:
        kernels = [f"ps_mixed_kernel x{nd + npf} ({nd} decode + {pre_note})"]
    else:
        kernels = ([f"ps_decode_kernel x{nd}"] if nd else []) + \
                  ([f"ps_prefill_kernel x{npf}"] if npf else [])
    if info["merge_items"]:
        kernels.append(f"ps_merge_kernel x{info['merge_items']}")
    # the launch's bound is the larger of its two ideal times: algorithmic
    # bytes at HBM peak, or its QK^T and PV flops at dense 16-bit MFMA peak
    # (fp32 rows run v_mfma_f32_16x16x4f32, priced at the fp32 matrix peak)
    t_hbm = dom_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (peak_mfma * 1e12)
    hbm_line = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    tflops_dom = flops / (ms_dom * 1e-3) / 1e12
    mfma_line = {"bound": "mfma", "achieved": round(tflops_dom, 1), "peak": peak_mfma,
                 "unit": "TFLOP/s", "frac": round(tflops_dom / peak_mfma, 4)}
    if t_mfma > t_hbm:
        roofline, other = dict(mfma_line), hbm_line
    else:
        roofline, other = dict(hbm_line), mfma_line
    roofline["traffic"] = traffic

    result = {
        "metric": "packed paged-attn query tok/s + KV-read HBM GB/s (% peak), 1 MI355X",
        "value": round(tok_s, 1),
        "unit": "query tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16", "bf16": "bf16"}[step.dtype_name],
        "data": "synthetic",
        "config": {"workload": step.name + (" +shared-prefix pass" if args.shared_prefix else ""),
                   "num_seqs": step.num_seqs, "num_tokens": T,
                   "num_q_heads": step.num_q_heads, "num_kv_heads": step.num_kv_heads,
                   "head_dim": step.head_dim, "block_size": 16, "num_blocks": step.num_blocks,
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "roofline_other_bound": other,
        "dominant": {"call": dom_call, "kernels": kernels,
                     "algorithmic_bytes_per_launch": dom_bytes, "flops_per_launch": flops,
                     "us_per_launch": round(ms_dom * 1e3, 3)},
        "prefill_alone": prefill_alone,
        "decode_alone": decode_alone,
        "attention_alone_us": round(ms_attn * 1e3, 3),
        # KV bytes over the attention call's time: unique (each physical
        # block once: what HBM can serve) and logical (once per sequence
        # that reads it; above HBM speed when blocks are shared and cached)
        "kv_read_gbs": round(info["kv_bytes_unique"] / (ms_attn * 1e-3) / 1e9, 1),
        "kv_read_logical_gbs": round(kv_bytes / (ms_attn * 1e-3) / 1e9, 1),
        "attention_tflops": round(flops / (ms_attn * 1e-3) / 1e12, 2),
        "scatter_us": round(ms_scatter * 1e3, 3),
        "host_plan_us": round(min(plan_us), 1),
        "host_plan_call_us": round(host_call_us, 1),
        "plan": {key: info[key] for key in ("decode_items", "prefill_items", "merge_items", "decode_split_keys",
                                            "prefill_split_keys", "decode_waves", "mixed_launch",
                                            "decode_stream_kv", "step_fused", "workspace_rows", "flags")},
        "pool_copies": nrot,
        "launch": "eager" if args.eager else "hip-graph replay",
        "gpu": torch.cuda.get_device_name(0),
        "torch": torch.__version__,
        "hip": torch.version.hip,
    }
    try:
        result["commit"] = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short", "HEAD"],
                                          capture_output=True, text=True, timeout=5).stdout.strip() or None
    except Exception:
        result["commit"] = None
    if args.copy_mb > 0:
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # the chip as the runtime reports it, and a measured device-to-device
    # copy: the HBM figures above against what a plain stream sustains
    props = torch.cuda.get_device_properties(0)
    result["device"] = {"arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count,
                        "memory_gib": round(props.total_memory / 2 ** 30, 1)}
    copy_gbs = measured_copy_gbs(dev)
    result["hbm_measured"] = {"copy_gbs": round(copy_gbs, 1),
                              "how": "1 GiB device-to-device copy with torch's copy kernel: bytes read + "
                                     "written over the time, best of 5"}
    for line in (result.get("roofline"), result.get("roofline_other_bound"), result.get("decode_alone")):
        if line and line.get("bound") == "hbm":
            line["frac_of_measured_copy"] = round(line["achieved"] / copy_gbs, 4)
    result["kernel_source_digest"] = kernel_source_digest()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline ...")
        result["cpu_baseline"] = cpu_baseline(step, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def measured_copy_gbs(dev, mib=1024, reps=5):
    """A device-to-device copy of `mib` MiB with torch's copy kernel, best of
    `reps`: bytes read plus bytes written over the time, GB/s."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(reps):
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del src, dst
    return 2 * (mib << 20) / (best * 1e-3) / 1e9


if __name__ == "__main__":
    main()
