#!/usr/bin/env python3
"""Throughput of the shared-prefix beam-decode step on one MI355X.

A step is one gr_decode_step over the whole batch of the headline workload
(256 requests, 600-token prompts, 8 heads x 64, beam 100, chains of 3 records,
256 codes per level, bf16): attention of every beam over its request's shared
prompt plus its own ancestor chain, codebook projection, log-softmax, prior
add and top-100 of 100 x 256 per request.  Inputs are seeded synthetic data
(workloads module), uploaded once and resident in HBM; independent copies
rotate between steps so that each step reads cold data (the working set of
one copy exceeds the 256 MB last-level cache).

The timed steps are independent batches.  By default they are spread over two
HIP streams (step i on stream i % 2, each stream with its own input copies,
outputs and workspace), as a serving process keeps two batches in flight:
one batch's scoring, a latency-bound pass with one workgroup per request,
overlaps the other's HBM-bound attention.  `value` is K steps over the time
of the whole timed region; the same K steps run back to back on one stream
give `ms_per_step_one_stream`, and a third pass with an event between the two
stages of every step gives the stage times and the attention roofline.

Printed: one JSON line with steps/s (value), beam-steps/s, algorithmic HBM
GB/s of the step, the attention kernel's roofline (algorithmic bytes per
launch / its event-timed average duration, against 8 TB/s), and the oracle
timed on a bounded sample of the same workload on the host CPU.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

With a whole-ID generation workload (--workload gen_beam100_p600) a step is
one complete generation instead: the q/k/v tables of the chosen codes
(one gr_code_table over the levels) and gr_generate (four decode steps with the chosen
codes' records appended in between, and the IDs traced back), captured once
in a HIP graph and replayed.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E, published peak
MFMA_BF16_PEAK_TFLOPS = 2500.0    # dense bf16 MFMA, published peak
COUNTERS = os.path.join(ROOT, "profiles", "attn_bf16_beam100_p600_counters.json")
ATTN_SOURCE = os.path.join(ROOT, "generative_recommendation_beam_amd", "csrc", "attn.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first (the GPU takes some tens of ms to reach steady clocks)")
    ap.add_argument("--workload", default="beam100_p600")
    ap.add_argument("--sets", type=int, default=0,
                    help="independent input copies rotated between steps (default: 2 per stream)")
    ap.add_argument("--streams", type=int, default=2,
                    help="HIP streams carrying independent batches concurrently (1 = one after another)")
    ap.add_argument("--attention", choices=["softmax", "linear"], default="softmax",
                    help="linear: linear-attention decoding over a shared prompt state (gr_linear_decode_step); "
                         "the state is computed once per input set before timing, as a prefill would")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time for the CPU sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration, copy bandwidth)")
    return ap.parse_args()


# ----------------------------------------------------------------- accounting
def chain_nodes(x):
    """Distinct arena nodes on the live beams' chains, per request (from the
    seeded parent draws: level l node j extends level l-1 node parent_beam)."""
    cfg = x.cfg
    if not x.levels:
        return [0] * cfg.R
    import numpy as np
    counts = np.zeros(cfg.R, np.int64)
    live = np.tile(np.arange(cfg.n_in), (cfg.R, 1))          # deepest-level indices
    for li in range(len(x.levels) - 1, -1, -1):
        for r in range(cfg.R):
            counts[r] += len(np.unique(live[r]))
        pb = x.levels[li][0]
        if pb is None:
            break
        live = np.take_along_axis(pb, live, axis=1)
    return counts.tolist()


def algorithmic(x):
    """Bytes the step must move and flops it must do (no re-reads, no padding,
    no debug outputs): the prompt window once per request, the queries, every
    distinct chain record once (k and v) with its parent id, the beam nodes, the
    codebook slice once, the prior, and the selected score/token/parent."""
    cfg = x.cfg
    es = 2 if cfg.dtype == "bf16" else 4
    D, R, B, Lw = cfg.D, cfg.R, cfg.n_in, cfg.Lw
    n_chain = sum(chain_nodes(x))
    prompt = R * Lw * D * 2 * es
    q = R * B * D * es
    records = n_chain * (D * 2 * es + 4) + (R * B * 4 if x.levels else 0)
    # attention output handed to the scoring stage: bf16 for the bf16
    # codebook path (it feeds the MFMA projection), fp32 otherwise
    attn_out = R * B * D * (2 if (cfg.dtype == "bf16" and cfg.vocab == 256) else 4)
    W = cfg.vocab * D * es
    prior = 0 if x.prior is None else R * B * 4
    outs = R * cfg.k * 12
    delta = cfg.depth
    flops = R * (4 * B * Lw * D + 4 * B * delta * D + 2 * B * D * cfg.vocab)
    return dict(step_bytes=prompt + q + records + W + prior + outs,
                attn_kernel_bytes=prompt + q + records + attn_out,
                prompt=prompt, q=q, records=records, n_chain_records=n_chain, flops=flops)


def algorithmic_linear(x):
    """Bytes of a linear-attention step: the shared state and normaliser of
    every (request, head) once (fp32), then as the softmax step without the
    prompt (queries, distinct chain records, codebook, priors, outputs)."""
    cfg = x.cfg
    a = algorithmic(x)
    state = cfg.R * cfg.H * (cfg.d * cfg.d + cfg.d) * 4
    step = a["step_bytes"] - a["prompt"] + state
    attn_out = cfg.R * cfg.n_in * cfg.D * (2 if (cfg.dtype == "bf16" and cfg.vocab == 256) else 4)
    flops = cfg.R * cfg.n_in * cfg.H * (2 * cfg.d * cfg.d + 4 * cfg.depth * cfg.d) + 2 * cfg.R * cfg.n_in * cfg.D * cfg.vocab
    return dict(step_bytes=step, attn_kernel_bytes=state + a["q"] + a["records"] + attn_out, state=state,
                flops=flops, n_chain_records=a["n_chain_records"])


# ------------------------------------------------------------------ devices
def clone_step(ds):
    """An independent device copy of one uploaded step (same values)."""
    import dataclasses
    from generative_recommendation_beam_amd import _lib as L
    c = lambda t: None if t is None else t.clone()
    ak, av, par = c(ds.arena_k), c(ds.arena_v), c(ds.parent)
    trie = None
    if ds.trie is not None:
        trie = L.Trie(k=ak.data_ptr(), v=av.data_ptr(), parent=par.data_ptr(),
                      capacity=ds.trie.capacity, max_depth=ds.trie.max_depth)
        trie._tensors = (ak, av, par)
    return dataclasses.replace(ds, prompt_k=c(ds.prompt_k), prompt_v=c(ds.prompt_v), q=c(ds.q), W=c(ds.W),
                               prior=c(ds.prior), arena_k=ak, arena_v=av, parent=par, trie=trie,
                               beam_node=c(ds.beam_node))


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_counters(attn_bytes_alg):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, or None when absent or taken on another version of the kernel."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha") != source_sha(ATTN_SOURCE):
        return None
    return int((c["fetch_kib"] * c["fetch_scale"] + c["write_kib"] * c["write_scale"]) * 1024)


def cpu_baseline(x, seconds, linear=False):
    """The oracle (plain NumPy, one BLAS thread) on the first requests of the
    same workload until `seconds` of work have accumulated (for linear
    attention the prompt state is computed outside the timed part, as on the
    GPU)."""
    import numpy as np
    import oracle
    from oracle import linear as LA
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:            # pragma: no cover
        threadpool_limits = None
    cfg = x.cfg
    done, spent, beams = 0, 0.0, 0
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        while done < cfg.R and (spent < seconds or done < 2):
            r = [done]
            sl = lambda a: None if a is None else a[r]
            ak, av, par = oracle.new_arena(1, max(cfg.capacity, 1), cfg.H, cfg.d)
            prev, base = None, 0
            for (pb, k, v) in x.levels:
                ak, av, par, prev = oracle.trie_append(ak, av, par, base, k[r], v[r], sl(pb), prev)
                base += k.shape[1]
            if linear:
                state = LA.prompt_state(x.prompt_k[r], x.prompt_v[r], cfg.window)
                t0 = time.perf_counter()
                o = LA.attend_linear_shared(x.prompt_k[r], x.prompt_v[r], x.q[r], par, ak, av, sl(x.beam_node),
                                            cfg.window, state=state)
                c = oracle.candidate_scores(oracle.codebook_logits(o, x.W), sl(x.prior), True)
                oracle.select_topk(c[0], cfg.k)
            else:
                t0 = time.perf_counter()
                oracle.decode_step(x.prompt_k[r], x.prompt_v[r], x.q[r], par, ak, av, sl(x.beam_node), x.W,
                                   sl(x.prior), cfg.k, use_log_softmax=cfg.vocab > 1, window=cfg.window)
            spent += time.perf_counter() - t0
            done += 1
            beams += cfg.n_in
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    steps_per_s = (done / cfg.R) / spent
    return {"value": steps_per_s, "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done} of {cfg.R} requests ({done * cfg.n_in} beams), "
                      f"{spent:.1f} s of oracle time, scaled to whole steps",
            "beam_steps_per_s": beams / spent}


def gen_accounting(g, steps):
    """Algorithmic bytes of one generation: per step, the prompt window once
    per request, the queries, every distinct record on a live chain once (k,
    v, parent id), the level's codebook, priors and outputs; per append, the
    written records, queries and node ids; the code tables (embeddings and
    projections read, tables written).  Distinct chain records are counted
    from the parents the run selected."""
    import numpy as np
    sh = g.shape
    es = 2 if sh.dtype == 1 else 4
    R, D, V = sh.R, sh.H * sh.head_dim, g.vocab
    Lw = sh.prompt_len if sh.window <= 0 else min(sh.window, sh.prompt_len)
    total, attn_prompt = 0, 0
    for lv, (n, k) in enumerate(g.sizes):
        total += R * Lw * D * 2 * es + R * n * D * es + V * D * es + R * k * 12 + (R * n * 4 if lv else 0)
        attn_prompt += R * Lw * D * 2 * es
        # records on the chains of step lv's n beams: levels lv, lv-1, .., 1
        if lv:
            live = np.tile(np.arange(n), (R, 1))
            for up in range(lv - 1, -1, -1):
                recs = sum(len(np.unique(live[r])) for r in range(R))
                total += recs * (D * 2 * es + 4)
                live = np.take_along_axis(steps[up]["parent"], live, axis=1)
        if lv + 1 < len(g.sizes):
            total += R * k * (3 * D * es + 4 + 8)
    total += (g.levels - 1) * (V * g.d_emb * es + 3 * D * g.d_emb * es + V * 3 * D * es)
    return total, attn_prompt


def bench_generate(args, cfg):
    import numpy as np
    import torch
    import workloads as W
    from generative_recommendation_beam_amd import harness as HN
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    x = W.make_generate_inputs(cfg)
    print(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    sets = [HN.upload_generate(x) for _ in range(args.sets if args.sets > 0 else 2)]
    torch.cuda.synchronize()
    print(f"[bench] {len(sets)} input set(s) resident on the GPU", file=sys.stderr, flush=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    def one(g):
        HN.code_tables(g, s)
        HN.generate(g, s)

    with torch.cuda.stream(s):
        for g in sets:
            one(g)
    torch.cuda.synchronize()
    graphs = []
    for g in sets:
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=s):
            one(g)
        graphs.append(gr)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        ev0.record(s)
        for i in range(args.steps):
            graphs[i % len(graphs)].replay()
        ev1.record(s)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    # the same generations launched eagerly (no graph), for the launch cost
    with torch.cuda.stream(s):
        ev0.record(s)
        for i in range(args.steps):
            one(sets[i % len(sets)])
        ev1.record(s)
    torch.cuda.synchronize()
    ms_eager = ev0.elapsed_time(ev1) / args.steps
    errs = [int(g.dev_err.item()) for g in sets]
    assert not any(errs), f"device error bits set: {errs}"
    host = HN.generate_to_host(sets[0])
    nbytes, prompt_bytes = gen_accounting(sets[0], host["steps"])
    gbps = nbytes / (ms * 1e-3) / 1e9
    gens = 1e3 / ms
    out = {
        "metric": "whole-ID generations/s, 4 levels, beam=100, prompt=600 tok (1 GPU)",
        "value": round(gens, 2), "unit": "generations/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) K/V, q0 and code embeddings, N(0,1/De) q/k/v projections, "
                "N(0,0.02) codebooks)",
        "config": {"workload": cfg.name, "requests": cfg.R, "prompt_len": cfg.Lp, "heads": cfg.H,
                   "head_dim": cfg.d, "beam_width": cfg.k, "levels": cfg.steps, "d_emb": x.d_emb,
                   "codes_per_level": cfg.vocab, "input_sets": len(sets), "hip_graph": True},
        "ids_per_s": round(gens * cfg.R * cfg.k, 0),
        "ms_per_generation_eager": round(ms_eager, 5),
        "algorithmic_bytes_per_generation": nbytes,
        "achieved_GBps": round(gbps, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "whole generation (all launches of one graph replay)",
                     "prompt_bytes_per_generation": prompt_bytes},
    }
    if not args.skip_cpu_baseline:
        print("[bench] timing the oracle on a sample of the same workload", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_generate(x, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline_generate(x, seconds):
    """The oracle's whole-ID generation (one BLAS thread) request by request
    until `seconds` of work have accumulated, scaled to whole batches."""
    from oracle import generate as OG
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:            # pragma: no cover
        threadpool_limits = None
    cfg = x.cfg
    done, spent = 0, 0.0
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        tables = [OG.code_table(e, x.w_qkv, cfg.H, cfg.d, cfg.dtype) for e in x.emb]
        while done < cfg.R and (spent < seconds or done < 2):
            r = [done]
            t0 = time.perf_counter()
            OG.generate(x.prompt_k[r], x.prompt_v[r], x.q0[r], x.W, tables, cfg.k)
            spent += time.perf_counter() - t0
            done += 1
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return {"value": (done / cfg.R) / spent, "unit": "generations/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done} of {cfg.R} requests, {spent:.1f} s of oracle time (code tables "
                      f"excluded), scaled to whole batches"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(requests are independent: see the sharding notes in the design document)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import workloads as W
    from generative_recommendation_beam_amd import _lib as L
    from generative_recommendation_beam_amd import harness as HN

    if args.workload in W.GEN_CONFIGS:
        bench_generate(args, W.GEN_CONFIGS[args.workload])
        return
    cfg = W.CONFIGS[args.workload]
    assert cfg.steps == 1, "the benchmark times single-step workloads"
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    x = W.make_step_inputs(cfg)
    print(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    acc = algorithmic(x)
    n_streams = max(1, args.streams)
    n_sets = args.sets if args.sets > 0 else 2 * n_streams
    assert n_sets % n_streams == 0, "every stream needs its own input sets"
    sets = [HN.upload_step(x)]
    for _ in range(n_sets - 1):
        sets.append(clone_step(sets[0]))
    bufs = [HN.decode_buffers(ds) for ds in sets]
    torch.cuda.synchronize()
    print(f"[bench] {len(sets)} input set(s) resident on the GPU", file=sys.stderr, flush=True)

    linear = args.attention == "linear"
    states = []
    prefill_ms = None
    if linear:
        acc = algorithmic_linear(x)
        HN.linear_state(sets[0])           # first launch (code object load) untimed
        torch.cuda.synchronize()
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record()
        for ds in sets:
            states.append(HN.linear_state(ds))
        p1.record()
        torch.cuda.synchronize()
        prefill_ms = p0.elapsed_time(p1) / len(sets)

    def step(i, flags_extra=0, stream=None):
        ds, buf = sets[i % len(sets)], bufs[i % len(bufs)]
        if linear:
            S, z = states[i % len(sets)]
            L.gr_linear_decode_step(ds.shape, S, z, ds.q, ds.n_beams, ds.trie, ds.beam_node, ds.W, ds.vocab,
                                    ds.prior, ds.k, ds.flags | flags_extra, buf.score, buf.token, buf.parent,
                                    None, None, buf.ws, buf.ws_bytes, ds.dev_err, stream)
            return
        L.gr_decode_step(ds.shape, ds.prompt_k, ds.prompt_v, ds.q, ds.n_beams, ds.trie, ds.beam_node, ds.W,
                         ds.vocab, ds.prior, ds.k, ds.flags | flags_extra, buf.score, buf.token, buf.parent,
                         None, None, buf.ws, buf.ws_bytes, ds.dev_err, stream)

    # Independent batches on several streams (a serving process keeping
    # several batches in flight, as concurrent workers sharing one GPU do):
    # step i runs on stream i % S with input set i % n_sets, so a stream
    # only ever touches its own sets, outputs and workspaces.  One batch's
    # scoring, a latency-bound pass with one workgroup per request, then
    # overlaps another batch's HBM-bound attention.
    main_stream = torch.cuda.current_stream()
    streams = [main_stream] + [torch.cuda.Stream() for _ in range(n_streams - 1)]

    def run_streams(k):
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(main_stream)
        for st in streams[1:]:
            st.wait_event(start)
        for i in range(k):
            step(i, stream=streams[i % n_streams])
        for st in streams[1:]:
            e = torch.cuda.Event()
            e.record(st)
            main_stream.wait_event(e)
        stop.record(main_stream)
        return start, stop

    for i in range(args.warmup):
        step(i)
    run_streams(args.warmup)
    torch.cuda.synchronize()

    # timed region 1: K whole steps, one call each
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_step_one_stream = ms_total / args.steps

    # timed region 1b: the same K steps spread over the streams
    ms_step = ms_step_one_stream
    if n_streams > 1:
        torch.cuda.synchronize()
        e0, e1 = run_streams(args.steps)
        torch.cuda.synchronize()
        ms_step = e0.elapsed_time(e1) / args.steps

    # timed region 2: the same K steps, each split into its two stages with
    # an event before, between and after them on the launch stream (same
    # kernels, same arguments, same order as in region 1; the input sets
    # still alternate, so every attention launch streams a prompt set the
    # previous one evicted).  Stage time = mean event-to-event interval.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(args.steps):
        step(i, L.GR_STEP_ATTENTION)
        ev[2 * i + 1].record()
        step(i, L.GR_STEP_SELECTION)
        ev[2 * i + 2].record()
    torch.cuda.synchronize()
    attn_avg_ms = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(args.steps)) / args.steps
    sel_avg_ms = sum(ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(args.steps)) / args.steps
    errs = [int(ds.dev_err.item()) for ds in sets]
    assert not any(errs), f"device error bits set: {errs}"

    copy_gbps = None
    if args.calibrate_copy:
        n = 512 * 1024 * 1024 // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(10):
            torch.mul(a, 1.0, out=b)
        c1.record()
        torch.cuda.synchronize()
        copy_gbps = 2 * n * 4 * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9

    steps_per_s = 1e3 / ms_step
    achieved = acc["attn_kernel_bytes"] / (attn_avg_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": None if linear else traffic_from_counters(acc["attn_kernel_bytes"]),
                "kernel": "linear_attn_kernel" if linear else "attn_bf16_kernel",
                "avg_launch_ms": round(attn_avg_ms, 5),
                "algorithmic_bytes_per_launch": acc["attn_kernel_bytes"]}
    step_gbps = acc["step_bytes"] / (ms_step * 1e-3) / 1e9
    out = {
        "metric": ("linear-attention " if linear else "") +
                  "beam decode steps/s & achieved HBM GB/s, beam=100, prompt=600 tok (1 GPU)",
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) K/V/Q, N(0,0.02) codebook, cumsum(-x^2) priors)",
        "config": {"workload": cfg.name, "requests": cfg.R, "prompt_len": cfg.Lp, "window": cfg.Lw,
                   "heads": cfg.H, "head_dim": cfg.d, "beams": cfg.n_in, "beam_width": cfg.k,
                   "chain_records": cfg.depth, "codes_per_level": cfg.vocab, "input_sets": len(sets),
                   "concurrent_batches": n_streams},
        "beam_steps_per_s": round(steps_per_s * cfg.R * cfg.n_in, 0),
        "achieved_GBps": round(step_gbps, 1),
        "hbm_frac_of_peak": round(step_gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": acc["step_bytes"],
        "flops_per_step": acc["flops"],
        "achieved_TFLOPs": round(acc["flops"] / (ms_step * 1e-3) / 1e12, 2),
        "streams": n_streams,
        "ms_per_step_one_stream": round(ms_step_one_stream, 5),
        "stage_ms": {"attention": round(attn_avg_ms, 5), "scoring_selection": round(sel_avg_ms, 5)},
        "roofline": roofline,
    }
    if copy_gbps is not None:
        out["copy_GBps"] = round(copy_gbps, 1)
    if linear:
        out["config"]["attention"] = "linear (elu+1 features, shared prompt state)"
        out["prefill_state_ms"] = round(prefill_ms, 5)
    if not args.skip_cpu_baseline:
        print("[bench] timing the oracle on a sample of the same workload", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds, linear)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
