#!/usr/bin/env python3
"""Throughput of the shared-prefix beam-decode step on one MI355X.

A step is one gr_decode_step over the whole batch of the headline workload
(256 requests, 600-token prompts, 8 heads x 64, beam 100, chains of 3 records,
256 codes per level, bf16): attention of every beam over its request's shared
prompt plus its own ancestor chain, codebook projection, log-softmax, prior
add and top-100 of 100 x 256 per request.  Inputs are seeded synthetic data
(workloads module), uploaded once and resident in HBM; independent copies
rotate between steps so that each step reads cold data (as many copies as
span 512 MiB of algorithmic bytes, twice the 256 MB last-level cache: two
for the headline, six for beam50_p600, eighteen for the 40 000-candidate
scalar workload).

Order of a run:
  1. the oracle on the host CPU, over the same workload (cpu_baseline), with
     one worker process per host core (before the GPU is touched);
  2. a plain device copy of 512 MiB each way, repeated for about 0.2 s and
     then timed (copy bandwidth, the practical HBM figure the step is also
     compared with; the GPU is at steady clocks afterwards);
  3. W warm-up steps, then K steps back to back on one stream between two
     events: `value` = 1 / step time, `ms_per_step`;
  4. K attention-only calls (GR_STEP_ATTENTION) back to back, then K
     selection-only calls (GR_STEP_SELECTION): stage times, and the attention
     kernel's roofline (its algorithmic bytes per launch over its mean launch
     time).
With --streams S > 1 the K steps also run spread over S streams (independent
batches in flight); that throughput is an extra field, never `value`.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

With a broadcast-scoring workload (--workload xf128d5l_u256_c40k) a step is
one gr_broadcast_score call: the user pass over 256 user tokens, 40 000
single-token candidates through 5 Pre-LN layers of width 128, their scores
and the top-2000; its roofline is the bf16 MFMA peak (FLOPs per call over
the call's time).

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
COLD_BYTES = 512 * 1024 * 1024    # input rotation span: twice the 256 MB last-level cache


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps first")
    ap.add_argument("--workload", default="beam100_p600")
    ap.add_argument("--sets", type=int, default=0,
                    help="independent input copies rotated between steps (default: enough to span 512 MiB of "
                         "algorithmic bytes, at least 2, per stream)")
    ap.add_argument("--streams", type=int, default=1,
                    help="also time the steps spread over this many HIP streams (extra field)")
    ap.add_argument("--attention", choices=["softmax", "linear"], default="softmax",
                    help="linear: linear-attention decoding over a shared prompt state (gr_linear_decode_step); "
                         "the state is computed once per input set before timing, as a prefill would")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="bound on the oracle's wall time (requests beyond it are not run)")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle worker processes (default: the host cores this process may use, at most 16)")
    ap.add_argument("--copy-seconds", type=float, default=0.2, help="device copy calibration time")
    ap.add_argument("--gemm-seconds", type=float, default=0.3, help="dense bf16 GEMM calibration time")
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
    # the attention launch: what it must read (prompt window, queries, chain
    # records with their parent ids, beam nodes); its output is handed on
    # through the workspace and counted as traffic, not as algorithmic bytes
    return dict(step_bytes=prompt + q + records + W + prior + outs,
                attn_kernel_bytes=prompt + q + records, attn_out_bytes=attn_out,
                prompt=prompt, q=q, records=records, n_chain_records=n_chain, flops=flops,
                prefix_flops=R * 4 * B * Lw * D)


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
    return dict(step_bytes=step, attn_kernel_bytes=state + a["q"] + a["records"], attn_out_bytes=attn_out,
                state=state, flops=flops, n_chain_records=a["n_chain_records"], prefix_flops=None)


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


def traffic_from_counters():
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


# The oracle runs in worker processes forked before the GPU is touched; a
# worker reads the workload from this module global (copy-on-write).
_ORACLE_INPUT = None


def host_cores(requested=0):
    """Worker processes for the oracle: the cores this process may run on
    (at most 16, the host share of one GPU), or the number asked for."""
    n = len(os.sched_getaffinity(0))
    return max(1, requested if requested > 0 else min(n, 16)), n


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:            # pragma: no cover
        pass


def _oracle_request(task):
    """The oracle's decode step for one request of the shared workload
    (its arena is built first, untimed).  Returns the step's seconds."""
    import oracle
    from oracle import linear as LA
    r, linear = task
    x = _ORACLE_INPUT
    cfg = x.cfg
    rr = [r]
    sl = lambda a: None if a is None else a[rr]
    ak, av, par = oracle.new_arena(1, max(cfg.capacity, 1), cfg.H, cfg.d)
    prev, base = None, 0
    for (pb, k, v) in x.levels:
        ak, av, par, prev = oracle.trie_append(ak, av, par, base, k[rr], v[rr], sl(pb), prev)
        base += k.shape[1]
    if linear:
        state = LA.prompt_state(x.prompt_k[rr], x.prompt_v[rr], cfg.window)
        t0 = time.perf_counter()
        o = LA.attend_linear_shared(x.prompt_k[rr], x.prompt_v[rr], x.q[rr], par, ak, av, sl(x.beam_node),
                                    cfg.window, state=state)
        c = oracle.candidate_scores(oracle.codebook_logits(o, x.W), sl(x.prior), True)
        oracle.select_topk(c[0], cfg.k)
    else:
        t0 = time.perf_counter()
        oracle.decode_step(x.prompt_k[rr], x.prompt_v[rr], x.q[rr], par, ak, av, sl(x.beam_node), x.W,
                           sl(x.prior), cfg.k, use_log_softmax=cfg.vocab > 1, window=cfg.window)
    return time.perf_counter() - t0


def _noop(_):
    return 0


def cpu_baseline(x, seconds, workers, linear=False):
    """The oracle (plain NumPy, fp64 accumulation) on the same workload, one
    request per task over `workers` forked processes with one BLAS thread
    each, in rounds of `workers` requests until every request is done or the
    wall time passes `seconds`.  Steps/s = requests done / R / wall time of
    the rounds (arena builds, and for linear attention the prompt state, are
    inside the wall time; see `decode_only_value` for the decode calls
    alone).  Must run before anything touches the GPU (the workers fork)."""
    import multiprocessing as mp
    global _ORACLE_INPUT
    _ORACLE_INPUT = x
    cfg = x.cfg
    done, times = 0, []
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_one_blas_thread) as pool:
        pool.map(_noop, range(workers))              # workers up (fork, imports) before the clock
        pool.map(_oracle_request, [(0, linear)] * min(workers, cfg.R))   # first-call costs, untimed
        t0 = time.perf_counter()
        while done < cfg.R:
            batch = [(r, linear) for r in range(done, min(cfg.R, done + workers))]
            times += pool.map(_oracle_request, batch, chunksize=1)
            done += len(batch)
            if time.perf_counter() - t0 > seconds:
                break
        wall = time.perf_counter() - t0
    _ORACLE_INPUT = None
    return {"value": (done / cfg.R) / wall, "unit": "steps/s", "cores": workers, "kind": "oracle",
            "sample": f"{done} of {cfg.R} requests ({done * cfg.n_in} beams), one per task over {workers} "
                      f"processes x 1 BLAS thread, {wall:.2f} s wall, scaled to whole steps",
            "beam_steps_per_s": done * cfg.n_in / wall,
            "decode_only_value": (done / cfg.R) / (sum(times) / workers),
            "cpu_model": cpu_model()}


def gen_accounting(g, steps):
    """Algorithmic bytes of one generation: per step, the prompt window once
    per request, the queries, every distinct record on a live chain once (k,
    v, parent id), the level's codebook, priors and outputs; per append, the
    written records, queries and node ids; the code tables (embeddings and
    projections read, tables written).  Distinct chain records are counted
    from the parents the run selected.  Where the records stay in the code
    tables (bf16, arenas of at most 4096 nodes) a chain node costs its parent
    id and table row index, each distinct table row (level, code) is read
    once for all requests (the queries of later steps too), and an append
    writes the node's row index instead of the query and the record."""
    import numpy as np
    sh = g.shape
    es = 2 if sh.dtype == 1 else 4
    R, D, V = sh.R, sh.H * sh.head_dim, g.vocab
    tab = sh.dtype == 1 and g.trie is not None and g.trie.capacity <= 4096
    Lw = sh.prompt_len if sh.window <= 0 else min(sh.window, sh.prompt_len)
    total, attn_prompt = 0, 0
    for lv, (n, k) in enumerate(g.sizes):
        q_bytes = R * n * D * es
        if tab and lv:
            q_bytes = np.unique(steps[lv - 1]["token"]).size * D * es
        total += R * Lw * D * 2 * es + q_bytes + V * D * es + R * k * 12 + (R * n * 4 if lv else 0)
        attn_prompt += R * Lw * D * 2 * es
        # records on the chains of step lv's n beams: levels lv, lv-1, .., 1
        if lv:
            live = np.tile(np.arange(n), (R, 1))
            for up in range(lv - 1, -1, -1):
                recs = sum(len(np.unique(live[r])) for r in range(R))
                if tab:
                    codes = np.unique(np.take_along_axis(steps[up]["token"], live, axis=1))
                    total += recs * 8 + codes.size * D * 2 * es
                else:
                    total += recs * (D * 2 * es + 4)
                live = np.take_along_axis(steps[up]["parent"], live, axis=1)
        if lv + 1 < len(g.sizes):
            total += R * k * (4 + 8 + 4 if tab else 3 * D * es + 4 + 8)
    total += (g.levels - 1) * (V * g.d_emb * es + 3 * D * g.d_emb * es + V * 3 * D * es)
    return total, attn_prompt


def bench_generate(args, cfg):
    import numpy as np
    import torch
    import workloads as W
    from generative_recommendation_beam_amd import harness as HN
    t0 = time.perf_counter()
    x = W.make_generate_inputs(cfg)
    print(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    cpu = None
    if not args.skip_cpu_baseline:
        workers, _ = host_cores(args.cpu_workers)
        print(f"[bench] the oracle on {workers} host cores", file=sys.stderr, flush=True)
        cpu = cpu_baseline_generate(x, args.cpu_seconds, workers)
    torch.cuda.set_device(0)
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
    copy_gbps = copy_bandwidth(args.copy_seconds)
    mfma_bandwidth(args.gemm_seconds)
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
        "copy_GBps": round(copy_gbps, 1),
        "frac_of_copy": round(gbps / copy_gbps, 4),
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def xf_flops(cfg):
    """FLOPs of one broadcast-scoring call, counted as the page counts a
    candidate's cost (2 per multiply-add): per layer and token 16 D^2 for
    the four projections and the FFN, plus 4 D per attended key (user
    tokens attend to L_u keys, candidates to L_u + their own), plus the
    score head (2 D per candidate).  Returns (total, candidate part)."""
    D, Lu, N, L = cfg.D, cfg.Lu, cfg.N, cfg.n_layers
    user = L * Lu * (16 * D * D + 4 * Lu * D)
    cand = L * N * (16 * D * D + 4 * (Lu + 1) * D) + 2 * D * N
    return cfg.R * (user + cand), cfg.R * cand


def bench_broadcast(args, cfg):
    import numpy as np
    import torch
    import workloads as W
    from generative_recommendation_beam_amd import harness as HN
    t0 = time.perf_counter()
    x = W.make_xf_inputs(cfg)
    print(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    cpu = None
    if not args.skip_cpu_baseline:
        cpu = cpu_baseline_broadcast(x, args.cpu_seconds)
    torch.cuda.set_device(0)
    n_sets = args.sets if args.sets > 0 else 2
    sets = [HN.upload_xf(x, all_scores=False)]
    for i in range(1, n_sets):
        xi = W.make_xf_inputs(cfg, seed=cfg.seed + 100 * i)
        sets.append(HN.upload_xf(xi, all_scores=False))
    torch.cuda.synchronize()
    print(f"[bench] {len(sets)} input set(s) resident on the GPU", file=sys.stderr, flush=True)
    copy_gbps = copy_bandwidth(args.copy_seconds)
    gemm_tflops = mfma_bandwidth(args.gemm_seconds)
    for i in range(args.warmup):
        HN.broadcast_score(sets[i % len(sets)])
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(args.steps):
        HN.broadcast_score(sets[i % len(sets)])
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    flops, cand_flops = xf_flops(cfg)
    tflops = flops / (ms * 1e-3) / 1e12
    calls = 1e3 / ms
    in_bytes = (x.user.size + x.cand.size + x.w_mat.size) * 2 + x.w_vec.size * 4
    out = {
        "metric": f"broadcast-scored candidates/s, {cfg.D}D-{cfg.n_layers}L, {cfg.N} candidates over "
                  f"{cfg.Lu} user tokens, top-{cfg.k} (1 GPU)",
        "value": round(calls * cfg.R * cfg.N, 0), "unit": "candidates/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) user and candidate tokens, N(0,1/fan_in) weights, N(0,0.02) biases, "
                "LayerNorm gains 1+N(0,0.1))",
        "config": {"workload": cfg.name, "requests": cfg.R, "candidates": cfg.N, "user_len": cfg.Lu,
                   "d_model": cfg.D, "heads": cfg.H, "layers": cfg.n_layers, "ffn": 2 * cfg.D, "k": cfg.k,
                   "input_sets": len(sets)},
        "calls_per_s": round(calls, 2),
        "flops_per_call": flops,
        "candidate_flops_per_call": cand_flops,
        "algorithmic_bytes_per_call": int(in_bytes + cfg.R * cfg.k * 8),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "gr_broadcast_score (user pass, candidate kernel, selection)"},
        "gemm_bf16_TFLOPs": round(gemm_tflops, 1),
        "frac_of_gemm": round(tflops / gemm_tflops, 4),
        "copy_GBps": round(copy_gbps, 1),
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def cpu_baseline_broadcast(x, seconds):
    """The oracle over chunks of 1000 candidates of request 0 (the user pass
    once, outside the wall time) until `seconds` have passed, with NumPy's
    BLAS on every host core; scaled to candidates/s."""
    from oracle import broadcast as BC
    cfg = x.cfg
    layers = [BC.LayerParams(**{k: lp[k] for k in (
        "w_qkv", "b_qkv", "w_o", "b_o", "w_1", "b_1", "w_2", "b_2",
        "ln1_g", "ln1_b", "ln2_g", "ln2_b")}) for lp in x.layers]
    P = BC.ModelParams(layers, x.lnf_g, x.lnf_b, x.w_score, x.b_score)
    cores, _ = host_cores(0)
    kv, _ = BC.user_forward(x.user[0], P, cfg.H)
    done, chunk = 0, 1000
    t0 = time.perf_counter()
    while done < cfg.N:
        n = min(chunk, cfg.N - done)
        BC.score_head(BC.candidate_forward(x.cand[0][done:done + n], kv, P, cfg.H), P)
        done += n
        if time.perf_counter() - t0 > seconds:
            break
    wall = time.perf_counter() - t0
    return {"value": round(done / wall, 1), "unit": "candidates/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {cfg.N} candidates of one request in chunks of {chunk}, user pass excluded, "
                      f"{wall:.2f} s wall, NumPy BLAS threads over {cores} cores",
            "cpu_model": cpu_model()}


def _oracle_generate(r):
    from oracle import generate as OG
    x, tables = _ORACLE_INPUT
    rr = [r]
    t0 = time.perf_counter()
    OG.generate(x.prompt_k[rr], x.prompt_v[rr], x.q0[rr], x.W, tables, x.cfg.k)
    return time.perf_counter() - t0


def cpu_baseline_generate(x, seconds, workers):
    """The oracle's whole-ID generation, one request per task over `workers`
    forked processes (one BLAS thread each), in rounds until every request
    is done or `seconds` of wall time have passed; the code tables are
    computed once beforehand (outside the wall time)."""
    import multiprocessing as mp
    from oracle import generate as OG
    global _ORACLE_INPUT
    cfg = x.cfg
    _one_blas_thread()
    tables = [OG.code_table(e, x.w_qkv, cfg.H, cfg.d, cfg.dtype) for e in x.emb]
    _ORACLE_INPUT = (x, tables)
    done = 0
    with mp.get_context("fork").Pool(workers, initializer=_one_blas_thread) as pool:
        pool.map(_noop, range(workers))
        t0 = time.perf_counter()
        while done < cfg.R:
            pool.map(_oracle_generate, list(range(done, min(cfg.R, done + workers))), chunksize=1)
            done += min(workers, cfg.R - done)
            if time.perf_counter() - t0 > seconds:
                break
        wall = time.perf_counter() - t0
    _ORACLE_INPUT = None
    return {"value": (done / cfg.R) / wall, "unit": "generations/s", "cores": workers, "kind": "oracle",
            "sample": f"{done} of {cfg.R} requests, one per task over {workers} processes x 1 BLAS thread, "
                      f"{wall:.2f} s wall (code tables excluded), scaled to whole batches",
            "cpu_model": cpu_model()}


def mfma_bandwidth(seconds):
    """A dense bf16 GEMM (torch.matmul, 8192^3, hipBLASLt): repeated for
    `seconds`, then 10 timed between events.  Returns TFLOP/s, the measured
    counterpart of the published dense bf16 MFMA peak.  Running right before
    the decode steps, it also brings the GPU to the clocks it holds under
    sustained load: from an idle GPU the first ~200 decode steps run up to
    30 % slower while the clocks rise."""
    import torch
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    c = torch.matmul(a, b)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(5):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    tf = 2 * n ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    return tf


def copy_bandwidth(seconds):
    """A plain device copy, 512 MiB each way (torch's copy kernel): repeated
    for `seconds`, then 20 copies timed between events.  Returns GB/s of
    bytes read plus bytes written.  Running first, it also brings the GPU to
    its steady clocks before the decode steps."""
    import torch
    n = 512 * 1024 * 1024 // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(20):
        b.copy_(a)
    c1.record()
    torch.cuda.synchronize()
    gbps = 2 * n * 4 * 20 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return gbps


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
    if args.workload in W.XF_CONFIGS:
        bench_broadcast(args, W.XF_CONFIGS[args.workload])
        return
    cfg = W.CONFIGS[args.workload]
    assert cfg.steps == 1, "the benchmark times single-step workloads"
    linear = args.attention == "linear"
    t0 = time.perf_counter()
    x = W.make_step_inputs(cfg)
    print(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    acc = algorithmic_linear(x) if linear else algorithmic(x)

    # 1. the oracle on the host cores, before the GPU is touched (its workers fork)
    cpu = None
    if not args.skip_cpu_baseline:
        workers, _ = host_cores(args.cpu_workers)
        print(f"[bench] the oracle on {workers} host cores", file=sys.stderr, flush=True)
        cpu = cpu_baseline(x, args.cpu_seconds, workers, linear)

    torch.cuda.set_device(0)
    n_streams = max(1, args.streams)
    # enough independent sets that the rotation spans more than twice the
    # 256 MB last-level cache: each step then reads data no earlier step left
    # there (at least two sets per stream)
    n_cold = -(-COLD_BYTES // max(1, acc["step_bytes"]))
    n_sets = args.sets if args.sets > 0 else max(2, n_cold) * n_streams
    assert n_sets % n_streams == 0, "every stream needs its own input sets"
    sets = [HN.upload_step(x)]
    for _ in range(n_sets - 1):
        sets.append(clone_step(sets[0]))
    bufs = [HN.decode_buffers(ds) for ds in sets]
    torch.cuda.synchronize()
    print(f"[bench] {len(sets)} input set(s) resident on the GPU", file=sys.stderr, flush=True)

    states = []
    prefill_ms = None
    if linear:
        HN.linear_state(sets[0])           # first launch (code object load) untimed
        torch.cuda.synchronize()
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record()
        for ds in sets:
            states.append(HN.linear_state(ds))
        p1.record()
        torch.cuda.synchronize()
        prefill_ms = p0.elapsed_time(p1) / len(sets)

    # 2. device copy bandwidth and a dense bf16 GEMM (measured counterparts of
    # the published HBM and MFMA peaks), right before the decode steps
    copy_gbps = copy_bandwidth(args.copy_seconds)
    gemm_tflops = mfma_bandwidth(args.gemm_seconds)

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

    # 3. W warm-up steps, then K whole steps back to back on one stream
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps

    # 4. each stage alone: K attention-only calls back to back between two
    # events (the input sets still alternate, so every launch streams a
    # prompt set the previous one evicted), then K selection-only calls
    # back to back (each re-scores its set's attention output, left in the
    # workspace by the attention-only calls).  Stage time = interval / K:
    # the kernels' own durations, without per-launch event gaps.
    def stage_ms(flag):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            step(i, flag)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    attn_avg_ms = stage_ms(L.GR_STEP_ATTENTION)
    sel_avg_ms = stage_ms(L.GR_STEP_SELECTION)

    # optional: the same K steps as independent batches spread over streams
    ms_multi = None
    if n_streams > 1:
        main_stream = torch.cuda.current_stream()
        streams = [main_stream] + [torch.cuda.Stream() for _ in range(n_streams - 1)]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(main_stream)
        for st in streams[1:]:
            st.wait_event(start)
        for i in range(args.steps):
            step(i, stream=streams[i % n_streams])
        for st in streams[1:]:
            e = torch.cuda.Event()
            e.record(st)
            main_stream.wait_event(e)
        stop.record(main_stream)
        torch.cuda.synchronize()
        ms_multi = start.elapsed_time(stop) / args.steps
    errs = [int(ds.dev_err.item()) for ds in sets]
    assert not any(errs), f"device error bits set: {errs}"

    steps_per_s = 1e3 / ms_step
    achieved = acc["attn_kernel_bytes"] / (attn_avg_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic_from_counters() if (cfg.name == W.HEADLINE and not linear) else None,
                "kernel": "linear_ring_bf16_kernel" if linear else "attn_bf16_kernel",
                "avg_launch_ms": round(attn_avg_ms, 5),
                "algorithmic_bytes_per_launch": acc["attn_kernel_bytes"],
                "output_bytes_per_launch": acc["attn_out_bytes"],
                "frac_of_copy": round(achieved / copy_gbps, 4)}
    step_gbps = acc["step_bytes"] / (ms_step * 1e-3) / 1e9
    out = {
        "metric": ("linear-attention " if linear else "") +
                  (f"beam decode steps/s & achieved HBM GB/s, beam={cfg.n_in}, prompt={cfg.Lp} tok" +
                   (f", window={cfg.Lw}" if cfg.Lw != cfg.Lp else "") + " (1 GPU)"),
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
                   "chain_records": cfg.depth, "codes_per_level": cfg.vocab, "input_sets": len(sets)},
        "beam_steps_per_s": round(steps_per_s * cfg.R * cfg.n_in, 0),
        "achieved_GBps": round(step_gbps, 1),
        "hbm_frac_of_peak": round(step_gbps / HBM_PEAK_GBPS, 4),
        "copy_GBps": round(copy_gbps, 1),
        "hbm_frac_of_copy": round(step_gbps / copy_gbps, 4),
        "gemm_bf16_TFLOPs": round(gemm_tflops, 1),
        "algorithmic_bytes_per_step": acc["step_bytes"],
        "flops_per_step": acc["flops"],
        "achieved_TFLOPs": round(acc["flops"] / (ms_step * 1e-3) / 1e12, 2),
        "stage_ms": {"attention": round(attn_avg_ms, 5), "scoring_selection": round(sel_avg_ms, 5)},
        "roofline": roofline,
    }
    if acc.get("prefix_flops"):
        # the prompt part of the attention is a dense contraction on bf16 MFMA
        tf = acc["prefix_flops"] / (attn_avg_ms * 1e-3) / 1e12
        out["prefix_mfma"] = {"flops_per_launch": acc["prefix_flops"], "achieved_TFLOPs": round(tf, 1),
                              "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                              "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                              "frac_of_gemm": round(tf / gemm_tflops, 4)}
    if ms_multi is not None:
        out["streams"] = n_streams
        out["ms_per_step_streams"] = round(ms_multi, 5)
        out["steps_per_s_streams"] = round(1e3 / ms_multi, 2)
    if linear:
        out["config"]["attention"] = "linear (elu+1 features, shared prompt state)"
        out["prefill_state_ms"] = round(prefill_ms, 5)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
