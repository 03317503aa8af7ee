"""The decode-step oracle over many requests in worker processes (test
infrastructure).

Workers are started with the "spawn" method, so they share nothing with the
test process (which holds the GPU): each draws the same seeded inputs from
workloads and runs the oracle on its requests.  Nothing here imports torch
or the HIP package.
"""
from __future__ import annotations

import multiprocessing as mp
import os

_X = None


def _init(name):
    global _X
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    import workloads as W
    _X = W.make_step_inputs(W.CONFIGS[name])


def oracle_requests(x, rs):
    """Oracle decode of requests rs of the workload inputs x (the trie built
    by the oracle's own append)."""
    import oracle
    cfg = x.cfg
    rs = list(rs)
    sl = lambda a: None if a is None else a[rs]
    levels = [(sl(pb), k[rs], v[rs]) for (pb, k, v) in x.levels]
    cap = max(sum(k.shape[1] for (_, k, _) in levels), 1)
    ak, av, par = oracle.new_arena(len(rs), cap, cfg.H, cfg.d)
    prev, base = None, 0
    for (pb, k, v) in levels:
        ak, av, par, prev = oracle.trie_append(ak, av, par, base, k, v, pb, prev)
        base += k.shape[1]
    return oracle.decode_step(x.prompt_k[rs], x.prompt_v[rs], x.q[rs], par, ak, av,
                              sl(x.beam_node), x.W, sl(x.prior), cfg.k,
                              use_log_softmax=cfg.vocab > 1, window=cfg.window)


def _one(r):
    return r, oracle_requests(_X, [r])


def oracle_many(name, rs, workers=None):
    """Per-request oracle results of workload `name` for requests rs, stacked
    in the order of rs (dict of arrays with a leading request axis)."""
    import numpy as np
    rs = list(rs)
    if workers is None:
        workers = max(1, min(16, len(os.sched_getaffinity(0)), len(rs)))
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers, initializer=_init, initargs=(name,)) as pool:
        out = dict(pool.imap_unordered(_one, rs, chunksize=1))
    keys = out[rs[0]].keys()
    return {k: np.concatenate([out[r][k] for r in rs], axis=0) for k in keys}
