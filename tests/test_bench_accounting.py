"""The benchmark's bookkeeping, on the CPU.

* Algorithmic bytes of the headline step: the prompt window (256 requests x
  600 rows x 512 dims x K and V x 2 bytes) and the queries exactly; the
  distinct chain records counted from the seeded trie equal a count made
  here with the oracle's own chain walk; the total is the 452 MB the
  workload's definition gives.
* `bench.py --gpus N` with N > 1 exits with status 2 and says why, before
  touching a GPU.
"""
import os
import subprocess
import sys

import numpy as np

import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_headline_algorithmic_bytes():
    cfg = W.CONFIGS["beam100_p600"]
    x = W.make_step_inputs(cfg)
    acc = bench.algorithmic(x)
    assert acc["prompt"] == 256 * 600 * 512 * 2 * 2
    assert acc["q"] == 256 * 100 * 512 * 2
    # distinct records on the live chains, walked with the oracle's chain()
    ak, av, par = oracle.new_arena(cfg.R, cfg.capacity, cfg.H, cfg.d)
    prev, base = None, 0
    for (pb, k, v) in x.levels:
        prev_nodes = prev
        nodes = np.tile(np.arange(base, base + k.shape[1], dtype=np.int32), (cfg.R, 1))
        for r in range(cfg.R):
            for j in range(k.shape[1]):
                par[r, base + j] = -1 if pb is None else prev_nodes[r, pb[r, j]]
        prev, base = nodes, base + k.shape[1]
    distinct = 0
    for r in range(cfg.R):
        seen = set()
        for b in range(cfg.n_in):
            seen.update(oracle.chain(par[r], int(x.beam_node[r, b]), 8))
        distinct += len(seen)
    assert acc["n_chain_records"] == distinct
    assert 200 < distinct / cfg.R < 220                  # about 210.7 per request
    assert abs(acc["step_bytes"] / 1e6 - 452.2) < 2.0


def test_bench_refuses_several_gpus():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_attention_launch_bytes_exclude_its_output():
    """The attention launch's algorithmic bytes are what it must read (prompt
    window, queries, distinct chain records with parent ids, beam nodes);
    the bf16 output it hands to the scoring stage is traffic, not
    algorithmic bytes."""
    cfg = W.CONFIGS["beam100_p600"]
    x = W.make_step_inputs(cfg)
    acc = bench.algorithmic(x)
    assert acc["attn_kernel_bytes"] == acc["prompt"] + acc["q"] + acc["records"]
    assert acc["attn_out_bytes"] == 256 * 100 * 512 * 2
    assert acc["records"] == acc["n_chain_records"] * (512 * 2 * 2 + 4) + 256 * 100 * 4


def test_cpu_baseline_uses_worker_processes():
    """The oracle baseline runs one request per task over several forked
    workers and reports how many it used."""
    cfg = W.reduced(W.CONFIGS["beam50_p600"], R=4, Lp=64, n_in=8, k=8, level_sizes=(8, 8))
    x = W.make_step_inputs(cfg)
    res = bench.cpu_baseline(x, 30.0, 2)
    assert res["cores"] == 2 and res["kind"] == "oracle"
    assert res["value"] > 0 and "4 of 4 requests" in res["sample"]
