"""GPU parity of the split prompt window (long prompts, few requests).

With fewer (request, head, beam group) units than it takes to fill the GPU,
the bf16 attention cuts each unit's prompt window into runs of 64-key tiles,
one workgroup each, and merges their partial softmax states with
log-sum-exp weights; the chain records go with the last run.  The oracle's
single softmax over the whole key set (and its split prefix/suffix form) is
the reference.

* gr_prefix_attn on long prompts: whole windows, sliding windows with a
  ragged last tile, two beam groups, prompt-only beams, the in-kernel and the
  pre-pass chain resolve; the run count the host picks is checked too.
* gr_decode_step end to end (attention, candidates, selection) on a long
  prompt with few requests.
* The same step with the split forced off is not available from the ABI; the
  split and unsplit paths meet in the generation tests (three requests, two
  runs) and the full-size workloads (no split).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from generative_recommendation_beam_amd import _lib as L
from generative_recommendation_beam_amd import harness as HN
from parity import announce, assert_close
from test_gpu_2_decode import compare, oracle_step

pytestmark = pytest.mark.gpu

CF = W.CONFIGS
LONG = {
    "long4k_beam50": W.reduced(CF["beam50_p600"], R=2, Lp=4096, H=4, level_sizes=(40, 50)),
    "long3k_window1000": W.reduced(CF["beam100_p600"], R=2, Lp=3000, window=1000, H=2,
                                   level_sizes=(90, 100, 100)),
    "long2k_two_groups": W.reduced(CF["beam100_p600"], R=1, Lp=2000, H=4, n_in=130, k=130,
                                   level_sizes=(100, 130, 130)),
    "long5k_prompt_only": W.reduced(CF["beam50_p600"], R=1, Lp=5000, H=8, n_in=64, k=64, depth=0,
                                    level_sizes=()),
    "long1k_d32": W.reduced(CF["beam50_p600"], R=3, Lp=1111, H=2, d=32, level_sizes=(30, 50)),
}


def expected_runs(cfg):
    """The host's choice, written out: units below 384 split into runs of at
    least 4 tiles, aiming at 384 workgroups."""
    waves = 1 if cfg.n_in <= 32 else (2 if cfg.n_in <= 64 else 4)
    per = waves * 32
    units = cfg.R * cfg.H * ((cfg.n_in + per - 1) // per)
    n_tiles = (cfg.Lw + 63) // 64
    if units >= 384:
        return 1
    ns = min(-(-384 // units), n_tiles // 4)
    if ns < 2:
        return 1
    tps = -(-n_tiles // ns)
    return -(-n_tiles // tps)


def oracle_arena(x):
    cfg = x.cfg
    ak, av, par = oracle.new_arena(cfg.R, max(cfg.capacity, 1), cfg.H, cfg.d)
    prev, base = None, 0
    for (pb, k, v) in x.levels:
        ak, av, par, prev = oracle.trie_append(ak, av, par, base, k, v, pb, prev)
        base += k.shape[1]
    return ak, av, par


@pytest.mark.parametrize("name", list(LONG))
def test_split_prefix_attn(name):
    cfg = LONG[name]
    runs = expected_runs(cfg)
    announce(f"gr_prefix_attn split window {name}: {runs} runs")
    assert runs > 1, "the case is meant to split"
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x)
    # the workspace holds the partial states: o [hd] plus (max, sum) per run, beam and head
    nb_pad = -(-cfg.n_in // 128) * 128 if cfg.n_in > 64 else (64 if cfg.n_in > 32 else 32)
    assert L.gr_attn_workspace_size(ds.shape, cfg.n_in) >= cfg.R * cfg.H * runs * nb_pad * (cfg.d + 2) * 4
    out = HN.prefix_attn(ds)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == 0
    ak, av, par = oracle_arena(x)
    ref = oracle.prefix_attn(x.prompt_k, x.prompt_v, x.q, par, ak, av, x.beam_node, window=cfg.window)
    assert_close(out.cpu().numpy(), ref, cfg.dtype, f"split {name}")


def test_split_prefix_attn_prepass_chains():
    """Arena above the in-kernel resolve limit: the chains come from the
    pre-pass and still go with the last run."""
    cfg = W.reduced(CF["beam50_p600"], R=2, Lp=2500, H=2, level_sizes=(50, 50))
    announce("gr_prefix_attn split window, pre-pass chains (5000-node arena)")
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x, capacity=5000)
    out = HN.prefix_attn(ds)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == 0
    ak, av, par = oracle_arena(x)
    ref = oracle.prefix_attn(x.prompt_k, x.prompt_v, x.q, par, ak, av, x.beam_node, window=cfg.window)
    assert_close(out.cpu().numpy(), ref, cfg.dtype, "split pre-pass chains")


@pytest.mark.parametrize("name", ["long4k_beam50", "long3k_window1000", "long2k_two_groups"])
def test_split_decode_step(name):
    cfg = LONG[name]
    announce(f"gr_decode_step split window {name}")
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x)
    buf = HN.decode_buffers(ds, debug_outputs=True)
    HN.decode_step(ds, buf)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == 0
    got = HN.results_to_host(buf)
    compare(cfg, got, oracle_step(x), list(range(cfg.R)), f"split {name}")
