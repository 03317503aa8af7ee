"""GPU parity of linear-attention decoding (gr_linear_state, gr_linear_attn,
gr_linear_decode_step) against the oracle (oracle/linear.py).

* The shared prompt state S_p and normaliser z_p of every (request, head)
  against the oracle's exact sums, with and without a window (bar on the
  whole tensor).
* gr_linear_attn against the oracle's shared-state form, for bf16 and fp32
  workloads, chains of 0..8 records, a one-token prompt and window.
* gr_linear_decode_step end to end on reduced versions of every workload
  family and the widest model (D = 4096), compared in full like the softmax
  step: attention outputs, all candidate scores, selected scores (bar), the
  index rule and the exact self-consistency of the selection; and the
  headline shape at full size on sampled requests.
* A chain longer than max_depth raises GR_DEVERR_DEPTH, corrupt parents
  GR_DEVERR_PARENT_ORDER / _RANGE (every form); two calls, and a call split
  by the stage bits, give bit-identical outputs.
* Both bf16 forms: arenas of up to 4096 nodes (records through the LDS DMA
  ring) and larger ones (per-lane loads).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import linear as LA
from generative_recommendation_beam_amd import _lib as L
from generative_recommendation_beam_amd import harness as HN
from parity import announce, assert_close
from test_gpu_2_decode import SMALL, compare

pytestmark = pytest.mark.gpu

CF = W.CONFIGS


def arena_of(x, rs=None):
    cfg = x.cfg
    rs = list(range(cfg.R)) if rs is None else list(rs)
    sl = lambda a: None if a is None else a[rs]
    cap = max(sum(k.shape[1] for (_, k, _) in x.levels), 1)
    ak, av, par = oracle.new_arena(len(rs), cap, cfg.H, cfg.d)
    prev, base = None, 0
    for (pb, k, v) in x.levels:
        ak, av, par, prev = oracle.trie_append(ak, av, par, base, k[rs], v[rs], sl(pb), prev)
        base += k.shape[1]
    return ak, av, par


def oracle_linear_step(x, rs=None):
    cfg = x.cfg
    rs = list(range(cfg.R)) if rs is None else list(rs)
    sl = lambda a: None if a is None else a[rs]
    ak, av, par = arena_of(x, rs)
    return LA.linear_decode_step(x.prompt_k[rs], x.prompt_v[rs], x.q[rs], par, ak, av, sl(x.beam_node), x.W,
                                 sl(x.prior), cfg.k, use_log_softmax=cfg.vocab > 1, window=cfg.window)


STATE_CASES = {
    "bf16_d64": W.reduced(CF["beam50_p600"], R=3, Lp=131),
    "bf16_d64_window": W.reduced(CF["beam512_p2048_w512"], R=2, Lp=300, window=130, H=4),
    "bf16_d32_short": W.reduced(CF["broadcast40k_u256"], n_in=8, k=8, level_sizes=(8,), Lp=37),
    "f32_d32": W.reduced(CF["beam100_p600"], R=2, Lp=40, H=4, d=32, n_in=16, k=16, level_sizes=(9, 16, 16),
                         dtype="f32"),
    "one_token": W.reduced(CF["beam50_p600"], R=2, Lp=1, level_sizes=(30, 50)),
}


@pytest.mark.parametrize("name", list(STATE_CASES))
def test_linear_state(name):
    cfg = STATE_CASES[name]
    announce(f"gr_linear_state {name}")
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x)
    S, z = HN.linear_state(ds)
    torch.cuda.synchronize()
    S_ref, z_ref = LA.prompt_state(x.prompt_k, x.prompt_v, cfg.window)
    assert_close(S.cpu().numpy(), S_ref, cfg.dtype, f"{name} state")
    assert_close(z.cpu().numpy(), z_ref, cfg.dtype, f"{name} norm")


ATTN_CASES = dict(STATE_CASES)
ATTN_CASES["depth8_chains"] = SMALL["depth8_chains"]
ATTN_CASES["beam130_two_chunks"] = SMALL["beam130_two_groups"]


@pytest.mark.parametrize("name", list(ATTN_CASES))
def test_linear_attn(name):
    cfg = ATTN_CASES[name]
    announce(f"gr_linear_attn {name}")
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x)
    S, z = HN.linear_state(ds)
    out = torch.empty((cfg.R, cfg.n_in, cfg.D), dtype=torch.float32, device="cuda")
    L.gr_linear_attn(ds.shape, S, z, ds.q, ds.n_beams, ds.trie, ds.beam_node, out, ds.dev_err)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == 0
    ak, av, par = arena_of(x)
    ref = LA.attend_linear_shared(x.prompt_k, x.prompt_v, x.q, par, ak, av, x.beam_node, cfg.window)
    assert_close(out.cpu().numpy(), ref, cfg.dtype, f"{name} linear attention")


STEP_CASES = ["beam50_small", "beam100_small", "beam100_flat_prior", "beam512_window_small", "beam130_two_groups",
              "scalar_small", "f32_beam16", "depth8_chains", "one_token_window", "single_beam",
              "max_width_h64_d64", "max_width_h128_d32", "max_width_f32",
              "max_width_long_window", "max_k_1024_beams"]


@pytest.mark.parametrize("name", STEP_CASES)
def test_linear_decode_step(name):
    cfg = SMALL[name]
    announce(f"gr_linear_decode_step {name}")
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x)
    S, z = HN.linear_state(ds)
    buf = HN.decode_buffers(ds, debug_outputs=True)
    HN.linear_decode_step(ds, buf, S, z)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == 0
    got = HN.results_to_host(buf)
    compare(cfg, got, oracle_linear_step(x), list(range(cfg.R)), f"linear {name}")


def test_linear_decode_full_size_sampled():
    cfg = CF["beam100_p600"]
    rs = [0, 131, 255]
    announce(f"gr_linear_decode_step beam100_p600 full size, oracle on requests {rs}")
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x)
    S, z = HN.linear_state(ds)
    buf = HN.decode_buffers(ds)
    HN.linear_decode_step(ds, buf, S, z)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == 0
    got = HN.results_to_host(buf)
    compare(cfg, got, oracle_linear_step(x, rs), rs, "linear beam100_p600", debug=False)
    # the same call again with debug outputs: attention and candidates
    buf2 = HN.decode_buffers(ds, debug_outputs=True)
    HN.linear_decode_step(ds, buf2, S, z)
    torch.cuda.synchronize()
    got2 = HN.results_to_host(buf2)
    np.testing.assert_array_equal(got2["token"], got["token"])
    np.testing.assert_array_equal(got2["score"], got["score"])
    ref = oracle_linear_step(x, rs)
    assert_close(got2["attn"][rs], ref["attn"], cfg.dtype, "linear beam100_p600 attention")
    assert_close(got2["cand"][rs], ref["cand"], cfg.dtype, "linear beam100_p600 candidates")


def test_linear_depth_error_and_determinism():
    cfg = SMALL["beam100_small"]
    announce("gr_linear_attn depth error, determinism")
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x, max_depth=2)       # chains of three records
    S, z = HN.linear_state(ds)
    out = torch.empty((cfg.R, cfg.n_in, cfg.D), dtype=torch.float32, device="cuda")
    L.gr_linear_attn(ds.shape, S, z, ds.q, ds.n_beams, ds.trie, ds.beam_node, out, ds.dev_err)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) & L.GR_DEVERR_DEPTH
    ds = HN.upload_step(x)
    S, z = HN.linear_state(ds)
    outs = []
    for _ in range(2):
        buf = HN.decode_buffers(ds, debug_outputs=True)
        HN.linear_decode_step(ds, buf, S, z)
        torch.cuda.synchronize()
        outs.append(HN.results_to_host(buf))
    for key in ("score", "token", "parent", "attn", "cand"):
        np.testing.assert_array_equal(outs[0][key], outs[1][key])


def test_linear_attn_large_arena():
    """Arenas above 4096 nodes per request take the per-lane-load form of the
    bf16 kernel instead of the ring form; same results."""
    cfg = SMALL["beam100_small"]
    announce("gr_linear_attn, 5000-node arena (per-lane loads)")
    x = W.make_step_inputs(cfg)
    outs = []
    for capacity in (None, 5000):
        ds = HN.upload_step(x, capacity=capacity)
        S, z = HN.linear_state(ds)
        out = torch.empty((cfg.R, cfg.n_in, cfg.D), dtype=torch.float32, device="cuda")
        L.gr_linear_attn(ds.shape, S, z, ds.q, ds.n_beams, ds.trie, ds.beam_node, out, ds.dev_err)
        torch.cuda.synchronize()
        assert int(ds.dev_err.item()) == 0
        outs.append(out.cpu().numpy())
    ak, av, par = arena_of(x)
    ref = LA.attend_linear_shared(x.prompt_k, x.prompt_v, x.q, par, ak, av, x.beam_node, cfg.window)
    assert_close(outs[0], ref, cfg.dtype, "linear attention, ring form")
    assert_close(outs[1], ref, cfg.dtype, "linear attention, per-lane form")


@pytest.mark.parametrize("capacity,dtype", [(None, "bf16"), (5000, "bf16"), (None, "f32")])
def test_linear_attn_device_errors(capacity, dtype):
    """Corrupt ancestry in each form (ring, per-lane loads, fp32): a parent
    newer than its child raises GR_DEVERR_PARENT_ORDER, a beam node outside
    the arena GR_DEVERR_PARENT_RANGE; nothing is read out of bounds."""
    cfg = W.reduced(CF["beam100_p600"], R=2, Lp=40, H=2, n_in=6, k=6, level_sizes=(3, 6, 6), dtype=dtype)
    announce(f"gr_linear_attn device errors, capacity {capacity}, {dtype}")
    x = W.make_step_inputs(cfg)
    out = torch.empty((cfg.R, cfg.n_in, cfg.D), dtype=torch.float32, device="cuda")

    def run(ds):
        S, z = HN.linear_state(ds)
        ds.dev_err.zero_()
        L.gr_linear_attn(ds.shape, S, z, ds.q, ds.n_beams, ds.trie, ds.beam_node, out, ds.dev_err)
        torch.cuda.synchronize()
        return int(ds.dev_err.item())

    ds = HN.upload_step(x, capacity=capacity)
    assert run(ds) == 0
    ds.parent[1, 9] = 12                         # a level-3 record gets a newer parent
    assert run(ds) & L.GR_DEVERR_PARENT_ORDER
    ds = HN.upload_step(x, capacity=capacity)
    ds.beam_node[0, 2] = 100000                  # outside the arena
    assert run(ds) == L.GR_DEVERR_PARENT_RANGE


@pytest.mark.parametrize("name", ["beam100_small", "one_token_window"])
def test_linear_stage_split_equals_whole(name):
    """The two stage bits of gr_linear_decode_step, called one after the
    other, give bit-identical results to one whole call."""
    cfg = SMALL[name]
    announce(f"gr_linear_decode_step stage split {name}")
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x)
    S, z = HN.linear_state(ds)
    outs = []
    for stages in ([0], [L.GR_STEP_ATTENTION, L.GR_STEP_SELECTION]):
        buf = HN.decode_buffers(ds, debug_outputs=True)
        for st in stages:
            L.gr_linear_decode_step(ds.shape, S, z, ds.q, ds.n_beams, ds.trie, ds.beam_node, ds.W, ds.vocab,
                                    ds.prior, ds.k, ds.flags | st, buf.score, buf.token, buf.parent, buf.attn,
                                    buf.cand, buf.ws, buf.ws_bytes, ds.dev_err)
        torch.cuda.synchronize()
        outs.append(HN.results_to_host(buf))
    assert int(ds.dev_err.item()) == 0
    for key in ("score", "token", "parent", "attn", "cand"):
        np.testing.assert_array_equal(outs[0][key], outs[1][key], err_msg=key)
