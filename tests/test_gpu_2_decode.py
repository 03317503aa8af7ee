"""GPU parity of gr_decode_step (the whole hot path) against the oracle.

* Reduced versions of every workload family (beam 50/100/512 with windows,
  scalar scoring) and the widest model the boundary takes (D = 4096),
  compared in full: attention outputs, all candidate scores,
  the selected scores (max|err|/RMS bar), the index rule and exact
  self-consistency of the selection with the GPU's own candidate scores.
* The tiny fp32 workload run end to end for three chained steps, the trie grown
  by the decode itself through gr_trie_append (teacher forcing only if a
  near-tie < 1e-3 swaps a pick).
* Every full-size workload in the launch configuration the benchmark times
  (no debug outputs), checked on sampled requests that the oracle computes in
  full, plus a second call with debug outputs for attention and candidates.
* Determinism: two calls give bit-identical outputs.
* Two batches in flight on two streams match one call alone, bit for bit.
* The attention-only and selection-only stage bits, called one after the
  other, give bit-identical results to one whole call.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from generative_recommendation_beam_amd import _lib as L
from generative_recommendation_beam_amd import harness as HN
from parity import (announce, assert_close, check_index_rule, check_self_consistent)
from oracle_pool import oracle_many

pytestmark = pytest.mark.gpu

CF = W.CONFIGS
SMALL = {
    "beam50_small": W.reduced(CF["beam50_p600"], R=5, Lp=131, n_in=50, level_sizes=(41, 50)),
    "beam100_small": W.reduced(CF["beam100_p600"], R=4, Lp=200, n_in=100,
                               level_sizes=(100, 100, 100)),
    "beam100_flat_prior": W.reduced(CF["beam100_p600"], R=3, Lp=77, n_in=100,
                                    level_sizes=(90, 100, 100), prior="flat"),
    "beam512_window_small": W.reduced(CF["beam512_p2048_w512"], R=2, Lp=300, window=130, H=4,
                                      level_sizes=(256, 512, 512, 512)),
    "beam130_two_groups": W.reduced(CF["beam100_p600"], R=2, Lp=90, n_in=130, k=130,
                                    level_sizes=(100, 130, 130), H=4),
    "scalar_small": W.reduced(CF["broadcast40k_u256"], n_in=3000, k=333, level_sizes=(3000,)),
    # the bounded selection at larger k: four picks per wave (k > 256), the
    # lane-maximum bound with near-equal running scores, lists above 256
    # entries ordered by the bucket pass
    "k300_four_picks": W.reduced(CF["beam100_p600"], R=2, Lp=90, n_in=128, k=300, level_sizes=(100, 128, 128), H=4),
    "k512_flat_prior": W.reduced(CF["beam100_p600"], R=2, Lp=90, n_in=128, k=512, level_sizes=(100, 128, 128), H=4,
                                 prior="flat"),
    "k200_zero_prior": W.reduced(CF["beam100_p600"], R=2, Lp=90, n_in=100, k=200, level_sizes=(100, 100, 100), H=4,
                                 prior="zero"),
    # 64-beam scoring groups with k above the bounded selection's 512: the
    # register-wide selection over 32 slots a lane, alone (at most 64 input
    # beams) and with a merge of four 64-beam groups (the last one of 8 beams)
    "k600_beam60_exact": W.reduced(CF["beam100_p600"], R=2, Lp=90, n_in=60, k=600, level_sizes=(40, 60, 60), H=4),
    "k600_beam200_groups64": W.reduced(CF["beam100_p600"], R=2, Lp=90, n_in=200, k=600,
                                       level_sizes=(100, 200, 200), H=4),
    "f32_beam16": W.reduced(CF["beam100_p600"], R=2, Lp=40, H=4, d=32, n_in=16, k=16,
                            level_sizes=(9, 16, 16), dtype="f32"),
    # edge cases: chains of the maximum depth (8 records), a one-token prompt,
    # a one-token window, a single live beam
    "depth8_chains": W.reduced(CF["beam100_p600"], R=2, Lp=70, H=2, n_in=40, k=40, depth=8,
                               level_sizes=(24, 40, 40, 40, 40, 40, 40, 40)),
    "one_token_prompt": W.reduced(CF["beam50_p600"], R=2, Lp=1, level_sizes=(30, 50)),
    "one_token_window": W.reduced(CF["beam50_p600"], R=2, Lp=100, window=1, level_sizes=(30, 50)),
    "single_beam": W.reduced(CF["beam50_p600"], R=3, Lp=64, n_in=1, k=1, level_sizes=(1, 1)),
    # the widest model the boundary takes: D = H * d = 4096 (64 heads of 64,
    # 128 heads of 32; bf16 and fp32).  Windows below D / 8 keys take the fp32
    # projection; the 600-key window keeps the bf16 codebook MFMA.
    # the largest selection a decode step takes: 1024 beams (8 groups of 128)
    # into k = GR_MAX_K = 2048, 8 x 2048 partial entries in the final merge
    "max_k_1024_beams": W.reduced(CF["beam512_p2048_w512"], R=1, Lp=128, window=0, H=2, n_in=1024, k=2048,
                                  depth=2, level_sizes=(256, 1024)),
    "max_width_long_window": W.reduced(CF["beam100_p600"], R=1, Lp=600, H=64, d=64, n_in=32, k=32,
                                       level_sizes=(20, 32)),
    "max_width_h64_d64": W.reduced(CF["beam100_p600"], R=2, Lp=96, H=64, d=64, n_in=40, k=40,
                                   level_sizes=(30, 40)),
    "max_width_h128_d32": W.reduced(CF["beam100_p600"], R=2, Lp=80, H=128, d=32, n_in=24, k=24,
                                    level_sizes=(20, 24, 24)),
    "max_width_f32": W.reduced(CF["beam100_p600"], R=1, Lp=50, H=128, d=32, n_in=16, k=16,
                               level_sizes=(9, 16), dtype="f32"),
}


def oracle_step(x, rsel=None):
    """Oracle decode of the requests in rsel (all when None)."""
    cfg = x.cfg
    rs = list(range(cfg.R)) if rsel is None else list(rsel)
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


def compare(cfg, got, ref, rs, name, debug=True):
    tol = cfg.dtype
    if debug:
        assert_close(got["attn"][rs], ref["attn"], tol, f"{name} attention")
        assert_close(got["cand"][rs], ref["cand"], tol, f"{name} candidates")
        check_self_consistent(got["cand"], got["token"], got["parent"])
    assert_close(got["score"][rs], ref["score"], tol, f"{name} selected scores")
    band = 0
    for i, r in enumerate(rs):
        band += check_index_rule(ref["cand"][i], got["token"][r], got["parent"][r])
    return band


@pytest.mark.parametrize("name", sorted(SMALL))
def test_decode_small_parity(name):
    cfg = SMALL[name]
    announce(f"gr_decode_step {name}")
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x)
    buf = HN.decode_buffers(ds, debug_outputs=True)
    HN.decode_step(ds, buf)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == 0
    got = HN.results_to_host(buf)
    ref = oracle_step(x)
    band = compare(cfg, got, ref, list(range(cfg.R)), name)
    print(f"{name}: picks in the near-tie band: {band}")


@pytest.mark.parametrize("prior", ["cumsum", "flat"])
def test_decode_zero_codebook_ties(prior):
    """W = 0: every code of a beam has the same log-probability, so the
    candidates tie within each beam (and across all beams with a flat prior).
    The selection must follow the flat index among equal scores exactly."""
    cfg = W.reduced(CF["beam100_p600"], R=3, Lp=50, H=2, n_in=100, level_sizes=(60, 100, 100),
                    prior=prior)
    announce(f"gr_decode_step zero codebook, {prior} prior")
    x = W.make_step_inputs(cfg)
    x.W = np.zeros_like(x.W)
    ds = HN.upload_step(x)
    buf = HN.decode_buffers(ds, debug_outputs=True)
    HN.decode_step(ds, buf)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == 0
    got = HN.results_to_host(buf)
    check_self_consistent(got["cand"], got["token"], got["parent"])
    ref = oracle_step(x)
    compare(cfg, got, ref, list(range(cfg.R)), f"zero codebook {prior}")
    if prior == "cumsum":
        # the best beam's codes 0 .. k-1, in index order
        best = np.argmax(x.prior, axis=1)
        for r in range(cfg.R):
            np.testing.assert_array_equal(got["parent"][r], np.full(cfg.k, best[r]))
            np.testing.assert_array_equal(got["token"][r], np.arange(cfg.k))


def test_chained_fp32_three_steps():
    cfg = CF["tiny_f32_3step"]
    announce("gr_decode_step tiny_f32_3step chained")
    ci = W.make_chained_inputs(cfg)
    R, H, d, k = cfg.R, cfg.H, cfg.d, cfg.k
    shape = HN.make_shape(R, H, d, cfg.Lp, 0, L.GR_F32)
    pk, pv = HN.to_dev(ci.prompt_k, L.GR_F32), HN.to_dev(ci.prompt_v, L.GR_F32)
    cap = k * (cfg.steps - 1)
    ak_d, av_d, par_d, trie = HN.new_arena(shape, cap)
    ak, av, par = oracle.new_arena(R, cap, H, d)
    dev_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    node_d, node = None, None
    prior_d, prior = torch.zeros((R, 1), device="cuda"), ci.prior0
    base, forced = 0, 0
    for s in range(cfg.steps):
        q = ci.q[s]
        n_in = q.shape[1]
        ds = HN.DeviceStep(shape, pk, pv, HN.to_dev(q, L.GR_F32), HN.to_dev(ci.W[s], L.GR_F32), prior_d,
                           ak_d, av_d, par_d, trie if node_d is not None else None, node_d, n_in, k, 256,
                           L.GR_TOPK_LOG_SOFTMAX, dev_err)
        buf = HN.decode_buffers(ds, debug_outputs=True)
        HN.decode_step(ds, buf)
        torch.cuda.synchronize()
        assert int(dev_err.item()) == 0
        got = HN.results_to_host(buf)
        ref = oracle.decode_step(ci.prompt_k, ci.prompt_v, q, par, ak, av, node, ci.W[s], prior, k)
        compare(cfg, got, ref, list(range(R)), f"step {s}")
        same = (np.array_equal(got["token"], ref["token"]) and np.array_equal(got["parent"], ref["parent"]))
        if not same:
            forced += 1            # continue both sides from the oracle's picks
        tok, parent = ref["token"], ref["parent"]
        score_g = got["score"] if same else ref["score"]
        if s + 1 < cfg.steps:
            kn, vn = ci.rec[s]
            pb = parent if node is not None else None
            node_d = HN.append_level(shape, trie, base, kn, vn, pb, node_d, dev_err)
            ak, av, par, node = oracle.trie_append(ak, av, par, base, kn, vn, pb, node)
            base += k
            prior_d = torch.from_numpy(np.ascontiguousarray(score_g)).cuda()
            prior = ref["score"]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(node_d.cpu().numpy(), node)
    np.testing.assert_array_equal(par_d.cpu().numpy(), par)
    print(f"teacher-forced steps: {forced}")


# every request of the headline, the beam-50 and the scalar workloads, 8 of
# the 32 large-beam requests, and the 8192-key split-window workload in full
FULL = [("beam50_p600", None), ("beam100_p600", None),
        ("broadcast40k_u256", None), ("beam512_p2048_w512", [0, 5, 9, 13, 17, 22, 27, 31]),
        ("long8k_beam100", None)]


@pytest.mark.parametrize("name,rsel", FULL, ids=[n for n, _ in FULL])
def test_decode_full_size_sampled(name, rsel):
    cfg = CF[name]
    announce(f"gr_decode_step {name} full size")
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x)
    buf = HN.decode_buffers(ds, debug_outputs=False)       # as timed by the benchmark
    HN.decode_step(ds, buf)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == 0
    got = HN.results_to_host(buf)
    rs = list(range(cfg.R)) if rsel is None else rsel
    # the oracle over the requests in worker processes (one request each)
    ref = oracle_many(name, rs) if len(rs) > 1 else oracle_step(x, rs)
    compare(cfg, got, ref, rs, name, debug=False)
    # same call with the debug outputs: attention and every candidate score
    buf2 = HN.decode_buffers(ds, debug_outputs=True)
    HN.decode_step(ds, buf2)
    torch.cuda.synchronize()
    got2 = HN.results_to_host(buf2)
    for key in ("score", "token", "parent"):
        np.testing.assert_array_equal(got2[key], got[key])
    compare(cfg, got2, ref, rs, name, debug=True)


def test_determinism():
    cfg = SMALL["beam100_small"]
    announce("gr_decode_step determinism")
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x)
    outs = []
    for _ in range(2):
        buf = HN.decode_buffers(ds, debug_outputs=True)
        HN.decode_step(ds, buf)
        torch.cuda.synchronize()
        outs.append(HN.results_to_host(buf))
    for key in outs[0]:
        np.testing.assert_array_equal(outs[0][key], outs[1][key], err_msg=key)


@pytest.mark.parametrize("name", ["beam100_small", "one_token_window", "scalar_small", "f32_beam16"])
def test_stage_split_equals_whole(name):
    """GR_STEP_ATTENTION then GR_STEP_SELECTION on the same workspace (the
    split the benchmark times) gives bit-identical results to one whole call,
    on the bf16 codebook MFMA, the fp32 projection and scalar scoring."""
    cfg = SMALL[name]
    announce(f"gr_decode_step stage split {name}")
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x)
    outs = []
    for stages in ([0], [L.GR_STEP_ATTENTION, L.GR_STEP_SELECTION]):
        buf = HN.decode_buffers(ds, debug_outputs=True)
        for st in stages:
            L.gr_decode_step(ds.shape, ds.prompt_k, ds.prompt_v, ds.q, ds.n_beams, ds.trie, ds.beam_node, ds.W,
                             ds.vocab, ds.prior, ds.k, ds.flags | st, buf.score, buf.token, buf.parent, buf.attn,
                             buf.cand, buf.ws, buf.ws_bytes, ds.dev_err)
        torch.cuda.synchronize()
        outs.append(HN.results_to_host(buf))
    assert int(ds.dev_err.item()) == 0
    for key in ("score", "token", "parent", "attn", "cand"):
        np.testing.assert_array_equal(outs[0][key], outs[1][key], err_msg=key)


@pytest.mark.parametrize("name", ["beam100_small", "f32_beam16", "scalar_small"])
def test_dim_major_codebook_equals_code_major(name):
    """W given dimension-major ([H*d][vocab], the pages' D x 256 orientation)
    with GR_W_DIM_MAJOR gives bit-identical results to the default
    code-major [vocab][H*d]."""
    cfg = SMALL[name]
    announce(f"gr_decode_step dimension-major W {name}")
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x)
    wt = ds.W.t().contiguous()
    outs = []
    for w, fl in ((ds.W, 0), (wt, L.GR_W_DIM_MAJOR)):
        buf = HN.decode_buffers(ds, debug_outputs=True)
        L.gr_decode_step(ds.shape, ds.prompt_k, ds.prompt_v, ds.q, ds.n_beams, ds.trie, ds.beam_node, w,
                         ds.vocab, ds.prior, ds.k, ds.flags | fl, buf.score, buf.token, buf.parent, buf.attn,
                         buf.cand, buf.ws, buf.ws_bytes, ds.dev_err)
        torch.cuda.synchronize()
        outs.append(HN.results_to_host(buf))
    assert int(ds.dev_err.item()) == 0
    for key in ("score", "token", "parent", "attn", "cand"):
        np.testing.assert_array_equal(outs[0][key], outs[1][key], err_msg=key)


def test_two_streams_concurrent():
    """Two batches in flight on two streams (each with its own workspace and
    outputs, as the benchmark runs them) give the results of one call alone,
    bit for bit: the library keeps no state between calls."""
    cfg = SMALL["beam100_small"]
    announce("gr_decode_step on two streams at once")
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x)
    ref = HN.decode_buffers(ds, debug_outputs=True)
    HN.decode_step(ds, ref)
    torch.cuda.synchronize()
    want = HN.results_to_host(ref)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    bufs = [[HN.decode_buffers(ds, debug_outputs=True) for _ in range(3)] for _ in streams]
    torch.cuda.synchronize()
    for i in range(3):
        for s, b in zip(streams, bufs):
            HN.decode_step(ds, b[i], stream=s)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == 0
    for b in bufs:
        for buf in b:
            got = HN.results_to_host(buf)
            for key in ("score", "token", "parent", "attn", "cand"):
                np.testing.assert_array_equal(got[key], want[key], err_msg=key)
