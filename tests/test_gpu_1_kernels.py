"""GPU parity of the individual C-ABI entry points against the oracle.

gr_trie_append: bit-exact arena, parent ids and node ids; device error bits.
gr_prefix_attn: max|err|/RMS within the bf16 / fp32 bar on cases that span
several 64-key tiles with a ragged tail, ragged beam counts (1, 2, 4 waves per
workgroup and several beam groups), windows, chain depths 0..3, head dims 32
and 64; device error bits for corrupt parents and chains past max_depth.
gr_beam_topk: scores within the bar, the index rule, exact self-consistency,
exact ties, multi-group merges, scalar (vocab 1) selection of 2000 of 40000.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from generative_recommendation_beam_amd import _lib as L
from generative_recommendation_beam_amd import harness as HN
from parity import (announce, assert_close, check_index_rule, check_self_consistent, TOL)

pytestmark = pytest.mark.gpu

C2, C3 = W.CONFIGS["beam50_p600"], W.CONFIGS["beam100_p600"]

ATTN_CASES = {
    "bf16_d64_ragged_nw2": W.reduced(C2, R=2, Lp=150, n_in=37, level_sizes=(20, 37)),
    "bf16_d32_window_nw4": W.reduced(C3, R=3, Lp=70, window=33, H=4, d=32, n_in=100,
                                     level_sizes=(30, 100, 100)),
    "bf16_prompt_only_nw1": W.reduced(C2, R=1, Lp=64, H=2, n_in=5, depth=0, level_sizes=()),
    "bf16_two_groups": W.reduced(C2, R=2, Lp=200, window=100, H=2, n_in=129, depth=1,
                                 level_sizes=(129,)),
    "bf16_short_prompt": W.reduced(C2, R=2, Lp=3, H=3, n_in=40, depth=2, level_sizes=(7, 40)),
    "f32_d32": W.reduced(C2, R=2, Lp=50, H=4, d=32, n_in=9, level_sizes=(4, 9), dtype="f32"),
    "f32_d64_window": W.reduced(C3, R=1, Lp=65, window=20, H=2, n_in=70,
                                level_sizes=(10, 40, 70), dtype="f32"),
}


def oracle_arena(x):
    cfg = x.cfg
    cap = max(sum(k.shape[1] for (_, k, _) in x.levels), 1)
    ak, av, par = oracle.new_arena(cfg.R, cap, cfg.H, cfg.d)
    prev, base = None, 0
    for (pb, k, v) in x.levels:
        ak, av, par, prev = oracle.trie_append(ak, av, par, base, k, v, pb, prev)
        base += k.shape[1]
    return ak, av, par


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_trie_append_bitexact(dtype):
    announce(f"gr_trie_append {dtype}")
    cfg = W.reduced(C3, R=3, Lp=8, H=4, d=32 if dtype == "f32" else 64, n_in=60,
                    level_sizes=(11, 33, 60), dtype=dtype)
    x = W.make_step_inputs(cfg)
    shape = HN.make_shape(cfg.R, cfg.H, cfg.d, cfg.Lp, 0, HN.dtype_code(dtype))
    dev_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ak_d, av_d, par_d, trie = HN.new_arena(shape, 110)
    ak, av, par = oracle.new_arena(cfg.R, 110, cfg.H, cfg.d)
    prev_d, prev, base = None, None, 3          # start past a few unused slots
    for (pb, k, v) in x.levels:
        prev_d = HN.append_level(shape, trie, base, k, v, pb, prev_d, dev_err)
        ak, av, par, prev = oracle.trie_append(ak, av, par, base, k, v, pb, prev)
        base += k.shape[1]
    torch.cuda.synchronize()
    assert int(dev_err.item()) == 0
    np.testing.assert_array_equal(prev_d.cpu().numpy(), prev)
    np.testing.assert_array_equal(par_d.cpu().numpy(), par)
    np.testing.assert_array_equal(ak_d.float().cpu().numpy(), ak)
    np.testing.assert_array_equal(av_d.float().cpu().numpy(), av)


def test_trie_append_device_errors():
    announce("gr_trie_append device errors")
    shape = HN.make_shape(2, 2, 32, 4, 0, L.GR_BF16)
    dev_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ak_d, av_d, par_d, trie = HN.new_arena(shape, 16)
    rng = np.random.default_rng(0)
    k = rng.standard_normal((2, 3, 2, 32)).astype(np.float32)
    nodes = HN.append_level(shape, trie, 0, k, k, None, None, dev_err)
    bad_pb = np.array([[0, 5, 1], [2, 2, -1]], np.int32)          # 5 and -1 out of range
    HN.append_level(shape, trie, 3, k, k, bad_pb, nodes, dev_err)
    torch.cuda.synchronize()
    assert int(dev_err.item()) == L.GR_DEVERR_BEAM_RANGE
    p = par_d.cpu().numpy()
    assert p[0, 4] == -1 and p[1, 5] == -1 and p[0, 3] == 0 and p[1, 3] == 2
    dev_err.zero_()
    late = torch.tensor([[9, 1, 2], [0, 1, 2]], dtype=torch.int32, device="cuda")  # node 9 is newer
    HN.append_level(shape, trie, 6, k, k, np.zeros((2, 3), np.int32), late, dev_err)
    torch.cuda.synchronize()
    assert int(dev_err.item()) == L.GR_DEVERR_PARENT_ORDER


@pytest.mark.parametrize("name", sorted(ATTN_CASES))
def test_prefix_attn_parity(name):
    cfg = ATTN_CASES[name]
    announce(f"gr_prefix_attn {name}")
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x)
    out = HN.prefix_attn(ds)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == 0
    ak, av, par = oracle_arena(x)
    ref = oracle.prefix_attn(x.prompt_k, x.prompt_v, x.q, par, ak, av, x.beam_node,
                             window=cfg.window)
    e = assert_close(out.cpu().numpy(), ref, cfg.dtype, name)
    print(f"{name}: max|err|/RMS = {e:.3e}")


# Arenas of up to 4096 nodes per request have their chains resolved inside
# the attention kernel (parents staged in LDS); larger ones through the
# chain-resolve pre-pass.  Both paths are exercised.
LARGE_ARENA = 5000


def test_prefix_attn_parity_large_arena():
    announce("gr_prefix_attn bf16 chains in a 5000-node arena")
    cfg = ATTN_CASES["bf16_d64_ragged_nw2"]
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x, capacity=LARGE_ARENA)
    out = HN.prefix_attn(ds)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == 0
    ak, av, par = oracle_arena(x)
    ref = oracle.prefix_attn(x.prompt_k, x.prompt_v, x.q, par, ak, av, x.beam_node, window=cfg.window)
    assert_close(out.cpu().numpy(), ref, cfg.dtype, "bf16_large_arena")


def relocated(ds, off):
    """The same step with its arena moved up by `off` slots (node ids and
    parent links shift by off) and the slots below it holding NaN."""
    R, cap = ds.parent.shape
    ak = torch.full((R, cap + off) + tuple(ds.arena_k.shape[2:]), float("nan"), dtype=ds.arena_k.dtype,
                    device=ds.arena_k.device)
    av = ak.clone()
    ak[:, off:] = ds.arena_k
    av[:, off:] = ds.arena_v
    par = torch.full((R, cap + off), -1, dtype=torch.int32, device=ds.parent.device)
    par[:, off:] = torch.where(ds.parent >= 0, ds.parent + off, ds.parent)
    trie = L.Trie(k=ak.data_ptr(), v=av.data_ptr(), parent=par.data_ptr(), capacity=cap + off,
                  max_depth=ds.trie.max_depth)
    trie._tensors = (ak, av, par)
    bn = torch.where(ds.beam_node >= 0, ds.beam_node + off, ds.beam_node)
    return dataclasses.replace(ds, arena_k=ak, arena_v=av, parent=par, trie=trie, beam_node=bn)


# 128-beam workgroups fold each chain level as one product over the tile of
# all their beams' rows; beams without a record at a level must not bring in
# arena slots that hold no record.  Mixed chain depths (prompt-only beams,
# one-record chains, full chains) over an arena whose unused slots hold NaN.
MIXED_DEPTHS = W.reduced(W.CONFIGS["beam100_p600"], R=2, Lp=90, n_in=100, level_sizes=(60, 100, 100), H=4)


def mixed_depth_step(capacity):
    x = W.make_step_inputs(MIXED_DEPTHS)
    ds = HN.upload_step(x, capacity=capacity)
    ds.beam_node[:, ::5] = -1                    # prompt only
    ds.beam_node[:, 1::5] = 7                    # a level-1 node: a one-record chain
    return ds


@pytest.mark.parametrize("capacity", [None, LARGE_ARENA])
def test_decode_step_never_reads_unused_arena_slots(capacity):
    announce(f"decode step, mixed chain depths, arena moved over NaN slots, capacity {capacity}")
    ds = mixed_depth_step(capacity)
    outs = []
    for d in (ds, relocated(ds, 37)):
        buf = HN.decode_buffers(d, debug_outputs=True)
        HN.decode_step(d, buf)
        torch.cuda.synchronize()
        outs.append(buf)
    assert int(ds.dev_err.item()) == 0
    a, b = outs
    assert torch.isfinite(b.attn).all() and torch.isfinite(b.score).all()
    for name in ("attn", "cand", "score", "token", "parent"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


def test_linear_step_never_reads_unused_arena_slots():
    announce("linear decode step, mixed chain depths, arena moved over NaN slots")
    ds = mixed_depth_step(None)
    S, z = HN.linear_state(ds)
    outs = []
    for d in (ds, relocated(ds, 37)):
        buf = HN.decode_buffers(d, debug_outputs=True)
        HN.linear_decode_step(d, buf, S, z)
        torch.cuda.synchronize()
        outs.append(buf)
    assert int(ds.dev_err.item()) == 0
    a, b = outs
    assert torch.isfinite(b.attn).all() and torch.isfinite(b.score).all()
    for name in ("attn", "cand", "score", "token", "parent"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


@pytest.mark.parametrize("capacity", [None, LARGE_ARENA])
def test_prefix_attn_device_errors(capacity):
    announce(f"gr_prefix_attn device errors, capacity {capacity}")
    cfg = W.reduced(C3, R=2, Lp=40, H=2, n_in=6, level_sizes=(3, 6, 6))
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x, max_depth=2, capacity=capacity)   # chains have 3 records
    HN.prefix_attn(ds)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == L.GR_DEVERR_DEPTH
    ds = HN.upload_step(x, capacity=capacity)
    ds.parent[1, 9] = 12                         # beam 0's record gets a newer parent
    ds.dev_err.zero_()
    HN.prefix_attn(ds)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) & L.GR_DEVERR_PARENT_ORDER
    ds = HN.upload_step(x, capacity=capacity)
    ds.beam_node[0, 2] = 100000                  # outside the arena
    ds.dev_err.zero_()
    HN.prefix_attn(ds)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == L.GR_DEVERR_PARENT_RANGE


TOPK_CASES = {
    "beam100": dict(R=3, n_in=100, vocab=256, k=100, lsm=True, prior="cumsum"),
    "three_groups_merge": dict(R=2, n_in=300, vocab=256, k=100, lsm=True, prior="cumsum"),
    "flat_prior": dict(R=2, n_in=64, vocab=256, k=64, lsm=True, prior="flat"),
    "exact_ties": dict(R=2, n_in=50, vocab=256, k=50, lsm=False, prior="int", quant=True),
    "take_all": dict(R=2, n_in=7, vocab=256, k=1792, lsm=True, prior="cumsum"),
    "single_root": dict(R=4, n_in=1, vocab=256, k=8, lsm=True, prior="zero"),
    "scalar_2000_of_40000": dict(R=1, n_in=40000, vocab=1, k=2000, lsm=False, prior="none"),
    "scalar_ties": dict(R=2, n_in=5000, vocab=1, k=700, lsm=False, prior="none", quant=True),
    "max_k": dict(R=2, n_in=20, vocab=256, k=2048, lsm=True, prior="cumsum"),   # k = GR_MAX_K
    # final merge over several groups: exact ties across group boundaries, and
    # 3 x 2048 partial entries ranked by several blocks per request
    "merge_ties": dict(R=2, n_in=200, vocab=256, k=300, lsm=False, prior="int", quant=True),
    "merge_max_k": dict(R=2, n_in=300, vocab=256, k=2048, lsm=True, prior="cumsum"),
    # integer-valued scores with many exact ties: the selection lists (about
    # 1000 and 1700 entries) crowd single buckets of the bucket sort, so they
    # are ordered by the merge sort (runs of 2 and 4 entries per thread)
    "ties_merge_sort_1k": dict(R=2, n_in=64, vocab=256, k=1000, lsm=False, prior="int", quant=True),
    "ties_merge_sort_2k": dict(R=2, n_in=40, vocab=256, k=1500, lsm=False, prior="int", quant=True),
}


@pytest.mark.parametrize("name", sorted(TOPK_CASES))
def test_beam_topk_parity(name):
    c = TOPK_CASES[name]
    announce(f"gr_beam_topk {name}")
    check_topk_case(name, c, np.random.default_rng(len(name)))


def check_topk_case(name, c, rng):
    """gr_beam_topk on seeded logits (N(0, 0.1) codes or N(0, 1) scalars,
    optionally rounded to multiples of 1/40 for exact ties) against the
    oracle: exact values and indices without the log-softmax, the index rule
    with it, and exact self-consistency with the returned candidate scores."""
    R, n_in, V, k = c["R"], c["n_in"], c["vocab"], c["k"]
    z = rng.standard_normal((R, n_in, V)).astype(np.float32) * (0.1 if V == 256 else 1.0)
    if c.get("quant"):
        z = np.round(z * 40).astype(np.float32)
    prior = None
    if c["prior"] == "cumsum":
        prior = np.cumsum(-rng.standard_normal((R, n_in)) ** 2, axis=1).astype(np.float32)
    elif c["prior"] in ("flat", "zero"):
        prior = np.zeros((R, n_in), np.float32)
    elif c["prior"] == "int":
        prior = -rng.integers(0, 6, size=(R, n_in)).astype(np.float32)
    flags = L.GR_TOPK_LOG_SOFTMAX if c["lsm"] else 0
    zd = torch.from_numpy(z).cuda()
    pd = None if prior is None else torch.from_numpy(prior).cuda()
    score, token, parent, cand = HN.beam_topk(zd, pd, k, flags)
    torch.cuda.synchronize()
    score, token, parent, cand = (t.cpu().numpy() for t in (score, token, parent, cand))
    ref = oracle.beam_topk(z, prior, k, c["lsm"])
    check_self_consistent(cand, token, parent)
    if not c["lsm"]:
        # integer-valued or plain sums: both sides compute the same fp32 values
        np.testing.assert_array_equal(cand, ref["cand"])
        np.testing.assert_array_equal(token, ref["token"])
        np.testing.assert_array_equal(parent, ref["parent"])
    assert_close(cand, ref["cand"], "f32", f"{name} candidates")
    assert_close(score, ref["score"], "f32", f"{name} scores")
    for r in range(R):
        check_index_rule(ref["cand"][r], token[r], parent[r])
