"""Pins of the oracle's attention stage (CPU only).

What pins what:
* library special case: with no chain the operation is plain scaled dot-product
  attention, so the oracle must equal torch's SDPA (CPU, float64), with and
  without a window; with a chain it equals SDPA over [prompt ; all records]
  with a boolean mask that opens the window and the beam's own branch.
* invariant: the materialised, explicit-mask and split/log-sum-exp forms agree
  to float64 rounding (they share no arithmetic beyond the chain walk, which is
  pinned separately by the hand-worked fixtures).
* closed forms: one key -> its value; equal keys or q = 0 -> mean of the values
  of the key set; a window >= Lp -> full attention.
* own-branch rule (Engineering Exploration of Generative Recall, §4.4):
  changing a record that is not an ancestor of a beam (sibling, cousin, other
  request) leaves that beam's output bit-identical; changing an ancestor
  changes it; relabelling arena slots (parents stay older) changes nothing.
* hand-derived fixtures under tests/golden/.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(x):
    if isinstance(x, str):
        if x.startswith("ln"):
            return math.log(float(Fraction(x[2:].strip("()"))))
        return float(Fraction(x))
    return float(x)


def _arr(v, dtype=np.float32):
    return np.array([[_num(e) for e in row] for row in v], dtype=dtype)


def _build(cfg, seed=None):
    x = W.make_step_inputs(cfg, seed)
    ak, av, par = oracle.new_arena(cfg.R, max(cfg.capacity, 1), cfg.H, cfg.d)
    prev, base = None, 0
    for (pb, k, v) in x.levels:
        ak, av, par, prev = oracle.trie_append(ak, av, par, base, k, v, pb, prev)
        base += k.shape[1]
    return x, ak, av, par


SMALL = W.reduced(W.CONFIGS["beam50_p600"], R=3, Lp=23, n_in=7,
                  level_sizes=(5, 7), H=2, d=8)
SMALL_D3 = W.reduced(W.CONFIGS["beam100_p600"], R=2, Lp=17, n_in=6,
                     level_sizes=(4, 6, 6), H=3, d=4)


@pytest.mark.parametrize("window", [0, 5])
def test_prompt_only_equals_torch_sdpa(window):
    cfg = SMALL
    x, *_ = _build(cfg)
    o = oracle.attend_materialized(x.prompt_k, x.prompt_v, x.q, window=window,
                                   out_dtype=np.float64)
    Lw = cfg.Lp if window == 0 else window
    q = torch.from_numpy(x.q.astype(np.float64)).permute(0, 2, 1, 3)
    k = torch.from_numpy(x.prompt_k[:, cfg.Lp - Lw:].astype(np.float64)).permute(0, 2, 1, 3)
    v = torch.from_numpy(x.prompt_v[:, cfg.Lp - Lw:].astype(np.float64)).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)
    ref = ref.permute(0, 2, 1, 3).reshape(cfg.R, cfg.n_in, cfg.D).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("cfg,window", [(SMALL, 0), (SMALL, 9), (SMALL_D3, 0)])
def test_tree_mask_equals_torch_sdpa_with_bool_mask(cfg, window):
    x, ak, av, par = _build(cfg)
    o = oracle.attend_materialized(x.prompt_k, x.prompt_v, x.q, par, ak, av,
                                   x.beam_node, window=window, out_dtype=np.float64)
    Lp, Lw = cfg.Lp, (cfg.Lp if window == 0 else window)
    for r in range(cfg.R):
        K = np.concatenate([x.prompt_k[r], ak[r]], 0).astype(np.float64)
        V = np.concatenate([x.prompt_v[r], av[r]], 0).astype(np.float64)
        mask = np.zeros((cfg.n_in, K.shape[0]), bool)
        mask[:, Lp - Lw:Lp] = True
        for b in range(cfg.n_in):
            n = int(x.beam_node[r, b])
            while n != -1:                       # walk written out independently
                mask[b, Lp + n] = True
                n = int(par[r, n])
        q = torch.from_numpy(x.q[r].astype(np.float64)).permute(1, 0, 2)
        kt = torch.from_numpy(K).permute(1, 0, 2)
        vt = torch.from_numpy(V).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, kt, vt, attn_mask=torch.from_numpy(mask))
        ref = ref.permute(1, 0, 2).reshape(cfg.n_in, cfg.D).numpy()
        np.testing.assert_allclose(o[r], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("cfg,window", [(SMALL, 0), (SMALL, 4), (SMALL_D3, 0),
                                        (SMALL_D3, 1)])
def test_three_forms_agree(cfg, window):
    x, ak, av, par = _build(cfg)
    args = (x.prompt_k, x.prompt_v, x.q, par, ak, av, x.beam_node)
    a = oracle.attend_materialized(*args, window=window, out_dtype=np.float64)
    b = oracle.attend_masked(*args, window=window, out_dtype=np.float64)
    c = oracle.attend_split(*args, window=window, out_dtype=np.float64)
    assert np.abs(a - b).max() <= 1e-12
    assert np.abs(a - c).max() <= 1e-12
    # the float32 results differ by at most one rounding
    a32 = oracle.attend_materialized(*args, window=window)
    assert np.all(np.abs(a32 - a) <= np.spacing(np.abs(a32)))


def test_window_at_least_prompt_is_full():
    x, ak, av, par = _build(SMALL)
    args = (x.prompt_k, x.prompt_v, x.q, par, ak, av, x.beam_node)
    full = oracle.attend_materialized(*args, window=0)
    for w in (SMALL.Lp, SMALL.Lp + 1, 10 * SMALL.Lp):
        np.testing.assert_array_equal(oracle.attend_materialized(*args, window=w), full)


def test_closed_forms():
    rng = np.random.default_rng(7)
    H, d = 2, 4
    # single key -> its value
    pk = rng.standard_normal((1, 1, H, d)).astype(np.float32)
    pv = rng.standard_normal((1, 1, H, d)).astype(np.float32)
    q = rng.standard_normal((1, 3, H, d)).astype(np.float32)
    o = oracle.attend_materialized(pk, pv, q, out_dtype=np.float64)
    for b in range(3):
        np.testing.assert_allclose(o[0, b], pv[0, 0].reshape(-1), rtol=0, atol=1e-15)
    # all keys equal (prompt and chain) -> mean of the values
    Lp = 6
    krow = rng.standard_normal((H, d)).astype(np.float32)
    pk = np.broadcast_to(krow, (1, Lp, H, d)).copy()
    pv = rng.standard_normal((1, Lp, H, d)).astype(np.float32)
    ak, av, par = oracle.new_arena(1, 2, H, d)
    ak[0, :] = krow
    av[0] = rng.standard_normal((2, H, d)).astype(np.float32)
    par[0] = [-1, 0]
    q = rng.standard_normal((1, 1, H, d)).astype(np.float32)
    o = oracle.attend_materialized(pk, pv, q, par, ak, av, np.array([[1]], np.int32),
                                   out_dtype=np.float64)
    mean = (pv[0].astype(np.float64).sum(0) + av[0].astype(np.float64).sum(0)) / (Lp + 2)
    np.testing.assert_allclose(o[0, 0], mean.reshape(-1), rtol=1e-13, atol=1e-13)
    # q = 0 -> mean of the values of the beam's key set, with a window
    pk = rng.standard_normal((1, Lp, H, d)).astype(np.float32)
    q0 = np.zeros((1, 1, H, d), np.float32)
    o = oracle.attend_materialized(pk, pv, q0, par, ak, av, np.array([[0]], np.int32),
                                   window=2, out_dtype=np.float64)
    mean = (pv[0, Lp - 2:].astype(np.float64).sum(0) + av[0, 0].astype(np.float64)) / 3
    np.testing.assert_allclose(o[0, 0], mean.reshape(-1), rtol=1e-13, atol=1e-13)


def test_own_branch_perturbations():
    cfg = SMALL_D3
    x, ak, av, par = _build(cfg)
    args = lambda ak_, av_: (x.prompt_k, x.prompt_v, x.q, par, ak_, av_, x.beam_node)
    base = oracle.attend_materialized(*args(ak, av))
    r, b = 1, 2
    node = int(x.beam_node[r, b])
    anc = set(oracle.chain(par[r], node, 8))
    checked_off = checked_on = 0
    for n in range(cfg.capacity):
        ak2, av2 = ak.copy(), av.copy()
        ak2[r, n] += 1.5
        av2[r, n] -= 2.0
        o = oracle.attend_materialized(*args(ak2, av2))
        if n in anc:
            assert not np.array_equal(o[r, b], base[r, b])
            checked_on += 1
        else:
            np.testing.assert_array_equal(o[r, b], base[r, b])
            checked_off += 1
        np.testing.assert_array_equal(o[1 - r], base[1 - r])   # other request
    assert checked_on == cfg.depth and checked_off == cfg.capacity - cfg.depth


def test_relabelled_arena_gives_identical_outputs():
    cfg = SMALL_D3
    x, ak, av, par = _build(cfg)
    base = oracle.attend_materialized(x.prompt_k, x.prompt_v, x.q, par, ak, av,
                                      x.beam_node)
    # interleave the levels with unused slots and reverse order within a level;
    # parents stay older than their children
    cap = cfg.capacity
    new_id = np.zeros(cap, np.int64)
    offs = np.cumsum([0] + list(cfg.level_sizes))
    nxt = 0
    for li, n in enumerate(cfg.level_sizes):
        for j in reversed(range(n)):
            new_id[offs[li] + j] = nxt + 1      # one free slot before each node
            nxt += 2
    cap2 = 2 * cap + 1
    ak2, av2, par2 = oracle.new_arena(cfg.R, cap2, cfg.H, cfg.d)
    for r in range(cfg.R):
        for n in range(cap):
            m = new_id[n]
            ak2[r, m], av2[r, m] = ak[r, n], av[r, n]
            par2[r, m] = -1 if par[r, n] < 0 else new_id[par[r, n]]
    bn2 = new_id[x.beam_node].astype(np.int32)
    o = oracle.attend_materialized(x.prompt_k, x.prompt_v, x.q, par2, ak2, av2, bn2)
    np.testing.assert_array_equal(o, base)
    o_m = oracle.attend_masked(x.prompt_k, x.prompt_v, x.q, par2, ak2, av2, bn2)
    np.testing.assert_allclose(o_m, base, rtol=0, atol=4 * np.spacing(np.abs(base).max()))


def test_golden_attention_cases():
    with open(os.path.join(GOLDEN, "attention_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        pk = _arr(c["prompt_k"])[None, :, None, :]
        pv = _arr(c["prompt_v"])[None, :, None, :]
        q = _arr(c["q"])[None, :, None, :]
        kw = dict(window=c["window"], scale=1.0, out_dtype=np.float64)
        if c["beam_node"] is None:
            o = oracle.attend_materialized(pk, pv, q, **kw)
        else:
            ak = _arr(c["arena_k"])[None, :, None, :]
            av = _arr(c["arena_v"])[None, :, None, :]
            par = np.array([c["parent"]], np.int32)
            bn = np.array([c["beam_node"]], np.int32)
            o = oracle.attend_materialized(pk, pv, q, par, ak, av, bn, **kw)
            o2 = oracle.attend_masked(pk, pv, q, par, ak, av, bn, **kw)
            np.testing.assert_allclose(o2[0, :, 0], [_num(e) for e in c["expected"]],
                                       rtol=1e-6, err_msg=c["name"])
        np.testing.assert_allclose(o[0, :, 0], [_num(e) for e in c["expected"]],
                                   rtol=1e-6, err_msg=c["name"])


def test_chain_errors():
    par = np.array([-1, 0, 1, 2, 2, 7], np.int32)
    assert oracle.chain(par, 3, 8) == [0, 1, 2, 3]
    assert oracle.chain(par, 4, 8) == [0, 1, 2, 4]
    with pytest.raises(oracle.TrieError):
        oracle.chain(par, 3, 3)                 # depth 4 > max 3
    with pytest.raises(oracle.TrieError):
        oracle.chain(par, 5, 8)                 # parent 7 is not older than 5
    with pytest.raises(oracle.TrieError):
        oracle.chain(par, 6, 8)                 # outside the arena
    with pytest.raises(oracle.TrieError):
        oracle.chain(np.array([0], np.int32), 0, 8)   # self-parent (cycle)
