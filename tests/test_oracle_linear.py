"""Pins of the oracle's linear attention (CPU only).

What pins what:
* the feature map elu(x) + 1 at hand-derived points, including both sides of
  zero;
* library special case: with all-positive weights w_j, normalised linear
  attention equals softmax attention whose scores are log w_j.  torch's SDPA
  (float64) with a zero query and log w_j as its additive mask must give the
  oracle's output, the weights computed here with plain Python floats;
* the three formulations (per-beam materialised sum, per-beam recurrent state
  built token by token, shared prompt state plus the beam's records) agree to
  1e-12, with and without a window and on chains of one to three records;
* closed forms: one key gives its value; identical keys give the mean value;
* the own-branch rule: changing a non-ancestor record leaves every output
  bit-identical, changing an ancestor changes it;
* the shared prompt state equals explicit sums over the window rows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import linear as LA


def _build(cfg, seed=None):
    x = W.make_step_inputs(cfg, seed)
    ak, av, par = oracle.new_arena(cfg.R, max(cfg.capacity, 1), cfg.H, cfg.d)
    prev, base = None, 0
    for (pb, k, v) in x.levels:
        ak, av, par, prev = oracle.trie_append(ak, av, par, base, k, v, pb, prev)
        base += k.shape[1]
    return x, ak, av, par


SMALL = W.reduced(W.CONFIGS["beam50_p600"], R=3, Lp=23, n_in=7, level_sizes=(5, 7), H=2, d=8)
SMALL_D3 = W.reduced(W.CONFIGS["beam100_p600"], R=2, Lp=17, n_in=6, level_sizes=(4, 6, 6), H=3, d=4)


def _phi_py(x):
    return x + 1.0 if x > 0 else math.exp(x)


def test_phi_hand_values():
    xs = np.array([0.0, 1.0, -1.0, 2.5, -3.0, 1e-300, -1e-300])
    want = np.array([1.0, 2.0, math.exp(-1.0), 3.5, math.exp(-3.0), 1.0, 1.0])
    np.testing.assert_array_equal(LA.phi(xs), want)


@pytest.mark.parametrize("cfg,window", [(SMALL, 0), (SMALL, 6), (SMALL_D3, 0)])
def test_equals_sdpa_with_log_weight_mask(cfg, window):
    x, ak, av, par = _build(cfg)
    o = LA.attend_linear_materialized(x.prompt_k, x.prompt_v, x.q, par, ak, av, x.beam_node, window,
                                      out_dtype=np.float64)
    Lp, Lw, H, d = cfg.Lp, (cfg.Lp if window == 0 else window), cfg.H, cfg.d
    for r in range(cfg.R):
        for b in range(cfg.n_in):
            keys, vals = [], []
            for j in range(Lp - Lw, Lp):
                keys.append(x.prompt_k[r, j]); vals.append(x.prompt_v[r, j])
            nodes, n = [], int(x.beam_node[r, b])
            while n != -1:                          # the chain, walked independently
                nodes.append(n)
                n = int(par[r, n])
            for n in reversed(nodes):
                keys.append(ak[r, n]); vals.append(av[r, n])
            for h in range(H):
                w = [sum(_phi_py(float(x.q[r, b, h, i])) * _phi_py(float(k[h, i])) for i in range(d)) for k in keys]
                mask = torch.tensor([[math.log(v) for v in w]], dtype=torch.float64)
                q0 = torch.zeros((1, d), dtype=torch.float64)
                kt = torch.zeros((len(keys), d), dtype=torch.float64)
                vt = torch.tensor(np.array([v[h] for v in vals], np.float64))
                ref = torch.nn.functional.scaled_dot_product_attention(q0, kt, vt, attn_mask=mask).numpy()[0]
                np.testing.assert_allclose(o[r, b, h * d:(h + 1) * d], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("cfg,window", [(SMALL, 0), (SMALL, 4), (SMALL_D3, 0), (SMALL_D3, 1)])
def test_three_forms_agree(cfg, window):
    x, ak, av, par = _build(cfg)
    args = (x.prompt_k, x.prompt_v, x.q, par, ak, av, x.beam_node, window)
    a = LA.attend_linear_materialized(*args, out_dtype=np.float64)
    b = LA.attend_linear_recurrent(*args, out_dtype=np.float64)
    c = LA.attend_linear_shared(*args, out_dtype=np.float64)
    assert np.abs(a - b).max() <= 1e-12
    assert np.abs(a - c).max() <= 1e-12


def test_closed_forms():
    rng = np.random.default_rng(8)
    H, d = 2, 5
    pk = rng.standard_normal((1, 1, H, d))
    pv = rng.standard_normal((1, 1, H, d))
    q = rng.standard_normal((1, 3, H, d))
    o = LA.attend_linear_shared(pk, pv, q, out_dtype=np.float64)
    for b in range(3):
        np.testing.assert_allclose(o[0, b], pv[0, 0].reshape(-1), rtol=1e-14, atol=1e-14)
    pk = np.repeat(rng.standard_normal((1, 1, H, d)), 9, axis=1)
    pv = rng.standard_normal((1, 9, H, d))
    o = LA.attend_linear_shared(pk, pv, q, out_dtype=np.float64)
    np.testing.assert_allclose(o[0, 1], pv[0].mean(axis=0).reshape(-1), rtol=1e-13, atol=1e-13)


def test_own_branch_rule():
    cfg = SMALL_D3
    x, ak, av, par = _build(cfg)
    args = lambda a_k, a_v: (x.prompt_k, x.prompt_v, x.q, par, a_k, a_v, x.beam_node, 0)
    base = LA.attend_linear_shared(*args(ak, av))
    on_chain = set()
    for r in range(cfg.R):
        for b in range(cfg.n_in):
            on_chain |= {(r, n) for n in oracle.chain(par[r], int(x.beam_node[r, b]), 8)}
    changed_any = False
    for r in range(cfg.R):
        for n in range(ak.shape[1]):
            k2, v2 = ak.copy(), av.copy()
            k2[r, n] += 0.5
            v2[r, n] -= 0.25
            o = LA.attend_linear_shared(*args(k2, v2))
            if (r, n) in on_chain:
                assert not np.array_equal(o, base)
                changed_any = True
            else:
                np.testing.assert_array_equal(o, base)
    assert changed_any


def test_prompt_state_equals_explicit_sums():
    rng = np.random.default_rng(9)
    R, Lp, H, d, win = 2, 6, 2, 3, 4
    pk = rng.standard_normal((R, Lp, H, d)).astype(np.float32)
    pv = rng.standard_normal((R, Lp, H, d)).astype(np.float32)
    S, z = LA.prompt_state(pk, pv, win)
    for r in range(R):
        for h in range(H):
            for a in range(d):
                zz = math.fsum(_phi_py(float(pk[r, j, h, a])) for j in range(Lp - win, Lp))
                assert abs(z[r, h, a] - zz) <= 1e-14 * max(1.0, abs(zz))
                for c in range(d):
                    s = math.fsum(_phi_py(float(pk[r, j, h, a])) * float(pv[r, j, h, c])
                                  for j in range(Lp - win, Lp))
                    assert abs(S[r, h, a, c] - s) <= 1e-13
