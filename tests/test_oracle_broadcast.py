"""Pins of the multi-layer broadcast-scoring oracle (oracle/broadcast.py).

What fixes each function, independently of the oracle's own code:
* the layer stack (Pre-LN, ReLU FFN of width 2D, biases, LayerNorm eps
  1e-5): torch.nn.TransformerEncoderLayer with norm_first=True,
  activation="relu", dim_feedforward=2D, no dropout, in float64, on the whole
  sequence [user tokens; one candidate] with a mask that keeps the user rows
  off the candidate (readings X5, X6).  Every user hidden state and the
  candidate's final state must agree; a dropped residual, a wrong head split,
  a transposed weight or a missing self key fails this.
* candidate_attention: the decode step's attention oracle (already pinned by
  torch SDPA) with the user keys as the prompt and each candidate's own key
  as its one-record chain -- the one-layer core of the broadcast-scoring
  workload with the scalar score.
* layer_norm / score_head: hand-computed fixtures.
* isolation (X6): candidates scored together equal candidates scored one by
  one, and a permutation of the candidates permutes the scores; the user
  keys and values do not depend on the candidates (X5).
* broadcast_score's selection: sorted by (score desc, index asc), and equal
  to a plain Python sort of the returned scores.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import broadcast as BC
import workloads as W


def _params(x: W.XFInputs) -> BC.ModelParams:
    layers = [BC.LayerParams(**{k: lp[k] for k in (
        "w_qkv", "b_qkv", "w_o", "b_o", "w_1", "b_1", "w_2", "b_2",
        "ln1_g", "ln1_b", "ln2_g", "ln2_b")}) for lp in x.layers]
    return BC.ModelParams(layers, x.lnf_g, x.lnf_b, x.w_score, x.b_score)


SMALL = W.XFConfig("xf_small", 60, R=1, Lu=6, N=5, D=64, n_layers=2, k=3)


def _torch_stack(x: W.XFInputs, n_heads: int):
    D = x.cfg.D
    mods = []
    for lp in x.layers:
        m = torch.nn.TransformerEncoderLayer(D, n_heads, dim_feedforward=2 * D, dropout=0.0,
                                             activation="relu", layer_norm_eps=1e-5,
                                             batch_first=True, norm_first=True,
                                             dtype=torch.float64)
        with torch.no_grad():
            t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
            m.self_attn.in_proj_weight.copy_(t(lp["w_qkv"]))
            m.self_attn.in_proj_bias.copy_(t(lp["b_qkv"]))
            m.self_attn.out_proj.weight.copy_(t(lp["w_o"]))
            m.self_attn.out_proj.bias.copy_(t(lp["b_o"]))
            m.linear1.weight.copy_(t(lp["w_1"]))
            m.linear1.bias.copy_(t(lp["b_1"]))
            m.linear2.weight.copy_(t(lp["w_2"]))
            m.linear2.bias.copy_(t(lp["b_2"]))
            m.norm1.weight.copy_(t(lp["ln1_g"]))
            m.norm1.bias.copy_(t(lp["ln1_b"]))
            m.norm2.weight.copy_(t(lp["ln2_g"]))
            m.norm2.bias.copy_(t(lp["ln2_b"]))
        m.train()          # dropout 0: the plain (non-fused) math path
        mods.append(m)
    return mods


def test_layer_stack_matches_torch_pre_ln_encoder():
    x = W.make_xf_inputs(SMALL)
    P = _params(x)
    n_heads = 2
    Lu = SMALL.Lu
    kv, xs = BC.user_forward(x.user[0], P, n_heads)
    final = BC.candidate_forward(x.cand[0], kv, P, n_heads)
    mods = _torch_stack(x, n_heads)
    # user rows may not attend to the candidate (True = blocked)
    mask = torch.zeros(Lu + 1, Lu + 1, dtype=torch.bool)
    mask[:Lu, Lu] = True
    for i in range(SMALL.N):
        seq = np.concatenate([x.user[0], x.cand[0][i:i + 1]], axis=0)
        h = torch.from_numpy(seq.astype(np.float64))[None]
        for m in mods:
            h = m(h, src_mask=mask)
        h = h[0].detach().numpy()
        np.testing.assert_allclose(final[i], h[Lu], rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(xs[-1], h[:Lu], rtol=1e-10, atol=1e-10)


def test_candidate_attention_is_the_decode_attention_with_a_self_record():
    rng = np.random.default_rng(7)
    Lu, N, H, d = 9, 6, 2, 32
    D = H * d
    ku, vu = rng.standard_normal((Lu, D)), rng.standard_normal((Lu, D))
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    got = BC.candidate_attention(q, k, v, ku, vu, H)
    ak, av, par = oracle.new_arena(1, N, H, d)
    ak[0] = k.reshape(N, H, d)
    av[0] = v.reshape(N, H, d)
    ref = oracle.prefix_attn(ku.reshape(1, Lu, H, d).astype(np.float32),
                             vu.reshape(1, Lu, H, d).astype(np.float32),
                             q.reshape(1, N, H, d).astype(np.float32), par, ak, av,
                             np.arange(N, dtype=np.int32)[None])
    # the decode oracle stores float32 inputs: compare on those values
    got32 = BC.candidate_attention(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                                   ku.astype(np.float32), vu.astype(np.float32), H)
    np.testing.assert_allclose(got32, ref[0], rtol=1e-6, atol=1e-6)
    assert got.shape == (N, D)


def test_layer_norm_fixture():
    # x = [1, 2, 3, 4]: mean 2.5, biased variance 1.25
    y = BC.layer_norm(np.array([[1.0, 2.0, 3.0, 4.0]]), np.array([1.0, 2.0, 1.0, 1.0]),
                      np.array([0.0, 0.0, 0.5, 0.0]), eps=0.0)
    s = math.sqrt(1.25)
    np.testing.assert_allclose(y[0], [-1.5 / s, 2 * (-0.5 / s), 0.5 / s + 0.5, 1.5 / s], rtol=1e-14)
    # eps enters under the root
    y = BC.layer_norm(np.array([[0.0, 2.0]]), np.ones(2), np.zeros(2), eps=3.0)
    np.testing.assert_allclose(y[0], [-1 / 2, 1 / 2], rtol=1e-14)


def test_score_head_fixture():
    P = BC.ModelParams([], np.array([1.0, 1.0]), np.array([0.0, 0.0]), np.array([2.0, -1.0]), 0.25)
    # LN([3, 5]) = [-1, 1] (eps negligible at this precision): 2 * -1 - 1 * 1 + 0.25
    np.testing.assert_allclose(BC.score_head(np.array([[3.0, 5.0]]), P), [-2.75], rtol=1e-5)


def test_candidates_are_isolated_and_the_user_side_is_shared():
    x = W.make_xf_inputs(SMALL)
    P = _params(x)
    kv, _ = BC.user_forward(x.user[0], P, 2)
    together = BC.candidate_forward(x.cand[0], kv, P, 2)
    alone = np.concatenate([BC.candidate_forward(x.cand[0][i:i + 1], kv, P, 2) for i in range(SMALL.N)])
    np.testing.assert_allclose(together, alone, rtol=1e-12, atol=1e-12)
    perm = np.array([3, 0, 4, 1, 2])
    np.testing.assert_allclose(BC.candidate_forward(x.cand[0][perm], kv, P, 2), together[perm],
                               rtol=1e-12, atol=1e-12)
    # chunking changes nothing
    np.testing.assert_allclose(BC.candidate_forward(x.cand[0], kv, P, 2, chunk=2), together,
                               rtol=1e-12, atol=1e-12)
    # other candidates, same user keys and values
    x2 = W.make_xf_inputs(SMALL, seed=999)
    kv2, _ = BC.user_forward(x.user[0], P, 2)
    for (k1, v1), (k2, v2) in zip(kv, kv2):
        np.testing.assert_array_equal(k1, k2)
        np.testing.assert_array_equal(v1, v2)
    assert not np.array_equal(x2.cand, x.cand)


def test_broadcast_score_selection_order():
    cfg = W.XFConfig("xf_sel", 61, R=2, Lu=8, N=40, D=64, n_layers=1, k=7)
    x = W.make_xf_inputs(cfg)
    P = _params(x)
    res = BC.broadcast_score(x.user, x.cand, P, cfg.k, n_heads=2)
    for r in range(cfg.R):
        s = res["all"][r]
        order = sorted(range(cfg.N), key=lambda i: (-float(s[i]), i))[:cfg.k]
        assert res["index"][r].tolist() == order
        np.testing.assert_array_equal(res["score"][r], s[order])


@pytest.mark.parametrize("D", [64, 128])
def test_default_heads_are_32_wide(D):
    cfg = W.XFConfig("xf_heads", 62, R=1, Lu=4, N=3, D=D, n_layers=1, k=2)
    x = W.make_xf_inputs(cfg)
    P = _params(x)
    a = BC.broadcast_score(x.user, x.cand, P, 2)
    b = BC.broadcast_score(x.user, x.cand, P, 2, n_heads=D // 32)
    np.testing.assert_array_equal(a["all"], b["all"])
