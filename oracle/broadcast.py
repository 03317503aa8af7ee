"""Multi-layer broadcast scoring of single-token candidates (oracle).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg use this module.

Sources (TransRetrieval: Scaling Up Transformer-Based Retrieval for
Industrial Recommendation):
* Architecture Overview, stage (4): the tokens go through an N-layer Pre-LN
  Transformer whose feed-forward network uses ReLU; the user-side keys and
  values of a request are cached once and reused by all of its candidates.
* The per-candidate cost paragraph: a candidate needs its own Q/K/V/output
  projections and FFN, 16 L_t D^2 FLOPs per layer, plus attention over the
  whole user sequence, 4 L_t L_u D FLOPs per layer; after target compression
  L_t = 1 (one token per candidate).
* Hardware-aware inference optimization: the one user cache is broadcast to
  every candidate without copies; single-token candidates are packed into
  one batched computation and kept apart by masking.
* GPU retrieval: the candidate selection runs on the device.
* Model-based Retrieval: about 4 x 10^4 candidates per request; Recall@2000
  (experiments) gives the 2000 kept.

Readings (the pages leave these open):
* X1  Layer: x <- x + MHA(LN1(x)); x <- x + FFN(LN2(x)), FFN(h) =
      ReLU(h W1^T + b1) W2^T + b2.  The FFN width is 2D: the four D x D
      projections take 8 D^2 FLOPs per token, so the cost's 16 D^2 leaves
      8 D^2 = 2 * 2 * D * F for the two FFN products, F = 2D.
* X2  LayerNorm over the D features with the biased variance, eps = 1e-5,
      a gain and a bias per feature.
* X3  Every projection has a bias (standard linear layers, weight [out][in]).
* X4  Heads of 32 dimensions (D = 128: 4 heads), scores scaled by
      1/sqrt(32), one softmax per head.
* X5  User tokens attend to every user token (feature fields have no order)
      and never to a candidate: that is what lets their keys and values be
      computed once per request and shared.
* X6  A candidate token attends to the L_u user keys of the layer and to its
      own key (it forms its own K and V; nothing else reads them).
      Candidates never see one another.
* X7  After the last layer a final LayerNorm and a linear head give the
      scalar score s = LN_f(x) . w + b.
* X8  The selection keeps the k best scores of each request, ties broken by
      the lower candidate index (the beam step's rule).
* X9  The inputs are the tokens as they enter the Transformer (feature
      aggregation, target compression and the domain embedding happen
      upstream and are not part of this computation).

Arithmetic: float64 throughout from the (bf16-representable) float32 inputs;
scores are rounded to float32, and the selection is decided on them.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List

import numpy as np

from .beam import select_topk

_F64 = np.float64
LN_EPS = 1e-5
HEAD_DIM = 32


@dataclasses.dataclass
class LayerParams:
    """One layer's weights: w_qkv [3D][D] (rows: the query, key and value
    output features), b_qkv [3D], w_o [D][D], b_o [D], w_1 [2D][D], b_1 [2D],
    w_2 [D][2D], b_2 [D], ln1_g, ln1_b, ln2_g, ln2_b [D]."""
    w_qkv: np.ndarray
    b_qkv: np.ndarray
    w_o: np.ndarray
    b_o: np.ndarray
    w_1: np.ndarray
    b_1: np.ndarray
    w_2: np.ndarray
    b_2: np.ndarray
    ln1_g: np.ndarray
    ln1_b: np.ndarray
    ln2_g: np.ndarray
    ln2_b: np.ndarray


@dataclasses.dataclass
class ModelParams:
    """The layer stack plus the final LayerNorm (lnf_g, lnf_b [D]) and the
    scoring head (w_score [D], b_score scalar)."""
    layers: List[LayerParams]
    lnf_g: np.ndarray
    lnf_b: np.ndarray
    w_score: np.ndarray
    b_score: float

    @property
    def D(self) -> int:
        return int(self.lnf_g.shape[0])


def layer_norm(x, g, b, eps=LN_EPS):
    """(x - mean) / sqrt(var + eps) * g + b over the last axis, var biased
    (reading X2)."""
    x = np.asarray(x, _F64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(g, _F64) + np.asarray(b, _F64)


def _linear(x, w, b):
    return x @ np.asarray(w, _F64).T + np.asarray(b, _F64)


def _heads(x, n_heads):
    n, D = x.shape
    return x.reshape(n, n_heads, D // n_heads)


def user_attention(q, k, v, n_heads):
    """Every user token over every user token (reading X5): q, k, v [Lu][D]
    -> [Lu][D]."""
    qh, kh, vh = _heads(q, n_heads), _heads(k, n_heads), _heads(v, n_heads)
    d = qh.shape[-1]
    s = np.einsum("ihd,jhd->hij", qh, kh) / math.sqrt(d)
    s -= s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return np.einsum("hij,jhd->ihd", p, vh).reshape(q.shape)


def candidate_attention(q, k, v, k_user, v_user, n_heads):
    """Each candidate over the layer's user keys and its own key (reading
    X6): q, k, v [N][D] (the candidates' own), k_user, v_user [Lu][D] ->
    [N][D].  The user cache is read in place by every candidate (the
    broadcast), the own key enters as one more score per candidate."""
    qh, kh, vh = _heads(q, n_heads), _heads(k, n_heads), _heads(v, n_heads)
    kuh, vuh = _heads(k_user, n_heads), _heads(v_user, n_heads)
    d = qh.shape[-1]
    s_user = np.einsum("nhd,jhd->nhj", qh, kuh) / math.sqrt(d)          # [N][H][Lu]
    s_self = np.einsum("nhd,nhd->nh", qh, kh)[..., None] / math.sqrt(d)  # [N][H][1]
    s = np.concatenate([s_user, s_self], axis=-1)
    s -= s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    o = np.einsum("nhj,jhd->nhd", p[..., :-1], vuh) + p[..., -1:] * vh
    return o.reshape(q.shape)


def _qkv(h, lp):
    D = h.shape[-1]
    qkv = _linear(h, lp.w_qkv, lp.b_qkv)
    return qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:]


def _ffn(h, lp):
    return _linear(np.maximum(_linear(h, lp.w_1, lp.b_1), 0.0), lp.w_2, lp.b_2)


def user_forward(u, P: ModelParams, n_heads):
    """The user tokens u [Lu][D] through the layer stack.  Returns (kv, xs):
    kv[l] = (K_l, V_l) [Lu][D], the keys and values every candidate reads at
    layer l, and xs[l] the user hidden states entering layer l (xs[L] after
    the last one)."""
    x = np.asarray(u, _F64)
    kv, xs = [], [x]
    for lp in P.layers:
        q, k, v = _qkv(layer_norm(x, lp.ln1_g, lp.ln1_b), lp)
        kv.append((k, v))
        x = x + _linear(user_attention(q, k, v, n_heads), lp.w_o, lp.b_o)
        x = x + _ffn(layer_norm(x, lp.ln2_g, lp.ln2_b), lp)
        xs.append(x)
    return kv, xs


def candidate_forward(c, kv, P: ModelParams, n_heads, chunk=2048):
    """The candidate tokens c [N][D] through the layer stack, each attending
    to the cached user keys/values kv[l] and to itself.  Returns the final
    hidden states [N][D] (before the final LayerNorm).  Candidates are
    independent; they are processed in chunks only to bound memory."""
    c = np.asarray(c, _F64)
    out = np.empty_like(c)
    for s0 in range(0, c.shape[0], chunk):
        x = c[s0:s0 + chunk]
        for lp, (ku, vu) in zip(P.layers, kv):
            q, k, v = _qkv(layer_norm(x, lp.ln1_g, lp.ln1_b), lp)
            x = x + _linear(candidate_attention(q, k, v, ku, vu, n_heads), lp.w_o, lp.b_o)
            x = x + _ffn(layer_norm(x, lp.ln2_g, lp.ln2_b), lp)
        out[s0:s0 + chunk] = x
    return out


def score_head(x, P: ModelParams):
    """s = LN_f(x) . w + b (reading X7), float64."""
    return layer_norm(x, P.lnf_g, P.lnf_b) @ np.asarray(P.w_score, _F64) + float(P.b_score)


def broadcast_score(user_tok, cand_tok, P: ModelParams, k, n_heads=None):
    """The whole computation for R requests: user_tok [R][Lu][D], cand_tok
    [R][N][D].  Returns dict(score [R][k], index [R][k] (int32), all [R][N]
    float32 candidate scores)."""
    R, N, D = cand_tok.shape
    n_heads = D // HEAD_DIM if n_heads is None else n_heads
    k = min(int(k), N)
    allsc = np.zeros((R, N), np.float32)
    score = np.zeros((R, k), np.float32)
    index = np.zeros((R, k), np.int32)
    for r in range(R):
        kv, _ = user_forward(user_tok[r], P, n_heads)
        x = candidate_forward(cand_tok[r], kv, P, n_heads)
        allsc[r] = score_head(x, P).astype(np.float32)
        score[r], _, index[r] = select_topk(allsc[r][:, None], k)
    return dict(score=score, index=index, all=allsc)
