"""Codebook scoring, log-softmax, prior add and exact top-k (oracle).

Sources:
* Engineering Exploration of Generative Recall, §4.2 Custom Beam Search: the
  vocabulary is n x 256 codes, but each position has only 256 valid codes, so
  the step scores and ranks those 256 only (the current level's slice of the
  codebook).  The running beam score plus the code's log-probability ranks the
  B_in x 256 candidates, and the best B become the next beams.
* Same page, §4.4 Tree-Based Attention: beam widths 50 and 100.
* TransRetrieval, Model-based Retrieval / Hardware-aware inference
  optimization: each candidate is one query token over a shared user cache and
  gets one scalar score; candidate selection keeps the best (Recall@2000
  measures the 2000 kept).

Readings where the pages are silent (listed with the others in the design
notes): one root hypothesis enters the first step; the log-softmax runs over
the 256 codes of the current level only; no length normalisation; ties are
broken by the lower flat index f = b * vocab + t; the selection is made on
float32 scores.
"""
from __future__ import annotations

import numpy as np

from .attention import prefix_attn
from .trie import trie_append, new_arena

_F64 = np.float64


def codebook_logits(o, W):
    """z[r][b][t] = sum_i o[r][b][i] * W[t][i] (float64).  W is [vocab][D]:
    row t is code t's projection vector of the current level."""
    return np.einsum("rbi,ti->rbt", o.astype(_F64), W.astype(_F64))


def log_softmax(z):
    """lp = z - (max z + log sum exp(z - max z)) over the last axis."""
    z = np.asarray(z, _F64)
    m = z.max(axis=-1, keepdims=True)
    return z - (m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))


def candidate_scores(z, prior=None, use_log_softmax=True):
    """c[r][b][t] = prior[r][b] + lp[r][b][t] (or + z when the log-softmax is
    off), rounded to float32."""
    lp = log_softmax(z) if use_log_softmax else np.asarray(z, _F64)
    if prior is not None:
        lp = lp + np.asarray(prior, _F64)[..., None]
    return lp.astype(np.float32)


def select_topk(c, k):
    """Exact top-k of one request's candidates c [n_in][vocab] (float32):
    order by score descending, then flat index f = b * vocab + t ascending.
    Returns (score [k] float32, token [k] = f mod vocab, parent [k] = f div
    vocab), both int32."""
    n_in, vocab = c.shape
    flat = c.reshape(-1)
    f = np.arange(flat.size, dtype=np.int64)
    order = np.lexsort((f, -flat))[:k]
    return (flat[order].astype(np.float32), (order % vocab).astype(np.int32),
            (order // vocab).astype(np.int32))


def _select_all(c, k):
    R = c.shape[0]
    score = np.zeros((R, k), np.float32)
    token = np.zeros((R, k), np.int32)
    par = np.zeros((R, k), np.int32)
    for r in range(R):
        score[r], token[r], par[r] = select_topk(c[r], k)
    return score, token, par


def scalar_scores(o, w, prior=None):
    """One score per candidate: o[r][i] . w (+ prior[r][i]), float32."""
    s = np.einsum("rbi,i->rb", o.astype(_F64), np.asarray(w, _F64).reshape(-1))
    if prior is not None:
        s = s + np.asarray(prior, _F64)
    return s.astype(np.float32)


def beam_topk(logits, prior, k, use_log_softmax=True):
    """The selection stage on given logits [R][n_in][vocab]: candidate scores
    then exact top-k per request.  Returns dict(score, token, parent, cand)."""
    c = candidate_scores(logits, prior, use_log_softmax)
    score, token, par = _select_all(c, k)
    return dict(score=score, token=token, parent=par, cand=c)


def decode_step(prompt_k, prompt_v, q, parent, arena_k, arena_v, beam_node,
                W, prior, k, use_log_softmax=True, window=0, scale=None,
                max_depth=8):
    """One decode step: attention of every beam over the shared prompt and its
    own chain, codebook logits of the current level, log-softmax, prior add,
    exact top-k.  W is [vocab][D]; with vocab == 1 the step is scalar scoring
    (score = o . w, no log-softmax).  Returns dict(score, token, parent, attn,
    cand) with attn [R][n][D] float32 and cand [R][n][vocab] float32."""
    o = prefix_attn(prompt_k, prompt_v, q, parent, arena_k, arena_v,
                    beam_node, window, scale, max_depth)
    if W.shape[0] == 1 and not use_log_softmax:
        c = scalar_scores(o, W[0], prior)[..., None]
    else:
        c = candidate_scores(codebook_logits(o, W), prior, use_log_softmax)
    score, token, par = _select_all(c, k)
    return dict(score=score, token=token, parent=par, attn=o, cand=c)


def run_chained(prompt_k, prompt_v, W_levels, q_steps, rec_steps, prior0, k,
                window=0, scale=None, max_depth=8):
    """Free-running chained decode: step 0 has one prompt-only hypothesis per
    request; after step s the record (k, v) of every output slot j is appended
    with parent = node of the beam it extends (-1 after step 0), and the slot's
    score becomes its prior.  Each step keeps min(k, n_in * vocab) beams (a
    step cannot keep more candidates than it has).  q_steps[s] [R][n_s][H][d]; rec_steps[s] is
    either a pair of arrays [R][k][H][d] (slot-indexed) or a callable
    (s, token, parent) -> (k, v).  Returns the per-step results and the
    final arena."""
    R, Lp, H, d = prompt_k.shape
    steps = len(W_levels)
    ak, av, par = new_arena(R, max(k * (steps - 1), 1), H, d)
    beam_node, prior, base = None, prior0, 0
    results = []
    for s in range(steps):
        q = q_steps[s] if not callable(q_steps) else q_steps(s, results)
        ks = min(k, q.shape[1] * W_levels[s].shape[0])
        res = decode_step(prompt_k, prompt_v, q, par, ak, av, beam_node,
                          W_levels[s], prior, ks, True, window, scale, max_depth)
        results.append(res)
        if s + 1 < steps:
            rec = rec_steps[s]
            kn, vn = rec(s, res["token"], res["parent"]) if callable(rec) else rec
            pb = res["parent"] if beam_node is not None else None
            ak, av, par, beam_node = trie_append(
                ak, av, par, base, kn, vn, pb, beam_node)
            base += ks
            prior = res["score"]
    return results, (ak, av, par)

