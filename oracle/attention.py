"""Attention of every beam over the shared prompt plus its own ancestor chain
(oracle, float64 arithmetic, float32 outputs).

The operation (per request r, live beam b, head h):

    keys(b)  = prompt rows [Lp - Lw, Lp)  followed by  chain(beam_node[b])
    s_j      = (q[b,h] . k_j[h]) * scale            scale = 1/sqrt(d) default
    p        = softmax(s)   over keys(b)            (one softmax, no dropout)
    o[b, h*d + i] = sum_j p_j v_j[h][i]

Sources:
* Engineering Exploration of Generative Recall, §4.1 Superman Optimizer: the
  attention steps are QK^T, scaling, mask, softmax, (dropout, off at
  inference) and the weighted sum, done as one SDPA call.
* Same page, §4.4 Tree-Based Attention: the shared prefix is stored once and a
  tree-aware mask lets each token see only ancestors on its own branch.
* Same page, §4.5 Sliding-Window Attention: the prompt part may be limited to
  a window of the most recent omega tokens; the chain is never windowed.
* TransRetrieval, Hardware-aware inference optimization: one user KV cache is
  broadcast to every candidate without copies, and packed single-query
  candidates are kept apart by masking.
* OneLA, Abstract: shared prompt state plus per-beam append-only records.

Three formulations are given; they are algebraically identical and are
cross-checked in the tests:
  attend_materialized  copies each beam's full key/value sequence (the
                       "full state per beam" baseline OneLA describes)
  attend_masked        one sequence = prompt + every arena record of the
                       request, with an explicit ancestor mask (-inf off
                       branch), i.e. the tree-aware mask of §4.4 written out
  attend_split         softmax over the prompt part and over the chain part
                       separately, merged with their log-sum-exp weights
"""
from __future__ import annotations

import math

import numpy as np

from .trie import chain

_F64 = np.float64


def _window(Lp: int, window: int) -> int:
    return Lp if (window is None or window <= 0) else min(int(window), Lp)


def _scale(d: int, scale) -> float:
    return 1.0 / math.sqrt(d) if (scale is None or scale == 0) else float(scale)


def _chains(parent, beam_node, r, nb, max_depth):
    if beam_node is None:
        return [[] for _ in range(nb)]
    return [chain(parent[r], int(beam_node[r, b]), max_depth) for b in range(nb)]


def attend_materialized(prompt_k, prompt_v, q, parent=None, arena_k=None,
                        arena_v=None, beam_node=None, window=0, scale=None,
                        max_depth=8, out_dtype=np.float32):
    """Per beam: build K_b, V_b = [prompt window ; chain records] as real
    copies ([Lw + delta][H][d]), then softmax attention per head.  Returns
    o [R][n_beams][H*d] (float32 unless out_dtype says otherwise)."""
    R, Lp, H, d = prompt_k.shape
    nb = q.shape[1]
    Lw = _window(Lp, window)
    sc = _scale(d, scale)
    out = np.zeros((R, nb, H * d), out_dtype)
    for r in range(R):
        pk = prompt_k[r, Lp - Lw:].astype(_F64)
        pv = prompt_v[r, Lp - Lw:].astype(_F64)
        chains = _chains(parent, beam_node, r, nb, max_depth)
        for b in range(nb):
            ch = chains[b]
            if ch:
                Kb = np.concatenate([pk, arena_k[r, ch].astype(_F64)], axis=0)
                Vb = np.concatenate([pv, arena_v[r, ch].astype(_F64)], axis=0)
            else:
                Kb, Vb = pk.copy(), pv.copy()
            qb = q[r, b].astype(_F64)                      # [H][d]
            for h in range(H):
                s = (Kb[:, h, :] @ qb[h]) * sc              # [n_keys]
                p = np.exp(s - s.max())
                p /= p.sum()
                out[r, b, h * d:(h + 1) * d] = p @ Vb[:, h, :]
    return out


def attend_masked(prompt_k, prompt_v, q, parent=None, arena_k=None,
                  arena_v=None, beam_node=None, window=0, scale=None,
                  max_depth=8, n_nodes=None, out_dtype=np.float32):
    """One key sequence per request: all Lp prompt rows followed by the first
    n_nodes arena records.  Mask M[b][j] is open for prompt rows inside the
    window and for records on chain(b); every other score is -inf before the
    softmax.  Returns o [R][n_beams][H*d] (float32 unless out_dtype says
    otherwise)."""
    R, Lp, H, d = prompt_k.shape
    nb = q.shape[1]
    Lw = _window(Lp, window)
    sc = _scale(d, scale)
    if arena_k is None or beam_node is None:
        n_nodes = 0
    elif n_nodes is None:
        n_nodes = arena_k.shape[1]
    out = np.zeros((R, nb, H * d), out_dtype)
    for r in range(R):
        if n_nodes:
            K = np.concatenate([prompt_k[r], arena_k[r, :n_nodes]], 0).astype(_F64)
            V = np.concatenate([prompt_v[r], arena_v[r, :n_nodes]], 0).astype(_F64)
        else:
            K = prompt_k[r].astype(_F64)
            V = prompt_v[r].astype(_F64)
        nk = K.shape[0]
        mask = np.zeros((nb, nk), bool)
        mask[:, Lp - Lw:Lp] = True
        chains = _chains(parent, beam_node, r, nb, max_depth)
        for b in range(nb):
            for n in chains[b]:
                mask[b, Lp + n] = True
        qr = q[r].astype(_F64)                               # [nb][H][d]
        for h in range(H):
            S = (qr[:, h, :] @ K[:, h, :].T) * sc            # [nb][nk]
            S = np.where(mask, S, -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            out[r, :, h * d:(h + 1) * d] = P @ V[:, h, :]
    return out


def attend_split(prompt_k, prompt_v, q, parent=None, arena_k=None,
                 arena_v=None, beam_node=None, window=0, scale=None,
                 max_depth=8, out_dtype=np.float32):
    """Softmax over the prompt window alone -> (m1, l1, o1) and over the chain
    alone -> (m2, l2, o2), where m is the max score, l = sum exp(s - m) and o
    the normalised output of that part; then
        m = max(m1, m2),  o = (l1 e^{m1-m} o1 + l2 e^{m2-m} o2)
                              / (l1 e^{m1-m} + l2 e^{m2-m}).
    Returns o [R][n_beams][H*d] (float32 unless out_dtype says otherwise)."""
    R, Lp, H, d = prompt_k.shape
    nb = q.shape[1]
    Lw = _window(Lp, window)
    sc = _scale(d, scale)
    out = np.zeros((R, nb, H * d), out_dtype)
    for r in range(R):
        pk = prompt_k[r, Lp - Lw:].astype(_F64)
        pv = prompt_v[r, Lp - Lw:].astype(_F64)
        chains = _chains(parent, beam_node, r, nb, max_depth)
        for b in range(nb):
            qb = q[r, b].astype(_F64)
            ch = chains[b]
            for h in range(H):
                s1 = (pk[:, h, :] @ qb[h]) * sc
                m1 = s1.max()
                e1 = np.exp(s1 - m1)
                l1 = e1.sum()
                o1 = (e1 @ pv[:, h, :]) / l1
                if not ch:
                    out[r, b, h * d:(h + 1) * d] = o1
                    continue
                ck = arena_k[r, ch, h, :].astype(_F64)
                cv = arena_v[r, ch, h, :].astype(_F64)
                s2 = (ck @ qb[h]) * sc
                m2 = s2.max()
                e2 = np.exp(s2 - m2)
                l2 = e2.sum()
                o2 = (e2 @ cv) / l2
                m = max(m1, m2)
                w1 = l1 * math.exp(m1 - m)
                w2 = l2 * math.exp(m2 - m)
                out[r, b, h * d:(h + 1) * d] = (w1 * o1 + w2 * o2) / (w1 + w2)
    return out


def prefix_attn(prompt_k, prompt_v, q, parent=None, arena_k=None,
                arena_v=None, beam_node=None, window=0, scale=None,
                max_depth=8):
    """The attention stage of the decode step: the materialised form."""
    return attend_materialized(prompt_k, prompt_v, q, parent, arena_k,
                               arena_v, beam_node, window, scale, max_depth)
