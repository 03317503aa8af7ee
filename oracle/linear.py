"""Linear attention over the shared prompt plus each beam's own records
(oracle, float64 arithmetic, float32 outputs).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg use this module.

Source: OneLA, Abstract.  Large-beam decoding with recurrent linear
attention; instead of a full recurrent state per beam (or replaying the shared
history), every beam's state is one shared prompt-derived state plus compact
append-only records of its own divergent transitions, found through a light
ancestry index, and only the state information a step needs is computed.

The operation (per request r, live beam b, head h), with the positive feature
map phi(x) = elu(x) + 1 applied elementwise:

    keys(b)   = prompt rows [Lp - Lw, Lp)  followed by  chain(beam_node[b])
    S_b       = sum_{j in keys(b)} phi(k_j) v_j^T        ([d][d])
    z_b       = sum_{j in keys(b)} phi(k_j)              ([d])
    o[b, h*d + i] = (phi(q) . S_b[:, i]) / (phi(q) . z_b)

Readings (the abstract names neither): the feature map is elu + 1, the common
choice that keeps every weight positive so the normaliser cannot vanish, and
the output is normalised by phi(q) . z (attention weights that sum to one, as
in the softmax form); no score scale; the window and the chain are those of
the softmax form.

Three formulations, cross-checked in the tests:
  attend_linear_materialized  per beam, its full key/value sequence as a
                              real copy, weights phi(q).phi(k_j) summed
                              directly (no state at all)
  attend_linear_recurrent     per beam, the recurrent state built token by
                              token: S_t = S_{t-1} + phi(k_t) v_t^T over the
                              prompt then the chain (the "full state per
                              beam" a linear-attention server would keep)
  attend_linear_shared        the shared prompt state (prompt_state) plus the
                              beam's chain records, as OneLA represents it
"""
from __future__ import annotations

import numpy as np

from .trie import chain

_F64 = np.float64


def phi(x):
    """elu(x) + 1: x + 1 for x > 0, exp(x) otherwise (float64)."""
    x = np.asarray(x, _F64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def _window(Lp: int, window: int) -> int:
    return Lp if (window is None or window <= 0) else min(int(window), Lp)


def _chains(parent, beam_node, r, nb, max_depth):
    if beam_node is None:
        return [[] for _ in range(nb)]
    return [chain(parent[r], int(beam_node[r, b]), max_depth) for b in range(nb)]


def prompt_state(prompt_k, prompt_v, window=0):
    """The shared prompt-derived state of every (request, head): S [R][H][d][d]
    = sum over the window rows of phi(k) v^T, z [R][H][d] = sum of phi(k);
    float64."""
    R, Lp, H, d = prompt_k.shape
    Lw = _window(Lp, window)
    fk = phi(prompt_k[:, Lp - Lw:])                       # [R][Lw][H][d]
    v = np.asarray(prompt_v[:, Lp - Lw:], _F64)
    S = np.einsum("rjhk,rjhv->rhkv", fk, v)
    z = fk.sum(axis=1)
    return S, z


def attend_linear_materialized(prompt_k, prompt_v, q, parent=None, arena_k=None, arena_v=None,
                               beam_node=None, window=0, max_depth=8, out_dtype=np.float32):
    R, Lp, H, d = prompt_k.shape
    nb = q.shape[1]
    Lw = _window(Lp, window)
    out = np.zeros((R, nb, H * d), out_dtype)
    for r in range(R):
        chains = _chains(parent, beam_node, r, nb, max_depth)
        for b in range(nb):
            ch = chains[b]
            Kb = np.concatenate([prompt_k[r, Lp - Lw:], arena_k[r, ch]], 0) if ch else prompt_k[r, Lp - Lw:]
            Vb = np.concatenate([prompt_v[r, Lp - Lw:], arena_v[r, ch]], 0) if ch else prompt_v[r, Lp - Lw:]
            fq = phi(q[r, b])                              # [H][d]
            fk = phi(Kb)                                   # [n][H][d]
            for h in range(H):
                w = fk[:, h, :] @ fq[h]                    # [n] weights, all positive
                out[r, b, h * d:(h + 1) * d] = (w @ np.asarray(Vb[:, h, :], _F64)) / w.sum()
    return out


def attend_linear_recurrent(prompt_k, prompt_v, q, parent=None, arena_k=None, arena_v=None,
                            beam_node=None, window=0, max_depth=8, out_dtype=np.float32):
    R, Lp, H, d = prompt_k.shape
    nb = q.shape[1]
    Lw = _window(Lp, window)
    out = np.zeros((R, nb, H * d), out_dtype)
    for r in range(R):
        chains = _chains(parent, beam_node, r, nb, max_depth)
        for b in range(nb):
            seq_k = [prompt_k[r, j] for j in range(Lp - Lw, Lp)] + [arena_k[r, n] for n in chains[b]]
            seq_v = [prompt_v[r, j] for j in range(Lp - Lw, Lp)] + [arena_v[r, n] for n in chains[b]]
            S = np.zeros((H, d, d), _F64)
            z = np.zeros((H, d), _F64)
            for kt, vt in zip(seq_k, seq_v):
                fk = phi(kt)
                S += fk[:, :, None] * np.asarray(vt, _F64)[:, None, :]
                z += fk
            fq = phi(q[r, b])
            for h in range(H):
                out[r, b, h * d:(h + 1) * d] = (fq[h] @ S[h]) / (fq[h] @ z[h])
    return out


def attend_linear_shared(prompt_k, prompt_v, q, parent=None, arena_k=None, arena_v=None,
                         beam_node=None, window=0, max_depth=8, state=None, out_dtype=np.float32):
    """o from the shared prompt state plus the beam's own records:
    numerator phi(q)^T S_p + sum_n (phi(q).phi(k_n)) v_n, denominator
    phi(q).z_p + sum_n phi(q).phi(k_n).  `state` = prompt_state(...) may be
    passed in."""
    R, Lp, H, d = prompt_k.shape
    nb = q.shape[1]
    S, z = prompt_state(prompt_k, prompt_v, window) if state is None else state
    out = np.zeros((R, nb, H * d), out_dtype)
    for r in range(R):
        chains = _chains(parent, beam_node, r, nb, max_depth)
        for b in range(nb):
            fq = phi(q[r, b])                              # [H][d]
            num = np.einsum("hk,hkv->hv", fq, S[r])
            den = np.einsum("hk,hk->h", fq, z[r])
            for n in chains[b]:
                w = np.einsum("hk,hk->h", fq, phi(arena_k[r, n]))
                num += w[:, None] * np.asarray(arena_v[r, n], _F64)
                den += w
            out[r, b] = (num / den[:, None]).reshape(H * d)
    return out


def linear_decode_step(prompt_k, prompt_v, q, parent, arena_k, arena_v, beam_node, W, prior, k,
                       use_log_softmax=True, window=0, max_depth=8):
    """A decode step with linear attention: attend_linear_shared, then the
    same scoring as the softmax step (codebook logits, log-softmax, prior add,
    exact top-k; with vocab == 1 and no log-softmax, scalar scores o . w).
    Returns dict(score, token, parent, attn, cand)."""
    from .beam import codebook_logits, candidate_scores, scalar_scores, _select_all
    o = attend_linear_shared(prompt_k, prompt_v, q, parent, arena_k, arena_v, beam_node, window,
                             max_depth)
    if W.shape[0] == 1 and not use_log_softmax:
        c = scalar_scores(o, W[0], prior)[..., None]
    else:
        c = candidate_scores(codebook_logits(o, W), prior, use_log_softmax)
    score, token, par = _select_all(c, k)
    return dict(score=score, token=token, parent=par, attn=o, cand=c)
