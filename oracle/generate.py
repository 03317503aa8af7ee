"""Whole semantic-ID generation on the device's terms (oracle).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg use this module.

Sources:
* Engineering Exploration of Generative Recall, §4.2 Custom Beam Search: an
  item ID is a sequence of codes, one per level; the vocabulary is n x 256 and
  each position has its own 256 valid codes, so level l is scored against its
  own slice (W_l) and the best B partial IDs survive each step.
* Same page, §4.1 Superman Optimizer: attention starts from the query, key
  and value computed for each token.
* OneLA, Abstract: every surviving beam adds one compact record of its new
  transition to an append-only store; the ancestry index links it to the
  beam it extends.
* TransRetrieval, GPU retrieval: the scoring and selection of every
  iteration stay in one device-resident pipeline, with no host round trip.

Readings (the pages do not spell the step between two levels out):
* The code chosen at step l enters step l+1 as a token.  Its embedding is row
  t of the level's table emb_l [V][De] (the level's slice of the n x 256
  vocabulary), and the model's projections give q = emb_l[t] Wq^T,
  k = emb_l[t] Wk^T, v = emb_l[t] Wv^T, with w_qkv = [Wq; Wk; Wv] of shape
  [3D][De].  k, v become the beam's new record; q is its next query.
* These vectors depend on (level, code) only, so projecting the V rows of a
  level once and looking up the chosen code gives exactly the values of
  projecting each chosen token: code_table() computes that table.
* Step 0 has one root hypothesis per request whose query q0 is given (the
  prompt's own last position); its prior is 0.  Step l keeps
  k_l = min(B, n_l * V) beams, n_0 = 1, n_{l+1} = k_l.
* The stored table is rounded once to the storage dtype (round to nearest
  even for bf16) from the exact (float64) dot products.
"""
from __future__ import annotations

import numpy as np

from .beam import run_chained


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned
    as float32 (every bfloat16 value is one).  bfloat16 keeps 7 of the 52
    explicit mantissa bits of a float64: the low 45 bits are dropped with
    round-to-nearest-even on the bit pattern, which carries into the exponent
    where it must.  Finite, normal inputs within the float32 range."""
    a = np.ascontiguousarray(np.asarray(x, np.float64))
    bits = a.view(np.uint64)
    drop = np.uint64(45)
    lsb = (bits >> drop) & np.uint64(1)
    half = np.uint64((1 << 44) - 1)
    kept = (bits + half + lsb) & ~np.uint64((1 << 45) - 1)
    return kept.view(np.float64).astype(np.float32)


def level_sizes(levels: int, k: int, vocab: int = 256):
    """(n_l, k_l) for l = 0 .. levels-1: beams entering and leaving each step."""
    n, out = 1, []
    for _ in range(levels):
        kl = min(k, n * vocab)
        out.append((n, kl))
        n = kl
    return out


def code_table(emb, w_qkv, H: int, d: int, dtype: str = "f32"):
    """q, k, v of every code of one level.  emb [V][De], w_qkv [3D][De]
    (rows: the D query features, then the key and value features), D = H*d.
    Returns [V][3][H][d] float32: T[t][c] = sum_i emb[t][i] w_qkv[c][i],
    summed in float64 and rounded once to the storage dtype ("f32" or
    "bf16")."""
    e = np.asarray(emb, np.float64)
    w = np.asarray(w_qkv, np.float64)
    V, De = e.shape
    assert w.shape == (3 * H * d, De)
    t = e @ w.T
    t = t.astype(np.float32) if dtype == "f32" else round_to_bf16(t)
    return t.reshape(V, 3, H, d)


def backtrack_ids(results) -> np.ndarray:
    """Code sequence of every final beam: ids[r][j][l] for the beams leaving
    the last step, following out_parent back through the steps."""
    last = results[-1]
    R, k = last["token"].shape
    L = len(results)
    ids = np.zeros((R, k, L), np.int32)
    for r in range(R):
        for j in range(k):
            ids[r, j, L - 1] = last["token"][r, j]
            p = int(last["parent"][r, j])
            for lv in range(L - 2, -1, -1):
                ids[r, j, lv] = results[lv]["token"][r, p]
                p = int(results[lv]["parent"][r, p])
    return ids


def generate(prompt_k, prompt_v, q0, W_levels, tables, k, window=0,
             scale=None, max_depth=8):
    """All levels of the ID.  q0 [R][1][H][d]; W_levels[l] [V][D] (level l's
    codebook projection); tables[l] [V][3][H][d] for l < levels-1 (the
    projection of level l's chosen codes, code_table()).  Returns
    (results, ids, arena): per-step dicts as decode_step returns them, the
    final beams' code sequences [R][k_last][levels], and the final arena."""
    levels = len(W_levels)
    assert len(tables) >= levels - 1

    def q_steps(s, results):
        if s == 0:
            return q0
        return tables[s - 1][:, 0][results[-1]["token"]]

    def rec(s, token, parent):
        return tables[s][:, 1][token], tables[s][:, 2][token]

    R = prompt_k.shape[0]
    results, arena = run_chained(prompt_k, prompt_v, W_levels, q_steps,
                                 [rec] * (levels - 1),
                                 np.zeros((R, 1), np.float32), k, window,
                                 scale, max_depth)
    return results, backtrack_ids(results), arena
