"""Pins of the oracle's whole-ID generation (CPU only).

What pins what:
* bfloat16 storage rounding: hand-derived halfway and above-halfway cases
  (ties go to the even mantissa, carries reach the exponent), and agreement
  with the input generators' own float32 -> bfloat16 rounding on float32
  values (a separate implementation).
* code table: every entry equals an explicit math.fsum dot product; an
  identity-block projection returns the embedding rows themselves.
* level sizes: one root, then min(B, n * V) beams per step.
* generation: for a vocabulary of 4 and 3 levels, where a code's query, key
  and value are looked up from its level's table, an exhaustive enumeration of
  all 64 IDs with its own minimal attention (no oracle code) ranks them by
  total log-probability; beam search through the oracle with B = 64 returns
  exactly that ranking (IDs and scores), and B = 1 returns the greedy ID.
  The IDs come from following out_parent back through the steps, so the
  enumeration also pins the backtracking.
"""
import math

import numpy as np
import pytest

import workloads as W
from oracle import generate as G

# ------------------------------------------------------------- bf16 rounding


def test_round_to_bf16_hand_cases():
    u = 2.0 ** -7                    # bf16 spacing in [1, 2)
    cases = [
        (1.0 + u / 2, 1.0),                          # halfway, even below
        (1.0 + 3 * u / 2, 1.0 + 2 * u),              # halfway, even above
        (-(1.0 + 3 * u / 2), -(1.0 + 2 * u)),        # the sign only rides along
        (1.0 + u / 2 + 2.0 ** -30, 1.0 + u),         # just above halfway
        (1.0 + u / 2 - 2.0 ** -30, 1.0),             # just below halfway
        (2.0 - u / 2, 2.0),                          # carry into the exponent
        (0.1, 0.10009765625),                        # 0x3DCD
        (3.0, 3.0),
    ]
    got = G.round_to_bf16(np.array([c for c, _ in cases]))
    np.testing.assert_array_equal(got, np.array([w for _, w in cases], np.float32))


def test_round_to_bf16_matches_generator_rounding_on_float32():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-8, 8, 20000))).astype(np.float32)
    np.testing.assert_array_equal(G.round_to_bf16(x.astype(np.float64)), W.bf16_round(x.copy()))


# ---------------------------------------------------------------- code table


def test_code_table_equals_explicit_sums():
    rng = np.random.default_rng(4)
    V, De, H, d = 5, 12, 2, 3
    emb = rng.standard_normal((V, De)).astype(np.float32)
    w = rng.standard_normal((3 * H * d, De)).astype(np.float32)
    for dtype in ("f32", "bf16"):
        t = G.code_table(emb, w, H, d, dtype)
        assert t.shape == (V, 3, H, d)
        flat = t.reshape(V, 3 * H * d)
        for a in range(V):
            for c in range(3 * H * d):
                exact = math.fsum(float(emb[a, i]) * float(w[c, i]) for i in range(De))
                want = np.float32(exact) if dtype == "f32" else G.round_to_bf16(np.array([exact]))[0]
                assert flat[a, c] == want, (dtype, a, c)


def test_code_table_identity_projection_returns_embeddings():
    rng = np.random.default_rng(5)
    H, d = 2, 4
    D = H * d
    emb = W.bf16_round(rng.standard_normal((7, D)).astype(np.float32))
    eye = np.eye(D, dtype=np.float32)
    t = G.code_table(emb, np.concatenate([eye, 2 * eye, -eye]), H, d, "bf16")
    np.testing.assert_array_equal(t[:, 0].reshape(7, D), emb)
    np.testing.assert_array_equal(t[:, 1].reshape(7, D), 2 * emb)
    np.testing.assert_array_equal(t[:, 2].reshape(7, D), -emb)


def test_level_sizes():
    assert G.level_sizes(4, 100) == [(1, 100), (100, 100), (100, 100), (100, 100)]
    assert G.level_sizes(3, 300) == [(1, 256), (256, 300), (300, 300)]
    assert G.level_sizes(3, 16, vocab=4) == [(1, 4), (4, 16), (16, 16)]


# ------------------------------------------------------- exhaustive search
V_T, L_T, H_T, D_T, LP_T = 4, 3, 2, 4, 5


def _world():
    g = np.random.default_rng(21)
    pk = g.standard_normal((1, LP_T, H_T, D_T)).astype(np.float32)
    pv = g.standard_normal((1, LP_T, H_T, D_T)).astype(np.float32)
    q0 = g.standard_normal((1, 1, H_T, D_T)).astype(np.float32)
    Ws = [(g.standard_normal((V_T, H_T * D_T)) * 1.5).astype(np.float32) for _ in range(L_T)]
    tables = [g.standard_normal((V_T, 3, H_T, D_T)).astype(np.float32) for _ in range(L_T - 1)]
    return pk, pv, q0, Ws, tables


def _softmax_attend(q, keys, vals):
    out = []
    for h in range(H_T):
        s = [sum(float(q[h][i]) * float(k[h][i]) for i in range(D_T)) / math.sqrt(D_T) for k in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        tot = sum(e)
        for i in range(D_T):
            out.append(sum(e[j] * float(vals[j][h][i]) for j in range(len(keys))) / tot)
    return out


def _lp(world, prefix):
    pk, pv, q0, Ws, tables = world
    q = q0[0, 0] if not prefix else tables[len(prefix) - 1][prefix[-1], 0]
    keys = [pk[0, j] for j in range(LP_T)] + [tables[i][prefix[i], 1] for i in range(len(prefix))]
    vals = [pv[0, j] for j in range(LP_T)] + [tables[i][prefix[i], 2] for i in range(len(prefix))]
    o = _softmax_attend(q, keys, vals)
    z = [sum(float(Ws[len(prefix)][t][i]) * o[i] for i in range(H_T * D_T)) for t in range(V_T)]
    m = max(z)
    lse = m + math.log(sum(math.exp(x - m) for x in z))
    return [x - lse for x in z]


def _all_ids(world):
    seqs = []
    for a in range(V_T):
        for b in range(V_T):
            for c in range(V_T):
                path = (a, b, c)
                seqs.append((sum(_lp(world, path[:l])[path[l]] for l in range(L_T)), path))
    seqs.sort(key=lambda x: -x[0])
    return seqs


def test_generation_equals_exhaustive_ranking():
    world = _world()
    pk, pv, q0, Ws, tables = world
    want = _all_ids(world)
    results, ids, (ak, av, par) = G.generate(pk, pv, q0, Ws, tables, 64)
    assert [tuple(int(x) for x in row) for row in ids[0]] == [p for _, p in want]
    np.testing.assert_allclose(results[-1]["score"][0], [s for s, _ in want], rtol=0, atol=2e-5)
    # the arena holds one record per kept beam of the first two steps
    assert par.shape[1] >= 4 + 16


def test_generation_with_one_beam_is_greedy():
    world = _world()
    pk, pv, q0, Ws, tables = world
    path = ()
    for _ in range(L_T):
        lp = _lp(world, path)
        path = path + (int(np.argmax(lp)),)
    _, ids, _ = G.generate(pk, pv, q0, Ws, tables, 1)
    assert tuple(int(x) for x in ids[0, 0]) == path


@pytest.mark.parametrize("k", [3, 10])
def test_generation_narrow_beam_keeps_best_extensions(k):
    """With a narrow beam every kept ID is one of the k best one-code
    extensions of the beams kept before it (recomputed by enumeration)."""
    world = _world()
    pk, pv, q0, Ws, tables = world
    results, ids, _ = G.generate(pk, pv, q0, Ws, tables, k)
    kept = [()]
    scores = {(): 0.0}
    for lv in range(L_T):
        cand = []
        for b, p in enumerate(kept):
            lp = _lp(world, p)
            for t in range(V_T):
                cand.append((scores[p] + lp[t], b * V_T + t, p + (t,)))
        cand.sort(key=lambda x: (-x[0], x[1]))
        kl = min(k, len(cand))
        kept = [c[2] for c in cand[:kl]]
        for s, _, p in cand[:kl]:
            scores[p] = s
    assert [tuple(int(x) for x in row) for row in ids[0]] == kept
