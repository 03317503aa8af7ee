"""Pins of the oracle's scoring, selection and whole-search logic (CPU only).

What pins what:
* log-softmax: probabilities sum to one; shifting the logits changes nothing;
  the log-softmax over the 256 codes of the current level equals a softmax
  over an n x 256 vocabulary with the other levels masked out (Engineering
  Exploration of Generative Recall, §4.2: only the current position's 256
  codes are valid); hand-derived fixture.
* top-k: equals Python's own sort on (score desc, flat index asc), including
  exact ties; k = n returns the whole ranking; the defining property (no
  unselected candidate beats a selected one) holds; hand-derived fixture.
* codebook logits / scalar scores: one-hot projections pick single components.
* the whole search: exhaustive enumeration of every sequence of a tiny trie
  (vocab 4, 3 levels), computed with its own minimal attention (no oracle
  code), equals beam search through the oracle's arena when the beam keeps
  every prefix, and greedy decoding when the beam is 1.
* trie append: records land at base + j, parents map through the previous
  beams, existing records are never touched (OneLA, Abstract), bad input
  raises.
* memory accounting of §4.4: the arena holds sum_l n_l records while a
  materialised cache holds B (Lp + delta) rows per head.
"""
import json
import math
import os
import zlib
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(x):
    if isinstance(x, str):
        if x.startswith("ln"):
            return math.log(float(Fraction(x[2:].strip("()"))))
        return float(Fraction(x))
    return float(x)


# ---------------------------------------------------------------- log-softmax
def test_log_softmax_normalised_and_shift_invariant():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((4, 5, 256)) * 3
    lp = oracle.log_softmax(z)
    np.testing.assert_allclose(np.exp(lp).sum(-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(oracle.log_softmax(z + 123.25), lp, atol=1e-12)
    assert np.all(lp <= 0)


def test_level_slice_equals_masked_full_vocab():
    rng = np.random.default_rng(4)
    n_levels, V = 4, 256
    z_full = rng.standard_normal((3, n_levels * V))
    for lvl in range(n_levels):
        masked = np.full_like(z_full, -np.inf)
        masked[:, lvl * V:(lvl + 1) * V] = z_full[:, lvl * V:(lvl + 1) * V]
        with np.errstate(divide="ignore", invalid="ignore"):
            m = masked.max(-1, keepdims=True)
            full_lp = masked - m - np.log(np.exp(masked - m).sum(-1, keepdims=True))
        np.testing.assert_allclose(oracle.log_softmax(z_full[:, lvl * V:(lvl + 1) * V]),
                                   full_lp[:, lvl * V:(lvl + 1) * V], atol=1e-12)


def test_golden_log_softmax():
    with open(os.path.join(GOLDEN, "select_worked.json")) as f:
        g = json.load(f)["log_softmax"]
    z = np.array([_num(e) for e in g["z"]])
    np.testing.assert_allclose(oracle.log_softmax(z), [_num(e) for e in g["lp"]],
                               rtol=1e-14)


# -------------------------------------------------------------------- top-k
def _python_sort(c, k):
    n_in, V = c.shape
    items = sorted(((-float(c[b, t]), b * V + t) for b in range(n_in) for t in range(V)))
    items = items[:k]
    return ([-s for s, _ in items], [f % V for _, f in items], [f // V for _, f in items])


@pytest.mark.parametrize("n_in,V,k,quant", [(7, 16, 5, None), (7, 16, 112, None),
                                            (9, 8, 20, 0.5), (3, 256, 256, 0.25),
                                            (5, 1, 3, 1.0), (40, 1, 17, None)])
def test_select_matches_python_sort(n_in, V, k, quant):
    rng = np.random.default_rng(n_in * 100 + k)
    c = rng.standard_normal((n_in, V)).astype(np.float32)
    if quant:
        c = (np.round(c / quant) * quant).astype(np.float32)   # many exact ties
    s, t, p = oracle.select_topk(c, k)
    rs, rt, rp = _python_sort(c, k)
    np.testing.assert_array_equal(s, np.array(rs, np.float32))
    np.testing.assert_array_equal(t, rt)
    np.testing.assert_array_equal(p, rp)
    # defining property: nothing unselected ranks above the last selected
    chosen = set(zip(p.tolist(), t.tolist()))
    last = (-float(s[-1]), int(p[-1]) * V + int(t[-1]))
    for b in range(n_in):
        for tt in range(V):
            if (b, tt) not in chosen:
                assert (-float(c[b, tt]), b * V + tt) > last


def test_golden_select():
    with open(os.path.join(GOLDEN, "select_worked.json")) as f:
        g = json.load(f)["topk_no_log_softmax"]
    res = oracle.beam_topk(np.array([g["logits"]], np.float32),
                           np.array([g["prior"]], np.float32), g["k"],
                           use_log_softmax=False)
    np.testing.assert_array_equal(res["score"][0], g["score"])
    np.testing.assert_array_equal(res["token"][0], g["token"])
    np.testing.assert_array_equal(res["parent"][0], g["parent"])


def test_onehot_projection_and_scalar_scores():
    rng = np.random.default_rng(5)
    o = rng.standard_normal((2, 3, 8)).astype(np.float32)
    Wm = np.zeros((4, 8), np.float32)
    picks = [5, 0, 7, 2]
    for t, i in enumerate(picks):
        Wm[t, i] = 1.0
    z = oracle.codebook_logits(o, Wm)
    np.testing.assert_array_equal(z, o[..., picks].astype(np.float64))
    w = np.zeros(8, np.float32)
    w[3] = 1.0
    np.testing.assert_array_equal(oracle.scalar_scores(o, w), o[..., 3])
    prior = rng.standard_normal((2, 3)).astype(np.float32)
    np.testing.assert_allclose(oracle.scalar_scores(o, w, prior),
                               o[..., 3].astype(np.float64) + prior, rtol=1e-7)


# ------------------------------------------------------- exhaustive search
V_T, L_T, H_T, D_T, LP_T = 4, 3, 2, 4, 5


def _path_rng(tag, path):
    return np.random.default_rng(zlib.crc32(repr((tag, tuple(path))).encode()))


def _qfun(path):
    return _path_rng("q", path).standard_normal((H_T, D_T)).astype(np.float32)


def _recfun(path):
    g = _path_rng("kv", path)
    return (g.standard_normal((H_T, D_T)).astype(np.float32),
            g.standard_normal((H_T, D_T)).astype(np.float32))


def _tiny_world():
    g = np.random.default_rng(11)
    pk = g.standard_normal((1, LP_T, H_T, D_T)).astype(np.float32)
    pv = g.standard_normal((1, LP_T, H_T, D_T)).astype(np.float32)
    Ws = [(g.standard_normal((V_T, H_T * D_T)) * 1.5).astype(np.float32)
          for _ in range(L_T)]
    return pk, pv, Ws


def _own_attention(q, keys, vals):
    """Minimal softmax attention with explicit loops, independent of oracle/."""
    out = []
    for h in range(H_T):
        s = [sum(float(q[h][i]) * float(k[h][i]) for i in range(D_T)) / math.sqrt(D_T)
             for k in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        tot = sum(e)
        for i in range(D_T):
            out.append(sum(e[j] * float(vals[j][h][i]) for j in range(len(keys))) / tot)
    return out


def _lp_at(pk, pv, Ws, prefix):
    keys = [pk[0, j] for j in range(LP_T)] + [_recfun(prefix[:i + 1])[0] for i in range(len(prefix))]
    vals = [pv[0, j] for j in range(LP_T)] + [_recfun(prefix[:i + 1])[1] for i in range(len(prefix))]
    o = _own_attention(_qfun(prefix), keys, vals)
    z = [sum(float(Ws[len(prefix)][t][i]) * o[i] for i in range(H_T * D_T)) for t in range(V_T)]
    m = max(z)
    lse = m + math.log(sum(math.exp(x - m) for x in z))
    return [x - lse for x in z]


def _enumerate_all(pk, pv, Ws):
    seqs = []
    for a in range(V_T):
        for b in range(V_T):
            for c in range(V_T):
                path = (a, b, c)
                tot = sum(_lp_at(pk, pv, Ws, path[:l])[path[l]] for l in range(L_T))
                seqs.append((tot, path))
    seqs.sort(key=lambda x: -x[0])
    return seqs


def _beam_search(pk, pv, Ws, k):
    paths = {0: [()]}

    def qsteps(s, results):
        if s > 0:
            res = results[-1]
            prev = paths[s - 1]
            paths[s] = [prev[int(p)] + (int(t),) for t, p in zip(res["token"][0], res["parent"][0])]
        return np.stack([_qfun(p) for p in paths[s]])[None]

    def recs(s, token, parent):
        prev = paths[s]
        new = [prev[int(p)] + (int(t),) for t, p in zip(token[0], parent[0])]
        kv = [_recfun(p) for p in new]
        return (np.stack([a for a, _ in kv])[None], np.stack([b for _, b in kv])[None])

    results, arena = oracle.run_chained(pk, pv, Ws, qsteps, [recs] * (L_T - 1),
                                        np.zeros((1, 1), np.float32), k)
    final = results[-1]
    prev = paths[L_T - 1]
    out = [prev[int(p)] + (int(t),) for t, p in zip(final["token"][0], final["parent"][0])]
    return out, final["score"][0], results, arena


@pytest.mark.parametrize("k", [16, 64])
def test_beam_search_equals_exhaustive_when_beam_keeps_all_prefixes(k):
    pk, pv, Ws = _tiny_world()
    allseq = _enumerate_all(pk, pv, Ws)
    got, score, _, _ = _beam_search(pk, pv, Ws, k)
    want = allseq[:k]
    assert [tuple(p) for p in got] == [p for _, p in want]
    np.testing.assert_allclose(score, [s for s, _ in want], rtol=0, atol=2e-5)


def test_beam_one_is_greedy():
    pk, pv, Ws = _tiny_world()
    path = ()
    for _ in range(L_T):
        lp = _lp_at(pk, pv, Ws, path)
        path = path + (int(np.argmax(lp)),)
    got, score, _, _ = _beam_search(pk, pv, Ws, 1)
    assert tuple(got[0]) == path


def test_final_score_is_sum_along_trie_chain():
    pk, pv, Ws = _tiny_world()
    got, score, results, (ak, av, par) = _beam_search(pk, pv, Ws, 16)
    for j, path in enumerate(got):
        tot = sum(_lp_at(pk, pv, Ws, tuple(path[:l]))[path[l]] for l in range(L_T))
        assert abs(tot - float(score[j])) < 2e-5
    # the arena chain of each second-level node reproduces its path's records
    last_nodes = np.arange(4, 4 + 16)
    for n in last_nodes:
        ch = oracle.chain(par[0], int(n), 8)
        assert len(ch) == 2 and ch[0] < 4


# ------------------------------------------------------------- trie append
def test_trie_append_semantics_and_append_only():
    rng = np.random.default_rng(9)
    R, H, d = 2, 2, 3
    ak, av, par = oracle.new_arena(R, 10, H, d)
    k1 = rng.standard_normal((R, 3, H, d)).astype(np.float32)
    v1 = rng.standard_normal((R, 3, H, d)).astype(np.float32)
    ak, av, par, nodes1 = oracle.trie_append(ak, av, par, 0, k1, v1)
    np.testing.assert_array_equal(nodes1, [[0, 1, 2]] * R)
    assert np.all(par[:, :3] == -1)
    snap = (ak.copy(), av.copy(), par.copy())
    k2 = rng.standard_normal((R, 4, H, d)).astype(np.float32)
    v2 = rng.standard_normal((R, 4, H, d)).astype(np.float32)
    pb = np.array([[2, 0, 0, 1], [1, 1, 2, 0]], np.int32)
    ak, av, par, nodes2 = oracle.trie_append(ak, av, par, 3, k2, v2, pb, nodes1)
    np.testing.assert_array_equal(nodes2, [[3, 4, 5, 6]] * R)
    np.testing.assert_array_equal(par[:, 3:7], np.take_along_axis(nodes1, pb, 1))
    np.testing.assert_array_equal(ak[:, 3:7], k2)
    np.testing.assert_array_equal(av[:, 3:7], v2)
    # nothing already stored moved or changed
    np.testing.assert_array_equal(ak[:, :3], snap[0][:, :3])
    np.testing.assert_array_equal(av[:, :3], snap[1][:, :3])
    np.testing.assert_array_equal(par[:, :3], snap[2][:, :3])
    with pytest.raises(oracle.TrieError):
        oracle.trie_append(ak, av, par, 8, k2, v2, pb, nodes1)          # capacity
    with pytest.raises(oracle.TrieError):
        oracle.trie_append(ak, av, par, 7, k2[:, :2], v2[:, :2],
                           np.array([[0, 3], [0, 0]], np.int32), nodes1)  # beam index
    with pytest.raises(oracle.TrieError):
        oracle.trie_append(ak, av, par, 0, k2[:, :1], v2[:, :1],
                           np.zeros((R, 1), np.int32), nodes2)          # parent >= own id


def test_memory_accounting_of_shared_prefix_storage():
    """§4.4: a trie stores each shared prefix record once.  For the beam-100
    workload the arena holds 300 records per request where a materialised
    per-beam cache holds 100 x (600 + 3) rows."""
    cfg = W.CONFIGS["beam100_p600"]
    arena_rows = sum(cfg.level_sizes)
    prompt_rows = cfg.Lp
    materialised_rows = cfg.n_in * (cfg.Lp + cfg.depth)
    shared_rows = prompt_rows + arena_rows
    assert arena_rows == 300 and materialised_rows == 60300
    assert shared_rows / materialised_rows < 0.02


# ----------------------------------------------------------------- workloads
def test_workload_generators_are_seeded_and_shaped():
    cfg = W.reduced(W.CONFIGS["beam100_p600"], R=3, Lp=11, n_in=6, level_sizes=(4, 6, 6))
    a, b = W.make_step_inputs(cfg), W.make_step_inputs(cfg)
    np.testing.assert_array_equal(a.prompt_k, b.prompt_k)
    np.testing.assert_array_equal(a.q, b.q)
    assert a.prompt_k.shape == (3, 11, cfg.H, cfg.d) and a.W.shape == (256, cfg.D)
    assert np.array_equal(W.bf16_round(a.prompt_k), a.prompt_k)
    assert np.all(np.diff(a.prior, axis=1) <= 0)
    for li, (pb, k, v) in enumerate(a.levels):
        if li == 0:
            assert pb is None
        else:
            assert pb.min() >= 0 and pb.max() < cfg.level_sizes[li - 1]
    np.testing.assert_array_equal(a.beam_node[0], np.arange(10, 16))
    x = np.array([1.0, 1.00390625, 1.005859375, -3.1415927, 65504.0], np.float32)
    np.testing.assert_array_equal(W.bf16_round(x), [1.0, 1.0, 1.0078125, -3.140625, 65536.0])
    # bit-level definition of round-to-nearest-even on the upper 16 bits
    y = np.random.default_rng(1).standard_normal(100000).astype(np.float32) * 10
    u = y.view(np.uint32).astype(np.uint64)
    ref = ((u + ((u >> 16) & 1) + 0x7FFF) & 0xFFFF0000).astype(np.uint32).view(np.float32)
    np.testing.assert_array_equal(W.bf16_round(y), ref)
