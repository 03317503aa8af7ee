"""GPU parity of whole-ID generation: gr_code_table, gr_append_codes and
gr_generate against the oracle (oracle/generate.py).

* Code tables: every entry of the GPU table within one storage rounding plus
  the fp32 accumulation bound of the oracle's exactly rounded entry, and the
  whole table within the max|err|/RMS bar.
* gr_append_codes: arena records, parent links, node ids and next queries
  bit-exact against the oracle's trie_append of the table rows, over two
  levels; a code outside the vocabulary raises GR_DEVERR_TOKEN_RANGE.
* gr_generate, free running, against the oracle's generation with the same
  code tables: every step's selected scores (bar) and picks (index rule); a
  request is followed while its picks equal the oracle's (the fp32 workload
  is followed through all four levels, with the final IDs exact).
* Teacher-forced chain through the single-step entry points (gr_decode_step,
  gr_append_codes fed the oracle's picks) at the headline shape with fewer
  requests: every level's candidate scores, selected scores and picks against
  the oracle, so levels after a bf16 near-tie are still checked.
* gr_generate equals, bit for bit, the same chain of single-step entry points
  run from the host (its orchestration: buffers, offsets, priors, nodes; in
  bf16 its records read from the code tables against the arena copies), also
  with an arena too large for the table path and at the maximum depth.
* Beam width above 256 (the first step keeps 256, later steps more) and a
  single-level generation.
* One HIP graph holding the tables and the whole generation, replayed three
  times with other work in between: every replay equals the eager result.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import generate as OG
from generative_recommendation_beam_amd import _lib as L
from generative_recommendation_beam_amd import harness as HN
from parity import announce, assert_close, check_index_rule

pytestmark = pytest.mark.gpu

GC = W.GEN_CONFIGS
TINY = GC["gen_tiny_f32"]
MID = W.reduced(GC["gen_beam100_p600"], R=3)
WIDE = W.reduced(GC["gen_beam100_p600"], R=2, Lp=40, H=2, d=32, k=300, steps=3,
                 level_sizes=(256, 300))


def oracle_tables(x):
    cfg = x.cfg
    return [OG.code_table(e, x.w_qkv, cfg.H, cfg.d, cfg.dtype) for e in x.emb]


def setup(cfg, seed=None, tables="oracle", capacity=None):
    x = W.make_generate_inputs(cfg, seed=seed, R=cfg.R)
    g = HN.upload_generate(x, capacity=capacity)
    tabs = oracle_tables(x)
    if g.levels > 1:
        if tables == "oracle":
            g.tables.copy_(HN.to_dev(np.stack(tabs), g.shape.dtype))
        else:
            HN.code_tables(g)
    return x, g, tabs


def ulp_bf16(x):
    """Spacing of bfloat16 values at |x| (x nonzero, normal)."""
    e = np.floor(np.log2(np.abs(x.astype(np.float64))))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("cfg", [TINY, MID], ids=["f32", "bf16"])
def test_code_table(cfg):
    announce(f"gr_code_table {cfg.name} {cfg.dtype}")
    x = W.make_generate_inputs(cfg, R=1)
    g = HN.upload_generate(x)
    HN.code_tables(g)
    torch.cuda.synchronize()
    got = g.tables.float().cpu().numpy()
    want = np.stack(oracle_tables(x))
    assert_close(got, want, cfg.dtype, f"{cfg.name} code table")
    # Entry-wise bound: one rounding to the storage type of a value whose fp32
    # accumulation over d_emb terms is off by at most d_emb 2^-24 sum|e_i w_i|.
    e = np.stack(x.emb).astype(np.float64)
    absdot = np.abs(e) @ np.abs(x.w_qkv.astype(np.float64)).T
    acc_bound = x.d_emb * 2.0 ** -24 * absdot.reshape(want.shape)
    diff = np.abs(got.astype(np.float64) - want)
    if cfg.dtype == "bf16":
        step = ulp_bf16(np.where(want != 0, want, 1.0)) * (want != 0)
    else:
        step = np.abs(want.astype(np.float64)) * 2.0 ** -23
    assert np.all(diff <= step + acc_bound), "an entry is off by more than its rounding and accumulation bound"
    print(f"[info] entries that differ: {int(np.count_nonzero(diff))} of {diff.size}")


def test_append_codes_bit_exact():
    cfg = W.reduced(TINY, R=3, H=2, d=64, dtype="bf16")
    announce("gr_append_codes two levels, bf16")
    rng = np.random.default_rng(44)
    H, d, V, R = cfg.H, cfg.d, 256, cfg.R
    table = W.bf16_round(rng.standard_normal((V, 3, H, d)).astype(np.float32))
    shape = HN.make_shape(R, H, d, cfg.Lp, 0, L.GR_BF16)
    n1, n2 = 5, 9
    cap = n1 + n2 + 2
    ak_d, av_d, par_d, trie = HN.new_arena(shape, cap)
    ak, av, par = oracle.new_arena(R, cap, H, d)
    tab_d = HN.to_dev(table, L.GR_BF16)
    dev_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    tok1 = rng.integers(0, V, (R, n1)).astype(np.int32)
    tok2 = rng.integers(0, V, (R, n2)).astype(np.int32)
    pb2 = rng.integers(0, n1, (R, n2)).astype(np.int32)
    q1 = torch.empty((R, n1, H, d), dtype=torch.bfloat16, device="cuda")
    q2 = torch.empty((R, n2, H, d), dtype=torch.bfloat16, device="cuda")
    node1 = torch.empty((R, n1), dtype=torch.int32, device="cuda")
    node2 = torch.empty((R, n2), dtype=torch.int32, device="cuda")
    L.gr_append_codes(shape, trie, 1, n1, tab_d, V, HN.to_dev_i32(tok1), None, None, 0, q1, node1, dev_err)
    L.gr_append_codes(shape, trie, 1 + n1, n2, tab_d, V, HN.to_dev_i32(tok2), HN.to_dev_i32(pb2), node1, n1, q2,
                      node2, dev_err)
    torch.cuda.synchronize()
    assert int(dev_err.item()) == 0
    ak, av, par, o1 = oracle.trie_append(ak, av, par, 1, table[:, 1][tok1], table[:, 2][tok1], None, None)
    ak, av, par, o2 = oracle.trie_append(ak, av, par, 1 + n1, table[:, 1][tok2], table[:, 2][tok2], pb2, o1)
    np.testing.assert_array_equal(ak_d.float().cpu().numpy(), ak)
    np.testing.assert_array_equal(av_d.float().cpu().numpy(), av)
    np.testing.assert_array_equal(par_d.cpu().numpy(), par)
    np.testing.assert_array_equal(node1.cpu().numpy(), o1)
    np.testing.assert_array_equal(node2.cpu().numpy(), o2)
    np.testing.assert_array_equal(q1.float().cpu().numpy(), table[:, 0][tok1])
    np.testing.assert_array_equal(q2.float().cpu().numpy(), table[:, 0][tok2])
    # a code outside [0, 256) is reported by the kernel's own check
    bad = tok2.copy()
    bad[1, 3] = 256
    L.gr_append_codes(shape, trie, 1 + n1, n2, tab_d, V, HN.to_dev_i32(bad), HN.to_dev_i32(pb2), node1, n1, q2,
                      node2, dev_err)
    torch.cuda.synchronize()
    assert int(dev_err.item()) == L.GR_DEVERR_TOKEN_RANGE


def compare_free_running(cfg, got, res, ids):
    """Level by level while a request's picks equal the oracle's; at the
    level where they first differ, the index rule must hold.  Returns the
    number of levels each request was followed through."""
    R = cfg.R
    live = list(range(R))
    followed = [0] * R
    for lv, ref in enumerate(res):
        if not live:
            break
        gs = got["steps"][lv]
        assert_close(gs["score"][live], ref["score"][live], cfg.dtype, f"{cfg.name} level {lv} scores")
        nxt = []
        for r in live:
            check_index_rule(ref["cand"][r], gs["token"][r], gs["parent"][r])
            followed[r] = lv + 1
            if np.array_equal(gs["token"][r], ref["token"][r]) and np.array_equal(gs["parent"][r], ref["parent"][r]):
                nxt.append(r)
        live = nxt
    for r in live:     # followed through every level: the IDs are exact
        np.testing.assert_array_equal(got["ids"][r], ids[r])
    return followed


@pytest.mark.parametrize("cfg", [TINY, MID, WIDE], ids=["f32", "bf16", "wide"])
def test_generate_free_running(cfg):
    announce(f"gr_generate {cfg.name} R={cfg.R} B={cfg.k} levels={cfg.steps} {cfg.dtype}")
    x, g, tabs = setup(cfg)
    HN.generate(g)
    torch.cuda.synchronize()
    assert int(g.dev_err.item()) == 0
    got = HN.generate_to_host(g)
    res, ids, _ = OG.generate(x.prompt_k, x.prompt_v, x.q0, x.W, tabs, cfg.k)
    followed = compare_free_running(cfg, got, res, ids)
    print(f"[info] levels followed per request: {followed}")
    if cfg is TINY:
        assert followed == [cfg.steps] * cfg.R
    # every final beam's ID traces back through the GPU's own picks
    for r in range(cfg.R):
        for j in range(g.sizes[-1][1]):
            slot = j
            for lv in range(cfg.steps - 1, -1, -1):
                assert got["ids"][r, j, lv] == got["steps"][lv]["token"][r, slot]
                slot = got["steps"][lv]["parent"][r, slot]
            assert slot == 0


def test_generate_teacher_forced_chain():
    """Single-step entry points fed the oracle's picks after every level."""
    cfg = MID
    announce(f"teacher-forced chain {cfg.name} R={cfg.R}")
    x, g, tabs = setup(cfg)
    res, _, _ = OG.generate(x.prompt_k, x.prompt_v, x.q0, x.W, tabs, cfg.k)
    shape, V, R = g.shape, g.vocab, cfg.R
    ws = torch.empty(max(L.gr_decode_workspace_size(shape, n, V, k) for n, k in g.sizes), dtype=torch.uint8,
                     device="cuda")
    q, nodes, prior, base = g.q0, None, None, 0
    for lv, (n, k) in enumerate(g.sizes):
        sc = torch.empty((R, k), device="cuda")
        tk = torch.empty((R, k), dtype=torch.int32, device="cuda")
        pa = torch.empty((R, k), dtype=torch.int32, device="cuda")
        cand = torch.empty((R, n, V), device="cuda")
        L.gr_decode_step(shape, g.prompt_k, g.prompt_v, q, n, g.trie if lv else None, nodes, g.W[lv], V, prior, k,
                         L.GR_TOPK_LOG_SOFTMAX, sc, tk, pa, None, cand, ws, ws.numel(), g.dev_err)
        torch.cuda.synchronize()
        assert int(g.dev_err.item()) == 0
        ref = res[lv]
        assert_close(sc.cpu().numpy(), ref["score"], cfg.dtype, f"forced level {lv} scores")
        assert_close(cand.cpu().numpy(), ref["cand"], cfg.dtype, f"forced level {lv} candidates")
        for r in range(R):
            check_index_rule(ref["cand"][r], tk[r].cpu().numpy(), pa[r].cpu().numpy())
        if lv + 1 < len(g.sizes):
            qn = torch.empty((R, k, cfg.H, cfg.d), dtype=torch.bfloat16, device="cuda")
            nn = torch.empty((R, k), dtype=torch.int32, device="cuda")
            L.gr_append_codes(shape, g.trie, base, k, g.tables[lv], V, HN.to_dev_i32(ref["token"]),
                              HN.to_dev_i32(ref["parent"]) if lv else None, nodes, n, qn, nn, g.dev_err)
            q, nodes, base = qn, nn, base + k
            prior = torch.from_numpy(np.ascontiguousarray(ref["score"])).cuda()


def host_chain(g):
    """The same generation through the single-step entry points, host-driven."""
    shape, V, R = g.shape, g.vocab, g.shape.R
    ws = torch.empty(max(L.gr_decode_workspace_size(shape, n, V, k) for n, k in g.sizes), dtype=torch.uint8,
                     device="cuda")
    q, nodes, prior, base = g.q0, None, None, 0
    steps = []
    for lv, (n, k) in enumerate(g.sizes):
        sc = torch.empty((R, k), device="cuda")
        tk = torch.empty((R, k), dtype=torch.int32, device="cuda")
        pa = torch.empty((R, k), dtype=torch.int32, device="cuda")
        L.gr_decode_step(shape, g.prompt_k, g.prompt_v, q, n, g.trie if lv else None, nodes, g.W[lv], V, prior, k,
                         L.GR_TOPK_LOG_SOFTMAX, sc, tk, pa, None, None, ws, ws.numel(), g.dev_err)
        steps.append((sc, tk, pa))
        if lv + 1 < len(g.sizes):
            qn = torch.empty((R, k, shape.H, shape.head_dim), dtype=g.q0.dtype, device="cuda")
            nn = torch.empty((R, k), dtype=torch.int32, device="cuda")
            L.gr_append_codes(shape, g.trie, base, k, g.tables[lv], V, tk, pa if lv else None, nodes, n, qn, nn,
                              g.dev_err)
            q, nodes, prior, base = qn, nn, sc, base + k
    torch.cuda.synchronize()
    return [tuple(t.cpu().numpy() for t in s) for s in steps]


DEEP_BF16 = W.reduced(GC["gen_tiny_f32"], R=2, Lp=40, H=2, d=64, k=40, steps=L.GR_MAX_DEPTH + 1,
                      level_sizes=(40,) * L.GR_MAX_DEPTH, dtype="bf16")
NARROW = W.reduced(MID, k=20, level_sizes=(20, 20, 20))


# In bf16 with an arena of at most 4096 nodes gr_generate's attention reads the
# chain records from the code tables, while the single-step entry points read
# the copies gr_append_codes wrote into the arena: the two must agree bit for
# bit.  Capacity 5000 keeps gr_generate on the arena (chain pre-pass) path.
@pytest.mark.parametrize("cfg,capacity", [(MID, None), (WIDE, None), (NARROW, None), (MID, 5000), (DEEP_BF16, None)],
                         ids=["bf16", "wide", "bf16_beam20", "bf16_arena5000", "bf16_max_levels"])
def test_generate_equals_host_driven_chain(cfg, capacity):
    announce(f"gr_generate vs host-driven chain {cfg.name} capacity={capacity}")
    x, g, _ = setup(cfg, capacity=capacity)
    chain = host_chain(g)
    HN.generate(g)
    torch.cuda.synchronize()
    assert int(g.dev_err.item()) == 0
    got = HN.generate_to_host(g)
    for lv, (sc, tk, pa) in enumerate(chain):
        np.testing.assert_array_equal(got["steps"][lv]["score"], sc)
        np.testing.assert_array_equal(got["steps"][lv]["token"], tk)
        np.testing.assert_array_equal(got["steps"][lv]["parent"], pa)


def test_generate_single_level():
    cfg = W.reduced(MID, steps=1, level_sizes=())
    announce("gr_generate one level")
    x, g, _ = setup(cfg)
    HN.generate(g)
    torch.cuda.synchronize()
    assert int(g.dev_err.item()) == 0
    got = HN.generate_to_host(g)
    res, ids, _ = OG.generate(x.prompt_k, x.prompt_v, x.q0, x.W, [], cfg.k)
    compare_free_running(cfg, got, res, ids)
    np.testing.assert_array_equal(got["ids"][..., 0], got["steps"][0]["token"])


def test_generate_graph_replays():
    cfg = MID
    announce(f"gr_generate in a HIP graph {cfg.name}")
    x, g, _ = setup(cfg, tables="gpu")
    HN.generate(g)
    torch.cuda.synchronize()
    assert int(g.dev_err.item()) == 0
    eager = HN.generate_to_host(g)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        g.dev_err.zero_()          # a fill kernel, not a memset node
        HN.code_tables(g, s)
        HN.generate(g, s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        g.dev_err.zero_()
        HN.code_tables(g, s)
        HN.generate(g, s)
    torch.cuda.synchronize()
    for rep in range(3):
        g.out_score.fill_(float("nan"))
        g.out_token.fill_(-7)
        g.out_ids.fill_(-7)
        g.tables.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(g.dev_err.item()) == 0
        got = HN.generate_to_host(g)
        for lv in range(g.levels):
            for key in ("score", "token", "parent"):
                np.testing.assert_array_equal(got["steps"][lv][key], eager["steps"][lv][key],
                                              err_msg=f"replay {rep} level {lv} {key}")
        np.testing.assert_array_equal(got["ids"], eager["ids"], err_msg=f"replay {rep} ids")
        # eager work on the default stream between replays
        torch.matmul(torch.randn(256, 256, device="cuda"), torch.randn(256, 256, device="cuda")).sum().item()


def test_generate_maximum_levels():
    """GR_MAX_DEPTH + 1 levels: the last step's chains hold GR_MAX_DEPTH
    records, and the trace-back walks nine levels."""
    cfg = W.reduced(GC["gen_tiny_f32"], R=2, Lp=40, H=2, d=32, k=4, steps=L.GR_MAX_DEPTH + 1,
                    level_sizes=(4,) * L.GR_MAX_DEPTH)
    announce(f"gr_generate {cfg.steps} levels, beam 4, fp32")
    x, g, tabs = setup(cfg)
    assert g.trie.max_depth == L.GR_MAX_DEPTH
    HN.generate(g)
    torch.cuda.synchronize()
    assert int(g.dev_err.item()) == 0
    got = HN.generate_to_host(g)
    res, ids, _ = OG.generate(x.prompt_k, x.prompt_v, x.q0, x.W, tabs, cfg.k)
    followed = compare_free_running(cfg, got, res, ids)
    print(f"[info] levels followed per request: {followed}")
    assert got["ids"].shape == (cfg.R, cfg.k, cfg.steps)
