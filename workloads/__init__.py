"""Seeded synthetic inputs for the shared-prefix beam-decode step.

This module draws random numbers and lays them out; it holds none of the
method's arithmetic (no attention, no softmax, no selection).  Both the
oracle-side tests and the HIP-side tests and benchmark take their inputs from
here, so the two implementations always see the same values.

Workload shapes follow the pages:

* Engineering Exploration of Generative Recall (ASGR), §4.2 Custom Beam
  Search: each semantic-ID level has 256 codes; §4.4 Tree-Based Attention:
  beam widths 50 and 100 over a trie of shared prefixes; §4.5 Sliding-Window
  Attention: inputs of about 600 tokens with a window over the most recent
  ones.
* TransRetrieval, Model-based Retrieval and Hardware-aware inference
  optimization: about 4x10^4 candidates per request, each a single query token
  that shares one user KV cache; Recall@2000 gives the 2000 selected.
* OneLA, Abstract: large beams (hundreds of candidates) over one shared prompt
  plus short append-only suffix records.

The pages' datasets are not available, so every value is drawn from a seeded
generator: prompt and record K/V and queries ~ N(0, 1), codebook projections
~ N(0, 0.02), prior beam scores = cumsum(-x^2) with x ~ N(0, 1) (already sorted
descending, like the running log-probabilities of a beam).  bf16 workloads are
rounded to bf16 (round to nearest even) on the host, and both sides consume
those same values.

Draw order for one generator (numpy default_rng(seed)), all float32:
prompt K, prompt V, codebook W (one per level for chained runs), prior x,
trie parents level by level, record k then v level by level, queries.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "Config", "CONFIGS", "HEADLINE", "bf16_round", "make_step_inputs",
    "make_chained_inputs", "StepInputs", "ChainedInputs", "reduced",
    "GEN_CONFIGS", "GenInputs", "make_generate_inputs",
    "XFConfig", "XF_CONFIGS", "XFInputs", "make_xf_inputs",
]


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload.  Symbols: R requests, Lp prompt tokens, window (0 = all),
    H heads of head_dim d, n_in live beams entering the step, k selected
    (beam width out), depth = records per beam chain including its own,
    level_sizes = arena nodes per trie level, vocab = codes per level (256)
    or 1 for scalar scoring."""
    name: str
    index: int          # seed = 1000 + index
    R: int
    Lp: int
    window: int
    H: int
    d: int
    n_in: int
    k: int
    depth: int
    level_sizes: tuple
    dtype: str          # "f32" or "bf16"
    vocab: int
    prior: str          # "zero", "cumsum", "flat", "none"
    steps: int = 1      # >1: chained decode grown by the decode itself

    @property
    def D(self) -> int:
        return self.H * self.d

    @property
    def Lw(self) -> int:
        return self.Lp if self.window <= 0 else min(self.window, self.Lp)

    @property
    def capacity(self) -> int:
        return int(sum(self.level_sizes))

    @property
    def seed(self) -> int:
        return 1000 + self.index


CONFIGS: Dict[str, Config] = {c.name: c for c in [
    # three chained fp32 steps, trie grown by the decode (B = 8 per level)
    Config("tiny_f32_3step", 1, R=1, Lp=64, window=0, H=4, d=32, n_in=1, k=8,
           depth=0, level_sizes=(8, 8), dtype="f32", vocab=256, prior="zero",
           steps=3),
    Config("beam50_p600", 2, R=64, Lp=600, window=0, H=8, d=64, n_in=50, k=50,
           depth=2, level_sizes=(50, 50), dtype="bf16", vocab=256,
           prior="cumsum"),
    # the headline workload: beam 100 over a 600-token prompt, 256 requests
    Config("beam100_p600", 3, R=256, Lp=600, window=0, H=8, d=64, n_in=100,
           k=100, depth=3, level_sizes=(100, 100, 100), dtype="bf16",
           vocab=256, prior="cumsum"),
    Config("broadcast40k_u256", 4, R=1, Lp=256, window=0, H=4, d=32,
           n_in=40000, k=2000, depth=1, level_sizes=(40000,), dtype="bf16",
           vocab=1, prior="none"),
    Config("beam512_p2048_w512", 5, R=32, Lp=2048, window=512, H=16, d=64,
           n_in=512, k=512, depth=4, level_sizes=(256, 512, 512, 512),
           dtype="bf16", vocab=256, prior="cumsum"),
    # long prompts, few requests: the regime of the split prompt window
    Config("long8k_beam100", 8, R=4, Lp=8192, window=0, H=8, d=64, n_in=100,
           k=100, depth=3, level_sizes=(100, 100, 100), dtype="bf16",
           vocab=256, prior="cumsum"),
]}

HEADLINE = "beam100_p600"


def reduced(cfg: Config, **changes) -> Config:
    """A copy of `cfg` with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(cfg, **changes)


def bf16_round(x: np.ndarray, inplace: bool = False) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even) and return
    them as float32 (every result is exactly representable in bf16).  Uses
    torch's float32 -> bfloat16 conversion (round to nearest even) for speed;
    the tests pin it against the bit-level definition."""
    import torch
    if inplace and isinstance(x, np.ndarray) and x.dtype == np.float32 and x.flags.c_contiguous:
        t = torch.from_numpy(x)
        t.copy_(t.to(torch.bfloat16))
        return x
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _maybe_round(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(x, inplace=True) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def _normal(rng, shape, std=1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


@dataclasses.dataclass
class StepInputs:
    """Inputs of one decode step.  Layouts (row-major):
    prompt_k/v [R][Lp][H][d]; W [vocab][D]; prior [R][n_in] or None;
    levels: list of (parent_beam [R][n_l] int32 or None for level 1,
    k [R][n_l][H][d], v [R][n_l][H][d]); q [R][n_in][H][d];
    beam_node [R][n_in] int32 arena node of each live beam (None = prompt
    only).  Nodes are numbered level by level: level l occupies
    [offset_l, offset_l + n_l)."""
    cfg: Config
    prompt_k: np.ndarray
    prompt_v: np.ndarray
    W: np.ndarray
    prior: Optional[np.ndarray]
    levels: List[tuple]
    q: np.ndarray
    beam_node: Optional[np.ndarray]

    def level_offsets(self) -> List[int]:
        offs, o = [], 0
        for (_, k, _) in self.levels:
            offs.append(o)
            o += k.shape[1]
        return offs


def _prior(rng, cfg: Config) -> Optional[np.ndarray]:
    if cfg.prior == "none":
        return None
    if cfg.prior in ("zero", "flat"):
        return np.zeros((cfg.R, cfg.n_in), np.float32)
    x = _normal(rng, (cfg.R, cfg.n_in))
    return np.cumsum(-(x.astype(np.float64) ** 2), axis=1).astype(np.float32)


def make_step_inputs(cfg: Config, seed: Optional[int] = None) -> StepInputs:
    """Draw one single-step workload.  Level sizes are cfg.level_sizes (level
    1 is at most 256 wide in the beam configs); parents of level l >= 2 are
    uniform over level l-1 of the same request (drawn with replacement); the
    live beam b owns node b of the deepest level."""
    assert cfg.steps == 1
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    R, Lp, H, d = cfg.R, cfg.Lp, cfg.H, cfg.d
    pk = _maybe_round(_normal(rng, (R, Lp, H, d)), cfg.dtype)
    pv = _maybe_round(_normal(rng, (R, Lp, H, d)), cfg.dtype)
    W = _maybe_round(_normal(rng, (cfg.vocab, cfg.D), 0.02), cfg.dtype)
    prior = _prior(rng, cfg)
    sizes = list(cfg.level_sizes[:cfg.depth])
    parents = [None]
    for li in range(1, len(sizes)):
        parents.append(rng.integers(0, sizes[li - 1], size=(R, sizes[li]),
                                    dtype=np.int64).astype(np.int32))
    recs = []
    for n in sizes:
        k = _maybe_round(_normal(rng, (R, n, H, d)), cfg.dtype)
        v = _maybe_round(_normal(rng, (R, n, H, d)), cfg.dtype)
        recs.append((k, v))
    q = _maybe_round(_normal(rng, (R, cfg.n_in, H, d)), cfg.dtype)
    levels = [(parents[i], recs[i][0], recs[i][1]) for i in range(len(sizes))]
    if sizes:
        assert sizes[-1] >= cfg.n_in
        off = int(sum(sizes[:-1]))
        beam_node = np.tile(np.arange(off, off + cfg.n_in, dtype=np.int32), (R, 1))
    else:
        beam_node = None
    return StepInputs(cfg, pk, pv, W, prior, levels, q, beam_node)


@dataclasses.dataclass
class ChainedInputs:
    """Inputs of a chained run of cfg.steps decode steps.  Slot-indexed
    draws: q[s] [R][n_s][H][d] is the query of live slot j at step s (n_0 =
    cfg.n_in, later steps cfg.k); rec[s] = (k, v) [R][k][H][d] is the record
    appended for output slot j after step s; W[s] [vocab][D]."""
    cfg: Config
    prompt_k: np.ndarray
    prompt_v: np.ndarray
    W: List[np.ndarray]
    prior0: np.ndarray
    rec: List[tuple]
    q: List[np.ndarray]


def make_chained_inputs(cfg: Config, seed: Optional[int] = None) -> ChainedInputs:
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    R, Lp, H, d = cfg.R, cfg.Lp, cfg.H, cfg.d
    pk = _maybe_round(_normal(rng, (R, Lp, H, d)), cfg.dtype)
    pv = _maybe_round(_normal(rng, (R, Lp, H, d)), cfg.dtype)
    W = [_maybe_round(_normal(rng, (cfg.vocab, cfg.D), 0.02), cfg.dtype)
         for _ in range(cfg.steps)]
    prior0 = np.zeros((R, cfg.n_in), np.float32)
    rec = []
    for _ in range(cfg.steps - 1):
        k = _maybe_round(_normal(rng, (R, cfg.k, H, d)), cfg.dtype)
        v = _maybe_round(_normal(rng, (R, cfg.k, H, d)), cfg.dtype)
        rec.append((k, v))
    q = []
    for s in range(cfg.steps):
        n = cfg.n_in if s == 0 else cfg.k
        q.append(_maybe_round(_normal(rng, (R, n, H, d)), cfg.dtype))
    return ChainedInputs(cfg, pk, pv, W, prior0, rec, q)


# Whole-ID generation: `steps` levels, one root hypothesis per request, beam
# width k; level_sizes are the records appended between the steps (the kept
# beams of every step but the last).
GEN_CONFIGS: Dict[str, Config] = {c.name: c for c in [
    Config("gen_tiny_f32", 6, R=2, Lp=64, window=0, H=4, d=32, n_in=1, k=8,
           depth=0, level_sizes=(8, 8, 8), dtype="f32", vocab=256,
           prior="zero", steps=4),
    # four-level IDs at the headline shape (beam 100, 600-token prompt)
    Config("gen_beam100_p600", 7, R=256, Lp=600, window=0, H=8, d=64, n_in=1,
           k=100, depth=0, level_sizes=(100, 100, 100), dtype="bf16",
           vocab=256, prior="zero", steps=4),
]}


@dataclasses.dataclass
class GenInputs:
    """Inputs of a whole-ID generation.  q0 [R][1][H][d] is the root
    hypothesis's query; W[l] [vocab][D] level l's codebook projection;
    emb[l] [vocab][d_emb] the embeddings of the codes chosen at step l
    (l < steps - 1); w_qkv [3D][d_emb] the query, key and value projections
    stacked by rows."""
    cfg: Config
    d_emb: int
    prompt_k: np.ndarray
    prompt_v: np.ndarray
    q0: np.ndarray
    W: List[np.ndarray]
    emb: List[np.ndarray]
    w_qkv: np.ndarray


def make_generate_inputs(cfg: Config, d_emb: Optional[int] = None,
                         seed: Optional[int] = None, R: Optional[int] = None) -> GenInputs:
    """Draw order: prompt K, prompt V, W per level, embeddings per level,
    w_qkv, q0.  Embeddings ~ N(0, 1) and w_qkv ~ N(0, 1/d_emb) give q, k, v of
    unit variance like the other queries and records.  R overrides the
    request count (fewer requests of the same shape for parity runs)."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    R = cfg.R if R is None else R
    d_emb = cfg.D if d_emb is None else d_emb
    H, d, D = cfg.H, cfg.d, cfg.D
    pk = _maybe_round(_normal(rng, (R, cfg.Lp, H, d)), cfg.dtype)
    pv = _maybe_round(_normal(rng, (R, cfg.Lp, H, d)), cfg.dtype)
    Wl = [_maybe_round(_normal(rng, (cfg.vocab, D), 0.02), cfg.dtype) for _ in range(cfg.steps)]
    emb = [_maybe_round(_normal(rng, (cfg.vocab, d_emb)), cfg.dtype) for _ in range(cfg.steps - 1)]
    w_qkv = _maybe_round(_normal(rng, (3 * D, d_emb), float(d_emb) ** -0.5), cfg.dtype)
    q0 = _maybe_round(_normal(rng, (R, 1, H, d)), cfg.dtype)
    return GenInputs(cfg, d_emb, pk, pv, q0, Wl, emb, w_qkv)


# ---------------------------------------------------------------------------
# Multi-layer broadcast scoring (TransRetrieval, Architecture Overview and
# Model-based Retrieval: an xD-yL Pre-LN Transformer scoring ~4 x 10^4
# single-token candidates per request against one user sequence; 128D-5L is
# the largest configuration the page evaluates, Recall@2000 the cut).

@dataclasses.dataclass(frozen=True)
class XFConfig:
    """R requests, each with Lu user tokens and N candidate tokens of width
    D = 32 * heads, n_layers layers, k kept."""
    name: str
    index: int          # seed = 1000 + index
    R: int
    Lu: int
    N: int
    D: int
    n_layers: int
    k: int

    @property
    def H(self) -> int:
        return self.D // 32

    @property
    def seed(self) -> int:
        return 1000 + self.index


XF_CONFIGS: Dict[str, XFConfig] = {c.name: c for c in [
    XFConfig("xf128d5l_u256_c40k", 9, R=1, Lu=256, N=40000, D=128, n_layers=5, k=2000),
]}


@dataclasses.dataclass
class XFInputs:
    """Tokens and weights of a broadcast-scoring run, both as named arrays
    (layers[l] is a dict: w_qkv [3D][D], b_qkv [3D], w_o [D][D], b_o [D],
    w_1 [2D][D], b_1 [2D], w_2 [D][2D], b_2 [D], ln1_g, ln1_b, ln2_g, ln2_b
    [D]; final lnf_g, lnf_b, w_score [D], b_score) and packed for the
    device: w_mat bf16 values as float32, per layer w_qkv, w_o, w_1, w_2
    (8 D^2 values); w_vec float32, per layer b_qkv, b_o, b_1, b_2, ln1_g,
    ln1_b, ln2_g, ln2_b (11 D values), then lnf_g, lnf_b, w_score, b_score
    (3 D + 1)."""
    cfg: XFConfig
    user: np.ndarray        # [R][Lu][D]
    cand: np.ndarray        # [R][N][D]
    layers: List[dict]
    lnf_g: np.ndarray
    lnf_b: np.ndarray
    w_score: np.ndarray
    b_score: float
    w_mat: np.ndarray
    w_vec: np.ndarray


XF_MAT_KEYS = ("w_qkv", "w_o", "w_1", "w_2")
XF_VEC_KEYS = ("b_qkv", "b_o", "b_1", "b_2", "ln1_g", "ln1_b", "ln2_g", "ln2_b")


def make_xf_inputs(cfg: XFConfig, seed: Optional[int] = None, R: Optional[int] = None,
                   N: Optional[int] = None) -> XFInputs:
    """Draw order: user tokens, candidate tokens, then per layer w_qkv, w_o,
    w_1, w_2, b_qkv, b_o, b_1, b_2, ln1_g, ln1_b, ln2_g, ln2_b, then lnf_g,
    lnf_b, w_score, b_score.  Tokens ~ N(0, 1); weight matrices ~
    N(0, 1/fan_in) (unit-variance activations through the stack); biases ~
    N(0, 0.02); LayerNorm gains 1 + N(0, 0.1), biases N(0, 0.1).  Tokens and
    weight matrices are rounded to bf16.  R and N override the request and
    candidate counts (smaller parity runs draw the same way)."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    R = cfg.R if R is None else R
    N = cfg.N if N is None else N
    D = cfg.D
    user = bf16_round(_normal(rng, (R, cfg.Lu, D)), inplace=True)
    cand = bf16_round(_normal(rng, (R, N, D)), inplace=True)
    layers = []
    for _ in range(cfg.n_layers):
        lp = {}
        lp["w_qkv"] = bf16_round(_normal(rng, (3 * D, D), D ** -0.5), inplace=True)
        lp["w_o"] = bf16_round(_normal(rng, (D, D), D ** -0.5), inplace=True)
        lp["w_1"] = bf16_round(_normal(rng, (2 * D, D), D ** -0.5), inplace=True)
        lp["w_2"] = bf16_round(_normal(rng, (D, 2 * D), (2 * D) ** -0.5), inplace=True)
        lp["b_qkv"] = _normal(rng, (3 * D,), 0.02)
        lp["b_o"] = _normal(rng, (D,), 0.02)
        lp["b_1"] = _normal(rng, (2 * D,), 0.02)
        lp["b_2"] = _normal(rng, (D,), 0.02)
        for nm in ("ln1", "ln2"):
            lp[nm + "_g"] = (1.0 + _normal(rng, (D,), 0.1)).astype(np.float32)
            lp[nm + "_b"] = _normal(rng, (D,), 0.1)
        layers.append(lp)
    lnf_g = (1.0 + _normal(rng, (D,), 0.1)).astype(np.float32)
    lnf_b = _normal(rng, (D,), 0.1)
    w_score = _normal(rng, (D,), D ** -0.5)
    b_score = float(_normal(rng, (1,), 0.02)[0])
    w_mat = np.concatenate([lp[k].reshape(-1) for lp in layers for k in XF_MAT_KEYS]).astype(np.float32)
    w_vec = np.concatenate([lp[k].reshape(-1) for lp in layers for k in XF_VEC_KEYS] +
                           [lnf_g, lnf_b, w_score, np.array([b_score], np.float32)]).astype(np.float32)
    return XFInputs(cfg, user, cand, layers, lnf_g, lnf_b, w_score, b_score, w_mat, w_vec)
