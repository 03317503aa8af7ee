"""Seeded sweeps of small random shapes against the oracle.

Each case draws its shape from a fixed seed: requests, prompt length and
window (sometimes below 64 keys, which takes the fp32 projection), heads and
head dim (odd D / 32 included, so the scoring ring ends on an odd chunk),
live beams (1..300, one or several beam groups), chain depth (0..5), beam
width (up to the candidate count or GR_MAX_K), dtype and prior.  Every case
is compared in full (attention outputs, all candidate scores, the selected
scores, the index rule and the exact self-consistency of the selection).

The top-k sweep draws requests, candidate counts (up to 120 000, several
selection groups and the final merge), k (1 .. GR_MAX_K), the 256-code or
scalar mode, the log-softmax, priors and exact ties, covering the counting
rank, bucket, bitonic and merge orderings of the selection list.

Twelve of the decode shapes also go through gr_linear_decode_step, and ten
long-prompt shapes (500 .. 3000 keys, few requests and heads, so that the
prompt window is split into runs) through gr_decode_step.
"""
import numpy as np
import pytest
import torch

import workloads as W
from generative_recommendation_beam_amd import _lib as L
from generative_recommendation_beam_amd import harness as HN
from parity import announce
from test_gpu_1_kernels import check_topk_case
from test_gpu_2_decode import compare, oracle_step

pytestmark = pytest.mark.gpu

N_CASES = 24


def random_config(seed: int) -> W.Config:
    rng = np.random.default_rng(5000 + seed)
    dtype = "f32" if seed % 6 == 5 else "bf16"
    H = int(rng.integers(1, 5))
    d = int(rng.choice([32, 64]))
    R = int(rng.integers(1, 4))
    Lp = int(rng.choice([1, 7, 40, 65, 130, 257]))
    window = int(rng.choice([0, 0, 1, 33, 64, 100])) if Lp > 1 else 0
    n_in = int(rng.choice([1, 5, 31, 32, 33, 64, 100, 129, 200, 300]))
    depth = int(rng.integers(0, 6))
    if depth == 0 and n_in > 256:
        n_in = 256                        # a prompt-only step has at most one level of beams
    sizes = []
    for li in range(depth):
        sizes.append(n_in if li == depth - 1 else int(rng.integers(1, 2 * n_in + 1)))
    sizes = tuple(sizes)
    if sizes:
        sizes = tuple(min(s, 256) if i == 0 and len(sizes) > 1 else s for i, s in enumerate(sizes))
    cand = n_in * 256
    k = int(min(cand, L.GR_MAX_K, rng.choice([1, 8, 50, 100, 257, 700])))
    prior = str(rng.choice(["cumsum", "flat", "zero"]))
    return W.reduced(W.CONFIGS["beam100_p600"], R=R, Lp=Lp, window=window, H=H, d=d, n_in=n_in, k=k,
                     depth=depth, level_sizes=sizes, dtype=dtype, prior=prior)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_decode_random_shapes(seed):
    cfg = random_config(seed)
    announce(f"gr_decode_step random case {seed}: R={cfg.R} Lp={cfg.Lp} window={cfg.window} H={cfg.H} "
             f"d={cfg.d} n_in={cfg.n_in} k={cfg.k} levels={cfg.level_sizes} {cfg.dtype} prior={cfg.prior}")
    x = W.make_step_inputs(cfg, seed=9000 + seed)
    ds = HN.upload_step(x)
    buf = HN.decode_buffers(ds, debug_outputs=True)
    HN.decode_step(ds, buf)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == 0
    got = HN.results_to_host(buf)
    ref = oracle_step(x)
    compare(cfg, got, ref, list(range(cfg.R)), f"random {seed}")


def random_topk_case(seed: int) -> dict:
    rng = np.random.default_rng(7000 + seed)
    vocab = int(rng.choice([1, 256, 256]))
    R = int(rng.integers(1, 4))
    n_in = int(rng.choice([1, 3, 40, 129, 300, 470])) if vocab == 256 else int(rng.choice([5, 700, 9000, 40000, 120000]))
    k = int(min(n_in * vocab, L.GR_MAX_K, rng.choice([1, 7, 100, 256, 300, 1000, 2048])))
    lsm = vocab == 256 and bool(rng.integers(0, 2))
    quant = not lsm and bool(rng.integers(0, 2))
    prior = str(rng.choice(["cumsum", "flat", "int", "none"]))
    return dict(R=R, n_in=n_in, vocab=vocab, k=k, lsm=lsm, prior=prior, quant=quant)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_topk_random_shapes(seed):
    c = random_topk_case(seed)
    announce(f"gr_beam_topk random case {seed}: {c}")
    check_topk_case(f"random {seed}", c, np.random.default_rng(8000 + seed))


@pytest.mark.parametrize("seed", range(12))
def test_linear_decode_random_shapes(seed):
    """The same random shapes through gr_linear_decode_step."""
    from oracle import linear as LA
    from test_gpu_5_linear import arena_of
    cfg = random_config(seed)
    announce(f"gr_linear_decode_step random case {seed}: R={cfg.R} Lp={cfg.Lp} window={cfg.window} H={cfg.H} "
             f"d={cfg.d} n_in={cfg.n_in} k={cfg.k} levels={cfg.level_sizes} {cfg.dtype}")
    x = W.make_step_inputs(cfg, seed=9000 + seed)
    ds = HN.upload_step(x)
    S, z = HN.linear_state(ds)
    buf = HN.decode_buffers(ds, debug_outputs=True)
    HN.linear_decode_step(ds, buf, S, z)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == 0
    got = HN.results_to_host(buf)
    ak, av, par = arena_of(x)
    ref = LA.linear_decode_step(x.prompt_k, x.prompt_v, x.q, par, ak, av, x.beam_node, x.W, x.prior, cfg.k,
                                window=cfg.window)
    compare(cfg, got, ref, list(range(cfg.R)), f"linear random {seed}")


def random_long_config(seed: int) -> W.Config:
    """Few requests and heads with prompts of 500 .. 3000 keys: the prompt
    window is split into runs (bf16)."""
    rng = np.random.default_rng(6000 + seed)
    R = int(rng.integers(1, 3))
    H = int(rng.integers(1, 4))
    d = int(rng.choice([32, 64]))
    Lp = int(rng.integers(500, 3001))
    window = int(rng.choice([0, 0, int(rng.integers(300, Lp))]))
    n_in = int(rng.choice([7, 50, 100, 129]))
    depth = int(rng.integers(0, 4))
    sizes = tuple(n_in for _ in range(depth))
    k = int(min(n_in * 256, rng.choice([10, 100, 300])))
    return W.reduced(W.CONFIGS["beam100_p600"], R=R, Lp=Lp, window=window, H=H, d=d, n_in=n_in, k=k,
                     depth=depth, level_sizes=sizes, dtype="bf16", prior="cumsum")


@pytest.mark.parametrize("seed", range(10))
def test_split_window_random_shapes(seed):
    cfg = random_long_config(seed)
    announce(f"gr_decode_step split-window random case {seed}: R={cfg.R} Lp={cfg.Lp} window={cfg.window} "
             f"H={cfg.H} d={cfg.d} n_in={cfg.n_in} k={cfg.k} depth={cfg.depth}")
    x = W.make_step_inputs(cfg, seed=9500 + seed)
    ds = HN.upload_step(x)
    buf = HN.decode_buffers(ds, debug_outputs=True)
    HN.decode_step(ds, buf)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == 0
    got = HN.results_to_host(buf)
    compare(cfg, got, oracle_step(x), list(range(cfg.R)), f"split random {seed}")
