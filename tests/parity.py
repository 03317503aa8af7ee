"""Comparison rules between the HIP path and the oracle.

* Floating-point tensors (attention outputs, candidate scores, selected
  scores): max |gpu - oracle| / RMS(oracle) <= 2e-2 for bf16 workloads
  (bf16 inputs, fp32 accumulation) and <= 1e-5 for the fp32 workload.
* Selected indices (token, parent): let c_(k+1) be the oracle's (k+1)-th
  candidate score.  (i) every oracle pick scoring above c_(k+1) + 1e-3 is in
  the GPU selection with the same (parent, token); (ii) no GPU pick has an
  oracle score below c_(k+1) - 1e-3; (iii) consecutive GPU output slots are in
  the oracle's order whenever their oracle scores differ by more than 1e-3.
* Self-consistency (exact): the GPU selection equals the exact order of the
  GPU's own candidate scores (score desc, flat index asc).
"""
from __future__ import annotations

import sys

import numpy as np

TOL = {"bf16": 2e-2, "f32": 1e-5}
GAP = 1e-3


def announce(msg: str) -> None:
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(np.asarray(gpu, np.float64) - ref))) / max(rms, 1e-30)


def assert_close(gpu, ref, dtype: str, what: str) -> float:
    e = rel_err(gpu, ref)
    print(f"[err] {what}: max|err|/RMS = {e:.3e} (bar {TOL[dtype]:.0e})", file=sys.stderr, flush=True)
    assert e <= TOL[dtype], f"{what}: max|err|/RMS = {e:.3e} > {TOL[dtype]:.0e}"
    return e


def exact_order(c: np.ndarray, k: int):
    """(parent, token) of the k best of one request's candidates c [n][V]."""
    n, V = c.shape
    flat = c.reshape(-1)
    order = np.lexsort((np.arange(flat.size), -flat))[:k]
    return order // V, order % V


def check_self_consistent(cand: np.ndarray, token: np.ndarray, parent: np.ndarray) -> None:
    """Per request: the GPU picks are exactly the top-k of its own scores."""
    R, k = token.shape
    for r in range(R):
        p, t = exact_order(cand[r], k)
        np.testing.assert_array_equal(parent[r], p, err_msg=f"request {r}: parent")
        np.testing.assert_array_equal(token[r], t, err_msg=f"request {r}: token")


def check_index_rule(oracle_cand: np.ndarray, token: np.ndarray, parent: np.ndarray, gap: float = GAP):
    """The index rule above for one request; returns the number of picks that
    sit inside the near-tie band (informational)."""
    n, V = oracle_cand.shape
    k = token.shape[0]
    flat = oracle_cand.reshape(-1).astype(np.float64)
    order = np.lexsort((np.arange(flat.size), -flat))
    ck1 = flat[order[k]] if flat.size > k else -np.inf
    gpu_f = parent.astype(np.int64) * V + token.astype(np.int64)
    gpu_set = set(gpu_f.tolist())
    assert len(gpu_set) == k, "duplicate picks"
    band = 0
    for j in range(k):
        f = int(order[j])
        if flat[f] > ck1 + gap:
            assert f in gpu_set, f"oracle pick {j} (f={f}, c={flat[f]:.6f}) missing; c_k+1={ck1:.6f}"
        else:
            band += 1
    for f in gpu_f.tolist():
        assert flat[f] >= ck1 - gap, f"GPU pick f={f} has oracle score {flat[f]:.6f} < c_k+1 - gap"
    cs = flat[gpu_f]
    for j in range(k - 1):
        if abs(cs[j] - cs[j + 1]) > gap:
            assert cs[j] > cs[j + 1], f"slots {j},{j+1} out of order: {cs[j]:.6f} vs {cs[j+1]:.6f}"
    return band
