"""gr_decode_step_noalloc: the decode step on the library's static device
scratch, for callers that cannot allocate.

* Host side (CPU): a step whose workspace exceeds the static buffer is
  refused with GR_ERR_SCRATCH_LIMIT before any device call.
* GPU: two calls in a row through the C ABI, the second with a smaller
  input than the first, each equal bit for bit to gr_decode_step with a
  caller workspace on the same inputs (scores, tokens, parents, attention
  outputs, candidate scores); no device error bits.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from generative_recommendation_beam_amd import _lib as L
from generative_recommendation_beam_amd import harness as HN

FAKE = 0x10000


def test_oversized_step_is_refused_before_any_device_call():
    big = L.Shape(R=1024, H=8, head_dim=64, prompt_len=600, window=0, dtype=L.GR_BF16, scale=0.0)
    assert L.gr_decode_workspace_size(big, 100, 256, 100) > L.GR_NOALLOC_SCRATCH_BYTES
    tr = L.Trie(k=FAKE, v=FAKE, parent=FAKE, capacity=300, max_depth=8)
    st = L._lib.gr_decode_step_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, 100, ctypes.byref(tr), FAKE, FAKE,
                                       256, FAKE, 100, L.GR_TOPK_LOG_SOFTMAX, FAKE, FAKE, FAKE, None, None,
                                       FAKE, None)
    assert st == L.GR_ERR_SCRATCH_LIMIT
    assert "static" in L.status_string(st)
    # the full-size headline step fits
    head = L.Shape(R=256, H=8, head_dim=64, prompt_len=600, window=0, dtype=L.GR_BF16, scale=0.0)
    assert L.gr_decode_workspace_size(head, 100, 256, 100) <= L.GR_NOALLOC_SCRATCH_BYTES


def _run_both(cfg):
    x = W.make_step_inputs(cfg)
    ds = HN.upload_step(x)
    ref = HN.decode_buffers(ds, debug_outputs=True)
    HN.decode_step(ds, ref)
    got = HN.decode_buffers(ds, debug_outputs=True)
    got.ws = None
    print(f"noalloc: {cfg.name} R={cfg.R} Lp={cfg.Lp} beams={cfg.n_in} k={cfg.k}", flush=True)
    L.gr_decode_step_noalloc(ds.shape, ds.prompt_k, ds.prompt_v, ds.q, ds.n_beams, ds.trie, ds.beam_node, ds.W,
                             ds.vocab, ds.prior, ds.k, ds.flags, got.score, got.token, got.parent, got.attn,
                             got.cand, ds.dev_err)
    torch.cuda.synchronize()
    assert int(ds.dev_err.item()) == 0
    a, b = HN.results_to_host(ref), HN.results_to_host(got)
    for key in ("score", "token", "parent", "attn", "cand"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.gpu
def test_noalloc_matches_workspace_call_twice_second_smaller():
    first = W.reduced(W.CONFIGS["beam100_p600"], R=24)
    second = W.reduced(W.CONFIGS["beam50_p600"], R=3, Lp=131, level_sizes=(41, 50))
    _run_both(first)
    _run_both(second)
