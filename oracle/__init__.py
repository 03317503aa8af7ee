"""CPU oracle for the shared-prefix beam-decode step -- TEST INFRASTRUCTURE.

This package is a plain, slow, obviously-correct NumPy implementation of what
the decode step computes.  It is test infrastructure only: the tests, the smoke
check and the benchmark's CPU-baseline leg may import it; the product library
(the HIP kernels behind the C ABI and its Python binding) never does, and it
shares no code, table or helper with that path.

Precision: inputs are float32 arrays (bf16 workloads hold bf16-representable
values); every dot product, softmax and sum is evaluated in float64 and the
results are rounded to float32 where a stored tensor is produced (attention
outputs, candidate scores).  Selections are decided on those float32 scores,
the same precision the GPU path decides in.

Modules:
  trie       append-only record arena with parent indices; ancestor chains
  attention  attention of each beam over the shared prompt plus its own chain,
             in three independent formulations (materialised, explicit mask,
             split prefix/suffix with a log-sum-exp merge)
  beam       codebook logits, log-softmax, prior add, exact top-k, the whole
             decode step, chained decoding, scalar scoring
  linear     linear attention (feature map elu + 1) over the shared prompt
             state plus each beam's records, in three formulations
  generate   whole-ID generation: the q/k/v table of each level's codes,
             every level's step with the chosen codes' records appended in
             between, and the final IDs traced back through the parents
  broadcast  multi-layer broadcast scoring: a Pre-LN Transformer stack over
             one user sequence (keys and values computed once) and many
             single-token candidates, a scalar score each, exact top-k

Pins: every function here is checked in tests/test_oracle_*.py against closed
forms, library special cases, invariants and brute force (see the docstrings
of those tests).  Parity of the absolute values to the pages is unpinned: the
pages print no worked example of this computation.
"""
from .trie import trie_append, chain, TrieError, new_arena
from .attention import (attend_materialized, attend_masked, attend_split,
                        prefix_attn)
from .beam import (codebook_logits, log_softmax, candidate_scores,
                   select_topk, decode_step, scalar_scores, beam_topk,
                   run_chained)
from . import generate, linear, broadcast

__all__ = [
    "trie_append", "chain", "TrieError", "new_arena", "attend_materialized",
    "attend_masked", "attend_split", "prefix_attn", "codebook_logits",
    "log_softmax", "candidate_scores", "select_topk", "decode_step",
    "scalar_scores", "beam_topk", "run_chained", "generate", "linear",
    "broadcast",
]
