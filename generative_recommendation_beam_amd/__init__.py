"""Shared-prefix large-beam decode step for MI355X (gfx950).

The product is the C ABI in include/gr_beam.h, implemented by hand-written HIP
kernels in csrc/ and built into libgrbeam.so; `_lib` is its ctypes binding and
`harness` holds small device-side helpers that allocate tensors and call the
binding (no arithmetic of the method runs in Python).  Build with
`python generative_recommendation_beam_amd/build.py`.
"""
from . import _lib  # noqa: F401  (fails loudly when libgrbeam.so is missing)
from ._lib import (GrError, Shape, Trie, gr_trie_append, gr_prefix_attn,  # noqa: F401
                   gr_beam_topk, gr_decode_step, gr_linear_state, gr_linear_attn,
                   gr_linear_decode_step, gr_code_table, gr_append_codes, gr_generate,
                   gr_attn_workspace_size, gr_topk_workspace_size, gr_decode_workspace_size,
                   gr_generate_workspace_size, status_string,
                   GR_BF16, GR_F32, GR_TOPK_LOG_SOFTMAX, GR_MAX_DEPTH, GR_MAX_K)
