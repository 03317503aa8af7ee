"""Device-side harness around the C ABI: uploads host arrays, builds the trie
arena with gr_trie_append, allocates outputs and workspace, and calls
gr_prefix_attn / gr_beam_topk / gr_decode_step through the binding.

No arithmetic of the method runs here; every step of the decode runs in the
HIP kernels.  Inputs are host arrays (numpy, float32 values that the bf16
workloads already hold in bf16-representable form) in the C ABI's layouts.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

from . import _lib as L

_TORCH = {L.GR_BF16: torch.bfloat16, L.GR_F32: torch.float32}


def dtype_code(name: str) -> int:
    return {"bf16": L.GR_BF16, "f32": L.GR_F32}[name]


def to_dev(a: np.ndarray, dtype_code_: int, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device=device, dtype=_TORCH[dtype_code_]).contiguous()


def to_dev_i32(a: Optional[np.ndarray], device="cuda") -> Optional[torch.Tensor]:
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


@dataclasses.dataclass
class DeviceStep:
    shape: L.Shape
    prompt_k: torch.Tensor
    prompt_v: torch.Tensor
    q: torch.Tensor
    W: torch.Tensor
    prior: Optional[torch.Tensor]
    arena_k: Optional[torch.Tensor]
    arena_v: Optional[torch.Tensor]
    parent: Optional[torch.Tensor]
    trie: Optional[L.Trie]
    beam_node: Optional[torch.Tensor]
    n_beams: int
    k: int
    vocab: int
    flags: int
    dev_err: torch.Tensor

    @property
    def R(self) -> int:
        return self.shape.R

    @property
    def D(self) -> int:
        return self.shape.H * self.shape.head_dim


def make_shape(R, H, hd, Lp, window, dtype: int, scale=0.0) -> L.Shape:
    return L.Shape(R=R, H=H, head_dim=hd, prompt_len=Lp, window=window, dtype=dtype, scale=scale)


def new_arena(shape: L.Shape, capacity: int, max_depth: int = L.GR_MAX_DEPTH, device="cuda"):
    R, H, hd = shape.R, shape.H, shape.head_dim
    ak = torch.zeros((R, capacity, H, hd), dtype=_TORCH[shape.dtype], device=device)
    av = torch.zeros_like(ak)
    par = torch.full((R, capacity), -1, dtype=torch.int32, device=device)
    trie = L.Trie(k=ak.data_ptr(), v=av.data_ptr(), parent=par.data_ptr(), capacity=capacity,
                  max_depth=max_depth)
    trie._tensors = (ak, av, par)    # the struct holds raw pointers: keep the storage alive
    return ak, av, par, trie


def append_level(shape, trie, base, k_new, v_new, parent_beam, prev_nodes, dev_err, device="cuda"):
    """gr_trie_append of one level; returns the node ids (device int32)."""
    kn = to_dev(k_new, shape.dtype, device)
    vn = to_dev(v_new, shape.dtype, device)
    pb = to_dev_i32(parent_beam, device)
    n_new = kn.shape[1]
    nodes = torch.empty((shape.R, n_new), dtype=torch.int32, device=device)
    n_prev = 0 if prev_nodes is None else prev_nodes.shape[1]
    L.gr_trie_append(shape, trie, base, n_new, kn, vn, pb, prev_nodes, n_prev, nodes, dev_err)
    return nodes


def upload_step(x, window=None, device="cuda", max_depth: int = L.GR_MAX_DEPTH, flags=None,
                capacity: Optional[int] = None) -> DeviceStep:
    """Upload one single-step workload (an object with the fields of
    workloads.StepInputs) and build its arena level by level through
    gr_trie_append.  `capacity` (default: exactly the appended records)
    sizes the arena; extra slots stay unused."""
    cfg = x.cfg
    dt = dtype_code(cfg.dtype)
    R, Lp, H, hd = x.prompt_k.shape
    shape = make_shape(R, H, hd, Lp, cfg.window if window is None else window, dt)
    dev_err = torch.zeros(1, dtype=torch.int32, device=device)
    pk, pv = to_dev(x.prompt_k, dt, device), to_dev(x.prompt_v, dt, device)
    q = to_dev(x.q, dt, device)
    W = to_dev(x.W, dt, device)
    prior = None if x.prior is None else torch.from_numpy(x.prior).to(device)
    ak = av = par = trie = None
    beam_node = None
    if x.levels:
        cap = sum(k.shape[1] for (_, k, _) in x.levels)
        ak, av, par, trie = new_arena(shape, max(cap, capacity or 0), max_depth, device)
        prev, base = None, 0
        for (pb, kk, vv) in x.levels:
            prev = append_level(shape, trie, base, kk, vv, pb, prev, dev_err, device)
            base += kk.shape[1]
        beam_node = to_dev_i32(x.beam_node, device)
    vocab = x.W.shape[0]
    if flags is None:
        flags = L.GR_TOPK_LOG_SOFTMAX if vocab > 1 else 0
    return DeviceStep(shape, pk, pv, q, W, prior, ak, av, par, trie, beam_node, q.shape[1], cfg.k,
                      vocab, flags, dev_err)


def prefix_attn(ds: DeviceStep, stream=None) -> torch.Tensor:
    out = torch.empty((ds.R, ds.n_beams, ds.D), dtype=torch.float32, device=ds.q.device)
    nbytes = L.gr_attn_workspace_size(ds.shape, ds.n_beams)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=ds.q.device)
    L.gr_prefix_attn(ds.shape, ds.prompt_k, ds.prompt_v, ds.q, ds.n_beams, ds.trie, ds.beam_node, out,
                     ws, nbytes, ds.dev_err, stream)
    return out


@dataclasses.dataclass
class DecodeBuffers:
    score: torch.Tensor
    token: torch.Tensor
    parent: torch.Tensor
    attn: Optional[torch.Tensor]
    cand: Optional[torch.Tensor]
    ws: torch.Tensor
    ws_bytes: int


def decode_buffers(ds: DeviceStep, debug_outputs: bool = False) -> DecodeBuffers:
    dev = ds.q.device
    k = ds.k
    score = torch.empty((ds.R, k), dtype=torch.float32, device=dev)
    token = torch.empty((ds.R, k), dtype=torch.int32, device=dev)
    parent = torch.empty((ds.R, k), dtype=torch.int32, device=dev)
    attn = cand = None
    if debug_outputs:
        attn = torch.empty((ds.R, ds.n_beams, ds.D), dtype=torch.float32, device=dev)
        cand = torch.empty((ds.R, ds.n_beams, ds.vocab), dtype=torch.float32, device=dev)
    nbytes = L.gr_decode_workspace_size(ds.shape, ds.n_beams, ds.vocab, k)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    return DecodeBuffers(score, token, parent, attn, cand, ws, nbytes)


def decode_step(ds: DeviceStep, buf: DecodeBuffers, stream=None) -> None:
    L.gr_decode_step(ds.shape, ds.prompt_k, ds.prompt_v, ds.q, ds.n_beams, ds.trie, ds.beam_node, ds.W,
                     ds.vocab, ds.prior, ds.k, ds.flags, buf.score, buf.token, buf.parent, buf.attn,
                     buf.cand, buf.ws, buf.ws_bytes, ds.dev_err, stream)


def linear_state(ds: DeviceStep, stream=None):
    """gr_linear_state of an uploaded step's prompt: (state, norm)."""
    R, H, hd = ds.shape.R, ds.shape.H, ds.shape.head_dim
    S = torch.empty((R, H, hd, hd), dtype=torch.float32, device=ds.q.device)
    z = torch.empty((R, H, hd), dtype=torch.float32, device=ds.q.device)
    L.gr_linear_state(ds.shape, ds.prompt_k, ds.prompt_v, S, z, stream)
    return S, z


def linear_decode_step(ds: DeviceStep, buf: DecodeBuffers, state, norm, stream=None) -> None:
    L.gr_linear_decode_step(ds.shape, state, norm, ds.q, ds.n_beams, ds.trie, ds.beam_node, ds.W, ds.vocab,
                            ds.prior, ds.k, ds.flags, buf.score, buf.token, buf.parent, buf.attn, buf.cand,
                            buf.ws, buf.ws_bytes, ds.dev_err, stream)


def beam_topk(logits: torch.Tensor, prior: Optional[torch.Tensor], k: int, flags: int, cand: bool = True):
    R, n_in, vocab = logits.shape
    dev = logits.device
    score = torch.empty((R, k), dtype=torch.float32, device=dev)
    token = torch.empty((R, k), dtype=torch.int32, device=dev)
    parent = torch.empty((R, k), dtype=torch.int32, device=dev)
    cand_out = torch.empty_like(logits) if cand else None
    nbytes = L.gr_topk_workspace_size(R, n_in, vocab, k)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    L.gr_beam_topk(R, n_in, vocab, k, flags, logits, prior, score, token, parent, cand_out, ws, nbytes)
    return score, token, parent, cand_out


def results_to_host(buf: DecodeBuffers) -> dict:
    out = dict(score=buf.score.cpu().numpy(), token=buf.token.cpu().numpy(),
               parent=buf.parent.cpu().numpy())
    if buf.attn is not None:
        out["attn"] = buf.attn.cpu().numpy()
    if buf.cand is not None:
        out["cand"] = buf.cand.cpu().numpy()
    return out


# ------------------------------------------------------- whole-ID generation


def level_sizes(levels: int, beam_width: int, vocab: int = 256):
    """(n_l, k_l) of every step of a generation: beams in and kept."""
    n, out = 1, []
    for _ in range(levels):
        k = min(beam_width, n * vocab)
        out.append((n, k))
        n = k
    return out


@dataclasses.dataclass
class DeviceGen:
    """A whole-ID generation on the device: inputs, the code tables, the
    arena, outputs and workspace, ready for gr_generate."""
    shape: L.Shape
    levels: int
    beam_width: int
    vocab: int
    d_emb: int
    prompt_k: torch.Tensor
    prompt_v: torch.Tensor
    q0: torch.Tensor
    W: torch.Tensor            # [levels][vocab][D]
    emb: Optional[torch.Tensor]      # [levels-1][vocab][d_emb]
    w_qkv: torch.Tensor        # [3D][d_emb]
    tables: Optional[torch.Tensor]   # [levels-1][vocab][3][H][hd]
    trie: Optional[L.Trie]
    out_score: torch.Tensor
    out_token: torch.Tensor
    out_parent: torch.Tensor
    out_ids: torch.Tensor
    ws: torch.Tensor
    dev_err: torch.Tensor
    sizes: list

    def level(self, name: str, lv: int) -> torch.Tensor:
        """Step lv's block [R][k_l] of out_score / out_token / out_parent."""
        R = self.shape.R
        off = R * sum(k for _, k in self.sizes[:lv])
        k = self.sizes[lv][1]
        return getattr(self, name)[off:off + R * k].view(R, k)


def upload_generate(x, device="cuda", capacity: Optional[int] = None) -> DeviceGen:
    """Upload a workloads.GenInputs and allocate everything gr_generate needs
    (the code tables are left empty: code_tables() fills them).  `capacity`
    (default: exactly the appended records) sizes the trie arena."""
    cfg = x.cfg
    dt = dtype_code(cfg.dtype)
    R = x.prompt_k.shape[0]
    shape = make_shape(R, cfg.H, cfg.d, cfg.Lp, cfg.window, dt)
    levels, B, V = cfg.steps, cfg.k, cfg.vocab
    sizes = level_sizes(levels, B, V)
    total = R * sum(k for _, k in sizes)
    trie, tables, emb = None, None, None
    if levels > 1:
        cap = max(sum(k for _, k in sizes[:-1]), capacity or 0)
        trie = new_arena(shape, cap, max_depth=max(levels - 1, 1), device=device)[3]
        emb = to_dev(np.stack(x.emb), dt, device)
        tables = torch.empty((levels - 1, V, 3, cfg.H, cfg.d), dtype=_TORCH[dt], device=device)
    ws_bytes = L.gr_generate_workspace_size(shape, levels, V, B)
    return DeviceGen(shape, levels, B, V, x.d_emb, to_dev(x.prompt_k, dt, device), to_dev(x.prompt_v, dt, device),
                     to_dev(x.q0, dt, device), to_dev(np.stack(x.W), dt, device), emb,
                     to_dev(x.w_qkv, dt, device), tables, trie,
                     torch.empty(total, dtype=torch.float32, device=device),
                     torch.empty(total, dtype=torch.int32, device=device),
                     torch.empty(total, dtype=torch.int32, device=device),
                     torch.empty((R, sizes[-1][1], levels), dtype=torch.int32, device=device),
                     torch.empty(ws_bytes, dtype=torch.uint8, device=device),
                     torch.zeros(1, dtype=torch.int32, device=device), sizes)


def code_tables(g: DeviceGen, stream=None) -> None:
    """gr_code_table over every level whose chosen codes become records."""
    L.gr_code_table(g.shape, g.levels - 1, g.vocab, g.d_emb, g.emb, g.w_qkv, g.tables, stream)


def generate(g: DeviceGen, stream=None) -> None:
    L.gr_generate(g.shape, g.prompt_k, g.prompt_v, g.q0, g.levels, g.W, g.tables, g.vocab, g.beam_width, g.trie,
                  g.out_score, g.out_token, g.out_parent, g.out_ids, g.ws, g.ws.numel(), g.dev_err, stream)


def generate_to_host(g: DeviceGen) -> dict:
    """Per-step results and the final IDs as numpy arrays."""
    steps = [dict(score=g.level("out_score", lv).cpu().numpy(), token=g.level("out_token", lv).cpu().numpy(),
                  parent=g.level("out_parent", lv).cpu().numpy()) for lv in range(g.levels)]
    return dict(steps=steps, ids=g.out_ids.cpu().numpy())


@dataclasses.dataclass
class DeviceXf:
    """A broadcast-scoring run on the device: tokens, packed weights,
    outputs and workspace, ready for gr_broadcast_score."""
    shape: L.XfShape
    k: int
    user: torch.Tensor         # [R][Lu][D] bf16
    cand: torch.Tensor         # [R][N][D] bf16
    w_mat: torch.Tensor        # bf16, per layer w_qkv, w_o, w_1, w_2
    w_vec: torch.Tensor        # fp32, per layer vectors then the final ones
    out_score: torch.Tensor    # [R][k]
    out_index: torch.Tensor    # [R][k]
    cand_scores: Optional[torch.Tensor]   # [R][N] or None
    ws: torch.Tensor


def upload_xf(x, k: Optional[int] = None, all_scores: bool = True, device="cuda") -> DeviceXf:
    """Upload a workloads.XFInputs and allocate the outputs and workspace."""
    cfg = x.cfg
    R, N, D = x.cand.shape
    k = cfg.k if k is None else int(k)
    shape = L.XfShape(R, N, x.user.shape[1], D, len(x.layers))
    ws_bytes = L.gr_broadcast_workspace_size(shape, k)
    return DeviceXf(shape, k, to_dev(x.user, L.GR_BF16, device), to_dev(x.cand, L.GR_BF16, device),
                    to_dev(x.w_mat, L.GR_BF16, device), to_dev(x.w_vec, L.GR_F32, device),
                    torch.empty((R, k), dtype=torch.float32, device=device),
                    torch.empty((R, k), dtype=torch.int32, device=device),
                    torch.empty((R, N), dtype=torch.float32, device=device) if all_scores else None,
                    torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=device))


def broadcast_score(d: DeviceXf, stream=None) -> None:
    L.gr_broadcast_score(d.shape, d.user, d.cand, d.w_mat, d.w_vec, d.k, d.out_score, d.out_index, d.cand_scores,
                         d.ws, d.ws.numel(), stream)


def xf_to_host(d: DeviceXf) -> dict:
    return dict(score=d.out_score.cpu().numpy(), index=d.out_index.cpu().numpy(),
                all=None if d.cand_scores is None else d.cand_scores.cpu().numpy())
