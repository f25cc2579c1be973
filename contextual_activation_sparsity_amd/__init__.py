"""Contextually sparse decoder-layer step on MI355X (gfx950): Python binding.

The functions below carry the C ABI's names (include/dejavu_hip.h) and only marshal
torch tensors (device memory) and the current HIP stream into the library. Every step of
the layer runs in hand-written HIP kernels; there is no CPU or torch fallback.

Typical use::

    import contextual_activation_sparsity_amd as dv
    dims = dv.Dims(d_model=4096, d_ffn=16384, n_heads=32, head_dim=128, rank_mlp=512,
                   rank_head=512, t_max=2049, dtype="f16")
    ws = dv.workspace(dims, B=1, k=820, kh=7)
    dv.dv_layer_step(dims, layer, pred, x, x, 820, 7, None, None, kc, vc, 2048, x_out, ws=ws)
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Dict, Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import DV_IDX_DUPLICATE, DV_IDX_ORDER, DV_IDX_RANGE, DejavuError  # noqa: F401

__all__ = ["Dims", "LayerWeights", "PredictorWeights", "workspace", "stack_workspace", "dv_predict",
           "dv_topk", "dv_sparse_mlp", "dv_sparse_attn", "dv_layer_step", "dv_layer_step_noalloc", "dv_lookahead_stack",
           "dv_decode_step", "dv_layer_labels", "dv_predictor_train_workspace_bytes", "dv_predictor_train_step",
           "dv_workspace_bytes", "dv_stack_workspace_bytes", "dv_topk_workspace_bytes", "dv_block_scores",
           "dv_sparse_mlp_blocked", "dv_check_indices", "require_gpu", "DejavuError",
           "DV_IDX_RANGE", "DV_IDX_ORDER", "DV_IDX_DUPLICATE"]

_DT = {"f32": (_lib.DV_F32, torch.float32), "f16": (_lib.DV_F16, torch.float16)}


@dataclasses.dataclass(frozen=True)
class Dims:
    d_model: int
    d_ffn: int
    n_heads: int
    head_dim: int
    rank_mlp: int
    rank_head: int
    t_max: int
    dtype: str = "f16"

    def c(self) -> _lib.DvDims:
        return _lib.DvDims(self.d_model, self.d_ffn, self.n_heads, self.head_dim, self.rank_mlp,
                           self.rank_head, self.t_max, _DT[self.dtype][0])

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DT[self.dtype][1]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


@dataclasses.dataclass
class LayerWeights:
    """Device tensors of one layer (storage layouts as in include/dejavu_hip.h)."""
    g1: torch.Tensor
    g2: torch.Tensor
    wqkv: torch.Tensor
    bqkv: torch.Tensor
    wo: torch.Tensor
    bo: torch.Tensor
    w1t: torch.Tensor
    b1: torch.Tensor
    w2: torch.Tensor
    b2: torch.Tensor

    def c(self) -> _lib.DvLayer:
        return _lib.DvLayer(*[_ptr(getattr(self, f.name)) for f in dataclasses.fields(self)])


@dataclasses.dataclass
class PredictorWeights:
    p1_mlp: torch.Tensor
    p2_mlp: torch.Tensor
    p1_head: torch.Tensor
    p2_head: torch.Tensor

    def c(self) -> _lib.DvPredictor:
        return _lib.DvPredictor(*[_ptr(getattr(self, f.name)) for f in dataclasses.fields(self)])


def require_gpu() -> None:
    """Load the library and check that a GPU is visible; raise otherwise."""
    _lib.lib()
    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible: the sparse layer step runs only on the GPU")


def dv_workspace_bytes(dims: Dims, B: int, k: int, kh: int) -> int:
    d = dims.c()
    return int(_lib.lib().dv_workspace_bytes(ctypes.byref(d), B, k, kh))


def dv_topk_workspace_bytes(B: int, n: int) -> int:
    return int(_lib.lib().dv_topk_workspace_bytes(B, n))


def dv_stack_workspace_bytes(dims: Dims, B: int, k: int, kh: int) -> int:
    d = dims.c()
    return int(_lib.lib().dv_stack_workspace_bytes(ctypes.byref(d), B, k, kh))


def _alloc_ws(n: int, device) -> torch.Tensor:
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def workspace(dims: Dims, B: int, k: int, kh: int, device="cuda") -> torch.Tensor:
    return _alloc_ws(dv_workspace_bytes(dims, B, k, kh), device)


def stack_workspace(dims: Dims, B: int, k: int, kh: int, device="cuda") -> torch.Tensor:
    return _alloc_ws(dv_stack_workspace_bytes(dims, B, k, kh), device)


def _ws(ws: Optional[torch.Tensor]) -> Tuple[Optional[int], int]:
    if ws is None:
        return None, 0
    return ws.data_ptr(), ws.numel() * ws.element_size()


def dv_predict(dims: Dims, pred: PredictorWeights, x_pred: torch.Tensor, s_mlp: torch.Tensor,
               s_head: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    d, p = dims.c(), pred.c()
    wp, wn = _ws(ws)
    st = _lib.lib().dv_predict(ctypes.byref(d), ctypes.byref(p), _ptr(x_pred), x_pred.shape[0], _ptr(s_mlp),
                               _ptr(s_head), wp, wn, _stream(stream))
    _lib.check("dv_predict", st)


def dv_topk(scores: torch.Tensor, k: int, idx: torch.Tensor, ws: Optional[torch.Tensor] = None,
            stream=None) -> None:
    B, n = scores.shape
    if ws is None and k > 0:
        ws = _alloc_ws(dv_topk_workspace_bytes(B, n), scores.device)
    wp, wn = _ws(ws)
    st = _lib.lib().dv_topk(_ptr(scores), B, n, k, _ptr(idx), wp, wn, _stream(stream))
    _lib.check("dv_topk", st)


def dv_block_scores(scores: torch.Tensor, bs: int, out: torch.Tensor, stream=None) -> None:
    B, n = scores.shape
    st = _lib.lib().dv_block_scores(_ptr(scores), B, n, bs, _ptr(out), _stream(stream))
    _lib.check("dv_block_scores", st)


def dv_check_indices(idx: Optional[torch.Tensor], n: int, status: torch.Tensor, k: Optional[int] = None,
                     stream=None) -> None:
    """status[b] (int32 device tensor [B]) = OR of DV_IDX_RANGE / DV_IDX_ORDER / DV_IDX_DUPLICATE
    for row b of idx [B][k] (int32 device tensor) against the bound n; 0 when the row is valid."""
    B = status.numel()
    if k is None:
        k = 0 if idx is None else idx.shape[-1]
    st = _lib.lib().dv_check_indices(_ptr(idx), B, k, n, _ptr(status), _stream(stream))
    _lib.check("dv_check_indices", st)


def dv_sparse_mlp_blocked(dims: Dims, layer: LayerWeights, xn: torch.Tensor, blocks: Optional[torch.Tensor], kb: int,
                          bs: int, y: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    d, L = dims.c(), layer.c()
    wp, wn = _ws(ws)
    st = _lib.lib().dv_sparse_mlp_blocked(ctypes.byref(d), ctypes.byref(L), _ptr(xn), xn.shape[0], _ptr(blocks), kb,
                                          bs, _ptr(y), wp, wn, _stream(stream))
    _lib.check("dv_sparse_mlp_blocked", st)


def dv_layer_labels(dims: Dims, layer: LayerWeights, x: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    t_past: int, fire: Optional[torch.Tensor] = None, preact: Optional[torch.Tensor] = None,
                    head_norm: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """Dense-layer training targets: fire [B][F] uint8, preact [B][F] fp32, head_norm [B][H] fp32."""
    d, L = dims.c(), layer.c()
    if ws is None:
        ws = workspace(dims, x.shape[0], dims.d_ffn, dims.n_heads)
    wp, wn = _ws(ws)
    st = _lib.lib().dv_layer_labels(ctypes.byref(d), ctypes.byref(L), _ptr(x), x.shape[0], _ptr(k_cache),
                                    _ptr(v_cache), t_past, _ptr(fire), _ptr(preact), _ptr(head_norm), wp, wn,
                                    _stream(stream))
    _lib.check("dv_layer_labels", st)


def dv_predictor_train_workspace_bytes(M: int, d: int, N: int, r: int) -> int:
    return int(_lib.lib().dv_predictor_train_workspace_bytes(M, d, N, r))


def dv_predictor_train_step(x: torch.Tensor, y: torch.Tensor, p1: torch.Tensor, p2: torch.Tensor, v1: torch.Tensor,
                            v2: torch.Tensor, lr: float, momentum: float, loss: torch.Tensor,
                            ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """One full-batch step on x [M][d] fp32, y [M][N] uint8, p1 [r][d], p2 [N][r] (updated in place)."""
    M, d = x.shape
    N, r = p2.shape
    if y.dtype != torch.uint8 or tuple(y.shape) != (M, N) or tuple(p1.shape) != (r, d):
        raise ValueError("shapes: x [M][d], y [M][N] uint8, p1 [r][d], p2 [N][r]")
    for name, t in (("x", x), ("p1", p1), ("p2", p2), ("v1", v1), ("v2", v2), ("loss", loss)):
        if t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
    if v1.shape != p1.shape or v2.shape != p2.shape:
        raise ValueError("momentum buffers must match the factors")
    if ws is None:
        ws = _alloc_ws(dv_predictor_train_workspace_bytes(M, d, N, r), x.device)
    wp, wn = _ws(ws)
    st = _lib.lib().dv_predictor_train_step(_ptr(x), M, d, _ptr(y), N, r, _ptr(p1), _ptr(p2), _ptr(v1), _ptr(v2),
                                            float(lr), float(momentum), _ptr(loss), wp, wn, _stream(stream))
    _lib.check("dv_predictor_train_step", st)


def dv_sparse_mlp(dims: Dims, layer: LayerWeights, xn: torch.Tensor, idx: Optional[torch.Tensor], k: int,
                  y: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    d, L = dims.c(), layer.c()
    wp, wn = _ws(ws)
    st = _lib.lib().dv_sparse_mlp(ctypes.byref(d), ctypes.byref(L), _ptr(xn), xn.shape[0], _ptr(idx), k,
                                  _ptr(y), wp, wn, _stream(stream))
    _lib.check("dv_sparse_mlp", st)


def dv_sparse_attn(dims: Dims, layer: LayerWeights, xn: torch.Tensor, heads: Optional[torch.Tensor], kh: int,
                   k_cache: torch.Tensor, v_cache: torch.Tensor, t_past: int, y: torch.Tensor,
                   ws: torch.Tensor, stream=None) -> None:
    d, L = dims.c(), layer.c()
    wp, wn = _ws(ws)
    st = _lib.lib().dv_sparse_attn(ctypes.byref(d), ctypes.byref(L), _ptr(xn), xn.shape[0], _ptr(heads), kh,
                                   _ptr(k_cache), _ptr(v_cache), t_past, _ptr(y), wp, wn, _stream(stream))
    _lib.check("dv_sparse_attn", st)


def dv_layer_step(dims: Dims, layer: LayerWeights, pred: Optional[PredictorWeights], x: torch.Tensor,
                  x_pred: Optional[torch.Tensor], k: int, kh: int, idx_in: Optional[torch.Tensor],
                  heads_in: Optional[torch.Tensor], k_cache: torch.Tensor, v_cache: torch.Tensor,
                  t_past: int, x_out: torch.Tensor, idx_out: Optional[torch.Tensor] = None,
                  heads_out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                  stream=None) -> None:
    d, L = dims.c(), layer.c()
    p = pred.c() if pred is not None else None
    wp, wn = _ws(ws)
    st = _lib.lib().dv_layer_step(ctypes.byref(d), ctypes.byref(L), ctypes.byref(p) if p is not None else None,
                                  _ptr(x), _ptr(x_pred), x.shape[0], k, kh, _ptr(idx_in), _ptr(heads_in),
                                  _ptr(k_cache), _ptr(v_cache), t_past, _ptr(x_out), _ptr(idx_out),
                                  _ptr(heads_out), wp, wn, _stream(stream))
    _lib.check("dv_layer_step", st)


def dv_layer_step_noalloc(dims: Dims, layer: LayerWeights, pred: Optional[PredictorWeights], x: torch.Tensor,
                          x_pred: Optional[torch.Tensor], k: int, kh: int, idx_in: Optional[torch.Tensor],
                          heads_in: Optional[torch.Tensor], k_cache: torch.Tensor, v_cache: torch.Tensor,
                          t_past: int, x_out: torch.Tensor, idx_out: Optional[torch.Tensor] = None,
                          heads_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """dv_layer_step without a workspace: the library's fixed per-GPU scratch array serves as one."""
    d, L = dims.c(), layer.c()
    p = pred.c() if pred is not None else None
    st = _lib.lib().dv_layer_step_noalloc(ctypes.byref(d), ctypes.byref(L), ctypes.byref(p) if p is not None else None,
                                          _ptr(x), _ptr(x_pred), x.shape[0], k, kh, _ptr(idx_in), _ptr(heads_in),
                                          _ptr(k_cache), _ptr(v_cache), t_past, _ptr(x_out), _ptr(idx_out),
                                          _ptr(heads_out), _stream(stream))
    _lib.check("dv_layer_step_noalloc", st)


def dv_lookahead_stack(dims: Dims, layers: Sequence[LayerWeights], preds: Sequence[PredictorWeights],
                       x: torch.Tensor, k: int, kh: int, k_caches: Sequence[torch.Tensor],
                       v_caches: Sequence[torch.Tensor], t_past: int, y: torch.Tensor,
                       h_all: Optional[torch.Tensor] = None, idx_out: Optional[torch.Tensor] = None,
                       heads_out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                       stream=None, side_stream=None) -> None:
    n = len(layers)
    d = dims.c()
    Ls = (_lib.DvLayer * n)(*[l.c() for l in layers])
    Ps = (_lib.DvPredictor * n)(*[p.c() for p in preds])
    kcs = (ctypes.c_void_p * n)(*[_ptr(t) for t in k_caches])
    vcs = (ctypes.c_void_p * n)(*[_ptr(t) for t in v_caches])
    wp, wn = _ws(ws)
    main = _stream(stream)
    side = main if side_stream is None else side_stream.cuda_stream
    st = _lib.lib().dv_lookahead_stack(ctypes.byref(d), Ls, Ps, n, _ptr(x), x.shape[0], k, kh, kcs, vcs, t_past,
                                       _ptr(y), _ptr(h_all), _ptr(idx_out), _ptr(heads_out), wp, wn, main, side)
    _lib.check("dv_lookahead_stack", st)


def dv_decode_step(dims: Dims, layers: Sequence[LayerWeights], preds: Sequence[PredictorWeights],
                   x: torch.Tensor, k: int, kh: int, k_caches: Sequence[torch.Tensor],
                   v_caches: Sequence[torch.Tensor], t_rows: torch.Tensor, y: torch.Tensor, advance: bool = False,
                   h_all: Optional[torch.Tensor] = None, idx_out: Optional[torch.Tensor] = None,
                   heads_out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                   stream=None, side_stream=None) -> None:
    """t_rows: int32 device tensor [B] of per-row past lengths (advanced in place if advance)."""
    if t_rows.dtype != torch.int32 or not t_rows.is_cuda or t_rows.numel() != x.shape[0]:
        raise ValueError("t_rows must be an int32 device tensor with one length per row")
    n = len(layers)
    d = dims.c()
    Ls = (_lib.DvLayer * n)(*[l.c() for l in layers])
    Ps = (_lib.DvPredictor * n)(*[p.c() for p in preds])
    kcs = (ctypes.c_void_p * n)(*[_ptr(t) for t in k_caches])
    vcs = (ctypes.c_void_p * n)(*[_ptr(t) for t in v_caches])
    wp, wn = _ws(ws)
    main = _stream(stream)
    side = main if side_stream is None else side_stream.cuda_stream
    st = _lib.lib().dv_decode_step(ctypes.byref(d), Ls, Ps, n, _ptr(x), x.shape[0], k, kh, kcs, vcs, _ptr(t_rows),
                                   int(bool(advance)), _ptr(y), _ptr(h_all), _ptr(idx_out), _ptr(heads_out), wp, wn,
                                   main, side)
    _lib.check("dv_decode_step", st)
