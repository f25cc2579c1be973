"""Device-side generation of the seeded synthetic inputs (bit-identical to synth's host draws),
and a plain streaming-read measurement for the bench.

Large workloads (the OPT-175B-shaped 24-layer stack holds ~93 GB of fp16 weights, caches
and predictors) are drawn directly in HBM by synth/libdv_synth.so; the host regenerates any
row it needs from the same counters. This module draws numbers only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict

import numpy as np
import torch

from . import Workload, layer_shapes, scale_f32

_LIB = None
_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdv_synth.so")


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_PATH):
            raise RuntimeError(f"{_PATH} is missing: build with `python -m contextual_activation_sparsity_amd.build`")
        L = ctypes.CDLL(_PATH)
        L.dv_synth_fill.restype = ctypes.c_int
        L.dv_synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_ulonglong,
                                    ctypes.c_float, ctypes.c_longlong, ctypes.c_void_p]
        L.dv_synth_stream_read.restype = ctypes.c_int
        L.dv_synth_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_void_p]
        _LIB = L
    return _LIB


def fill_(t: torch.Tensor, key: int, sigma: float, start: int = 0) -> torch.Tensor:
    """Fill a contiguous fp32/fp16 device tensor with the stream `key` from counter `start`."""
    assert t.is_cuda and t.is_contiguous()
    if sigma == 0.0:
        return t.zero_()
    dt = {torch.float32: 0, torch.float16: 1}[t.dtype]
    rc = _lib().dv_synth_fill(t.data_ptr(), t.numel(), dt, key, float(scale_f32(sigma)), start,
                              torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"dv_synth_fill failed with hip error {rc}")
    return t


def _tdt(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "f16": torch.float16}[dtype]


def layer_on_device(w: Workload, layer: int = 0, device="cuda") -> Dict[str, torch.Tensor]:
    """All tensors of one layer (weights, predictor, gains) drawn in device memory."""
    if w.b1_mean != 0.0:
        raise ValueError("layer_on_device draws unshifted biases; use layer_tensors for b1_mean != 0")
    out = {}
    for name, (shp, sg, dt) in layer_shapes(w).items():
        t = torch.empty(shp, dtype=_tdt(dt), device=device)
        out[name] = fill_(t, w.key(name, layer), sg)
    out["g1"] = torch.ones(w.d_model, dtype=torch.float32, device=device)
    out["g2"] = torch.ones(w.d_model, dtype=torch.float32, device=device)
    return out


def kv_on_device(w: Workload, which: str, layer: int = 0, device="cuda") -> torch.Tensor:
    shp = (w.batch, w.n_heads, w.t_max, w.head_dim)
    t = torch.empty(shp, dtype=_tdt(w.dtype), device=device)
    fill_(t, w.key(which, layer), w.kv_sigma)
    t[:, :, w.t_past:, :] = 0
    return t


def x_on_device(w: Workload, step: int = 0, layer: int = 0, device="cuda") -> torch.Tensor:
    t = torch.empty((w.batch, w.d_model), dtype=torch.float32, device=device)
    return fill_(t, w.key("x", layer, step), w.x_sigma)


def to_device(arrs: Dict[str, np.ndarray], device="cuda") -> Dict[str, torch.Tensor]:
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(device) for k, v in arrs.items()}


def stream_read_gbps(nbytes: int = 4 << 30, reps: int = 5) -> float:
    """Best read bandwidth (GB/s) of the plain streaming-read kernel over a device buffer of
    nbytes (well beyond the 256 MB Infinity Cache), timed with HIP events on the current stream.
    A measurement reference for the bench; it draws no numbers."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    props = torch.cuda.get_device_properties(torch.cuda.current_device())
    blocks = 8 * props.multi_processor_count
    sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    best = 0.0
    for _ in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = _lib().dv_synth_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, stream)
        e1.record()
        if rc != 0:
            raise RuntimeError(f"dv_synth_stream_read failed with hip error {rc}")
        torch.cuda.synchronize()
        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf, sink
    return best
