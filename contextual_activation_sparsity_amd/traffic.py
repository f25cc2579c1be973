"""Memory-traffic model of decode: the bytes a step must move and the time they bound.

Host-side bookkeeping used to turn measured times into achieved bandwidth. It
computes no part of the layer step.

Two models live here:

* The page's model. DejaVu Guide, "Mathematical Modeling: Memory Traffic and
  Speedup Bounds": dense weight traffic per token is
  N_layers * (4 d^2 + n_mlp * d * d_ffn) * P bytes, the sparse traffic scales the
  attention term by the active-head fraction and the MLP term by the active
  neuron fraction, and a memory-bound decode step takes at least traffic /
  bandwidth. The page's worked example (LLaMA-3-70B shapes, SwiGLU, so three
  MLP matrices) pins these functions in the tests.
* The algorithmic bytes counted here per layer-token: every weight row, bias, gain
  and KV entry the sparse step must read, the KV entries it appends and the
  residual-stream vector it reads and writes. Intermediates a fused kernel
  could keep on chip (scores, q/k/v, partial sums) are not counted.
"""
from __future__ import annotations

from typing import Dict


def dense_weight_bytes_per_layer(d_model: int, d_ffn: int, p_bytes: int, n_mlp_mats: int = 3) -> int:
    """Dense weight bytes of one layer: (4 d^2 + n_mlp d d_ffn) * P."""
    return (4 * d_model * d_model + n_mlp_mats * d_model * d_ffn) * p_bytes


def attn_weight_bytes_per_layer(d_model: int, p_bytes: int) -> int:
    return 4 * d_model * d_model * p_bytes


def mlp_weight_bytes_per_layer(d_model: int, d_ffn: int, p_bytes: int, n_mlp_mats: int = 3) -> int:
    return n_mlp_mats * d_model * d_ffn * p_bytes


def sparse_weight_bytes_per_layer(d_model: int, d_ffn: int, p_bytes: int, s_attn: float,
                                  s_mlp: float, n_mlp_mats: int = 3) -> float:
    """Sparse weight bytes of one layer: active fractions times the two dense terms."""
    return (s_attn * attn_weight_bytes_per_layer(d_model, p_bytes)
            + s_mlp * mlp_weight_bytes_per_layer(d_model, d_ffn, p_bytes, n_mlp_mats))


def stream_time_lower_bound_s(n_bytes: float, bandwidth_bytes_per_s: float) -> float:
    """A memory-bound step cannot finish faster than bytes / bandwidth."""
    return n_bytes / bandwidth_bytes_per_s


def step_bytes(d_model: int, d_ffn: int, n_heads: int, head_dim: int, rank: int, t_past: int,
               k_union: int, kh_union: int, wb: int, batch: int = 1, kh_rows_kv: int = None,
               predictor: bool = True) -> Dict[str, int]:
    """Algorithmic HBM bytes of one sparse layer step (all batch rows).

    k_union / kh_union: distinct neurons / heads whose weights are read (the
    per-row sets' union; equal to k / kh at batch 1). kh_rows_kv: the sum over
    batch rows of each row's head count (each row reads its own KV cache);
    defaults to batch * kh_union.
    """
    d, F, H, dh, r, T = d_model, d_ffn, n_heads, head_dim, rank, t_past
    if kh_rows_kv is None:
        kh_rows_kv = batch * kh_union
    f32 = 4
    parts = {
        "predictor": (2 * r * d + r * (F + H)) * wb if predictor else 0,
        "qkv": 3 * kh_union * dh * d * wb + 3 * kh_union * dh * f32,
        "kv_read": 2 * kh_rows_kv * dh * T * wb,
        "kv_append": 2 * kh_rows_kv * dh * wb,
        "wo": kh_union * dh * d * wb + d * f32,
        "w1": k_union * d * wb + k_union * f32,
        "w2": k_union * d * wb + d * f32,
        "gains": 2 * d * f32,
        "vectors": 2 * batch * d * f32 + (batch * d * f32 if predictor else 0),
    }
    parts["total"] = sum(parts.values())
    return parts


def dense_layer_bytes(d_model: int, d_ffn: int, n_heads: int, head_dim: int, t_past: int, wb: int,
                      batch: int = 1) -> int:
    """Bytes of the dense decoder layer at the same shape (no predictor)."""
    d, F, H, dh, T = d_model, d_ffn, n_heads, head_dim, t_past
    return ((3 * H * dh * d + H * dh * d + 2 * F * d) * wb
            + batch * 2 * H * dh * (T + 1) * wb
            + (3 * H * dh + 2 * d + F + 2 * d) * 4 + 2 * batch * d * 4)


def step_flops(d_model: int, d_ffn: int, n_heads: int, head_dim: int, rank: int, t_past: int,
               k: int, kh: int, batch: int = 1) -> int:
    """Multiply-add flops (2 per MAC) of one sparse layer step."""
    d, F, H, dh, r, T = d_model, d_ffn, n_heads, head_dim, rank, t_past
    per_row = 2 * (2 * r * d + r * (F + H) + 3 * kh * dh * d + 2 * kh * dh * (T + 1)
                   + kh * dh * d + 2 * k * d)
    return batch * per_row
