"""Seeded synthetic inputs for the sparse decode layer step.

This module is shared by the oracle tests, the GPU tests and the bench. It
draws numbers and holds workload shapes; it performs no step of the method
(no projection, selection, norm, attention or MLP arithmetic).

Generator
---------
Every tensor element is a pure function of (stream key, element counter), so a
row of a 1.2 GB matrix can be regenerated on the host without generating the
rest, and the device filler in ``synth/fill.hip`` produces bit-identical values.

* Bits: the SplitMix64 output function (Steele, Lea and Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014) applied to
  ``key + (i + 1) * 0x9E3779B97F4A7C15`` (wrapping 64-bit arithmetic), i.e. the
  i-th output of a SplitMix64 stream seeded with ``key``.
* Near-Gaussian values: the four 16-bit lanes of the 64-bit output are summed
  (an Irwin-Hall(4) variate), centred exactly in integers, converted exactly to
  fp32 and multiplied once by the fp32 constant ``sigma / SD_IH4``. That single
  correctly rounded fp32 multiply, followed by round-to-nearest-even to fp16
  where the storage type is fp16, is reproduced bit for bit by the device
  filler. The variate has mean 0 and standard deviation ``sigma``; it stands in
  for the N(0, sigma) draws of the OPT-shaped workloads.
* Uniforms in [0, 1) (host only): the top 53 bits times 2**-53.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

GOLDEN = 0x9E3779B97F4A7C15
MIX_M1 = 0xBF58476D1CE4E5B9
MIX_M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

# Standard deviation of the sum of four independent uniform integers on [0, 65535].
SD_IH4 = math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)
IH4_CENTER = 2 * 65535  # mean of that sum, an exact integer


def mix64_int(z: int) -> int:
    """SplitMix64 output mixing function on a Python int (64-bit wrapping)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX_M1) & MASK64
    z = ((z ^ (z >> 27)) * MIX_M2) & MASK64
    return z ^ (z >> 31)


def mix64(z: np.ndarray) -> np.ndarray:
    """Vectorised SplitMix64 output mixing function on a uint64 array."""
    z = z.astype(np.uint64, copy=True)
    z ^= z >> np.uint64(30)
    z *= np.uint64(MIX_M1)
    z ^= z >> np.uint64(27)
    z *= np.uint64(MIX_M2)
    z ^= z >> np.uint64(31)
    return z


# Tensor identifiers: part of every stream key, so each tensor of each layer
# is an independent stream.
TENSOR_IDS: Dict[str, int] = {
    "p1_mlp": 1, "p2_mlp": 2, "p1_head": 3, "p2_head": 4,
    "g1": 5, "g2": 6, "wqkv": 7, "bqkv": 8, "wo": 9, "bo": 10,
    "w1t": 11, "b1": 12, "w2": 13, "b2": 14,
    "k_cache": 15, "v_cache": 16, "x": 17, "sel_mlp": 18, "sel_head": 19, "scores": 20,
    "x_basis": 21, "x_coef": 22, "x_noise": 23, "labels": 24,
}


def stream_key(seed: int, workload: int, layer: int, tensor: int, step: int = 0) -> int:
    """64-bit stream key for one tensor of one layer (and one step, for x)."""
    k = mix64_int(GOLDEN)
    for part in (seed, workload, layer, tensor, step):
        k = mix64_int((k ^ (part & MASK64)) + GOLDEN)
    return k


def raw_bits(key: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` of the SplitMix64 stream ``key``."""
    return raw_bits_at(key, np.arange(start, start + count, dtype=np.uint64))


def raw_bits_at(key: int, counters: np.ndarray) -> np.ndarray:
    """Outputs of the SplitMix64 stream ``key`` at arbitrary (0-based) counters."""
    ctr = np.asarray(counters, dtype=np.uint64) + np.uint64(1)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + ctr * np.uint64(GOLDEN)
    return mix64(z)


def scale_f32(sigma: float) -> np.float32:
    """The single fp32 multiplier that maps a centred Irwin-Hall(4) integer to std ``sigma``."""
    return np.float32(sigma / SD_IH4)


def normal_f32(key: int, start: int, count: int, sigma: float) -> np.ndarray:
    """Near-Gaussian fp32 values (mean 0, std sigma) for counters start..start+count-1."""
    return normal_f32_at(key, np.arange(start, start + count, dtype=np.uint64), sigma)


def _normal_chunk(key: int, ctr: np.ndarray, scale: np.float32, out: np.ndarray) -> None:
    b = raw_bits_at(key, ctr)
    m = np.uint64(0xFFFF)
    s = (b & m) + ((b >> np.uint64(16)) & m) + ((b >> np.uint64(32)) & m) + (b >> np.uint64(48))
    z = s.astype(np.int64) - IH4_CENTER
    np.multiply(z.astype(np.float32), scale, out=out)


_CHUNK = 1 << 16


def normal_f32_at(key: int, counters: np.ndarray, sigma: float) -> np.ndarray:
    """Near-Gaussian fp32 values at arbitrary counters.

    Large requests are cut into cache-sized chunks spread over threads; every element
    is computed by the same operations either way.
    """
    counters = np.asarray(counters, dtype=np.uint64).reshape(-1)
    n = counters.size
    out = np.empty(n, np.float32)
    scale = scale_f32(sigma)
    if n <= 4 * _CHUNK:
        _normal_chunk(key, counters, scale, out)
        return out
    starts = range(0, n, _CHUNK)
    with _pool() as ex:
        list(ex.map(lambda a: _normal_chunk(key, counters[a:a + _CHUNK], scale, out[a:a + _CHUNK]), starts))
    return out


def _pool():
    import concurrent.futures as cf
    import os
    return cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))


def uniform01(key: int, start: int, count: int) -> np.ndarray:
    """Uniform fp64 values in [0, 1) from the top 53 bits (host only)."""
    b = raw_bits(key, start, count)
    return (b >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def np_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16}[dtype]


def tensor(key: int, shape: Tuple[int, ...], sigma: float, dtype: str,
           row_start: int = 0, n_rows: Optional[int] = None) -> np.ndarray:
    """Draw a tensor (or a contiguous range of its leading-axis rows).

    The counter of element e is its flat index in the full tensor, so a row
    range drawn alone equals the same rows of the full tensor.
    """
    shape = tuple(int(s) for s in shape)
    row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    if n_rows is None:
        n_rows = shape[0] - row_start
    vals = normal_f32(key, row_start * row, n_rows * row, sigma) if sigma != 0.0 else \
        np.zeros(n_rows * row, np.float32)
    return vals.astype(np_dtype(dtype)).reshape((n_rows,) + shape[1:])


def rows(key: int, shape: Tuple[int, ...], sigma: float, dtype: str, row_ids) -> np.ndarray:
    """Draw an arbitrary list of leading-axis rows of a tensor (random access)."""
    row_ids = np.asarray(row_ids, dtype=np.int64).reshape(-1)
    row = int(np.prod(shape[1:]))
    out = np.empty((row_ids.size, row), np_dtype(dtype))
    step = max(1, (1 << 22) // max(row, 1))
    for a in range(0, row_ids.size, step):
        r = row_ids[a:a + step]
        ctr = (r[:, None] * row + np.arange(row, dtype=np.int64)[None, :]).astype(np.uint64)
        vals = normal_f32_at(key, ctr.reshape(-1), sigma) if sigma != 0.0 else np.zeros(ctr.size, np.float32)
        out[a:a + step] = vals.astype(np_dtype(dtype)).reshape(r.size, row)
    return out.reshape((row_ids.size,) + tuple(shape[1:]))


# --------------------------------------------------------------------------
# Workload presets: OPT-shaped synthetic decoder layers.
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # workload id, part of every stream key
    d_model: int
    d_ffn: int
    n_heads: int
    head_dim: int
    rank: int           # predictor rank (MLP and head predictors alike)
    t_past: int         # past KV length
    k: int              # neurons kept per token
    kh: int             # heads kept per token
    dtype: str          # weight and KV storage type
    n_layers: int = 1
    batch: int = 1
    w_sigma: float = 0.02
    p_sigma: float = 0.05
    x_sigma: float = 1.0
    kv_sigma: float = 1.0
    bias_sigma: float = 0.0
    b1_mean: float = 0.0  # added to every up-projection bias (sets how often a neuron fires)
    seed: int = 0

    @property
    def t_max(self) -> int:
        return self.t_past + 1

    def key(self, tensor_name: str, layer: int = 0, step: int = 0) -> int:
        return stream_key(self.seed, self.wid, layer, TENSOR_IDS[tensor_name], step)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Tiny OPT-125m-shaped layer, fp32 (parity workload).
OPT125M_LAYER = Workload("opt125m-layer-fp32", 1, 768, 3072, 12, 64, 128, 128, 307, 3, "f32")
# OPT-6.7B-shaped layer, fp16 weights, predictor rank 512, 5 % neurons / 20 % heads.
OPT6P7B_LAYER = Workload("opt6.7b-layer-fp16", 2, 4096, 16384, 32, 128, 512, 2048, 820, 7, "f16")
# OPT-66B-shaped layer, fp16, rank 1000 (density sweep; k set per point).
OPT66B_LAYER = Workload("opt66b-layer-fp16", 3, 9216, 36864, 72, 128, 1000, 2048, 1843, 14, "f16")
# OPT-175B-shaped 24-layer stack, fp16, rank 1000, 5 % neurons / 20 % heads, KV 2048 per layer.
OPT175B_STACK = Workload("opt175b-stack24-fp16", 4, 12288, 49152, 96, 128, 1000, 2048, 2458, 19,
                         "f16", n_layers=24)
# OPT-175B-shaped single layer, batched decode, KV 1024 per sequence.
OPT175B_BATCHED = Workload("opt175b-batched-fp16", 5, 12288, 49152, 96, 128, 1000, 1024, 2458, 19,
                           "f16")

# OPT-125m-shaped layer, fp32, for predictor training: up-projection biases shifted to -0.7
# so that about 10 % of the neurons fire (pre-activation std ~ 0.02 * sqrt(768) = 0.55);
# k = 10 % of the neurons, kh = 3 of 12 heads. Samples are single tokens (no past KV), so
# every head's output is its value vector, a function of the sample alone.
OPT125M_TRAIN = Workload("opt125m-train-fp32", 6, 768, 3072, 12, 64, 128, 0, 307, 3, "f32",
                         bias_sigma=0.02, b1_mean=-0.7)

WORKLOADS = {w.name: w for w in (OPT125M_LAYER, OPT6P7B_LAYER, OPT66B_LAYER, OPT175B_STACK,
                                 OPT175B_BATCHED, OPT125M_TRAIN)}

# Density sweep points of the OPT-66B-shaped layer.
SWEEP_MLP = (0.02, 0.05, 0.10, 0.25, 0.50, 1.00)
SWEEP_HEAD = (0.10, 0.20, 0.50, 1.00)


def count_at(density: float, n: int) -> int:
    """Kept count for a density: round half up of density * n."""
    return int(math.floor(density * n + 0.5))


def layer_shapes(w: Workload) -> Dict[str, Tuple[Tuple[int, ...], float, str]]:
    """Per-layer tensors: storage shape, std, storage type (vectors are fp32)."""
    d, F, H, dh, r = w.d_model, w.d_ffn, w.n_heads, w.head_dim, w.rank
    return {
        "p1_mlp": ((r, d), w.p_sigma, w.dtype),
        "p2_mlp": ((F, r), w.p_sigma, w.dtype),      # neuron-major: row j scores neuron j
        "p1_head": ((r, d), w.p_sigma, w.dtype),
        "p2_head": ((H, r), w.p_sigma, w.dtype),
        "wqkv": ((H, 3, dh, d), w.w_sigma, w.dtype),
        "bqkv": ((H, 3, dh), w.bias_sigma, "f32"),
        "wo": ((H, dh, d), w.w_sigma, w.dtype),
        "bo": ((d,), w.bias_sigma, "f32"),
        "w1t": ((F, d), w.w_sigma, w.dtype),
        "b1": ((F,), w.bias_sigma, "f32"),
        "w2": ((F, d), w.w_sigma, w.dtype),
        "b2": ((d,), w.bias_sigma, "f32"),
    }


def gains(w: Workload) -> np.ndarray:
    """RMSNorm gains: ones (the usual initialisation)."""
    return np.ones(w.d_model, np.float32)


def layer_tensors(w: Workload, layer: int = 0) -> Dict[str, np.ndarray]:
    """All tensors of one layer on the host (small workloads only)."""
    out = {name: tensor(w.key(name, layer), shp, sg, dt)
           for name, (shp, sg, dt) in layer_shapes(w).items()}
    out["g1"] = gains(w)
    out["g2"] = gains(w)
    if w.b1_mean != 0.0:
        out["b1"] = (out["b1"] + np.float32(w.b1_mean)).astype(np.float32)
    return out


def kv_shape(w: Workload) -> Tuple[int, int, int, int]:
    return (w.batch, w.n_heads, w.t_max, w.head_dim)


def kv_cache(w: Workload, which: str, layer: int = 0) -> np.ndarray:
    """Past KV cache [B][H][t_max][dh]; slots t_past..t_max-1 are zero."""
    shp = kv_shape(w)
    full = tensor(w.key(which, layer), shp, w.kv_sigma, w.dtype)
    full[:, :, w.t_past:, :] = 0
    return full


def x_input(w: Workload, step: int = 0, layer: int = 0) -> np.ndarray:
    """Layer input x [B][d] fp32 for one decode step."""
    return tensor(w.key("x", layer, step), (w.batch, w.d_model), w.x_sigma, "f32")


def zipf_scores(w: Workload, n: int, tensor_name: str, exponent: float = 1.1) -> np.ndarray:
    """Per-row selection scores for Zipf-skewed popularity (batched workload).

    Item popularity is rank**-exponent over a seeded random ranking; each row
    adds independent Gumbel noise to the log popularity. Keeping the k largest
    of these scores draws k items without replacement with probability
    proportional to popularity (the Gumbel-top-k construction).
    """
    key_perm = w.key(tensor_name, 0, 1 << 20)
    u = uniform01(key_perm, 0, n)
    ranks = np.argsort(np.argsort(u, kind="stable"), kind="stable") + 1   # seeded permutation of 1..n
    logw = -exponent * np.log(ranks.astype(np.float64))
    out = np.empty((w.batch, n), np.float32)
    for b in range(w.batch):
        ub = uniform01(w.key(tensor_name, 0, b), 0, n)
        ub = np.clip(ub, 1e-300, None)
        out[b] = (logw - np.log(-np.log(ub))).astype(np.float32)
    return out


def lowdim_x(w: Workload, n: int, dim: int = 32, noise: float = 0.1, mean_sigma: float = 1.0,
             split: int = 0) -> np.ndarray:
    """Layer inputs [n][d] fp32 near a seeded affine subspace of dimension dim.

    x = mu + g . U^T + e: a shared mean vector mu (elements of std `mean_sigma`), U [d][dim]
    of std 1/sqrt(dim) (so each element of g . U^T has variance about 1), coefficients
    g [n][dim] of std 1 and isotropic noise e of std `noise`. Formed in float64 and rounded
    once to fp32. `split` selects an independent draw of g and e (0: training samples,
    1: held-out samples) over the same mu and U. Stands in for hidden states, which have a
    shared mean direction and low intrinsic dimension; both are what let a linear predictor
    see which neurons fire and which heads are large.
    """
    mu = tensor(w.key("x_basis", 0, 1), (w.d_model,), mean_sigma, "f32").astype(np.float64)
    u = tensor(w.key("x_basis"), (w.d_model, dim), 1.0 / math.sqrt(dim), "f32").astype(np.float64)
    g = tensor(w.key("x_coef", 0, split), (n, dim), 1.0, "f32").astype(np.float64)
    e = tensor(w.key("x_noise", 0, split), (n, w.d_model), noise, "f32").astype(np.float64)
    return (mu[None] + g @ u.T + e).astype(np.float32)


def random_labels(w: Workload, n: int, width: int, p: float, split: int = 0) -> np.ndarray:
    """0/1 labels [n][width] uint8, each 1 with probability p (independent uniforms)."""
    u = uniform01(w.key("labels", 0, split), 0, n * width).reshape(n, width)
    return (u < p).astype(np.uint8)
