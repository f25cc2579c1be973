// Device helpers shared by the gfx950 kernels: 16-byte vector loads of the storage
// type, fp32 widening, wavefront reductions. Wavefronts are 64 lanes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dv {

constexpr int kWave = 64;

typedef _Float16 half_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Number of storage elements in one 16-byte chunk.
template <typename WT> struct Vec;
template <> struct Vec<half_t> { static constexpr int N = 8; };
template <> struct Vec<float> { static constexpr int N = 4; };

// One 16-byte chunk of weights, kept packed until it is consumed.
template <typename WT> struct Chunk { u32x4 raw; };

template <typename WT>
__device__ __forceinline__ Chunk<WT> load_chunk(const WT* p) {
  Chunk<WT> c;
  c.raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return c;
}

template <typename WT>
__device__ __forceinline__ Chunk<WT> load_chunk_cached(const WT* p) {
  Chunk<WT> c;
  c.raw = *reinterpret_cast<const u32x4*>(p);
  return c;
}

// Widen element e of a chunk to fp32.
__device__ __forceinline__ void widen(const Chunk<half_t>& c, float* out) {
  h16x8 h = __builtin_bit_cast(h16x8, c.raw);
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = static_cast<float>(h[e]);
}
__device__ __forceinline__ void widen(const Chunk<float>& c, float* out) {
  f32x4 f = __builtin_bit_cast(f32x4, c.raw);
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = f[e];
}

template <typename WT> __device__ __forceinline__ WT narrow(float v);
template <> __device__ __forceinline__ half_t narrow<half_t>(float v) { return static_cast<half_t>(v); }
template <> __device__ __forceinline__ float narrow<float>(float v) { return v; }

// Sum over groups of `width` consecutive lanes (width a power of two <= 64); every lane of
// the group receives the group's total. The xor-butterfly gives every lane the same bits.
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = width / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

template <int width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int off = width / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace dv
