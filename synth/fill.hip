// Device filler for the seeded synthetic inputs (the same generator as synth/__init__.py).
//
// Element i of a stream with key K is the SplitMix64 output mix64(K + (i+1)*0x9E3779B97F4A7C15)
// (Steele, Lea and Flood, OOPSLA 2014). Its four 16-bit lanes are summed, the sum is centred
// by the exact integer 2*65535, converted exactly to fp32 and multiplied once by an fp32
// scale; fp16 storage rounds that product to nearest-even (explicitly, below). The host implementation does the
// same operations, so both produce identical bits. This file draws numbers only.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float draw(uint64_t key, uint64_t ctr, float scale) {
  const uint64_t b = mix64(key + (ctr + 1ull) * 0x9E3779B97F4A7C15ull);
  const int s = (int)(b & 0xFFFFu) + (int)((b >> 16) & 0xFFFFu) + (int)((b >> 32) & 0xFFFFu) + (int)(b >> 48);
  const float z = (float)(s - 131070);
  return __fmul_rn(z, scale);
}

// IEEE 754 binary32 -> binary16, round to nearest, ties to even, written out in integer
// arithmetic so the result does not depend on which conversion instruction the compiler
// picks (the packed conversion rounded an exact tie differently from the host).
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  const uint32_t x = __float_as_uint(f);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) return (uint16_t)(sign | 0x7c00u | (ax > 0x7f800000u ? 0x200u : 0u));  // inf, nan
  if (ax >= 0x47800000u) return (uint16_t)(sign | 0x7c00u);   // overflow to inf (|f| >= 65536)
  if (ax < 0x38800000u) {                                     // below the smallest normal half
    if (ax < 0x33000000u) return (uint16_t)sign;              // below half the smallest subnormal
    const uint32_t m = (ax & 0x7fffffu) | 0x800000u;
    const int sh = 126 - (int)(ax >> 23);                     // 14..24
    uint32_t q = m >> sh;
    const uint32_t rem = m & ((1u << sh) - 1u), half = 1u << (sh - 1);
    q += (rem > half) || (rem == half && (q & 1u));
    return (uint16_t)(sign | q);
  }
  const uint32_t t = ax - 0x38000000u;                        // rebias the exponent 127 -> 15
  uint32_t q = t >> 13;
  const uint32_t rem = t & 0x1fffu;
  q += (rem > 0x1000u) || (rem == 0x1000u && (q & 1u));       // a carry may bump the exponent
  return (uint16_t)(sign | q);
}

__global__ void fill_f32_kernel(float* out, long long n, uint64_t key, float scale, long long start) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = draw(key, (uint64_t)(start + i), scale);
}

__global__ void fill_f16_kernel(uint16_t* out, long long n, uint64_t key, float scale, long long start) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = f32_to_f16_rne(draw(key, (uint64_t)(start + i), scale));
}

}  // namespace

extern "C" {

// dtype 0 = fp32, 1 = fp16. Returns a hipError_t value (0 on success).
int dv_synth_fill(void* out, long long n, int dtype, unsigned long long key, float scale, long long start,
                  hipStream_t stream) {
  if (out == nullptr || n < 0 || (dtype != 0 && dtype != 1)) return (int)hipErrorInvalidValue;
  if (n == 0) return 0;
  const int threads = 256;
  long long blocks = (n + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  if (dtype == 0)
    hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       static_cast<float*>(out), n, (uint64_t)key, scale, start);
  else
    hipLaunchKernelGGL(fill_f16_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       static_cast<uint16_t*>(out), n, (uint64_t)key, scale, start);
  return (int)hipGetLastError();
}

}  // extern "C"
