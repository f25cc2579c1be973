// Device filler for the seeded synthetic inputs (the same generator as synth/__init__.py).
//
// Element i of a stream with key K is the SplitMix64 output mix64(K + (i+1)*0x9E3779B97F4A7C15)
// (Steele, Lea and Flood, OOPSLA 2014). Its four 16-bit lanes are summed, the sum is centred
// by the exact integer 2*65535, converted exactly to fp32 and multiplied once by an fp32
// scale; fp16 storage rounds that product to nearest-even. The host implementation does the
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

template <typename T>
__global__ void fill_kernel(T* out, long long n, uint64_t key, float scale, long long start) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = (T)draw(key, (uint64_t)(start + i), scale);
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
    hipLaunchKernelGGL(fill_kernel<float>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       static_cast<float*>(out), n, (uint64_t)key, scale, start);
  else
    hipLaunchKernelGGL(fill_kernel<_Float16>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       static_cast<_Float16*>(out), n, (uint64_t)key, scale, start);
  return (int)hipGetLastError();
}

}  // extern "C"
