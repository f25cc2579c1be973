// A plain streaming read, the bench's reference for what a read-only kernel reaches on this
// GPU: every 16-byte chunk of a buffer is loaded once (non-temporal, eight loads in flight per
// thread, grid-stride), folded with XOR, and a word is stored only on an improbable fold value
// so the loads stay live without writing anything in practice.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* p, long long n, uint32_t* sink) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

// Reads bytes (a multiple of 16) from the 16-byte aligned device buffer p with `blocks`
// blocks of 256 threads; sink holds `blocks` words. Returns the HIP error code (0 = success).
extern "C" int dv_synth_stream_read(const void* p, long long bytes, void* sink, int blocks, hipStream_t s) {
  if (p == nullptr || sink == nullptr || bytes <= 0 || bytes % 16 != 0 || blocks <= 0) return (int)hipErrorInvalidValue;
  if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<const u32x4*>(p), bytes / 16,
                     reinterpret_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}
