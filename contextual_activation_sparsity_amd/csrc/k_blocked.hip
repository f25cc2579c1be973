// Block scores for blocked-channel sparsity (DejaVu Guide, "Blocked Channel Sparsity"):
// neurons are grouped into contiguous blocks of bs and a block is loaded whole when it holds
// a highly active neuron, so a block ranks by its largest member score. NaN members count as
// lowest (a block of NaNs scores -inf, below every number).
#include "dv_device.h"
#include "dv_kernels.h"

namespace dv {

constexpr int kBlockScoreThreads = 256;

// One thread per (row, block); the block's members are read as 16-byte chunks, 4 in flight.
__global__ __launch_bounds__(kBlockScoreThreads) void block_scores_kernel(const float* scores, int B, int n, int bs,
                                                                          float* out) {
  const int nb = n / bs;
  const long long t = blockIdx.x * (long long)kBlockScoreThreads + threadIdx.x;
  if (t >= (long long)B * nb) return;
  const int b = (int)(t / nb), j = (int)(t - (long long)b * nb);
  const float* p = scores + (long long)b * n + (long long)j * bs;
  float m = -INFINITY;
  int e = 0;
  if ((bs & 3) == 0) {
    for (; e + 16 <= bs; e += 16) {
      f32x4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const f32x4*>(p + e + 4 * q);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) m = fmaxf(m, v[q][c] != v[q][c] ? -INFINITY : v[q][c]);
    }
  }
  for (; e < bs; ++e) {
    const float v = p[e];
    m = fmaxf(m, v != v ? -INFINITY : v);
  }
  out[(long long)b * nb + j] = m;
}

hipError_t launch_block_scores(const float* scores, int B, int n, int bs, float* out, hipStream_t s) {
  if (B < 1 || bs < 1 || n < bs || n % bs != 0) return hipErrorInvalidValue;
  const long long total = (long long)B * (n / bs);
  hipLaunchKernelGGL(block_scores_kernel, dim3((unsigned)((total + kBlockScoreThreads - 1) / kBlockScoreThreads)),
                     dim3(kBlockScoreThreads), 0, s, scores, B, n, bs, out);
  return hipGetLastError();
}

}  // namespace dv
