// Opt-in validation of caller-supplied index lists.
//
// The sparse gathers take the active neurons and heads as ascending lists of unique indices,
// the form the predictor's top-k hands over (DejaVu Guide, "Step-by-Step Implementation":
// the predictor returns sorted indices and the sparse forward consumes them). A list that
// breaks that form gives results that depend on the path: the row-wise gathers add a
// repeated neuron twice, while the batched path's union bitmap keeps it once. This kernel
// reports, per row, which rule a list breaks, so a caller can check its lists before use.
//
// One block per row. Thread t looks at entries t, t + 256, ... and compares each with its
// predecessor; the flags are OR-reduced over the wavefront with shuffles and over the
// block's waves through LDS, and thread 0 writes the row's status word. OR is order
// independent, so the result does not depend on scheduling.
#include "dv_device.h"
#include "dv_kernels.h"

namespace dv {

constexpr int kCheckBlock = 256;

__global__ __launch_bounds__(kCheckBlock) void check_indices_kernel(const int32_t* idx, int k, int n,
                                                                    int32_t* status) {
  __shared__ int s_flags[kCheckBlock / kWave];
  const int b = blockIdx.x;
  const int32_t* row = idx + (long long)b * k;
  int flags = 0;
  for (int j = threadIdx.x; j < k; j += kCheckBlock) {
    const int cur = row[j];
    if (cur < 0 || cur >= n) flags |= kIdxRange;
    if (j > 0) {
      const int prev = row[j - 1];
      if (cur < prev) flags |= kIdxOrder;
      if (cur == prev) flags |= kIdxDuplicate;
    }
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) flags |= __shfl_xor(flags, off, kWave);
  if ((threadIdx.x % kWave) == 0) s_flags[threadIdx.x / kWave] = flags;
  __syncthreads();
  if (threadIdx.x == 0) {
    int all = 0;
#pragma unroll
    for (int w = 0; w < kCheckBlock / kWave; ++w) all |= s_flags[w];
    status[b] = all;
  }
}

hipError_t launch_check_indices(const int32_t* idx, int B, int k, int n, int32_t* status, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_indices_kernel, dim3(B), dim3(kCheckBlock), 0, s, idx, k, n, status);
  return hipGetLastError();
}

}  // namespace dv
