// Device body of the ordered reduce that finishes a row-axpy: out = sum of the row groups'
// partials in group order + bias + residual, 4 columns per thread.
#pragma once
#include "dv_device.h"
#include "dv_kernels.h"

namespace dv {

constexpr int kAxpyMaxRG = 32;

// Block bx of NT threads, batch row b: columns (bx * NT + thread) * 4 .. + 3.
template <int NT>
__device__ __forceinline__ void axpy_reduce_block(const RowAxpyArgs& a, int bx, int b) {
  const int c0 = (bx * NT + (int)threadIdx.x) * 4;
  if (c0 >= a.d) return;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if (a.partial != nullptr) {   // no partials: bias + residual only
    const float* p = a.partial + (long long)b * a.RG * a.d + c0;
    f32x4 v[kAxpyMaxRG];
#pragma unroll
    for (int r = 0; r < kAxpyMaxRG; ++r)
      if (r < a.RG) v[r] = *reinterpret_cast<const f32x4*>(p + (long long)r * a.d);
#pragma unroll
    for (int r = 0; r < kAxpyMaxRG; ++r)
      if (r < a.RG) s += v[r];
  }
  if (a.bias) s += *reinterpret_cast<const f32x4*>(a.bias + c0);
  if (a.resid) s += *reinterpret_cast<const f32x4*>(a.resid + (long long)b * a.ldr + c0);
  *reinterpret_cast<f32x4*>(a.out + (long long)b * a.ldo + c0) = s;
}

}  // namespace dv
