// Gather row-axpy kernel ("GEMV2" shape): out = sum over selected rows of coef * row.
//
// Used for the active-neuron down-projection (u . W2[S, :]) and the head-sparse output
// projection (o_h . Wo_h), DejaVu Guide, sparse MLP of "Step-by-Step Implementation" and
// "Head-Pruned Attention Dispatch". Both weights are stored with one contiguous row per
// neuron / per head element, so a selected row is a contiguous burst.
//
// Tiling: grid.x = column slices of TPC*VEC columns (one 16-byte chunk per thread and
// row), grid.y = row groups, grid.z = batch row. Inside a block, 256/TPC row lanes walk
// the group's rows with U rows in flight each and accumulate fp32 columns in registers.
// Row lanes are summed through LDS in lane order; row groups write fp32 partials and the
// last block to finish a slice (device-scope counter) sums the partials in group order,
// adds bias and residual and writes the output. The result is bitwise deterministic.
#include "dv_device.h"
#include "dv_kernels.h"

namespace dv {

constexpr int kAxpyBlock = 256;
constexpr int kAxpyMaxRG = 32;
constexpr int kAxpyU = 4;

template <typename WT, int TPC>
__global__ __launch_bounds__(kAxpyBlock) void rowaxpy_kernel(RowAxpyArgs a) {
  constexpr int VEC = Vec<WT>::N;
  constexpr int RL = kAxpyBlock / TPC;
  constexpr int CS = TPC * VEC;
  constexpr int U = kAxpyU;
  __shared__ float s_acc[RL][CS];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int rl = tid / TPC;
  const int cl = tid % TPC;
  const int slice = blockIdx.x;
  const int rg = blockIdx.y;
  const int b = blockIdx.z;
  const int col0 = slice * CS + cl * VEC;
  const bool colv = col0 < a.d;

  const int rpg = (a.n_rows + a.RG - 1) / a.RG;
  const int r_begin = rg * rpg;
  const int r_end = min(a.n_rows, r_begin + rpg);

  const WT* W = reinterpret_cast<const WT*>(a.W);
  const float* coef = a.coef + (long long)b * a.ldc;
  const int32_t* idxb = a.idx ? a.idx + (long long)b * a.idx_bstride : nullptr;

  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  for (int base = r_begin; base < r_end; base += RL * U) {
    // Row indices and coefficients first (wave-uniform when a wave is one row lane, so
    // they are scalar loads), then all U weight loads back to back.
    long long roff[U];
    float cf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int i = base + rl + u * RL;
      if constexpr (TPC == kWave) i = wave_uniform(i);
      cf[u] = 0.f;
      roff[u] = -1;
      if (i < r_end) {
        const int g = i / a.G;
        const int wi = i - g * a.G;
        const int grp = idxb ? idxb[g] : g;
        if ((unsigned)grp < (unsigned)a.n_groups) {
          cf[u] = coef[i];
          roff[u] = ((long long)grp * a.G + wi) * a.ld;
        }
      }
    }
    Chunk<WT> w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (colv && roff[u] >= 0) w[u] = load_chunk<WT>(W + roff[u] + col0);
      else w[u].raw = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float wf[VEC];
      widen(w[u], wf);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = fmaf(cf[u], wf[e], acc[e]);
    }
  }

#pragma unroll
  for (int e = 0; e < VEC; ++e) s_acc[rl][cl * VEC + e] = acc[e];
  __syncthreads();

  const long long obase = (long long)b * a.ldo;
  for (int c = tid; c < CS; c += kAxpyBlock) {
    const int col = slice * CS + c;
    if (col >= a.d) continue;
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < RL; ++r) v += s_acc[r][c];
    if (a.RG == 1) {
      if (a.bias) v += a.bias[col];
      if (a.resid) v += a.resid[(long long)b * a.ldr + col];
      a.out[obase + col] = v;
    } else {
      a.partial[((long long)b * a.RG + rg) * a.d + col] = v;
    }
  }
  if (a.RG == 1) return;

  // Publish this group's partial; the last group of the slice reduces.
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int prev = atomicAdd(&a.counters[b * a.n_slices + slice], 1);
    s_last = (prev == a.RG - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int c = tid; c < CS; c += kAxpyBlock) {
    const int col = slice * CS + c;
    if (col >= a.d) continue;
    float v = 0.f;
    const float* p = a.partial + (long long)b * a.RG * a.d + col;
    for (int r = 0; r < a.RG; ++r) v += p[(long long)r * a.d];
    if (a.bias) v += a.bias[col];
    if (a.resid) v += a.resid[(long long)b * a.ldr + col];
    a.out[obase + col] = v;
  }
  if (tid == 0) a.counters[b * a.n_slices + slice] = 0;
}

int rowaxpy_max_rg() { return kAxpyMaxRG; }

void rowaxpy_plan(int d, int n_rows, bool f16, int B, int cus, int* tpc, int* n_slices, int* RG) {
  const int vec = f16 ? 8 : 4;
  const int t = 64;
  const int cs = t * vec;
  const int ns = (d + cs - 1) / cs;
  const int rl = kAxpyBlock / t;
  long long target = (long long)cus * 3;
  long long rg = target / ((long long)ns * (B > 0 ? B : 1));
  const long long rows_cap = n_rows / (rl * kAxpyU);  // at least RL*U rows per group
  if (rg > rows_cap) rg = rows_cap;
  if (rg > kAxpyMaxRG) rg = kAxpyMaxRG;
  if (rg < 1) rg = 1;
  *tpc = t;
  *n_slices = ns;
  *RG = (int)rg;
}

hipError_t launch_rowaxpy(const RowAxpyArgs& a, bool f16, int tpc, int B, hipStream_t s) {
  if (tpc != 64) return hipErrorInvalidValue;
  dim3 grid(a.n_slices, a.RG, B);
  if (f16) hipLaunchKernelGGL((rowaxpy_kernel<half_t, 64>), grid, dim3(kAxpyBlock), 0, s, a);
  else hipLaunchKernelGGL((rowaxpy_kernel<float, 64>), grid, dim3(kAxpyBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace dv
