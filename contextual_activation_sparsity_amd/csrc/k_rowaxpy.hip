// Gather row-axpy ("GEMV2" shape): out = sum over selected rows of coef * row (+ bias + resid).
//
// Used for the active-neuron down-projection (u . W2[S, :]) and the head-sparse output
// projection (o_h . Wo_h), DejaVu Guide, sparse MLP of "Step-by-Step Implementation" and
// "Head-Pruned Attention Dispatch". Both weights are stored with one contiguous row per
// neuron / per head element, so a selected row is a contiguous burst.
//
// Two kernels, no block ever waits on another (an in-kernel device-scope fence writes back
// an XCD's whole L2, which serialises badly on MI355X):
//  1. rowaxpy_part_kernel: grid = column slices x row groups x batch. A block owns a slice
//     of TPC 16-byte chunks (512 B of each fp16 row for TPC = 32, four whole cache lines)
//     and one group of consecutive selected rows. The group's row ids and coefficients are
//     staged in LDS first (all loads issued together), then 256/TPC row lanes stream the
//     rows with U loads in flight each and accumulate fp32 in registers; row lanes are
//     summed through LDS in lane order and the slice's partial is written.
//  2. rowaxpy_reduce_kernel: out = sum of the row groups' partials in group order + bias +
//     resid. With a single row group the first kernel writes the output directly.
// The sum order is fixed, so results are bitwise reproducible.
#include "reduce_body.h"

namespace dv {

#ifndef DV_AXPY_TPC
#define DV_AXPY_TPC 32     // threads per row slice: 32 x 16 B = 512 B of each fp16 row
#endif
#ifndef DV_AXPY_BPC
#define DV_AXPY_BPC 3      // target resident blocks per CU when choosing the row groups
#endif
#ifndef DV_AXPY_U
#define DV_AXPY_U 8        // rows in flight per thread
#endif
constexpr int kAxpyBlock = 256;
constexpr int kAxpyTpc = DV_AXPY_TPC;
constexpr int kAxpyU = DV_AXPY_U;
constexpr int kAxpyStage = 1024;  // rows whose ids/coefficients are staged per sweep

template <typename WT, int TPC>
__global__ __launch_bounds__(kAxpyBlock) void rowaxpy_part_kernel(RowAxpyArgs a) {
  constexpr int VEC = Vec<WT>::N;
  constexpr int RL = kAxpyBlock / TPC;   // row lanes
  constexpr int CS = TPC * VEC;          // columns per slice
  constexpr int U = kAxpyU;
  constexpr int PT = kAxpyStage / kAxpyBlock;
  __shared__ int s_row[kAxpyStage];
  __shared__ float s_coef[kAxpyStage];
  __shared__ float s_red[RL][CS];

  const int tid = threadIdx.x;
  const int rl = tid / TPC;
  const int cl = tid % TPC;
  const int slice = blockIdx.x;
  const int rg = blockIdx.y;
  const int b = blockIdx.z;
  const int col0 = slice * CS + cl * VEC;
  const bool colv = col0 < a.d;
  const int rpg = (a.n_rows + a.RG - 1) / a.RG;
  const int r_begin = min(a.n_rows, rg * rpg);
  const int r_end = min(a.n_rows, r_begin + rpg);

  const WT* W = reinterpret_cast<const WT*>(a.W);
  const float* coef = a.coef + (long long)b * a.ldc;
  const int32_t* idxb = a.idx ? a.idx + (long long)b * a.idx_bstride : nullptr;

  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  for (int r0 = r_begin; r0 < r_end; r0 += kAxpyStage) {  // block-uniform
    const int nst = min(kAxpyStage, r_end - r0);
    __syncthreads();
    int grp[PT], wi[PT];
    float cv[PT];
#pragma unroll
    for (int q = 0; q < PT; ++q) {  // every index/coefficient load is issued before any is used
      const int i = tid + q * kAxpyBlock;
      const int ii = r0 + i;
      const int g = ii / a.G;
      wi[q] = ii - g * a.G;
      grp[q] = -1;
      cv[q] = 0.f;
      if (i < nst) {
        grp[q] = idxb ? idxb[g] : g;
        cv[q] = coef[ii];
      }
    }
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int i = tid + q * kAxpyBlock;
      if (i < nst) {
        const bool ok = (unsigned)grp[q] < (unsigned)a.n_groups;
        s_row[i] = ok ? grp[q] * a.G + wi[q] : -1;
        s_coef[i] = ok ? cv[q] : 0.f;
      }
    }
    __syncthreads();
    for (int j0 = rl; j0 < nst; j0 += RL * U) {
      Chunk<WT> w[U];
      float cf[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * RL;
        const int ro = j < nst ? s_row[j] : -1;
        cf[u] = j < nst ? s_coef[j] : 0.f;
        if (colv && ro >= 0) w[u] = load_chunk<WT>(W + (long long)ro * a.ld + col0);
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
  }

#pragma unroll
  for (int e = 0; e < VEC; ++e) s_red[rl][cl * VEC + e] = acc[e];
  __syncthreads();
  for (int c = tid; c < CS; c += kAxpyBlock) {
    const int col = slice * CS + c;
    if (col >= a.d) continue;
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < RL; ++r) v += s_red[r][c];
    if (a.RG == 1) {
      if (a.bias) v += a.bias[col];
      if (a.resid) v += a.resid[(long long)b * a.ldr + col];
      a.out[(long long)b * a.ldo + col] = v;
    } else {
      a.partial[((long long)b * a.RG + rg) * a.d + col] = v;
    }
  }
}

// out[b][c] = sum_rg partial[b][rg][c] (group order; none if partial is null) + bias[c] + resid[b][c]; 4 columns per
// thread, small blocks so the few hundred KB of partials are read by many CUs at once.
constexpr int kReduceBlock = 64;
__global__ __launch_bounds__(kReduceBlock) void rowaxpy_reduce_kernel(RowAxpyArgs a) {
  axpy_reduce_block<kReduceBlock>(a, blockIdx.x, blockIdx.y);
}

int rowaxpy_max_rg() { return kAxpyMaxRG; }

void rowaxpy_plan(int d, int n_rows, bool f16, int B, int cus, int* tpc, int* n_slices, int* RG) {
  const int vec = f16 ? 8 : 4;
  const int t = kAxpyTpc;
  const int cs = t * vec;
  const int ns = (d + cs - 1) / cs;
  const int rl = kAxpyBlock / t;
  long long rg = (long long)cus * DV_AXPY_BPC / ((long long)ns * (B > 0 ? B : 1));
  const long long rows_cap = n_rows / (rl * 4);  // at least 4 rows per row lane and group
  if (rg > rows_cap) rg = rows_cap;
  if (rg > kAxpyMaxRG) rg = kAxpyMaxRG;
  if (rg < 1) rg = 1;
  *tpc = t;
  *n_slices = ns;
  *RG = (int)rg;
}

hipError_t launch_rowaxpy_part(const RowAxpyArgs& a, bool f16, int tpc, int B, hipStream_t s) {
  if (tpc != kAxpyTpc) return hipErrorInvalidValue;
  dim3 grid(a.n_slices, a.RG, B);
  if (f16) hipLaunchKernelGGL((rowaxpy_part_kernel<half_t, kAxpyTpc>), grid, dim3(kAxpyBlock), 0, s, a);
  else hipLaunchKernelGGL((rowaxpy_part_kernel<float, kAxpyTpc>), grid, dim3(kAxpyBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rowaxpy(const RowAxpyArgs& a, bool f16, int tpc, int B, hipStream_t s) {
  hipError_t e = launch_rowaxpy_part(a, f16, tpc, B, s);
  if (e != hipSuccess || a.RG == 1) return e;
  return launch_axpy_reduce(a, B, s);
}

hipError_t launch_axpy_reduce(const RowAxpyArgs& a, int B, hipStream_t s) {
  if (a.RG < 1 || a.RG > kAxpyMaxRG || a.d % 4 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rowaxpy_reduce_kernel, dim3((a.d / 4 + kReduceBlock - 1) / kReduceBlock, B),
                     dim3(kReduceBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace dv
