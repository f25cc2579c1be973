// Predictor training: targets from the dense layer and gradient steps of the rank-r score map
// (DejaVu Guide, "Mathematical Formulation of Lookahead Predictors": the head predictor marks
// the heads with the largest attention norms, the neuron predictor the neurons that fire; blog
// summary "What Is Contextual Sparsity?": the classifiers are trained offline on the dense
// model's activations, with the layer input as features).
//
// Loss: mean binary cross-entropy of the scores (logits) over every (sample, output) pair,
// computed in the epilogue of the product that forms the scores;
// optimiser: full-batch gradient descent with heavy-ball momentum. The contractions are fp32
// GEMMs on the matrix cores; every reduction runs in a fixed order, so a step is bitwise
// reproducible.
#include <algorithm>

#include "dv_device.h"
#include "dv_kernels.h"

namespace dv {

constexpr int kGemmK = 16;
constexpr int kGemmThreads = 256;

// ---------------------------------------------------------------------------
// Targets
// ---------------------------------------------------------------------------
__global__ void iota_rows_kernel(int32_t* out, int rows, int n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (long long)rows * n) out[i] = (int32_t)(i % n);
}

// ||o_h||_2 for every (row, head); o is [B][H][dh] fp32.
__global__ void head_norm_kernel(const float* o, int BH, int dh, float* norm) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= BH) return;
  const float* v = o + (long long)i * dh;
  float s = 0.f;
  for (int e = 0; e < dh; ++e) s = fmaf(v[e], v[e], s);
  norm[i] = sqrtf(s);
}

__global__ void fire_kernel(const float* a, long long n, uint8_t* fire) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) fire[i] = a[i] > 0.f ? 1 : 0;
}

hipError_t launch_iota_rows(int32_t* out, int rows, int n, hipStream_t s) {
  const long long total = (long long)rows * n;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(iota_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, out, rows, n);
  return hipGetLastError();
}

hipError_t launch_head_norm(const float* o, int BH, int dh, float* norm, hipStream_t s) {
  if (BH <= 0) return hipSuccess;
  hipLaunchKernelGGL(head_norm_kernel, dim3((BH + 255) / 256), dim3(256), 0, s, o, BH, dh, norm);
  return hipGetLastError();
}

hipError_t launch_fire(const float* a, long long n, uint8_t* fire, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fire_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, n, fire);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 GEMM with strided operands on the matrix cores: C[i][j] = sum_k A(i,k) B(k,j),
// A(i,k) = A[i*sai + k*sak], B(k,j) = B[k*sbk + j*sbj]. A 128 x 128 output tile per block of
// 4 waves (64 x 64 per wave, 4 x 4 tiles of v_mfma_f32_16x16x4f32), K in steps of 16 staged
// in LDS k-major (each operand loaded along its contiguous axis), the next step's loads in
// flight during the MFMAs. With more than one slice, slice z of the K range writes its
// partial tile to C + z*M*N and a second kernel sums the slices in order.
// ---------------------------------------------------------------------------
typedef float f4t __attribute__((ext_vector_type(4)));
constexpr int kMT = 128;                       // output tile edge
constexpr int kMLd = kMT + 4;                  // padded LDS row (floats)
constexpr int kMLoads = kMT * kGemmK / kGemmThreads;   // operand elements per thread per step

__global__ __launch_bounds__(kGemmThreads) void gemm_f32_kernel(GemmF32Args a, int k_per_slice) {
  __shared__ float As[kGemmK][kMLd];
  __shared__ float Bs[kGemmK][kMLd];
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int lr = lane % 16, lg = lane / 16;
  const int wi = (wv / 2) * 64, wj = (wv % 2) * 64;   // this wave's 64 x 64 quarter
  const int i0 = blockIdx.y * kMT, j0 = blockIdx.x * kMT;
  const int kb = blockIdx.z * k_per_slice;
  const int ke = min(a.K, kb + k_per_slice);
  const bool a_kfast = a.sak == 1;
  const bool b_jfast = a.sbj == 1;
  float ra[kMLoads], rb[kMLoads];
  auto load = [&](int k0) {
#pragma unroll
    for (int q = 0; q < kMLoads; ++q) {
      const int e = tid + q * kGemmThreads;
      const int ii = a_kfast ? e / kGemmK : e % kMT;
      const int kk = a_kfast ? e % kGemmK : e / kMT;
      const int gi = i0 + ii, gk = k0 + kk;
      ra[q] = (gi < a.M && gk < ke) ? a.A[(long long)gi * a.sai + (long long)gk * a.sak] : 0.f;
      const int jj = b_jfast ? e % kMT : e / kGemmK;
      const int k2 = b_jfast ? e / kMT : e % kGemmK;
      const int gj = j0 + jj, gk2 = k0 + k2;
      rb[q] = (gj < a.N && gk2 < ke) ? a.B[(long long)gk2 * a.sbk + (long long)gj * a.sbj] : 0.f;
    }
  };
  f4t acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f4t{0.f, 0.f, 0.f, 0.f};
  if (kb < ke) load(kb);
  for (int k0 = kb; k0 < ke; k0 += kGemmK) {   // block-uniform
    __syncthreads();   // the previous step's readers are done
#pragma unroll
    for (int q = 0; q < kMLoads; ++q) {
      const int e = tid + q * kGemmThreads;
      As[a_kfast ? e % kGemmK : e / kMT][a_kfast ? e / kGemmK : e % kMT] = ra[q];
      Bs[b_jfast ? e / kMT : e % kGemmK][b_jfast ? e % kMT : e / kGemmK] = rb[q];
    }
    __syncthreads();
    if (k0 + kGemmK < ke) load(k0 + kGemmK);
#pragma unroll
    for (int ks = 0; ks < kGemmK / 4; ++ks) {
      const int k = 4 * ks + lg;   // A: row lr, k = lg; B: column lr, k = lg
      float av[4], bv[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) av[m] = As[k][wi + 16 * m + lr];
#pragma unroll
      for (int n = 0; n < 4; ++n) bv[n] = Bs[k][wj + 16 * n + lr];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[m], bv[n], acc[m][n], 0, 0, 0);
    }
  }
  // D layout: lane holds column lr of its tile, rows 4*lg + e
  float* C = a.C + (long long)blockIdx.z * a.M * a.N;
  float lsum = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int gi = i0 + wi + 16 * m + 4 * lg + e;
      if (gi >= a.M) continue;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int gj = j0 + wj + 16 * n + lr;
        if (gj >= a.N) continue;
        const long long o = (long long)gi * a.N + gj;
        float v = acc[m][n][e];
        if (a.bce_y) {   // loss term softplus(s) - y s, and the gradient (sigmoid(s) - y) / n
          const float t = a.bce_y[o] ? 1.f : 0.f;
          const float ex = expf(-fabsf(v));
          lsum += fmaxf(v, 0.f) + log1pf(ex) - t * v;
          const float sig = v >= 0.f ? 1.f / (1.f + ex) : ex / (1.f + ex);
          v = (sig - t) * a.inv_n;
        }
        C[o] = v;
      }
    }
  if (a.bce_y) {   // block sum in a fixed order: lanes by butterfly, then waves in order
    __shared__ float s_loss[kGemmThreads / kWave];
    lsum = group_sum<kWave>(lsum);
    if (lane == 0) s_loss[wv] = lsum;
    __syncthreads();
    if (tid == 0) {
      float t = 0.f;
      for (int w = 0; w < kGemmThreads / kWave; ++w) t += s_loss[w];
      a.bce_part[blockIdx.y * gridDim.x + blockIdx.x] = t;
    }
  }
}

__global__ void sum_slices_kernel(const float* part, int slices, long long n, float* out) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = part[i];
  for (int z = 1; z < slices; ++z) s += part[(long long)z * n + i];
  out[i] = s;
}

int gemm_f32_slices(int M, int N, int K, int cus) {
  const long long tiles = (long long)((M + kMT - 1) / kMT) * ((N + kMT - 1) / kMT);
  const long long want = 2LL * cus;
  int ks = (int)std::min<long long>((want + tiles - 1) / tiles, std::max(1, K / 256));
  return std::max(1, std::min(ks, kGemmMaxSlices));
}

// C = op(A) op(B); with more than one slice, `scratch` holds slices*M*N floats.
hipError_t launch_gemm_f32(GemmF32Args a, int slices, float* scratch, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.K <= 0 || slices < 1) return hipErrorInvalidValue;
  if (a.bce_y != nullptr && slices != 1) return hipErrorInvalidValue;   // the epilogue needs whole sums
  int kps = (a.K + slices - 1) / slices;
  kps = (kps + kGemmK - 1) / kGemmK * kGemmK;
  slices = std::max(1, (a.K + kps - 1) / kps);
  float* dst = a.C;
  if (slices > 1) a.C = scratch;
  dim3 grid((a.N + kMT - 1) / kMT, (a.M + kMT - 1) / kMT, slices);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(kGemmThreads), 0, s, a, std::max(kps, 1));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || slices == 1) return e;
  const long long n = (long long)a.M * a.N;
  hipLaunchKernelGGL(sum_slices_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, scratch, slices, n, dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Loss: the cross-entropy epilogue's block parts summed by one block in a fixed order (each
// thread adds a fixed strided subset in index order, then a pairwise tree over the threads).
// ---------------------------------------------------------------------------
constexpr int kFinishThreads = 1024;
__global__ __launch_bounds__(kFinishThreads) void loss_finish_kernel(const float* part, int n_part, float inv_n,
                                                                     float* loss) {
  __shared__ float s_t[kFinishThreads];
  float t = 0.f;
  for (int i = threadIdx.x; i < n_part; i += kFinishThreads) t += part[i];
  s_t[threadIdx.x] = t;
  __syncthreads();
  for (int w = kFinishThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) s_t[threadIdx.x] += s_t[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = s_t[0] * inv_n;
}

hipError_t launch_loss_finish(const float* part, int n_part, float inv_n, float* loss, hipStream_t s) {
  hipLaunchKernelGGL(loss_finish_kernel, dim3(1), dim3(kFinishThreads), 0, s, part, n_part, inv_n, loss);
  return hipGetLastError();
}

int gemm_f32_blocks(int M, int N) { return ((M + kMT - 1) / kMT) * ((N + kMT - 1) / kMT); }

// v = mu v + g; p = p - lr v, over two parameter arrays in one launch.
__global__ void momentum_step_kernel(float* p1, float* v1, const float* g1, long long n1, float* p2, float* v2,
                                     const float* g2, long long n2, float lr, float mu) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  float *p, *v;
  const float* g;
  if (i < n1) {
    p = p1; v = v1; g = g1;
  } else {
    i -= n1;
    if (i >= n2) return;
    p = p2; v = v2; g = g2;
  }
  const float vn = fmaf(mu, v[i], g[i]);
  v[i] = vn;
  p[i] = p[i] - lr * vn;
}

hipError_t launch_momentum_step(float* p1, float* v1, const float* g1, long long n1, float* p2, float* v2,
                                const float* g2, long long n2, float lr, float mu, hipStream_t s) {
  const long long n = n1 + n2;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(momentum_step_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p1, v1, g1, n1, p2,
                     v2, g2, n2, lr, mu);
  return hipGetLastError();
}

}  // namespace dv
