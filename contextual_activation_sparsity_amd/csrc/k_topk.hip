// Exact top-k of predictor scores by radix select (DejaVu Guide, "Mathematical
// Formulation of Lookahead Predictors": the active sets are the top-k of the scores;
// the guide's predictor returns the indices sorted).
//
// One block per (row, problem). Each thread owns a contiguous run of indices and keeps
// their 32-bit order keys in registers: finite floats map monotonically to unsigned
// keys with -0.0 folded onto +0.0, and every NaN maps to 0, below -inf. Four passes over
// 8-bit digits (histograms privatised per wavefront in LDS, then summed) find the k-th
// largest key tau and how many keys equal to tau are still needed. The output is written
// in ascending index order from a block-wide exclusive scan of per-thread counts: every
// key above tau, plus the lowest-index keys equal to tau. Integer-exact and unique.
#include "dv_device.h"
#include "dv_kernels.h"

namespace dv {

__device__ __forceinline__ unsigned order_key(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: lowest
  if (u == 0x80000000u) u = 0u;                     // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int BS>
__device__ __forceinline__ void block_excl_scan2(unsigned a, unsigned b, unsigned* ea, unsigned* eb,
                                                 unsigned (*s)[BS / kWave]) {
  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  unsigned ia = a, ib = b;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const unsigned ta = __shfl_up(ia, off, kWave);
    const unsigned tb = __shfl_up(ib, off, kWave);
    if (lane >= off) { ia += ta; ib += tb; }
  }
  if (lane == kWave - 1) { s[0][w] = ia; s[1][w] = ib; }
  __syncthreads();
  unsigned pa = 0, pb = 0;
  for (int i = 0; i < w; ++i) { pa += s[0][i]; pb += s[1][i]; }
  *ea = pa + ia - a;
  *eb = pb + ib - b;
}

template <int BS, int KPT>
__global__ __launch_bounds__(BS) void topk_kernel(TopkArgs a) {
  constexpr int NW = BS / kWave;
  __shared__ unsigned s_hist[NW][256];
  __shared__ unsigned s_tot[256];
  __shared__ unsigned s_sel[2];
  __shared__ unsigned s_scan[2][NW];

  const TopkProb& P = blockIdx.y == 0 ? a.p[0] : a.p[1];
  const int b = blockIdx.x;
  const int n = P.n;
  const int k = P.k;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  if (k <= 0) return;
  int32_t* out = P.out + (long long)b * k;
  if (k >= n) {
    for (int i = tid; i < n; i += BS) out[i] = i;
    return;
  }
  const float* sc = P.scores + (long long)b * n;
  const int per = (n + BS - 1) / BS;
  const int beg = tid * per;
  const int nv = max(0, min(per, n - beg));

  unsigned key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) key[j] = (j < nv) ? order_key(sc[beg + j]) : 0u;

  unsigned prefix = 0u, pmask = 0u, krem = (unsigned)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < NW * 256; i += BS) (&s_hist[0][0])[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (j < nv && (key[j] & pmask) == prefix) atomicAdd(&s_hist[w][(key[j] >> shift) & 255u], 1u);
    __syncthreads();
    for (int i = tid; i < 256; i += BS) {
      unsigned t = 0;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) t += s_hist[ww][i];
      s_tot[i] = t;
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l owns bins 255-4l .. 252-4l (descending digit order)
      unsigned cnt[4], tot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { cnt[j] = s_tot[255 - 4 * tid - j]; tot += cnt[j]; }
      unsigned incl = tot;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const unsigned t = __shfl_up(incl, off, kWave);
        if (tid >= off) incl += t;
      }
      unsigned before = incl - tot;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (before < krem && krem <= before + cnt[j]) {
          s_sel[0] = 255u - 4u * tid - j;
          s_sel[1] = krem - before;
        }
        before += cnt[j];
      }
    }
    __syncthreads();
    const unsigned dgt = s_sel[0];
    krem = s_sel[1];
    prefix |= dgt << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  const unsigned tau = prefix;

  unsigned gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (j < nv) { gt += key[j] > tau; eq += key[j] == tau; }
  }
  unsigned gt_before, eq_before;
  block_excl_scan2<BS>(gt, eq, &gt_before, &eq_before, s_scan);
  unsigned pos = gt_before + min(eq_before, krem);
  unsigned eq_seen = eq_before;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (j < nv) {
      if (key[j] > tau) {
        out[pos++] = beg + j;
      } else if (key[j] == tau) {
        if (eq_seen < krem) out[pos++] = beg + j;
        ++eq_seen;
      }
    }
  }
}

template <int BS, int KPT>
static void launch_one(const TopkArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL((topk_kernel<BS, KPT>), dim3(B, a.nprob), dim3(BS), 0, s, a);
}

hipError_t launch_topk(const TopkArgs& a, int B, hipStream_t s) {
  int nmax = 0;
  for (int i = 0; i < a.nprob; ++i) nmax = max(nmax, a.p[i].n);
  if (nmax > 65536) return hipErrorInvalidValue;
  if (nmax <= 1024) launch_one<256, 4>(a, B, s);
  else if (nmax <= 4096) launch_one<1024, 4>(a, B, s);
  else if (nmax <= 16384) launch_one<1024, 16>(a, B, s);
  else launch_one<1024, 64>(a, B, s);
  return hipGetLastError();
}

}  // namespace dv
