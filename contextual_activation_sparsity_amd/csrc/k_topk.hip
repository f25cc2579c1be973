// Exact top-k of predictor scores by radix select (DejaVu Guide, "Mathematical
// Formulation of Lookahead Predictors": the active sets are the top-k of the scores;
// the guide's predictor returns the indices sorted).
//
// One block per (row, problem). Each thread owns a contiguous run of indices and keeps
// their 32-bit order keys in registers: finite floats map monotonically to unsigned
// keys with -0.0 folded onto +0.0, and every NaN maps to 0, below -inf. Three passes over
// 11/11/10-bit digits (LDS histograms in four copies to spread atomics) find the k-th
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

// Exclusive scan over the block of up to two per-thread counts (thread order).
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
  __syncthreads();
}

constexpr int kTopkBins = 2048;   // 11-bit digits: passes over bits 31..21, 20..10, 9..0
constexpr int kTopkCopies = 4;    // histogram copies (wave w uses copy w % 4) to spread LDS atomics

template <int BS, int KPT>
__global__ __launch_bounds__(BS) void topk_kernel(TopkArgs a) {
  constexpr int NW = BS / kWave;
  constexpr int BPT = kTopkBins / BS;  // bins per thread in the digit search
  __shared__ unsigned s_hist[kTopkCopies][kTopkBins];
  __shared__ unsigned s_sel[2];
  __shared__ unsigned s_scan[2][NW];

  const TopkProb& P = blockIdx.y == 0 ? a.p[0] : a.p[1];
  const int b = blockIdx.x;
  const int n = P.n;
  const int k = P.k;
  const int tid = threadIdx.x;
  const int copy = (tid / kWave) % kTopkCopies;
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
  if ((per % 4) == 0 && (n % 4) == 0 && (reinterpret_cast<uintptr_t>(sc) & 15u) == 0) {
#pragma unroll
    for (int j = 0; j < KPT; j += 4) {
      if (j < nv) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(sc + beg + j);
        key[j] = order_key(v[0]); key[j + 1] = order_key(v[1]);
        key[j + 2] = order_key(v[2]); key[j + 3] = order_key(v[3]);
      } else {
        key[j] = key[j + 1] = key[j + 2] = key[j + 3] = 0u;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = (j < nv) ? order_key(sc[beg + j]) : 0u;
  }

  if (tid == 0) { s_sel[0] = 0u; s_sel[1] = 1u; }
  unsigned prefix = 0u, pmask = 0u, krem = (unsigned)k;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const unsigned dmask = pass == 2 ? 1023u : 2047u;
    for (int i = tid; i < kTopkCopies * kTopkBins; i += BS) (&s_hist[0][0])[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (j < nv && (key[j] & pmask) == prefix) atomicAdd(&s_hist[copy][(key[j] >> shift) & dmask], 1u);
    __syncthreads();
    // thread t owns BPT consecutive bins in descending digit order
    unsigned cnt[BPT], tot = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int bin = kTopkBins - 1 - (tid * BPT + j);
      unsigned c = 0;
#pragma unroll
      for (int q = 0; q < kTopkCopies; ++q) c += s_hist[q][bin];
      cnt[j] = c;
      tot += c;
    }
    unsigned before, unused;
    block_excl_scan2<BS>(tot, 0u, &before, &unused, s_scan);
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      if (before < krem && krem <= before + cnt[j]) {
        s_sel[0] = (unsigned)(kTopkBins - 1 - (tid * BPT + j));
        s_sel[1] = krem - before;
      }
      before += cnt[j];
    }
    __syncthreads();
    const unsigned dgt = s_sel[0];
    krem = s_sel[1];
    prefix |= dgt << shift;
    pmask |= dmask << shift;
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
      // pos < k always holds for a correct selection; the bound keeps writes in range regardless
      if (key[j] > tau) {
        if (pos < (unsigned)k) out[pos] = beg + j;
        ++pos;
      } else if (key[j] == tau) {
        if (eq_seen < krem) {
          if (pos < (unsigned)k) out[pos] = beg + j;
          ++pos;
        }
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
