// Exact top-k of predictor scores (DejaVu Guide, "Mathematical Formulation of Lookahead
// Predictors": the active sets are the top-k of the scores; the guide's predictor returns
// the indices sorted).
//
// Order: scores map to 32-bit unsigned keys that order like the floats, with -0.0 folded
// onto +0.0 and every NaN mapped to 0 (below -inf). The k largest keys win; among equal
// keys the lower index wins. Output is the selected indices in ascending order.
//
// One block of 1024 threads per (row, problem); one CU retires 64 lane-ops per clock, so
// the design minimises sweeps over the keys:
//  1. Coalesced striped load (element t + 1024 j goes to thread t, register j), fused with
//     the histogram of the top 11 key bits (LDS, four copies to spread atomics). A scan of
//     the 2048 bins gives the bin holding the k-th largest key and how many keys above it
//     are already taken.
//  2. The keys of that bin are compacted into LDS (typically 1-3 % of n) and the remaining
//     21 bits are resolved there (11 + 10 bit passes). If the bin holds more keys than the
//     LDS list, the two passes run over the registers instead.
//  3. The threshold key tau and the number r of keys equal to tau still needed are known.
//     Each wave ballots "key > tau" and "key == tau" for each register row; one block scan
//     of the per-(row, wave) counts in index order gives every selected element its output
//     position, and a tie is taken iff fewer than r ties precede it in index order.
// Integer-exact and unique.
#include "dv_device.h"
#include "dv_kernels.h"

namespace dv {

__device__ __forceinline__ unsigned order_key(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: lowest
  if (u == 0x80000000u) u = 0u;                     // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkBlock = 1024;
constexpr int kTopkWaves = kTopkBlock / kWave;
constexpr int kTopkBins = 2048;   // 11-bit digits: bits 31..21, then 20..10, then 9..0
constexpr int kTopkCopies = 4;    // histogram copies (wave w uses copy w % 4)
constexpr int kTopkCand = 4096;   // LDS list for the keys of the threshold bin

// Exclusive scan over the block of two per-thread counts (thread order); also returns the totals.
__device__ __forceinline__ void block_scan2(unsigned a, unsigned b, unsigned* ea, unsigned* eb,
                                            unsigned* ta, unsigned* tb, unsigned (*s)[kTopkWaves]) {
  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  unsigned ia = a, ib = b;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const unsigned xa = __shfl_up(ia, off, kWave);
    const unsigned xb = __shfl_up(ib, off, kWave);
    if (lane >= off) { ia += xa; ib += xb; }
  }
  if (lane == kWave - 1) { s[0][w] = ia; s[1][w] = ib; }
  __syncthreads();
  unsigned pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int i = 0; i < kTopkWaves; ++i) {
    if (i < w) { pa += s[0][i]; pb += s[1][i]; }
    sa += s[0][i]; sb += s[1][i];
  }
  *ea = pa + ia - a;
  *eb = pb + ib - b;
  *ta = sa;
  *tb = sb;
  __syncthreads();
}

// Finds the digit bin holding the krem-th largest key (counting from the top) in a histogram
// of nbins bins; returns the bin in s_sel[0] and the rank inside it in s_sel[1].
__device__ __forceinline__ void find_bin(const unsigned (*hist)[kTopkBins], int nbins, unsigned krem,
                                         unsigned* s_sel, unsigned (*s_scan)[kTopkWaves]) {
  constexpr int BPT = kTopkBins / kTopkBlock;  // 2 bins per thread, descending digit order
  const int tid = threadIdx.x;
  unsigned cnt[BPT], tot = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int bin = nbins - 1 - (tid * BPT + j);
    unsigned c = 0;
    if (bin >= 0)
#pragma unroll
      for (int q = 0; q < kTopkCopies; ++q) c += hist[q][bin];
    cnt[j] = c;
    tot += c;
  }
  unsigned before, unused, t0, t1;
  block_scan2(tot, 0u, &before, &unused, &t0, &t1, s_scan);
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    if (before < krem && krem <= before + cnt[j]) {
      s_sel[0] = (unsigned)(nbins - 1 - (tid * BPT + j));
      s_sel[1] = krem - before;
    }
    before += cnt[j];
  }
  __syncthreads();
}

template <int KPT>
__global__ __launch_bounds__(kTopkBlock) void topk_kernel(TopkArgs a) {
  __shared__ unsigned s_hist[kTopkCopies][kTopkBins];
  __shared__ unsigned s_cand[kTopkCand];
  __shared__ unsigned s_cnt[2][KPT][kTopkWaves];
  __shared__ unsigned s_sel[2];
  __shared__ unsigned s_ncand;
  __shared__ unsigned s_scan[2][kTopkWaves];

  const TopkProb& P = blockIdx.y == 0 ? a.p[0] : a.p[1];
  const int b = blockIdx.x;
  const int n = P.n;
  const int k = P.k;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int w = tid / kWave;
  const int copy = w % kTopkCopies;
  if (k <= 0) return;
  int32_t* out = P.out + (long long)b * k;
  if (k >= n) {
    for (int i = tid; i < n; i += kTopkBlock) out[i] = i;
    return;
  }
  const float* sc = P.scores + (long long)b * n;

  for (int i = tid; i < kTopkCopies * kTopkBins; i += kTopkBlock) (&s_hist[0][0])[i] = 0u;
  if (tid == 0) { s_sel[0] = 0u; s_sel[1] = 1u; s_ncand = 0u; }
  __syncthreads();

  // 1. coalesced load + histogram of bits 31..21
  unsigned key[KPT];
  // branch-free: every load is issued before the first one is consumed
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = tid + j * kTopkBlock;
    const float v = sc[min(i, n - 1)];
    key[j] = order_key(v) & (0u - (unsigned)(i < n));   // arithmetic mask, no branch
  }
  // Positions past n hold key 0 (the NaN key): they lose every comparison and come last by
  // index, so with k <= n they are never selected and need no further bounds checks.
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    atomicAdd(&s_hist[copy][key[j] >> 21], 1u);
    __builtin_amdgcn_sched_barrier(0);  // one row at a time: keeps register pressure flat
  }
  __syncthreads();
  find_bin(s_hist, kTopkBins, (unsigned)k, s_sel, s_scan);
  const unsigned d0 = s_sel[0];
  unsigned krem = s_sel[1];
  unsigned bin_count = 0;
#pragma unroll
  for (int q = 0; q < kTopkCopies; ++q) bin_count += s_hist[q][d0];
  unsigned prefix = d0 << 21, pmask = 2047u << 21;

  // 2. resolve the low 21 bits among the keys of bin d0
  const bool compact = bin_count <= (unsigned)kTopkCand;  // block-uniform (padding counts too)
  if (compact) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if ((key[j] >> 21) == d0) s_cand[atomicAdd(&s_ncand, 1u)] = key[j];
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();
  const int ncand = (int)s_ncand;
#pragma unroll
  for (int pass = 1; pass < 3; ++pass) {
    const int shift = pass == 1 ? 10 : 0;
    const unsigned dmask = pass == 1 ? 2047u : 1023u;
    for (int i = tid; i < kTopkCopies * kTopkBins; i += kTopkBlock) (&s_hist[0][0])[i] = 0u;
    __syncthreads();
    if (compact) {
      for (int i = tid; i < ncand; i += kTopkBlock) {
        const unsigned kv = s_cand[i];
        if ((kv & pmask) == prefix) atomicAdd(&s_hist[copy][(kv >> shift) & dmask], 1u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPT; ++j)
      {
        if ((key[j] & pmask) == prefix) atomicAdd(&s_hist[copy][(key[j] >> shift) & dmask], 1u);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    find_bin(s_hist, (int)dmask + 1, krem, s_sel, s_scan);
    prefix |= s_sel[0] << shift;
    pmask |= dmask << shift;
    krem = s_sel[1];
  }
  const unsigned tau = prefix;  // the k-th largest key; krem of the keys equal to it are taken
  __shared__ unsigned s_tk[3];
  if (tid == 0) { s_tk[0] = tau; s_tk[1] = krem; s_tk[2] = 0u; }

  // 3. positions in ascending index order from per-(row, wave) ballot counts
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const unsigned long long gm = __ballot(key[j] > tau);
    const unsigned long long em = __ballot(key[j] == tau);
    if (lane == 0) {
      s_cnt[0][j][w] = (unsigned)__popcll(gm);
      s_cnt[1][j][w] = (unsigned)__popcll(em);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  // exclusive scan of the KPT*16 (row, wave) counts in index order; thread t holds entries
  // t*CPT .. t*CPT+CPT-1
  constexpr int NE = KPT * kTopkWaves;
  constexpr int CPT = (NE + kTopkBlock - 1) / kTopkBlock;
  unsigned cg[CPT], ce[CPT], sg = 0, se = 0;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int e = tid * CPT + c;
    cg[c] = e < NE ? (&s_cnt[0][0][0])[e] : 0u;
    ce[c] = e < NE ? (&s_cnt[1][0][0])[e] : 0u;
    sg += cg[c];
    se += ce[c];
  }
  unsigned bg, be, tg, te;
  block_scan2(sg, se, &bg, &be, &tg, &te, s_scan);
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int e = tid * CPT + c;
    if (e < NE) { (&s_cnt[0][0][0])[e] = bg; (&s_cnt[1][0][0])[e] = be; }
    bg += cg[c];
    be += ce[c];
  }
  __syncthreads();
  // tau and krem re-read after the barrier: the per-row comparisons of the counting loop
  // are then recomputed here instead of being kept alive (96 masks would spill)
  const unsigned tau2 = s_tk[0], krem2 = s_tk[1];
  const int zero = (int)s_tk[2];  // element indices are recomputed from it, not kept from the load loop
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = zero + tid + j * kTopkBlock;
    const bool gt = key[j] > tau2;
    const bool eq = key[j] == tau2;
    const unsigned long long gm = __ballot(gt);
    const unsigned long long em = __ballot(eq);
    const unsigned gb = s_cnt[0][j][w] + (unsigned)__popcll(gm & below);
    const unsigned eb = s_cnt[1][j][w] + (unsigned)__popcll(em & below);
    if (gt || (eq && eb < krem2)) {
      const unsigned pos = gb + min(eb, krem2);
      if (pos < (unsigned)k) out[pos] = i;   // always true for a correct selection
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int KPT>
static void launch_one(const TopkArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL((topk_kernel<KPT>), dim3(B, a.nprob), dim3(kTopkBlock), 0, s, a);
}

hipError_t launch_topk(const TopkArgs& a, int B, hipStream_t s) {
  int nmax = 0;
  for (int i = 0; i < a.nprob; ++i) nmax = max(nmax, a.p[i].n);
  if (nmax > 65536) return hipErrorInvalidValue;
  if (nmax <= 1024) launch_one<1>(a, B, s);
  else if (nmax <= 4096) launch_one<4>(a, B, s);
  else if (nmax <= 16384) launch_one<16>(a, B, s);
  else if (nmax <= 49152) launch_one<48>(a, B, s);
  else launch_one<64>(a, B, s);
  return hipGetLastError();
}

}  // namespace dv
