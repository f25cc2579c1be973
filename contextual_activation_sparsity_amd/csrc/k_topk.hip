// Exact top-k of predictor scores (DejaVu Guide, "Mathematical Formulation of Lookahead
// Predictors": the active sets are the top-k of the scores; the guide's predictor returns
// the indices sorted).
//
// Order: scores map to 32-bit unsigned keys that order like the floats, with -0.0 folded
// onto +0.0 and every NaN mapped to 0 (below -inf). The k largest keys win; among equal
// keys the lower index wins. Output is the selected indices in ascending order.
//
// A radix select spread over many CUs. Three kernels, and no block ever waits on another
// (the kernel boundaries order them):
//  1. topk_hist_kernel: one block per 4096-score chunk writes the chunk's histogram of the
//     top 11 key bits.
//  2. topk_classify_kernel: every chunk block sums the chunk histograms, finds the bin d0
//     holding the k-th largest key, and sorts its own scores into "above d0" (ballots
//     straight into a bitmap of selected positions) and "in d0" (candidates, compacted in
//     index order into the chunk's list).
//  Problems of at most 256 scores (the heads) are selected whole by one block of the first
//  launch (rank by counting), and the other two kernels skip them. When no problem of the
//  launch has more than 16384 scores, one block per row selects each problem whole instead
//  (topk_single_kernel: the same radix passes over keys held in registers), in one launch.
//  3. topk_finish_kernel: one block per row gathers the candidates (typically 1-3 % of n),
//     resolves the remaining 21 key bits with two more histogram passes, takes the ties at
//     the threshold key in index order, sets their bits, and turns the bitmap into the
//     ascending index list with one block scan of per-word popcounts.
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

constexpr int kTkBlock = 1024;
constexpr int kTkWaves = kTkBlock / kWave;
constexpr int kTkEpt = kTopkChunk / kTkBlock;   // scores per thread per chunk (4)
constexpr int kTkBins = 2048;                    // 11-bit digits: bits 31..21, 20..10, 9..0
constexpr int kTkCopies = 2;                     // LDS histogram copies (wave w uses w % 2)
constexpr int kTkCandLds = 8192;                 // candidates resolved from LDS
static_assert(kTkEpt * kTkBlock == kTopkChunk, "chunk must be a whole number of block sweeps");
static_assert(kTopkChunk % 64 == 0, "a chunk is whole waves");

// Exclusive scan over the block of one per-thread count (thread order); also returns the total.
__device__ __forceinline__ unsigned block_scan(unsigned a, unsigned* total, unsigned* s) {
  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  unsigned ia = a;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const unsigned x = __shfl_up(ia, off, kWave);
    if (lane >= off) ia += x;
  }
  if (lane == kWave - 1) s[w] = ia;
  __syncthreads();
  unsigned p = 0, t = 0;
#pragma unroll
  for (int i = 0; i < kTkWaves; ++i) {
    if (i < w) p += s[i];
    t += s[i];
  }
  __syncthreads();
  *total = t;
  return p + ia - a;
}

// Bin of a histogram (nbins <= 2048, thread t holds bins nbins-1-2t and nbins-2-2t, i.e.
// descending digit order) that holds the krem-th largest key; returns {bin, rank inside it,
// keys in it} through s_sel. 1 <= krem <= total is required.
__device__ __forceinline__ void select_bin(unsigned c0, unsigned c1, int nbins, unsigned krem, unsigned* s_sel,
                                           unsigned* s_scan) {
  const int t = threadIdx.x;
  unsigned total;
  const unsigned before = block_scan(c0 + c1, &total, s_scan);
  if (before < krem && krem <= before + c0) {
    s_sel[0] = (unsigned)(nbins - 1 - 2 * t);
    s_sel[1] = krem - before;
    s_sel[2] = c0;
  } else if (before + c0 < krem && krem <= before + c0 + c1) {
    s_sel[0] = (unsigned)(nbins - 2 - 2 * t);
    s_sel[1] = krem - before - c0;
    s_sel[2] = c1;
  }
  __syncthreads();
}

__device__ __forceinline__ const TopkProb& prob_of(const TopkArgs& a) {
  return blockIdx.z == 0 ? a.p[0] : a.p[1];
}

// Problems of at most kTkSmall scores (the heads) are selected whole by one block inside the
// first launch: the rank of score i is the number of scores ahead of it (a larger key, or the
// same key at a lower index), score i is selected when its rank is below k, and a block scan of
// the selected flags gives the ascending list. Exact, with the same keys and tie rule.
constexpr int kTkSmall = 256;
static_assert(kTkSmall <= kTkBlock, "one score per thread");
__device__ __forceinline__ void topk_small(const TopkProb& P, int b, unsigned* s_key, unsigned* s_scan) {
  const int n = P.n, k = P.k, tid = threadIdx.x;
  const float* sc = P.scores + (long long)b * n;
  const unsigned key = tid < n ? order_key(sc[tid]) : 0u;
  // keys padded with 0 to a multiple of 4: a pad (index >= n > tid) is never ahead of a score
  if (tid < ((n + 3) & ~3)) s_key[tid] = key;
  __syncthreads();
  bool sel = false;
  if (tid < n) {
    unsigned r = 0;
    const u32x4* k4 = reinterpret_cast<const u32x4*>(s_key);
#pragma unroll 4
    for (int j4 = 0; j4 < (n + 3) / 4; ++j4) {
      const u32x4 v = k4[j4];
      const int j = 4 * j4;
      r += (v.x > key || (v.x == key && j < tid)) ? 1u : 0u;
      r += (v.y > key || (v.y == key && j + 1 < tid)) ? 1u : 0u;
      r += (v.z > key || (v.z == key && j + 2 < tid)) ? 1u : 0u;
      r += (v.w > key || (v.w == key && j + 3 < tid)) ? 1u : 0u;
    }
    sel = r < (unsigned)k;
  }
  unsigned tot;
  const unsigned pos = block_scan(sel ? 1u : 0u, &tot, s_scan);
  if (sel) P.out[(long long)b * k + pos] = tid;
}

// 1. per-chunk histograms of bits 31..21 -> part[b][chunk][2048]
__global__ __launch_bounds__(kTkBlock) void topk_hist_kernel(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned s_hist[kTkCopies][kTkBins];
  const TopkProb& P = prob_of(a);
  const int c = blockIdx.x, b = blockIdx.y, n = P.n, tid = threadIdx.x;
  const int nch = (n + kTopkChunk - 1) / kTopkChunk;
  if (n <= kTkSmall) {   // block-uniform: the whole problem in this launch
    if (c == 0 && P.k > 0) topk_small(P, b, &s_hist[0][0], &s_hist[1][0]);
    return;
  }
  if (P.k <= 0 || P.k >= n || c >= nch) return;
  const float* sc = P.scores + (long long)b * n;
  for (int i = tid; i < kTkCopies * kTkBins; i += kTkBlock) (&s_hist[0][0])[i] = 0u;
  unsigned key[kTkEpt];
#pragma unroll
  for (int j = 0; j < kTkEpt; ++j) {
    const int i = c * kTopkChunk + j * kTkBlock + tid;
    key[j] = i < n ? order_key(sc[i]) : 0u;
  }
  __syncthreads();
  const int copy = (tid / kWave) % kTkCopies;
#pragma unroll
  for (int j = 0; j < kTkEpt; ++j) {
    const int i = c * kTopkChunk + j * kTkBlock + tid;
    if (i < n) atomicAdd(&s_hist[copy][key[j] >> 21], 1u);   // padding is not counted
  }
  __syncthreads();
  unsigned* part = P.ws.part + ((long long)b * nch + c) * kTkBins;
  for (int bin = tid; bin < kTkBins; bin += kTkBlock) {
    unsigned v = 0;
#pragma unroll
    for (int q = 0; q < kTkCopies; ++q) v += s_hist[q][bin];
    part[bin] = v;
  }
}

// 2. threshold bin from the summed histogram; above-bin bits and in-bin candidates per chunk
__global__ __launch_bounds__(kTkBlock) void topk_classify_kernel(TopkArgs a) {
  __shared__ unsigned s_scan[kTkWaves];
  __shared__ unsigned s_sel[3];
  __shared__ unsigned s_cnt[kTkEpt * kTkWaves];
  const TopkProb& P = prob_of(a);
  const int c = blockIdx.x, b = blockIdx.y, n = P.n, k = P.k, tid = threadIdx.x;
  const int lane = tid % kWave, w = tid / kWave;
  const int nch = (n + kTopkChunk - 1) / kTopkChunk;
  if (n <= kTkSmall || k <= 0 || k >= n || c >= nch) return;   // small problems are done
  const float* sc = P.scores + (long long)b * n;
  // every load of the block is issued before the first one is used
  unsigned key[kTkEpt];
#pragma unroll
  for (int j = 0; j < kTkEpt; ++j) {
    const int i = c * kTopkChunk + j * kTkBlock + tid;
    key[j] = order_key(sc[min(i, n - 1)]);
  }
  // thread t owns bins 2047-2t (c0) and 2046-2t (c1); stored pairs are (2046-2t, 2047-2t)
  const unsigned* part = P.ws.part + (long long)b * nch * kTkBins;
  uint2 pv[kTopkMaxChunks];
#pragma unroll
  for (int q = 0; q < kTopkMaxChunks; ++q)   // all chunk loads in flight together
    pv[q] = q < nch ? *reinterpret_cast<const uint2*>(part + (long long)q * kTkBins + (kTkBins - 2 - 2 * tid))
                    : make_uint2(0u, 0u);
  unsigned c0 = 0, c1 = 0;
#pragma unroll
  for (int q = 0; q < kTopkMaxChunks; ++q) {
    c1 += pv[q].x;
    c0 += pv[q].y;
  }
  select_bin(c0, c1, kTkBins, (unsigned)k, s_sel, s_scan);
  const unsigned d0 = s_sel[0];
  if (c == 0 && tid == 0) {   // the threshold bin, keys above it, keys in it
    unsigned* sel = P.ws.sel + (long long)b * 4;
    sel[0] = d0;
    sel[1] = (unsigned)k - s_sel[1];
    sel[2] = s_sel[2];
    sel[3] = 0u;
  }
  // above-bin positions: each (sweep j, wave w) covers 64 consecutive scores = 2 bitmap words
  unsigned* bits = P.ws.bits + (long long)b * nch * (kTopkChunk / 32);
  bool eq[kTkEpt];
#pragma unroll
  for (int j = 0; j < kTkEpt; ++j) {
    const int i = c * kTopkChunk + j * kTkBlock + tid;
    const unsigned dg = key[j] >> 21;
    const bool ok = i < n;
    const unsigned long long gm = __ballot(ok && dg > d0);
    eq[j] = ok && dg == d0;
    const unsigned long long em = __ballot(eq[j]);
    if (lane == 0) {
      *reinterpret_cast<uint2*>(bits + c * (kTopkChunk / 32) + j * (kTkBlock / 32) + w * 2) =
          make_uint2((unsigned)gm, (unsigned)(gm >> 32));
      s_cnt[j * kTkWaves + w] = (unsigned)__popcll(em);
    }
  }
  __syncthreads();
  // exclusive scan of the (sweep, wave) candidate counts in index order, by wave 0
  if (w == 0) {
    const unsigned v = lane < kTkEpt * kTkWaves ? s_cnt[lane] : 0u;
    unsigned s = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const unsigned x = __shfl_up(s, off, kWave);
      if (lane >= off) s += x;
    }
    if (lane < kTkEpt * kTkWaves) s_cnt[lane] = s - v;
    if (lane == kWave - 1) P.ws.ccnt[(long long)b * nch + c] = s;
  }
  static_assert(kTkEpt * kTkWaves <= kWave, "one wave scans the candidate counts");
  __syncthreads();
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  unsigned* ckey = P.ws.ckey + (long long)b * nch * kTopkChunk + c * kTopkChunk;
  unsigned* cidx = P.ws.cidx + (long long)b * nch * kTopkChunk + c * kTopkChunk;
#pragma unroll
  for (int j = 0; j < kTkEpt; ++j) {
    const unsigned long long em = __ballot(eq[j]);
    if (eq[j]) {
      const unsigned pos = s_cnt[j * kTkWaves + w] + (unsigned)__popcll(em & below);
      ckey[pos] = key[j];
      cidx[pos] = (unsigned)(c * kTopkChunk + j * kTkBlock + tid);
    }
  }
}

// 3. resolve the threshold bin, take the ties in index order, bitmap -> ascending list
__global__ __launch_bounds__(kTkBlock) void topk_finish_kernel(TopkArgs a) {
  __shared__ unsigned s_bits[kTopkMaxChunks * (kTopkChunk / 32)];
  __shared__ unsigned s_hist[kTkCopies][kTkBins];
  __shared__ unsigned s_ck[kTkCandLds];
  __shared__ unsigned s_ci[kTkCandLds];
  __shared__ unsigned s_scan[kTkWaves];
  __shared__ unsigned s_sel[3];
  __shared__ unsigned s_pre[kTopkMaxChunks + 1];
  __shared__ unsigned s_tk[2];
  const TopkProb& P = prob_of(a);
  const int b = blockIdx.x, n = P.n, k = P.k, tid = threadIdx.x;
  const int copy = (tid / kWave) % kTkCopies;
  if (k <= 0 || n <= kTkSmall) return;   // small problems are done
  int32_t* out = P.out + (long long)b * k;
  if (k >= n) {
    for (int i = tid; i < n; i += kTkBlock) out[i] = i;
    return;
  }
  const int nch = (n + kTopkChunk - 1) / kTopkChunk;
  const int nwords = nch * (kTopkChunk / 32);
  const unsigned* sel = P.ws.sel + (long long)b * 4;
  const unsigned* ccnt = P.ws.ccnt + (long long)b * nch;
  const unsigned* gbits = P.ws.bits + (long long)b * nwords;
  const unsigned* gck = P.ws.ckey + (long long)b * nch * kTopkChunk;
  const unsigned* gci = P.ws.cidx + (long long)b * nch * kTopkChunk;

  // independent loads first: bitmap words, per-chunk candidate counts, the threshold record
  const unsigned bw0 = tid < nwords ? gbits[tid] : 0u;
  const unsigned bw1 = tid + kTkBlock < nwords ? gbits[tid + kTkBlock] : 0u;
  const unsigned cq = tid < nch ? ccnt[tid] : 0u;
  const unsigned d0 = sel[0];
  const unsigned above = sel[1];
  static_assert(2 * kTkBlock >= kTopkMaxChunks * (kTopkChunk / 32), "two bitmap words per thread");
  if (tid < nwords) s_bits[tid] = bw0;
  if (tid + kTkBlock < nwords) s_bits[tid + kTkBlock] = bw1;
  if (tid < kWave) {   // exclusive scan of the chunk counts by wave 0
    unsigned sc = cq;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const unsigned t = __shfl_up(sc, off, kWave);
      if (tid >= off) sc += t;
    }
    if (tid <= nch) s_pre[tid] = sc - cq;   // s_pre[nch] = total (cq = 0 there)
  }
  static_assert(kTopkMaxChunks < kWave, "one wave scans the chunk counts");
  __syncthreads();
  const unsigned ncand = s_pre[nch];   // == keys in bin d0
  const bool in_lds = ncand <= (unsigned)kTkCandLds;   // block-uniform
  // candidate g (0 <= g < ncand, index order) lives in chunk q at offset g - s_pre[q]
  auto gpos = [&](unsigned g) -> long long {
    int q = 0;
    while (q + 1 < nch && s_pre[q + 1] <= g) ++q;
    return (long long)q * kTopkChunk + (g - s_pre[q]);
  };
  if (in_lds) {
    for (unsigned g = tid; g < ncand; g += kTkBlock) {
      const long long p = gpos(g);
      s_ck[g] = gck[p];
      s_ci[g] = gci[p];
    }
  }
  __syncthreads();
  auto cand_key = [&](unsigned g) -> unsigned { return in_lds ? s_ck[g] : gck[gpos(g)]; };
  auto cand_idx = [&](unsigned g) -> unsigned { return in_lds ? s_ci[g] : gci[gpos(g)]; };

  unsigned krem = (unsigned)k - above;   // 1 <= krem <= ncand
  unsigned prefix = d0 << 21, pmask = 2047u << 21;
#pragma unroll
  for (int pass = 1; pass < 3; ++pass) {
    const int shift = pass == 1 ? 10 : 0;
    const int nb = pass == 1 ? 2048 : 1024;
    const unsigned dmask = (unsigned)nb - 1u;
    for (int i = tid; i < kTkCopies * kTkBins; i += kTkBlock) (&s_hist[0][0])[i] = 0u;
    __syncthreads();
    for (unsigned g = tid; g < ncand; g += kTkBlock) {
      const unsigned kv = cand_key(g);
      if ((kv & pmask) == prefix) atomicAdd(&s_hist[copy][(kv >> shift) & dmask], 1u);
    }
    __syncthreads();
    unsigned h0 = 0, h1 = 0;
    const int b0 = nb - 1 - 2 * tid, b1 = nb - 2 - 2 * tid;
#pragma unroll
    for (int q = 0; q < kTkCopies; ++q) {
      if (b0 >= 0) h0 += s_hist[q][b0];
      if (b1 >= 0) h1 += s_hist[q][b1];
    }
    select_bin(h0, h1, nb, krem, s_sel, s_scan);
    prefix |= s_sel[0] << shift;
    pmask |= dmask << shift;
    krem = s_sel[1];
  }
  // tau = the k-th largest key; krem of the keys equal to tau are taken, lowest index first
  if (tid == 0) { s_tk[0] = prefix; s_tk[1] = krem; }
  __syncthreads();
  const unsigned tau = s_tk[0], take = s_tk[1];
  unsigned taken = 0;   // ties already taken in earlier sweeps (block-uniform)
  for (unsigned g0 = 0; g0 < ncand; g0 += kTkBlock) {
    const unsigned g = g0 + tid;
    unsigned kv = 0, ix = 0;
    if (g < ncand) { kv = cand_key(g); ix = cand_idx(g); }
    const bool gt = g < ncand && kv > tau;
    const bool eq = g < ncand && kv == tau;
    unsigned tot;
    const unsigned rank = taken + block_scan(eq ? 1u : 0u, &tot, s_scan);
    if (gt || (eq && rank < take)) atomicOr(&s_bits[ix >> 5], 1u << (ix & 31u));
    taken += tot;
  }
  __syncthreads();
  // bitmap -> ascending list: thread t owns words 2t and 2t+1
  const int w0 = 2 * tid;
  const unsigned m0 = w0 < nwords ? s_bits[w0] : 0u;
  const unsigned m1 = w0 + 1 < nwords ? s_bits[w0 + 1] : 0u;
  unsigned tot;
  unsigned pos = block_scan((unsigned)__popc(m0) + (unsigned)__popc(m1), &tot, s_scan);
  static_assert(2 * kTkBlock >= kTopkMaxChunks * (kTopkChunk / 32), "two bitmap words per thread");
  unsigned m = m0;
  for (int h = 0; h < 2; ++h) {
    const int base = (w0 + h) * 32;
    while (m != 0u) {
      const int bit = __builtin_ctz(m);
      m &= m - 1u;
      if (pos < (unsigned)k) out[pos] = base + bit;   // always true for a correct selection
      ++pos;
    }
    m = m1;
  }
}

// Problems of at most kTkSingle scores (and more than kTkSmall) are selected whole by one
// block per row, in one launch: thread t holds the keys of the EPT consecutive positions from
// EPT*t in registers; three histogram passes over their 11/11/10-bit digits (each pass counts
// only the keys that share the digits found so far) find tau, the k-th largest key, and how
// many keys equal to tau are taken. A block scan of the per-thread counts of tau-keys gives each
// thread the ties at lower positions (the lower index wins), and a scan of the per-thread
// selected counts places each thread's picks in the ascending list. Same keys, same tie rule.
constexpr int kTkSingle = 16384;   // measured: at 36864 scores the three launches over many CUs win

template <int EPT>
__global__ __launch_bounds__(kTkBlock) void topk_single_kernel(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned s_hist[kTkBins];
  __shared__ unsigned s_scan[kTkWaves];
  __shared__ unsigned s_sel[3];
  static_assert(EPT * kTkBlock >= kTkSingle, "the largest single-block problem fits");
  const TopkProb& P = prob_of(a);
  const int b = blockIdx.x, n = P.n, k = P.k, tid = threadIdx.x;
  if (k <= 0) return;
  if (n <= kTkSmall) {   // block-uniform
    topk_small(P, b, s_hist, s_scan);
    return;
  }
  int32_t* out = P.out + (long long)b * k;
  if (k >= n) {
    for (int i = tid; i < n; i += kTkBlock) out[i] = i;
    return;
  }
  const float* sc = P.scores + (long long)b * n;
  const int i0 = tid * EPT;
  unsigned key[EPT];
  if ((EPT % 4) == 0 && (reinterpret_cast<uintptr_t>(sc) & 15u) == 0 && i0 + EPT <= n) {
#pragma unroll
    for (int j = 0; j < EPT; j += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(sc + i0 + j);
      key[j] = order_key(v[0]); key[j + 1] = order_key(v[1]);
      key[j + 2] = order_key(v[2]); key[j + 3] = order_key(v[3]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPT; ++j) key[j] = i0 + j < n ? order_key(sc[i0 + j]) : 0u;
  }
  const int nv = max(0, min(EPT, n - i0));   // valid positions of this thread
  unsigned krem = (unsigned)k, prefix = 0u, pmask = 0u;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    const unsigned dmask = (unsigned)nb - 1u;
    for (int i = tid; i < kTkBins; i += kTkBlock) s_hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < EPT; ++j)
      if (j < nv && (key[j] & pmask) == prefix) atomicAdd(&s_hist[(key[j] >> shift) & dmask], 1u);
    __syncthreads();
    const int b0 = nb - 1 - 2 * tid, b1 = nb - 2 - 2 * tid;
    const unsigned h0 = b0 >= 0 ? s_hist[b0] : 0u;
    const unsigned h1 = b1 >= 0 ? s_hist[b1] : 0u;
    select_bin(h0, h1, nb, krem, s_sel, s_scan);
    prefix |= s_sel[0] << shift;
    pmask |= dmask << shift;
    krem = s_sel[1];
  }
  const unsigned tau = prefix, take = krem;   // take of the keys equal to tau, lowest positions first
  unsigned ne = 0;
#pragma unroll
  for (int j = 0; j < EPT; ++j) ne += (j < nv && key[j] == tau) ? 1u : 0u;
  unsigned tot;
  unsigned eq_seen = block_scan(ne, &tot, s_scan);   // tau-keys at lower positions
  unsigned cnt = 0;
  unsigned selbits = 0u;   // bit j: position i0 + j is selected
  static_assert(EPT <= 32, "one word of selection bits per thread");
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    bool on = false;
    if (j < nv) {
      if (key[j] > tau) {
        on = true;
      } else if (key[j] == tau) {
        on = eq_seen < take;
        ++eq_seen;
      }
    }
    if (on) {
      ++cnt;
      selbits |= 1u << j;
    }
  }
  unsigned pos = block_scan(cnt, &tot, s_scan);
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    if ((selbits >> j) & 1u) {
      if (pos < (unsigned)k) out[pos] = i0 + j;   // always true for a correct selection
      ++pos;
    }
  }
}

size_t topk_ws_bytes(int B, int n) {
  const size_t nch = (size_t)((n + kTopkChunk - 1) / kTopkChunk);
  const size_t per_row = nch * kTkBins        // part
                       + nch * (kTopkChunk / 32)   // bits
                       + 2 * nch * kTopkChunk      // ckey, cidx
                       + nch                       // ccnt
                       + 4;                        // sel
  return (size_t)B * per_row * sizeof(unsigned) + 6 * 256;
}

TopkWs topk_ws_carve(void* base, int B, int n) {
  const size_t nch = (size_t)((n + kTopkChunk - 1) / kTopkChunk);
  char* p = static_cast<char*>(base);
  auto take = [&](size_t words) {
    unsigned* r = reinterpret_cast<unsigned*>(p);
    p += ((words * sizeof(unsigned)) + 255u) & ~size_t(255u);
    return r;
  };
  TopkWs w{};
  w.part = take((size_t)B * nch * kTkBins);
  w.bits = take((size_t)B * nch * (kTopkChunk / 32));
  w.ckey = take((size_t)B * nch * kTopkChunk);
  w.cidx = take((size_t)B * nch * kTopkChunk);
  w.ccnt = take((size_t)B * nch);
  w.sel = take((size_t)B * 4);
  return w;
}

hipError_t launch_topk(const TopkArgs& a, int B, hipStream_t s) {
  int nmax = 0;
  for (int i = 0; i < a.nprob; ++i) {
    if (a.p[i].n > kTopkMaxChunks * kTopkChunk) return hipErrorInvalidValue;
    nmax = max(nmax, a.p[i].n);
  }
  if (nmax > kTkSmall && nmax <= kTkSingle) {   // one block per row and problem, one launch
    const dim3 g1(B, 1, a.nprob);
    hipLaunchKernelGGL(topk_single_kernel<kTkSingle / kTkBlock>, g1, dim3(kTkBlock), 0, s, a);
    return hipGetLastError();
  }
  const int nch = (nmax + kTopkChunk - 1) / kTopkChunk;
  const dim3 grid(nch, B, a.nprob);
  hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kTkBlock), 0, s, a);
  if (nmax <= kTkSmall) return hipGetLastError();   // every problem was selected whole
  hipLaunchKernelGGL(topk_classify_kernel, grid, dim3(kTkBlock), 0, s, a);
  hipLaunchKernelGGL(topk_finish_kernel, dim3(B, 1, a.nprob), dim3(kTkBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace dv
