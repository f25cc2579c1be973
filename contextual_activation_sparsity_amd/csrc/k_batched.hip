// Batched decode (B >= 2 rows per step) on the union of the rows' selections.
//
// Each row keeps its own selection (the step is per-row masked, DejaVu Guide, "Head-Pruned
// Attention Dispatch" and the sparse MLP of "Step-by-Step Implementation", applied row by
// row); the union only shares the weight traffic: every selected weight row is read once
// and multiplied against all B activation rows on the matrix cores.
//
//  * union_rows / union_or / union_list: per-row bitmaps of the selected groups (neurons or
//    heads, from the rows' ascending lists by binary search in LDS, no atomics), then their
//    OR with a count per block of words, then the OR as an ascending list (each block starts
//    at the counts of the blocks before it) with its length in device memory.
//  * rows_norm_f16: RMSNorm of each row, rounded to fp16 (the MFMA operand type).
//  * gemm_rows (up-projection, q/k/v and W1; both predictor factors): out[b][i] =
//    act(W[row_i] . X[b] + bias), masked per row. A block stages 64 gathered weight rows and
//    the B activation rows through LDS in K chunks (contiguous 512-byte row pieces per load
//    instruction); a wave owns 16 rows, fp32 accumulation with v_mfma_f32_16x16x32_f16.
//    With a low part X_lo the product is taken twice (W . X_hi + W . X_lo): the fp16 weights
//    are exact, so the result then carries fp32-like activation precision (used for the
//    predictor's scores; its first factor takes the fp32 input and splits it into the two
//    parts while staging it). Short launches split K over blocks and add the slices in order.
//  * gemm_cols (down-projection, Wo and W2): partial[b][rg][c] = sum over the rows of row
//    group rg of C[b][k] * W[row_k][c]. Weight rows are read in 512-byte strips, transposed
//    8 x 8 in registers and staged in LDS so each lane's B fragment (8 consecutive k at one
//    column) is one 16-byte LDS read. The weight rows of a block's union positions are
//    staged in LDS a sweep at a time, so no tile waits on an index load. The row groups are
//    summed by the ordered reduce kernel of the gather-axpy.
// Every sum has a fixed order: results are bitwise reproducible.
#include <algorithm>

#include "dv_device.h"
#include "dv_kernels.h"

namespace dv {

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bool bit_of(const unsigned* bits, int j) { return (bits[j >> 5] >> (j & 31)) & 1u; }

// Number of set bits of `bits` below position j (the rank of j in an ascending list).
__device__ __forceinline__ int rank_below(const unsigned* bits, int j) {
  int r = 0;
  for (int w = 0; w < (j >> 5); ++w) r += __popc(bits[w]);
  return r + __popc(bits[j >> 5] & ((1u << (j & 31)) - 1u));
}

// ---------------------------------------------------------------------------
// union of the rows' selections
// ---------------------------------------------------------------------------
// Row bitmaps without atomics: thread (row b, word w) finds the first entry >= 32w of the row's
// ascending list by binary search and sets the bits of the entries below 32(w+1) (entries
// outside [0, n) select nothing). Every word is written whole, so no clearing pass is needed.
constexpr int kUnionRowsBlock = 256;    // bitmap words per block
constexpr int kUnionRowsLds = 16384;    // a row's list is searched in LDS up to this length
constexpr int kUnionRowsLdsPT = 16;     // list entries each thread stages per sweep
__global__ __launch_bounds__(kUnionRowsBlock) void union_rows_kernel(UnionArgs a) {
  __shared__ int32_t s_l[kUnionRowsLds];
  const UnionProb& P = blockIdx.z == 0 ? a.p[0] : a.p[1];
  const int tid = threadIdx.x;
  const int words = (P.n + 31) / 32;
  const int b = blockIdx.y;
  const int w0 = blockIdx.x * kUnionRowsBlock;
  if (w0 >= words) return;   // block-uniform: the other problem may have more words
  const int32_t* L = P.idx + (long long)b * P.idx_bstride;
  // Row b's ascending list, staged in LDS with every load of a sweep in flight together, so
  // the searches below wait on LDS instead of on a chain of dependent global loads.
  const bool lds = P.k <= kUnionRowsLds;   // block-uniform
  if (lds) {
    for (int i0 = 0; i0 < P.k; i0 += kUnionRowsBlock * kUnionRowsLdsPT) {
      int32_t v[kUnionRowsLdsPT];
#pragma unroll
      for (int q = 0; q < kUnionRowsLdsPT; ++q) {
        const int i = i0 + q * kUnionRowsBlock + tid;
        v[q] = i < P.k ? L[i] : 0;
      }
#pragma unroll
      for (int q = 0; q < kUnionRowsLdsPT; ++q) {
        const int i = i0 + q * kUnionRowsBlock + tid;
        if (i < P.k) s_l[i] = v[q];
      }
    }
    __syncthreads();
  }
  const int w = w0 + tid;
  if (w >= words) return;
  auto at = [&](int i) -> int32_t { return lds ? s_l[i] : L[i]; };
  const int lo_v = 32 * w, hi_v = min(32 * w + 32, P.n);
  int lo = 0, hi = P.k;   // first position with L[pos] >= lo_v
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (at(mid) < lo_v) lo = mid + 1;
    else hi = mid;
  }
  unsigned m = 0u;
  for (int i = lo; i < P.k && at(i) < hi_v; ++i) m |= 1u << (at(i) - lo_v);
  P.bits[(long long)b * words + w] = m;
}

// OR of the row bitmaps (kept as row B), kUnionWpb words per block: four groups of eight rows
// per word with every load in flight, then the set bits of the block's words.
constexpr int kUnionOrBlock = 4 * kUnionWpb;
static_assert(kBatchMax <= 32, "four groups of eight rows cover a batch");
__global__ __launch_bounds__(kUnionOrBlock) void union_or_kernel(UnionArgs a) {
  __shared__ unsigned s_or[4][kUnionWpb];
  const UnionProb& P = blockIdx.y == 0 ? a.p[0] : a.p[1];
  const int words = (P.n + 31) / 32;
  const int w0 = blockIdx.x * kUnionWpb;
  if (w0 >= words) return;   // block-uniform: the other problem may have more words
  const int tid = threadIdx.x, wl = tid % kUnionWpb, rg = tid / kUnionWpb;
  const int w = w0 + wl;
  unsigned r[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int b = 8 * rg + q;
    r[q] = (w < words && b < a.B) ? P.bits[(long long)b * words + w] : 0u;
  }
  unsigned u = 0u;
#pragma unroll
  for (int q = 0; q < 8; ++q) u |= r[q];
  s_or[rg][wl] = u;
  __syncthreads();
  if (tid < kUnionWpb) {   // wave 0: one word per lane
    const unsigned v = s_or[0][tid] | s_or[1][tid] | s_or[2][tid] | s_or[3][tid];
    if (w < words) P.bits[(long long)a.B * words + w] = v;
    unsigned c = (unsigned)__popc(v);
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) c += __shfl_xor(c, off, kWave);
    if (tid == 0) P.bcnt[blockIdx.x] = c;
  }
}
static_assert(kUnionWpb == kWave, "the list kernel is one wave per block of words");

// The OR as an ascending list: block x (one wave, one word per lane) starts at the set bits of
// the blocks before it, scans its words' counts, stages its part of the list in LDS and
// writes it with coalesced stores; the last block writes the list's length.
__global__ __launch_bounds__(kUnionWpb) void union_list_kernel(UnionArgs a) {
  __shared__ int32_t s_l[kUnionWpb * 32];
  const UnionProb& P = blockIdx.y == 0 ? a.p[0] : a.p[1];
  const int words = (P.n + 31) / 32;
  const int nblk = (words + kUnionWpb - 1) / kUnionWpb;
  const int x = blockIdx.x;
  if (x >= nblk) return;   // block-uniform
  const int lane = threadIdx.x;
  static_assert(kUnionMaxN / 32 / kUnionWpb <= kWave, "one lane per earlier block");
  unsigned off = lane < x ? P.bcnt[lane] : 0u;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) off += __shfl_xor(off, o, kWave);
  const int w = x * kUnionWpb + lane;
  const unsigned v = w < words ? P.bits[(long long)a.B * words + w] : 0u;
  const unsigned pc = (unsigned)__popc(v);
  unsigned incl = pc;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const unsigned t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  const unsigned tot = __shfl(incl, kWave - 1, kWave);
  unsigned p = incl - pc;
  unsigned m = v;
  while (m != 0u) {
    const int bit = __builtin_ctz(m);
    m &= m - 1u;
    s_l[p++] = w * 32 + bit;
  }
  __syncthreads();
  for (unsigned i = lane; i < tot; i += kUnionWpb) P.list[off + i] = s_l[i];
  if (x == nblk - 1 && lane == 0) *P.count = (int)(off + tot);
}

// ---------------------------------------------------------------------------
// RMSNorm of each row (or a plain copy when g is null), rounded to fp16; with out_lo the
// rounding remainder goes there too (v = hi + lo to about 22 bits, for the split products)
// ---------------------------------------------------------------------------
constexpr int kNormBlock = 1024;
constexpr int kNormPT = 4;   // f32x4 chunks per thread per sweep, all loads issued together
__global__ __launch_bounds__(kNormBlock) void rows_norm_f16_kernel(const float* x, long long ldx, const float* g, int d,
                                                                    float eps, _Float16* out, _Float16* out_lo,
                                                                    long long ldo) {
  __shared__ float s_red[kNormBlock / kWave];
  const int b = blockIdx.x, tid = threadIdx.x;
  const float* xb = x + (long long)b * ldx;
  _Float16* ob = out + (long long)b * ldo;
  _Float16* lb = out_lo ? out_lo + (long long)b * ldo : nullptr;
  if (d <= kNormBlock * 4 * kNormPT) {
    // One sweep: the row and its gains are loaded together and kept in registers.
    f32x4 t[kNormPT], gg[kNormPT];
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < kNormPT; ++q) {
      const int c = (q * kNormBlock + tid) * 4;
      const bool ok = c < d;
      t[q] = ok ? *reinterpret_cast<const f32x4*>(xb + c) : f32x4{0.f, 0.f, 0.f, 0.f};
      gg[q] = (ok && g) ? *reinterpret_cast<const f32x4*>(g + c) : f32x4{1.f, 1.f, 1.f, 1.f};
    }
#pragma unroll
    for (int q = 0; q < kNormPT; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = fmaf(t[q][e], t[q][e], ss);
    ss = group_sum<kWave>(ss);
    if (tid % kWave == 0) s_red[tid / kWave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kNormBlock / kWave; ++i) tot += s_red[i];
    const float inv = g ? 1.0f / sqrtf(tot / (float)d + eps) : 1.0f;   // no gain: plain cast
#pragma unroll
    for (int q = 0; q < kNormPT; ++q) {
      const int c = (q * kNormBlock + tid) * 4;
      if (c >= d) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = t[q][e] * inv * gg[q][e];
        const _Float16 hi = static_cast<_Float16>(v);
        ob[c + e] = hi;
        if (lb) lb[c + e] = static_cast<_Float16>(v - static_cast<float>(hi));
      }
    }
    return;
  }
  float ss = 0.f;
  for (int c0 = 0; c0 < d; c0 += kNormBlock * 4 * kNormPT) {
    f32x4 t[kNormPT];
#pragma unroll
    for (int q = 0; q < kNormPT; ++q) {
      const int c = c0 + (q * kNormBlock + tid) * 4;
      t[q] = c < d ? *reinterpret_cast<const f32x4*>(xb + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int q = 0; q < kNormPT; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = fmaf(t[q][e], t[q][e], ss);
  }
  ss = group_sum<kWave>(ss);
  if (tid % kWave == 0) s_red[tid / kWave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kNormBlock / kWave; ++i) tot += s_red[i];
  const float inv = g ? 1.0f / sqrtf(tot / (float)d + eps) : 1.0f;   // no gain: plain cast
  for (int c0 = 0; c0 < d; c0 += kNormBlock * 4 * kNormPT) {
    f32x4 t[kNormPT], gg[kNormPT];
#pragma unroll
    for (int q = 0; q < kNormPT; ++q) {
      const int c = c0 + (q * kNormBlock + tid) * 4;
      const bool ok = c < d;
      t[q] = ok ? *reinterpret_cast<const f32x4*>(xb + c) : f32x4{0.f, 0.f, 0.f, 0.f};
      gg[q] = (ok && g) ? *reinterpret_cast<const f32x4*>(g + c) : f32x4{1.f, 1.f, 1.f, 1.f};
    }
#pragma unroll
    for (int q = 0; q < kNormPT; ++q) {
      const int c = c0 + (q * kNormBlock + tid) * 4;
      if (c >= d) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = t[q][e] * inv * gg[q][e];
        const _Float16 hi = static_cast<_Float16>(v);
        ob[c + e] = hi;
        if (lb) lb[c + e] = static_cast<_Float16>(v - static_cast<float>(hi));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// gemm_rows: up-projection over gathered rows
// ---------------------------------------------------------------------------
constexpr int kGemmBlock = 256;   // 4 waves

// K slices of a launch whose split follows the device-side tile count.
__device__ __forceinline__ int rows_dyn_ks(const GemmRowsArgs& a, int tiles) {
  const int ks = tiles > 0 ? a.dyn_slots / tiles : 1;
  return ks < 1 ? 1 : (ks > a.ksplit ? a.ksplit : ks);
}

// Epilogue of one output (gathered row i, batch row b): bias, ReLU, the row's own mask, and
// the store in the launch's output mode.
__device__ __forceinline__ void rows_store(const GemmRowsArgs& a, int i, int b, float acc) {
  const int g = i / a.G;
  const int wi = i - g * a.G;
  const int grp = a.sel ? a.sel[g] : g;
  const bool gv = (unsigned)grp < (unsigned)a.n_groups;
  const long long row = gv ? (long long)grp * a.G + wi : 0;
  const float bias = (gv && a.bias) ? a.bias[row] : 0.f;
  const unsigned* rb = a.rowbits ? a.rowbits + (long long)b * a.bits_words : nullptr;
  const bool on = gv && (rb == nullptr || bit_of(rb, grp));
  float v = acc + bias;
  if (a.relu) v = fmaxf(v, 0.f);
  if (a.mode == kGemmOutF16) {
    const float vv = on ? v : 0.f;
    const _Float16 hi = static_cast<_Float16>(vv);
    a.outh[(long long)b * a.ldo + i] = hi;
    if (a.outh_lo) a.outh_lo[(long long)b * a.ldo + i] = static_cast<_Float16>(vv - static_cast<float>(hi));
  } else if (a.mode == kGemmOutF32) {
    if (a.outf_b != nullptr && i >= a.n_rows_a) a.outf_b[(long long)b * a.ldo_b + (i - a.n_rows_a)] = on ? v : 0.f;
    else a.outf[(long long)b * a.ldo + i] = on ? v : 0.f;
  } else if (on && rb != nullptr) {   // q/k/v into the row's own slot order
    const int slot = rank_below(rb, grp);
    a.outf[((long long)b * a.kh + slot) * a.G + wi] = v;
  }
}

// Up-projections: a block of 4 waves owns 64 gathered rows (a 16-row MFMA tile per wave) over
// its slice of K (all of K unless a short launch splits K over blocks; then each slice writes
// partial sums that the finishing kernel adds in slice order), staged through LDS in chunks of
// kRowsKC: one load instruction of a
// wave covers 2 rows x 512 contiguous bytes, and the activation rows (and their remainders)
// are staged once per block instead of once per wave. The next chunk's loads are in flight
// while the MFMAs consume the current one. No cross-wave sum: each wave owns its rows.
// With XF the activations come as fp32 and are split into an fp16 part and its fp16
// remainder while they are staged (the same bits a separate conversion pass would write).
constexpr int kRowsKC = 256;
constexpr int kRowsLdk = kRowsKC + 8;
template <int NT, bool SPLIT, bool XF = false>
__global__ __launch_bounds__(256) void gemm_rows_lds_kernel(GemmRowsArgs a) {
  static_assert(SPLIT || !XF, "fp32 activations are staged as a part and its remainder");
  constexpr int NX = NT * 16;                   // staged activation rows
  constexpr int XL = SPLIT ? 2 : 1;
  constexpr int XLD = NX * kRowsKC / 8 / 256;   // 16-byte activation loads per thread per array
  __shared__ __attribute__((aligned(16))) half_t s_w[64 * kRowsLdk];
  __shared__ __attribute__((aligned(16))) _Float16 s_x[XL][NX * kRowsLdk];
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int lr = lane % 16, lg = lane / 16;
  const int nrows = (a.n_groups_sel ? *a.n_groups_sel : a.n_groups) * a.G;
  // (row tile, K slice) of this block: grid.y slices, or with a device-side split the slices
  // that keep about dyn_slots blocks busy for the union's actual number of tiles.
  int tile = blockIdx.x, slice = blockIdx.y, ks = gridDim.y;
  if (a.dyn_slots > 0) {
    const int tiles = (nrows + 63) / 64;
    ks = rows_dyn_ks(a, tiles);
    if ((int)blockIdx.x >= tiles * ks) return;   // block-uniform
    tile = blockIdx.x / ks;
    slice = blockIdx.x - tile * ks;
  }
  const int r0 = tile * 64;
  if (r0 >= nrows) return;   // block-uniform
  const half_t* W = reinterpret_cast<const half_t*>(a.W);
  // loader: thread -> rows lrow + 8*q (q < 8), 8 halfs at k = kk
  const int lrow = tid / 32, kk = 8 * (tid % 32);
  const half_t* wp[8];
  bool wok[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int i = r0 + lrow + 8 * q;
    long long wrow = -1;
    if (i < nrows) {
      const int g = i / a.G;
      const int grp = a.sel ? a.sel[g] : g;
      if ((unsigned)grp < (unsigned)a.n_groups) wrow = (long long)grp * a.G + (i - g * a.G);
    }
    const half_t* base = W;
    if (a.W_b != nullptr && wrow >= a.n_rows_a) {   // second matrix of a two-matrix launch
      base = reinterpret_cast<const half_t*>(a.W_b);
      wrow -= a.n_rows_a;
    }
    wok[q] = wrow >= 0;
    wp[q] = base + (wrow >= 0 ? wrow : 0) * a.ld + kk;
  }
  // A block's 64 rows all belong to one matrix of a two-matrix launch, hence to one input.
  const bool second = a.X_b != nullptr && r0 >= a.n_rows_a;
  const _Float16* Xs = second ? a.X_b : a.X;
  const _Float16* XLs = second ? a.X_lo_b : a.X_lo;
  u32x4 wreg[8];
  h8v xreg[XL][XLD];
  f32x4 xraw[XF ? XLD : 1][2];   // XF: the fp32 activations of the chunk in flight
  auto load = [&](int k0) {
    const bool kok = k0 + kk < a.d;   // d is a multiple of 8: a chunk is wholly in or out
#pragma unroll
    for (int q = 0; q < 8; ++q)
      wreg[q] = (kok && wok[q]) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp[q] + k0))
                                : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int p = 0; p < XLD; ++p) {
      const int b = lrow + 8 * p;
      const bool ok = kok && b < a.B;
      if constexpr (XF) {
        const float* xp = a.Xf + (long long)b * a.ldx + k0 + kk;
        xraw[p][0] = ok ? *reinterpret_cast<const f32x4*>(xp) : f32x4{0.f, 0.f, 0.f, 0.f};
        xraw[p][1] = ok ? *reinterpret_cast<const f32x4*>(xp + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
        xreg[0][p] = ok ? *reinterpret_cast<const h8v*>(Xs + (long long)b * a.ldx + k0 + kk)
                        : h8v{0, 0, 0, 0, 0, 0, 0, 0};
        if constexpr (SPLIT)
          xreg[1][p] = ok ? *reinterpret_cast<const h8v*>(XLs + (long long)b * a.ldx + k0 + kk)
                          : h8v{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  };
  f4v acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f4v{0.f, 0.f, 0.f, 0.f};
  // K chunks of this block's slice (grid.y slices when K is split over blocks)
  const int nch = (a.d + kRowsKC - 1) / kRowsKC;
  const int kfirst = (int)((long long)nch * slice / ks) * kRowsKC;
  const int klast = min(a.d, (int)((long long)nch * (slice + 1) / ks) * kRowsKC);
  if (kfirst < klast) load(kfirst);
  for (int k0 = kfirst; k0 < klast; k0 += kRowsKC) {   // block-uniform
    __syncthreads();   // the previous chunk's readers are done
#pragma unroll
    for (int q = 0; q < 8; ++q) *reinterpret_cast<u32x4*>(&s_w[(lrow + 8 * q) * kRowsLdk + kk]) = wreg[q];
    if constexpr (XF) {
#pragma unroll
      for (int p = 0; p < XLD; ++p)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = xraw[p][e / 4][e % 4];
          const _Float16 hi = static_cast<_Float16>(v);
          xreg[0][p][e] = hi;
          xreg[1][p][e] = static_cast<_Float16>(v - static_cast<float>(hi));
        }
    }
#pragma unroll
    for (int x = 0; x < XL; ++x)
#pragma unroll
      for (int p = 0; p < XLD; ++p) *reinterpret_cast<h8v*>(&s_x[x][(lrow + 8 * p) * kRowsLdk + kk]) = xreg[x][p];
    __syncthreads();
    if (k0 + kRowsKC < klast) load(k0 + kRowsKC);
    const int nks = min(kRowsKC, a.d - k0 + 31) / 32;   // k-steps holding data (the rest are zero)
    for (int kstep = 0; kstep < nks; ++kstep) {
      const h8v af = *reinterpret_cast<const h8v*>(&s_w[(16 * wv + lr) * kRowsLdk + 32 * kstep + 8 * lg]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const h8v bf = *reinterpret_cast<const h8v*>(&s_x[0][(16 * nt + lr) * kRowsLdk + 32 * kstep + 8 * lg]);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, acc[nt], 0, 0, 0);
        if constexpr (SPLIT) {
          const h8v bl = *reinterpret_cast<const h8v*>(&s_x[XL - 1][(16 * nt + lr) * kRowsLdk + 32 * kstep + 8 * lg]);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bl, acc[nt], 0, 0, 0);
        }
      }
    }
  }
  // D layout: lane holds batch row 16*nt + lr, gathered rows r0 + 16*wv + 4*lg + e
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = r0 + 16 * wv + 4 * lg + e;
    if (i >= nrows) continue;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int b = nt * 16 + lr;
      if (b >= a.B) continue;
      if (ks > 1) a.kpart[((long long)slice * a.B + b) * a.kld + i] = acc[nt][e];
      else rows_store(a, i, b, acc[nt][e]);
    }
  }
}

// Sum of the K slices of a split up-projection, in slice order, then the epilogue.
__global__ void gemm_rows_finish_kernel(GemmRowsArgs a) {
  const int nrows = (a.n_groups_sel ? *a.n_groups_sel : a.n_groups) * a.G;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int b = blockIdx.y;
  if (i >= nrows) return;
  const int ks = a.dyn_slots > 0 ? rows_dyn_ks(a, (nrows + 63) / 64) : a.ksplit;
  if (ks == 1) return;   // the up-projection stored its outputs itself
  float p[kRowsMaxSplit];   // every slice's partial in flight together, summed in slice order
#pragma unroll
  for (int q = 0; q < kRowsMaxSplit; ++q) p[q] = q < ks ? a.kpart[((long long)q * a.B + b) * a.kld + i] : 0.f;
  float v = 0.f;
#pragma unroll
  for (int q = 0; q < kRowsMaxSplit; ++q)
    if (q < ks) v += p[q];
  rows_store(a, i, b, v);
}

// ---------------------------------------------------------------------------
// gemm_cols: down-projection over gathered rows, row groups -> partials
// ---------------------------------------------------------------------------
#ifndef DV_ROWS_DYN_MAXB
#define DV_ROWS_DYN_MAXB 8    // union up-projections of at most this many rows split K on the device
#endif
static_assert(DV_ROWS_DYN_MAXB <= 16, "the device-side split launches the 16-row activation tile");
#ifndef DV_ROWS_DYN_BPC
#define DV_ROWS_DYN_BPC 3     // blocks per CU the device-side K split aims for
#endif
#ifndef DV_COLS_BPC
#define DV_COLS_BPC 3    // target blocks per CU when choosing the down-projection's row groups
#endif
#ifndef DV_COLS_CW
#define DV_COLS_CW 256   // output columns per block: 512-byte strips of every weight row
#endif

// LDS slot of tile column c: columns are rotated within each group of 8 by half the group
// number, so that the 16-byte transposed writes of 16 neighbouring lanes (columns 8 apart) and
// the B-fragment reads of 16 neighbouring columns each fall on 16 distinct bank quads with the
// 36-dword column pitch (the plain layout put 8 lanes on each quad of the writes).
__device__ __forceinline__ int cols_slot(int c) { return (c & ~7) | (((c & 7) + (c >> 4)) & 7); }

constexpr int kColsRowStage = 2048;   // union positions whose weight rows are staged in LDS per sweep

// A tile is KT gathered rows x CW columns (32 KB). Each thread loads the same 8 columns of 8
// consecutive rows (for a fixed row, a wave reads CW/8*16 contiguous bytes per row), transposes
// that 8 x 8 block in registers and writes each column's 8 rows as one 16-byte LDS store: the
// B fragment of the MFMA (8 consecutive k at one column) is then one 16-byte LDS read. The next
// tile's rows are in flight while the current one is transposed and consumed.
template <int MT, int CW>
__global__ __launch_bounds__(kGemmBlock) void gemm_cols_kernel(GemmColsArgs a) {
  constexpr int TPC = CW / 8;             // threads across the tile's columns
  constexpr int RGP = kGemmBlock / TPC;   // 8-row groups per tile
  constexpr int KT = 8 * RGP;             // rows per tile
  constexpr int LDK = KT + 8;             // halfs per transposed column (padded)
  constexpr int CTW = CW / 16 / (kGemmBlock / kWave);   // 16-column MFMA tiles per wave
  constexpr int KS = KT / 32;             // MFMA k-steps per tile
  static_assert(KT % 32 == 0 && CTW >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) half_t s_w[CW * LDK];
  __shared__ __attribute__((aligned(16))) _Float16 s_c[MT * 16 * LDK];   // coefficients [b][k] of the tile
  __shared__ int s_rows[kColsRowStage];   // weight rows of the staged sweep of union positions
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int lr = lane % 16, lg = lane / 16;
  const int tc = tid % TPC, trg = tid / TPC;
  const int c0 = blockIdx.x * CW;
  const int rg = blockIdx.y;
  const int K = *a.n_groups_sel * a.G;
  int rpg = (K + a.RG - 1) / a.RG;
  rpg = (rpg + KT - 1) / KT * KT;
  const int kb0 = min(K, rg * rpg);
  const int kend = min(K, kb0 + rpg);
  const half_t* W = reinterpret_cast<const half_t*>(a.W);
  const int col = c0 + 8 * tc;
  const bool colv = col < a.d;   // d is a multiple of 8: a chunk is wholly in or out
  auto row_of = [&](int k) -> int {   // weight row of union position k, -1 past the group
    if (k >= kend) return -1;
    const int g = k / a.G;
    const int grp = a.sel[g];
    if ((unsigned)grp >= (unsigned)a.n_groups) return -1;
    return grp * a.G + (k - g * a.G);
  };
  // The weight rows of the group's union positions are staged in LDS a sweep of
  // kColsRowStage positions at a time (every index load of the sweep in flight together), so
  // the tile loop takes them from LDS instead of waiting on a dependent global load per tile.
  int sweep0 = kb0;
  auto stage_rows = [&](int k0) {   // block-uniform; k0 is a tile boundary
    constexpr int PT = kColsRowStage / kGemmBlock;
    int v[PT];
#pragma unroll
    for (int q = 0; q < PT; ++q) v[q] = row_of(k0 + tid + q * kGemmBlock);
    __syncthreads();   // the previous sweep's readers are done
#pragma unroll
    for (int q = 0; q < PT; ++q) s_rows[tid + q * kGemmBlock] = v[q];
    __syncthreads();
    sweep0 = k0;
  };
  auto rows_for = [&](int* r, int kb) {   // the tile at kb lies in the staged sweep
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int k = kb + 8 * trg + q;
      r[q] = k < kend ? s_rows[k - sweep0] : -1;
    }
  };
  auto load_tile = [&](u32x4* wt, const int* r) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      wt[q] = (r[q] >= 0 && colv)
                  ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(W + (long long)r[q] * a.ld + col))
                  : u32x4{0u, 0u, 0u, 0u};
  };
  // Coefficient tile C[b][kb .. kb + KT) for the MT*16 batch rows, staged in LDS with the
  // weights: thread -> batch row tid / (KT/8), 8 consecutive k at 8 * (tid % (KT/8)).
  constexpr int CPR = KT / 8;   // 16-byte chunks per coefficient row
  const int cb = tid / CPR, ck = 8 * (tid % CPR);
  auto load_coef = [&](h8v& cf, int kb) {
    const int k = kb + ck;
    cf = h8v{0, 0, 0, 0, 0, 0, 0, 0};
    if (cb < MT * 16 && cb < a.B && k < kend) {
      const _Float16* cp = a.C + (long long)cb * a.ldc + k;
      if (k + 8 <= kend) {
        cf = *reinterpret_cast<const h8v*>(cp);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) cf[e] = (k + e < kend) ? cp[e] : static_cast<_Float16>(0.f);
      }
    }
  };
  f4v acc[CTW][MT];
#pragma unroll
  for (int i = 0; i < CTW; ++i)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[i][mt] = f4v{0.f, 0.f, 0.f, 0.f};
  u32x4 cur[8], nxt[8];
  h8v ccur, cnxt;
  int rn[8];
  if (kb0 < kend) {
    stage_rows(kb0);
    rows_for(rn, kb0);
    load_tile(cur, rn);
    load_coef(ccur, kb0);
  }
  for (int kb = kb0; kb < kend; kb += KT) {   // block-uniform
    const int kn = kb + KT;
    if (kn < kend) {
      if (kn >= sweep0 + kColsRowStage) stage_rows(kn);
      rows_for(rn, kn);   // no loads past the group's end (rows_for gives -1 there)
      load_tile(nxt, rn);
      load_coef(cnxt, kn);
    }
    h8v colv8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int q = 0; q < 8; ++q) colv8[j][q] = __builtin_bit_cast(h8v, cur[q])[j];
    __syncthreads();   // the previous tile's readers are done
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<h8v*>(&s_w[cols_slot(8 * tc + j) * LDK + 8 * trg]) = colv8[j];
    if (cb < MT * 16) *reinterpret_cast<h8v*>(&s_c[cb * LDK + ck]) = ccur;
    __syncthreads();
#pragma unroll
    for (int kstep = 0; kstep < KS; ++kstep)
#pragma unroll
      for (int i = 0; i < CTW; ++i) {
        const int cl = (wv * CTW + i) * 16 + lr;
        const h8v bf = *reinterpret_cast<const h8v*>(&s_w[cols_slot(cl) * LDK + 32 * kstep + 8 * lg]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const h8v af = *reinterpret_cast<const h8v*>(&s_c[(16 * mt + lr) * LDK + 32 * kstep + 8 * lg]);
          acc[i][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, acc[i][mt], 0, 0, 0);
        }
      }
#pragma unroll
    for (int q = 0; q < 8; ++q) cur[q] = nxt[q];
    ccur = cnxt;
  }
  // D layout: lane holds output column lr of its tile, batch rows 16*mt + 4*lg + e
#pragma unroll
  for (int i = 0; i < CTW; ++i) {
    const int c = c0 + (wv * CTW + i) * 16 + lr;
    if (c >= a.d) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int b = 16 * mt + 4 * lg + e;
        if (b < a.B) a.partial[((long long)b * a.RG + rg) * a.d + c] = acc[i][mt][e];
      }
  }
}

// o[b][slot][e] (fp32, the row's head order) -> C[b][u*dh + e] (fp16, union order, 0 where
// head u of the union is not selected by row b).
__global__ void heads_to_union_kernel(const float* o, int kh, int dh, const int32_t* uh, const int* n_uh,
                                      const unsigned* hbits, int hwords, int B, _Float16* C, long long ldc) {
  const int u = blockIdx.x, b = blockIdx.y, e = threadIdx.x;
  if (u >= *n_uh || e >= dh || b >= B) return;
  const int h = uh[u];
  const unsigned* rb = hbits + (long long)b * hwords;
  float v = 0.f;
  if (bit_of(rb, h)) v = o[((long long)b * kh + rank_below(rb, h)) * dh + e];
  C[(long long)b * ldc + (long long)u * dh + e] = static_cast<_Float16>(v);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
hipError_t launch_union(const UnionArgs& a, hipStream_t s) {
  for (int i = 0; i < a.nprob; ++i)
    if (a.p[i].n > kUnionMaxN || a.p[i].n <= 0) return hipErrorInvalidValue;
  int maxw = 1;
  for (int i = 0; i < a.nprob; ++i) maxw = max(maxw, (a.p[i].n + 31) / 32);
  hipLaunchKernelGGL(union_rows_kernel, dim3((maxw + kUnionRowsBlock - 1) / kUnionRowsBlock, a.B, a.nprob),
                     dim3(kUnionRowsBlock), 0, s, a);
  const int nblk = (maxw + kUnionWpb - 1) / kUnionWpb;
  hipLaunchKernelGGL(union_or_kernel, dim3(nblk, a.nprob), dim3(kUnionOrBlock), 0, s, a);
  hipLaunchKernelGGL(union_list_kernel, dim3(nblk, a.nprob), dim3(kUnionWpb), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rows_norm_f16(const float* x, long long ldx, const float* g, int d, float eps, int B, _Float16* out,
                                _Float16* out_lo, long long ldo, hipStream_t s) {
  if (d % 4 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rows_norm_f16_kernel, dim3(B), dim3(kNormBlock), 0, s, x, ldx, g, d, eps, out, out_lo, ldo);
  return hipGetLastError();
}

template <int NT, bool SPLIT>
static void launch_rows_lds(const GemmRowsArgs& a, int max_rows, int ks, hipStream_t s) {
  if (SPLIT && a.Xf != nullptr)
    hipLaunchKernelGGL((gemm_rows_lds_kernel<NT, SPLIT, SPLIT>), dim3((max_rows + 63) / 64, ks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((gemm_rows_lds_kernel<NT, SPLIT>), dim3((max_rows + 63) / 64, ks), dim3(256), 0, s, a);
}

// A short launch (fewer 64-row tiles than twice the CUs) splits K over blocks, up to
// kRowsMaxSplit slices of whole chunks, and the finishing kernel adds the slices in order.
hipError_t launch_gemm_rows(const GemmRowsArgs& a_in, int max_rows, int cus, hipStream_t s) {
  GemmRowsArgs a = a_in;
  if (a.d % 8 != 0 || a.B < 1 || a.B > kBatchMax || max_rows < 0) return hipErrorInvalidValue;   // tail K steps are guarded
  if (a.W_b != nullptr && (a.G != 1 || a.sel != nullptr || a.n_rows_a < 0 || a.n_rows_a > a.n_groups))
    return hipErrorInvalidValue;
  if (a.X_b != nullptr && (a.W_b == nullptr || a.n_rows_a % 64 != 0 || (a.X_lo != nullptr) != (a.X_lo_b != nullptr)))
    return hipErrorInvalidValue;
  if (a.Xf != nullptr && (a.X_b != nullptr || a.X_lo != nullptr)) return hipErrorInvalidValue;
  if (max_rows == 0) return hipSuccess;
  const bool split = a.X_lo != nullptr || a.Xf != nullptr;
  const int tiles = (max_rows + 63) / 64;
  const int nch = (a.d + kRowsKC - 1) / kRowsKC;
  int ks = 1;
  a.dyn_slots = 0;
  if (a.kpart != nullptr && max_rows <= kRowsSplitMaxRows && tiles < 2 * cus && a.kld >= max_rows) {
    ks = std::max(1, std::min({(2 * cus + tiles - 1) / tiles, nch, kRowsMaxSplit}));
  } else if (a.kpart != nullptr && a.n_groups_sel != nullptr && !split && a.B <= DV_ROWS_DYN_MAXB) {
    // A union launch: its row count is known only on the device, so blocks pick their K slice
    // from it, up to the slices the partial buffer holds at this launch's largest row count.
    const int cap = (int)std::min<long long>(kRowsMaxSplit, (long long)kRowsMaxSplit * kRowsSplitMaxRows / max_rows);
    const int kmax = std::min(nch, cap);
    if (kmax >= 2) {
      a.ksplit = kmax;
      a.dyn_slots = DV_ROWS_DYN_BPC * cus;
      a.kld = max_rows;
      hipLaunchKernelGGL((gemm_rows_lds_kernel<1, false>), dim3(tiles * kmax, 1), dim3(256), 0, s, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(gemm_rows_finish_kernel, dim3((max_rows + 255) / 256, a.B), dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
  a.ksplit = ks;
  if (a.B <= 16) {
    if (split) launch_rows_lds<1, true>(a, max_rows, ks, s);
    else launch_rows_lds<1, false>(a, max_rows, ks, s);
  } else {
    if (split) launch_rows_lds<2, true>(a, max_rows, ks, s);
    else launch_rows_lds<2, false>(a, max_rows, ks, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ks == 1) return e;
  hipLaunchKernelGGL(gemm_rows_finish_kernel, dim3((max_rows + 255) / 256, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

int gemm_cols_rg(int d, int max_rows, int B, int cus) {
  constexpr int KT = 8 * kGemmBlock / (DV_COLS_CW / 8);
  const int ctiles = (d + DV_COLS_CW - 1) / DV_COLS_CW;
  int rg = (DV_COLS_BPC * cus + ctiles - 1) / ctiles;     // about DV_COLS_BPC blocks per CU
  const int cap = max(1, max_rows / (2 * KT));            // at least 2 tiles of rows per group
  rg = min(rg, cap);
  rg = min(rg, kBatchMaxRG);
  while (rg > 1 && (long long)rg * B > 1024) --rg;        // bounds the partial buffer
  return max(rg, 1);
}

hipError_t launch_gemm_cols(const GemmColsArgs& a, hipStream_t s) {
  if (a.d % 8 != 0 || a.B < 1 || a.B > kBatchMax || a.RG < 1 || a.RG > kBatchMaxRG) return hipErrorInvalidValue;
  const dim3 grid((a.d + DV_COLS_CW - 1) / DV_COLS_CW, a.RG);
  if (a.B <= 16) hipLaunchKernelGGL((gemm_cols_kernel<1, DV_COLS_CW>), grid, dim3(kGemmBlock), 0, s, a);
  else hipLaunchKernelGGL((gemm_cols_kernel<2, DV_COLS_CW>), grid, dim3(kGemmBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_heads_to_union(const float* o, int kh, int dh, const int32_t* uh, const int* n_uh, const unsigned* hbits,
                                 int hwords, int B, int max_uh, _Float16* C, long long ldc, hipStream_t s) {
  if (dh > 1024 || max_uh < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(heads_to_union_kernel, dim3(max_uh, B), dim3(dh), 0, s, o, kh, dh, uh, n_uh, hbits, hwords, B, C, ldc);
  return hipGetLastError();
}

}  // namespace dv
