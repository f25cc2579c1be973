// Gather row-dot kernel ("GEMV1" shape): one fp32 dot product per selected weight row.
//
// Used for the predictor's two factors, the head-sparse q/k/v projection and the
// active-neuron up-projection (DejaVu Guide, "Mathematical Formulation of Lookahead
// Predictors", "Head-Pruned Attention Dispatch" and the sparse MLP of "Step-by-Step
// Implementation"). Rows are neuron-major, so every selected row is one contiguous burst.
//
// Tiling: TPR threads share one row; each thread owns CH 16-byte chunks of the row
// (chunk c = lane + TPR*j) and keeps the matching slice of the (normalised) input vector
// in registers for the whole kernel, so the input is read from L2 once per block. A block
// keeps R rows per row-slot in flight (R*CH 16-byte loads per thread) to cover HBM latency.
// Rows are dealt to row-slots round-robin across the grid. The dot product is summed in
// a fixed order (per-thread chunks, xor butterfly, waves in order): bitwise deterministic.
#include <hip/hip_ext.h>

#include "dv_device.h"
#include "dv_kernels.h"

namespace dv {

constexpr int kRowdotBlock = 256;
// Tile parameters (compile-time; the defaults are the tuned values).
#ifndef DV_ROWDOT_BPC_BIG
#define DV_ROWDOT_BPC_BIG 2  // target resident blocks per CU for long rows (>= 5 chunks/thread)
#endif
#ifndef DV_ROWDOT_BPC
#define DV_ROWDOT_BPC 2      // target resident blocks per CU otherwise
#endif
#ifndef DV_ROWDOT_RBIG
#define DV_ROWDOT_RBIG 4     // rows in flight per row-slot when a thread holds >= 5 chunks
#endif
#ifndef DV_ROWDOT_WAVES_PER_EU
#define DV_ROWDOT_WAVES_PER_EU 1  // lower bound on resident waves per SIMD the registers must allow
#endif

#ifndef DV_ROWDOT_RMID
#define DV_ROWDOT_RMID 4     // rows in flight per row-slot when a thread holds 3 or 4 chunks
#endif

__host__ __device__ constexpr int rowdot_rows_in_flight(int ch) {
  return ch >= 5 ? DV_ROWDOT_RBIG : (ch >= 3 ? DV_ROWDOT_RMID : (ch == 2 ? 6 : 8));
}

// TAG only separates launch sites in profiles (1 = head-sparse q/k/v projection).
template <typename WT, int TPR, int CH, int TAG>
__global__ __launch_bounds__(kRowdotBlock) __attribute__((amdgpu_waves_per_eu(DV_ROWDOT_WAVES_PER_EU)))
void rowdot_kernel(RowDotArgs a) {
  constexpr int VEC = Vec<WT>::N;
  constexpr int SLOTS = kRowdotBlock / TPR;
  constexpr int R = rowdot_rows_in_flight(CH);
  constexpr int GW = TPR < kWave ? TPR : kWave;       // lanes per in-wave reduction
  constexpr int WPR = TPR > kWave ? TPR / kWave : 1;  // waves per row
  __shared__ float s_red[R][SLOTS][WPR];
  __shared__ float s_norm[SLOTS][WPR];

  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  int bx = blockIdx.x;
  int si = 0;
  if (a.nseg > 1 && bx >= a.seg[0].blocks) {
    bx -= a.seg[0].blocks;
    si = 1;
    if (a.nseg > 2 && bx >= a.seg[1].blocks) {
      bx -= a.seg[1].blocks;
      si = 2;
    }
  }
  static_assert(kRowdotMaxSeg == 3, "segment selection covers three segments");
  const RowDotSeg S = si == 0 ? a.seg[0] : (si == 1 ? a.seg[1] : a.seg[2]);

  const int slot = tid / TPR;
  const int lr = tid % TPR;
  const int wr = lr / kWave;  // wave index within the row (0 when TPR <= 64)
  const int nchunk = a.d / VEC;
  const WT* W = reinterpret_cast<const WT*>(S.W);
  const int TS = S.blocks * SLOTS;  // row-slots of this segment
  const int32_t* idxb = S.idx ? S.idx + (long long)b * S.idx_bstride : nullptr;
  float* outb = S.out + (long long)b * S.ldo;

  // Input slice of this thread, widened to fp32, in registers (requested first).
  float xr[CH][VEC];
  const float* xb = S.x + (long long)b * S.ldx;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = lr + TPR * j;
    if (c < nchunk) {
#pragma unroll
      for (int v = 0; v < VEC / 4; ++v) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(xb + c * VEC + 4 * v);
        xr[j][4 * v + 0] = t[0]; xr[j][4 * v + 1] = t[1];
        xr[j][4 * v + 2] = t[2]; xr[j][4 * v + 3] = t[3];
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) xr[j][e] = 0.f;
    }
  }

  // Rows of the batch starting at `base` and their weight loads. The first batch is
  // requested before the input norm is computed so the two latencies overlap.
  long long row[R];
  bool rv[R];
  Chunk<WT> w[R][CH];
  auto issue = [&](int base) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = base + slot + r * TS;
      rv[r] = false;
      row[r] = 0;
      if (i < S.n_out) {
        int g = i / S.G;
        // With TPR >= 64 a wave serves one row: keep its index scalar so the index load
        // does not queue behind the weight loads of the vector-memory counter.
        if constexpr (TPR >= kWave) g = wave_uniform(g);
        const int wi = i - g * S.G;
        const int grp = idxb ? idxb[g] : g;
        if ((unsigned)grp < (unsigned)S.n_groups) {
          rv[r] = true;
          row[r] = (long long)grp * S.G + wi;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int c = lr + TPR * j;
        if (rv[r] && c < nchunk) w[r][j] = load_chunk<WT>(W + row[r] * S.ld + (long long)c * VEC);
        else w[r][j].raw = u32x4{0u, 0u, 0u, 0u};
      }
  };
  int base = bx * SLOTS;
  if (base < S.n_out) issue(base);

  if (S.norm_g != nullptr) {
    // RMSNorm folded into the prologue: the threads of a row-slot hold the whole vector.
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int e = 0; e < VEC; ++e) ss = fmaf(xr[j][e], xr[j][e], ss);
    ss = group_sum<GW>(ss);
    if constexpr (WPR > 1) {
      if ((lr % kWave) == 0) s_norm[slot][wr] = ss;
      __syncthreads();
      ss = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < WPR; ++w2) ss += s_norm[slot][w2];
    }
    const float inv = 1.0f / sqrtf(ss / (float)a.d + a.eps);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = lr + TPR * j;
      if (c < nchunk) {
#pragma unroll
        for (int v = 0; v < VEC / 4; ++v) {
          const f32x4 g = *reinterpret_cast<const f32x4*>(S.norm_g + c * VEC + 4 * v);
#pragma unroll
          for (int e = 0; e < 4; ++e) xr[j][4 * v + e] = xr[j][4 * v + e] * inv * g[e];
        }
      }
    }
  }

  // Block-uniform loop so the barriers below are reached by every thread.
  for (; base < S.n_out; base += TS * R) {
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc[r] = 0.f;
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        float wf[VEC];
        widen(w[r][j], wf);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[r] = fmaf(wf[e], xr[j][e], acc[r]);
      }
      acc[r] = group_sum<GW>(acc[r]);
    }
    long long row_done[R];
    bool rv_done[R];
#pragma unroll
    for (int r = 0; r < R; ++r) { row_done[r] = row[r]; rv_done[r] = rv[r]; }
    // next batch's loads go out before this batch's reduction and store
    if (base + TS * R < S.n_out) issue(base + TS * R);
    if constexpr (WPR > 1) {
      if ((lr % kWave) == 0)
#pragma unroll
        for (int r = 0; r < R; ++r) s_red[r][slot][wr] = acc[r];
      __syncthreads();
      if (lr == 0)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float t = 0.f;
#pragma unroll
          for (int w2 = 0; w2 < WPR; ++w2) t += s_red[r][slot][w2];
          acc[r] = t;
        }
      __syncthreads();
    }
    if (lr == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int i = base + slot + r * TS;
        if (i < S.n_out) {
          float v = 0.f;
          if (rv_done[r]) {
            v = acc[r] + (S.bias ? S.bias[row_done[r]] : 0.f);
            if (S.relu) v = fmaxf(v, 0.f);
          }
          outb[i] = v;
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// host side: tiling choice and dispatch
// --------------------------------------------------------------------------

// Among tilings with the same lane utilisation the one with the fewest threads per row wins:
// rows shared by at most one wave reduce with shuffles only (no LDS round and no barrier).
static const int kTprs[] = {32, 64, 128, 256};

static bool ch_supported(int ch) { return ch == 1 || ch == 2 || ch == 3 || ch == 4 || ch == 5 || ch == 6 || ch == 8; }

bool rowdot_plan(int d, bool f16, int* tpr, int* ch) {
  const int vec = f16 ? 8 : 4;
  if (d <= 0 || d % vec) return false;
  const int nchunk = d / vec;
  double best = -1.0;
  for (int t : kTprs) {
    int c = (nchunk + t - 1) / t;
    while (c <= 8 && !ch_supported(c)) ++c;
    if (c > 8) continue;
    const double util = (double)nchunk / (double)(t * c);
    if (util > best + 1e-9) { best = util; *tpr = t; *ch = c; }
  }
  return best > 0.0;
}

int rowdot_rows_per_slot(long long total_rows, int tpr, int ch, int cus) {
  const int slots = kRowdotBlock / tpr;
  const long long target = (long long)cus * (ch >= 5 ? DV_ROWDOT_BPC_BIG : DV_ROWDOT_BPC);
  if (total_rows < 1) total_rows = 1;
  return (int)((total_rows + target * slots - 1) / (target * slots));
}

int rowdot_blocks_for(int n_out, int tpr, int per_slot) {
  if (n_out <= 0) return 1;
  const int slots = kRowdotBlock / tpr;
  long long blocks = ((long long)n_out + (long long)per_slot * slots - 1) / ((long long)per_slot * slots);
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

typedef void (*RowdotFn)(RowDotArgs);

template <typename WT, int TPR, int TAG>
static RowdotFn pick_ch(int ch) {
  switch (ch) {
    case 1: return rowdot_kernel<WT, TPR, 1, TAG>;
    case 2: return rowdot_kernel<WT, TPR, 2, TAG>;
    case 3: return rowdot_kernel<WT, TPR, 3, TAG>;
    case 4: return rowdot_kernel<WT, TPR, 4, TAG>;
    case 5: return rowdot_kernel<WT, TPR, 5, TAG>;
    case 6: return rowdot_kernel<WT, TPR, 6, TAG>;
    case 8: return rowdot_kernel<WT, TPR, 8, TAG>;
  }
  return nullptr;
}

template <typename WT, int TAG>
static RowdotFn pick(int tpr, int ch) {
  switch (tpr) {
    case 256: return pick_ch<WT, 256, TAG>(ch);
    case 128: return pick_ch<WT, 128, TAG>(ch);
    case 64: return pick_ch<WT, 64, TAG>(ch);
    case 32: return pick_ch<WT, 32, TAG>(ch);
  }
  return nullptr;
}

hipError_t launch_rowdot(const RowDotArgs& a, bool f16, int B, hipStream_t s, int tag, hipEvent_t ev_begin,
                         hipEvent_t ev_end) {
  int tpr = 0, ch = 0;
  if (!rowdot_plan(a.d, f16, &tpr, &ch)) return hipErrorInvalidValue;
  RowdotFn fn = tag == 1 ? (f16 ? pick<half_t, 1>(tpr, ch) : pick<float, 1>(tpr, ch))
                         : (f16 ? pick<half_t, 0>(tpr, ch) : pick<float, 0>(tpr, ch));
  if (fn == nullptr) return hipErrorInvalidValue;
  int blocks = 0;
  for (int i = 0; i < a.nseg; ++i) blocks += a.seg[i].blocks;
  if (ev_begin != nullptr || ev_end != nullptr) {
    // The events take this dispatch's own begin/end timestamps (not markers around it).
    hipExtLaunchKernelGGL(fn, dim3(blocks, B), dim3(kRowdotBlock), 0, s, ev_begin, ev_end, 0u, a);
  } else {
    hipLaunchKernelGGL(fn, dim3(blocks, B), dim3(kRowdotBlock), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dv
