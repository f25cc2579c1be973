// Device body of the gather row-dot (one block of kRowdotBlock threads), a device function
// so that a kernel can run row-dot blocks among other work. The tiling and the fixed
// summation order are described in k_rowdot.hip.
#pragma once
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


// Block bx0 of the row-dot over segments a.seg (blocks numbered across the segments), batch
// row b. Every thread of the block must call it (it synchronises the block).
template <typename WT, int TPR, int CH>
__device__ __forceinline__ void rowdot_block(const RowDotArgs& a, int bx0, int b) {
  int bx = bx0;
  constexpr int VEC = Vec<WT>::N;
  constexpr int SLOTS = kRowdotBlock / TPR;
  constexpr int R = rowdot_rows_in_flight(CH);
  constexpr int GW = TPR < kWave ? TPR : kWave;       // lanes per in-wave reduction
  constexpr int WPR = TPR > kWave ? TPR / kWave : 1;  // waves per row
  __shared__ float s_red[R][SLOTS][WPR];
  __shared__ float s_norm[SLOTS][WPR];

  const int tid = threadIdx.x;
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

}  // namespace dv
