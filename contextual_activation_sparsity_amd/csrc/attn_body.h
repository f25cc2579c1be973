// Device bodies of the head-sparse decode attention (split-T partials and their combine), as
// device functions of one block each. The method and the fixed combination order are
// described in k_attn.hip.
#pragma once
#include "dv_device.h"
#include "dv_kernels.h"

namespace dv {

constexpr int kAttnBlock = 256;
constexpr int kAttnStage = 40;  // chunk partials staged in LDS per sweep of the combine

// Block (chunk c, selected head s, batch row b) of the split-T attention. Every thread of
// the block must call it (it synchronises the block).
template <typename WT, int DH, int NPASS>
__device__ __forceinline__ void attn_block(const AttnArgs& a, int c, int s, int b) {
  constexpr int VEC = Vec<WT>::N;
  constexpr int TPK = DH / VEC;
  constexpr int KPP = kAttnBlock / TPK;
  constexpr int TC = KPP * NPASS;
  constexpr int NW = kAttnBlock / kWave;
  static_assert(TPK <= kWave, "one key per wave at most");
  static_assert(DH <= kAttnBlock, "one thread per output element in the combine");
  __shared__ float s_o[KPP][DH];
  __shared__ float s_l[KPP];
  __shared__ float s_m[NW];

  const int tid = threadIdx.x;
  const int ks = tid / TPK;
  const int kl = tid % TPK;
  const int h = a.heads[(long long)b * a.kh + s];
  const bool hv = (unsigned)h < (unsigned)a.n_heads;
  const int t_past = a.t_rows ? min(max(a.t_rows[b], 0), a.t_past) : a.t_past;
  const float LOG2E = 1.4426950408889634f;

  const float* qkv = a.qkv + ((long long)b * a.kh + s) * 3 * DH;
  float q[VEC], kcur[VEC], vcur[VEC];
  const float qscale = LOG2E / sqrtf((float)DH);
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    q[e] = qkv[kl * VEC + e] * qscale;
    kcur[e] = qkv[DH + kl * VEC + e];
    vcur[e] = qkv[2 * DH + kl * VEC + e];
  }

  const long long hoff = hv ? (((long long)b * a.n_heads + h) * a.t_max) * DH : 0;
  WT* K = reinterpret_cast<WT*>(a.k_cache) + hoff;
  WT* V = reinterpret_cast<WT*>(a.v_cache) + hoff;
  const int t0 = c * TC;

  Chunk<WT> kc[NPASS], vc[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int t = t0 + p * KPP + ks;
    if (hv && t < t_past) {
      kc[p] = load_chunk<WT>(K + (long long)t * DH + kl * VEC);
      vc[p] = load_chunk<WT>(V + (long long)t * DH + kl * VEC);
    } else {
      kc[p].raw = u32x4{0u, 0u, 0u, 0u};
      vc[p].raw = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // Scores (log2 domain) and the block maximum.
  float sc[NPASS];
  float m = -INFINITY;
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int t = t0 + p * KPP + ks;
    float kf[VEC];
    if (t < t_past) widen(kc[p], kf);
    else
#pragma unroll
      for (int e = 0; e < VEC; ++e) kf[e] = kcur[e];
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) dot = fmaf(q[e], kf[e], dot);
    dot = group_sum<TPK>(dot);
    sc[p] = (hv && t <= t_past) ? dot : -INFINITY;
    m = fmaxf(m, sc[p]);
  }
  m = group_max<kWave>(m);
  if ((tid % kWave) == 0) s_m[tid / kWave] = m;
  __syncthreads();
  m = s_m[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) m = fmaxf(m, s_m[w]);

  // p . V and sum p (only chunks with at least one valid key reach a finite m).
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  float l = 0.f;
  if (m > -INFINITY) {
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int t = t0 + p * KPP + ks;
      const float pw = (sc[p] > -INFINITY) ? exp2f(sc[p] - m) : 0.f;
      float vf[VEC];
      if (t < t_past) widen(vc[p], vf);
      else
#pragma unroll
        for (int e = 0; e < VEC; ++e) vf[e] = (t == t_past) ? vcur[e] : 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = fmaf(pw, vf[e], acc[e]);
      l += pw;
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) s_o[ks][kl * VEC + e] = acc[e];
  if (kl == 0) s_l[ks] = l;

  // Append the current token's k, v to the cache of this head.
  if (hv && t_past >= t0 && t_past < t0 + TC) {
    const int own = (t_past - t0) % KPP;  // key slot that met position t_past
    if (ks == own) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        K[(long long)t_past * DH + kl * VEC + e] = narrow<WT>(kcur[e]);
        V[(long long)t_past * DH + kl * VEC + e] = narrow<WT>(vcur[e]);
      }
    }
  }
  __syncthreads();

  float* part = a.partial + (((long long)b * a.kh + s) * a.n_chunks + c) * (DH + 2);
  for (int e = tid; e < DH; e += kAttnBlock) {
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < KPP; ++r) v += s_o[r][e];
    part[2 + e] = v;
  }
  if (tid == 0) {
    float lt = 0.f;
#pragma unroll
    for (int r = 0; r < KPP; ++r) lt += s_l[r];
    part[0] = m;
    part[1] = lt;
  }

}

// Combine the chunk partials of one (batch row, selected head):
// o = sum_c o_c 2^(m_c - M) / sum_c l_c 2^(m_c - M) with M = max m_c (scores in the log2
// domain), in chunk order (deterministic). The partials are staged in LDS with coalesced
// sweeps of kAttnStage chunks, every load of a sweep issued before any is stored; the attention
// plan keeps a head's chunks within one sweep where it can. Over several sweeps the sums are
// kept relative to the running maximum and rescaled when a later sweep raises it, so every
// partial is loaded once.
template <int DH>
__device__ __forceinline__ void attn_combine_block(const AttnArgs& a, int s, int b) {
  __shared__ float s_part[kAttnStage * (DH + 2)];
  const int tid = threadIdx.x;
  const float* base = a.partial + ((long long)b * a.kh + s) * a.n_chunks * (DH + 2);
  float* o = a.o + ((long long)b * a.kh + s) * DH;
  const int e = tid;
  float M = -INFINITY, L = 0.f, O = 0.f;
  constexpr int QMAX = (kAttnStage * (DH + 2) + kAttnBlock - 1) / kAttnBlock;
  for (int c0 = 0; c0 < a.n_chunks; c0 += kAttnStage) {   // block-uniform
    const int nb = min(kAttnStage, a.n_chunks - c0);
    const int n = nb * (DH + 2);
    const float* src = base + (long long)c0 * (DH + 2);
    float v[QMAX];
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      const int i = tid + q * kAttnBlock;
      v[q] = i < n ? src[i] : 0.f;
    }
    __syncthreads();   // the previous sweep's readers are done
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      const int i = tid + q * kAttnBlock;
      if (i < n) s_part[i] = v[q];
    }
    __syncthreads();
    float Ms = M;
    for (int cc = 0; cc < nb; ++cc) Ms = fmaxf(Ms, s_part[cc * (DH + 2)]);
    if (e < DH && Ms > -INFINITY) {
      if (M > -INFINITY && Ms > M) {   // a later sweep raised the maximum: rescale the sums
        const float r = exp2f(M - Ms);
        L *= r;
        O *= r;
      }
      for (int cc = 0; cc < nb; ++cc) {
        const float mc = s_part[cc * (DH + 2)];
        const float f = (mc > -INFINITY) ? exp2f(mc - Ms) : 0.f;
        L = fmaf(s_part[cc * (DH + 2) + 1], f, L);
        O = fmaf(s_part[cc * (DH + 2) + 2 + e], f, O);
      }
    }
    M = Ms;
  }
  if (e < DH) o[e] = (L > 0.f) ? O / L : 0.f;
}

}  // namespace dv
