// Head-sparse decode attention (DejaVu Guide, "Head-Pruned Attention Dispatch").
//
// Only the selected heads are visited: a block handles one (batch row, selected head,
// chunk of key positions). Positions 0..t_past-1 come from the head's cache region
// [t_max][dh] (head-major, so a selected head reads one contiguous span); position t_past
// is the current token, whose k and v come from the fp32 projection and are appended to
// the cache (rounded to the storage type) by the block that owns that position.
//
// Rows may have their own past lengths (a device array read by every block, clamped to
// [0, bound]); chunks past a row's length see no valid key and leave an empty partial
// (m = -inf, l = 0) that the combine weighs with zero.
//
// Per block: scores s_t = q.K_t / sqrt(dh) with TPK = dh/VEC threads per key (a 16-byte
// chunk each, summed by an xor butterfly), the chunk maximum m, p_t = exp(s_t - m), the
// unnormalised p.V in fp32 and l = sum p. Partials (m, l, o) go to the workspace and a
// second kernel rescales and sums them in chunk order:
// o_h = sum_c o_c e^(m_c - M) / sum_c l_c e^(m_c - M). Deterministic; no block waits on
// another inside a kernel.
#include "dv_device.h"
#include "dv_kernels.h"

namespace dv {

constexpr int kAttnBlock = 256;
constexpr int kAttnStage = 40;  // chunk partials staged in LDS per sweep of the combine

template <typename WT, int DH, int NPASS>
__global__ __launch_bounds__(kAttnBlock) void attn_kernel(AttnArgs a) {
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
  const int c = blockIdx.x;
  const int s = blockIdx.y;
  const int b = blockIdx.z;
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

// Combine the chunk partials of one (batch row, selected head): M = max m_c,
// o = sum_c o_c e^(m_c - M) / sum_c l_c e^(m_c - M), in chunk order (deterministic). The
// partials are staged in LDS with coalesced sweeps.
template <int DH>
__global__ __launch_bounds__(kAttnBlock) void attn_combine_kernel(AttnArgs a) {
  __shared__ float s_part[kAttnStage * (DH + 2)];
  const int tid = threadIdx.x;
  const int s = blockIdx.x;
  const int b = blockIdx.y;
  const float* base = a.partial + ((long long)b * a.kh + s) * a.n_chunks * (DH + 2);
  float* o = a.o + ((long long)b * a.kh + s) * DH;
  const int e = tid;
  float M = -INFINITY, L = 0.f, O = 0.f;
  const bool one_sweep = a.n_chunks <= kAttnStage;
  // all loads of a sweep are issued before any is stored
  constexpr int QMAX = (kAttnStage * (DH + 2) + kAttnBlock - 1) / kAttnBlock;
  auto stage = [&](int c0, int nb) {
    const int n = nb * (DH + 2);
    const float* src = base + (long long)c0 * (DH + 2);
    float v[QMAX];
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      const int i = tid + q * kAttnBlock;
      v[q] = i < n ? src[i] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      const int i = tid + q * kAttnBlock;
      if (i < n) s_part[i] = v[q];
    }
    __syncthreads();
  };
  for (int c0 = 0; c0 < a.n_chunks; c0 += kAttnStage) {
    const int nb = min(kAttnStage, a.n_chunks - c0);
    stage(c0, nb);
    for (int cc = 0; cc < nb; ++cc) M = fmaxf(M, s_part[cc * (DH + 2)]);
    if (one_sweep) break;
  }
  for (int c0 = 0; c0 < a.n_chunks; c0 += kAttnStage) {
    const int nb = min(kAttnStage, a.n_chunks - c0);
    if (!one_sweep) stage(c0, nb);
    if (e < DH && M > -INFINITY) {
      for (int cc = 0; cc < nb; ++cc) {
        const float mc = s_part[cc * (DH + 2)];
        const float f = (mc > -INFINITY) ? exp2f(mc - M) : 0.f;
        L = fmaf(s_part[cc * (DH + 2) + 1], f, L);
        O = fmaf(s_part[cc * (DH + 2) + 2 + e], f, O);
      }
    }
  }
  if (e < DH) o[e] = (L > 0.f) ? O / L : 0.f;
}

bool attn_plan(int dh, bool f16, int t_total, int kh, int B, int cus, int* chunk, int* n_chunks) {
  const int vec = f16 ? 8 : 4;
  if (dh != 64 && dh != 128) return false;
  const int tpk = dh / vec;
  const int kpp = kAttnBlock / tpk;
  const long long want = 2LL * cus;
  int npass = 2;
  for (int np : {8, 4}) {
    const long long nc = (t_total + kpp * np - 1) / (kpp * np);
    if (nc * kh * B >= want) { npass = np; break; }
  }
  *chunk = kpp * npass;
  *n_chunks = (t_total + *chunk - 1) / *chunk;
  return true;
}

template <typename WT, int DH>
static hipError_t launch_dh(const AttnArgs& a, int B, hipStream_t s) {
  constexpr int VEC = Vec<WT>::N;
  constexpr int KPP = kAttnBlock / (DH / VEC);
  dim3 grid(a.n_chunks, a.kh, B);
  switch (a.chunk / KPP) {
    case 2: hipLaunchKernelGGL((attn_kernel<WT, DH, 2>), grid, dim3(kAttnBlock), 0, s, a); break;
    case 4: hipLaunchKernelGGL((attn_kernel<WT, DH, 4>), grid, dim3(kAttnBlock), 0, s, a); break;
    case 8: hipLaunchKernelGGL((attn_kernel<WT, DH, 8>), grid, dim3(kAttnBlock), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_combine_kernel<DH>), dim3(a.kh, B), dim3(kAttnBlock), 0, s, a);
  return hipGetLastError();
}

__global__ void advance_lengths_kernel(int32_t* t, int B, int cap) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) t[b] = min(t[b] + 1, cap);
}

hipError_t launch_advance_lengths(int32_t* t, int B, int cap, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(advance_lengths_kernel, dim3((B + 63) / 64), dim3(64), 0, s, t, B, cap);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, bool f16, int B, hipStream_t s) {
  if (a.kh == 0) return hipSuccess;
  if (f16) return a.dh == 128 ? launch_dh<half_t, 128>(a, B, s) : launch_dh<half_t, 64>(a, B, s);
  return a.dh == 128 ? launch_dh<float, 128>(a, B, s) : launch_dh<float, 64>(a, B, s);
}

}  // namespace dv
