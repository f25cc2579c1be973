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
#include "attn_body.h"

namespace dv {

template <typename WT, int DH, int NPASS>
__global__ __launch_bounds__(kAttnBlock) void attn_kernel(AttnArgs a) {
  attn_block<WT, DH, NPASS>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

template <int DH>
__global__ __launch_bounds__(kAttnBlock) void attn_combine_kernel(AttnArgs a) {
  attn_combine_block<DH>(a, blockIdx.x, blockIdx.y);
}

// Keys per block: the longest chunk (fewest partials) that still gives about two blocks per CU,
// among chunkings whose partials fit one combine sweep; when none gives that many blocks, the
// shortest chunk that fits one sweep (a latency-bound launch gains little from more blocks,
// and a second sweep costs the combine a dependent round); when none fits, the longest chunk.
bool attn_plan(int dh, bool f16, int t_total, int kh, int B, int cus, int* chunk, int* n_chunks) {
  const int vec = f16 ? 8 : 4;
  if (dh != 64 && dh != 128) return false;
  const int tpk = dh / vec;
  const int kpp = kAttnBlock / tpk;
  const long long want = 2LL * cus;
  auto nc_of = [&](int np) { return (t_total + kpp * np - 1) / (kpp * np); };
  int npass = 0;
  for (int np : {8, 4, 2})
    if ((long long)nc_of(np) * kh * B >= want && nc_of(np) <= kAttnStage) { npass = np; break; }
  if (npass == 0)
    for (int np : {2, 4, 8})
      if (nc_of(np) <= kAttnStage) { npass = np; break; }
  if (npass == 0) npass = 8;
  *chunk = kpp * npass;
  *n_chunks = nc_of(npass);
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
