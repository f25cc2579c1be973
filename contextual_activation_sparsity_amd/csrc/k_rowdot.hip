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

#include "rowdot_body.h"

namespace dv {

// TAG only separates launch sites in profiles (1 = head-sparse q/k/v projection).
template <typename WT, int TPR, int CH, int TAG>
__global__ __launch_bounds__(kRowdotBlock) __attribute__((amdgpu_waves_per_eu(DV_ROWDOT_WAVES_PER_EU)))
void rowdot_kernel(RowDotArgs a) {
  rowdot_block<WT, TPR, CH>(a, blockIdx.x, blockIdx.y);
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
