// Internal launch interface between the C ABI (dv_api.hip) and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dejavu_hip.h"

namespace dv {

// Host side: sets the thread's dv_last_error() text and returns s.
dv_status record_error(dv_status s, const char* msg);

// ---------------------------------------------------------------------------
// Gather row-dot ("GEMV1"): out[b][i] = act(dot(W[row_b(i)], xhat_b) + bias[row_b(i)])
//   row_b(i) = grp * G + (i % G), grp = idx ? idx[b*idx_bstride + i/G] : i/G.
//   xhat_b = norm_g ? norm_g * x_b / sqrt(mean(x_b^2) + eps) : x_b.
// A group id outside [0, n_groups) yields 0 and is never dereferenced.
// ---------------------------------------------------------------------------
struct RowDotSeg {
  const void* W;
  long long ld;             // row stride (elements)
  int n_out;                // outputs per batch row
  int G;                    // consecutive rows per selected group
  int n_groups;
  const int32_t* idx;       // nullable -> identity
  long long idx_bstride;
  const float* x;           // [B][ldx]
  long long ldx;
  const float* norm_g;      // nullable -> no norm
  const float* bias;        // nullable
  float* out;               // [B][ldo]
  long long ldo;
  int relu;
  int blocks;               // blocks (grid.x) given to this segment
};

constexpr int kRowdotMaxSeg = 3;
struct RowDotArgs {
  RowDotSeg seg[kRowdotMaxSeg];   // independent row sets sharing the row length d
  int nseg;
  int d;                    // row length (elements), shared by both segments
  float eps;
};

// Chooses the tiling for row length d (elements) and storage type; returns false if d is
// not supported. rows_in_flight: rows one block keeps loading at once.
bool rowdot_plan(int d, bool f16, int* tpr, int* ch);
// Rows per row-slot so that all segments together fill the chip once; blocks of a segment
// with n_out rows at that depth.
int rowdot_rows_per_slot(long long total_rows, int tpr, int ch, int cus);
int rowdot_blocks_for(int n_out, int tpr, int per_slot);
hipError_t launch_rowdot(const RowDotArgs& a, bool f16, int B, hipStream_t s, int tag,
                         hipEvent_t ev_begin = nullptr, hipEvent_t ev_end = nullptr);

// ---------------------------------------------------------------------------
// Gather row-axpy ("GEMV2"): out[b][c] = sum_i coef[b][i] * W[row_b(i)][c] + bias[c] + resid[b][c]
//   Column slices x row groups write fp32 partials; a second kernel sums them in group
//   order (no in-kernel cross-block communication).
// ---------------------------------------------------------------------------
struct RowAxpyArgs {
  const void* W;
  long long ld;
  int d;
  int n_rows;               // rows per batch row
  int G;
  int n_groups;
  const int32_t* idx;
  long long idx_bstride;
  const float* coef;        // [B][ldc]
  long long ldc;
  const float* bias;        // [d] nullable
  const float* resid;       // [B][ldr] nullable
  long long ldr;
  float* out;               // [B][ldo]
  long long ldo;
  float* partial;           // [B][RG][d] (used when RG > 1)
  int RG;
  int n_slices;
};

void rowaxpy_plan(int d, int n_rows, bool f16, int B, int cus, int* tpc, int* n_slices, int* RG);
int rowaxpy_max_rg();
hipError_t launch_rowaxpy(const RowAxpyArgs& a, bool f16, int tpc, int B, hipStream_t s);

// ---------------------------------------------------------------------------
// Head-sparse decode attention: split-T partials, then a combine kernel.
// ---------------------------------------------------------------------------
struct AttnArgs {
  const float* qkv;         // [B][kh][3][dh] fp32 (q, k, v of each selected head)
  const int32_t* heads;     // [B][kh]
  int kh;
  int n_heads;
  int dh;
  int t_past;               // past length of every row; with t_rows: the largest allowed
  const int32_t* t_rows;    // [B] per-row past lengths on the device, or null
  int t_max;
  void* k_cache;            // [B][H][t_max][dh]
  void* v_cache;
  int chunk;                // keys per block
  int n_chunks;
  float* partial;           // [B][kh][n_chunks][dh + 2]: (m, l, o[dh]) per chunk
  float* o;                 // [B][kh][dh]
};
bool attn_plan(int dh, bool f16, int t_total, int kh, int B, int cus, int* chunk, int* n_chunks);
hipError_t launch_attn(const AttnArgs& a, bool f16, int B, hipStream_t s);
// t[b] = min(t[b] + 1, cap) for b < B (per-row lengths after a decode step).
hipError_t launch_advance_lengths(int32_t* t, int B, int cap, hipStream_t s);

// The row-axpy's column-slice partials only (launch_axpy_reduce finishes them when RG > 1).
hipError_t launch_rowaxpy_part(const RowAxpyArgs& a, bool f16, int tpc, int B, hipStream_t s);


// ---------------------------------------------------------------------------
// Exact top-k by radix select over many CUs (three kernels, see k_topk.hip).
// ---------------------------------------------------------------------------
constexpr int kTopkChunk = 4096;     // scores per chunk block
constexpr int kTopkMaxChunks = 16;   // n <= 65536
struct TopkWs {                      // per problem, rows b = 0..B-1 (caller workspace)
  unsigned* part;                    // [B][chunks][2048] chunk histograms of bits 31..21
  unsigned* bits;                    // [B][chunks * 128] bitmap of selected positions
  unsigned* ckey;                    // [B][chunks][4096] candidate keys of the threshold bin
  unsigned* cidx;                    // [B][chunks][4096] their positions
  unsigned* ccnt;                    // [B][chunks] candidates per chunk
  unsigned* sel;                     // [B][4] threshold bin, keys above it, keys in it
};
struct TopkProb {
  const float* scores;      // [B][n]
  int n;
  int k;
  int32_t* out;             // [B][k]
  TopkWs ws;
};
struct TopkArgs {
  TopkProb p[2];
  int nprob;
};
size_t topk_ws_bytes(int B, int n);              // scratch of one problem
TopkWs topk_ws_carve(void* base, int B, int n);  // base: 256-byte aligned, topk_ws_bytes long
hipError_t launch_topk(const TopkArgs& a, int B, hipStream_t s);

// ---------------------------------------------------------------------------
// Batched decode on the union of the rows' selections (k_batched.hip).
// ---------------------------------------------------------------------------
constexpr int kUnionMaxN = 65536;    // groups (neurons or heads) per problem
constexpr int kBatchMax = 32;        // rows per batched launch
constexpr int kBatchMaxRG = 32;      // row groups of the down-projection
constexpr int kUnionWpb = 64;        // bitmap words per block of the union's OR and list
struct UnionProb {
  const int32_t* idx;       // [B][idx_bstride]: the row's k selected groups (ascending)
  long long idx_bstride;
  int n;                    // groups
  int k;                    // selected per row
  unsigned* bits;           // [B + 1][ceil(n/32)]: row bitmaps, then their OR
  int32_t* list;            // [n]: the OR as an ascending list
  int* count;               // its length
  unsigned* bcnt;           // [kUnionMaxN / 32 / kUnionWpb] scratch: set bits per block of words
};
struct UnionArgs {
  UnionProb p[2];
  int nprob;
  int B;
};
hipError_t launch_union(const UnionArgs& a, hipStream_t s);
hipError_t launch_rows_norm_f16(const float* x, long long ldx, const float* g, int d, float eps, int B, _Float16* out,
                                _Float16* out_lo, long long ldo, hipStream_t s);

constexpr int kGemmOutF16 = 0;       // outh[b][i], fp16, 0 where the row does not select the group
constexpr int kGemmOutQkv = 1;       // outf[b][slot][G], only groups the row selects (slot = rank)
constexpr int kGemmOutF32 = 2;       // outf[b][i], fp32, 0 where the row does not select the group
struct GemmRowsArgs {                // out[b][i] = act(W[row_i] . X[b] + bias[row_i]), MFMA
  const void* W;                     // fp16 rows [n_groups * G][ld]
  long long ld;
  int d;                             // row length (multiple of 8)
  const int32_t* sel;                // selected groups (ascending; nullable = all)
  const int* n_groups_sel;           // device count of sel (nullable = n_groups)
  int G;
  int n_groups;
  int B;
  const _Float16* X;                 // [B][ldx]
  const _Float16* X_lo;              // nullable: rounding remainders of X (same layout)
  const float* Xf;                   // nullable: fp32 activations [B][ldx] instead of X and X_lo, split
                                     //   into an fp16 part and its fp16 remainder as they are staged
  long long ldx;
  const float* bias;                 // nullable
  int relu;
  const unsigned* rowbits;           // [B][bits_words] (nullable = every row selects every group)
  int bits_words;
  int mode;
  _Float16* outh;
  _Float16* outh_lo;                 // nullable: remainders of outh (kGemmOutF16)
  float* outf;
  long long ldo;
  int kh;                            // slots per row (kGemmOutQkv)
  float* kpart;                      // nullable: [kRowsMaxSplit][B][kld] partial sums when K is split over blocks
  long long kld;
  int ksplit;                        // set by the launcher
  const void* W_b;                   // nullable: rows i >= n_rows_a are row i - n_rows_a of W_b (same ld;
  int n_rows_a;                      //   G = 1 and no sel), so two matrices share a launch
  const _Float16* X_b;               // nullable: activations (and X_lo_b remainders) of W_b's rows; then
  const _Float16* X_lo_b;            //   n_rows_a is a multiple of 64, so a block's rows use one input
  float* outf_b;                     // nullable (kGemmOutF32): outputs of W_b's rows, [B][ldo_b]
  long long ldo_b;
  int dyn_slots;                     // set by the launcher: > 0 when the K split follows the device-side row
                                     //   count (ks = dyn_slots / tiles, at most ksplit)
};
constexpr int kRowsMaxSplit = 32;       // K slices of a short up-projection
constexpr int kRowsSplitMaxRows = 4096; // only launches of at most this many rows split K
hipError_t launch_gemm_rows(const GemmRowsArgs& a, int max_rows, int cus, hipStream_t s);

struct GemmColsArgs {                // partial[b][rg][c] = sum_k C[b][k] W[row_k][c], MFMA
  const void* W;                     // fp16 rows [n_groups * G][ld]
  long long ld;
  int d;                             // output columns (multiple of 8)
  const int32_t* sel;
  const int* n_groups_sel;
  int G;
  int n_groups;
  int B;
  const _Float16* C;                 // [B][ldc] coefficients in the union's row order
  long long ldc;
  float* partial;                    // [B][RG][d]
  int RG;
};
int gemm_cols_rg(int d, int max_rows, int B, int cus);
hipError_t launch_gemm_cols(const GemmColsArgs& a, hipStream_t s);
hipError_t launch_heads_to_union(const float* o, int kh, int dh, const int32_t* uh, const int* n_uh, const unsigned* hbits,
                                 int hwords, int B, int max_uh, _Float16* C, long long ldc, hipStream_t s);
// out[b][c] = sum_rg partial[b][rg][c] (group order) + bias[c] + resid[b][c]
hipError_t launch_axpy_reduce(const RowAxpyArgs& a, int B, hipStream_t s);

// Index-list validation (k_check.hip): status[b] = OR of the flags row b's list breaks.
constexpr int kIdxRange = 1;       // an entry outside [0, n)
constexpr int kIdxOrder = 2;       // an entry smaller than its predecessor
constexpr int kIdxDuplicate = 4;   // an entry equal to its predecessor
hipError_t launch_check_indices(const int32_t* idx, int B, int k, int n, int32_t* status, hipStream_t s);

// Blocked-channel scores (k_blocked.hip): out[b][j] = max of scores[b][j*bs .. j*bs+bs-1].
hipError_t launch_block_scores(const float* scores, int B, int n, int bs, float* out, hipStream_t s);

// Predictor training (k_train.hip).
hipError_t launch_iota_rows(int32_t* out, int rows, int n, hipStream_t s);   // out[b][i] = i
hipError_t launch_head_norm(const float* o, int BH, int dh, float* norm, hipStream_t s);
hipError_t launch_fire(const float* a, long long n, uint8_t* fire, hipStream_t s);   // fire = a > 0

// C [M][N] = op(A) op(B) in fp32, A(i,k) = A[i*sai + k*sak], B(k,j) = B[k*sbk + j*sbj].
struct GemmF32Args {
  const float* A;
  long long sai, sak;
  const float* B;
  long long sbk, sbj;
  float* C;
  int M, N, K;
  // Optional cross-entropy epilogue (one K slice only): with bce_y set, C receives
  // (sigmoid(S) - y) * inv_n instead of S, and block b adds its loss terms
  // softplus(s) - y*s in a fixed order into bce_part[b].
  const uint8_t* bce_y;
  float* bce_part;
  float inv_n;
};
constexpr int kGemmMaxSlices = 32;
int gemm_f32_slices(int M, int N, int K, int cus);   // K slices that fill `cus` compute units
// With slices > 1, scratch holds slices * M * N floats (partial products summed in slice order).
hipError_t launch_gemm_f32(GemmF32Args a, int slices, float* scratch, hipStream_t s);
// Blocks of the cross-entropy epilogue of an M x N product (the size of its bce_part array).
int gemm_f32_blocks(int M, int N);
// *loss = inv_n * (sum of part[0..n_part) in a fixed order).
hipError_t launch_loss_finish(const float* part, int n_part, float inv_n, float* loss, hipStream_t s);
hipError_t launch_momentum_step(float* p1, float* v1, const float* g1, long long n1, float* p2, float* v2,
                                const float* g2, long long n2, float lr, float mu, hipStream_t s);

}  // namespace dv
