// C ABI of the sparse decoder-layer step: argument validation, workspace layout and the
// launch sequence of each call. See include/dejavu_hip.h for the contract.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "dejavu_hip.h"
#include "dv_kernels.h"

namespace {

thread_local std::string g_err;

dv_status fail(dv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

}  // namespace

// Records the detail of a failed call for dv_last_error() (other sources of the library).
dv_status dv::record_error(dv_status s, const char* msg) { return fail(s, "%s", msg); }

namespace {

#define DV_HIP(call)                                                                      \
  do {                                                                                    \
    hipError_t e_ = (call);                                                               \
    if (e_ != hipSuccess) return fail(DV_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

#define DV_TRY(expr)                 \
  do {                               \
    dv_status s_ = (expr);           \
    if (s_ != DV_OK) return s_;      \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t align256(size_t x) { return (x + 255u) & ~size_t(255u); }

// Compute units of the current device (queried on every call: the library keeps no cache).
struct DeviceInfo {
  int cus = 0;
};

dv_status device_info(DeviceInfo* out) {
  int dev = 0;
  DV_HIP(hipGetDevice(&dev));
  int n = 0;
  DV_HIP(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev));
  out->cus = n > 0 ? n : 1;
  return DV_OK;
}

// The fork/join events of one stack call: created by the call and destroyed when it returns
// (a recorded event may be destroyed before the work it marks has run; waits already queued on
// it, or captured into a graph, are unaffected), so calls from different host threads never
// share an event and nothing outlives the call.
struct StackEvents {
  hipEvent_t in = nullptr, sel[2] = {nullptr, nullptr};
  ~StackEvents() {
    for (hipEvent_t e : {in, sel[0], sel[1]})
      if (e != nullptr) (void)hipEventDestroy(e);
  }
  dv_status create() {
    DV_HIP(hipEventCreateWithFlags(&in, hipEventDisableTiming));
    DV_HIP(hipEventCreateWithFlags(&sel[0], hipEventDisableTiming));
    DV_HIP(hipEventCreateWithFlags(&sel[1], hipEventDisableTiming));
    return DV_OK;
  }
};

bool is_f16(const dv_dims* d) { return d->dtype == DV_F16; }
int vec_of(const dv_dims* d) { return is_f16(d) ? 8 : 4; }

dv_status check_dims(const dv_dims* d) {
  if (d == nullptr) return fail(DV_ERR_NULL, "dims is NULL");
  if (d->dtype != DV_F32 && d->dtype != DV_F16) return fail(DV_ERR_DTYPE, "unknown dtype %d", d->dtype);
  if (d->d_model <= 0 || d->d_ffn <= 0 || d->n_heads <= 0 || d->head_dim <= 0 || d->rank_mlp <= 0 ||
      d->rank_head <= 0 || d->t_max <= 0)
    return fail(DV_ERR_DIMS, "all dims must be positive");
  if ((long long)d->n_heads * d->head_dim != d->d_model)
    return fail(DV_ERR_DIMS, "d_model %d != n_heads %d * head_dim %d", d->d_model, d->n_heads, d->head_dim);
  const int v = vec_of(d);
  if (d->d_model % v || d->rank_mlp % v || d->rank_head % v)
    return fail(DV_ERR_ALIGN, "d_model and ranks must be multiples of %d", v);
  if (d->head_dim != 64 && d->head_dim != 128) return fail(DV_ERR_DIMS, "head_dim must be 64 or 128");
  int t, c;
  if (!dv::rowdot_plan(d->d_model, is_f16(d), &t, &c)) return fail(DV_ERR_DIMS, "d_model %d unsupported", d->d_model);
  if (!dv::rowdot_plan(d->rank_mlp, is_f16(d), &t, &c) || !dv::rowdot_plan(d->rank_head, is_f16(d), &t, &c))
    return fail(DV_ERR_DIMS, "predictor rank unsupported");
  if (d->d_ffn > 65536 || d->n_heads > 65536) return fail(DV_ERR_DIMS, "d_ffn and n_heads must be <= 65536");
  return DV_OK;
}

dv_status check_k(const dv_dims* d, int B, int k, int kh) {
  if (B <= 0) return fail(DV_ERR_DIMS, "batch must be positive");
  if (k < 0 || k > d->d_ffn) return fail(DV_ERR_K, "k=%d outside [0, %d]", k, d->d_ffn);
  if (kh < 0 || kh > d->n_heads) return fail(DV_ERR_K, "kh=%d outside [0, %d]", kh, d->n_heads);
  return DV_OK;
}

dv_status check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(DV_ERR_NULL, "%s is NULL", name);
  if (!aligned16(p)) return fail(DV_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return DV_OK;
}

dv_status check_layer(const dv_layer* L, bool attn, bool mlp) {
  if (L == nullptr) return fail(DV_ERR_NULL, "layer is NULL");
  if (attn) {
    DV_TRY(check_ptr(L->wqkv, "wqkv")); DV_TRY(check_ptr(L->bqkv, "bqkv"));
    DV_TRY(check_ptr(L->wo, "wo")); DV_TRY(check_ptr(L->bo, "bo"));
  }
  if (mlp) {
    DV_TRY(check_ptr(L->w1t, "w1t")); DV_TRY(check_ptr(L->b1, "b1"));
    DV_TRY(check_ptr(L->w2, "w2")); DV_TRY(check_ptr(L->b2, "b2"));
  }
  return DV_OK;
}

dv_status check_pred(const dv_predictor* P) {
  if (P == nullptr) return fail(DV_ERR_NULL, "predictor is NULL");
  DV_TRY(check_ptr(P->p1_mlp, "p1_mlp")); DV_TRY(check_ptr(P->p2_mlp, "p2_mlp"));
  DV_TRY(check_ptr(P->p1_head, "p1_head")); DV_TRY(check_ptr(P->p2_head, "p2_head"));
  return DV_OK;
}

// ---------------------------------------------------------------------------
// Workspace layout (sized with the largest tiling any device can pick).
// ---------------------------------------------------------------------------
struct Layout {
  size_t z, s_mlp, s_head, idx, heads, qkv, apart, o, h1, u, part, tk_mlp, tk_head, kpart, total;
  // batched path (B >= 2): union bitmaps and lists, fp16 operands
  size_t ubits, hbits, ulist, uhlist, counts, ucnt, xh, zh, zl, cu, co;
  int max_u, max_uh;
  int max_chunks;
};

Layout layout_of(const dv_dims* d, int B, int k, int kh) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
  const size_t f = 4, Bz = (size_t)B;
  const int v = vec_of(d);
  const int tpk = d->head_dim / v;
  const int kpp = 256 / tpk;
  L.max_chunks = (d->t_max + 2 * kpp - 1) / (2 * kpp);
  L.z = take(f * Bz * (d->rank_mlp + d->rank_head));
  L.s_mlp = take(f * Bz * d->d_ffn);
  L.s_head = take(f * Bz * d->n_heads);
  L.idx = take(f * Bz * k);
  L.heads = take(f * Bz * kh);
  L.qkv = take(f * Bz * kh * 3 * d->head_dim);
  L.apart = take(f * Bz * kh * L.max_chunks * (d->head_dim + 2));
  L.o = take(f * Bz * kh * d->head_dim);
  L.h1 = take(f * Bz * d->d_model);
  L.u = take(f * Bz * k);
  L.part = take(f * Bz * dv::rowaxpy_max_rg() * d->d_model);
  L.tk_mlp = take(dv::topk_ws_bytes(B, d->d_ffn));
  L.tk_head = take(dv::topk_ws_bytes(B, d->n_heads));
  if (B >= 2) {
    const size_t fw = (size_t)(d->d_ffn + 31) / 32, hw = (size_t)(d->n_heads + 31) / 32;
    L.max_u = (int)std::min<long long>(d->d_ffn, (long long)B * k);
    L.max_uh = (int)std::min<long long>(d->n_heads, (long long)B * kh);
    L.ubits = take(4 * (Bz + 1) * fw);
    L.hbits = take(4 * (Bz + 1) * hw);
    L.ulist = take(4 * (size_t)d->d_ffn);
    L.uhlist = take(4 * (size_t)d->n_heads);
    L.counts = take(4 * 4);
    L.ucnt = take(4 * 2 * (size_t)(dv::kUnionMaxN / 32 / dv::kUnionWpb));
    L.xh = take(2 * Bz * d->d_model);
    L.zh = take(2 * Bz * (d->rank_mlp + d->rank_head));
    L.zl = take(2 * Bz * (d->rank_mlp + d->rank_head));
    L.cu = take(2 * Bz * (size_t)L.max_u);
    L.co = take(2 * Bz * (size_t)L.max_uh * d->head_dim);
    L.kpart = take(4 * (size_t)dv::kRowsMaxSplit * Bz * dv::kRowsSplitMaxRows);
  }
  L.total = off;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

dv_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return DV_OK;
  if (ws == nullptr) return fail(DV_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(DV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(DV_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", have, need);
  return DV_OK;
}

// ---------------------------------------------------------------------------
// Launch sequences (arguments already validated).
// ---------------------------------------------------------------------------
dv::RowDotSeg seg_of(const void* W, long long ld, int n_out, int G, int n_groups, const int32_t* idx,
                     long long idx_bstride, const float* x, long long ldx, const float* norm_g,
                     const float* bias, float* out, long long ldo, int relu) {
  dv::RowDotSeg s{};
  s.W = W; s.ld = ld; s.n_out = n_out; s.G = G; s.n_groups = n_groups; s.idx = idx;
  s.idx_bstride = idx_bstride; s.x = x; s.ldx = ldx; s.norm_g = norm_g; s.bias = bias;
  s.out = out; s.ldo = ldo; s.relu = relu; s.blocks = 0;
  return s;
}

// Optional timing of the q/k/v projection launches (dv_timing_start / dv_timing_stop).
struct TimingHook {
  std::mutex mu;
  std::vector<hipEvent_t> start, end;
  int cursor = 0;
  bool active = false;
};
TimingHook g_timing;

dv_status run_rowdot(dv::RowDotArgs& a, bool f16, int B, int cus, hipStream_t st, int tag = 0) {
  int tpr = 0, ch = 0;
  if (!dv::rowdot_plan(a.d, f16, &tpr, &ch)) return fail(DV_ERR_DIMS, "row length %d unsupported", a.d);
  if (a.nseg < 1 || a.nseg > dv::kRowdotMaxSeg) return fail(DV_ERR_DIMS, "internal: %d row-dot segments", a.nseg);
  long long total = 0;
  for (int i = 0; i < a.nseg; ++i) total += a.seg[i].n_out;
  const int per_slot = dv::rowdot_rows_per_slot(total, tpr, ch, cus);
  for (int i = 0; i < a.nseg; ++i) a.seg[i].blocks = dv::rowdot_blocks_for(a.seg[i].n_out, tpr, per_slot);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (tag == 1 && g_timing.active) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (g_timing.active && g_timing.cursor < (int)g_timing.start.size()) {
      e0 = g_timing.start[g_timing.cursor];
      e1 = g_timing.end[g_timing.cursor];
      ++g_timing.cursor;
    }
  }
  DV_HIP(dv::launch_rowdot(a, f16, B, st, tag, e0, e1));
  return DV_OK;
}

// Predictor stage 1 as two row-dot segments: z[b] = [P1_mlp; P1_head] . x[b] (no norm).
void predict_stage1_segs(const dv_dims* d, const dv_predictor* P, const float* x, float* z, dv::RowDotSeg* out) {
  const int rm = d->rank_mlp, rh = d->rank_head, D = d->d_model;
  out[0] = seg_of(P->p1_mlp, D, rm, 1, rm, nullptr, 0, x, D, nullptr, nullptr, z, rm + rh, 0);
  out[1] = seg_of(P->p1_head, D, rh, 1, rh, nullptr, 0, x, D, nullptr, nullptr, z + rm, rm + rh, 0);
}

dv_status run_predict_stage2(const dv_dims* d, const dv_predictor* P, int B, float* s_mlp, float* s_head,
                             const float* z, int cus, hipStream_t st);

// The batched path (union of the rows' selections on the matrix cores) serves fp16 weights
// and 3..32 rows; other batches run every row through the single-row kernels.
#ifndef DV_BATCH_MIN
#define DV_BATCH_MIN 3   // measured crossover at OPT-175B shape: below it, rows run one by one faster
#endif
bool batched(const dv_dims* d, int B) { return B >= DV_BATCH_MIN && B <= dv::kBatchMax && is_f16(d); }

dv::GemmRowsArgs rows_args(const void* W, long long ld, int dlen, const int32_t* sel, const int* nsel, int G,
                           int n_groups, int B, const _Float16* X, long long ldx, float* kpart) {
  dv::GemmRowsArgs g{};
  g.kpart = kpart; g.kld = dv::kRowsSplitMaxRows;
  g.W = W; g.ld = ld; g.d = dlen; g.sel = sel; g.n_groups_sel = nsel; g.G = G; g.n_groups = n_groups; g.B = B;
  g.X = X; g.ldx = ldx;
  return g;
}

// Batched predictor: both factors as dense MFMA products over all B rows. The activations
// (x, then z) enter as fp16 high parts plus fp16 remainders, so the scores keep fp32-like
// precision (the fp16 weights are exact).
dv_status run_predict_batched(const dv_dims* d, const dv_predictor* P, const float* x, int B, float* s_mlp,
                              float* s_head, const Layout& L, void* ws, int cus, hipStream_t st) {
  const int rm = d->rank_mlp, rh = d->rank_head, D = d->d_model;
  _Float16* zh = at<_Float16>(ws, L.zh);
  _Float16* zl = at<_Float16>(ws, L.zl);
  // both stage-1 factors in one launch: rows [0, rm) of P1_mlp, then rows of P1_head (z = [z_m; z_h]);
  // x enters in fp32 and is split into an fp16 part and its remainder as it is staged
  dv::GemmRowsArgs a = rows_args(P->p1_mlp, D, D, nullptr, nullptr, 1, rm + rh, B, nullptr, D, at<float>(ws, L.kpart));
  a.W_b = P->p1_head; a.n_rows_a = rm;
  a.Xf = x; a.mode = dv::kGemmOutF16; a.outh = zh; a.outh_lo = zl; a.ldo = rm + rh;
  DV_HIP(dv::launch_gemm_rows(a, rm + rh, cus, st));
  a.W_b = nullptr; a.n_rows_a = 0;
  a = rows_args(P->p2_mlp, rm, rm, nullptr, nullptr, 1, d->d_ffn, B, zh, rm + rh, at<float>(ws, L.kpart));
  a.X_lo = zl; a.mode = dv::kGemmOutF32; a.outf = s_mlp; a.ldo = d->d_ffn;
  if (rm == rh && d->d_ffn % 64 == 0) {
    // the head scores' rows ride in the neuron scores' launch (their own input z_h and output)
    a.n_groups = d->d_ffn + d->n_heads;
    a.W_b = P->p2_head; a.n_rows_a = d->d_ffn; a.X_b = zh + rm; a.X_lo_b = zl + rm;
    a.outf_b = s_head; a.ldo_b = d->n_heads;
    DV_HIP(dv::launch_gemm_rows(a, d->d_ffn + d->n_heads, cus, st));
    return DV_OK;
  }
  DV_HIP(dv::launch_gemm_rows(a, d->d_ffn, cus, st));
  a = rows_args(P->p2_head, rh, rh, nullptr, nullptr, 1, d->n_heads, B, zh + rm, rm + rh, at<float>(ws, L.kpart));
  a.X_lo = zl + rm; a.mode = dv::kGemmOutF32; a.outf = s_head; a.ldo = d->n_heads;
  DV_HIP(dv::launch_gemm_rows(a, d->n_heads, cus, st));
  return DV_OK;
}

dv_status run_predict(const dv_dims* d, const dv_predictor* P, const float* x, int B, float* s_mlp,
                      float* s_head, const Layout& L, void* ws, int cus, hipStream_t st) {
  if (batched(d, B)) return run_predict_batched(d, P, x, B, s_mlp, s_head, L, ws, cus, st);
  float* z = at<float>(ws, L.z);
  const bool f16 = is_f16(d);
  dv::RowDotArgs a{};
  a.nseg = 2; a.d = d->d_model; a.eps = 0.f;
  predict_stage1_segs(d, P, x, z, a.seg);
  DV_TRY(run_rowdot(a, f16, B, cus, st));
  return run_predict_stage2(d, P, B, s_mlp, s_head, z, cus, st);
}

// Predictor stage 2: s_mlp[b] = P2_mlp . z_mlp[b], s_head[b] = P2_head . z_head[b].
dv_status run_predict_stage2(const dv_dims* d, const dv_predictor* P, int B, float* s_mlp, float* s_head,
                             const float* z, int cus, hipStream_t st) {
  const bool f16 = is_f16(d);
  const int rm = d->rank_mlp, rh = d->rank_head;
  dv::RowDotSeg sm = seg_of(P->p2_mlp, rm, d->d_ffn, 1, d->d_ffn, nullptr, 0, z, rm + rh, nullptr, nullptr,
                            s_mlp, d->d_ffn, 0);
  dv::RowDotSeg sh = seg_of(P->p2_head, rh, d->n_heads, 1, d->n_heads, nullptr, 0, z + rm, rm + rh, nullptr,
                            nullptr, s_head, d->n_heads, 0);
  if (rm == rh) {
    dv::RowDotArgs b{};
    b.nseg = 2; b.d = rm; b.seg[0] = sm; b.seg[1] = sh;
    DV_TRY(run_rowdot(b, f16, B, cus, st));
  } else {
    dv::RowDotArgs b{};
    b.nseg = 1; b.d = rm; b.seg[0] = sm;
    DV_TRY(run_rowdot(b, f16, B, cus, st));
    dv::RowDotArgs c{};
    c.nseg = 1; c.d = rh; c.seg[0] = sh;
    DV_TRY(run_rowdot(c, f16, B, cus, st));
  }
  return DV_OK;
}

dv_status run_topk2(const float* s_mlp, int F, int k, int32_t* idx, const float* s_head, int H, int kh,
                    int32_t* heads, int B, void* ws_mlp, void* ws_head, hipStream_t st) {
  dv::TopkArgs t{};
  t.nprob = 2;
  t.p[0] = {s_mlp, F, k, idx, dv::topk_ws_carve(ws_mlp, B, F)};
  t.p[1] = {s_head, H, kh, heads, dv::topk_ws_carve(ws_head, B, H)};
  DV_HIP(dv::launch_topk(t, B, st));
  return DV_OK;
}

// Past KV length: one length t for every row, or per-row lengths on the device (rows) with
// t their largest allowed value.
struct KvLen {
  int t;
  const int32_t* rows;
};

// y = resid + (sum over selected heads of o_h . Wo_h + bo), x normalised with norm_g if given.
dv_status run_attn(const dv_dims* d, const dv_layer* Lw, const float* x, const float* norm_g, int B,
                   const int32_t* heads, int kh, void* kc, void* vc, KvLen kv, float* y,
                   const float* resid, const Layout& L, void* ws, int cus, hipStream_t st,
                   hipEvent_t ev_after_qkv = nullptr, const dv::RowDotSeg* extra = nullptr, int n_extra = 0) {
  const bool f16 = is_f16(d);
  const int D = d->d_model, dh = d->head_dim, H = d->n_heads;
  float* qkv = at<float>(ws, L.qkv);
  float* o = at<float>(ws, L.o);
  // Independent rows of the same length (the next layer's predictor stage 1) ride in the
  // q/k/v launch as further segments.
  dv::RowDotArgs a{};
  a.nseg = 0; a.d = D; a.eps = 1e-5f;
  if (kh > 0)
    a.seg[a.nseg++] = seg_of(Lw->wqkv, D, kh * 3 * dh, 3 * dh, H, heads, kh, x, D, norm_g, Lw->bqkv, qkv,
                             (long long)kh * 3 * dh, 0);
  for (int i = 0; i < n_extra; ++i) a.seg[a.nseg++] = extra[i];
  if (a.nseg > 0) DV_TRY(run_rowdot(a, f16, B, cus, st, /*tag=*/kh > 0 ? 1 : 0));
  if (ev_after_qkv) DV_HIP(hipEventRecord(ev_after_qkv, st));
  if (kh > 0) {
    dv::AttnArgs at_{};
    at_.qkv = qkv; at_.heads = heads; at_.kh = kh; at_.n_heads = H; at_.dh = dh; at_.t_past = kv.t; at_.t_rows = kv.rows;
    at_.t_max = d->t_max; at_.k_cache = kc; at_.v_cache = vc; at_.partial = at<float>(ws, L.apart);
    at_.o = o;
    if (!dv::attn_plan(dh, f16, kv.t + 1, kh, B, cus, &at_.chunk, &at_.n_chunks))
      return fail(DV_ERR_DIMS, "head_dim unsupported");
    if (at_.n_chunks > L.max_chunks) return fail(DV_ERR_DIMS, "internal: attention chunk plan");
    DV_HIP(dv::launch_attn(at_, f16, B, st));
  }
  dv::RowAxpyArgs r{};
  int tpc = 0;
  dv::rowaxpy_plan(D, kh * dh, f16, B, cus, &tpc, &r.n_slices, &r.RG);
  r.W = Lw->wo; r.ld = D; r.d = D; r.n_rows = kh * dh; r.G = dh; r.n_groups = H; r.idx = heads;
  r.idx_bstride = kh; r.coef = o; r.ldc = (long long)kh * dh; r.bias = Lw->bo; r.resid = resid; r.ldr = D;
  r.out = y; r.ldo = D; r.partial = at<float>(ws, L.part);
  DV_HIP(dv::launch_rowaxpy(r, f16, tpc, B, st));
  return DV_OK;
}

// k selected groups of G consecutive neurons each (G = 1: single neurons; G > 1: blocks).
dv_status run_mlp(const dv_dims* d, const dv_layer* Lw, const float* x, const float* norm_g, int B,
                  const int32_t* idx, int k, float* y, const float* resid, const Layout& L, void* ws, int cus,
                  hipStream_t st, int G = 1) {
  const bool f16 = is_f16(d);
  const int D = d->d_model, F = d->d_ffn;
  const int rows = k * G;
  float* u = at<float>(ws, L.u);
  if (k > 0) {
    dv::RowDotArgs a{};
    a.nseg = 1; a.d = D; a.eps = 1e-5f;
    a.seg[0] = seg_of(Lw->w1t, D, rows, G, F / G, idx, k, x, D, norm_g, Lw->b1, u, rows, 1);
    DV_TRY(run_rowdot(a, f16, B, cus, st));
  }
  dv::RowAxpyArgs r{};
  int tpc = 0;
  dv::rowaxpy_plan(D, rows, f16, B, cus, &tpc, &r.n_slices, &r.RG);
  r.W = Lw->w2; r.ld = D; r.d = D; r.n_rows = rows; r.G = G; r.n_groups = F / G; r.idx = idx; r.idx_bstride = k;
  r.coef = u; r.ldc = rows; r.bias = Lw->b2; r.resid = resid; r.ldr = D; r.out = y; r.ldo = D;
  r.partial = at<float>(ws, L.part);
  DV_HIP(dv::launch_rowaxpy(r, f16, tpc, B, st));
  return DV_OK;
}

// Union of the rows' neuron sets (problem 0) and/or head sets (problem 1).
dv_status run_union(const dv_dims* d, int B, const int32_t* idx, int k, const int32_t* heads, int kh, const Layout& L,
                    void* ws, hipStream_t st) {
  dv::UnionArgs u{};
  u.B = B;
  int* counts = at<int>(ws, L.counts);
  unsigned* bcnt = at<unsigned>(ws, L.ucnt);
  constexpr int nb = dv::kUnionMaxN / 32 / dv::kUnionWpb;
  if (idx != nullptr)
    u.p[u.nprob++] = {idx, k, d->d_ffn, k, at<unsigned>(ws, L.ubits), at<int32_t>(ws, L.ulist), counts, bcnt};
  if (heads != nullptr)
    u.p[u.nprob++] = {heads, kh, d->n_heads, kh, at<unsigned>(ws, L.hbits), at<int32_t>(ws, L.uhlist), counts + 1,
                      bcnt + nb};
  if (u.nprob == 0) return DV_OK;
  if (u.nprob == 1) u.p[1] = u.p[0];
  DV_HIP(dv::launch_union(u, st));
  return DV_OK;
}

// Batched head-sparse attention: q/k/v over the union of the rows' heads (MFMA), decode
// attention per (row, selected head), output projection over the union (MFMA) + reduce.
dv_status run_attn_batched(const dv_dims* d, const dv_layer* Lw, const float* x, const float* norm_g, int B,
                           const int32_t* heads, int kh, void* kc, void* vc, KvLen kv, float* y, const float* resid,
                           const Layout& L, void* ws, int cus, hipStream_t st, hipEvent_t ev_after_qkv, bool union_done) {
  const int D = d->d_model, dh = d->head_dim, H = d->n_heads;
  const int hw = (H + 31) / 32;
  const int* counts = at<int>(ws, L.counts);
  float* qkv = at<float>(ws, L.qkv);
  float* o = at<float>(ws, L.o);
  if (kh > 0) {
    if (!union_done) DV_TRY(run_union(d, B, nullptr, 0, heads, kh, L, ws, st));
    _Float16* xh = at<_Float16>(ws, L.xh);
    DV_HIP(dv::launch_rows_norm_f16(x, D, norm_g, D, 1e-5f, B, xh, nullptr, D, st));
    dv::GemmRowsArgs q = rows_args(Lw->wqkv, D, D, at<int32_t>(ws, L.uhlist), counts + 1, 3 * dh, H, B, xh, D,
                                   at<float>(ws, L.kpart));
    q.bias = Lw->bqkv; q.rowbits = at<unsigned>(ws, L.hbits); q.bits_words = hw;
    q.mode = dv::kGemmOutQkv; q.outf = qkv; q.kh = kh;
    DV_HIP(dv::launch_gemm_rows(q, L.max_uh * 3 * dh, cus, st));
  }
  if (ev_after_qkv) DV_HIP(hipEventRecord(ev_after_qkv, st));
  if (kh > 0) {
    dv::AttnArgs at_{};
    at_.qkv = qkv; at_.heads = heads; at_.kh = kh; at_.n_heads = H; at_.dh = dh; at_.t_past = kv.t; at_.t_rows = kv.rows;
    at_.t_max = d->t_max; at_.k_cache = kc; at_.v_cache = vc; at_.partial = at<float>(ws, L.apart);
    at_.o = o;
    if (!dv::attn_plan(dh, true, kv.t + 1, kh, B, cus, &at_.chunk, &at_.n_chunks))
      return fail(DV_ERR_DIMS, "head_dim unsupported");
    if (at_.n_chunks > L.max_chunks) return fail(DV_ERR_DIMS, "internal: attention chunk plan");
    DV_HIP(dv::launch_attn(at_, true, B, st));
    _Float16* co = at<_Float16>(ws, L.co);
    const long long ldc = (long long)L.max_uh * dh;
    DV_HIP(dv::launch_heads_to_union(o, kh, dh, at<int32_t>(ws, L.uhlist), counts + 1, at<unsigned>(ws, L.hbits), hw,
                                     B, L.max_uh, co, ldc, st));
  }
  dv::GemmColsArgs c{};
  c.W = Lw->wo; c.ld = D; c.d = D; c.sel = at<int32_t>(ws, L.uhlist); c.n_groups_sel = counts + 1; c.G = dh;
  c.n_groups = H; c.B = B; c.C = at<_Float16>(ws, L.co); c.ldc = (long long)L.max_uh * dh;
  c.partial = at<float>(ws, L.part); c.RG = dv::gemm_cols_rg(D, std::max(1, L.max_uh * dh), B, cus);
  dv::RowAxpyArgs r{};
  r.d = D; r.partial = c.partial; r.RG = c.RG; r.bias = Lw->bo; r.resid = resid; r.ldr = D; r.out = y; r.ldo = D;
  if (kh > 0) {
    DV_HIP(dv::launch_gemm_cols(c, st));
  } else {
    r.partial = nullptr;   // no heads: bias + residual only
    r.RG = 1;
  }
  DV_HIP(dv::launch_axpy_reduce(r, B, st));
  return DV_OK;
}

// Batched sparse MLP: up-projection over the union of the rows' neurons with per-row ReLU
// outputs (zero where a row does not select the neuron), down-projection over the union.
dv_status run_mlp_batched(const dv_dims* d, const dv_layer* Lw, const float* x, const float* norm_g, int B,
                          const int32_t* idx, int k, float* y, const float* resid, const Layout& L, void* ws, int cus,
                          hipStream_t st, bool union_done) {
  const int D = d->d_model, F = d->d_ffn;
  const int* counts = at<int>(ws, L.counts);
  dv::RowAxpyArgs r{};
  r.d = D; r.partial = at<float>(ws, L.part); r.bias = Lw->b2; r.resid = resid; r.ldr = D; r.out = y; r.ldo = D;
  if (k == 0) {   // no neurons: bias + residual only
    r.partial = nullptr;
    r.RG = 1;
    DV_HIP(dv::launch_axpy_reduce(r, B, st));
    return DV_OK;
  }
  if (!union_done) DV_TRY(run_union(d, B, idx, k, nullptr, 0, L, ws, st));
  _Float16* xh = at<_Float16>(ws, L.xh);
  DV_HIP(dv::launch_rows_norm_f16(x, D, norm_g, D, 1e-5f, B, xh, nullptr, D, st));
  _Float16* cu = at<_Float16>(ws, L.cu);
  dv::GemmRowsArgs a = rows_args(Lw->w1t, D, D, at<int32_t>(ws, L.ulist), counts, 1, F, B, xh, D,
                                 at<float>(ws, L.kpart));
  a.bias = Lw->b1; a.relu = 1; a.rowbits = at<unsigned>(ws, L.ubits); a.bits_words = (F + 31) / 32;
  a.mode = dv::kGemmOutF16; a.outh = cu; a.ldo = L.max_u;
  DV_HIP(dv::launch_gemm_rows(a, L.max_u, cus, st));
  dv::GemmColsArgs c{};
  c.W = Lw->w2; c.ld = D; c.d = D; c.sel = at<int32_t>(ws, L.ulist); c.n_groups_sel = counts; c.G = 1; c.n_groups = F;
  c.B = B; c.C = cu; c.ldc = L.max_u; c.partial = r.partial; c.RG = dv::gemm_cols_rg(D, L.max_u, B, cus);
  r.RG = c.RG;
  DV_HIP(dv::launch_gemm_cols(c, st));
  DV_HIP(dv::launch_axpy_reduce(r, B, st));
  return DV_OK;
}

dv_status run_layer(const dv_dims* d, const dv_layer* Lw, const float* x, int B, const int32_t* idx, int k,
                    const int32_t* heads, int kh, void* kc, void* vc, KvLen kv, float* x_out,
                    const Layout& L, void* ws, int cus, hipStream_t st, hipEvent_t ev_after_qkv = nullptr,
                    const dv::RowDotSeg* extra = nullptr, int n_extra = 0) {
  float* h1 = at<float>(ws, L.h1);
  if (batched(d, B)) {
    if (n_extra != 0) return fail(DV_ERR_DIMS, "internal: fused segments on the batched path");
    DV_TRY(run_union(d, B, k > 0 ? idx : nullptr, k, kh > 0 ? heads : nullptr, kh, L, ws, st));
    DV_TRY(run_attn_batched(d, Lw, x, Lw->g1, B, heads, kh, kc, vc, kv, h1, x, L, ws, cus, st, ev_after_qkv, true));
    return run_mlp_batched(d, Lw, h1, Lw->g2, B, idx, k, x_out, h1, L, ws, cus, st, true);
  }
  DV_TRY(run_attn(d, Lw, x, Lw->g1, B, heads, kh, kc, vc, kv, h1, x, L, ws, cus, st, ev_after_qkv, extra,
                  n_extra));
  DV_TRY(run_mlp(d, Lw, h1, Lw->g2, B, idx, k, x_out, h1, L, ws, cus, st));
  return DV_OK;
}

dv_status check_layer_all(const dv_dims* d, const dv_layer* Lw) {
  DV_TRY(check_layer(Lw, true, true));
  DV_TRY(check_ptr(Lw->g1, "g1"));
  DV_TRY(check_ptr(Lw->g2, "g2"));
  (void)d;
  return DV_OK;
}

dv_status check_kv(const dv_dims* d, void* kc, void* vc, int t_past) {
  DV_TRY(check_ptr(kc, "k_cache"));
  DV_TRY(check_ptr(vc, "v_cache"));
  if (t_past < 0 || t_past + 1 > d->t_max)
    return fail(DV_ERR_KV, "t_past=%d needs t_max >= t_past+1 (t_max=%d)", t_past, d->t_max);
  return DV_OK;
}

}  // namespace

// ===========================================================================
// exported
// ===========================================================================
extern "C" {

const char* dv_status_str(dv_status s) {
  switch (s) {
    case DV_OK: return "ok";
    case DV_ERR_NULL: return "null pointer";
    case DV_ERR_DIMS: return "bad dimensions";
    case DV_ERR_K: return "k out of range";
    case DV_ERR_DTYPE: return "bad dtype";
    case DV_ERR_ALIGN: return "misaligned pointer or row length";
    case DV_ERR_KV: return "kv cache position out of range";
    case DV_ERR_WORKSPACE: return "workspace too small";
    case DV_ERR_HIP: return "hip error";
  }
  return "unknown status";
}

const char* dv_last_error(void) { return g_err.c_str(); }

const char* dv_version(void) { return "dejavu_hip 0.1 gfx950"; }

int32_t dv_timing_start(int32_t n) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (g_timing.active || n <= 0) return -1;
  g_timing.start.assign(n, nullptr);
  g_timing.end.assign(n, nullptr);
  for (int i = 0; i < n; ++i) {
    if (hipEventCreate(&g_timing.start[i]) != hipSuccess || hipEventCreate(&g_timing.end[i]) != hipSuccess) {
      for (auto e : g_timing.start) if (e) (void)hipEventDestroy(e);
      for (auto e : g_timing.end) if (e) (void)hipEventDestroy(e);
      g_timing.start.clear();
      g_timing.end.clear();
      fail(DV_ERR_HIP, "hipEventCreate failed");
      return -1;
    }
  }
  g_timing.cursor = 0;
  g_timing.active = true;
  return n;
}

int32_t dv_timing_stop(float* ms, int32_t n) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (!g_timing.active) return -1;
  const int used = g_timing.cursor;
  int rc = used;
  for (int i = 0; i < used; ++i) {
    float t = -1.f;
    if (hipEventSynchronize(g_timing.end[i]) != hipSuccess ||
        hipEventElapsedTime(&t, g_timing.start[i], g_timing.end[i]) != hipSuccess)
      rc = -1;
    if (ms != nullptr && i < n) ms[i] = t;
  }
  for (auto e : g_timing.start) (void)hipEventDestroy(e);
  for (auto e : g_timing.end) (void)hipEventDestroy(e);
  g_timing.start.clear();
  g_timing.end.clear();
  g_timing.cursor = 0;
  g_timing.active = false;
  return rc;
}

size_t dv_workspace_bytes(const dv_dims* dims, int32_t B, int32_t k, int32_t kh) {
  if (check_dims(dims) != DV_OK || B <= 0 || k < 0 || kh < 0) return 0;
  return layout_of(dims, B, k, kh).total;
}

size_t dv_stack_workspace_bytes(const dv_dims* dims, int32_t B, int32_t k, int32_t kh) {
  if (check_dims(dims) != DV_OK || B <= 0 || k < 0 || kh < 0) return 0;
  const Layout L = layout_of(dims, B, k, kh);
  size_t off = align256(L.total);
  off += align256(L.total);                                     // side-stream layout
  off += 2 * align256(4 * (size_t)B * k) + 2 * align256(4 * (size_t)B * kh);  // set rings
  off += 2 * align256(4 * (size_t)B * dims->d_model);           // residual ping-pong
  return off;
}

dv_status dv_predict(const dv_dims* dims, const dv_predictor* pred, const float* x_pred, int32_t B,
                     float* s_mlp, float* s_head, void* ws, size_t ws_bytes, hipStream_t stream) {
  DV_TRY(check_dims(dims));
  DV_TRY(check_pred(pred));
  if (B <= 0) return fail(DV_ERR_DIMS, "batch must be positive");
  DV_TRY(check_ptr(x_pred, "x_pred"));
  DV_TRY(check_ptr(s_mlp, "s_mlp"));
  DV_TRY(check_ptr(s_head, "s_head"));
  const Layout L = layout_of(dims, B, 0, 0);
  DV_TRY(check_ws(ws, ws_bytes, L.total));
  DeviceInfo dinfo;
  DV_TRY(device_info(&dinfo));
  const DeviceInfo* di = &dinfo;
  return run_predict(dims, pred, x_pred, B, s_mlp, s_head, L, ws, di->cus, stream);
}

size_t dv_topk_workspace_bytes(int32_t B, int32_t n) {
  if (B <= 0 || n <= 0 || n > dv::kTopkMaxChunks * dv::kTopkChunk) return 0;
  return align256(dv::topk_ws_bytes(B, n));
}

dv_status dv_topk(const float* scores, int32_t B, int32_t n, int32_t k, int32_t* idx, void* ws,
                  size_t ws_bytes, hipStream_t stream) {
  if (B <= 0 || n <= 0) return fail(DV_ERR_DIMS, "B and n must be positive");
  if (n > dv::kTopkMaxChunks * dv::kTopkChunk) return fail(DV_ERR_DIMS, "n must be <= 65536");
  if (k < 0 || k > n) return fail(DV_ERR_K, "k=%d outside [0, %d]", k, n);
  if (scores == nullptr) return fail(DV_ERR_NULL, "scores is NULL");
  if (k > 0 && idx == nullptr) return fail(DV_ERR_NULL, "idx is NULL");
  if (k == 0) return DV_OK;
  DV_TRY(check_ws(ws, ws_bytes, dv_topk_workspace_bytes(B, n)));
  dv::TopkArgs t{};
  t.nprob = 1;
  t.p[0] = {scores, n, k, idx, dv::topk_ws_carve(ws, B, n)};
  t.p[1] = t.p[0];
  DV_HIP(dv::launch_topk(t, B, stream));
  return DV_OK;
}

dv_status dv_sparse_mlp(const dv_dims* dims, const dv_layer* layer, const float* xn, int32_t B,
                        const int32_t* idx, int32_t k, float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  DV_TRY(check_dims(dims));
  DV_TRY(check_layer(layer, false, true));
  DV_TRY(check_k(dims, B, k, 0));
  DV_TRY(check_ptr(xn, "xn"));
  DV_TRY(check_ptr(y, "y"));
  if (k > 0 && idx == nullptr) return fail(DV_ERR_NULL, "idx is NULL");
  const Layout L = layout_of(dims, B, k, 0);
  DV_TRY(check_ws(ws, ws_bytes, L.total));
  DeviceInfo dinfo;
  DV_TRY(device_info(&dinfo));
  const DeviceInfo* di = &dinfo;
  if (batched(dims, B)) return run_mlp_batched(dims, layer, xn, nullptr, B, idx, k, y, nullptr, L, ws, di->cus, stream, false);
  return run_mlp(dims, layer, xn, nullptr, B, idx, k, y, nullptr, L, ws, di->cus, stream);
}

dv_status dv_block_scores(const float* scores, int32_t B, int32_t n, int32_t bs, float* out, hipStream_t stream) {
  if (B <= 0 || n <= 0) return fail(DV_ERR_DIMS, "B and n must be positive");
  if (bs < 1 || bs > 4096 || n % bs != 0) return fail(DV_ERR_DIMS, "block size %d must divide n=%d (1..4096)", bs, n);
  if (scores == nullptr || out == nullptr) return fail(DV_ERR_NULL, "scores and out must be given");
  DV_TRY(check_ptr(scores, "scores"));   // read as 16-byte chunks when bs % 4 == 0
  DV_HIP(dv::launch_block_scores(scores, B, n, bs, out, stream));
  return DV_OK;
}

dv_status dv_check_indices(const int32_t* idx, int32_t B, int32_t k, int32_t n, int32_t* status, hipStream_t stream) {
  if (B <= 0 || n <= 0) return fail(DV_ERR_DIMS, "B and n must be positive");
  if (k < 0 || k > n) return fail(DV_ERR_K, "k=%d outside [0, %d]", k, n);
  if (status == nullptr) return fail(DV_ERR_NULL, "status is NULL");
  if (k > 0 && idx == nullptr) return fail(DV_ERR_NULL, "idx is NULL");
  if (reinterpret_cast<uintptr_t>(status) % alignof(int32_t) != 0 ||
      reinterpret_cast<uintptr_t>(idx) % alignof(int32_t) != 0)
    return fail(DV_ERR_ALIGN, "idx and status must be 4-byte aligned");
  DV_HIP(dv::launch_check_indices(idx, B, k, n, status, stream));
  return DV_OK;
}

dv_status dv_sparse_mlp_blocked(const dv_dims* dims, const dv_layer* layer, const float* xn, int32_t B,
                                const int32_t* blocks, int32_t kb, int32_t bs, float* y, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  DV_TRY(check_dims(dims));
  DV_TRY(check_layer(layer, false, true));
  if (bs < 1 || dims->d_ffn % bs != 0) return fail(DV_ERR_DIMS, "block size %d must divide d_ffn=%d", bs, dims->d_ffn);
  if (B <= 0) return fail(DV_ERR_DIMS, "batch must be positive");
  if (kb < 0 || kb > dims->d_ffn / bs) return fail(DV_ERR_K, "kb=%d outside [0, %d]", kb, dims->d_ffn / bs);
  DV_TRY(check_ptr(xn, "xn"));
  DV_TRY(check_ptr(y, "y"));
  if (kb > 0 && blocks == nullptr) return fail(DV_ERR_NULL, "blocks is NULL");
  const Layout L = layout_of(dims, B, kb * bs, 0);
  DV_TRY(check_ws(ws, ws_bytes, L.total));
  DeviceInfo dinfo;
  DV_TRY(device_info(&dinfo));
  const DeviceInfo* di = &dinfo;
  // whole blocks through the single-row gather kernels (rows of a block are contiguous)
  return run_mlp(dims, layer, xn, nullptr, B, blocks, kb, y, nullptr, L, ws, di->cus, stream, bs);
}

dv_status dv_layer_labels(const dv_dims* dims, const dv_layer* layer, const float* x, int32_t B, void* k_cache,
                          void* v_cache, int32_t t_past, uint8_t* fire, float* preact, float* head_norm, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  DV_TRY(check_dims(dims));
  DV_TRY(check_layer_all(dims, layer));
  if (B <= 0) return fail(DV_ERR_DIMS, "batch must be positive");
  DV_TRY(check_ptr(x, "x"));
  DV_TRY(check_kv(dims, k_cache, v_cache, t_past));
  if (fire == nullptr && preact == nullptr && head_norm == nullptr)
    return fail(DV_ERR_NULL, "give at least one of fire, preact, head_norm");
  if (preact != nullptr) DV_TRY(check_ptr(preact, "preact"));
  if (head_norm != nullptr) DV_TRY(check_ptr(head_norm, "head_norm"));
  const int D = dims->d_model, F = dims->d_ffn, H = dims->n_heads;
  const Layout L = layout_of(dims, B, F, H);
  DV_TRY(check_ws(ws, ws_bytes, L.total));
  DeviceInfo dinfo;
  DV_TRY(device_info(&dinfo));
  const DeviceInfo* di = &dinfo;
  // the dense layer's attention block: every head of every row (row-wise kernels)
  int32_t* heads = at<int32_t>(ws, L.heads);
  DV_HIP(dv::launch_iota_rows(heads, B, H, stream));
  float* h1 = at<float>(ws, L.h1);
  DV_TRY(run_attn(dims, layer, x, layer->g1, B, heads, H, k_cache, v_cache, KvLen{t_past, nullptr}, h1, x, L, ws,
                  di->cus, stream));
  if (head_norm) DV_HIP(dv::launch_head_norm(at<float>(ws, L.o), B * H, dims->head_dim, head_norm, stream));
  // up-projection pre-activations of every neuron on RMSNorm(h1) (identity row list, no ReLU)
  if (fire != nullptr || preact != nullptr) {
    float* a = preact ? preact : at<float>(ws, L.u);
    dv::RowDotArgs r{};
    r.nseg = 1; r.d = D; r.eps = 1e-5f;
    r.seg[0] = seg_of(layer->w1t, D, F, 1, F, nullptr, 0, h1, D, layer->g2, layer->b1, a, F, 0);
    DV_TRY(run_rowdot(r, is_f16(dims), B, di->cus, stream));
    if (fire) DV_HIP(dv::launch_fire(a, (long long)B * F, fire, stream));
  }
  return DV_OK;
}

namespace {
struct TrainPlan {
  int ks[5];                 // K slices of the five products
  size_t z, s, dz, g1, g2, scratch, part, total;
};

// The slice plan is fixed (planned for 256 compute units), so a step gives the same bits on
// any device.
TrainPlan train_plan(int M, int d, int N, int r) {
  TrainPlan p{};
  const int outs[5][3] = {{M, r, d}, {M, N, r}, {N, r, M}, {M, r, N}, {r, d, M}};
  size_t scratch = 0;
  for (int i = 0; i < 5; ++i) {
    // the scores product (i = 1) carries the cross-entropy epilogue, which needs whole sums
    p.ks[i] = i == 1 ? 1 : dv::gemm_f32_slices(outs[i][0], outs[i][1], outs[i][2], 256);
    if (p.ks[i] > 1) scratch = std::max(scratch, (size_t)p.ks[i] * outs[i][0] * outs[i][1]);
  }
  size_t off = 0;
  auto take = [&](size_t n) { const size_t o = off; off = align256(off + 4 * n); return o; };
  p.z = take((size_t)M * r);
  p.s = take((size_t)M * N);
  p.dz = take((size_t)M * r);
  p.g1 = take((size_t)r * d);
  p.g2 = take((size_t)N * r);
  p.scratch = take(scratch);
  p.part = take((size_t)dv::gemm_f32_blocks(M, N));
  p.total = off;
  return p;
}
}  // namespace

size_t dv_predictor_train_workspace_bytes(int32_t M, int32_t d, int32_t N, int32_t r) {
  if (M <= 0 || d <= 0 || N <= 0 || r <= 0) return 0;
  return train_plan(M, d, N, r).total;
}

dv_status dv_predictor_train_step(const float* x, int32_t M, int32_t d, const uint8_t* y, int32_t N, int32_t r,
                                  float* p1, float* p2, float* v1, float* v2, float lr, float momentum, float* loss,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
  if (M <= 0 || d <= 0 || N <= 0 || r <= 0) return fail(DV_ERR_DIMS, "M, d, N and r must be positive");
  if (!(lr >= 0.f) || !(momentum >= 0.f) || !std::isfinite(lr) || !std::isfinite(momentum))
    return fail(DV_ERR_DIMS, "lr and momentum must be finite and non-negative");
  DV_TRY(check_ptr(x, "x"));
  DV_TRY(check_ptr(y, "y"));
  DV_TRY(check_ptr(p1, "p1"));
  DV_TRY(check_ptr(p2, "p2"));
  DV_TRY(check_ptr(v1, "v1"));
  DV_TRY(check_ptr(v2, "v2"));
  if (loss == nullptr) return fail(DV_ERR_NULL, "loss is NULL");
  if (reinterpret_cast<uintptr_t>(loss) % alignof(float) != 0) return fail(DV_ERR_ALIGN, "loss is not 4-byte aligned");
  const TrainPlan P = train_plan(M, d, N, r);
  DV_TRY(check_ws(ws, ws_bytes, P.total));
  float* Z = at<float>(ws, P.z);
  float* S = at<float>(ws, P.s);
  float* dZ = at<float>(ws, P.dz);
  float* g1 = at<float>(ws, P.g1);
  float* g2 = at<float>(ws, P.g2);
  float* scr = at<float>(ws, P.scratch);
  // Z = x P1^T  [M][r]
  DV_HIP(dv::launch_gemm_f32({x, d, 1, p1, 1, d, Z, M, r, d}, P.ks[0], scr, stream));
  // S = Z P2^T  [M][N], turned by the epilogue into G = (sigmoid(S) - y) / (M N), with the
  // loss terms summed per block; then the loss
  const float inv_n = 1.f / ((float)M * (float)N);
  dv::GemmF32Args sg{Z, r, 1, p2, 1, r, S, M, N, r};
  sg.bce_y = y;
  sg.bce_part = at<float>(ws, P.part);
  sg.inv_n = inv_n;
  DV_HIP(dv::launch_gemm_f32(sg, P.ks[1], scr, stream));
  DV_HIP(dv::launch_loss_finish(at<float>(ws, P.part), dv::gemm_f32_blocks(M, N), inv_n, loss, stream));
  // dL/dP2 = G^T Z  [N][r]
  DV_HIP(dv::launch_gemm_f32({S, 1, N, Z, r, 1, g2, N, r, M}, P.ks[2], scr, stream));
  // dL/dZ = G P2  [M][r]
  DV_HIP(dv::launch_gemm_f32({S, N, 1, p2, r, 1, dZ, M, r, N}, P.ks[3], scr, stream));
  // dL/dP1 = dZ^T x  [r][d]
  DV_HIP(dv::launch_gemm_f32({dZ, 1, r, x, d, 1, g1, r, d, M}, P.ks[4], scr, stream));
  DV_HIP(dv::launch_momentum_step(p1, v1, g1, (long long)r * d, p2, v2, g2, (long long)N * r, lr, momentum, stream));
  return DV_OK;
}

dv_status dv_sparse_attn(const dv_dims* dims, const dv_layer* layer, const float* xn, int32_t B,
                         const int32_t* heads, int32_t kh, void* k_cache, void* v_cache, int32_t t_past,
                         float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  DV_TRY(check_dims(dims));
  DV_TRY(check_layer(layer, true, false));
  DV_TRY(check_k(dims, B, 0, kh));
  DV_TRY(check_ptr(xn, "xn"));
  DV_TRY(check_ptr(y, "y"));
  DV_TRY(check_kv(dims, k_cache, v_cache, t_past));
  if (kh > 0 && heads == nullptr) return fail(DV_ERR_NULL, "heads is NULL");
  const Layout L = layout_of(dims, B, 0, kh);
  DV_TRY(check_ws(ws, ws_bytes, L.total));
  DeviceInfo dinfo;
  DV_TRY(device_info(&dinfo));
  const DeviceInfo* di = &dinfo;
  if (batched(dims, B))
    return run_attn_batched(dims, layer, xn, nullptr, B, heads, kh, k_cache, v_cache, KvLen{t_past, nullptr}, y, nullptr, L, ws,
                            di->cus, stream, nullptr, false);
  return run_attn(dims, layer, xn, nullptr, B, heads, kh, k_cache, v_cache, KvLen{t_past, nullptr}, y, nullptr, L, ws,
                  di->cus, stream);
}

dv_status dv_layer_step(const dv_dims* dims, const dv_layer* layer, const dv_predictor* pred, const float* x,
                        const float* x_pred, int32_t B, int32_t k, int32_t kh, const int32_t* idx_in,
                        const int32_t* heads_in, void* k_cache, void* v_cache, int32_t t_past, float* x_out,
                        int32_t* idx_out, int32_t* heads_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  DV_TRY(check_dims(dims));
  DV_TRY(check_layer_all(dims, layer));
  DV_TRY(check_k(dims, B, k, kh));
  DV_TRY(check_ptr(x, "x"));
  DV_TRY(check_ptr(x_out, "x_out"));
  DV_TRY(check_kv(dims, k_cache, v_cache, t_past));
  const bool inline_pred = (idx_in == nullptr && heads_in == nullptr);
  if (!inline_pred && (idx_in == nullptr || heads_in == nullptr))
    return fail(DV_ERR_NULL, "give both idx_in and heads_in, or neither");
  if (inline_pred) {
    DV_TRY(check_pred(pred));
    DV_TRY(check_ptr(x_pred, "x_pred"));
  }
  const Layout L = layout_of(dims, B, k, kh);
  DV_TRY(check_ws(ws, ws_bytes, L.total));
  DeviceInfo dinfo;
  DV_TRY(device_info(&dinfo));
  const DeviceInfo* di = &dinfo;
  const int32_t* idx = idx_in;
  const int32_t* heads = heads_in;
  if (inline_pred) {
    int32_t* io = idx_out ? idx_out : at<int32_t>(ws, L.idx);
    int32_t* ho = heads_out ? heads_out : at<int32_t>(ws, L.heads);
    DV_TRY(run_predict(dims, pred, x_pred, B, at<float>(ws, L.s_mlp), at<float>(ws, L.s_head), L, ws, di->cus,
                       stream));
    DV_TRY(run_topk2(at<float>(ws, L.s_mlp), dims->d_ffn, k, io, at<float>(ws, L.s_head), dims->n_heads, kh,
                     ho, B, at<char>(ws, L.tk_mlp), at<char>(ws, L.tk_head), stream));
    idx = io;
    heads = ho;
  } else {
    if (idx_out && k > 0)
      DV_HIP(hipMemcpyAsync(idx_out, idx_in, sizeof(int32_t) * B * k, hipMemcpyDeviceToDevice, stream));
    if (heads_out && kh > 0)
      DV_HIP(hipMemcpyAsync(heads_out, heads_in, sizeof(int32_t) * B * kh, hipMemcpyDeviceToDevice, stream));
  }
  return run_layer(dims, layer, x, B, idx, k, heads, kh, k_cache, v_cache, KvLen{t_past, nullptr}, x_out, L, ws, di->cus,
                   stream);
}

}  // extern "C"

namespace {

// The lookahead stack over KV lengths kv; with advance != null the per-row lengths there
// are advanced by one once every layer has run (on `stream`, after the last attention).
dv_status run_stack(const dv_dims* dims, const dv_layer* layers, const dv_predictor* preds, int32_t n_layers,
                    const float* x, int32_t B, int32_t k, int32_t kh, void* const* k_caches,
                    void* const* v_caches, KvLen kv, int32_t* advance, float* y, float* h_all, int32_t* idx_out,
                    int32_t* heads_out, void* ws, size_t ws_bytes, hipStream_t stream, hipStream_t side_stream) {
  if (layers == nullptr || preds == nullptr || k_caches == nullptr || v_caches == nullptr)
    return fail(DV_ERR_NULL, "layers, preds and cache arrays must be given");
  if (n_layers <= 0) return fail(DV_ERR_DIMS, "n_layers must be positive");
  DV_TRY(check_k(dims, B, k, kh));
  DV_TRY(check_ptr(x, "x"));
  DV_TRY(check_ptr(y, "y"));
  if (h_all != nullptr) DV_TRY(check_ptr(h_all, "h_all"));
  for (int l = 0; l < n_layers; ++l) {
    DV_TRY(check_layer_all(dims, &layers[l]));
    DV_TRY(check_pred(&preds[l]));
    DV_TRY(check_kv(dims, k_caches[l], v_caches[l], kv.t));
  }
  const Layout L = layout_of(dims, B, k, kh);
  const size_t need = dv_stack_workspace_bytes(dims, B, k, kh);
  DV_TRY(check_ws(ws, ws_bytes, need));
  DeviceInfo dinfo;
  DV_TRY(device_info(&dinfo));
  const int cus = dinfo.cus;
  StackEvents ev;
  const int D = dims->d_model;

  // carve: main layout, side layout, set rings, residual ping-pong
  size_t off = align256(L.total);
  void* ws_side = static_cast<char*>(ws) + off;
  off += align256(L.total);
  int32_t* ring_idx[2];
  int32_t* ring_heads[2];
  for (int i = 0; i < 2; ++i) { ring_idx[i] = at<int32_t>(ws, off); off += align256(4 * (size_t)B * k); }
  for (int i = 0; i < 2; ++i) { ring_heads[i] = at<int32_t>(ws, off); off += align256(4 * (size_t)B * kh); }
  float* pp[2];
  for (int i = 0; i < 2; ++i) { pp[i] = at<float>(ws, off); off += align256(4 * (size_t)B * D); }

  const size_t vecb = sizeof(float) * (size_t)B * D;
  auto h_in = [&](int l) -> const float* {
    if (h_all) return h_all + (size_t)l * B * D;
    return l == 0 ? x : pp[l % 2];
  };
  auto h_outp = [&](int l) -> float* {
    if (h_all) return h_all + (size_t)(l + 1) * B * D;
    return l == n_layers - 1 ? y : pp[(l + 1) % 2];
  };
  auto sel_idx = [&](int l) -> int32_t* { return idx_out ? idx_out + (size_t)l * B * k : ring_idx[l % 2]; };
  auto sel_heads = [&](int l) -> int32_t* {
    return heads_out ? heads_out + (size_t)l * B * kh : ring_heads[l % 2];
  };
  auto topk_sets = [&](int l, void* w, hipStream_t st) -> dv_status {
    return run_topk2(at<float>(w, L.s_mlp), dims->d_ffn, k, sel_idx(l), at<float>(w, L.s_head), dims->n_heads,
                     kh, sel_heads(l), B, at<char>(w, L.tk_mlp), at<char>(w, L.tk_head), st);
  };

  const bool two = side_stream != stream;
  hipStream_t st_side = two ? side_stream : stream;
  if (two) DV_TRY(ev.create());
  if (h_all) DV_HIP(hipMemcpyAsync(h_all, x, vecb, hipMemcpyDeviceToDevice, stream));
  // Layer 0's sets come from the stack input, before any layer runs.
  DV_TRY(run_predict(dims, &preds[0], h_in(0), B, at<float>(ws, L.s_mlp), at<float>(ws, L.s_head), L, ws, cus,
                     stream));
  DV_TRY(topk_sets(0, ws, stream));
  for (int l = 0; l < n_layers; ++l) {
    if (two && l >= 1) DV_HIP(hipStreamWaitEvent(stream, ev.sel[l % 2], 0));
    // The sets of layer l+1 are predicted from the input of layer l: predictor stage 1 reads
    // the same vector as layer l's q/k/v projection and rides in that launch; stage 2 and the
    // top-k then run on the side stream while layer l finishes.
    const bool ahead = l + 1 < n_layers;
    const bool fuse = ahead && !batched(dims, B);
    dv::RowDotSeg p1[2];
    if (fuse) predict_stage1_segs(dims, &preds[l + 1], h_in(l), at<float>(ws_side, L.z), p1);
    DV_TRY(run_layer(dims, &layers[l], h_in(l), B, sel_idx(l), k, sel_heads(l), kh, k_caches[l], v_caches[l],
                     kv, h_outp(l), L, ws, cus, stream, (ahead && two) ? ev.in : nullptr,
                     fuse ? p1 : nullptr, fuse ? 2 : 0));
    if (ahead) {
      if (two) DV_HIP(hipStreamWaitEvent(st_side, ev.in, 0));
      // Stage 2 is planned for three quarters of the CUs: it starts together with layer l's
      // attention, and a grid over every CU holds them all while attention waits (measured on
      // the 24-layer OPT-175B-shaped stack: 123.9 against 126.9 us per layer-token).
      if (fuse)
        DV_TRY(run_predict_stage2(dims, &preds[l + 1], B, at<float>(ws_side, L.s_mlp), at<float>(ws_side, L.s_head),
                                  at<float>(ws_side, L.z), two ? std::max(1, cus * 3 / 4) : cus, st_side));
      else
        DV_TRY(run_predict(dims, &preds[l + 1], h_in(l), B, at<float>(ws_side, L.s_mlp), at<float>(ws_side, L.s_head),
                           L, ws_side, cus, st_side));
      DV_TRY(topk_sets(l + 1, ws_side, st_side));
      if (two) DV_HIP(hipEventRecord(ev.sel[(l + 1) % 2], st_side));
    }
  }
  if (advance) DV_HIP(dv::launch_advance_lengths(advance, B, dims->t_max - 1, stream));
  if (h_all && y != h_all + (size_t)n_layers * B * D)
    DV_HIP(hipMemcpyAsync(y, h_all + (size_t)n_layers * B * D, vecb, hipMemcpyDeviceToDevice, stream));
  return DV_OK;
}

}  // namespace

extern "C" {

dv_status dv_lookahead_stack(const dv_dims* dims, const dv_layer* layers, const dv_predictor* preds,
                             int32_t n_layers, const float* x, int32_t B, int32_t k, int32_t kh,
                             void* const* k_caches, void* const* v_caches, int32_t t_past, float* y, float* h_all,
                             int32_t* idx_out, int32_t* heads_out, void* ws, size_t ws_bytes, hipStream_t stream,
                             hipStream_t side_stream) {
  DV_TRY(check_dims(dims));
  return run_stack(dims, layers, preds, n_layers, x, B, k, kh, k_caches, v_caches, KvLen{t_past, nullptr}, nullptr, y,
                   h_all, idx_out, heads_out, ws, ws_bytes, stream, side_stream);
}

dv_status dv_decode_step(const dv_dims* dims, const dv_layer* layers, const dv_predictor* preds, int32_t n_layers,
                         const float* x, int32_t B, int32_t k, int32_t kh, void* const* k_caches,
                         void* const* v_caches, int32_t* t_rows, int32_t advance, float* y, float* h_all,
                         int32_t* idx_out, int32_t* heads_out, void* ws, size_t ws_bytes, hipStream_t stream,
                         hipStream_t side_stream) {
  DV_TRY(check_dims(dims));
  if (t_rows == nullptr) return fail(DV_ERR_NULL, "t_rows is NULL");
  if (reinterpret_cast<uintptr_t>(t_rows) % alignof(int32_t) != 0)
    return fail(DV_ERR_ALIGN, "t_rows is not 4-byte aligned");
  return run_stack(dims, layers, preds, n_layers, x, B, k, kh, k_caches, v_caches, KvLen{dims->t_max - 1, t_rows},
                   advance ? t_rows : nullptr, y, h_all, idx_out, heads_out, ws, ws_bytes, stream, side_stream);
}

}  // extern "C"
