/*
 * dejavu_hip.h -- C ABI of the contextually sparse decoder-layer step on MI355X (gfx950).
 *
 * What the step computes (DejaVu Guide: Contextual Sparsity for LLM Inference):
 *   - "Mathematical Formulation of Lookahead Predictors": per layer, a linear map scores
 *     every MLP neuron and every attention head from an activation available before the
 *     layer runs; the active sets are the top-k of those scores.
 *   - "The Synchronous Prediction Dilemma" and "Step-by-Step Implementation": the MLP
 *     computes act(x W1) W2 over the active neurons only (ReLU here), inside a pre-norm
 *     residual layer.
 *   - "Head-Pruned Attention Dispatch": an inactive head reads none of its q/k/v or
 *     output-projection weights and none of its KV cache.
 *   - "Pipelined Overlap Execution": the prediction for layer l+1 runs on its own stream
 *     while layer l computes.
 * The summary page "Deja Vu: How Contextual Sparsity Accelerates LLM Inference by 6x"
 * ("What Is Contextual Sparsity?") gives the sparsity levels the workloads use.
 *
 * Conventions for every call
 *   - All tensor pointers are DEVICE memory owned by the caller. The library never
 *     allocates or frees device memory. Scratch space is the caller's workspace `ws`
 *     of at least dv_workspace_bytes(...) bytes (256-byte aligned); its contents need no
 *     initialisation and are garbage after the call.
 *   - State the library keeps between calls: the device array that dv_layer_step_noalloc
 *     uses as its workspace (with its per-device address), the thread's dv_last_error()
 *     text, and the q/k/v timing hook while dv_timing_start is active. Nothing else: device
 *     properties are queried per call and the stack's events live for one call.
 *   - Calls are asynchronous on `stream`; outputs are valid once the stream is synchronised
 *     or an event recorded after the call has completed. Two calls that share a workspace
 *     must be ordered (same stream, or an event between them).
 *   - Arguments are validated on the host before anything is launched; a failed check
 *     returns a status and launches nothing. DV_ERR_HIP means a launch failed; the text is
 *     in dv_last_error() (thread-local).
 *   - Weight/KV storage type is dims->dtype (fp32 or fp16); gains and biases are always
 *     fp32; activations, scores and outputs are fp32; accumulation is fp32.
 *   - Weights are stored NEURON-MAJOR so every selected row is one contiguous burst:
 *     w1t[j] is column j of W1, w2[j] is row j of W2, p2_mlp[j] scores neuron j.
 *   - Index lists are int32, ascending, unique and in range (dv_topk produces exactly
 *     that; dv_check_indices checks lists from elsewhere). An out-of-range entry
 *     contributes nothing (it is never dereferenced).
 *   - Row length d_model and both predictor ranks must be multiples of 8 (fp16) or 4
 *     (fp32), every pointer 16-byte aligned (DV_ERR_ALIGN otherwise).
 */
#ifndef DEJAVU_HIP_H
#define DEJAVU_HIP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DV_OK = 0,
  DV_ERR_NULL = 1,       /* a required pointer is NULL */
  DV_ERR_DIMS = 2,       /* non-positive size, d_model != n_heads*head_dim, unsupported shape */
  DV_ERR_K = 3,          /* k outside [0, n] */
  DV_ERR_DTYPE = 4,      /* unknown storage type */
  DV_ERR_ALIGN = 5,      /* pointer not 16-byte aligned or row length not a vector multiple */
  DV_ERR_KV = 6,         /* t_past < 0 or t_past + 1 > t_max */
  DV_ERR_WORKSPACE = 7,  /* workspace NULL/too small/misaligned */
  DV_ERR_HIP = 8         /* a HIP call or launch failed */
} dv_status;

typedef enum { DV_F32 = 0, DV_F16 = 1 } dv_dtype;

/* Shapes of one decoder layer. d_model = n_heads * head_dim. */
typedef struct {
  int32_t d_model, d_ffn, n_heads, head_dim, rank_mlp, rank_head, t_max;
  int32_t dtype; /* dv_dtype: storage type of weights and KV cache */
} dv_dims;

/* Low-rank lookahead predictor of one layer (storage type dims->dtype).
 * Score of neuron j = p2_mlp[j] . (p1_mlp x); score of head h = p2_head[h] . (p1_head x). */
typedef struct {
  const void* p1_mlp;  /* [rank_mlp][d_model]  */
  const void* p2_mlp;  /* [d_ffn][rank_mlp]    */
  const void* p1_head; /* [rank_head][d_model] */
  const void* p2_head; /* [n_heads][rank_head] */
} dv_predictor;

/* Weights of one decoder layer. */
typedef struct {
  const float* g1;   /* [d] RMSNorm gain before attention */
  const float* g2;   /* [d] RMSNorm gain before the MLP */
  const void* wqkv;  /* [H][3][dh][d]: row (h,m,e) gives element e of q (m=0), k (1), v (2) */
  const float* bqkv; /* [H][3][dh] */
  const void* wo;    /* [H][dh][d]: row (h,e) is multiplied by o_h[e] */
  const float* bo;   /* [d] */
  const void* w1t;   /* [F][d]: row j is W1[:, j] */
  const float* b1;   /* [F] */
  const void* w2;    /* [F][d]: row j is W2[j, :] */
  const float* b2;   /* [d] */
} dv_layer;

/* Predictor scores (DejaVu Guide, "Mathematical Formulation of Lookahead Predictors").
 *   x_pred [B][d] fp32 -> s_mlp [B][F], s_head [B][H] fp32. No bias, no activation. */
dv_status dv_predict(const dv_dims* dims, const dv_predictor* pred, const float* x_pred, int32_t B,
                     float* s_mlp, float* s_head, void* ws, size_t ws_bytes, hipStream_t stream);

/* Exact top-k per row (same section; indices sorted as the guide's predictor returns them).
 *   scores [B][n] fp32 -> idx [B][k] int32, ascending. The k largest scores win; equal
 *   scores go to the lower index; -0.0 == +0.0; NaN ranks below -inf. 0 <= k <= n <= 65536.
 *   Workspace: dv_topk_workspace_bytes(B, n) bytes (may be NULL when k == 0). */
dv_status dv_topk(const float* scores, int32_t B, int32_t n, int32_t k, int32_t* idx, void* ws,
                  size_t ws_bytes, hipStream_t stream);

/* Sparse ReLU MLP over the active neurons ("Step-by-Step Implementation", sparse MLP).
 *   xn [B][d] fp32 (already normalised), idx [B][k] ->
 *   y [B][d] = relu(xn . W1[:, S_b] + b1[S_b]) . W2[S_b, :] + b2   (no residual).
 *   k = 0 gives y = b2. */
dv_status dv_sparse_mlp(const dv_dims* dims, const dv_layer* layer, const float* xn, int32_t B,
                        const int32_t* idx, int32_t k, float* y, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Blocked-channel scores ("Blocked Channel Sparsity": contiguous blocks of neurons are
 *   loaded whole when they hold a highly active neuron). scores [B][n] fp32 ->
 *   out [B][n/bs]: the largest member score of each block, NaN counting as lowest (a block of
 *   NaNs scores -inf). 1 <= bs <= 4096 and n % bs == 0; scores 16-byte aligned. Rank blocks
 *   with dv_topk. */
dv_status dv_block_scores(const float* scores, int32_t B, int32_t n, int32_t bs, float* out, hipStream_t stream);

/* Opt-in validation of index lists a caller supplies instead of taking them from dv_topk.
 * Every call that gathers by index (dv_sparse_mlp, dv_sparse_attn, dv_layer_step, the
 * blocked MLP) expects each row's list ascending, without repeats and inside [0, n): the
 * form the predictor hands the sparse forward in DejaVu Guide, "Step-by-Step
 * Implementation" (sorted indices). A list that breaks it gives path-dependent results (a
 * repeated neuron counts twice on the row-wise path and once on the batched union path).
 *   idx [B][k] int32 (device), n the exclusive bound (d_ffn, n_heads or the block count);
 *   status [B] int32 (device) receives, per row, the OR of:
 *     DV_IDX_RANGE     an entry < 0 or >= n,
 *     DV_IDX_ORDER     an entry smaller than the one before it,
 *     DV_IDX_DUPLICATE an entry equal to the one before it;
 *   0 means the row's list is valid. In an ascending list every repeat is adjacent, so a
 *   row with DV_IDX_ORDER clear has DV_IDX_DUPLICATE set exactly when it repeats an entry;
 *   with DV_IDX_ORDER set, repeats that are not adjacent go unreported.
 *   B >= 1, n >= 1, 0 <= k <= n (idx may be NULL when k == 0); idx and status 4-byte
 *   aligned. Asynchronous on `stream`; nothing is read back to the host. */
enum { DV_IDX_RANGE = 1, DV_IDX_ORDER = 2, DV_IDX_DUPLICATE = 4 };
dv_status dv_check_indices(const int32_t* idx, int32_t B, int32_t k, int32_t n, int32_t* status,
                           hipStream_t stream);

/* Sparse ReLU MLP over whole blocks of bs consecutive neurons (same section).
 *   blocks [B][kb]: ascending block ids (block j is neurons j*bs .. j*bs+bs-1); the result
 *   equals dv_sparse_mlp on the expanded neuron list. d_ffn % bs == 0, 0 <= kb <= d_ffn/bs.
 *   Workspace: dv_workspace_bytes(dims, B, kb * bs, 0). */
dv_status dv_sparse_mlp_blocked(const dv_dims* dims, const dv_layer* layer, const float* xn, int32_t B,
                                const int32_t* blocks, int32_t kb, int32_t bs, float* y, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* Head-sparse decode attention ("Head-Pruned Attention Dispatch").
 *   xn [B][d] fp32 (already normalised), heads [B][kh]; k_cache/v_cache [B][H][t_max][dh].
 *   For each active head h: q,k,v = xn . W_h + b_h; k,v are written to slot t_past of head h
 *   (inactive heads' caches are neither read nor written); o_h = softmax(K q / sqrt(dh)) V
 *   over the t_past cached entries plus the current one.
 *   y [B][d] = sum_h o_h . Wo_h + bo   (no residual). kh = 0 gives y = bo. */
dv_status dv_sparse_attn(const dv_dims* dims, const dv_layer* layer, const float* xn, int32_t B,
                         const int32_t* heads, int32_t kh, void* k_cache, void* v_cache,
                         int32_t t_past, float* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* One sparse decoder layer ("Step-by-Step Implementation", layer; attention also sparse):
 *   h1 = x + Attn_Sh(RMSNorm_g1(x));  x_out = h1 + MLP_S(RMSNorm_g2(h1)).
 *   Sets: if idx_in and heads_in are both non-NULL they are used; if both are NULL the
 *   sets are predicted inline from x_pred with `pred` (dv_predict + dv_topk); any other
 *   combination is DV_ERR_NULL. idx_out/heads_out (nullable) receive the sets used.
 *   x_out may equal x; x_pred may equal x. RMSNorm eps = 1e-5. */
dv_status dv_layer_step(const dv_dims* dims, const dv_layer* layer, const dv_predictor* pred,
                        const float* x, const float* x_pred, int32_t B, int32_t k, int32_t kh,
                        const int32_t* idx_in, const int32_t* heads_in, void* k_cache,
                        void* v_cache, int32_t t_past, float* x_out, int32_t* idx_out,
                        int32_t* heads_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* dv_layer_step for callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid allocation): the same arguments without the
 * workspace, whose role a fixed device array of the library takes, DV_NOALLOC_SCRATCH_BYTES
 * long. Each GPU holds its own copy of that array from the first use of the library there
 * until the process ends; the call allocates nothing.
 *   - Shapes whose dv_workspace_bytes(dims, B, k, kh) exceeds DV_NOALLOC_SCRATCH_BYTES are
 *     refused with DV_ERR_WORKSPACE before anything is launched (32 MiB holds every batch up
 *     to 8 rows at the OPT-175B layer shape, k 2458, kh 19, and any one-row layer up to it).
 *   - All calls on one GPU share its copy of the array: calls that overlap on one GPU (other
 *     streams, other host threads) race on it and must be ordered by the caller.
 *   - Results are bitwise those of dv_layer_step with the same arguments. */
#define DV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
dv_status dv_layer_step_noalloc(const dv_dims* dims, const dv_layer* layer, const dv_predictor* pred,
                                const float* x, const float* x_pred, int32_t B, int32_t k, int32_t kh,
                                const int32_t* idx_in, const int32_t* heads_in, void* k_cache,
                                void* v_cache, int32_t t_past, float* x_out, int32_t* idx_out,
                                int32_t* heads_out, hipStream_t stream);

/* A stack of n_layers sparse layers with lookahead prediction ("Asynchronous Lookahead
 * Predictors", "Pipelined Overlap Execution"). The sets of layer l+1 are predicted from
 * the input of layer l on `side_stream` while layer l runs on `stream`; layer 0's sets are
 * predicted from the stack input first. layers/preds/k_caches/v_caches are HOST arrays of
 * n_layers entries (the pointers inside are device memory).
 *   x [B][d]: stack input; y [B][d]: stack output (may equal x).
 *   h_all (nullable) [n_layers+1][B][d]: receives every layer's input and the final output.
 *   idx_out [n_layers][B][k], heads_out [n_layers][B][kh] (nullable): the sets used.
 *   side_stream may equal stream (then everything is serial). Results are bitwise identical
 *   either way. Workspace: dv_stack_workspace_bytes(). The call creates its own fork/join
 *   events and destroys them before returning (also under stream capture: the captured
 *   graph keeps the dependencies, not the events). */
dv_status dv_lookahead_stack(const dv_dims* dims, const dv_layer* layers, const dv_predictor* preds,
                             int32_t n_layers, const float* x, int32_t B, int32_t k, int32_t kh,
                             void* const* k_caches, void* const* v_caches, int32_t t_past,
                             float* y, float* h_all, int32_t* idx_out, int32_t* heads_out,
                             void* ws, size_t ws_bytes, hipStream_t stream,
                             hipStream_t side_stream);

/* One decode token through the lookahead stack, with a past KV length per row held in
 * device memory, so rows of a batch can sit at different positions and a captured graph of
 * the call can be replayed for consecutive tokens ("Asynchronous Lookahead Predictors";
 * the skip of an inactive head's KV from "Head-Pruned Attention Dispatch").
 *   t_rows [B] int32, DEVICE memory: row b has t_rows[b] past entries in every layer's
 *   cache and writes the token's k/v at slot t_rows[b] of each head it selects. A head that
 *   a row does not select leaves that slot as it was (a zero slot of a fresh cache stays
 *   zero, and later tokens read it as a zero key and value). The kernels read t_rows on the
 *   device, so the host cannot check it: values outside [0, t_max-1] are clamped into that
 *   range, which keeps every access inside the cache (the row then attends as if it had
 *   the clamped length).
 *   advance != 0: after the last layer, t_rows[b] = min(t_rows[b] + 1, t_max - 1), ordered
 *   on `stream` after every read of t_rows.
 *   Everything else is as dv_lookahead_stack (same workspace size); dv_lookahead_stack with
 *   t_past = T equals this call with every t_rows[b] = T. */
dv_status dv_decode_step(const dv_dims* dims, const dv_layer* layers, const dv_predictor* preds,
                         int32_t n_layers, const float* x, int32_t B, int32_t k, int32_t kh,
                         void* const* k_caches, void* const* v_caches, int32_t* t_rows,
                         int32_t advance, float* y, float* h_all, int32_t* idx_out,
                         int32_t* heads_out, void* ws, size_t ws_bytes, hipStream_t stream,
                         hipStream_t side_stream);

/* Training targets of one layer for the lookahead predictors, from the dense layer (every head
 * and every neuron selected): DejaVu Guide, "Mathematical Formulation of Lookahead
 * Predictors" (the head predictor targets the heads with the largest attention norms, the
 * neuron predictor the neurons that fire); blog summary "What Is Contextual Sparsity?" (the
 * offline phase records each input's active heads and neurons).
 *   x [B][d] fp32 layer inputs; caches as dv_sparse_attn (slot t_past of every head is
 *   written with the input's k/v, as a dense layer step would).
 *   fire [B][F] uint8 (nullable): 1 where the up-projection pre-activation on RMSNorm(h1),
 *   h1 = x + Attn(RMSNorm(x)), is positive (ReLU passes it), else 0.
 *   preact [B][F] fp32 (nullable): those pre-activations (bias included).
 *   head_norm [B][H] fp32 (nullable): ||o_h||_2 of every head's attention output; the head
 *   targets are its top-kh per row (dv_topk).
 *   At least one output must be given. Workspace: dv_workspace_bytes(dims, B, d_ffn,
 *   n_heads). */
dv_status dv_layer_labels(const dv_dims* dims, const dv_layer* layer, const float* x, int32_t B,
                          void* k_cache, void* v_cache, int32_t t_past, uint8_t* fire, float* preact,
                          float* head_norm, void* ws, size_t ws_bytes, hipStream_t stream);

/* One full-batch training step of a rank-r predictor (blog summary "What Is Contextual
 * Sparsity?": a small classifier per layer, trained on the layer's input; the scores of
 * "Mathematical Formulation of Lookahead Predictors" are its logits). All fp32, device memory:
 *   x [M][d] inputs, y [M][N] uint8 0/1 targets, p1 [r][d] and p2 [N][r] the two factors
 *   (scores s = (x p1^T) p2^T), v1/v2 their momentum buffers (zero before the first step).
 *   Loss: mean binary cross-entropy of s against y over all M*N pairs; *loss (device) gets
 *   its value at the parameters before the update. Update (heavy-ball momentum):
 *   v <- momentum * v + grad, p <- p - lr * v, for both factors.
 *   x, y, p1, p2, v1, v2 16-byte aligned; loss 4-byte aligned.
 *   Deterministic: the same inputs give the same bits on any device. Workspace:
 *   dv_predictor_train_workspace_bytes(M, d, N, r). */
size_t dv_predictor_train_workspace_bytes(int32_t M, int32_t d, int32_t N, int32_t r);
dv_status dv_predictor_train_step(const float* x, int32_t M, int32_t d, const uint8_t* y, int32_t N,
                                  int32_t r, float* p1, float* p2, float* v1, float* v2, float lr,
                                  float momentum, float* loss, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* Workspace bytes for every single-layer call above at this shape (the maximum). */
size_t dv_workspace_bytes(const dv_dims* dims, int32_t B, int32_t k, int32_t kh);
/* Workspace of dv_topk for B rows of n scores (0 if B or n is out of range). */
size_t dv_topk_workspace_bytes(int32_t B, int32_t n);
/* Workspace bytes for dv_lookahead_stack. */
size_t dv_stack_workspace_bytes(const dv_dims* dims, int32_t B, int32_t k, int32_t kh);

/* Observability: time the head-sparse q/k/v projection launch (the step's largest gather).
 * dv_timing_start(n) creates n event pairs and returns n (-1 if already active or n <= 0);
 * while active, each q/k/v launch of any call takes the next pair as the begin/end
 * timestamps of its own dispatch (hipExtLaunchKernel start/stop events) until n are used. dv_timing_stop(ms, n) waits for the recorded pairs, writes the
 * duration of each in milliseconds to ms[0..] (at most n; ms may be NULL), destroys the
 * events and returns the number recorded (-1 on a HIP error or if not active). */
int32_t dv_timing_start(int32_t n);
int32_t dv_timing_stop(float* ms, int32_t n);

const char* dv_status_str(dv_status status);
const char* dv_last_error(void);
/* Library version string. */
const char* dv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DEJAVU_HIP_H */
