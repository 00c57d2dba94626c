/*
 * path_attn.h -- C ABI of the MI355X (gfx950) PaTH attention library
 * (libpath_attn.so).
 *
 * PaTH attention ("PaTH Attention: Position Encoding via Accumulating
 * Householder Transformations"): causal softmax attention whose logit between
 * query i and key j <= i is
 *
 *     scale * k_j^T (H_{j+1} H_{j+2} ... H_i) q_i  [+ sum_{s=j+1}^{i} log f_s]
 *
 * with data-dependent transitions H_t = I - beta_t w_t w_t^T (Dutch technical
 * summary section 2, "Kernmechanisme"; Chinese notes, "overall framework" and
 * "key design"), the optional bracketed term being the PaTH-FoX forget gate
 * (Chinese notes, "PaTH-FoX").  Indices are 0-based, so H_0, beta_0 and f_0
 * never enter a logit.  The scale multiplies only the bilinear term.
 *
 * Conventions shared by every entry point
 *   - Pointers named q/k/v/w/out/k_cache/v_cache/workspace/beta/log_f/lse are
 *     DEVICE pointers (HIP device memory, or any pointer the device can
 *     read/write); all sizes are element counts unless named *_bytes.
 *   - Tensors are contiguous, row-major, [B][H][L][d] (per-token vectors) or
 *     [B][H][L] (per-token scalars).  Rows must be 16-byte aligned (d * elem
 *     size is a multiple of 16 for every supported d).
 *   - dtype: PATH_F32 (q,k,v,w,out in float32) or PATH_BF16 (bfloat16).
 *     beta, log_f and lse are always float32.
 *   - The caller owns every buffer, including the workspace; the library
 *     allocates nothing and keeps no global state apart from a per-device
 *     cache of one occupancy query (filled on the first decode call on a
 *     device, thread-safe) and the fixed device array that
 *     path_decode_step_noalloc uses instead of a workspace, so calls on
 *     different streams with different workspaces may run concurrently.
 *     Calls that share a workspace, a cache or that array race unless
 *     ordered by the caller.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream).  Argument checks run on the host before any HIP call;
 *     a negative path_status_t is returned and nothing is launched.  A failed
 *     launch returns PATH_ERR_HIP.
 *   - beta is used as given (no clipping); log_f holds log f_t (<= 0 for a
 *     forget gate, any finite value is accepted).
 */
#ifndef PATH_ATTN_H
#define PATH_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PATH_F32 = 0, PATH_BF16 = 1 } path_dtype_t;

typedef enum {
    PATH_OK = 0,
    PATH_ERR_INVALID = -1,      /* null pointer, bad size, bad dtype */
    PATH_ERR_UNSUPPORTED = -2,  /* valid but not implemented (d, chunk) */
    PATH_ERR_HIP = -3,          /* a HIP launch or runtime call failed */
    PATH_ERR_WORKSPACE = -4     /* workspace missing or too small */
} path_status_t;

/* Human-readable text for a status code (static storage). */
const char* path_status_string(int status);

/* Library version string (static storage). */
const char* path_version(void);

/*
 * Workspace size in bytes needed by path_attn_fwd for these sizes, or 0 if
 * the arguments are invalid/unsupported.  chunk: 0 = library default.
 */
size_t path_attn_fwd_workspace_bytes(int B, int H, int L, int d, int dtype,
                                     int chunk);

/*
 * PaTH attention forward (prefill) for all B*H heads.
 *
 * Computes, per head and every row i < L,
 *     out_i = sum_{j<=i} softmax_j(logit_ij) v_j,   lse_i = log sum_j exp(logit_ij)
 * with logit_ij as in the file header, using the pages' blockwise algorithm:
 * per chunk of `chunk` tokens the product of its transitions is held in the
 * UT-transform form I - W^T T^{-1} W, T^{-1} = (I + strictLower(D W W^T))^{-1} D
 * (Chinese notes, training strategy), and each query tile scans the key
 * chunks right to left, carrying the query through every chunk it passes
 * (Dutch summary section 3, FlashAttention-style algorithm).
 *
 *   q, k, v, w  [B][H][L][d] dtype.  w need not be unit-norm.
 *   beta        [B][H][L] float32.
 *   log_f       [B][H][L] float32, or NULL for PaTH without the forget gate.
 *   out         [B][H][L][d] dtype (written).
 *   lse         [B][H][L] float32 natural-log log-sum-exp, or NULL.
 *   d           PATH_BF16: 64 or 128.  PATH_F32: 16, 32, 64 (and 128 with
 *               chunk <= 32).
 *   chunk       0 = default (64 for bf16, 16 for f32 with d <= 32, else 32);
 *               PATH_BF16 supports 64, PATH_F32 supports 16, 32, 64.
 *   L >= 1 (any length: a ragged last chunk is padded internally); B, H >= 1.
 *   workspace   at least path_attn_fwd_workspace_bytes(...) bytes, 256-byte
 *               aligned; its contents on entry are ignored.
 * Inputs are not modified.
 */
int path_attn_fwd(const void* q, const void* k, const void* v, const void* w,
                  const float* beta, const float* log_f,
                  void* out, float* lse,
                  int B, int H, int L, int d, float scale,
                  int dtype, int chunk,
                  void* workspace, size_t ws_bytes, void* stream);

/*
 * The two stages of path_attn_fwd, for callers that time or schedule them
 * separately.  Same arguments, layouts and errors as path_attn_fwd.
 *
 * path_attn_fwd_prepare: the per-chunk stage (the pages' boundary-adjusted
 *   keys and queries computed beforehand, Dutch summary section 3): the UT
 *   transform of every chunk and the chunk-local forget-gate sums, written
 *   to `workspace`; for bf16 with d = 64 also each query chunk's step with
 *   its own chunk (queries carried to the chunk start, the probabilities of
 *   the chunk's own keys), which needs q and scale.  Reads q, k, v, w, beta,
 *   log_f.
 * path_attn_fwd_scan: the right-to-left scan of each query tile over the key
 *   chunks (Dutch summary section 3), reading q and the workspace written by
 *   a preceding path_attn_fwd_prepare with the same q, B, H, L, d, scale,
 *   dtype, chunk and the same log_f presence (the workspace must not be
 *   modified in between).  Writes out and lse.
 */
int path_attn_fwd_prepare(const void* q, const void* k, const void* v, const void* w,
                          const float* beta, const float* log_f,
                          int B, int H, int L, int d, float scale, int dtype, int chunk,
                          void* workspace, size_t ws_bytes, void* stream);

int path_attn_fwd_scan(const void* q, const void* k, const void* v, const void* w,
                       const float* log_f, void* out, float* lse,
                       int B, int H, int L, int d, float scale,
                       int dtype, int chunk,
                       const void* workspace, size_t ws_bytes, void* stream);

/*
 * Workspace size in bytes for path_attn_bwd, or 0 if the arguments are
 * invalid or unsupported (dtype other than PATH_BF16, d other than 64).
 * Grows as B*H*L^2/64 * 16 bytes: two 64 x 64 bf16 tiles per pair of
 * chunks (b < a) per head, plus O(B*H*L*d) for the per-chunk quantities.
 */
size_t path_attn_bwd_workspace_bytes(int B, int H, int L, int d, int dtype);

/*
 * Gradients of path_attn_fwd (training; the pages train with the same
 * blockwise algorithm as the forward: English summary, Dutch summary
 * section 3).  Given the forward's inputs, its out and lse, and d_out =
 * dLoss/d out, writes dLoss/d of every input, the exact gradient of the
 * blockwise computation read back step by step (Chinese notes, training
 * strategy: the UT transform, a block's full-matrix form, the right-to-left
 * transport of queries); the softmax part follows the usual
 * rowsum(d_out o out) form of attention's backward.
 *
 *   q, k, v, w     [B][H][L][d] bf16, as given to path_attn_fwd.
 *   beta           [B][H][L] float32.
 *   log_f          [B][H][L] float32 or NULL (no forget gate).
 *   out, lse       the forward's outputs for these inputs (out bf16, lse
 *                  float32 natural log).
 *   d_out          [B][H][L][d] bf16.
 *   dq, dk, dv, dw [B][H][L][d] float32 (written, every element).
 *   dbeta          [B][H][L] float32 (written).
 *   dlog_f         [B][H][L] float32 (written), NULL exactly when log_f is
 *                  NULL; dlog_f[0] of each head is 0 up to rounding (f_0
 *                  never enters a logit).
 *   dtype          PATH_BF16 only; d = 64 only (else PATH_ERR_UNSUPPORTED).
 *   workspace      at least path_attn_bwd_workspace_bytes(...) bytes,
 *                  256-byte aligned; contents on entry ignored.
 * Gradients are accumulated in float32 from bf16 MFMA products; the per-pair
 * states the algorithm stores are bf16.  A null pointer, a bad size or
 * log_f/dlog_f given without the other is PATH_ERR_INVALID.  Inputs are not
 * modified.  Asynchronous on `stream`.
 */
int path_attn_bwd(const void* q, const void* k, const void* v, const void* w,
                  const float* beta, const float* log_f, const void* out,
                  const float* lse, const void* d_out, float* dq, float* dk,
                  float* dv, float* dw, float* dbeta, float* dlog_f,
                  int B, int H, int L, int d, float scale, int dtype,
                  void* workspace, size_t ws_bytes, void* stream);

/*
 * Workspace size in bytes for path_kcache_from_prefill, or 0 if invalid.
 */
size_t path_kcache_workspace_bytes(int B, int H, int L, int d, int dtype);

/*
 * Key/value cache after a prefill of L tokens, for the decode steps that
 * follow (Dutch summary section 3, "Inferentie": cached keys are updated in
 * place, so no separate cache of transition vectors is kept).
 *
 *   k_cache[b][h][j] = H_{L-1} ... H_{j+1} k_j   for j < L   (written)
 *   v_cache[b][h][j] = v_j                       for j < L   (written)
 * Slots j >= L are not touched.
 *   k, v, w     [B][H][L][d] dtype;  beta [B][H][L] float32.
 *   k_cache, v_cache  [B][H][T_max][d] dtype, T_max >= L.
 *   dtype       PATH_BF16 with d in {64, 128}.
 *   workspace   >= path_kcache_workspace_bytes(B,H,L,d,dtype) bytes.
 */
int path_kcache_from_prefill(const void* k, const void* v, const void* w,
                             const float* beta, void* k_cache, void* v_cache,
                             int B, int H, int L, int T_max, int d, int dtype,
                             void* workspace, size_t ws_bytes, void* stream);

/*
 * The same caches from the workspace of a path_attn_fwd (bf16, d in {64,
 * 128}, default chunk) that has just run on the same k, w, beta (Dutch
 * summary section 3, "Inferentie": the cache as above).  The forward's
 * workspace holds every key carried to its chunk end and each chunk's whole
 * product, so the keys' per-chunk transform is not computed again.
 *
 *   fwd_workspace  the forward's workspace, fwd_ws_bytes >=
 *                  path_attn_fwd_workspace_bytes(B,H,L,d,dtype,0); read
 *                  only.  Its contents must be those the forward wrote
 *                  (the gate does not matter); nothing checks this.
 *   v              [B][H][L][d] dtype, copied into v_cache.
 *   k_cache, v_cache, T_max, B, H, L, d, dtype: as path_kcache_from_prefill.
 *   workspace      >= path_kcache_workspace_bytes(B,H,L,d,dtype) bytes.
 * Errors as path_kcache_from_prefill; a forward workspace that is null,
 * too small or not 256-byte aligned: PATH_ERR_WORKSPACE.  The results agree
 * with path_kcache_from_prefill to bf16 rounding (the chunk products enter
 * as d x d bf16 tiles instead of W and T^-T W).
 */
int path_kcache_from_forward(const void* fwd_workspace, size_t fwd_ws_bytes, const void* v,
                             void* k_cache, void* v_cache, int B, int H, int L, int T_max,
                             int d, int dtype, void* workspace, size_t ws_bytes, void* stream);

/*
 * Workspace size in bytes for path_decode_step, or 0 if invalid.
 */
size_t path_decode_workspace_bytes(int B, int H, int T_max, int d, int dtype);

/*
 * One decode step at position t (Dutch summary section 3, "Inferentie";
 * Chinese notes, inference paragraph): every cached key is first updated in
 * place with the new transition,
 *     k_cache[j] <- (I - beta_t w_t w_t^T) k_cache[j]     for j < t,
 * then k_t, v_t are stored at slot t, and q_t attends over slots 0..t:
 *     out_t = sum_{j<=t} softmax_j(scale * q_t . k_cache[j]) v_cache[j].
 * The updated keys are written back in the cache dtype (rounded to nearest
 * even for bf16).  No forget gate.
 *
 *   k_cache, v_cache  [B][H][T_max][d] dtype; slots [0,t) updated in place,
 *                     slot t written.
 *   q_t, k_t, v_t, w_t  [B][H][d] dtype;  beta_t [B][H] float32.
 *   out_t       [B][H][d] dtype;  lse_t [B][H] float32 or NULL.
 *   0 <= t < T_max.  dtype PATH_BF16 with d in {64, 128}.
 *   workspace   >= path_decode_workspace_bytes(B,H,T_max,d,dtype) bytes.
 */
int path_decode_step(void* k_cache, void* v_cache,
                     const void* q_t, const void* k_t, const void* v_t,
                     const void* w_t, const float* beta_t,
                     void* out_t, float* lse_t,
                     int B, int H, int t, int T_max, int d, float scale,
                     int dtype, void* workspace, size_t ws_bytes,
                     void* stream);

/*
 * path_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, same kernels and the
 * same results as path_decode_step (bit for bit), but the split partials go
 * to an array the library keeps in device memory, one per device
 * (8 MiB, held until the process ends; its address is looked up on the first
 * call on each device).  Nothing is allocated or freed by this call.
 *
 * Limit: B*H * ceil((t+1)/64) * (d+2) * 4 bytes must not exceed 8 MiB
 * (e.g. B*H = 64, d = 128: t < 16128); larger calls return
 * PATH_ERR_WORKSPACE before any HIP call.  Argument errors are those of
 * path_decode_step.
 *
 * Every call on one device shares that device's array, and each call
 * overwrites it before reading it (no clearing is needed): calls that overlap
 * on one device (different streams or threads, no ordering between them)
 * race and give undefined results.  Calls on one stream are ordered.
 */
int path_decode_step_noalloc(void* k_cache, void* v_cache,
                             const void* q_t, const void* k_t, const void* v_t,
                             const void* w_t, const float* beta_t,
                             void* out_t, float* lse_t,
                             int B, int H, int t, int T_max, int d, float scale,
                             int dtype, void* stream);

/*
 * PaTH-FoX decode (the forget gate of PaTH-FoX in the decode step).  The
 * PaTH-FoX weight multiplies the PaTH one by the product of the forget gates
 * f_{j+1} .. f_t (Chinese notes, PaTH-FoX extension), i.e. adds
 * F_t - F_j to the logit of key j, with F_t = sum_{s<=t} log f_s (natural
 * log); the in-place key update and the rest of the step are those of
 * path_decode_step.  The gate cache holds F_j per slot.
 *
 * path_fcache_from_prefill fills f_cache[0..L) from a prefill's log f:
 *   log_f       [B][H][L] float32 (log f, not f).
 *   f_cache     [B][H][T_max] float32, T_max >= L; slots [0, L) written
 *               (accumulated in fp64, stored as fp32).
 *
 * path_decode_step_gated is path_decode_step plus:
 *   f_cache     [B][H][T_max] float32 holding F_0 .. F_{t-1}; slot t is
 *               written with F_t = F_{t-1} + log_f_t (F_{-1} = 0).
 *   log_f_t     [B][H] float32, log f of token t.
 * Both return PATH_ERR_INVALID for a null gate pointer or bad sizes, checked
 * before any launch; the caller owns the gate cache.
 */
int path_fcache_from_prefill(const float* log_f, float* f_cache, int B, int H, int L,
                             int T_max, void* stream);
int path_decode_step_gated(void* k_cache, void* v_cache, float* f_cache,
                           const void* q_t, const void* k_t, const void* v_t,
                           const void* w_t, const float* beta_t, const float* log_f_t,
                           void* out_t, float* lse_t,
                           int B, int H, int t, int T_max, int d, float scale,
                           int dtype, void* workspace, size_t ws_bytes,
                           void* stream);

/*
 * Paged key/value cache.  With the keys updated in place, decoding is plain
 * softmax decoding over one cache, so paged caches and split-sequence
 * decoding apply unchanged (Chinese notes, inference paragraph; Dutch
 * summary section 3, "Inferentie").  The cache is a pool of pages instead of
 * one [B][H][T_max][d] array:
 *
 *   k_pool, v_pool  [num_blocks][H][page][d] dtype: page p holds `page`
 *                   consecutive slots of every head of one sequence.
 *   block_table     [B][max_blocks] int32 (device): slot j of sequence b is
 *                   slot j % page of page block_table[b][j / page].
 *   page            a positive multiple of 64; the capacity of a sequence is
 *                   max_blocks * page slots.
 * The caller owns the pool and the table and must keep the table's entries
 * for every slot a call touches within [0, num_blocks): an entry outside
 * that range gives undefined results (no status reports it).  Such a page
 * number is never dereferenced, so it cannot fault: its slots are left out
 * of the update and the attention, and a new key or value for one of them
 * is not stored.
 *
 * path_kcache_from_prefill_paged is path_kcache_from_prefill writing the
 * transformed keys and the values through the table (slots [0, L); L <=
 * max_blocks * page); workspace as path_kcache_workspace_bytes.
 *
 * path_decode_step_paged is path_decode_step (and, with f_cache and log_f_t
 * both non-NULL, path_decode_step_gated) on a paged cache: the in-place key
 * update, the append at slot t and the attention go through the table, with
 * t < max_blocks * page.  f_cache, if given, is contiguous
 * [B][H][max_blocks * page] float32.  Workspace: path_decode_workspace_bytes
 * with T_max = max_blocks * page.  The arithmetic and the split of the keys
 * are those of the contiguous call, so the results are identical to it.
 * Bad sizes, a null table or only one of f_cache / log_f_t:
 * PATH_ERR_INVALID; a page that is not a multiple of 64: PATH_ERR_UNSUPPORTED.
 */
int path_kcache_from_prefill_paged(const void* k, const void* v, const void* w,
                                   const float* beta, void* k_pool, void* v_pool,
                                   const int* block_table, int num_blocks, int max_blocks,
                                   int page, int B, int H, int L, int d, int dtype,
                                   void* workspace, size_t ws_bytes, void* stream);
int path_decode_step_paged(void* k_pool, void* v_pool, const int* block_table,
                           int num_blocks, int max_blocks, int page,
                           float* f_cache, const float* log_f_t,
                           const void* q_t, const void* k_t, const void* v_t,
                           const void* w_t, const float* beta_t,
                           void* out_t, float* lse_t,
                           int B, int H, int t, int d, float scale, int dtype,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * Transition parameters of every token from the layer input, the step ahead
 * of the attention (Chinese notes, "key design": w_t from a low-rank linear
 * layer, a short convolution of filter size 3 and an L2 normalisation;
 * beta_t = 2 sigmoid(u^T x_t + b); Dutch summary section 2, "Kernmechanisme"):
 * for token t and head h,
 *     z_t    = W_up (W_down x_t)                           (low-rank map)
 *     c_t    = conv[:,0] * z_t + conv[:,1] * z_{t-1} + conv[:,2] * z_{t-2}
 *              (depthwise and causal; z before the first token is 0)
 *     w_t    = c_t[h*d .. h*d+d) / || c_t[h*d .. h*d+d) ||   (0 if that is 0)
 *     beta_t = 2 sigmoid(u_h . x_t + b_h)
 * Readings where the pages are silent: no bias in the low-rank map, no bias
 * or activation in the convolution, one norm per head's d-vector.
 *
 *   x       [B][L][Dm]   bf16   layer input (token-major)
 *   w_down  [r][Dm]      bf16
 *   w_up    [H*d][r]     bf16
 *   conv    [H*d][3]     float32, tap k multiplies z_{t-k}
 *   u       [H][Dm]      bf16
 *   b       [H]          float32
 *   w       [B][H][L][d] bf16 out, the layout path_attn_fwd takes
 *   beta    [B][H][L]    float32 out
 * dtype must be PATH_BF16 (PATH_F32: PATH_ERR_UNSUPPORTED).  Supported sizes:
 * d in {64, 128}, r in {32, 64}, r + H <= 128, Dm a positive multiple of 128
 * (else PATH_ERR_UNSUPPORTED); a null pointer or a size below 1 is
 * PATH_ERR_INVALID.  Products accumulate in float32 (the low-rank
 * intermediate W_down x_t enters the second product as a bf16 pair, high and
 * low part); w is rounded to bf16 once, after the normalisation.  The inputs
 * are only read; w and beta are overwritten.
 */
int path_transition_prep(const void* x, const void* w_down, const void* w_up,
                         const float* conv, const void* u, const float* b,
                         void* w, float* beta, int B, int L, int Dm, int r, int H,
                         int d, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PATH_ATTN_H */
