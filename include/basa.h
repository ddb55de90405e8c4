/*
 * basa.h -- C ABI of libbasa: BASA sparse attention on AMD gfx950.
 *
 * BASA ("Backend-Agnostic Sparse Attention for Fast High-Resolution Visual
 * Generation", arXiv 2610.08772v1; paperlayer.ai summary) replaces a
 * diffusion transformer's visual self-attention by attention inside regular
 * local windows of the latent token grid whose partition is cyclically
 * shifted from block to block (sec. 3.1, A.1), plus a pooled global K/V
 * memory every window attends to (sec. 3.2, A.1), plus -- for video -- whole
 * windows of original K/V routed to each window by content (sec. 3.3, A.2),
 * all under one joint softmax (A.1).
 *
 * One DiT block runs, on one HIP stream, in this order:
 *     basa_pool_kv        (if the plan pools)
 *     basa_route_windows  (if the plan routes)
 *     basa_window_attn_fwd   (or basa_window_attn_fwd_split, the branch form)
 *     basa_text_attn_fwd     (joint blocks with text rows: the text queries)
 * and, when training through it (the pages' sparse adaptation, sec. 3.4):
 *     basa_window_attn_bwd  (same inputs, the forward's out and lse, dL/dout)
 *
 * Conventions shared by every call below
 * --------------------------------------
 * Tensors.  Every tensor argument is a device pointer owned by the caller,
 * contiguous, 16-byte aligned, in the layouts stated per call.  Token tensors
 * are [B, H, N, d] with the N tokens of the (T, Hg, Wg) grid in raster order
 * (t, y, x), x fastest.  Element type is the plan's dtype: BASA_BF16 means
 * bfloat16 in and out; BASA_F32 means float32 in and out (values are rounded to
 * bfloat16 as they are staged for the matrix cores; accumulation is float32).
 * The library keeps no pointer after a call returns and allocates no device
 * memory: scratch space is passed in by the caller (route, backward,
 * branch-split and text-query workspaces, sized in basa_plan_info).
 * Streams.  `stream` is a hipStream_t passed as void*; NULL is the null stream.
 * Work is enqueued asynchronously; the call does not synchronise.
 * Errors.  Arguments are checked before anything is enqueued; on a bad
 * argument the call returns a status, leaves all outputs untouched and records
 * a message for basa_last_error() (per host thread).  BASA_ERR_HIP reports a
 * failed launch.  Faults inside kernels surface at the caller's next
 * synchronisation.  The library never prints and never aborts.
 * Plans.  A plan is host memory only, immutable once built, and may be shared
 * by any number of threads and streams.  One plan describes one block's shift;
 * a model alternating shifts uses one plan per shift.
 */
#ifndef BASA_H
#define BASA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BASA_OK = 0,
  BASA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, size or range out of bounds */
  BASA_ERR_NOT_DIVISIBLE = 2,    /* pool cell does not tile the grid */
  BASA_ERR_UNSUPPORTED = 3,      /* valid request outside what the kernels implement */
  BASA_ERR_HIP = 4,              /* a HIP runtime call or kernel launch failed */
  BASA_ERR_OUT_OF_MEMORY = 5     /* host allocation of the plan failed */
} basa_status;

typedef enum { BASA_BF16 = 0, BASA_F32 = 1 } basa_dtype;

typedef struct basa_plan_s* basa_plan_t;

/* Problem description of one block (paperlayer.ai summary, A.1 and A.2).
 * 2D grids use grid[0] = window[0] = 1.  All sizes are in tokens. */
typedef struct {
  int32_t batch;          /* B >= 1 */
  int32_t heads;          /* H >= 1; every head is independent (routing is per head) */
  int32_t head_dim;       /* d: 64 or 128 */
  int32_t grid[3];        /* {T, Hg, Wg} latent token grid */
  int32_t window[3];      /* local window {wt, wh, ww}, 1 <= window[i] <= grid[i].  The
                             windows tile the rolled grid padded up to a window
                             multiple; padding is not a token, so the last
                             window along an axis the window does not divide is
                             short: it holds the grid[i] mod window[i] real
                             positions left, and its slots (queries and keys)
                             are numbered over those alone */
  int32_t shift[3];       /* cyclic partition offset, 0 <= shift[i] < grid[i].  The grid
                             is rolled by -shift and cut into windows: window 0 starts
                             at original coordinate `shift`; windows wrap around the
                             grid edge and are not masked */
  int32_t pool[3];        /* avg-pool cell, must divide grid; {0,0,0} disables the
                             pooled global memory.  Cells tile the unshifted grid */
  int32_t route_topk;     /* routed windows per window, 0 disables routing, else
                             1 .. min(nW - 1, 16) */
  int32_t route_radius;   /* candidate windows for routing (paperlayer.ai summary, A.2:
                             "candidate-window radius is one" for video): -1 = every
                             other window; r >= 0 = windows whose window-grid
                             coordinates differ from the query window's by at most r
                             on every axis (no wrap-around).  With r >= 0 every
                             window, corners included, must have route_topk
                             candidates */
  basa_dtype dtype;       /* element type of q, k, v, k_pool, v_pool, out, x, x_win */
  float softmax_scale;    /* scale on q.k; 0 selects 1/sqrt(head_dim) */
  int32_t global_tokens;  /* X >= 0 extra global K/V rows every window attends to, stored
                             after the G pooled cells in k_pool / v_pool (e.g. the text
                             tokens of an MM-DiT: paperlayer.ai A.1 evaluates a
                             "text/global-memory" branch under the same softmax).  The
                             caller writes them; basa_pool_kv writes rows 0..G-1 only */
} basa_params;

/* Sizes derived by a plan.  "Pairs" count (query, key) products over all
 * B*H heads; FLOPs count 4*d per pair (q.k and p.v, multiply and add), with
 * no padding.  With short windows the routed part is counted at M keys per
 * routed window, an upper bound (which windows are routed is known only at
 * run time).  The dense figures are for full attention over the same grid. */
typedef struct {
  int64_t n_tokens;              /* N = T*Hg*Wg */
  int64_t n_windows;             /* nW = prod ceil(grid[i] / window[i]) */
  int64_t window_tokens;         /* M = wt*wh*ww (slots of a full window) */
  int64_t pooled_tokens;         /* G, 0 if pooling is off */
  int64_t keys_per_query;        /* L = M + G + X + route_topk*M (the most any list holds) */
  int64_t route_workspace_bytes; /* device scratch basa_route_windows needs (0 if no routing) */
  double pairs_sparse, pairs_dense;
  double flops_sparse, flops_dense;
  int64_t global_tokens;         /* X (extra global rows after the pooled cells) */
  int64_t bwd_workspace_bytes;   /* device scratch basa_window_attn_bwd needs */
  int64_t split_workspace_bytes; /* device scratch basa_window_attn_fwd_split needs */
  int64_t text_splits;           /* parts of the text queries' key list (1: one pass) */
  int64_t text_workspace_bytes;  /* device scratch basa_text_attn_fwd needs (0: none) */
} basa_plan_info;

/* Validates `params` and builds a plan (host only; no HIP call is made).
 * Errors: INVALID_ARGUMENT (null pointer, non-positive size, window larger
 * than the grid, shift out of range, route_topk out of range, route_radius <
 * -1 or leaving a corner window fewer than route_topk candidates, bad scale
 * or dtype), NOT_DIVISIBLE (a pool cell does not divide the grid),
 * UNSUPPORTED (head_dim not 64/128,
 * route_topk > 16, routing with more than 8192 windows, more than 2^24 tokens,
 * more than 2^31 elements per tensor), OUT_OF_MEMORY. */
basa_status basa_plan(const basa_params* params, basa_plan_t* plan);

/* Frees a plan; NULL is ignored. */
void basa_plan_destroy(basa_plan_t plan);

/* Copies the plan's derived sizes into *info. */
basa_status basa_plan_get_info(basa_plan_t plan, basa_plan_info* info);

/* Exact count of the (query, key) pairs a forward of this plan computes with
 * a given route table (host only, no HIP call).  The plan's own counts
 * (basa_plan_info) take every routed window at M keys; with short windows
 * the routed windows' real sizes are known only once routing has run.
 * route: a HOST copy of the [B, H, nW, topk] table (NULL iff the plan does
 * not route).  *pairs receives the sum over heads and windows of M_w * (M_w +
 * G + X + sum_r M_{route[w][r]}), M_w the real tokens of window w; *flops
 * (may be NULL) 4 * d * pairs.  Errors: INVALID_ARGUMENT (null plan or pairs,
 * route presence not matching the plan, an entry outside [0, nW)). */
basa_status basa_plan_pairs(basa_plan_t plan, const int32_t* route, double* pairs,
                            double* flops);

/* Shift schedule across layers and denoising steps (paperlayer.ai, sec. 3.1:
 * window boundaries vary from block to block; a schedule interleaves
 * candidate offsets across layers before advancing them across denoising
 * steps).  Reading: the n_offsets candidates along axis a are
 * c * window[a] / n_offsets (integer division), c = 0 .. n_offsets - 1; block
 * `layer` at denoising step `step` takes candidate (layer + step) mod
 * n_offsets, so consecutive layers interleave the candidates and each step
 * advances every layer by one.  axes: bit a set = axis a (0 = T, 1 = H, 2 =
 * W) is offset, else its shift is 0 (6 = spatial only: a window spanning the
 * whole temporal axis gains nothing from a temporal offset).  Writes
 * shift[3], each in [0, window[a]): a valid basa_params.shift for any grid
 * at least one window wide.  Host only.  Errors: INVALID_ARGUMENT (null
 * pointer, n_offsets < 1, negative layer or step, axes outside [0, 7], a
 * window extent < 1). */
basa_status basa_shift_schedule(const int32_t window[3], int32_t layer, int32_t step,
                                int32_t n_offsets, int32_t axes, int32_t shift[3]);

/* Pooled global memory (paperlayer.ai, sec. 3.2 and A.1: a regular spatial
 * reduction by average pooling).  k, v: [B, H, N, d].  k_pool, v_pool:
 * [B, H, G + X, d] (X = global_tokens); rows 0..G-1 receive the cells in
 * raster order of the pooled grid, each the mean of its cell's tokens
 * (float32 accumulation, one rounding to the dtype); rows G.. are untouched.
 * Errors: INVALID_ARGUMENT if the plan does not pool or a pointer is
 * null/misaligned; HIP. */
basa_status basa_pool_kv(basa_plan_t plan, const void* k, const void* v, void* k_pool,
                         void* v_pool, void* stream);

/* Content-adaptive window routing (paperlayer.ai, sec. 3.3 and A.2).  For
 * every head and window i, the route_topk other windows j with the largest
 * score(i, j) = (sum of q over window i) . (sum of k over window j), in
 * descending score, ties to the smaller j.  Sums and the dot product are
 * float64: the window sums of bf16 input are exact (so independent of the
 * summation order) while the inputs' exponent span plus log2 of the window
 * size fits float64's 53-bit significand; float input sums round as any
 * float64 sum does.  The dot product runs in channel order with separate
 * multiply and add, so the result is reproducible bit for bit.  A NaN score
 * (non-finite input) ranks below every number, NaNs among themselves by
 * window index, so every entry of the table is still written.
 * q, k: [B, H, N, d].
 * route: [B, H, nW, route_topk] int32 (4-byte aligned).  workspace: device
 * scratch of at least info.route_workspace_bytes bytes, 256-byte aligned;
 * its contents on entry do not matter and on exit are unspecified.
 * Errors: INVALID_ARGUMENT if the plan does not route, a pointer is
 * null/misaligned or workspace_bytes is too small; HIP. */
basa_status basa_route_windows(basa_plan_t plan, const void* q, const void* k, int32_t* route,
                               void* workspace, size_t workspace_bytes, void* stream);

/* basa_route_windows for callers that cannot allocate device memory or pass
 * a workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same routing, with its scratch in a device
 * array the library holds, one per GPU, of at most 64 MiB (the plan's
 * info.route_workspace_bytes must not exceed it).  The call allocates
 * nothing.  Every call on a GPU shares that GPU's scratch and leaves its
 * contents behind; calls that overlap on one GPU (different streams or
 * threads) race and must be serialised by the caller.  Arguments as for
 * basa_route_windows without the workspace.  Errors: INVALID_ARGUMENT (the
 * plan does not route, a null or misaligned pointer), UNSUPPORTED (the
 * plan's scratch exceeds 64 MiB), HIP (the scratch lookup or a launch
 * failed). */
basa_status basa_route_windows_noalloc(basa_plan_t plan, const void* q, const void* k,
                                       int32_t* route, void* stream);

/* Fused window attention forward (paperlayer.ai, A.1: one softmax over the
 * concatenated K/V).  For query token n in window i, the key list is
 *   [window i's tokens in slot order] ++ [the G pooled cells] ++ [the X
 *   extra global rows] ++ [tokens of route[i][0]] ++ ... ++ [tokens of
 *   route[i][topk-1]]
 * and out[n] = softmax(scale * q_n . K_list^T) V_list, written at n's own
 * position.  q, k, v, out: [B, H, N, d].  k_pool, v_pool: [B, H, G + X, d],
 * the cells written by basa_pool_kv and the extra rows by the caller (NULL
 * iff G + X = 0).  route:
 * [B, H, nW, topk] as written by basa_route_windows (NULL iff topk == 0); an
 * entry outside [0, nW) is never used as an address and makes every output
 * row (and lse) of that window NaN, so a corrupt table shows in the result.
 * lse: optional float32 [B, H, N] natural-log log-sum-exp of the scaled
 * logits (NULL to skip).  A plan with window = grid, shift 0, no pooling and
 * no routing computes full dense attention.
 * Errors: INVALID_ARGUMENT (null/misaligned pointer, or pool/route pointer
 * presence not matching the plan); HIP. */
basa_status basa_window_attn_fwd(basa_plan_t plan, const void* q, const void* k, const void* v,
                                 const void* k_pool, const void* v_pool, const int32_t* route,
                                 void* out, float* lse, void* stream);

/* Text queries of a joint (MM-DiT) block.  The pages take the text tokens
 * as a branch of the image queries' softmax (paperlayer.ai, A.1) and say
 * nothing of the text tokens' own queries; read plainly, BASA sparsifies the
 * visual self-attention only, so each text query attends densely:
 *   out_text[s] = softmax(scale * q_text[s] . [K ++ K_text]^T) [V ++ V_text]
 * over all N image tokens and all X text rows.  q_text, out_text:
 * [B, H, X, d] in the plan dtype (X = global_tokens); k, v: [B, H, N, d];
 * k_global, v_global: [B, H, G + X, d], the buffers basa_window_attn_fwd
 * reads (the text rows follow the G pooled cells, which are not keys here).
 * lse_text: optional float32 [B, H, X], natural log.  When the text rows
 * are too few to fill the GPU, the key list is cut into info.text_splits
 * consecutive parts whose results are merged exactly by their log-sum-exps
 * (as the branch-split forms are); the parts' outputs and lse go to
 * workspace: device scratch of at least info.text_workspace_bytes bytes,
 * 256-byte aligned (may be NULL when that is 0).  The result then agrees
 * with one pass up to the rounding of the parts' outputs to the plan dtype.
 * Errors: INVALID_ARGUMENT (the plan has no text rows, a null or misaligned
 * pointer, or a small workspace); HIP. */
basa_status basa_text_attn_fwd(basa_plan_t plan, const void* q_text, const void* k,
                               const void* v, const void* k_global, const void* v_global,
                               void* out_text, float* lse_text, void* workspace,
                               size_t workspace_bytes, void* stream);

/* The same attention, executed as the pages do on stock backends
 * (paperlayer.ai, A.1): the key-list segments are evaluated as separate
 * branches and merged exactly by their log-sum-exps,
 *   out = sum_b exp(lse_b - lse) out_b,  lse = log sum_b exp(lse_b).
 * ways = 2: {window tokens, routed windows} and {global rows: pooled cells
 * and extra rows}; ways = 3: {window tokens}, {routed windows}, {global
 * rows}.  Branches without keys in this plan are dropped (with one branch
 * left, it is the joint computation).  Arguments as for
 * basa_window_attn_fwd, plus workspace: device scratch of at least
 * info.split_workspace_bytes bytes, 256-byte aligned, that holds each
 * branch's output (plan dtype) and lse.  The result agrees with
 * basa_window_attn_fwd up to the rounding of the branch outputs.
 * Errors: as basa_window_attn_fwd; INVALID_ARGUMENT for ways not 2 or 3 or
 * a small or misaligned workspace. */
basa_status basa_window_attn_fwd_split(basa_plan_t plan, const void* q, const void* k,
                                       const void* v, const void* k_pool, const void* v_pool,
                                       const int32_t* route, void* out, float* lse, int ways,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Gradients of basa_window_attn_fwd (the pages adapt the sparse model by
 * training, paperlayer.ai sec. 3.4).  Inputs as for the forward, plus out and
 * lse (float32 [B, H, N], required) of that forward and d_out = dL/d(out)
 * [B, H, N, d] in the plan's dtype.  Outputs, all float32: d_q, d_k, d_v
 * [B, H, N, d] and d_k_global, d_v_global [B, H, G + X, d] (the gradients of
 * the pooled cells and extra rows; NULL iff G + X = 0).  d_k, d_v include the
 * pooled cells' share carried back to their tokens (1/P of the cell's
 * gradient each); routing is a selection and has no gradient.  A route
 * entry outside [0, nW) routes nothing and makes that window's d_q rows NaN.
 * The products run on bf16 operands with float32 accumulation (P and dS
 * rounded to bf16); P is recomputed from lse, no score matrix is stored.  workspace: device
 * scratch of at least info.bwd_workspace_bytes bytes, 256-byte aligned (delta
 * = d_out . out and lse scaled to base 2, per token, the inverse route table, per-range partial sums of
 * the global rows' gradients, and for BASA_F32 plans bf16 copies of q, k, v,
 * d_out and the global rows).  Every output is deterministic: no atomics.
 * Errors: INVALID_ARGUMENT (null/misaligned pointer, pointer presence not
 * matching the plan, workspace too small); HIP (a kernel launch failed). */
basa_status basa_window_attn_bwd(basa_plan_t plan, const void* q, const void* k, const void* v,
                                 const void* k_pool, const void* v_pool, const int32_t* route,
                                 const void* out, const float* lse, const void* d_out,
                                 float* d_q, float* d_k, float* d_v, float* d_k_global,
                                 float* d_v_global, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Test hook: the plan's window partition (paperlayer.ai, A.1).  win_id[n] and
 * slot[n] (int32 [N], 4-byte aligned) give the window and the slot of token n
 * (slots of a short window run over its real positions only).
 * Errors: INVALID_ARGUMENT; HIP. */
basa_status basa_window_index(basa_plan_t plan, int32_t* win_id, int32_t* slot, void* stream);

/* Test and measurement hook: the shift-aware gather on its own -- the
 * window tensor that the pages' roll + reshape + permute of the token grid
 * forms (paperlayer.ai, A.1), which the attention kernel never materialises.
 * x: [B, H, N, d] -> x_win: [B, H, nW, M, d], x_win[b, h, i, s] = x[b, h,
 * token of slot s of window i], zero past a short window's slots.
 * Errors: INVALID_ARGUMENT; HIP. */
basa_status basa_gather_windows(basa_plan_t plan, const void* x, void* x_win, void* stream);

/* Measurement hook: the bf16 matrix-core rate this GPU sustains and its
 * clock under that load, to read the attention kernel's fraction of the
 * nominal peak against (the pages rate kernels by MFU against a nominal peak:
 * thelatestinai.com card, Table 3).  Launches n_workgroups workgroups of 256
 * threads; every wave runs four independent chains of iters
 * v_mfma_f32_32x32x16_bf16 products.  mode 0: constant operands (2^-6);
 * mode 1: operands whose bits change from one product to the next, as real
 * data's do (per-lane pseudo-random bf16 values, alternating with a
 * reordered, negated copy that cancels the previous product exactly); the
 * chip's clock under load depends on how many operand bits switch.
 * sink: device float32 [n_workgroups * 256], 4-byte aligned; each element
 * receives 4 * iters * 2^-8 in mode 0 and 0 in mode 1 (both exact).
 * clocks: device uint64 [n_workgroups * 4], 8-byte aligned; per workgroup the
 * shader clock (s_memtime) at start and end, then the 100 MHz constant clock
 * (s_memrealtime) at start and end.  flops: host double, NULL or receives
 * the launch's flop count (2 * 32 * 32 * 16 per product).  The caller owns
 * every buffer and times the launch (e.g. with events on `stream`).
 * Errors: INVALID_ARGUMENT (iters outside [1, 2^24), an odd iters in mode 1,
 * mode not 0 or 1, n_workgroups outside [1, 2^20], a null or misaligned
 * pointer); HIP (the launch failed). */
basa_status basa_probe_mfma(int32_t iters, int32_t mode, int32_t n_workgroups, float* sink,
                            uint64_t* clocks, double* flops, void* stream);

/* Name of a status code (static string). */
const char* basa_status_string(basa_status s);

/* Message of the last failed call on this host thread ("" if none). */
const char* basa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BASA_H */
