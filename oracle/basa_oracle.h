/*
 * basa_oracle.h -- plain CPU reference for BASA attention (TEST INFRASTRUCTURE).
 *
 * This library exists only so that tests, the package's smoke check and the
 * benchmark's CPU-baseline leg can check the GPU path against something slow
 * and obviously correct.  Nothing in the product path may link or call it.
 * It shares no code, header, table or helper with the GPU library.
 *
 * Source: "Backend-Agnostic Sparse Attention for Fast High-Resolution Visual
 * Generation" (BASA), as summarised on the paperlayer.ai page for arXiv
 * 2610.08772v1 (sections 3.1-3.3, A.1, A.2) and the thelatestinai.com card of
 * the same paper (Table 3).  Every function cites the passage it follows.
 *
 * Arithmetic: inputs arrive as float32 (bf16 values upcast exactly); every
 * accumulation, softmax and pooled value is carried in float64, compiled with
 * -ffp-contract=off and no fast-math, so the oracle's own rounding is far
 * below the bf16 tolerances it is used to check.
 *
 * Layouts (all row-major, contiguous):
 *   q, k, v      [B, H, N, d]      N tokens in raster order (t, y, x), x fastest
 *   kp, vp       [B, H, G + X, d]  pooled cells in raster order of the pooled grid,
 *                                  then the X extra global rows (bo_pool writes
 *                                  [B, H, G, d], the cells only)
 *   route        [B, H, nW, topk]  routed window ids, best first
 *   out          [B, H, N, d]      written at each query's original position
 *   lse          [B, H, N]         natural-log log-sum-exp of the scaled logits
 *
 * Parity status per function (the pins live in tests/test_oracle_*.py):
 *   bo_partition   pinned (roll/reshape/permute brute force, bijection)
 *   bo_pool        pinned (reshape-mean brute force, pool = grid, pool = 1)
 *   bo_route       pinned (argsort brute force, planted ranking, exact window
 *                  sums in any order for bf16 inputs)
 *   bo_attend*     pinned (dense masked attention brute force, SDPA at
 *                  window = grid, closed forms, branch-merge equivalence)
 *   bo_attend_bwd* pinned (central finite differences of bo_attend, torch
 *                  float64 autograd of dense masked attention)
 */
#ifndef BASA_ORACLE_H
#define BASA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  BO_OK = 0,
  BO_EINVAL = 1,       /* null pointer, non-positive size, bad scale */
  BO_ENOTDIV = 2,      /* pool does not divide the grid */
  BO_ERANGE = 3,       /* window above grid, shift outside [0, grid), topk outside
                          [0, nW-1] or above
                          the candidates a corner window has within the radius */
  BO_ENOMEM = 4
};

typedef struct {
  int64_t batch, heads, dim;
  int64_t grid[3];     /* {T, H, W}; T = 1 for images */
  int64_t window[3];   /* local window extent per axis */
  int64_t shift[3];    /* cyclic shift of the partition for this block */
  int64_t pool[3];     /* avg-pool cell per axis; {0,0,0} = no pooled memory */
  int64_t topk;        /* routed windows per query window; 0 = no routing */
  double scale;        /* softmax scale on q.k (the caller passes 1/sqrt(d)) */
  int64_t radius;      /* routing candidates: -1 = every other window; r >= 0 =
                          windows at most r window steps away on every axis */
  int64_t global_tokens;  /* X extra global K/V rows after the pooled cells
                             (e.g. text tokens), attended by every window */
} bo_params;

int bo_check(const bo_params* p);

/* Derived sizes (valid only after bo_check returned BO_OK). */
int64_t bo_tokens(const bo_params* p);          /* N = T*H*W */
int64_t bo_windows(const bo_params* p);         /* nW */
int64_t bo_window_tokens(const bo_params* p);   /* M (slots of a full window) */
int64_t bo_window_real_tokens(const bo_params* p, int64_t w);  /* slots of window w */
int64_t bo_pooled_tokens(const bo_params* p);   /* G, 0 when pooling is off */
int64_t bo_keys_per_query(const bo_params* p);  /* M + G + X + topk*M (the most any list has) */

/* Window partition of one block: win_id[n], slot[n] for every token and the
 * inverse table tok[w*M + s] (-1 past a short window's slots).  Any of the
 * three outputs may be NULL. */
int bo_partition(const bo_params* p, int32_t* win_id, int32_t* slot, int32_t* tok);

/* Average-pooled memory: xp[b,h,c,:] = mean of x over pooling cell c. */
int bo_pool(const bo_params* p, const float* x, double* xp);

/* Routing: route[b,h,i,0..topk) and, if score != NULL, the full window-score
 * matrix score[b,h,i,j]. */
int bo_route(const bo_params* p, const float* q, const float* k,
             int32_t* route, double* score);

/* Full attention output for every query of every window. kp/vp are NULL iff
 * pooling is off; route is NULL iff topk == 0; lse may be NULL. */
int bo_attend(const bo_params* p, const float* q, const float* k, const float* v,
              const double* kp, const double* vp, const int32_t* route,
              double* out, double* lse);

/* Same as bo_attend for a list of query rows only: rows[r] = (b*H + h)*N + n.
 * out is [n_rows, d], lse (nullable) is [n_rows]. */
int bo_attend_rows(const bo_params* p, const float* q, const float* k, const float* v,
                   const double* kp, const double* vp, const int32_t* route,
                   int64_t n_rows, const int64_t* rows, double* out, double* lse);

/* The softmax row of one query over its key list, in key-list order
 * (local window, pooled cells, routed windows).  probs has room for
 * bo_keys_per_query(p) values; key_id (nullable) receives each key's source:
 * a token index n >= 0, or -1 - c for pooled cell c.  A list shorter than
 * bo_keys_per_query(p) (short windows) ends with probability 0 and key id
 * INT64_MIN. */
int bo_softmax_row(const bo_params* p, const float* q, const float* k,
                   const double* kp, const int32_t* route, int64_t row,
                   double* probs, int64_t* key_id);

/* Gradients of bo_attend's output for the incoming gradient dout [B, H, N, d]:
 * dq, dk, dv [B, H, N, d] and, when the key lists have global rows, dkg, dvg
 * [B, H, G + X, d] (the gradients of the pooled cells and extra rows).  dk and
 * dv include the pooled cells' share carried back through the mean (each
 * token of a cell receives the cell's gradient / cell size); dkg, dvg hold
 * the gradients of the global rows themselves.  Routing has no gradient. */
int bo_attend_bwd(const bo_params* p, const float* q, const float* k, const float* v,
                  const double* kp, const double* vp, const int32_t* route, const float* dout,
                  double* dq, double* dk, double* dv, double* dkg, double* dvg);

/* dq of selected query rows only: rows[r] = (b*H + h)*N + n, dq [n_rows, d]. */
int bo_attend_bwd_dq_rows(const bo_params* p, const float* q, const float* k, const float* v,
                          const double* kp, const double* vp, const int32_t* route,
                          const float* dout, int64_t n_rows, const int64_t* rows, double* dq);

/* Key gradients of window w's tokens for one bh = b*H + h from every query
 * whose key list holds them, before the pooled cells' share: dk, dv [M, d]
 * in slot order (rows past a short window's slots are zero). */
int bo_attend_bwd_window_keys(const bo_params* p, const float* q, const float* k, const float* v,
                              const double* kp, const double* vp, const int32_t* route,
                              const float* dout, int64_t bh, int64_t w, double* dk, double* dv);

/* Number of threads the attention loops use (OpenMP), for reporting. */
int bo_num_threads(void);

/* Sets the number of threads later calls use (n >= 1; no effect without
 * OpenMP). */
void bo_set_num_threads(int n);

#ifdef __cplusplus
}
#endif

#endif /* BASA_ORACLE_H */
