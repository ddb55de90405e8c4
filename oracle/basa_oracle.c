/*
 * basa_oracle.c -- plain CPU reference for BASA attention (TEST INFRASTRUCTURE).
 *
 * Only tests, the package smoke check and the benchmark's CPU-baseline leg use
 * this file.  It is deliberately slow and literal: one query at a time, one key
 * at a time, float64 throughout, no blocking, no fusion.
 *
 * Method source: BASA (arXiv 2610.08772v1) as summarised on the paperlayer.ai
 * page: shifted regular windows (sec. 3.1 and A.1), K/V-pooled global memory
 * (sec. 3.2, A.1), content-adaptive routed windows (sec. 3.3, A.2), one joint
 * softmax over the concatenated key list (A.1).  Readings of points the pages
 * leave open are stated at each function.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).
 */
#include "basa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ sizes */

static int pool_on(const bo_params* p) {
  return p->pool[0] != 0 || p->pool[1] != 0 || p->pool[2] != 0;
}

/* Windows along axis a: the grid padded up to a window multiple. */
static int64_t nwin(const bo_params* p, int a) {
  return (p->grid[a] + p->window[a] - 1) / p->window[a];
}

/* Real extent of window w along each axis: the window extent, except for the
 * last window along an axis the window does not divide, which keeps what is
 * left of the grid. */
static void win_extents(const bo_params* p, int64_t w, int64_t e[3]) {
  int64_t nwy = nwin(p, 1), nwx = nwin(p, 2);
  int64_t c[3] = {w / (nwy * nwx), (w / nwx) % nwy, w % nwx};
  for (int a = 0; a < 3; ++a) {
    int64_t last = nwin(p, a) - 1;
    e[a] = c[a] < last ? p->window[a] : p->grid[a] - last * p->window[a];
  }
}

/* Routing candidates (paperlayer.ai, A.2: for video the candidate-window
 * radius is one unless stated otherwise).  Reading: window j is a candidate
 * for window i when their coordinates in the window grid (a, b, c) =
 * (w / (nWy nWx), (w / nWx) mod nWy, w mod nWx) differ by at most radius on
 * every axis, compared as plain integers (the window grid does not wrap);
 * radius -1 makes every window a candidate. */
static int candidate(const bo_params* p, int64_t i, int64_t j) {
  if (p->radius < 0) return 1;
  int64_t nwy = nwin(p, 1), nwx = nwin(p, 2);
  int64_t ci[3] = {i / (nwy * nwx), (i / nwx) % nwy, i % nwx};
  int64_t cj[3] = {j / (nwy * nwx), (j / nwx) % nwy, j % nwx};
  for (int a = 0; a < 3; ++a) {
    int64_t dlt = ci[a] > cj[a] ? ci[a] - cj[a] : cj[a] - ci[a];
    if (dlt > p->radius) return 0;
  }
  return 1;
}

/* Validation.  The pages form windows by cyclic shift + reshape + permute
 * "for divisible resolutions" (paperlayer.ai, A.1); pooling cells must tile
 * the grid exactly.  A window extent that does not divide the grid is read as
 * padding the rolled grid up to a window multiple, where padding is not a
 * token: the last window along that axis holds only its real positions (see
 * token_of).  A window may not exceed the grid; the shift is a cyclic offset
 * in [0, grid). */
int bo_check(const bo_params* p) {
  if (!p) return BO_EINVAL;
  if (p->batch < 1 || p->heads < 1 || p->dim < 1) return BO_EINVAL;
  if (!(p->scale > 0.0) || !isfinite(p->scale)) return BO_EINVAL;
  for (int a = 0; a < 3; ++a) {
    if (p->grid[a] < 1 || p->window[a] < 1) return BO_EINVAL;
    if (p->window[a] > p->grid[a]) return BO_ERANGE;
    if (p->shift[a] < 0 || p->shift[a] >= p->grid[a]) return BO_ERANGE;
  }
  if (pool_on(p)) {
    for (int a = 0; a < 3; ++a) {
      if (p->pool[a] < 1) return BO_EINVAL;
      if (p->grid[a] % p->pool[a] != 0) return BO_ENOTDIV;
    }
  }
  int64_t nw = bo_windows(p);
  if (p->topk < 0 || p->topk > nw - 1) return BO_ERANGE;
  if (p->global_tokens < 0) return BO_EINVAL;
  if (p->radius < -1) return BO_EINVAL;
  if (p->topk > 0 && p->radius >= 0) {
    /* Every window needs topk candidates; count them for each window. */
    for (int64_t i = 0; i < nw; ++i) {
      int64_t n = 0;
      for (int64_t j = 0; j < nw; ++j)
        if (j != i && candidate(p, i, j)) ++n;
      if (n < p->topk) return BO_ERANGE;
    }
  }
  return BO_OK;
}

int64_t bo_tokens(const bo_params* p) { return p->grid[0] * p->grid[1] * p->grid[2]; }

int64_t bo_windows(const bo_params* p) { return nwin(p, 0) * nwin(p, 1) * nwin(p, 2); }

int64_t bo_window_real_tokens(const bo_params* p, int64_t w) {
  int64_t e[3];
  win_extents(p, w, e);
  return e[0] * e[1] * e[2];
}

int64_t bo_window_tokens(const bo_params* p) { return p->window[0] * p->window[1] * p->window[2]; }

int64_t bo_pooled_tokens(const bo_params* p) {
  if (!pool_on(p)) return 0;
  return (p->grid[0] / p->pool[0]) * (p->grid[1] / p->pool[1]) * (p->grid[2] / p->pool[2]);
}

int64_t bo_keys_per_query(const bo_params* p) {
  return bo_window_tokens(p) + bo_pooled_tokens(p) + p->global_tokens +
         p->topk * bo_window_tokens(p);
}

int bo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void bo_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* -------------------------------------------------------------- partition */

/* Token of slot s in window w (paperlayer.ai, A.1: cyclic shift, then a
 * reshape/permute into non-overlapping windows).  Reading: the grid is rolled
 * by -shift before it is cut, so window 0 begins at original coordinate
 * `shift` and windows that cross the grid edge wrap around (no mask).  The
 * slots of a window run over its real positions in raster order of
 * (t, y, x) inside the window; a short window (see win_extents) has fewer. */
static int64_t token_of(const bo_params* p, int64_t w, int64_t s) {
  int64_t nwy = nwin(p, 1), nwx = nwin(p, 2);
  int64_t wa = w / (nwy * nwx), wb = (w / nwx) % nwy, wc = w % nwx;
  int64_t e[3];
  win_extents(p, w, e);
  int64_t it = s / (e[1] * e[2]);
  int64_t iy = (s / e[2]) % e[1];
  int64_t ix = s % e[2];
  int64_t t = (wa * p->window[0] + it + p->shift[0]) % p->grid[0];
  int64_t y = (wb * p->window[1] + iy + p->shift[1]) % p->grid[1];
  int64_t x = (wc * p->window[2] + ix + p->shift[2]) % p->grid[2];
  return (t * p->grid[1] + y) * p->grid[2] + x;
}

int bo_partition(const bo_params* p, int32_t* win_id, int32_t* slot, int32_t* tok) {
  int rc = bo_check(p);
  if (rc) return rc;
  int64_t nw = bo_windows(p), m = bo_window_tokens(p);
  int64_t nwy = nwin(p, 1), nwx = nwin(p, 2);
  for (int64_t w = 0; w < nw; ++w) {
    int64_t mw = bo_window_real_tokens(p, w);
    for (int64_t s = 0; s < m; ++s) {
      int64_t n = s < mw ? token_of(p, w, s) : -1;
      if (tok) tok[w * m + s] = (int32_t)n;
    }
  }
  /* The inverse map is computed from its own formula (token -> shifted
   * coordinate -> window, slot), not by inverting tok. */
  int64_t N = bo_tokens(p);
  for (int64_t n = 0; n < N; ++n) {
    int64_t t = n / (p->grid[1] * p->grid[2]);
    int64_t y = (n / p->grid[2]) % p->grid[1];
    int64_t x = n % p->grid[2];
    int64_t ut = (t - p->shift[0] + p->grid[0]) % p->grid[0];
    int64_t uy = (y - p->shift[1] + p->grid[1]) % p->grid[1];
    int64_t ux = (x - p->shift[2] + p->grid[2]) % p->grid[2];
    int64_t w = ((ut / p->window[0]) * nwy + uy / p->window[1]) * nwx + ux / p->window[2];
    int64_t e[3];
    win_extents(p, w, e);
    int64_t s = ((ut % p->window[0]) * e[1] + uy % p->window[1]) * e[2] + ux % p->window[2];
    if (win_id) win_id[n] = (int32_t)w;
    if (slot) slot[n] = (int32_t)s;
  }
  return BO_OK;
}

/* ------------------------------------------------------------------- pool */

/* K/V-pooled global memory (paperlayer.ai, sec. 3.2 and A.1: a "regular
 * spatial reduction" by average pooling).  Readings: the unshifted grid is cut
 * into non-overlapping cells of size pool (stride = kernel); the cell's members
 * are summed in raster order and the sum is divided by the cell size. */
int bo_pool(const bo_params* p, const float* x, double* xp) {
  int rc = bo_check(p);
  if (rc) return rc;
  if (!pool_on(p) || !x || !xp) return BO_EINVAL;
  int64_t d = p->dim, N = bo_tokens(p), G = bo_pooled_tokens(p);
  int64_t gy = p->grid[1] / p->pool[1], gx = p->grid[2] / p->pool[2];
  int64_t cell = p->pool[0] * p->pool[1] * p->pool[2];
  int64_t bh_count = p->batch * p->heads;
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < bh_count; ++bh) {
    for (int64_t c = 0; c < G; ++c) {
      int64_t ct = c / (gy * gx), cy = (c / gx) % gy, cx = c % gx;
      double* dst = xp + (bh * G + c) * d;
      for (int64_t e = 0; e < d; ++e) dst[e] = 0.0;
      for (int64_t i = 0; i < p->pool[0]; ++i)
        for (int64_t j = 0; j < p->pool[1]; ++j)
          for (int64_t l = 0; l < p->pool[2]; ++l) {
            int64_t n = ((ct * p->pool[0] + i) * p->grid[1] + cy * p->pool[1] + j) * p->grid[2] +
                        cx * p->pool[2] + l;
            const float* src = x + (bh * N + n) * d;
            for (int64_t e = 0; e < d; ++e) dst[e] = dst[e] + (double)src[e];
          }
      for (int64_t e = 0; e < d; ++e) dst[e] = dst[e] / (double)cell;
    }
  }
  return BO_OK;
}

/* ------------------------------------------------------------------ route */

/* Content-adaptive routing (paperlayer.ai, sec. 3.3 and A.2: selected original
 * K/V windows are added to each window's context).  Readings: the routing unit
 * is the block's own local-window partition; the score of candidate window j
 * for query window i is the dot product of i's summed queries with j's summed
 * keys, per head (ranking by sums equals ranking by means); the window itself
 * is excluded; the top-k are ordered by score descending, then by smaller
 * window index; only candidates (see candidate()) are ranked.  Sums and dot
 * products run in float64 with separate multiply and add: a window's slots
 * are summed in slot order, the dot product runs in channel order.  (The
 * pages fix no summation order.  For bfloat16 inputs every window sum is
 * exact, whatever the order, while the inputs' exponent span plus log2 of
 * the window size fits float64's 53-bit significand; the tests check that
 * for their inputs.) */
int bo_route(const bo_params* p, const float* q, const float* k, int32_t* route, double* score) {
  int rc = bo_check(p);
  if (rc) return rc;
  if (!q || !k || (p->topk > 0 && !route)) return BO_EINVAL;
  int64_t d = p->dim, N = bo_tokens(p), nw = bo_windows(p), m = bo_window_tokens(p);
  int64_t bh_count = p->batch * p->heads, kk = p->topk;
  int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * nw * m);
  if (!tok) return BO_ENOMEM;
  bo_partition(p, NULL, NULL, tok);
  int fail = 0;
#pragma omp parallel for schedule(dynamic)
  for (int64_t bh = 0; bh < bh_count; ++bh) {
    double* sq = (double*)malloc(sizeof(double) * nw * d);
    double* sk = (double*)malloc(sizeof(double) * nw * d);
    double* sc = (double*)malloc(sizeof(double) * nw * nw);
    if (!sq || !sk || !sc) {
      free(sq); free(sk); free(sc);
#pragma omp atomic write
      fail = 1;
      continue;
    }
    for (int64_t w = 0; w < nw; ++w) {
      int64_t mw = bo_window_real_tokens(p, w);
      for (int64_t e = 0; e < d; ++e) {
        double aq = 0.0, ak = 0.0;
        for (int64_t s = 0; s < mw; ++s) {
          int64_t n = tok[w * m + s];
          aq = aq + (double)q[(bh * N + n) * d + e];
          ak = ak + (double)k[(bh * N + n) * d + e];
        }
        sq[w * d + e] = aq;
        sk[w * d + e] = ak;
      }
    }
    for (int64_t i = 0; i < nw; ++i)
      for (int64_t j = 0; j < nw; ++j) {
        double acc = 0.0;
        for (int64_t e = 0; e < d; ++e) {
          double prod = sq[i * d + e] * sk[j * d + e];
          acc = acc + prod;
        }
        sc[i * nw + j] = acc;
      }
    if (score) memcpy(score + bh * nw * nw, sc, sizeof(double) * nw * nw);
    /* Selection: repeatedly take the best remaining candidate. */
    for (int64_t i = 0; i < nw && kk > 0; ++i) {
      int32_t* out = route + (bh * nw + i) * kk;
      for (int64_t r = 0; r < kk; ++r) {
        int64_t best = -1;
        for (int64_t j = 0; j < nw; ++j) {
          if (j == i || !candidate(p, i, j)) continue;
          int taken = 0;
          for (int64_t u = 0; u < r; ++u) if (out[u] == j) taken = 1;
          if (taken) continue;
          if (best < 0 || sc[i * nw + j] > sc[i * nw + best]) best = j;  /* ties keep smaller j */
        }
        out[r] = (int32_t)best;
      }
    }
    free(sq); free(sk); free(sc);
  }
  free(tok);
  return fail ? BO_ENOMEM : BO_OK;
}

/* -------------------------------------------------------------- attention */

typedef struct {
  const bo_params* p;
  const float *q, *k, *v;
  const double *kp, *vp;
  const int32_t* route;
  const int32_t* tok;      /* [nW, M] */
  const int32_t* win_id;   /* [N] */
  int64_t N, M, G, L, d, nw;
} att_ctx;

/* Source of key j of window w's key list: the list is the window's own tokens
 * in slot order, then the G pooled cells, then each routed window's tokens in
 * slot order (paperlayer.ai, A.1: one softmax over the concatenated K/V).
 * Returns a token index, or -1 - c for pooled cell c. */
static int64_t key_source(const att_ctx* c, int64_t bh, int64_t w, int64_t j) {
  int64_t mw = bo_window_real_tokens(c->p, w);
  if (j < mw) return c->tok[w * c->M + j];
  j -= mw;
  if (j < c->G) return -1 - j;
  j -= c->G;
  for (int64_t r = 0; r < c->p->topk; ++r) {
    int64_t rw = c->route[(bh * c->nw + w) * c->p->topk + r];
    int64_t mr = bo_window_real_tokens(c->p, rw);
    if (j < mr) return c->tok[rw * c->M + j];
    j -= mr;
  }
  return INT64_MIN;  /* past the list: not reached */
}

/* Length of window w's key list. */
static int64_t list_len(const att_ctx* c, int64_t bh, int64_t w) {
  int64_t len = bo_window_real_tokens(c->p, w) + c->G;
  for (int64_t r = 0; r < c->p->topk; ++r)
    len += bo_window_real_tokens(c->p, c->route[(bh * c->nw + w) * c->p->topk + r]);
  return len;
}

/* One query: z_j = scale * q.k_j over the key list, p = softmax(z),
 * o = sum_j p_j v_j, lse = log sum_j exp(z_j).  z has room for L values. */
static void attend_one(const att_ctx* c, int64_t bh, int64_t n, double* z, double* o,
                       double* lse, double* probs, int64_t* key_id) {
  int64_t d = c->d, w = c->win_id[n], L = list_len(c, bh, w);
  const float* qr = c->q + (bh * c->N + n) * d;
  double zmax = -INFINITY;
  for (int64_t j = 0; j < L; ++j) {
    int64_t src = key_source(c, bh, w, j);
    double dot = 0.0;
    if (src >= 0) {
      const float* kr = c->k + (bh * c->N + src) * d;
      for (int64_t e = 0; e < d; ++e) dot = dot + (double)qr[e] * (double)kr[e];
    } else {
      const double* kr = c->kp + (bh * c->G + (-1 - src)) * d;
      for (int64_t e = 0; e < d; ++e) dot = dot + (double)qr[e] * kr[e];
    }
    z[j] = c->p->scale * dot;
    if (z[j] > zmax) zmax = z[j];
    if (key_id) key_id[j] = src;
  }
  double l = 0.0;
  for (int64_t j = 0; j < L; ++j) {
    z[j] = exp(z[j] - zmax);
    l = l + z[j];
  }
  if (probs) {
    for (int64_t j = 0; j < L; ++j) probs[j] = z[j] / l;
    for (int64_t j = L; j < c->L; ++j) probs[j] = 0.0;
  }
  if (key_id)
    for (int64_t j = L; j < c->L; ++j) key_id[j] = INT64_MIN;
  if (o) {
    for (int64_t e = 0; e < d; ++e) o[e] = 0.0;
    for (int64_t j = 0; j < L; ++j) {
      int64_t src = key_source(c, bh, w, j);
      if (src >= 0) {
        const float* vr = c->v + (bh * c->N + src) * d;
        for (int64_t e = 0; e < d; ++e) o[e] = o[e] + z[j] * (double)vr[e];
      } else {
        const double* vr = c->vp + (bh * c->G + (-1 - src)) * d;
        for (int64_t e = 0; e < d; ++e) o[e] = o[e] + z[j] * vr[e];
      }
    }
    for (int64_t e = 0; e < d; ++e) o[e] = o[e] / l;
  }
  if (lse) *lse = zmax + log(l);
}

static int ctx_init(att_ctx* c, const bo_params* p, const float* q, const float* k,
                    const float* v, const double* kp, const double* vp, const int32_t* route,
                    int need_v) {
  int rc = bo_check(p);
  if (rc) return rc;
  if (!q || !k || (need_v && !v)) return BO_EINVAL;
  if ((pool_on(p) || p->global_tokens > 0) && (!kp || (need_v && !vp))) return BO_EINVAL;
  if (p->topk > 0 && !route) return BO_EINVAL;
  memset(c, 0, sizeof(*c));
  c->p = p; c->q = q; c->k = k; c->v = v; c->kp = kp; c->vp = vp; c->route = route;
  /* The global part of every key list: the pooled cells, then the extra
   * global rows (paperlayer.ai A.1: text and global memory in one branch). */
  c->N = bo_tokens(p); c->M = bo_window_tokens(p); c->G = bo_pooled_tokens(p) + p->global_tokens;
  c->L = bo_keys_per_query(p); c->d = p->dim; c->nw = bo_windows(p);
  int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * c->nw * c->M);
  int32_t* wid = (int32_t*)malloc(sizeof(int32_t) * c->N);
  if (!tok || !wid) { free(tok); free(wid); return BO_ENOMEM; }
  bo_partition(p, wid, NULL, tok);
  c->tok = tok; c->win_id = wid;
  return BO_OK;
}

static void ctx_free(att_ctx* c) {
  free((void*)c->tok);
  free((void*)c->win_id);
}

int bo_attend(const bo_params* p, const float* q, const float* k, const float* v,
              const double* kp, const double* vp, const int32_t* route, double* out,
              double* lse) {
  att_ctx c;
  int rc = ctx_init(&c, p, q, k, v, kp, vp, route, 1);
  if (rc) return rc;
  if (!out) { ctx_free(&c); return BO_EINVAL; }
  int64_t tasks = p->batch * p->heads * c.nw;
  int fail = 0;
#pragma omp parallel for schedule(dynamic)
  for (int64_t t = 0; t < tasks; ++t) {
    int64_t bh = t / c.nw, w = t % c.nw;
    double* z = (double*)malloc(sizeof(double) * c.L);
    if (!z) {
#pragma omp atomic write
      fail = 1;
      continue;
    }
    for (int64_t s = 0; s < bo_window_real_tokens(p, w); ++s) {
      int64_t n = c.tok[w * c.M + s];
      attend_one(&c, bh, n, z, out + (bh * c.N + n) * c.d, lse ? lse + bh * c.N + n : NULL,
                 NULL, NULL);
    }
    free(z);
  }
  ctx_free(&c);
  return fail ? BO_ENOMEM : BO_OK;
}

int bo_attend_rows(const bo_params* p, const float* q, const float* k, const float* v,
                   const double* kp, const double* vp, const int32_t* route, int64_t n_rows,
                   const int64_t* rows, double* out, double* lse) {
  att_ctx c;
  int rc = ctx_init(&c, p, q, k, v, kp, vp, route, 1);
  if (rc) return rc;
  if (!out || (n_rows > 0 && !rows)) { ctx_free(&c); return BO_EINVAL; }
  int64_t total = p->batch * p->heads * c.N;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= total) { ctx_free(&c); return BO_ERANGE; }
  int fail = 0;
#pragma omp parallel for schedule(dynamic)
  for (int64_t r = 0; r < n_rows; ++r) {
    double* z = (double*)malloc(sizeof(double) * c.L);
    if (!z) {
#pragma omp atomic write
      fail = 1;
      continue;
    }
    int64_t bh = rows[r] / c.N, n = rows[r] % c.N;
    attend_one(&c, bh, n, z, out + r * c.d, lse ? lse + r : NULL, NULL, NULL);
    free(z);
  }
  ctx_free(&c);
  return fail ? BO_ENOMEM : BO_OK;
}

int bo_softmax_row(const bo_params* p, const float* q, const float* k, const double* kp,
                   const int32_t* route, int64_t row, double* probs, int64_t* key_id) {
  att_ctx c;
  int rc = ctx_init(&c, p, q, k, NULL, kp, NULL, route, 0);
  if (rc) return rc;
  if (!probs || row < 0 || row >= p->batch * p->heads * c.N) { ctx_free(&c); return BO_EINVAL; }
  double* z = (double*)malloc(sizeof(double) * c.L);
  if (!z) { ctx_free(&c); return BO_ENOMEM; }
  attend_one(&c, row / c.N, row % c.N, z, NULL, NULL, probs, key_id);
  free(z);
  ctx_free(&c);
  return BO_OK;
}

/* --------------------------------------------------------------- backward */

/* Gradients of the attention output (paperlayer.ai, sec. 3.4 adapts the sparse
 * model by training, which differentiates this operator).  For every query n
 * with key list K_L, V_L and P = softmax(z), z_j = scale q_n.k_j, and the
 * incoming gradient g = dO_n:
 *   dV_j += P_j g                  dP_j = g.v_j
 *   dS_j  = P_j (dP_j - sum_i P_i dP_i)
 *   dq_n  = scale sum_j dS_j k_j    dK_j += scale dS_j q_n
 * Keys are token rows (dk, dv) or global rows (dkg, dvg: the pooled cells,
 * then the extra rows).  The pooled cells' gradients are then carried back
 * to the tokens of their cell, each receiving dkg_c / P (the mean's
 * derivative).  Routing is a selection and has no gradient.  All float64,
 * one query at a time; the key gradients are accumulated serially. */
/* One query's part of the backward: dq_n into dqr, and, when dk is not NULL,
 * its contributions to the key gradients.  keys_of < 0: every key, dk/dv
 * [B*H, N, d] and dkg/dvg [B*H, G, d].  keys_of = w >= 0: only the token keys
 * of window w, into dk/dv [M, d] at their slots (slot[] maps token -> slot).
 * z, dp, src have room for c->L. */
static void bwd_one(const att_ctx* c, const bo_params* p, int64_t bh, int64_t n,
                    const float* q, const float* k, const float* v, const double* kp,
                    const double* vp, const float* dout, double* z, double* dp, int64_t* src,
                    double* dqr, double* dk, double* dv, double* dkg, double* dvg,
                    int64_t keys_of, const int32_t* slot) {
  int64_t d = c->d, N = c->N, G = c->G;
  int64_t w = c->win_id[n], L = list_len(c, bh, w);
  attend_one(c, bh, n, z, NULL, NULL, z, src);  /* z <- probabilities P */
  const float* g = dout + (bh * N + n) * d;
  const float* qr = q + (bh * N + n) * d;
  double dsum = 0.0;
  for (int64_t j = 0; j < L; ++j) {
    const double* vg = NULL;
    const float* vr = NULL;
    if (src[j] >= 0) vr = v + (bh * N + src[j]) * d;
    else vg = vp + (bh * G + (-1 - src[j])) * d;
    double acc = 0.0;
    for (int64_t e = 0; e < d; ++e) acc = acc + (double)g[e] * (vr ? (double)vr[e] : vg[e]);
    dp[j] = acc;
    dsum = dsum + z[j] * acc;
  }
  for (int64_t e = 0; e < d; ++e) dqr[e] = 0.0;
  for (int64_t j = 0; j < L; ++j) {
    double ds = z[j] * (dp[j] - dsum);
    double* dkr = NULL;
    double* dvr = NULL;
    const double* kg = NULL;
    const float* kr = NULL;
    if (src[j] >= 0) {
      kr = k + (bh * N + src[j]) * d;
      if (dk && keys_of < 0) {
        dkr = dk + (bh * N + src[j]) * d;
        dvr = dv + (bh * N + src[j]) * d;
      } else if (dk && c->win_id[src[j]] == keys_of) {
        dkr = dk + (int64_t)slot[src[j]] * d;
        dvr = dv + (int64_t)slot[src[j]] * d;
      }
    } else {
      kg = kp + (bh * G + (-1 - src[j])) * d;
      if (dk && keys_of < 0) {
        dkr = dkg + (bh * G + (-1 - src[j])) * d;
        dvr = dvg + (bh * G + (-1 - src[j])) * d;
      }
    }
    for (int64_t e = 0; e < d; ++e) {
      dqr[e] = dqr[e] + p->scale * ds * (kr ? (double)kr[e] : kg[e]);
      if (dkr) {
        dkr[e] = dkr[e] + p->scale * ds * (double)qr[e];
        dvr[e] = dvr[e] + z[j] * (double)g[e];
      }
    }
  }
}

int bo_attend_bwd(const bo_params* p, const float* q, const float* k, const float* v,
                  const double* kp, const double* vp, const int32_t* route, const float* dout,
                  double* dq, double* dk, double* dv, double* dkg, double* dvg) {
  att_ctx c;
  int rc = ctx_init(&c, p, q, k, v, kp, vp, route, 1);
  if (rc) return rc;
  if (!dout || !dq || !dk || !dv || (c.G > 0 && (!dkg || !dvg))) { ctx_free(&c); return BO_EINVAL; }
  int64_t d = c.d, N = c.N, G = c.G, BH = p->batch * p->heads;
  memset(dk, 0, sizeof(double) * BH * N * d);
  memset(dv, 0, sizeof(double) * BH * N * d);
  if (G > 0) {
    memset(dkg, 0, sizeof(double) * BH * G * d);
    memset(dvg, 0, sizeof(double) * BH * G * d);
  }
  double* z = (double*)malloc(sizeof(double) * c.L);
  double* dp = (double*)malloc(sizeof(double) * c.L);
  int64_t* src = (int64_t*)malloc(sizeof(int64_t) * c.L);
  if (!z || !dp || !src) { free(z); free(dp); free(src); ctx_free(&c); return BO_ENOMEM; }
  for (int64_t bh = 0; bh < BH; ++bh)
    for (int64_t n = 0; n < N; ++n)
      bwd_one(&c, p, bh, n, q, k, v, kp, vp, dout, z, dp, src, dq + (bh * N + n) * d, dk, dv,
              dkg, dvg, -1, NULL);
  free(z); free(dp); free(src);
  /* The pooled cells' share of dK, dV goes back to their tokens. */
  if (pool_on(p)) {
    int64_t Gp = bo_pooled_tokens(p);
    int64_t gy = p->grid[1] / p->pool[1], gx = p->grid[2] / p->pool[2];
    int64_t cell = p->pool[0] * p->pool[1] * p->pool[2];
    for (int64_t bh = 0; bh < BH; ++bh)
      for (int64_t cc = 0; cc < Gp; ++cc) {
        int64_t ct = cc / (gy * gx), cy = (cc / gx) % gy, cx = cc % gx;
        for (int64_t i = 0; i < p->pool[0]; ++i)
          for (int64_t jj = 0; jj < p->pool[1]; ++jj)
            for (int64_t l = 0; l < p->pool[2]; ++l) {
              int64_t n = ((ct * p->pool[0] + i) * p->grid[1] + cy * p->pool[1] + jj) * p->grid[2] +
                          cx * p->pool[2] + l;
              for (int64_t e = 0; e < d; ++e) {
                dk[(bh * N + n) * d + e] += dkg[(bh * G + cc) * d + e] / (double)cell;
                dv[(bh * N + n) * d + e] += dvg[(bh * G + cc) * d + e] / (double)cell;
              }
            }
      }
  }
  ctx_free(&c);
  return BO_OK;
}

/* dq of selected query rows only (rows[r] = (b*H + h)*N + n): each query's
 * dq depends on its own key list alone, so a row is computed exactly as in
 * bo_attend_bwd. */
int bo_attend_bwd_dq_rows(const bo_params* p, const float* q, const float* k, const float* v,
                          const double* kp, const double* vp, const int32_t* route,
                          const float* dout, int64_t n_rows, const int64_t* rows, double* dq) {
  att_ctx c;
  int rc = ctx_init(&c, p, q, k, v, kp, vp, route, 1);
  if (rc) return rc;
  if (!dout || !dq || (n_rows > 0 && !rows)) { ctx_free(&c); return BO_EINVAL; }
  int64_t total = p->batch * p->heads * c.N;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= total) { ctx_free(&c); return BO_ERANGE; }
  int fail = 0;
#pragma omp parallel for schedule(dynamic)
  for (int64_t r = 0; r < n_rows; ++r) {
    double* z = (double*)malloc(sizeof(double) * c.L);
    double* dp = (double*)malloc(sizeof(double) * c.L);
    int64_t* src = (int64_t*)malloc(sizeof(int64_t) * c.L);
    if (z && dp && src)
      bwd_one(&c, p, rows[r] / c.N, rows[r] % c.N, q, k, v, kp, vp, dout, z, dp, src,
              dq + r * c.d, NULL, NULL, NULL, NULL, -1, NULL);
    else {
#pragma omp atomic write
      fail = 1;
    }
    free(z); free(dp); free(src);
  }
  ctx_free(&c);
  return fail ? BO_ENOMEM : BO_OK;
}

/* The key gradients of window w's tokens for one (b, h) = bh, from every
 * query whose key list holds them (the queries of w and of every window that
 * routed w), before the pooled cells' share is added: dk, dv [M, d] in slot
 * order, rows past a short window's slots zero.  Each query's terms are
 * exactly those of bo_attend_bwd. */
int bo_attend_bwd_window_keys(const bo_params* p, const float* q, const float* k, const float* v,
                              const double* kp, const double* vp, const int32_t* route,
                              const float* dout, int64_t bh, int64_t w, double* dk, double* dv) {
  att_ctx c;
  int rc = ctx_init(&c, p, q, k, v, kp, vp, route, 1);
  if (rc) return rc;
  if (!dout || !dk || !dv) { ctx_free(&c); return BO_EINVAL; }
  if (bh < 0 || bh >= p->batch * p->heads || w < 0 || w >= c.nw) { ctx_free(&c); return BO_ERANGE; }
  int32_t* slot = (int32_t*)malloc(sizeof(int32_t) * c.N);
  if (!slot) { ctx_free(&c); return BO_ENOMEM; }
  rc = bo_partition(p, NULL, slot, NULL);
  if (rc) { free(slot); ctx_free(&c); return rc; }
  /* Every query whose key list holds window w's tokens adds its terms; the
   * queries are independent, so threads take them in fixed turns (chunks of
   * 64 in token order) into private copies of the window's dK, dV, which
   * are then added in thread order. */
  int nthr = 1;
#ifdef _OPENMP
  nthr = omp_get_max_threads();
#endif
  const int64_t md = c.M * c.d;
  double* part = (double*)calloc((size_t)(2 * md * nthr), sizeof(double));
  if (!part) { free(slot); ctx_free(&c); return BO_ENOMEM; }
  int fail = 0;
#pragma omp parallel num_threads(nthr)
  {
    int t = 0;
#ifdef _OPENMP
    t = omp_get_thread_num();
#endif
    double* z = (double*)malloc(sizeof(double) * c.L);
    double* dp = (double*)malloc(sizeof(double) * c.L);
    int64_t* src = (int64_t*)malloc(sizeof(int64_t) * c.L);
    double* dq = (double*)malloc(sizeof(double) * c.d);
    const int ok = z && dp && src && dq;
    if (!ok) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(static, 64)
    for (int64_t n = 0; n < c.N; ++n) {
      if (!ok) continue;
      int64_t wn = c.win_id[n];
      int holds = wn == w;
      for (int64_t r = 0; r < p->topk && !holds; ++r)
        holds = route[(bh * c.nw + wn) * p->topk + r] == w;
      if (holds)
        bwd_one(&c, p, bh, n, q, k, v, kp, vp, dout, z, dp, src, dq, part + 2 * md * t,
                part + 2 * md * t + md, NULL, NULL, w, slot);
    }
    free(z); free(dp); free(src); free(dq);
  }
  for (int64_t i = 0; i < md; ++i) { dk[i] = 0.0; dv[i] = 0.0; }
  for (int t = 0; t < nthr; ++t)
    for (int64_t i = 0; i < md; ++i) {
      dk[i] = dk[i] + part[2 * md * t + i];
      dv[i] = dv[i] + part[2 * md * t + md + i];
    }
  free(part); free(slot);
  ctx_free(&c);
  return fail ? BO_ENOMEM : BO_OK;
}
