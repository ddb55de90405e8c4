// plan.cpp -- basa_plan: parameter validation and derived geometry (host only).
//
// The partition follows the BASA summary on paperlayer.ai (A.1): windows are
// formed by a cyclic shift, reshape and permute of the grid.  Pooling cells
// must tile the grid exactly.  A window extent that does not divide the grid
// leaves the last window along that axis short (padding read as "not a
// token": the short window holds only the real positions).
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <new>

#include "basa_internal.hpp"

namespace basa {

namespace {
thread_local char g_error[512] = "";
constexpr int kMaxTopk = 16;
constexpr int kMaxRouteWindows = 8192;
constexpr int64_t kMaxTokens = int64_t(1) << 24;
constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;

}  // namespace

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
}

const char* last_error() { return g_error; }

static basa_status fail(basa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return s;
}

static basa_status build(const basa_params& p, basa_plan_s& out) {
  if (p.batch < 1 || p.heads < 1) return fail(BASA_ERR_INVALID_ARGUMENT, "batch and heads must be >= 1");
  if (p.head_dim != 64 && p.head_dim != 128)
    return fail(BASA_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128 are implemented", p.head_dim);
  if (p.dtype != BASA_BF16 && p.dtype != BASA_F32)
    return fail(BASA_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)p.dtype);
  for (int a = 0; a < 3; ++a) {
    if (p.grid[a] < 1 || p.window[a] < 1)
      return fail(BASA_ERR_INVALID_ARGUMENT, "grid and window extents must be >= 1 (axis %d)", a);
    if (p.window[a] > p.grid[a])
      return fail(BASA_ERR_INVALID_ARGUMENT, "window %d exceeds grid %d on axis %d",
                  p.window[a], p.grid[a], a);
    if (p.shift[a] < 0 || p.shift[a] >= p.grid[a])
      return fail(BASA_ERR_INVALID_ARGUMENT, "shift %d outside [0, %d) on axis %d", p.shift[a],
                  p.grid[a], a);
  }
  const bool pool_on = p.pool[0] != 0 || p.pool[1] != 0 || p.pool[2] != 0;
  if (pool_on) {
    for (int a = 0; a < 3; ++a) {
      if (p.pool[a] < 1) return fail(BASA_ERR_INVALID_ARGUMENT, "pool extent must be >= 1 (axis %d)", a);
      if (p.grid[a] % p.pool[a] != 0)
        return fail(BASA_ERR_NOT_DIVISIBLE, "pool %d does not divide grid %d on axis %d",
                    p.pool[a], p.grid[a], a);
    }
  }
  const int64_t N = int64_t(p.grid[0]) * p.grid[1] * p.grid[2];
  if (N > kMaxTokens) return fail(BASA_ERR_UNSUPPORTED, "%lld tokens exceed 2^24", (long long)N);
  const int64_t BH = int64_t(p.batch) * p.heads;
  if (BH * N * p.head_dim > kMaxElems)
    return fail(BASA_ERR_UNSUPPORTED, "a [B,H,N,d] tensor exceeds 2^31 elements");
  auto cdiv = [](int64_t a, int64_t b) { return (a + b - 1) / b; };
  const int64_t nWt = cdiv(p.grid[0], p.window[0]), nWy = cdiv(p.grid[1], p.window[1]),
                nWx = cdiv(p.grid[2], p.window[2]);
  const int64_t nW = nWt * nWy * nWx;
  const int64_t M = int64_t(p.window[0]) * p.window[1] * p.window[2];
  if (p.route_topk < 0 || p.route_topk > nW - 1)
    return fail(BASA_ERR_INVALID_ARGUMENT, "route_topk %d outside [0, nW-1 = %lld]", p.route_topk,
                (long long)(nW - 1));
  if (p.route_topk > kMaxTopk)
    return fail(BASA_ERR_UNSUPPORTED, "route_topk %d exceeds %d", p.route_topk, kMaxTopk);
  if (p.route_topk > 0 && nW > kMaxRouteWindows)
    return fail(BASA_ERR_UNSUPPORTED, "routing over %lld windows exceeds %d", (long long)nW,
                kMaxRouteWindows);
  if (p.route_radius < -1)
    return fail(BASA_ERR_INVALID_ARGUMENT, "route_radius %d: -1 (every window) or >= 0",
                p.route_radius);
  if (p.route_topk > 0 && p.route_radius >= 0) {
    // A corner window has the fewest candidates (the window grid does not wrap).
    const int64_t r = p.route_radius;
    const int64_t fewest =
        (std::min(r, nWt - 1) + 1) * (std::min(r, nWy - 1) + 1) * (std::min(r, nWx - 1) + 1) - 1;
    if (p.route_topk > fewest)
      return fail(BASA_ERR_INVALID_ARGUMENT,
                  "route_topk %d exceeds the %lld candidates within radius %d of a corner window",
                  p.route_topk, (long long)fewest, p.route_radius);
  }
  if (p.global_tokens < 0)
    return fail(BASA_ERR_INVALID_ARGUMENT, "global_tokens %d must be >= 0", p.global_tokens);
  float scale = p.softmax_scale;
  if (scale == 0.0f) scale = 1.0f / std::sqrt(float(p.head_dim));
  if (!(scale > 0.0f) || !std::isfinite(scale))
    return fail(BASA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");

  Geom& g = out.g;
  g.T = p.grid[0]; g.Hg = p.grid[1]; g.Wg = p.grid[2];
  g.wt = p.window[0]; g.wh = p.window[1]; g.ww = p.window[2];
  g.st = p.shift[0]; g.sy = p.shift[1]; g.sx = p.shift[2];
  g.nWt = int32_t(nWt); g.nWy = int32_t(nWy); g.nWx = int32_t(nWx);
  g.rt = int32_t(g.T - (nWt - 1) * g.wt);
  g.ry = int32_t(g.Hg - (nWy - 1) * g.wh);
  g.rx = int32_t(g.Wg - (nWx - 1) * g.ww);
  g.padded = (g.rt != g.wt || g.ry != g.wh || g.rx != g.ww) ? 1 : 0;
  g.pt = pool_on ? p.pool[0] : 1; g.ph = pool_on ? p.pool[1] : 1; g.pw = pool_on ? p.pool[2] : 1;
  g.gt = g.T / g.pt; g.gy = g.Hg / g.ph; g.gx = g.Wg / g.pw;
  const int64_t Gp = pool_on ? int64_t(g.gt) * g.gy * g.gx : 0;
  const int64_t G = Gp + p.global_tokens;  // every global row, pooled and extra
  const int64_t L = M + G + int64_t(p.route_topk) * M;
  if (L > kMaxTokens) return fail(BASA_ERR_UNSUPPORTED, "%lld keys per query exceed 2^24", (long long)L);
  g.N = int32_t(N); g.M = int32_t(M); g.nW = int32_t(nW); g.G = int32_t(G); g.Gp = int32_t(Gp);
  g.L = int32_t(L); g.topk = p.route_topk; g.D = p.head_dim; g.BH = int32_t(BH);
  g.radius = p.route_radius;

  const int64_t whw = int64_t(g.wh) * g.ww, HWg = int64_t(g.Hg) * g.Wg;
  const int64_t cell_yx = int64_t(g.ph) * g.pw, gyx = int64_t(g.gy) * g.gx;
  g.f_wt = make_fastdiv(g.wt); g.f_wh = make_fastdiv(g.wh); g.f_ww = make_fastdiv(g.ww);
  g.f_whw = make_fastdiv(uint32_t(whw));
  g.f_nwx = make_fastdiv(g.nWx); g.f_nwyx = make_fastdiv(uint32_t(nWy * nWx));
  g.f_Wg = make_fastdiv(g.Wg); g.f_HWg = make_fastdiv(uint32_t(HWg));
  g.f_M = make_fastdiv(uint32_t(M));
  g.f_pw = make_fastdiv(g.pw); g.f_phw = make_fastdiv(uint32_t(cell_yx));
  g.f_gx = make_fastdiv(g.gx); g.f_gyx = make_fastdiv(uint32_t(gyx));
  g.f_rx = make_fastdiv(g.rx);
  g.f_ryw = make_fastdiv(uint32_t(g.ry * g.ww));
  g.f_whr = make_fastdiv(uint32_t(g.wh * g.rx));
  g.f_ryr = make_fastdiv(uint32_t(g.ry * g.rx));

  out.params = p;
  out.params.softmax_scale = scale;
  out.pool_on = pool_on;
  out.global_on = G > 0;
  out.scale = scale;
  // Route workspace: float64 window sums of q and of k, [2, B*H, nW, d], then
  // the sums of 128-slot chunks of each window, [2, B*H, nW, ceil(M/128), d],
  // then the window sums of k channel-major, [B*H, d, nW].
  out.route_ws_bytes = p.route_topk > 0 ? BH * nW * p.head_dim * int64_t(sizeof(double)) *
                                              (2 * (1 + (M + 127) / 128) + 1)
                                        : 0;

  out.bwd_ws_bytes = int64_t(bwd_workspace_bytes(out));
  out.split_ws_bytes = int64_t(split_workspace_bytes(out));
  // Text queries: the key list (N image tokens, then X text rows) is cut into
  // parts so that the (query tile, part, head) workgroups fill about one
  // round of the compute units, each part at least 512 keys; the parts'
  // results are merged by their log-sum-exps.
  out.text_split = 1;
  out.text_split_len = int32_t(N + p.global_tokens);
  out.text_ws_bytes = 0;
  if (p.global_tokens > 0) {
    const int64_t X = p.global_tokens, total = N + X;
    const int64_t work = (X + kAttnQueryTile - 1) / kAttnQueryTile * BH;
    int64_t parts = work < kComputeUnits ? kComputeUnits / work : 1;
    parts = std::max<int64_t>(1, std::min<int64_t>(parts, total / 512));
    const int64_t len = ((total + parts - 1) / parts + 63) / 64 * 64;
    parts = (total + len - 1) / len;
    out.text_split = int32_t(parts);
    out.text_split_len = int32_t(len);
    const int64_t elem = p.dtype == BASA_F32 ? 4 : 2;
    auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
    if (parts > 1)
      out.text_ws_bytes = al(parts * BH * X * p.head_dim * elem) + al(parts * BH * X * 4);
  }

  basa_plan_info& in = out.info;
  in.n_tokens = N;
  in.n_windows = nW;
  in.window_tokens = M;
  in.pooled_tokens = Gp;
  in.global_tokens = p.global_tokens;
  in.bwd_workspace_bytes = out.bwd_ws_bytes;
  in.split_workspace_bytes = out.split_ws_bytes;
  in.text_splits = out.text_split;
  in.text_workspace_bytes = out.text_ws_bytes;
  in.keys_per_query = L;
  in.route_workspace_bytes = out.route_ws_bytes;
  // Pairs: sum over windows of M_w * (M_w + G) plus, per query, topk routed
  // windows.  With short windows a routed window may hold fewer than M keys;
  // the routed part is then counted at M keys each (an upper bound: which
  // windows are routed is known only at run time).  sum_w M_w^2 factors over
  // the axes because window extents do.
  double own_sq = 1.0;
  for (int a = 0; a < 3; ++a) {
    const double w = p.window[a], nwa = double((p.grid[a] + p.window[a] - 1) / p.window[a]);
    const double r = p.grid[a] - (nwa - 1) * w;
    own_sq *= (nwa - 1) * w * w + r * r;
  }
  in.pairs_sparse = double(BH) * (own_sq + double(N) * double(G) +
                                  double(N) * double(p.route_topk) * double(M));
  in.pairs_dense = double(BH) * double(N) * double(N);
  in.flops_sparse = 4.0 * p.head_dim * in.pairs_sparse;
  in.flops_dense = 4.0 * p.head_dim * in.pairs_dense;
  return BASA_OK;
}

}  // namespace basa

extern "C" {

basa_status basa_plan(const basa_params* params, basa_plan_t* plan) {
  if (!params || !plan) return basa::fail(BASA_ERR_INVALID_ARGUMENT, "null params or plan pointer");
  basa_plan_s tmp{};
  basa_status st = basa::build(*params, tmp);
  if (st != BASA_OK) return st;
  basa_plan_s* p = new (std::nothrow) basa_plan_s(tmp);
  if (!p) return basa::fail(BASA_ERR_OUT_OF_MEMORY, "plan allocation failed");
  *plan = p;
  basa::set_error("%s", "");
  return BASA_OK;
}

void basa_plan_destroy(basa_plan_t plan) { delete plan; }

basa_status basa_plan_get_info(basa_plan_t plan, basa_plan_info* info) {
  if (!plan || !info) return basa::fail(BASA_ERR_INVALID_ARGUMENT, "null plan or info pointer");
  *info = plan->info;
  return BASA_OK;
}

basa_status basa_plan_pairs(basa_plan_t plan, const int32_t* route, double* pairs,
                            double* flops) {
  if (!plan || !pairs) return basa::fail(BASA_ERR_INVALID_ARGUMENT, "null plan or pairs pointer");
  const basa::Geom& g = plan->g;
  const int32_t K = plan->params.route_topk;
  if ((K > 0) != (route != nullptr))
    return basa::fail(BASA_ERR_INVALID_ARGUMENT,
                      K > 0 ? "the plan routes: route is required" : "route given but the plan does not route");
  // Real tokens of window w: the window extent on each axis, except the last
  // window along an axis the window does not divide.
  auto real_tokens = [&](int64_t w) {
    const int64_t a = w / (int64_t(g.nWy) * g.nWx), b = (w / g.nWx) % g.nWy, c = w % g.nWx;
    return int64_t(a + 1 < g.nWt ? g.wt : g.rt) * (b + 1 < g.nWy ? g.wh : g.ry) *
           (c + 1 < g.nWx ? g.ww : g.rx);
  };
  double total = 0.0;
  for (int64_t bh = 0; bh < g.BH; ++bh) {
    for (int64_t w = 0; w < g.nW; ++w) {
      const int64_t mw = real_tokens(w);
      int64_t keys = mw + g.G;
      for (int32_t r = 0; r < K; ++r) {
        const int32_t j = route[(bh * g.nW + w) * K + r];
        if (j < 0 || j >= g.nW)
          return basa::fail(BASA_ERR_INVALID_ARGUMENT,
                            "route[%lld][%lld][%d] = %d is outside [0, %d)", (long long)bh,
                            (long long)w, r, j, g.nW);
        keys += real_tokens(j);
      }
      total += double(mw) * double(keys);
    }
  }
  *pairs = total;
  if (flops) *flops = 4.0 * plan->params.head_dim * total;
  basa::set_error("%s", "");
  return BASA_OK;
}

basa_status basa_shift_schedule(const int32_t window[3], int32_t layer, int32_t step,
                                int32_t n_offsets, int32_t axes, int32_t shift[3]) {
  if (!window || !shift) return basa::fail(BASA_ERR_INVALID_ARGUMENT, "null window or shift pointer");
  if (n_offsets < 1) return basa::fail(BASA_ERR_INVALID_ARGUMENT, "n_offsets %d must be >= 1", n_offsets);
  if (layer < 0 || step < 0)
    return basa::fail(BASA_ERR_INVALID_ARGUMENT, "layer %d and step %d must be >= 0", layer, step);
  if (axes < 0 || axes > 7)
    return basa::fail(BASA_ERR_INVALID_ARGUMENT, "axes mask %d outside [0, 7]", axes);
  for (int a = 0; a < 3; ++a)
    if (window[a] < 1)
      return basa::fail(BASA_ERR_INVALID_ARGUMENT, "window extent %d on axis %d must be >= 1",
                        window[a], a);
  // Candidate k = (layer + step) mod n: consecutive layers take consecutive
  // candidates and every step moves each layer on by one.
  const int64_t k = (int64_t(layer) + step) % n_offsets;
  for (int a = 0; a < 3; ++a)
    shift[a] = (axes >> a) & 1 ? int32_t(k * window[a] / n_offsets) : 0;
  basa::set_error("%s", "");
  return BASA_OK;
}

const char* basa_status_string(basa_status s) {
  switch (s) {
    case BASA_OK: return "BASA_OK";
    case BASA_ERR_INVALID_ARGUMENT: return "BASA_ERR_INVALID_ARGUMENT";
    case BASA_ERR_NOT_DIVISIBLE: return "BASA_ERR_NOT_DIVISIBLE";
    case BASA_ERR_UNSUPPORTED: return "BASA_ERR_UNSUPPORTED";
    case BASA_ERR_HIP: return "BASA_ERR_HIP";
    case BASA_ERR_OUT_OF_MEMORY: return "BASA_ERR_OUT_OF_MEMORY";
  }
  return "BASA_ERR_UNKNOWN";
}

const char* basa_last_error(void) { return basa::last_error(); }

}  // extern "C"
