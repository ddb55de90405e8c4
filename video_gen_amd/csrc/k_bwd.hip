// k_bwd.hip -- gradients of BASA window attention (the pages adapt the sparse
// model by training it, paperlayer.ai summary sec. 3.4, which differentiates
// this operator).
//
// For every query n with key list K_L, V_L (window, pooled and extra global
// rows, routed windows), P = softmax(scale q_n K_L^T) and incoming gradient
// g = dO_n:
//   dV_L += P^T g,  dP = g V_L^T,  dS = P * (dP - g.O_n),
//   dq_n = scale dS K_L,  dK_L += scale dS^T q_n.
// P is recomputed from the forward's log-sum-exp, so nothing of the forward
// is kept but O and lse.
//
// Work is done per item = one (batch*head, window): its queries and its key
// list are gathered into dense row blocks (Q, dO [M x d], K, V [Lmax x d],
// bf16), the five products run as strided batched GEMMs (rocBLAS, bf16
// inputs, float32 accumulation), the softmax part is one elementwise pass,
// and the row gradients are scattered back: dq to its token (each query once),
// dk, dv and the global rows' gradients by float32 atomic adds (a token is a
// key of its own window and of every window routed to it).  Items run in
// chunks that fit the workspace.  Rows past a short window's slots and keys
// past an item's list are zero and masked.  The pooled cells' gradients are
// finally carried back to the tokens of their cells (each gets 1/P of it).
#include <rocblas/rocblas.h>

#include "device_common.hpp"

namespace basa {

namespace {

constexpr int kMaxRoutes = 16;

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<__bf16>(__bf16 x) {
  return __uint_as_float(uint32_t(__builtin_bit_cast(uint16_t, x)) << 16);
}
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, __bf16(x));
}

// Length of item (bh, w)'s key list and the window each routed segment reads.
__device__ __forceinline__ int32_t list_length(const Geom& g, uint32_t w, const int32_t* route_bh,
                                               int32_t* routes) {
  int32_t L = window_tokens(g, w) + g.G;
  for (int r = 0; r < g.topk; ++r) {
    routes[r] = min(uint32_t(route_bh[size_t(w) * g.topk + r]), uint32_t(g.nW - 1));
    L += window_tokens(g, uint32_t(routes[r]));
  }
  return L;
}

// Source row of key j of window w's list: token n >= 0, global row -1 - c,
// or INT32_MIN past the list.
__device__ __forceinline__ int32_t key_source(const Geom& g, uint32_t w, const int32_t* routes,
                                              int32_t j) {
  const int32_t mw = window_tokens(g, w);
  if (j < mw) return window_token(g, w, j);
  j -= mw;
  if (j < g.G) return -1 - j;
  j -= g.G;
  for (int r = 0; r < g.topk; ++r) {
    const int32_t mr = window_tokens(g, uint32_t(routes[r]));
    if (j < mr) return window_token(g, uint32_t(routes[r]), j);
    j -= mr;
  }
  return INT32_MIN;
}

struct BwdBufs {            // per-chunk workspace regions (item-major)
  uint16_t *qb, *gb, *kb, *vb, *pb, *dsb;  // bf16 rows
  float *s, *dp, *dqb, *dkb, *dvb, *delta, *lse;
  int32_t* len;             // key list length per item
};

// One workgroup per (item, 64-row block) of queries: Q, dO rows as bf16,
// delta = dO . O and lse per query (lse = +inf for rows past the window, so
// that every P of the row is 0).
template <typename T>
__global__ __launch_bounds__(256) void gather_queries_kernel(Geom g, int32_t item0, const T* q,
                                                             const T* out, const T* dout,
                                                             const float* lse, BwdBufs b) {
  const int32_t it = blockIdx.y;                 // item within the chunk
  const int32_t item = item0 + it;
  const uint32_t w = uint32_t(item % g.nW);
  const size_t bh = size_t(item / g.nW);
  const int32_t mw = window_tokens(g, w);
  const int32_t row = blockIdx.x * 64 + (threadIdx.x >> 2);  // 4 threads per row
  const int part = threadIdx.x & 3;                            // d / 4 elements each
  if (row >= g.M) return;
  const int D = g.D, per = D / 4;
  uint16_t* qdst = b.qb + (size_t(it) * g.M + row) * D + part * per;
  uint16_t* gdst = b.gb + (size_t(it) * g.M + row) * D + part * per;
  float dot = 0.f;
  if (row < mw) {
    const int32_t n = window_token(g, w, row);
    const size_t src = (bh * g.N + n) * size_t(D) + part * per;
    for (int e = 0; e < per; ++e) {
      const float gv = to_f32<T>(dout[src + e]);
      qdst[e] = bf16_bits(to_f32<T>(q[src + e]));
      gdst[e] = bf16_bits(gv);
      dot += gv * to_f32<T>(out[src + e]);
    }
  } else {
    for (int e = 0; e < per; ++e) qdst[e] = gdst[e] = 0;
  }
  dot += __shfl_xor(dot, 1);
  dot += __shfl_xor(dot, 2);
  if (part == 0) {
    b.delta[size_t(it) * g.M + row] = dot;
    b.lse[size_t(it) * g.M + row] =
        row < mw ? lse[bh * g.N + window_token(g, w, row)] : __builtin_inff();
  }
}

// One workgroup per (item, 64-row block) of keys: K, V rows as bf16 (zero past
// the list); block 0 also records the list length.
template <typename T>
__global__ __launch_bounds__(256) void gather_keys_kernel(Geom g, int32_t item0, int32_t Lmax,
                                                          const T* k, const T* v, const T* kg,
                                                          const T* vg, const int32_t* route,
                                                          BwdBufs b) {
  const int32_t it = blockIdx.y;
  const int32_t item = item0 + it;
  const uint32_t w = uint32_t(item % g.nW);
  const size_t bh = size_t(item / g.nW);
  int32_t routes[kMaxRoutes];
  const int32_t L = list_length(g, w, route ? route + bh * g.nW * g.topk : nullptr, routes);
  if (blockIdx.x == 0 && threadIdx.x == 0) b.len[it] = L;
  const int32_t row = blockIdx.x * 64 + (threadIdx.x >> 2);
  const int part = threadIdx.x & 3;
  if (row >= Lmax) return;
  const int D = g.D, per = D / 4;
  uint16_t* kdst = b.kb + (size_t(it) * Lmax + row) * D + part * per;
  uint16_t* vdst = b.vb + (size_t(it) * Lmax + row) * D + part * per;
  const int32_t src = row < L ? key_source(g, w, routes, row) : INT32_MIN;
  if (src == INT32_MIN) {
    for (int e = 0; e < per; ++e) kdst[e] = vdst[e] = 0;
    return;
  }
  const T* ks = src >= 0 ? k + (bh * g.N + src) * size_t(D) : kg + (bh * g.G + (-1 - src)) * size_t(D);
  const T* vs = src >= 0 ? v + (bh * g.N + src) * size_t(D) : vg + (bh * g.G + (-1 - src)) * size_t(D);
  for (int e = 0; e < per; ++e) {
    kdst[e] = bf16_bits(to_f32<T>(ks[part * per + e]));
    vdst[e] = bf16_bits(to_f32<T>(vs[part * per + e]));
  }
}

// P = exp(scale s - lse) (0 past the list), dS = P (dP - delta); both bf16.
__global__ __launch_bounds__(256) void softmax_bwd_kernel(Geom g, int32_t Lmax, float scale,
                                                          BwdBufs b) {
  const int32_t it = blockIdx.y;
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  const size_t per_item = size_t(g.M) * Lmax;
  if (i >= per_item) return;
  const int32_t row = int32_t(i / Lmax), col = int32_t(i % Lmax);
  const size_t at = size_t(it) * per_item + i;
  float p = 0.f, ds = 0.f;
  if (col < b.len[it]) {
    p = __expf(scale * b.s[at] - b.lse[size_t(it) * g.M + row]);
    ds = p * (b.dp[at] - b.delta[size_t(it) * g.M + row]);
  }
  b.pb[at] = bf16_bits(p);
  b.dsb[at] = bf16_bits(ds);
}

// dq rows to their tokens; dk, dv rows added to their tokens or global rows.
__global__ __launch_bounds__(256) void scatter_kernel(Geom g, int32_t item0, int32_t Lmax,
                                                      const int32_t* route, BwdBufs b, float* dq,
                                                      float* dk, float* dv, float* dkg,
                                                      float* dvg) {
  const int32_t it = blockIdx.y;
  const int32_t item = item0 + it;
  const uint32_t w = uint32_t(item % g.nW);
  const size_t bh = size_t(item / g.nW);
  const int32_t row = blockIdx.x * 64 + (threadIdx.x >> 2);
  const int part = threadIdx.x & 3;
  const int D = g.D, per = D / 4;
  if (row < g.M && row < window_tokens(g, w)) {  // query rows
    const int32_t n = window_token(g, w, row);
    const float* src = b.dqb + (size_t(it) * g.M + row) * D + part * per;
    float* dst = dq + (bh * g.N + n) * size_t(D) + part * per;
    for (int e = 0; e < per; ++e) dst[e] = src[e];
  }
  if (row >= b.len[it]) return;                  // key rows
  int32_t routes[kMaxRoutes];
  list_length(g, w, route ? route + bh * g.nW * g.topk : nullptr, routes);
  const int32_t src = key_source(g, w, routes, row);
  float *kd, *vd;
  if (src >= 0) {
    kd = dk + (bh * g.N + src) * size_t(D);
    vd = dv + (bh * g.N + src) * size_t(D);
  } else {
    kd = dkg + (bh * g.G + (-1 - src)) * size_t(D);
    vd = dvg + (bh * g.G + (-1 - src)) * size_t(D);
  }
  const float* ks = b.dkb + (size_t(it) * Lmax + row) * D + part * per;
  const float* vs = b.dvb + (size_t(it) * Lmax + row) * D + part * per;
  for (int e = 0; e < per; ++e) {
    atomicAdd(kd + part * per + e, ks[e]);
    atomicAdd(vd + part * per + e, vs[e]);
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, size_t n) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += size_t(gridDim.x) * 256)
    p[i] = 0.f;
}

// The pooled cells' gradients back to their tokens: token n of cell c gets
// dkg[c] / P (one thread per element of [B*H, N, d]).
__global__ __launch_bounds__(256) void pool_bwd_kernel(Geom g, const float* dkg, const float* dvg,
                                                       float* dk, float* dv) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  const size_t total = size_t(g.BH) * g.N * g.D;
  if (i >= total) return;
  const int32_t e = int32_t(i % g.D);
  const size_t rowi = i / g.D;
  const int32_t n = int32_t(rowi % g.N);
  const size_t bh = rowi / g.N;
  const int32_t t = n / (g.Hg * g.Wg), y = (n / g.Wg) % g.Hg, x = n % g.Wg;
  const int32_t c = ((t / g.pt) * g.gy + y / g.ph) * g.gx + x / g.pw;
  const float inv = 1.f / float(g.pt * g.ph * g.pw);
  dk[i] += dkg[(bh * g.G + c) * g.D + e] * inv;
  dv[i] += dvg[(bh * g.G + c) * g.D + e] * inv;
}

uint32_t blocks_for(size_t n) { return uint32_t((n + 255) / 256); }

// Handles per device, created on first use (rocBLAS keeps its own scratch).
rocblas_handle blas_handle() {
  static rocblas_handle h[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  if (!h[dev] && rocblas_create_handle(&h[dev]) != rocblas_status_success) h[dev] = nullptr;
  return h[dev];
}

// Row-major, strided-batched C[m x n] (float32) = alpha op(A) op(B) with
// bf16 A, B, through rocBLAS's column-major interface (C^T = op(B)^T op(A)^T).
rocblas_status gemm_rm(rocblas_handle h, bool ta, bool tb, int m, int n, int k, float alpha,
                       const void* a, int lda, int64_t sa, const void* b, int ldb, int64_t sb,
                       float* c, int ldc, int64_t sc, int batch) {
  const float beta = 0.f;
  return rocblas_gemm_strided_batched_ex(
      h, tb ? rocblas_operation_transpose : rocblas_operation_none,
      ta ? rocblas_operation_transpose : rocblas_operation_none, n, m, k, &alpha, b,
      rocblas_datatype_bf16_r, ldb, sb, a, rocblas_datatype_bf16_r, lda, sa, &beta, c,
      rocblas_datatype_f32_r, ldc, sc, c, rocblas_datatype_f32_r, ldc, sc, batch,
      rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

// Bytes of one item's workspace, and the carve-up of a chunk of `items`.
size_t bwd_item_bytes(const Geom& g) {
  const size_t M = g.M, L = g.L, D = g.D;
  return align256(M * D * 2) * 2 + align256(L * D * 2) * 2 + align256(M * L * 4) * 2 +
         align256(M * L * 2) * 2 + align256(M * D * 4) + align256(L * D * 4) * 2 +
         align256(M * 4) * 2 + 256;
}

static BwdBufs carve(const Geom& g, void* ws, int32_t items) {
  const size_t M = g.M, L = g.L, D = g.D, n = size_t(items);
  char* p = static_cast<char*>(ws);
  auto take = [&](size_t bytes) {
    char* r = p;
    p += align256(bytes * n);
    return r;
  };
  BwdBufs b;
  b.qb = reinterpret_cast<uint16_t*>(take(M * D * 2));
  b.gb = reinterpret_cast<uint16_t*>(take(M * D * 2));
  b.kb = reinterpret_cast<uint16_t*>(take(L * D * 2));
  b.vb = reinterpret_cast<uint16_t*>(take(L * D * 2));
  b.s = reinterpret_cast<float*>(take(M * L * 4));
  b.dp = reinterpret_cast<float*>(take(M * L * 4));
  b.pb = reinterpret_cast<uint16_t*>(take(M * L * 2));
  b.dsb = reinterpret_cast<uint16_t*>(take(M * L * 2));
  b.dqb = reinterpret_cast<float*>(take(M * D * 4));
  b.dkb = reinterpret_cast<float*>(take(L * D * 4));
  b.dvb = reinterpret_cast<float*>(take(L * D * 4));
  b.delta = reinterpret_cast<float*>(take(M * 4));
  b.lse = reinterpret_cast<float*>(take(M * 4));
  b.len = reinterpret_cast<int32_t*>(take(4));
  return b;
}

hipError_t launch_attn_bwd(const basa_plan_s& p, const void* q, const void* k, const void* v,
                           const void* kg, const void* vg, const int32_t* route, const void* out,
                           const float* lse, const void* dout, float* dq, float* dk, float* dv,
                           float* dkg, float* dvg, void* ws, hipStream_t s, const char** why) {
  const Geom& g = p.g;
  rocblas_handle h = blas_handle();
  if (!h) {
    *why = "rocBLAS handle creation failed";
    return hipErrorUnknown;
  }
  if (rocblas_set_stream(h, s) != rocblas_status_success) {
    *why = "rocblas_set_stream failed";
    return hipErrorUnknown;
  }
  const bool f32 = p.params.dtype == BASA_F32;
  const size_t tok = size_t(g.BH) * g.N * g.D, glob = size_t(g.BH) * g.G * g.D;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0, s, dk, tok);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0, s, dv, tok);
  if (glob) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0, s, dkg, glob);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0, s, dvg, glob);
  }
  const int32_t n_items = g.BH * g.nW, chunk = p.bwd_chunk;
  const int M = g.M, L = g.L, D = g.D;
  for (int32_t i0 = 0; i0 < n_items; i0 += chunk) {
    const int32_t items = std::min(chunk, n_items - i0);
    const BwdBufs b = carve(g, ws, items);
    const dim3 qgrid((M + 63) / 64, items), kgrid((L + 63) / 64, items);
    if (f32) {
      hipLaunchKernelGGL(gather_queries_kernel<float>, qgrid, dim3(256), 0, s, g, i0,
                         static_cast<const float*>(q), static_cast<const float*>(out),
                         static_cast<const float*>(dout), lse, b);
      hipLaunchKernelGGL(gather_keys_kernel<float>, kgrid, dim3(256), 0, s, g, i0, L,
                         static_cast<const float*>(k), static_cast<const float*>(v),
                         static_cast<const float*>(kg), static_cast<const float*>(vg), route, b);
    } else {
      hipLaunchKernelGGL(gather_queries_kernel<__bf16>, qgrid, dim3(256), 0, s, g, i0,
                         static_cast<const __bf16*>(q), static_cast<const __bf16*>(out),
                         static_cast<const __bf16*>(dout), lse, b);
      hipLaunchKernelGGL(gather_keys_kernel<__bf16>, kgrid, dim3(256), 0, s, g, i0, L,
                         static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
                         static_cast<const __bf16*>(kg), static_cast<const __bf16*>(vg), route, b);
    }
    const int64_t sQ = int64_t(M) * D, sK = int64_t(L) * D, sS = int64_t(M) * L;
    rocblas_status st = rocblas_status_success;
    // S = Q K^T, dP = dO V^T
    st = st != rocblas_status_success ? st
         : gemm_rm(h, false, true, M, L, D, 1.f, b.qb, D, sQ, b.kb, D, sK, b.s, L, sS, items);
    st = st != rocblas_status_success ? st
         : gemm_rm(h, false, true, M, L, D, 1.f, b.gb, D, sQ, b.vb, D, sK, b.dp, L, sS, items);
    if (st != rocblas_status_success) {
      *why = "rocBLAS GEMM failed";
      return hipErrorUnknown;
    }
    hipLaunchKernelGGL(softmax_bwd_kernel, dim3(blocks_for(size_t(M) * L), items), dim3(256), 0,
                       s, g, L, p.scale, b);
    // dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO
    st = gemm_rm(h, false, false, M, D, L, p.scale, b.dsb, L, sS, b.kb, D, sK, b.dqb, D, sQ, items);
    st = st != rocblas_status_success ? st
         : gemm_rm(h, true, false, L, D, M, p.scale, b.dsb, L, sS, b.qb, D, sQ, b.dkb, D, sK, items);
    st = st != rocblas_status_success ? st
         : gemm_rm(h, true, false, L, D, M, 1.f, b.pb, L, sS, b.gb, D, sQ, b.dvb, D, sK, items);
    if (st != rocblas_status_success) {
      *why = "rocBLAS GEMM failed";
      return hipErrorUnknown;
    }
    hipLaunchKernelGGL(scatter_kernel, dim3((std::max(M, L) + 63) / 64, items), dim3(256), 0, s,
                       g, i0, L, route, b, dq, dk, dv, dkg, dvg);
  }
  if (g.Gp > 0)
    hipLaunchKernelGGL(pool_bwd_kernel, dim3(blocks_for(tok)), dim3(256), 0, s, g, dkg, dvg, dk,
                       dv);
  return hipGetLastError();
}

}  // namespace basa
