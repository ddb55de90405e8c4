// k_route.hip -- content-adaptive window routing (BASA, paperlayer.ai summary
// sec. 3.3 and A.2: whole windows of original K/V are routed to each window).
//
// Score of candidate window j for window i: (sum of q over i) . (sum of k over
// j), per head, float64, in a fixed order -- slots in slot order within
// chunks of kRouteChunk, chunk sums in chunk order, channels in order for the
// dot product, multiply and add rounded separately -- so that the selection is
// reproducible bit for bit.  Window i itself is excluded; with
// a candidate radius r >= 0 (A.2: radius one for video) so is every window
// more than r window steps from i on some axis of the window grid.  The top-k
// are listed by score descending, ties to the smaller window index.
//
// Three launches: chunk sums (one wave per chunk of a window, head and tensor,
// whole rows per load, every load of the chunk in flight; reads Q and K once,
// HBM-bound), window sums (one workgroup per window, head and tensor, adding
// the chunk sums in order), then scores + selection (one workgroup per window
// and head; the nW x d sums of k are L2-resident).
#include "device_common.hpp"

namespace basa {

typedef double f64x2 __attribute__((ext_vector_type(2)));

template <typename T>
__device__ __forceinline__ double load_as_f64(const T* p);
template <>
__device__ __forceinline__ double load_as_f64<__bf16>(const __bf16* p) {
  const uint16_t u = *reinterpret_cast<const uint16_t*>(p);
  return double(__uint_as_float(uint32_t(u) << 16));
}
template <>
__device__ __forceinline__ double load_as_f64<float>(const float* p) {
  return double(*p);
}

// Workspace: window sums [2][B*H][nW][D] float64 (tensor 0 = q, 1 = k), then
// chunk sums [2][B*H][nW][n_chunks][D] float64.
constexpr int kRouteChunk = 64;
constexpr int kChunkWaves = 4;    // chunks (one per wave) per workgroup
constexpr int kSumPiece = 32;     // chunk sums staged per round of the window sums

__host__ __device__ inline int32_t route_chunks(const Geom& g) {
  return (g.M + kRouteChunk - 1) / kRouteChunk;
}

// One wave per 64-slot chunk of a (tensor, b*h, window).  The chunk's rows
// come in 16 bytes per lane, whole rows per instruction, into the wave's own
// LDS area; lane l then adds channels l*CPL .. l*CPL + CPL - 1 over the rows in
// slot order.  Waves share no LDS, so the kernel needs no workgroup barrier.
template <int D, typename T>
__global__ __launch_bounds__(64 * kChunkWaves) void route_chunk_sums_kernel(Geom g, const T* q,
                                                                           const T* k,
                                                                           double* chunk_sums) {
  constexpr int RB = D * int(sizeof(T));   // bytes per row
  constexpr int LPR = RB / 16;             // lanes per row
  constexpr int RPI = 64 / LPR;            // rows per load instruction
  constexpr int NI = kRouteChunk / RPI;    // load instructions per chunk
  constexpr int CPL = D / 64;              // channels per lane
  static_assert(RB % 16 == 0 && 64 % LPR == 0, "row shape");
  __shared__ __attribute__((aligned(16))) uint8_t rows[kChunkWaves][kRouteChunk * RB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t nc = route_chunks(g);
  const int32_t ngrp = (nc + kChunkWaves - 1) / kChunkWaves;
  const uint32_t w = blockIdx.x / ngrp;
  const int32_t ci = int32_t(blockIdx.x - w * ngrp) * kChunkWaves + wave;
  const int32_t c0 = ci * kRouteChunk;
  const int32_t len = min(kRouteChunk, window_tokens(g, w) - c0);
  if (ci >= nc || len <= 0) return;  // past the window's slots
  const size_t bh = blockIdx.y;
  const uint8_t* src =
      reinterpret_cast<const uint8_t*>((blockIdx.z ? k : q) + bh * size_t(g.N) * D);
  const int sub = lane / LPR, part = lane % LPR;
  uint8_t* const mine = rows[wave];
  u32x4 x[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int u = i * RPI + sub;
    if (u < len) {
      const int32_t n = window_token(g, w, uint32_t(c0 + u));
      x[i] = *reinterpret_cast<const u32x4*>(src + size_t(n) * RB + 16 * part);
    }
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int u = i * RPI + sub;
    if (u < len) *reinterpret_cast<u32x4*>(mine + u * RB + 16 * part) = x[i];
  }
  // LDS requests of one wave complete in order: the reads below see the
  // writes above.
  double acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.0;
  const T* col = reinterpret_cast<const T*>(mine) + lane * CPL;
  if (len == kRouteChunk) {
#pragma unroll 16
    for (int u = 0; u < kRouteChunk; ++u)
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = __dadd_rn(acc[c], load_as_f64<T>(col + u * D + c));
  } else {  // the last, partial chunk of a window
    for (int u = 0; u < len; ++u)
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = __dadd_rn(acc[c], load_as_f64<T>(col + u * D + c));
  }
  double* dst = chunk_sums + (((size_t(blockIdx.z) * g.BH + bh) * g.nW + w) * nc + ci) * D +
                lane * CPL;
#pragma unroll
  for (int c = 0; c < CPL; ++c) dst[c] = acc[c];
}

// One workgroup per (tensor, b*h, window): the window's chunk sums come into
// LDS kSumPiece chunks at a time, every load of a piece in flight at once,
// and thread c < D adds channel c's chunk sums in chunk order.
template <int D>
__global__ __launch_bounds__(256) void route_window_sums_kernel(Geom g, const double* chunk_sums,
                                                                double* ws) {
  constexpr int PER = kSumPiece * D / 2 / 256;  // 16-byte loads per thread per piece
  __shared__ __attribute__((aligned(16))) double piece[kSumPiece * D];
  const size_t row = blockIdx.x;  // (tensor, bh, w)
  const int32_t nc = route_chunks(g);
  const int32_t ncw =
      (window_tokens(g, uint32_t(row % uint32_t(g.nW))) + kRouteChunk - 1) / kRouteChunk;
  const double* src = chunk_sums + row * nc * D;
  const int tid = threadIdx.x;
  double acc = 0.0;
  for (int32_t j0 = 0; j0 < ncw; j0 += kSumPiece) {
    const int32_t n2 = min(kSumPiece, ncw - j0) * D / 2;  // 16-byte words of this piece
    const f64x2* from = reinterpret_cast<const f64x2*>(src + size_t(j0) * D);
    f64x2 x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (tid + 256 * i < n2) x[i] = from[tid + 256 * i];
    __syncthreads();  // the previous piece has been added
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (tid + 256 * i < n2) reinterpret_cast<f64x2*>(piece)[tid + 256 * i] = x[i];
    __syncthreads();
    if (tid < D) {
      const int32_t np = n2 * 2 / D;
      for (int32_t j = 0; j < np; ++j) acc = __dadd_rn(acc, piece[j * D + tid]);
    }
  }
  if (tid < D) ws[row * D + tid] = acc;
}

// Is window j within the candidate radius of window i?  The window grid is
// not wrapped: coordinates are compared as they are.
__device__ __forceinline__ bool in_radius(const Geom& g, uint32_t i, uint32_t j) {
  if (g.radius < 0) return true;
  const uint32_t yx = uint32_t(g.nWy * g.nWx);
  const uint32_t ia = g.f_nwyx.div(i), ja = g.f_nwyx.div(j);
  const uint32_t ir = i - ia * yx, jr = j - ja * yx;
  const uint32_t ib = g.f_nwx.div(ir), jb = g.f_nwx.div(jr);
  const uint32_t ic = ir - ib * uint32_t(g.nWx), jc = jr - jb * uint32_t(g.nWx);
  auto far = [&](uint32_t x, uint32_t y) { return (x > y ? x - y : y - x) > uint32_t(g.radius); };
  return !(far(ia, ja) || far(ib, jb) || far(ic, jc));
}

// Is (sa, ja) a better candidate than (sb, jb)?  ja < 0 / jb < 0 mean "none".
__device__ __forceinline__ bool better(double sa, int32_t ja, double sb, int32_t jb) {
  if (ja < 0) return false;
  if (jb < 0) return true;
  return sa > sb || (sa == sb && ja < jb);
}

template <int D>
__global__ __launch_bounds__(256) void route_topk_kernel(Geom g, const double* ws, int32_t* route) {
  extern __shared__ double score[];  // [nW]
  __shared__ int32_t chosen[16];
  const int32_t i = blockIdx.x;
  const size_t bh = blockIdx.y;
  const double* sq = ws + (bh * g.nW + i) * D;
  const double* sk = ws + (size_t(g.BH) + bh) * g.nW * D;
  for (int32_t j = threadIdx.x; j < g.nW; j += 256) {
    const double* kj = sk + size_t(j) * D;
    double acc = 0.0;
    for (int c = 0; c < D; ++c) acc = __dadd_rn(acc, __dmul_rn(sq[c], kj[c]));
    score[j] = acc;
  }
  __syncthreads();
  // Selection by wave 0: k rounds of a wave-wide argmax under better();
  // the other waves only keep the barrier count.
  const int lane = threadIdx.x;
  for (int r = 0; r < g.topk; ++r) {
    if (threadIdx.x < 64) {
      double bs = 0.0;
      int32_t bj = -1;
      for (int32_t j = lane; j < g.nW; j += 64) {
        bool skip = j == i || !in_radius(g, uint32_t(i), uint32_t(j));
        for (int u = 0; u < r; ++u) skip |= chosen[u] == j;
        if (!skip && better(score[j], j, bs, bj)) {
          bs = score[j];
          bj = j;
        }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const double os = __shfl_xor(bs, off);
        const int32_t oj = __shfl_xor(bj, off);
        if (better(os, oj, bs, bj)) {
          bs = os;
          bj = oj;
        }
      }
      if (lane == 0) {
        chosen[r] = bj;
        route[(bh * g.nW + i) * g.topk + r] = bj;
      }
    }
    __syncthreads();
  }
}

hipError_t launch_route(const basa_plan_s& p, const void* q, const void* k, int32_t* route,
                        void* workspace, hipStream_t s) {
  const Geom& g = p.g;
  auto ws = static_cast<double*>(workspace);
  double* chunk_sums = ws + size_t(2) * g.BH * g.nW * g.D;
  const bool f32 = p.params.dtype == BASA_F32;
  const uint32_t ngrp = uint32_t((route_chunks(g) + kChunkWaves - 1) / kChunkWaves);
  dim3 g1(uint32_t(g.nW) * ngrp, g.BH, 2);
#define BASA_CHUNKS(D_, T_)                                                                   \
  hipLaunchKernelGGL((route_chunk_sums_kernel<D_, T_>), g1, dim3(64 * kChunkWaves), 0, s, g,  \
                     static_cast<const T_*>(q), static_cast<const T_*>(k), chunk_sums)
  if (g.D == 128) {
    if (f32) BASA_CHUNKS(128, float); else BASA_CHUNKS(128, __bf16);
  } else {
    if (f32) BASA_CHUNKS(64, float); else BASA_CHUNKS(64, __bf16);
  }
#undef BASA_CHUNKS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t n_rows = uint32_t(size_t(2) * g.BH * g.nW);
  if (g.D == 128)
    hipLaunchKernelGGL(route_window_sums_kernel<128>, dim3(n_rows), dim3(256), 0, s, g,
                       chunk_sums, ws);
  else
    hipLaunchKernelGGL(route_window_sums_kernel<64>, dim3(n_rows), dim3(256), 0, s, g,
                       chunk_sums, ws);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(g.nW, g.BH);
  const size_t lds = size_t(g.nW) * sizeof(double);
  if (g.D == 128)
    hipLaunchKernelGGL(route_topk_kernel<128>, g2, dim3(256), lds, s, g, ws, route);
  else
    hipLaunchKernelGGL(route_topk_kernel<64>, g2, dim3(256), lds, s, g, ws, route);
  return hipGetLastError();
}

}  // namespace basa
