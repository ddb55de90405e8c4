// k_route.hip -- content-adaptive window routing (BASA, paperlayer.ai summary
// sec. 3.3 and A.2: whole windows of original K/V are routed to each window).
//
// Score of candidate window j for window i: (sum of q over i) . (sum of k over
// j), per head, float64, in a fixed order -- slot order for the sums, channel
// order for the dot product, multiply and add rounded separately -- so that
// the selection is reproducible bit for bit.  Window i itself is excluded; with
// a candidate radius r >= 0 (A.2: radius one for video) so is every window
// more than r window steps from i on some axis of the window grid.  The top-k
// are listed by score descending, ties to the smaller window index.
//
// Two launches: window sums (one wave per window, head and tensor; reads Q and
// K once, HBM-bound), then scores + selection (one workgroup per window and
// head; the nW x d sums of k are L2-resident).
#include "device_common.hpp"

namespace basa {

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

// ws layout: [2][B*H][nW][D] float64, tensor 0 = q sums, 1 = k sums.
template <int D, typename T>
__global__ __launch_bounds__(64) void route_sums_kernel(Geom g, const T* q, const T* k,
                                                        double* ws) {
  constexpr int CPL = D / 64;  // channels per lane
  const int lane = threadIdx.x;
  const uint32_t w = blockIdx.x;
  const size_t bh = blockIdx.y;
  const T* src = (blockIdx.z ? k : q) + bh * size_t(g.N) * D + lane * CPL;
  double acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.0;
  int32_t s = 0;
  // Loads are issued ahead in groups of 8; the adds stay in slot order.
  for (; s + 8 <= g.M; s += 8) {
    double x[8][CPL];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int32_t n = window_token(g, w, s + u);
#pragma unroll
      for (int c = 0; c < CPL; ++c) x[u][c] = load_as_f64<T>(src + size_t(n) * D + c);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = __dadd_rn(acc[c], x[u][c]);
  }
  for (; s < g.M; ++s) {
    const int32_t n = window_token(g, w, s);
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = __dadd_rn(acc[c], load_as_f64<T>(src + size_t(n) * D + c));
  }
  double* dst = ws + ((size_t(blockIdx.z) * g.BH + bh) * g.nW + w) * D + lane * CPL;
#pragma unroll
  for (int c = 0; c < CPL; ++c) dst[c] = acc[c];
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
  const bool f32 = p.params.dtype == BASA_F32;
  dim3 g1(g.nW, g.BH, 2);
  if (g.D == 128) {
    if (f32)
      hipLaunchKernelGGL((route_sums_kernel<128, float>), g1, dim3(64), 0, s, g,
                         static_cast<const float*>(q), static_cast<const float*>(k), ws);
    else
      hipLaunchKernelGGL((route_sums_kernel<128, __bf16>), g1, dim3(64), 0, s, g,
                         static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), ws);
  } else {
    if (f32)
      hipLaunchKernelGGL((route_sums_kernel<64, float>), g1, dim3(64), 0, s, g,
                         static_cast<const float*>(q), static_cast<const float*>(k), ws);
    else
      hipLaunchKernelGGL((route_sums_kernel<64, __bf16>), g1, dim3(64), 0, s, g,
                         static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), ws);
  }
  hipError_t e = hipGetLastError();
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
