// k_pool.hip -- K/V-pooled global memory (BASA, paperlayer.ai summary sec. 3.2
// and A.1: a regular spatial reduction by average pooling of K and V).
//
// One wave per (tensor, head, cell).  A wave reads whole 16-byte chunks of
// several member rows per step (coalesced 256-byte rows at d = 128 bf16),
// accumulates in float32 registers, folds the partial sums across lanes with
// shuffles and writes the cell's mean once.  HBM-bound: it reads K and V once
// (2 * B*H*N*d elements) and writes 2 * B*H*G*d elements.
#include "device_common.hpp"

namespace basa {

template <typename T>
__device__ __forceinline__ void accumulate16(const T* p, float* acc);

template <>
__device__ __forceinline__ void accumulate16<__bf16>(const __bf16* p, float* acc) {
  const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] += bf16_lo(u[e]);
    acc[2 * e + 1] += bf16_hi(u[e]);
  }
}

template <>
__device__ __forceinline__ void accumulate16<float>(const float* p, float* acc) {
  const f32x4 u = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] += u[e];
}

template <typename T>
__device__ __forceinline__ void store16(T* p, const float* v);

template <>
__device__ __forceinline__ void store16<__bf16>(__bf16* p, const float* v) {
  u32x4 u;
#pragma unroll
  for (int e = 0; e < 4; ++e) u[e] = pack_bf16(v[2 * e], v[2 * e + 1]);
  *reinterpret_cast<u32x4*>(p) = u;
}

template <>
__device__ __forceinline__ void store16<float>(float* p, const float* v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
}

template <int D, typename T>
__global__ __launch_bounds__(256) void pool_kernel(Geom g, const T* k, const T* v, T* kp, T* vp) {
  constexpr int EPC = 16 / int(sizeof(T));  // elements per 16-byte chunk
  constexpr int CH = D / EPC;               // chunks per row
  constexpr int RPS = 64 / CH;              // member rows per wave step
  const int lane = threadIdx.x & 63;
  const int32_t cell = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (cell >= g.Gp) return;
  const size_t bh = blockIdx.y;
  const T* src = (blockIdx.z ? v : k) + bh * size_t(g.N) * D;
  T* dst = (blockIdx.z ? vp : kp) + (bh * size_t(g.G) + cell) * D;  // head stride: all global rows
  const int c = lane % CH, r0 = lane / CH;

  const uint32_t ct = g.f_gyx.div(cell);
  const uint32_t cr = cell - ct * uint32_t(g.gy * g.gx);
  const uint32_t cy = g.f_gx.div(cr);
  const uint32_t cx = cr - cy * uint32_t(g.gx);
  const int32_t base = (int32_t(ct) * g.pt * g.Hg + int32_t(cy) * g.ph) * g.Wg + int32_t(cx) * g.pw;
  const int32_t P = g.pt * g.ph * g.pw;
  const uint32_t phw = uint32_t(g.ph * g.pw);

  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
#pragma unroll 4
  for (int32_t m = r0; m < P; m += RPS) {
    const uint32_t i = g.f_phw.div(m);
    const uint32_t r = m - i * phw;
    const uint32_t j = g.f_pw.div(r);
    const uint32_t l = r - j * uint32_t(g.pw);
    const int32_t n = base + (int32_t(i) * g.Hg + int32_t(j)) * g.Wg + int32_t(l);
    accumulate16<T>(src + size_t(n) * D + c * EPC, acc);
  }
#pragma unroll
  for (int off = CH; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] += __shfl_xor(acc[e], off);
  if (r0 == 0) {
    const float count = float(P);
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = acc[e] / count;
    store16<T>(dst + c * EPC, acc);
  }
}

hipError_t launch_pool(const basa_plan_s& p, const void* k, const void* v, void* kp, void* vp,
                       hipStream_t s) {
  const Geom& g = p.g;
  dim3 grid((g.Gp + 3) / 4, g.BH, 2);
#define BASA_POOL(D_, T_)                                                                     \
  hipLaunchKernelGGL((pool_kernel<D_, T_>), grid, dim3(256), 0, s, g,                       \
                     static_cast<const T_*>(k), static_cast<const T_*>(v), static_cast<T_*>(kp), \
                     static_cast<T_*>(vp))
  const bool f32 = p.params.dtype == BASA_F32;
  if (g.D == 128) {
    if (f32) BASA_POOL(128, float); else BASA_POOL(128, __bf16);
  } else {
    if (f32) BASA_POOL(64, float); else BASA_POOL(64, __bf16);
  }
#undef BASA_POOL
  return hipGetLastError();
}

}  // namespace basa
