// k_merge.hip -- branch-split execution of BASA attention.
//
// The pages evaluate the local-window branch and the text/global branch
// (and, for video, the routed branch) as separate attention calls and merge
// them exactly: a softmax over concatenated key lists equals the branch
// outputs weighted by exp(lse_b - lse), lse = log sum_b exp(lse_b)
// (paperlayer.ai summary, A.1; warm-up there picks the faster two- or
// three-way decomposition per shape).  Here each branch is a pass of the
// attention kernel restricted to its key-list segments, writing O_b and
// lse_b to the caller's workspace, and one kernel merges them.
#include "device_common.hpp"

namespace basa {

namespace {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&f)[8]);
template <>
__device__ __forceinline__ void load8<__bf16>(const __bf16* p, float (&f)[8]) {
  const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(u[i]);
    f[2 * i + 1] = bf16_hi(u[i]);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&f)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = a[i];
    f[4 + i] = b[i];
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&f)[8]);
template <>
__device__ __forceinline__ void store8<__bf16>(__bf16* p, const float (&f)[8]) {
  *reinterpret_cast<u32x4*>(p) = u32x4{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]),
                                       pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7])};
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&f)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{f[0], f[1], f[2], f[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
}

struct Branches {
  const void* o[3];
  const float* lse[3];
  int32_t n;
};

// One thread per 8 elements of [B*H, N, d]: out = sum_b w_b O_b / sum_b w_b
// with w_b = exp(lse_b - max lse), lse = max lse + log sum_b w_b.
template <typename T>
__global__ __launch_bounds__(256) void merge_branches_kernel(size_t rows, int32_t d, Branches br,
                                                             T* out, float* lse) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  const int32_t per_row = d / 8;
  if (i >= rows * per_row) return;
  const size_t row = i / per_row;
  float l[3], m = -INFINITY;
  for (int b = 0; b < br.n; ++b) {
    l[b] = br.lse[b][row];
    m = fmaxf(m, l[b]);
  }
  float acc[8] = {}, wsum = 0.f;
  for (int b = 0; b < br.n; ++b) {
    const float wgt = __expf(l[b] - m);
    float f[8];
    load8<T>(static_cast<const T*>(br.o[b]) + i * 8, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += wgt * f[e];
    wsum += wgt;
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= inv;
  store8<T>(out + i * 8, acc);
  if (lse && i % per_row == 0) lse[row] = m + __logf(wsum);
}

// Parts of one softmax (the text queries' key list cut into consecutive
// parts): the same merge over n_parts partial results stored part-major.
template <typename T>
__global__ __launch_bounds__(256) void merge_parts_kernel(size_t rows, int32_t d, int32_t n_parts,
                                                          const T* parts, const float* part_lse,
                                                          T* out, float* lse) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  const int32_t per_row = d / 8;
  if (i >= rows * per_row) return;
  const size_t row = i / per_row;
  float m = -INFINITY;
  for (int32_t q = 0; q < n_parts; ++q) m = fmaxf(m, part_lse[q * rows + row]);
  float acc[8] = {}, wsum = 0.f;
  for (int32_t q = 0; q < n_parts; ++q) {
    const float wgt = __expf(part_lse[q * rows + row] - m);
    float f[8];
    load8<T>(parts + q * rows * d + i * 8, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += wgt * f[e];
    wsum += wgt;
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= inv;
  store8<T>(out + i * 8, acc);
  if (lse && i % per_row == 0) lse[row] = m + __logf(wsum);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

hipError_t launch_merge_parts(const basa_plan_s& p, const void* parts, const float* part_lse,
                              int n_parts, size_t rows, void* out, float* lse, hipStream_t s) {
  const int32_t d = p.g.D;
  const dim3 grid(uint32_t((rows * (d / 8) + 255) / 256));
  if (p.params.dtype == BASA_F32)
    hipLaunchKernelGGL(merge_parts_kernel<float>, grid, dim3(256), 0, s, rows, d, n_parts,
                       static_cast<const float*>(parts), part_lse, static_cast<float*>(out), lse);
  else
    hipLaunchKernelGGL(merge_parts_kernel<__bf16>, grid, dim3(256), 0, s, rows, d, n_parts,
                       static_cast<const __bf16*>(parts), part_lse, static_cast<__bf16*>(out),
                       lse);
  return hipGetLastError();
}

size_t split_workspace_bytes(const basa_plan_s& p) {
  const Geom& g = p.g;
  const size_t elem = p.params.dtype == BASA_F32 ? 4 : 2;
  return 3 * (align256(size_t(g.BH) * g.N * g.D * elem) + align256(size_t(g.BH) * g.N * 4));
}

// Branch sets: two-way = {local, routed} + {global rows}; three-way =
// {local} + {routed} + {global rows}; sets without keys are dropped.
hipError_t launch_attn_split(const basa_plan_s& p, const void* q, const void* k, const void* v,
                             const void* kp, const void* vp, const int32_t* route, void* out,
                             float* lse, int ways, void* ws, hipStream_t s) {
  const Geom& g = p.g;
  int sets[3], n = 0;
  const bool routed = g.topk > 0, global = g.G > 0;
  if (ways == 2) {
    sets[n++] = 1 | (routed ? 4 : 0);
    if (global) sets[n++] = 2;
  } else {
    sets[n++] = 1;
    if (routed) sets[n++] = 4;
    if (global) sets[n++] = 2;
  }
  if (n == 1) return launch_attn(p, q, k, v, kp, vp, route, out, lse, s, sets[0]);
  const size_t elem = p.params.dtype == BASA_F32 ? 4 : 2;
  const size_t o_bytes = align256(size_t(g.BH) * g.N * g.D * elem);
  const size_t l_bytes = align256(size_t(g.BH) * g.N * 4);
  char* base = static_cast<char*>(ws);
  Branches br{};
  br.n = n;
  for (int b = 0; b < n; ++b) {
    void* ob = base + b * (o_bytes + l_bytes);
    float* lb = reinterpret_cast<float*>(base + b * (o_bytes + l_bytes) + o_bytes);
    const hipError_t e = launch_attn(p, q, k, v, kp, vp, route, ob, lb, s, sets[b]);
    if (e != hipSuccess) return e;
    br.o[b] = ob;
    br.lse[b] = lb;
  }
  const size_t rows = size_t(g.BH) * g.N;
  const size_t threads = rows * (g.D / 8);
  const dim3 grid(uint32_t((threads + 255) / 256));
  if (p.params.dtype == BASA_F32)
    hipLaunchKernelGGL(merge_branches_kernel<float>, grid, dim3(256), 0, s, rows, g.D, br,
                       static_cast<float*>(out), lse);
  else
    hipLaunchKernelGGL(merge_branches_kernel<__bf16>, grid, dim3(256), 0, s, rows, g.D, br,
                       static_cast<__bf16*>(out), lse);
  return hipGetLastError();
}

}  // namespace basa
