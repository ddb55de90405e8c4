// k_route.hip -- content-adaptive window routing (BASA, paperlayer.ai summary
// sec. 3.3 and A.2: whole windows of original K/V are routed to each window).
//
// Score of candidate window j for window i: (sum of q over i) . (sum of k over
// j), per head, in float64.  The sums are taken in this kernel's own order --
// chunks of kRouteChunk slots summed in parallel (within a chunk, rows
// strided over lanes, then a tree across lanes), chunk sums in chunk order.  For bf16 input the
// order does not matter: a bf16 value has 8 significant bits, so while the
// inputs' exponent span plus log2 of the window size stays within float64's
// 53, every partial sum is exact and any order gives the same bits.  Float
// input sums round, within the usual (M - 1) u sum|x| of any other order.
// The dot product runs in channel order, multiply and add rounded
// separately, so the scores, and the selection, are reproducible bit for
// bit.  Window i itself is excluded; with
// a candidate radius r >= 0 (A.2: radius one for video) so is every window
// more than r window steps from i on some axis of the window grid.  The top-k
// are listed by score descending, ties to the smaller window index.
//
// Two or three launches: chunk sums (one wave per chunk of a window, head and
// tensor, whole rows per load, every load of the chunk in flight, sums in
// registers; reads Q and K once, HBM-bound); window sums (one workgroup per
// window, head and tensor, adding the chunk sums in order), which the chunk
// kernel does itself when one workgroup holds every chunk of a window; then
// scores + selection (one workgroup per window and head).  The window sums
// of k are also kept channel-major, [B*H][d][nW], so that the lanes scoring
// consecutive candidates read consecutive addresses.
#include <mutex>

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
// chunk sums [2][B*H][nW][n_chunks][D] float64, then the window sums of k
// again, channel-major [B*H][D][nW].
// The value lane ^ off holds (off a power of two).  Strides 32 and 16 use the
// VALU lane swaps: with both operands x, lane l gets back x[l] and x[l ^ off],
// the partner's in the first result for lanes with that bit set, in the
// second otherwise.  Smaller strides go through a bpermute.
__device__ __forceinline__ uint32_t xor_lanes32(uint32_t v, int off) {
  const bool hi = (threadIdx.x & off) != 0;
  if (off == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return hi ? r[0] : r[1];
  }
  if (off == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return hi ? r[0] : r[1];
  }
  return uint32_t(__shfl_xor(int(v), off));
}

__device__ __forceinline__ double xor_lanes(double v, int off) {
  const uint64_t b = uint64_t(__double_as_longlong(v));
  const uint32_t lo = xor_lanes32(uint32_t(b), off), hi = xor_lanes32(uint32_t(b >> 32), off);
  return __longlong_as_double((long long)(uint64_t(hi) << 32 | lo));
}

constexpr int kRouteChunk = 128;
static_assert(kRouteChunk % 64 == 0, "a chunk is whole groups of 64 rows, one row per lane each");
constexpr int kChunkWaves = 4;    // chunks (one per wave) per workgroup
constexpr int kSumPiece = 32;     // chunk sums staged per round of the window sums

__host__ __device__ inline int32_t route_chunks(const Geom& g) {
  return (g.M + kRouteChunk - 1) / kRouteChunk;
}

// Writes window sum `acc` of channel c, tensor `tensor`, row (tensor, bh, w)
// of the window sums, and for k its channel-major copy.
__device__ __forceinline__ void put_window_sum(const Geom& g, double* ws, double* ws_kt,
                                               int tensor, size_t bh, uint32_t w, int c, int D,
                                               double acc) {
  ws[((size_t(tensor) * g.BH + bh) * g.nW + w) * D + c] = acc;
  if (tensor == 1) ws_kt[(bh * D + c) * g.nW + w] = acc;
}

// The chunk sum of one wave: chunk ci (slots c0 .. c0 + len - 1) of window w,
// head bh, tensor blockIdx.z; written to the workgroup's LDS slots (whole) or
// to the workspace.
template <int D, typename T>
__device__ __forceinline__ void chunk_sum_wave(const Geom& g, const T* q, const T* k,
                                               double* chunk_sums, double* part_sums, bool whole,
                                               uint32_t w, int32_t ci, int32_t c0, int32_t len,
                                               int32_t nc, size_t bh, int lane, int wave) {
  constexpr int RB = D * int(sizeof(T));   // bytes per row
  constexpr int LPR = RB / 16;             // lanes per row
  constexpr int RPI = 64 / LPR;            // rows per load instruction
  constexpr int NI = kRouteChunk / RPI;    // load instructions per chunk
  constexpr int EPL = 16 / int(sizeof(T)); // channels per lane
  static_assert(RB % 16 == 0 && 64 % LPR == 0 && LPR * EPL == D, "row shape");
  const uint8_t* src =
      reinterpret_cast<const uint8_t*>((blockIdx.z ? k : q) + bh * size_t(g.N) * D);
  const int sub = lane / LPR, part = lane % LPR;
  // Lane l finds the tokens of the chunk's rows l, l + 64, ... once; the
  // loads take each row's token from its lane.
  // Rows past a partial chunk's end load its first row and are dropped at
  // the sums, so the loads carry no condition and all go out at once.
  constexpr int TPL = kRouteChunk / 64;  // rows per lane
  int32_t tok[TPL];
#pragma unroll
  for (int h = 0; h < TPL; ++h) {
    const int32_t r = 64 * h + lane;
    tok[h] = window_token(g, w, uint32_t(c0 + (r < len ? r : 0)));
  }
  // Loads go out in rounds of at most 16 (64 registers, so that more waves
  // fit on a compute unit), every load of a round before any of its sums (the scheduler would otherwise start adding,
  // and waiting, after a few of them).
  constexpr int NL = NI < 16 ? NI : 16;  // loads per round
  static_assert(NI % NL == 0, "whole rounds");
  double acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0;
#pragma unroll
  for (int i0 = 0; i0 < NI; i0 += NL) {
    // A round whose rows all lie past a partial chunk's end is not loaded
    // (the same for every lane of the wave).
    if (i0 > 0 && i0 * RPI >= len) break;
    u32x4 x[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      // Row (i0 + j) * RPI + sub of the chunk: RPI divides 64, so every row
      // of one load sits in the same group of 64, whose tokens one lane each
      // holds.
      const int i = i0 + j;
      const int32_t n = __shfl(tok[(i * RPI) / 64], (i * RPI) % 64 + sub);
      // bf16: 32-bit byte offsets from the head's base (a head holds at most
      // 2^31 elements, so 2^32 bytes); float: 64-bit offsets.
      if constexpr (sizeof(T) == 2)
        x[j] = *reinterpret_cast<const u32x4*>(src + (uint32_t(n) * uint32_t(RB) + 16u * part));
      else
        x[j] = *reinterpret_cast<const u32x4*>(src + size_t(n) * RB + 16 * part);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int i = i0 + j;
      if (i * RPI + sub >= len) x[j] = u32x4{};
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        double v;
        if constexpr (sizeof(T) == 2) {
          const uint32_t wv = x[j][e / 2];
          v = double(e & 1 ? bf16_hi(wv) : bf16_lo(wv));
        } else {
          v = double(__uint_as_float(x[j][e]));
        }
        acc[e] = __dadd_rn(acc[e], v);
      }
    }
  }
  double sum[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) sum[e] = acc[e];
  // Across the lanes holding the same channels (lane xor LPR, 2 LPR, ...).
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) sum[e] = __dadd_rn(sum[e], xor_lanes(sum[e], off));
  }
  if (lane < LPR) {
    double* dst = whole ? part_sums + wave * D + part * EPL
                        : chunk_sums + (((size_t(blockIdx.z) * g.BH + bh) * g.nW + w) * nc + ci) * D +
                              part * EPL;
#pragma unroll
    for (int e = 0; e < EPL; e += 2)
      *reinterpret_cast<f64x2*>(dst + e) = f64x2{sum[e], sum[e + 1]};
  }
}

// One wave per 128-slot chunk of a (tensor, b*h, window).  Lane (sub, part)
// loads 16 bytes -- EPL channels starting at part * EPL -- of rows sub, sub +
// RPI, ... of the chunk (whole rows per instruction, 16 loads in flight),
// and adds its rows per channel in float64 in registers; then the RPI lanes
// that hold the same channels add their partial sums across lanes.  When one
// workgroup covers every chunk of its window (at most kChunkWaves chunks), it
// also adds the chunk sums in chunk order, through LDS, and writes the window
// sums; otherwise the chunk sums go to the workspace for
// route_window_sums_kernel.
template <int D, typename T>
__global__ __launch_bounds__(64 * kChunkWaves) void route_chunk_sums_kernel(Geom g, const T* q,
                                                                           const T* k,
                                                                           double* chunk_sums,
                                                                           double* ws,
                                                                           double* ws_kt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t nc = route_chunks(g);
  const int32_t ngrp = (nc + kChunkWaves - 1) / kChunkWaves;
  // Uniform over the grid: this workgroup holds every chunk of its window.
  const bool whole = ngrp == 1;
  __shared__ __attribute__((aligned(16))) double part_sums[kChunkWaves * D];
  const uint32_t w = blockIdx.x / ngrp;
  const int32_t ci = int32_t(blockIdx.x - w * ngrp) * kChunkWaves + wave;
  const int32_t c0 = ci * kRouteChunk;
  const int32_t wlen = window_tokens(g, w);
  const int32_t len = min(kRouteChunk, wlen - c0);
  const size_t bh = blockIdx.y;
  if (ci < nc && len > 0) chunk_sum_wave<D, T>(g, q, k, chunk_sums, part_sums, whole, w, ci, c0,
                                               len, nc, bh, lane, wave);
  if (!whole) return;
  __syncthreads();
  const int32_t ncw = (wlen + kRouteChunk - 1) / kRouteChunk;
  for (int c = threadIdx.x; c < D; c += 64 * kChunkWaves) {
    double acc = 0.0;
    for (int32_t j = 0; j < ncw; ++j) acc = __dadd_rn(acc, part_sums[j * D + c]);
    put_window_sum(g, ws, ws_kt, int(blockIdx.z), bh, w, c, D, acc);
  }
}

// One workgroup per (tensor, b*h, window): the window's chunk sums come into
// LDS kSumPiece chunks at a time, every load of a piece in flight at once,
// and thread c < D adds channel c's chunk sums in chunk order.
template <int D>
__global__ __launch_bounds__(256) void route_window_sums_kernel(Geom g, const double* chunk_sums,
                                                                double* ws, double* ws_kt) {
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
  if (tid < D) {
    const size_t per_tensor = size_t(g.BH) * g.nW;
    const int tensor = int(row / per_tensor);
    const size_t rem = row - size_t(tensor) * per_tensor;
    const size_t bh = rem / uint32_t(g.nW);
    put_window_sum(g, ws, ws_kt, tensor, bh, uint32_t(rem - bh * uint32_t(g.nW)), tid, D, acc);
  }
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
// A strict total order even with NaN scores (non-finite input): a NaN ranks
// below every number, and equal scores or two NaNs go to the smaller index,
// so the rank selection gives every candidate its own place.
__device__ __forceinline__ bool better(double sa, int32_t ja, double sb, int32_t jb) {
  if (ja < 0) return false;
  if (jb < 0) return true;
  const bool na = sa != sa, nb = sb != sb;
  if (na || nb) return na == nb ? ja < jb : nb;
  return sa > sb || (sa == sb && ja < jb);
}

// Selection by rank: with at most kRankMaxWindows windows, thread j counts
// the eligible candidates better() than candidate j; that count is j's place
// in the list (better() is a strict total order, so the places are distinct).
// More windows: route_topk rounds of a wave-wide argmax.
constexpr int kRankMaxWindows = 1024;

template <int D>
__global__ __launch_bounds__(256) void route_topk_kernel(Geom g, const double* ws,
                                                         const double* ws_kt, int32_t* route) {
  // [nW] scores; with the rank selection then [nW] int32 candidate ids (j, or
  // -1 for a window that is not a candidate).
  extern __shared__ double score[];
  const bool by_rank = g.nW <= kRankMaxWindows;
  int32_t* cand = reinterpret_cast<int32_t*>(score + g.nW);
  __shared__ int32_t chosen[16];
  __shared__ double sq[D];
  const int32_t i = blockIdx.x;
  const size_t bh = blockIdx.y;
  if (threadIdx.x < D) sq[threadIdx.x] = ws[(bh * g.nW + i) * D + threadIdx.x];
  __syncthreads();
  // Scores in channel order, multiply and add rounded separately; candidate
  // j's sums of k are column j of the channel-major copy, so the lanes of a
  // load read consecutive doubles.  Loads go out CB at a time before their
  // products.
  const double* kt = ws_kt + bh * size_t(D) * g.nW;
  constexpr int CB = 32;
  for (int32_t j = threadIdx.x; j < g.nW; j += 256) {
    double acc = 0.0;
#pragma unroll 1
    for (int c0 = 0; c0 < D; c0 += CB) {
      double kv[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u) kv[u] = kt[size_t(c0 + u) * g.nW + j];
#pragma unroll
      for (int u = 0; u < CB; ++u) acc = __dadd_rn(acc, __dmul_rn(sq[c0 + u], kv[u]));
    }
    score[j] = acc;
    if (by_rank) cand[j] = (j == i || !in_radius(g, uint32_t(i), uint32_t(j))) ? -1 : j;
  }
  __syncthreads();
  if (by_rank) {
    for (int32_t j = threadIdx.x; j < g.nW; j += 256) {
      if (cand[j] < 0) continue;
      const double sj = score[j];
      int32_t place = 0;
      for (int32_t m = 0; m < g.nW; ++m) place += better(score[m], cand[m], sj, j) ? 1 : 0;
      if (place < g.topk) route[(bh * g.nW + i) * g.topk + place] = j;
    }
    return;
  }
  // Wave 0 takes route_topk rounds; the other waves only keep the barrier
  // count.
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

// Scratch of basa_route_windows_noalloc: a file-scope device array, so each
// GPU the library runs on holds its own copy until the process ends.  Host
// code never passes the array's name to a kernel (in host code it is only a
// stand-in, not a device address): the entry point looks up this device's
// address once, with the device current, and passes that.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_route(const basa_plan_s& p, const void* q, const void* k, int32_t* route,
                        void* workspace, hipStream_t s) {
  const Geom& g = p.g;
  auto ws = static_cast<double*>(workspace);
  const int32_t nc = route_chunks(g);
  double* chunk_sums = ws + size_t(2) * g.BH * g.nW * g.D;
  double* ws_kt = chunk_sums + size_t(2) * g.BH * g.nW * nc * g.D;
  const bool f32 = p.params.dtype == BASA_F32;
  const uint32_t ngrp = uint32_t((nc + kChunkWaves - 1) / kChunkWaves);
  dim3 g1(uint32_t(g.nW) * ngrp, g.BH, 2);
#define BASA_CHUNKS(D_, T_)                                                                   \
  hipLaunchKernelGGL((route_chunk_sums_kernel<D_, T_>), g1, dim3(64 * kChunkWaves), 0, s, g,  \
                     static_cast<const T_*>(q), static_cast<const T_*>(k), chunk_sums, ws,     \
                     ws_kt)
  if (g.D == 128) {
    if (f32) BASA_CHUNKS(128, float); else BASA_CHUNKS(128, __bf16);
  } else {
    if (f32) BASA_CHUNKS(64, float); else BASA_CHUNKS(64, __bf16);
  }
#undef BASA_CHUNKS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ngrp > 1) {  // otherwise the chunk kernel wrote the window sums
    const uint32_t n_rows = uint32_t(size_t(2) * g.BH * g.nW);
    if (g.D == 128)
      hipLaunchKernelGGL(route_window_sums_kernel<128>, dim3(n_rows), dim3(256), 0, s, g,
                         chunk_sums, ws, ws_kt);
    else
      hipLaunchKernelGGL(route_window_sums_kernel<64>, dim3(n_rows), dim3(256), 0, s, g,
                         chunk_sums, ws, ws_kt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 g2(g.nW, g.BH);
  const size_t lds =
      size_t(g.nW) * (sizeof(double) + (g.nW <= kRankMaxWindows ? sizeof(int32_t) : 0));
  if (g.D == 128)
    hipLaunchKernelGGL(route_topk_kernel<128>, g2, dim3(256), lds, s, g, ws, ws_kt, route);
  else
    hipLaunchKernelGGL(route_topk_kernel<64>, g2, dim3(256), lds, s, g, ws, ws_kt, route);
  return hipGetLastError();
}

}  // namespace basa
