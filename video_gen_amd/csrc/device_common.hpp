// device_common.hpp -- index math and bf16 helpers shared by libbasa's kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "basa_internal.hpp"

namespace basa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A divisor of the parameter block in scalar registers, and a choice between
// two divisors by value.
__device__ __forceinline__ FastDiv scalar_div(const FastDiv& f) {
  return FastDiv{0, uint32_t(__builtin_amdgcn_readfirstlane(f.m)),
                 uint32_t(__builtin_amdgcn_readfirstlane(f.s1)),
                 uint32_t(__builtin_amdgcn_readfirstlane(f.s2))};
}
__device__ __forceinline__ FastDiv pick_div(bool c, const FastDiv& a, const FastDiv& b) {
  return FastDiv{0, c ? a.m : b.m, c ? a.s1 : b.s1, c ? a.s2 : b.s2};
}

// Token index of slot s of window w under the plan's cyclic shift (BASA,
// paperlayer.ai summary A.1: shift, reshape, permute).  The roll is folded
// into the coordinates: a window that runs past the grid edge wraps around.
// In a short window (last along an axis the window does not divide) the
// slots run over its real positions only, in the same raster order.  PAD =
// false is the form for plans without short windows.
template <bool PAD>
__device__ __forceinline__ int32_t window_token_t(const Geom& g, uint32_t w, uint32_t s) {
  const uint32_t wa = g.f_nwyx.div(w);
  const uint32_t wr = w - wa * uint32_t(g.nWy * g.nWx);
  const uint32_t wb = g.f_nwx.div(wr);
  const uint32_t wc = wr - wb * uint32_t(g.nWx);
  uint32_t it, iy, ix;
  if constexpr (!PAD) {
    it = g.f_whw.div(s);
    const uint32_t sr = s - it * uint32_t(g.wh * g.ww);
    iy = g.f_ww.div(sr);
    ix = sr - iy * uint32_t(g.ww);
  } else {
    const bool sy = wb == uint32_t(g.nWy - 1), sx = wc == uint32_t(g.nWx - 1);
    const uint32_t ey = sy ? g.ry : g.wh, ex = sx ? g.rx : g.ww;
    // Divisors picked by value, from scalar copies: a choice between two
    // fields of the parameter block would otherwise become a per-lane load
    // through a chosen address (a vector memory load, which waits behind
    // every load in flight).
    const FastDiv f_slab = pick_div(sy, pick_div(sx, scalar_div(g.f_ryr), scalar_div(g.f_ryw)),
                                    pick_div(sx, scalar_div(g.f_whr), scalar_div(g.f_whw)));
    const FastDiv f_row = pick_div(sx, scalar_div(g.f_rx), scalar_div(g.f_ww));
    it = f_slab.div(s);
    const uint32_t sr = s - it * ey * ex;
    iy = f_row.div(sr);
    ix = sr - iy * ex;
  }
  int32_t t = int32_t(wa) * g.wt + int32_t(it) + g.st;
  int32_t y = int32_t(wb) * g.wh + int32_t(iy) + g.sy;
  int32_t x = int32_t(wc) * g.ww + int32_t(ix) + g.sx;
  t -= t >= g.T ? g.T : 0;
  y -= y >= g.Hg ? g.Hg : 0;
  x -= x >= g.Wg ? g.Wg : 0;
  return (t * g.Hg + y) * g.Wg + x;
}

__device__ __forceinline__ int32_t window_token(const Geom& g, uint32_t w, uint32_t s) {
  return g.padded ? window_token_t<true>(g, w, s) : window_token_t<false>(g, w, s);
}

// Real positions (slots) of window w: M, or fewer for a short window.
__device__ __forceinline__ int32_t window_tokens(const Geom& g, uint32_t w) {
  if (!g.padded) return g.M;
  const uint32_t wa = g.f_nwyx.div(w);
  const uint32_t wr = w - wa * uint32_t(g.nWy * g.nWx);
  const uint32_t wb = g.f_nwx.div(wr);
  const uint32_t wc = wr - wb * uint32_t(g.nWx);
  const int32_t et = wa == uint32_t(g.nWt - 1) ? g.rt : g.wt;
  const int32_t ey = wb == uint32_t(g.nWy - 1) ? g.ry : g.wh;
  const int32_t ex = wc == uint32_t(g.nWx - 1) ? g.rx : g.ww;
  return et * ey * ex;
}

// Float pair -> packed bf16 pair (round to nearest even), low half = lo.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// 8 consecutive elements as packed bf16 (4 dwords); float32 input is rounded.
template <typename T>
__device__ __forceinline__ u32x4 load8_bf16(const T* p);

template <>
__device__ __forceinline__ u32x4 load8_bf16<__bf16>(const __bf16* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

template <>
__device__ __forceinline__ u32x4 load8_bf16<float>(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  u32x4 r;
  r[0] = pack_bf16(a[0], a[1]);
  r[1] = pack_bf16(a[2], a[3]);
  r[2] = pack_bf16(b[0], b[1]);
  r[3] = pack_bf16(b[2], b[3]);
  return r;
}

// Workgroup order: the hardware hands consecutive workgroup ids to the 8 XCDs
// in turn.  Remapping makes each XCD run a contiguous range of logical tiles,
// so tiles that read the same K/V (the Q tiles of one window) share an L2.
__device__ __forceinline__ int32_t xcd_remap(int32_t pid, int32_t n) {
  constexpr int32_t X = 8;
  const int32_t per = (n + X - 1) / X;
  const int32_t r = n % X;
  const int32_t tall = r == 0 ? X : r;
  const int32_t xcd = pid % X, local = pid / X;
  return xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
}

}  // namespace basa
