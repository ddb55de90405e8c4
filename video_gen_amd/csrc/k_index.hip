// k_index.hip -- the window partition as device code: the per-token index map
// and the stand-alone shift-aware gather (BASA, paperlayer.ai summary A.1:
// cyclic shift, reshape and permute fold the windows into the batch).
//
// The gather reads every source row whole (16-byte lanes, a row per 8 or 16
// lanes) and writes the windowed copy in slot order; no rolled copy of the
// grid is made.  It is HBM-bound: 2 * B*H*N*d*sizeof(elem) bytes per call.
#include "device_common.hpp"

namespace basa {

__global__ __launch_bounds__(256) void window_index_kernel(Geom g, int32_t* win_id,
                                                           int32_t* slot) {
  const int32_t n = blockIdx.x * 256 + threadIdx.x;
  if (n >= g.N) return;
  const uint32_t t = g.f_HWg.div(n);
  const uint32_t r = n - t * uint32_t(g.Hg * g.Wg);
  const uint32_t y = g.f_Wg.div(r);
  const uint32_t x = r - y * uint32_t(g.Wg);
  // Coordinates in the rolled grid: u = (p - shift) mod extent.
  int32_t ut = int32_t(t) - g.st, uy = int32_t(y) - g.sy, ux = int32_t(x) - g.sx;
  ut += ut < 0 ? g.T : 0;
  uy += uy < 0 ? g.Hg : 0;
  ux += ux < 0 ? g.Wg : 0;
  const uint32_t wa = g.f_wt.div(ut), wb = g.f_wh.div(uy), wc = g.f_ww.div(ux);
  const uint32_t it = ut - wa * g.wt, iy = uy - wb * g.wh, ix = ux - wc * g.ww;
  // Slots of a short window run over its own extents.
  const uint32_t ey = wb == uint32_t(g.nWy - 1) ? g.ry : g.wh;
  const uint32_t ex = wc == uint32_t(g.nWx - 1) ? g.rx : g.ww;
  win_id[n] = int32_t((wa * g.nWy + wb) * g.nWx + wc);
  slot[n] = int32_t((it * ey + iy) * ex + ix);
}

// One thread per 16-byte chunk of the output; blockIdx.y = b*H + h.  The
// output has nW * M rows per head; rows past a short window's real slots are
// zero.
template <int CH>
__global__ __launch_bounds__(256) void gather_kernel(Geom g, const u32x4* x, u32x4* xw) {
  const int64_t rows = int64_t(g.nW) * g.M;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= rows * CH) return;
  const int64_t row = idx / CH;
  const int32_t c = int32_t(idx - row * CH);
  // Plain division: row * M can pass 2^32 (window = grid on a large grid),
  // beyond the multiply-high divider's exact range.
  const uint32_t w = uint32_t(row / g.M);
  const uint32_t s = uint32_t(row - int64_t(w) * g.M);
  const size_t out = size_t(blockIdx.y) * size_t(rows) * CH + size_t(row) * CH + c;
  if (int32_t(s) >= window_tokens(g, w)) {
    xw[out] = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const int32_t n = window_token(g, w, s);
  xw[out] = x[size_t(blockIdx.y) * g.N * CH + size_t(n) * CH + c];
}

hipError_t launch_window_index(const basa_plan_s& p, int32_t* win_id, int32_t* slot,
                               hipStream_t s) {
  const Geom& g = p.g;
  dim3 grid((g.N + 255) / 256);
  hipLaunchKernelGGL(window_index_kernel, grid, dim3(256), 0, s, g, win_id, slot);
  return hipGetLastError();
}

hipError_t launch_gather(const basa_plan_s& p, const void* x, void* x_win, hipStream_t s) {
  const Geom& g = p.g;
  const int row_bytes = g.D * (p.params.dtype == BASA_F32 ? 4 : 2);
  const int ch = row_bytes / 16;
  dim3 grid(uint32_t((int64_t(g.nW) * g.M * ch + 255) / 256), g.BH);
  auto xs = static_cast<const u32x4*>(x);
  auto xd = static_cast<u32x4*>(x_win);
  switch (ch) {
    case 8: hipLaunchKernelGGL(gather_kernel<8>, grid, dim3(256), 0, s, g, xs, xd); break;
    case 16: hipLaunchKernelGGL(gather_kernel<16>, grid, dim3(256), 0, s, g, xs, xd); break;
    case 32: hipLaunchKernelGGL(gather_kernel<32>, grid, dim3(256), 0, s, g, xs, xd); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace basa
