// basa_internal.hpp -- plan layout and kernel launch interface inside libbasa.
//
// The host plan derives, once per (shape, shift), every size and the magic
// multipliers that let device code split a flat index into grid coordinates
// without integer division.  Kernels receive the plan's geometry by value.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/basa.h"

namespace basa {

constexpr int kAttnQueryTile = 256;  // query slots per attention workgroup
constexpr int kComputeUnits = 256;   // MI355X

// Division by an invariant d > 0, exact for every 32-bit n: the round-up
// method of Granlund and Montgomery ("Division by invariant integers using
// multiplication", PLDI 1994), in its branch-free form.  With
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
//   t = umulhi(n, m),  q = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0).
struct FastDiv {
  uint32_t d;
  uint32_t m;
  uint32_t s1, s2;
  __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
    const uint32_t t = uint32_t((uint64_t(n) * m) >> 32);
    return (t + ((n - t) >> s1)) >> s2;
  }
};

inline FastDiv make_fastdiv(uint32_t d) {
  if (d == 0) d = 1;  // an unused divisor (an absent extent)
  uint32_t l = 0;
  while (l < 32 && (uint64_t(1) << l) < d) ++l;
  FastDiv f;
  f.d = d;
  f.m = uint32_t((((uint64_t(1) << l) - d) << 32) / d + 1);
  f.s1 = l < 1 ? l : 1;
  f.s2 = l > 1 ? l - 1 : 0;
  return f;
}

// Geometry of one block's partition, pooling and routing (POD, kernel argument).
struct Geom {
  int32_t T, Hg, Wg;        // token grid
  int32_t wt, wh, ww;       // window extent
  int32_t st, sy, sx;       // cyclic shift of the partition
  int32_t nWt, nWy, nWx;    // windows per axis
  int32_t pt, ph, pw;       // pool cell (1,1,1 when pooling is off)
  int32_t gt, gy, gx;       // pooled grid
  int32_t N, M, nW, G, L, topk, D, BH;  // G: global key rows (pooled cells + extra rows)
  int32_t Gp;               // pooled cells (the first Gp of the G global rows)
  int32_t radius;           // routing candidate radius in window steps (-1: all)
  // Grids that a window does not divide: the last window along such an axis
  // keeps only the rt / ry / rx real positions (= wt / wh / ww elsewhere) and
  // its slots are numbered over them alone.  padded = any axis is short.
  int32_t rt, ry, rx;
  int32_t padded;
  FastDiv f_rx;                      // slot -> x in a window of width rx
  FastDiv f_ryw, f_whr, f_ryr;       // slot -> t for (ry, ww), (wh, rx), (ry, rx)
  FastDiv f_wt, f_wh, f_ww, f_whw;   // slot -> (it, iy, ix); token -> window
  FastDiv f_nwx, f_nwyx;             // window id -> (wa, wb, wc)
  FastDiv f_Wg, f_HWg;               // token -> (t, y, x)
  FastDiv f_M;                       // key index -> routed window, slot
  FastDiv f_pw, f_phw, f_gx, f_gyx;  // pooled cell / member -> coordinates
};

}  // namespace basa

struct basa_plan_s {
  basa_params params;
  basa::Geom g;
  bool pool_on;
  bool global_on;           // any global rows (pooled cells or extra rows)
  float scale;
  int64_t route_ws_bytes;
  int64_t bwd_ws_bytes;     // backward workspace (delta, inverse route table)
  int64_t split_ws_bytes;   // branch-split forward workspace (three branches)
  int32_t text_split;       // text queries: parts of the key list
  int32_t text_split_len;   // keys per part (the last may be shorter)
  int64_t text_ws_bytes;    // partial outputs and lse of the parts (0 with one part)
  basa_plan_info info;
};

namespace basa {

// Kernel launchers (one per device entry point); each returns the launch status.
hipError_t launch_window_index(const basa_plan_s& p, int32_t* win_id, int32_t* slot,
                               hipStream_t s);
hipError_t launch_gather(const basa_plan_s& p, const void* x, void* x_win, hipStream_t s);
hipError_t launch_pool(const basa_plan_s& p, const void* k, const void* v, void* kp, void* vp,
                       hipStream_t s);
hipError_t launch_route(const basa_plan_s& p, const void* q, const void* k, int32_t* route,
                        void* workspace, hipStream_t s);
// The routing scratch of the allocation-free entry point: its size, and this
// device's address of it (looked up on the first call on each device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out);
size_t bwd_workspace_bytes(const basa_plan_s& p);
hipError_t launch_attn_bwd(const basa_plan_s& p, const void* q, const void* k, const void* v,
                           const void* kg, const void* vg, const int32_t* route, const void* out,
                           const float* lse, const void* dout, float* dq, float* dk, float* dv,
                           float* dkg, float* dvg, void* ws, hipStream_t s);
size_t split_workspace_bytes(const basa_plan_s& p);
hipError_t launch_attn_split(const basa_plan_s& p, const void* q, const void* k, const void* v,
                             const void* kp, const void* vp, const int32_t* route, void* out,
                             float* lse, int ways, void* ws, hipStream_t s);
// Text queries of a joint block: every text row attends to every image token
// and every text row (the global rows after the pooled cells).
hipError_t launch_attn_text(const basa_plan_s& p, const void* q_text, const void* k,
                            const void* v, const void* kg, const void* vg, void* out_text,
                            float* lse_text, void* ws, hipStream_t s);
// out[r] = sum_p exp(lse_p[r] - lse[r]) parts_p[r], lse = log sum_p exp(lse_p):
// parts [n_parts][rows][d] in the plan dtype, part_lse [n_parts][rows].
hipError_t launch_merge_parts(const basa_plan_s& p, const void* parts, const float* part_lse,
                              int n_parts, size_t rows, void* out, float* lse, hipStream_t s);
// branches: key-list segments of the pass (1 local, 2 global rows, 4 routed);
// 7 is the joint pass.
hipError_t launch_attn(const basa_plan_s& p, const void* q, const void* k, const void* v,
                       const void* kp, const void* vp, const int32_t* route, void* out,
                       float* lse, hipStream_t s, int branches = 7);

// Matrix-core probe (a measurement hook): threads per workgroup, flops of a
// launch, and the launch itself.
int probe_threads_per_workgroup();
double probe_flops(int32_t iters, int32_t n_workgroups);
hipError_t launch_probe_mfma(int32_t iters, int32_t mode, int32_t n_workgroups, float* sink,
                             uint64_t* clocks, hipStream_t s);

// Per-thread error message used by the C entry points.
void set_error(const char* fmt, ...);

}  // namespace basa
