// api.cpp -- the C entry points of libbasa that enqueue device work.
//
// Each entry point checks its arguments against the plan before anything is
// enqueued, then calls one launcher.  No entry point allocates device memory
// or synchronises.
#include <cstdint>

#include "basa_internal.hpp"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

basa_status need_tensor(const void* p, const char* name) {
  if (!p) {
    basa::set_error("%s is null", name);
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (!aligned(p, 16)) {
    basa::set_error("%s is not 16-byte aligned", name);
    return BASA_ERR_INVALID_ARGUMENT;
  }
  return BASA_OK;
}

basa_status need_plan(basa_plan_t plan) {
  if (!plan) {
    basa::set_error("plan is null");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  return BASA_OK;
}

basa_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    basa::set_error("%s launch failed: %s", what, hipGetErrorString(e));
    return BASA_ERR_HIP;
  }
  basa::set_error("%s", "");
  return BASA_OK;
}

#define BASA_CHECK(expr)               \
  do {                                 \
    basa_status st_ = (expr);          \
    if (st_ != BASA_OK) return st_;    \
  } while (0)

}  // namespace

extern "C" {

basa_status basa_pool_kv(basa_plan_t plan, const void* k, const void* v, void* k_pool,
                         void* v_pool, void* stream) {
  BASA_CHECK(need_plan(plan));
  if (!plan->pool_on) {
    basa::set_error("the plan has no pooled memory (pool = {0,0,0})");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  BASA_CHECK(need_tensor(k, "k"));
  BASA_CHECK(need_tensor(v, "v"));
  BASA_CHECK(need_tensor(k_pool, "k_pool"));
  BASA_CHECK(need_tensor(v_pool, "v_pool"));
  return launched(basa::launch_pool(*plan, k, v, k_pool, v_pool, static_cast<hipStream_t>(stream)),
                  "pool");
}

basa_status basa_route_windows(basa_plan_t plan, const void* q, const void* k, int32_t* route,
                               void* workspace, size_t workspace_bytes, void* stream) {
  BASA_CHECK(need_plan(plan));
  if (plan->params.route_topk == 0) {
    basa::set_error("the plan does not route (route_topk = 0)");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  BASA_CHECK(need_tensor(q, "q"));
  BASA_CHECK(need_tensor(k, "k"));
  if (!route || !aligned(route, 4)) {
    basa::set_error("route is null or not 4-byte aligned");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (!workspace || !aligned(workspace, 256)) {
    basa::set_error("workspace is null or not 256-byte aligned");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (workspace_bytes < static_cast<size_t>(plan->route_ws_bytes)) {
    basa::set_error("workspace of %zu bytes is smaller than the %lld the plan needs",
                    workspace_bytes, static_cast<long long>(plan->route_ws_bytes));
    return BASA_ERR_INVALID_ARGUMENT;
  }
  return launched(basa::launch_route(*plan, q, k, route, workspace, static_cast<hipStream_t>(stream)),
                  "route");
}

basa_status basa_route_windows_noalloc(basa_plan_t plan, const void* q, const void* k,
                                       int32_t* route, void* stream) {
  BASA_CHECK(need_plan(plan));
  if (plan->params.route_topk == 0) {
    basa::set_error("the plan does not route (route_topk = 0)");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (static_cast<size_t>(plan->route_ws_bytes) > basa::noalloc_scratch_bytes()) {
    basa::set_error("the plan's routing scratch of %lld bytes exceeds the %zu bytes the "
                    "allocation-free entry point holds; use basa_route_windows with a workspace",
                    static_cast<long long>(plan->route_ws_bytes), basa::noalloc_scratch_bytes());
    return BASA_ERR_UNSUPPORTED;
  }
  BASA_CHECK(need_tensor(q, "q"));
  BASA_CHECK(need_tensor(k, "k"));
  if (!route || !aligned(route, 4)) {
    basa::set_error("route is null or not 4-byte aligned");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  void* ws = nullptr;
  const hipError_t e = basa::noalloc_scratch(&ws);
  if (e != hipSuccess) {
    basa::set_error("device scratch lookup failed: %s", hipGetErrorString(e));
    return BASA_ERR_HIP;
  }
  return launched(basa::launch_route(*plan, q, k, route, ws, static_cast<hipStream_t>(stream)),
                  "route (no allocation)");
}

namespace {

// The forward's argument checks, shared by the joint and the branch-split
// entry points.
basa_status check_fwd(basa_plan_t plan, const void* q, const void* k, const void* v,
                      const void* k_pool, const void* v_pool, const int32_t* route,
                      const void* out, const float* lse) {
  BASA_CHECK(need_plan(plan));
  BASA_CHECK(need_tensor(q, "q"));
  BASA_CHECK(need_tensor(k, "k"));
  BASA_CHECK(need_tensor(v, "v"));
  BASA_CHECK(need_tensor(out, "out"));
  if (plan->global_on) {
    BASA_CHECK(need_tensor(k_pool, "k_pool"));
    BASA_CHECK(need_tensor(v_pool, "v_pool"));
  } else if (k_pool || v_pool) {
    basa::set_error("k_pool/v_pool given but the plan has no global rows");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (plan->params.route_topk > 0) {
    if (!route || !aligned(route, 4)) {
      basa::set_error("route is null or not 4-byte aligned");
      return BASA_ERR_INVALID_ARGUMENT;
    }
  } else if (route) {
    basa::set_error("route given but the plan does not route");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (lse && !aligned(lse, 4)) {
    basa::set_error("lse is not 4-byte aligned");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  return BASA_OK;
}

}  // namespace

basa_status basa_window_attn_fwd(basa_plan_t plan, const void* q, const void* k, const void* v,
                                 const void* k_pool, const void* v_pool, const int32_t* route,
                                 void* out, float* lse, void* stream) {
  BASA_CHECK(check_fwd(plan, q, k, v, k_pool, v_pool, route, out, lse));
  return launched(basa::launch_attn(*plan, q, k, v, k_pool, v_pool, route, out, lse,
                                    static_cast<hipStream_t>(stream)),
                  "window attention");
}

basa_status basa_text_attn_fwd(basa_plan_t plan, const void* q_text, const void* k,
                               const void* v, const void* k_global, const void* v_global,
                               void* out_text, float* lse_text, void* workspace,
                               size_t workspace_bytes, void* stream) {
  BASA_CHECK(need_plan(plan));
  if (plan->g.G - plan->g.Gp <= 0) {
    basa::set_error("the plan has no text rows (global_tokens == 0)");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  BASA_CHECK(need_tensor(q_text, "q_text"));
  BASA_CHECK(need_tensor(k, "k"));
  BASA_CHECK(need_tensor(v, "v"));
  BASA_CHECK(need_tensor(k_global, "k_global"));
  BASA_CHECK(need_tensor(v_global, "v_global"));
  BASA_CHECK(need_tensor(out_text, "out_text"));
  if (lse_text && !aligned(lse_text, 4)) {
    basa::set_error("lse_text is not 4-byte aligned");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (plan->text_ws_bytes > 0) {
    if (!workspace || !aligned(workspace, 256)) {
      basa::set_error("workspace is null or not 256-byte aligned");
      return BASA_ERR_INVALID_ARGUMENT;
    }
    if (workspace_bytes < static_cast<size_t>(plan->text_ws_bytes)) {
      basa::set_error("workspace of %zu bytes is smaller than the %lld the plan needs",
                      workspace_bytes, static_cast<long long>(plan->text_ws_bytes));
      return BASA_ERR_INVALID_ARGUMENT;
    }
  }
  return launched(basa::launch_attn_text(*plan, q_text, k, v, k_global, v_global, out_text,
                                         lse_text, workspace, static_cast<hipStream_t>(stream)),
                  "text-query attention");
}

basa_status basa_window_attn_fwd_split(basa_plan_t plan, const void* q, const void* k,
                                       const void* v, const void* k_pool, const void* v_pool,
                                       const int32_t* route, void* out, float* lse, int ways,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  BASA_CHECK(check_fwd(plan, q, k, v, k_pool, v_pool, route, out, lse));
  if (ways != 2 && ways != 3) {
    basa::set_error("ways must be 2 or 3, got %d", ways);
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (!workspace || !aligned(workspace, 256)) {
    basa::set_error("workspace is null or not 256-byte aligned");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (workspace_bytes < static_cast<size_t>(plan->split_ws_bytes)) {
    basa::set_error("workspace of %zu bytes is smaller than the %lld the plan needs",
                    workspace_bytes, static_cast<long long>(plan->split_ws_bytes));
    return BASA_ERR_INVALID_ARGUMENT;
  }
  return launched(basa::launch_attn_split(*plan, q, k, v, k_pool, v_pool, route, out, lse, ways,
                                          workspace, static_cast<hipStream_t>(stream)),
                  "branch-split window attention");
}

basa_status basa_window_attn_bwd(basa_plan_t plan, const void* q, const void* k, const void* v,
                                 const void* k_pool, const void* v_pool, const int32_t* route,
                                 const void* out, const float* lse, const void* d_out,
                                 float* d_q, float* d_k, float* d_v, float* d_k_global,
                                 float* d_v_global, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  BASA_CHECK(need_plan(plan));
  BASA_CHECK(need_tensor(q, "q"));
  BASA_CHECK(need_tensor(k, "k"));
  BASA_CHECK(need_tensor(v, "v"));
  BASA_CHECK(need_tensor(out, "out"));
  BASA_CHECK(need_tensor(d_out, "d_out"));
  BASA_CHECK(need_tensor(d_q, "d_q"));
  BASA_CHECK(need_tensor(d_k, "d_k"));
  BASA_CHECK(need_tensor(d_v, "d_v"));
  if (!lse || !aligned(lse, 4)) {
    basa::set_error("lse is null or not 4-byte aligned");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (plan->global_on) {
    BASA_CHECK(need_tensor(k_pool, "k_pool"));
    BASA_CHECK(need_tensor(v_pool, "v_pool"));
    BASA_CHECK(need_tensor(d_k_global, "d_k_global"));
    BASA_CHECK(need_tensor(d_v_global, "d_v_global"));
  } else if (k_pool || v_pool || d_k_global || d_v_global) {
    basa::set_error("global rows given but the plan has none");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (plan->params.route_topk > 0) {
    if (!route || !aligned(route, 4)) {
      basa::set_error("route is null or not 4-byte aligned");
      return BASA_ERR_INVALID_ARGUMENT;
    }
  } else if (route) {
    basa::set_error("route given but the plan does not route");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (!workspace || !aligned(workspace, 256)) {
    basa::set_error("workspace is null or not 256-byte aligned");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (workspace_bytes < static_cast<size_t>(plan->bwd_ws_bytes)) {
    basa::set_error("workspace of %zu bytes is smaller than the %lld the plan needs",
                    workspace_bytes, static_cast<long long>(plan->bwd_ws_bytes));
    return BASA_ERR_INVALID_ARGUMENT;
  }
  hipError_t e = basa::launch_attn_bwd(*plan, q, k, v, k_pool, v_pool, route, out, lse, d_out,
                                       d_q, d_k, d_v, d_k_global, d_v_global, workspace,
                                       static_cast<hipStream_t>(stream));
  return launched(e, "attention backward");
}

basa_status basa_window_index(basa_plan_t plan, int32_t* win_id, int32_t* slot, void* stream) {
  BASA_CHECK(need_plan(plan));
  if (!win_id || !slot || !aligned(win_id, 4) || !aligned(slot, 4)) {
    basa::set_error("win_id/slot null or not 4-byte aligned");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  return launched(basa::launch_window_index(*plan, win_id, slot, static_cast<hipStream_t>(stream)),
                  "window index");
}

basa_status basa_gather_windows(basa_plan_t plan, const void* x, void* x_win, void* stream) {
  BASA_CHECK(need_plan(plan));
  BASA_CHECK(need_tensor(x, "x"));
  BASA_CHECK(need_tensor(x_win, "x_win"));
  return launched(basa::launch_gather(*plan, x, x_win, static_cast<hipStream_t>(stream)), "gather");
}

basa_status basa_probe_mfma(int32_t iters, int32_t mode, int32_t n_workgroups, float* sink,
                            uint64_t* clocks, double* flops, void* stream) {
  if (iters < 1 || iters >= (1 << 24)) {
    basa::set_error("iters must be in [1, 2^24), got %d", iters);
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (mode != 0 && mode != 1) {
    basa::set_error("mode must be 0 (constant operands) or 1 (switching operands), got %d", mode);
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (mode == 1 && (iters & 1)) {
    basa::set_error("mode 1 takes an even iters, got %d", iters);
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (n_workgroups < 1 || n_workgroups > (1 << 20)) {
    basa::set_error("n_workgroups must be in [1, 2^20], got %d", n_workgroups);
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (!sink || !aligned(sink, 4) || !clocks || !aligned(clocks, 8)) {
    basa::set_error("sink (4-byte aligned) and clocks (8-byte aligned) must be device pointers");
    return BASA_ERR_INVALID_ARGUMENT;
  }
  if (flops) *flops = basa::probe_flops(iters, n_workgroups);
  return launched(basa::launch_probe_mfma(iters, mode, n_workgroups, sink, clocks,
                                          static_cast<hipStream_t>(stream)),
                  "mfma probe");
}

}  // extern "C"
