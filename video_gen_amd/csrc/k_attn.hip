// k_attn.hip -- fused BASA window attention forward for gfx950.
//
// BASA (paperlayer.ai summary of arXiv 2610.08772v1, A.1) evaluates, for
// every query token of a window, one softmax over the concatenated keys
//     window's own tokens ++ pooled global cells ++ routed windows' tokens
// and returns softmax(scale q K^T) V at the query's own grid position.  The
// pages run this on stock attention with an explicit roll/reshape/permute
// and separate branches; here one kernel walks the key list directly: the
// cyclic shift is folded into per-row address math and the branches share a
// single online softmax, so no rolled copy and no branch merge exist.
//
// Work decomposition.  One workgroup = 4 waves = 128 query slots of one
// (batch*head, window); wave w owns slots [32w, 32w+32).  The key list is
// streamed through LDS in tiles of 64 rows, double-buffered; a ring of three
// 64-entry tables holds each tile's row codes (token n >= 0, pooled cell
// -1 - c, or past-the-end), computed two tiles ahead.
//
// Per wave and tile (bf16 matrix cores, v_mfma_f32_32x32x16_bf16):
//   S^T[64 keys x 32 queries] = K_tile . Q^T     A = K rows from LDS,
//                                                B = Q held in registers
//   online softmax in base 2, per query column: every lane holds one query
//     and 16 of its keys per 32-key block, so the row max / sum need one
//     cross-half exchange (v_permlane32_swap) and nothing else;
//   O^T[d x 32 queries] += V^T_tile . P^T        A = V^T rows from LDS,
//                                                B = P straight from the S^T
//                                                accumulator registers.
// V is transposed while it is staged (global -> registers -> LDS) and its
// keys are laid out in the order the S^T accumulator hands P to the second
// product, so P never moves between lanes.
// The running maximum is only raised when a tile's maximum exceeds it by
// more than 8 (log2 units), so exp2 arguments stay <= 8 and O is rescaled
// rarely; the final normalisation uses the same maximum, so the result is
// unchanged.
#include "device_common.hpp"

namespace basa {

namespace {

constexpr int kWaves = 4;
constexpr int BQ = 32 * kWaves;  // query slots per workgroup
constexpr int BK = 64;           // key rows per tile
constexpr int kMaxTopk = 16;
constexpr int32_t kNoRow = INT32_MIN;
constexpr float kRescaleSlack = 8.0f;  // log2 units

template <int D>
struct Smem {
  static constexpr int KP = D + 8;   // K tile row pitch (bf16)
  static constexpr int VP = BK + 8;  // V^T tile row pitch (bf16)
  uint16_t k[2][BK * KP];
  uint16_t vt[2][D * VP];
  int32_t code[3][BK];
  int32_t routes[kMaxTopk];
};

template <typename T>
struct AttnArgs {
  const T* q;
  const T* k;
  const T* v;
  const T* kp;
  const T* vp;
  const int32_t* route;
  T* out;
  float* lse;
  float scale_log2;  // softmax scale * log2(e)
  int32_t n_qt;      // query tiles per window
  int32_t n_blocks;
};

// Row code of key j of window `win`'s key list.
__device__ __forceinline__ int32_t key_code(const Geom& g, uint32_t win, const int32_t* routes,
                                            int32_t j) {
  if (j >= g.L) return kNoRow;
  if (j < g.M) return window_token(g, win, j);
  j -= g.M;
  if (j < g.G) return -1 - j;
  j -= g.G;
  const uint32_t r = g.f_M.div(j);
  return window_token(g, routes[r], j - r * uint32_t(g.M));
}

template <int D, typename T>
__device__ __forceinline__ u32x4 load_row8(const T* tok, const T* pooled, int32_t code, int c) {
  u32x4 r = {0u, 0u, 0u, 0u};
  if (code != kNoRow) {
    const T* row = code >= 0 ? tok + size_t(code) * D : pooled + size_t(-1 - code) * D;
    r = load8_bf16<T>(row + 8 * c);
  }
  return r;
}

// Column of key quad kq (keys 4kq .. 4kq+3 of a tile) inside a V^T row.  The
// S^T accumulator of 32 keys gives lane half h the keys {4h..4h+3, 8+4h..}
// of each 16-key step; storing quads 1 and 2 of every 16 swapped makes each
// lane's eight keys of a step contiguous.
__device__ __forceinline__ int vt_col(int kq) {
  return 16 * (kq >> 2) + 8 * (kq & 1) + 4 * ((kq >> 1) & 1);
}

template <typename T>
__device__ __forceinline__ void store_out4(T* p, const float* v);
template <>
__device__ __forceinline__ void store_out4<__bf16>(__bf16* p, const float* v) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
}
template <>
__device__ __forceinline__ void store_out4<float>(float* p, const float* v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
}

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace

template <int D, typename T>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void window_attn_fwd_kernel(Geom g, AttnArgs<T> a) {
  constexpr int KP = Smem<D>::KP, VP = Smem<D>::VP;
  constexpr int KS = D / 16;      // 16-wide k steps of q.k
  constexpr int DB = D / 32;      // 32-row blocks of O^T
  constexpr int CH = D / 8;       // 8-element chunks per row
  constexpr int RPP = 256 / CH;   // K rows staged per pass
  constexpr int KPASS = BK / RPP;
  constexpr int VITEMS = (BK / 4) * CH;  // (key quad, chunk) items of a V tile
  __shared__ Smem<D> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;

  const int32_t blk = xcd_remap(blockIdx.x, a.n_blocks);
  const int32_t qt = blk % a.n_qt;
  const int32_t rest = blk / a.n_qt;
  const uint32_t win = uint32_t(rest % g.nW);
  const size_t bh = size_t(rest / g.nW);

  const T* qh = a.q + bh * size_t(g.N) * D;
  const T* kh = a.k + bh * size_t(g.N) * D;
  const T* vh = a.v + bh * size_t(g.N) * D;
  const T* kph = a.kp ? a.kp + bh * size_t(g.G) * D : nullptr;
  const T* vph = a.vp ? a.vp + bh * size_t(g.G) * D : nullptr;

  // Routed window ids are clamped into [0, nW) so that a corrupt table can
  // only give wrong keys, never an out-of-bounds read.
  if (tid < g.topk)
    sm.routes[tid] = int32_t(min(uint32_t(a.route[(bh * g.nW + win) * g.topk + tid]),
                                 uint32_t(g.nW - 1)));
  __syncthreads();
  const int32_t n_tiles = (g.L + BK - 1) / BK;
  if (tid < 2 * BK) sm.code[tid / BK][tid % BK] = key_code(g, win, sm.routes, tid);

  // This lane's query: slot qs of the window, token qn.
  const int32_t qs = qt * BQ + wave * 32 + l32;
  const bool q_valid = qs < g.M;
  const bool wave_active = qt * BQ + wave * 32 < g.M;
  const int32_t qn = q_valid ? window_token(g, win, qs) : 0;
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 u = {0u, 0u, 0u, 0u};
    if (q_valid) u = load8_bf16<T>(qh + size_t(qn) * D + 16 * ks + 8 * half);
    qf[ks] = __builtin_bit_cast(bf16x8, u);
  }
  __syncthreads();

  // Staging registers for one tile.
  u32x4 kreg[KPASS];
  u32x4 vreg[4];
  const int kc = tid % CH, kr = tid / CH;          // K: chunk, row within pass
  const int vq = tid % (BK / 4), vc = tid / (BK / 4);  // V: key quad, chunk
  const bool v_item = tid < VITEMS;

  auto load_tile = [&](int t) {
    const int32_t* code = sm.code[t % 3];
#pragma unroll
    for (int p = 0; p < KPASS; ++p) kreg[p] = load_row8<D, T>(kh, kph, code[p * RPP + kr], kc);
    if (v_item) {
#pragma unroll
      for (int i = 0; i < 4; ++i) vreg[i] = load_row8<D, T>(vh, vph, code[4 * vq + i], vc);
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* ks_ = sm.k[buf];
#pragma unroll
    for (int p = 0; p < KPASS; ++p)
      *reinterpret_cast<u32x4*>(ks_ + (p * RPP + kr) * KP + 8 * kc) = kreg[p];
    if (v_item) {
      uint16_t* vt = sm.vt[buf] + vt_col(vq);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dw = e >> 1;
        uint32_t lo, hi;
        if (e & 1) {
          lo = (vreg[0][dw] >> 16) | (vreg[1][dw] & 0xffff0000u);
          hi = (vreg[2][dw] >> 16) | (vreg[3][dw] & 0xffff0000u);
        } else {
          lo = (vreg[0][dw] & 0xffffu) | (vreg[1][dw] << 16);
          hi = (vreg[2][dw] & 0xffffu) | (vreg[3][dw] << 16);
        }
        *reinterpret_cast<u32x2*>(vt + (8 * vc + e) * VP) = u32x2{lo, hi};
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_i = -INFINITY;  // running max of scaled logits (log2 units)
  float l_i = 0.f;        // this lane's partial sum of exp2 terms
  const float sl2 = a.scale_log2;

  for (int32_t t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 2 < n_tiles && tid < BK)
      sm.code[(t + 2) % 3][tid] = key_code(g, win, sm.routes, (t + 2) * BK + tid);
    if (t + 1 < n_tiles) load_tile(t + 1);

    if (wave_active) {
      const uint16_t* ks_ = sm.k[buf];
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const bf16x8 k0 =
            *reinterpret_cast<const bf16x8*>(ks_ + l32 * KP + 16 * kk + 8 * half);
        const bf16x8 k1 =
            *reinterpret_cast<const bf16x8*>(ks_ + (32 + l32) * KP + 16 * kk + 8 * half);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[kk], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[kk], s1, 0, 0, 0);
      }
      // Keys past the end of the list (last tile only) get -inf.
      if ((t + 1) * BK > g.L) {
        const int32_t base = t * BK + 4 * half;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int32_t kj = base + (i >> 2) * 8 + (i & 3);
          if (kj >= g.L) s0[i] = -INFINITY;
          if (kj + 32 >= g.L) s1[i] = -INFINITY;
        }
      }
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
      mx = pair_max(mx) * sl2;
      const float m_new = fmaxf(m_i, mx);
      if (__any(m_new > m_i + kRescaleSlack)) {
        const float alpha = m_i == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_i - m_new);
        l_i *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
        m_i = m_new;
      }
      // P = exp2(s * scale log2e - m); row sums; pack into the B operand.
      bf16x8 pb[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const f32x16& sv = st < 2 ? s0 : s1;
        const int i0 = 8 * (st & 1);
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[i0 + 2 * e], sl2, -m_i));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[i0 + 2 * e + 1], sl2, -m_i));
          l_i += p0 + p1;
          w4[e] = pack_bf16(p0, p1);
        }
        pb[st] = __builtin_bit_cast(bf16x8, u32x4{w4[0], w4[1], w4[2], w4[3]});
      }
      const uint16_t* vt = sm.vt[buf];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 vv =
              *reinterpret_cast<const bf16x8*>(vt + (32 * db + l32) * VP + 16 * st + 8 * half);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pb[st], o[db], 0, 0, 0);
        }
      }
    }

    if (t + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_active) return;
  const float l_tot = pair_sum(l_i);
  if (!q_valid) return;
  const float inv = 1.0f / l_tot;
  T* orow = a.out + (bh * g.N + qn) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      float v4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = o[db][4 * g4 + e] * inv;
      store_out4<T>(orow + 32 * db + 8 * g4 + 4 * half, v4);
    }
  }
  if (a.lse && half == 0) a.lse[bh * g.N + qn] = (m_i + log2f(l_tot)) * 0.69314718055994531f;
}

hipError_t launch_attn(const basa_plan_s& p, const void* q, const void* k, const void* v,
                       const void* kp, const void* vp, const int32_t* route, void* out,
                       float* lse, hipStream_t s) {
  const Geom& g = p.g;
  const int32_t n_qt = (g.M + BQ - 1) / BQ;
  const int64_t n_blocks = int64_t(n_qt) * g.nW * g.BH;
  if (n_blocks > INT32_MAX) return hipErrorInvalidValue;
  const float sl2 = float(double(p.scale) * 1.4426950408889634);
#define BASA_ATTN(D_, T_)                                                                        \
  do {                                                                                           \
    AttnArgs<T_> a{static_cast<const T_*>(q), static_cast<const T_*>(k), static_cast<const T_*>(v), \
                   static_cast<const T_*>(kp), static_cast<const T_*>(vp), route,                \
                   static_cast<T_*>(out), lse, sl2, n_qt, int32_t(n_blocks)};                    \
    hipLaunchKernelGGL((window_attn_fwd_kernel<D_, T_>), dim3(uint32_t(n_blocks)), dim3(256), 0, \
                       s, g, a);                                                                 \
  } while (0)
  const bool f32 = p.params.dtype == BASA_F32;
  if (g.D == 128) {
    if (f32) BASA_ATTN(128, float); else BASA_ATTN(128, __bf16);
  } else {
    if (f32) BASA_ATTN(64, float); else BASA_ATTN(64, __bf16);
  }
#undef BASA_ATTN
  return hipGetLastError();
}

}  // namespace basa
