// k_bwd.hip -- fused gradients of BASA window attention for gfx950.
//
// The pages adapt the sparse model by training it (paperlayer.ai summary of
// arXiv 2610.08772v1, sec. 3.4), which differentiates the attention operator
// of A.1: for every query n with key list K_L, V_L (its window's tokens, the
// global rows, the routed windows' tokens), P = softmax(scale q_n K_L^T) and
// incoming gradient g = dO_n,
//   dV_j += P_j g,   dP_j = g . v_j,   dS_j = P_j (dP_j - delta_n),
//   dq_n  = scale sum_j dS_j k_j,      dK_j += scale dS_j q_n,
// with delta_n = g . O_n (= sum_j P_j dP_j).  P is recomputed from the
// forward's log-sum-exp, so the forward keeps nothing but O and lse.
//
// Three kernels, none of which writes a score matrix to memory:
//   dq      one workgroup per 128 queries of one (batch*head, window); walks
//           the window's key list in the forward's order (K, V tiles through
//           LDS) and accumulates dQ^T in registers.  It also writes delta for
//           the other two kernels.
//   dkv_g   one workgroup per 128 global rows and one range of queries:
//           every query attends every global row, so the range is plain
//           token order; partial sums are added with float atomics.
//   dkv     one workgroup per 128 keys of one window; walks every query that
//           has those keys in its list: the window's own queries, then the
//           queries of each window that routed to it (an inverse route table
//           is built first).  dK^T and dV^T stay in registers and each key
//           row is written once, with its pooled cell's share added: token n
//           of cell c gets dK_c / P through the mean (dkv_g has finished).
//
// Matrix products (v_mfma_f32_32x32x16_bf16).  Every product keeps the
// register-resident side as the B operand and reads the LDS side as A:
//   dq:  S'^T = K (cQ)^T - lse2       (A = K rows,     B = cQ in registers)
//        dP^T = V dO^T - delta        (A = V rows,     B = dO in registers)
//        dQ^T += K^T dS^T             (A = K^T by transposing LDS reads,
//                                      B = dS from the accumulator layout)
//   dkv: S'   = Q (cK)^T - lse2       (A = Q rows,     B = cK in registers)
//        dP   = dO V^T - delta        (A = dO rows,    B = V in registers)
//        dV^T += dO^T P, dK^T += Q^T dS (A = transposing reads of the dO and
//                                      Q tiles, B = P and dS)
// c = scale * log2(e) and lse2 = log2(e) * lse; the subtracted terms enter as
// the accumulator input, so P = exp2(S') needs no other vector work.
//
// LDS tiles hold 64 rows of bf16 in the forward's grouped layout, [8-row
// group][d/32 block][8 rows][32 elements], with the four 16-byte chunks of
// each 64-byte row segment XOR-swizzled by bits 2-3 of the row; the
// transposing reads follow the swizzle lane by lane.  Each tile is loaded
// into registers one tile ahead and written to the other of two buffers.
#include "device_common.hpp"

namespace basa {

namespace {

constexpr int kNT = 256;          // threads per workgroup (4 waves)
constexpr int kBT = 64;           // rows per LDS tile
constexpr int kRows = 128;        // queries (dq) or keys (dkv) per workgroup
constexpr int kSplit = 2048;      // queries per dkv_g workgroup
constexpr int kMaxRoutes = 16;
constexpr int32_t kNone = INT32_MIN;
constexpr float kLog2e = 1.4426950408889634f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Element x of row r of a tile.
template <int D>
__device__ __forceinline__ int tile_off(int r, int x) {
  return (r >> 3) * (8 * D) + (x >> 5) * 256 + (r & 7) * 32 +
         8 * (((x >> 3) ^ (r >> 2)) & 3) + (x & 7);
}

// A operand of rows 32*blk + (lane % 32), k step ks: 8 consecutive elements.
template <int D>
__device__ __forceinline__ bf16x8 frag(const uint16_t* t, int blk, int ks, int lane) {
  return *reinterpret_cast<const bf16x8*>(t + tile_off<D>(32 * blk + (lane & 31),
                                                          16 * ks + 8 * (lane >> 5)));
}

// A operand of the transposed tile, X^T[32 d x 16 rows]: d block db, rows of
// 16-row sub-tile st.  Lane (g16, s16) reads 4 elements of row
// 16 st + 4 (g16 / 2) + s16 / 4 (and of that row + 8); the transposing read
// hands each lane one d column of four rows.  This row order is the one in
// which the accumulator layout of the products holds the B side.
template <int D>
__device__ __forceinline__ bf16x8 tfrag(const uint16_t* t, int st, int db, int lane) {
  const int g16 = lane >> 4, s16 = lane & 15;
  const int r = 16 * st + 4 * (g16 >> 1) + (s16 >> 2);
  const int x = 32 * db + 16 * (g16 & 1) + 4 * (s16 & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + tile_off<D>(r, x)));
  const s16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + tile_off<D>(r + 8, x)));
  return __builtin_bit_cast(
      bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                    __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
}

__device__ __forceinline__ f32x16 splat16(float x) {
  f32x16 r;
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = x;
  return r;
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 8 consecutive elements as float.
template <typename T>
__device__ __forceinline__ void load8_f32(const T* p, float (&f)[8]);
template <>
__device__ __forceinline__ void load8_f32<__bf16>(const __bf16* p, float (&f)[8]) {
  const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(u[i]);
    f[2 * i + 1] = bf16_hi(u[i]);
  }
}
template <>
__device__ __forceinline__ void load8_f32<float>(const float* p, float (&f)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = a[i];
    f[4 + i] = b[i];
  }
}

// 8 elements times c, rounded once to bf16.
__device__ __forceinline__ bf16x8 scale8(const float (&f)[8], float c) {
  return __builtin_bit_cast(bf16x8, u32x4{pack_bf16(f[0] * c, f[1] * c),
                                          pack_bf16(f[2] * c, f[3] * c),
                                          pack_bf16(f[4] * c, f[5] * c),
                                          pack_bf16(f[6] * c, f[7] * c)});
}

template <typename T>
struct BwdArgs {
  const T *q, *k, *v, *kg, *vg, *out, *dout;
  const float* lse;
  const int32_t* route;
  float *dq, *dk, *dv, *dkg, *dvg;
  float* delta;             // [B*H, N] workspace: dO . O
  int32_t* r_off;           // [B*H, nW + 1] inverse route table offsets
  int32_t* r_list;          // [B*H, nW * topk] windows that routed to each window
  float scale, c;           // softmax scale; scale * log2(e)
  int32_t n_blocks;         // workgroups of the launch
};

// Source of key j of window w's list, in the forward's order: token n >= 0,
// global row -1 - c, or kNone past the end.  rstart[r] = offset of routed
// window r inside the routed part, rstart[topk] = its length.
__device__ __forceinline__ int32_t key_src(const Geom& g, uint32_t w, int32_t Mw,
                                           const int32_t* routes, const int32_t* rstart,
                                           int32_t j) {
  if (j < Mw) return window_token(g, w, j);
  j -= Mw;
  if (j < g.G) return -1 - j;
  j -= g.G;
  if (j >= rstart[g.topk]) return kNone;
  int r = 0;
  while (r + 1 < g.topk && j >= rstart[r + 1]) ++r;
  return window_token(g, uint32_t(routes[r]), j - rstart[r]);
}

// Tile staging: thread tid moves 8 elements (chunk tid % (D/8)) of rows
// tid / (D/8) + i * (256 / (D/8)), i < NP.
template <int D>
struct Stage {
  static constexpr int CPR = D / 8, RPP = kNT / CPR, NP = kBT / RPP;
};

// ------------------------------------------------------------------ dq

template <int D, typename T>
__global__ __launch_bounds__(kNT) void bwd_dq_kernel(Geom g, BwdArgs<T> a) {
  constexpr int KS = D / 16, DB = D / 32;
  using SG = Stage<D>;
  __shared__ __attribute__((aligned(16))) uint16_t kt[2][kBT * D];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][kBT * D];
  __shared__ int32_t routes[kMaxRoutes];
  __shared__ int32_t rstart[kMaxRoutes + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int32_t n_qt = (g.M + kRows - 1) / kRows;
  const int32_t blk = xcd_remap(blockIdx.x, a.n_blocks);
  const int32_t qt = blk % n_qt, rest = blk / n_qt;
  const uint32_t w = uint32_t(rest % g.nW);
  const size_t bh = size_t(rest / g.nW);
  const int32_t Mw = window_tokens(g, w);
  if (qt * kRows >= Mw) return;

  // Routed window ids (clamped into [0, nW) as the forward clamps them) and
  // the offsets of their segments.
  if (tid < g.topk)
    routes[tid] = int32_t(min(uint32_t(a.route[(bh * g.nW + w) * g.topk + tid]), uint32_t(g.nW - 1)));
  __syncthreads();
  if (tid == 0) {
    int32_t acc = 0;
    for (int r = 0; r < g.topk; ++r) {
      rstart[r] = acc;
      acc += window_tokens(g, uint32_t(routes[r]));
    }
    rstart[g.topk] = acc;
  }
  __syncthreads();
  const int32_t L = Mw + g.G + rstart[g.topk];
  const int32_t n_tiles = (L + kBT - 1) / kBT;

  // This lane's query (lanes l32 and l32 + 32 share it, each holding half of
  // every 16-element k step).
  const int32_t qs = qt * kRows + wave * 32 + l32;
  const bool qv = qs < Mw;
  const int32_t qn = qv ? window_token(g, w, qs) : 0;
  const size_t qrow = (bh * g.N + qn) * size_t(D);
  bf16x8 qf[KS], gf[KS];
  float dsum = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float x[8] = {}, y[8] = {}, o[8] = {};
    if (qv) {
      load8_f32<T>(a.q + qrow + 16 * ks + 8 * half, x);
      load8_f32<T>(a.dout + qrow + 16 * ks + 8 * half, y);
      load8_f32<T>(a.out + qrow + 16 * ks + 8 * half, o);
    }
    qf[ks] = scale8(x, a.c);
    gf[ks] = scale8(y, 1.f);
#pragma unroll
    for (int e = 0; e < 8; ++e) dsum += float(gf[ks][e]) * o[e];
  }
  const float delta = pair_sum(dsum);
  if (qv && half == 0) a.delta[bh * g.N + qn] = delta;
  const f32x16 s_in = splat16(qv ? -kLog2e * a.lse[bh * g.N + qn] : -INFINITY);
  const f32x16 p_in = splat16(-delta);

  // Key tile t: rows of K and V into registers, then into an LDS buffer.
  const int sc = tid % SG::CPR, sr = tid / SG::CPR;
  const T* kh = a.k + bh * size_t(g.N) * D;
  const T* vh = a.v + bh * size_t(g.N) * D;
  const T* kgh = a.kg ? a.kg + bh * size_t(g.G) * D : kh;
  const T* vgh = a.vg ? a.vg + bh * size_t(g.G) * D : vh;
  u32x4 kr[SG::NP], vr[SG::NP];
  auto fetch = [&](int32_t t) {
#pragma unroll
    for (int i = 0; i < SG::NP; ++i) {
      const int32_t j = t * kBT + sr + i * SG::RPP;
      const int32_t src = j < L ? key_src(g, w, Mw, routes, rstart, j) : kNone;
      kr[i] = vr[i] = u32x4{0, 0, 0, 0};
      if (src != kNone) {
        const T* kp = src >= 0 ? kh + size_t(src) * D : kgh + size_t(-1 - src) * D;
        const T* vp = src >= 0 ? vh + size_t(src) * D : vgh + size_t(-1 - src) * D;
        kr[i] = load8_bf16<T>(kp + 8 * sc);
        vr[i] = load8_bf16<T>(vp + 8 * sc);
      }
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < SG::NP; ++i) {
      const int off = tile_off<D>(sr + i * SG::RPP, 8 * sc);
      *reinterpret_cast<u32x4*>(&kt[buf][off]) = kr[i];
      *reinterpret_cast<u32x4*>(&vt[buf][off]) = vr[i];
    }
  };

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x16{};
  fetch(0);
  put(0);
  __syncthreads();
  for (int32_t t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) fetch(t + 1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int32_t j0 = t * kBT + 32 * kb;
      if (j0 >= L) break;
      f32x16 s = s_in, p = p_in;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag<D>(kt[buf], kb, ks, lane), qf[ks], s, 0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag<D>(vt[buf], kb, ks, lane), gf[ks], p, 0, 0, 0);
      }
      // Lane (query, half) holds keys j0 + 8 gi + 4 half + 0..3 at 4 gi + 0..3.
      uint32_t dsw[8];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const int32_t key = j0 + 8 * (i >> 2) + 4 * half + (i & 3);
        const float p0 = key < L ? __builtin_amdgcn_exp2f(s[i]) : 0.f;
        const float p1 = key + 1 < L ? __builtin_amdgcn_exp2f(s[i + 1]) : 0.f;
        dsw[i / 2] = pack_bf16(p0 * p[i], p1 * p[i + 1]);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const bf16x8 bds = __builtin_bit_cast(
            bf16x8, u32x4{dsw[4 * jj], dsw[4 * jj + 1], dsw[4 * jj + 2], dsw[4 * jj + 3]});
#pragma unroll
        for (int db = 0; db < DB; ++db)
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tfrag<D>(kt[buf], 2 * kb + jj, db, lane),
                                                           bds, dq[db], 0, 0, 0);
      }
    }
    if (t + 1 < n_tiles) put(buf ^ 1);
    __syncthreads();
  }

  if (!qv) return;
  // Lane (query, half) holds d = 32 db + 8 gi + 4 half + 0..3 of its row.
  float* dst = a.dq + qrow;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * gi + 4 * half) =
          f32x4{dq[db][4 * gi] * a.scale, dq[db][4 * gi + 1] * a.scale,
                dq[db][4 * gi + 2] * a.scale, dq[db][4 * gi + 3] * a.scale};
    }
  }
}

// ------------------------------------------------------------------ dkv

// dK^T, dV^T of this lane's key (B operands kf = c*K, vf = V) over query
// tiles 0 .. n_tiles-1; row_of(t, r) gives the token of row r of tile t, or
// kNone.  Ends with a barrier, so the LDS buffers may be reused.
template <int D, typename T, typename RowOf>
__device__ __forceinline__ void key_pass(const Geom& g, const BwdArgs<T>& a, size_t bh,
                                         const bf16x8 (&kf)[D / 16], const bf16x8 (&vf)[D / 16],
                                         int32_t n_tiles, RowOf& row_of, uint16_t (*qt)[kBT * D],
                                         uint16_t (*gt)[kBT * D], float (*lse2)[kBT],
                                         float (*dlt)[kBT], f32x16 (&dk)[D / 32],
                                         f32x16 (&dv)[D / 32]) {
  constexpr int KS = D / 16, DB = D / 32;
  using SG = Stage<D>;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int sc = tid % SG::CPR, sr = tid / SG::CPR;
  const T* qh = a.q + bh * size_t(g.N) * D;
  const T* gh = a.dout + bh * size_t(g.N) * D;
  u32x4 qr[SG::NP], gr[SG::NP];
  float l_r = 0.f, d_r = 0.f;   // threads 0..63: lse2 and delta of row tid
  auto fetch = [&](int32_t t) {
#pragma unroll
    for (int i = 0; i < SG::NP; ++i) {
      const int32_t n = row_of(t, sr + i * SG::RPP);
      qr[i] = gr[i] = u32x4{0, 0, 0, 0};
      if (n != kNone) {
        qr[i] = load8_bf16<T>(qh + size_t(n) * D + 8 * sc);
        gr[i] = load8_bf16<T>(gh + size_t(n) * D + 8 * sc);
      }
    }
    if (tid < kBT) {
      const int32_t n = row_of(t, tid);
      l_r = n != kNone ? kLog2e * a.lse[bh * g.N + n] : INFINITY;
      d_r = n != kNone ? a.delta[bh * g.N + n] : 0.f;
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < SG::NP; ++i) {
      const int off = tile_off<D>(sr + i * SG::RPP, 8 * sc);
      *reinterpret_cast<u32x4*>(&qt[buf][off]) = qr[i];
      *reinterpret_cast<u32x4*>(&gt[buf][off]) = gr[i];
    }
    if (tid < kBT) {
      lse2[buf][tid] = l_r;
      dlt[buf][tid] = d_r;
    }
  };
  fetch(0);
  put(0);
  __syncthreads();
  for (int32_t t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) fetch(t + 1);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // This lane's rows in the accumulator layout: 32 qb + 8 gi + 4 half + 0..3.
      f32x16 s, p;
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2[buf][32 * qb + 8 * gi + 4 * half]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&dlt[buf][32 * qb + 8 * gi + 4 * half]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[4 * gi + i] = -l4[i];
          p[4 * gi + i] = -d4[i];
        }
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag<D>(qt[buf], qb, ks, lane), kf[ks], s, 0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag<D>(gt[buf], qb, ks, lane), vf[ks], p, 0, 0, 0);
      }
      uint32_t pw[8], dsw[8];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = __builtin_amdgcn_exp2f(s[i]), p1 = __builtin_amdgcn_exp2f(s[i + 1]);
        pw[i / 2] = pack_bf16(p0, p1);
        dsw[i / 2] = pack_bf16(p0 * p[i], p1 * p[i + 1]);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const bf16x8 bp = __builtin_bit_cast(
            bf16x8, u32x4{pw[4 * jj], pw[4 * jj + 1], pw[4 * jj + 2], pw[4 * jj + 3]});
        const bf16x8 bds = __builtin_bit_cast(
            bf16x8, u32x4{dsw[4 * jj], dsw[4 * jj + 1], dsw[4 * jj + 2], dsw[4 * jj + 3]});
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tfrag<D>(gt[buf], 2 * qb + jj, db, lane),
                                                           bp, dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tfrag<D>(qt[buf], 2 * qb + jj, db, lane),
                                                           bds, dk[db], 0, 0, 0);
        }
      }
    }
    if (t + 1 < n_tiles) put(buf ^ 1);
    __syncthreads();
  }
}

// This lane's key: c*K and V rows as B operands (zero when invalid).
template <int D, typename T>
__device__ __forceinline__ void load_key(const T* krow, const T* vrow, bool valid, float c,
                                         bf16x8 (&kf)[D / 16], bf16x8 (&vf)[D / 16]) {
  const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    float x[8] = {}, y[8] = {};
    if (valid) {
      load8_f32<T>(krow + 16 * ks + 8 * half, x);
      load8_f32<T>(vrow + 16 * ks + 8 * half, y);
    }
    kf[ks] = scale8(x, c);
    vf[ks] = scale8(y, 1.f);
  }
}

template <int D, typename T>
__global__ __launch_bounds__(kNT) void bwd_dkv_kernel(Geom g, BwdArgs<T> a) {
  constexpr int KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t qt[2][kBT * D];
  __shared__ __attribute__((aligned(16))) uint16_t gt[2][kBT * D];
  __shared__ __attribute__((aligned(16))) float lse2[2][kBT];
  __shared__ __attribute__((aligned(16))) float dlt[2][kBT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int32_t n_kt = (g.M + kRows - 1) / kRows;
  const int32_t blk = xcd_remap(blockIdx.x, a.n_blocks);
  const int32_t kt = blk % n_kt, rest = blk / n_kt;
  const uint32_t w = uint32_t(rest % g.nW);
  const size_t bh = size_t(rest / g.nW);
  const int32_t Mw = window_tokens(g, w);
  if (kt * kRows >= Mw) return;

  const int32_t kslot = kt * kRows + wave * 32 + l32;
  const bool kv = kslot < Mw;
  const int32_t kn = kv ? window_token(g, w, kslot) : 0;
  const size_t krow = (bh * g.N + kn) * size_t(D);
  bf16x8 kf[KS], vf[KS];
  load_key<D, T>(a.k + krow, a.v + krow, kv, a.c, kf, vf);

  // Query segments: this window, then every window that routed to it.
  const int32_t* rl = nullptr;
  int32_t n_seg = 1;
  if (g.topk > 0) {
    const int32_t* off = a.r_off + bh * size_t(g.nW + 1);
    rl = a.r_list + bh * size_t(g.nW) * g.topk + off[w];
    n_seg += off[w + 1] - off[w];
  }
  int32_t n_tiles = 0;
  for (int32_t sg = 0; sg < n_seg; ++sg)
    n_tiles += (window_tokens(g, sg == 0 ? w : uint32_t(rl[sg - 1])) + kBT - 1) / kBT;
  // Tiles are asked for in increasing order (every thread asks for the same
  // tiles), so a cursor over the segments maps tile -> (window, first slot).
  int32_t cur_seg = 0, cur_first = 0, cur_m = Mw;
  uint32_t cur_u = w;
  auto row_of = [&](int32_t t, int r) -> int32_t {
    while (t - cur_first >= (cur_m + kBT - 1) / kBT) {
      cur_first += (cur_m + kBT - 1) / kBT;
      ++cur_seg;
      cur_u = uint32_t(rl[cur_seg - 1]);
      cur_m = window_tokens(g, cur_u);
    }
    const int32_t slot = (t - cur_first) * kBT + r;
    return slot < cur_m ? window_token(g, cur_u, slot) : kNone;
  };

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dk[db] = dv[db] = f32x16{};
  key_pass<D, T>(g, a, bh, kf, vf, n_tiles, row_of, qt, gt, lse2, dlt, dk, dv);

  if (!kv) return;
  // The pooled cell's share: dK_c / P, dV_c / P.
  const float* pk = nullptr;
  const float* pv = nullptr;
  float inv = 0.f;
  if (g.Gp > 0) {
    const int32_t t = kn / (g.Hg * g.Wg), y = (kn / g.Wg) % g.Hg, x = kn % g.Wg;
    const int32_t cell = ((t / g.pt) * g.gy + y / g.ph) * g.gx + x / g.pw;
    pk = a.dkg + (bh * g.G + cell) * size_t(D);
    pv = a.dvg + (bh * g.G + cell) * size_t(D);
    inv = 1.f / float(g.pt * g.ph * g.pw);
  }
  float* dkr = a.dk + krow;
  float* dvr = a.dv + krow;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int d = 32 * db + 8 * gi + 4 * half;
      f32x4 ok = {dk[db][4 * gi] * a.scale, dk[db][4 * gi + 1] * a.scale,
                  dk[db][4 * gi + 2] * a.scale, dk[db][4 * gi + 3] * a.scale};
      f32x4 ov = {dv[db][4 * gi], dv[db][4 * gi + 1], dv[db][4 * gi + 2], dv[db][4 * gi + 3]};
      if (pk) {
        const f32x4 ck = *reinterpret_cast<const f32x4*>(pk + d);
        const f32x4 cv = *reinterpret_cast<const f32x4*>(pv + d);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ok[i] += ck[i] * inv;
          ov[i] += cv[i] * inv;
        }
      }
      *reinterpret_cast<f32x4*>(dkr + d) = ok;
      *reinterpret_cast<f32x4*>(dvr + d) = ov;
    }
  }
}

template <int D, typename T>
__global__ __launch_bounds__(kNT) void bwd_dkv_global_kernel(Geom g, BwdArgs<T> a) {
  constexpr int KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t qt[2][kBT * D];
  __shared__ __attribute__((aligned(16))) uint16_t gt[2][kBT * D];
  __shared__ __attribute__((aligned(16))) float lse2[2][kBT];
  __shared__ __attribute__((aligned(16))) float dlt[2][kBT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int32_t n_gt = (g.G + kRows - 1) / kRows;
  const int32_t n_sp = (g.N + kSplit - 1) / kSplit;
  const int32_t blk = blockIdx.x;
  const int32_t sp = blk % n_sp, rest = blk / n_sp;
  const int32_t gtile = rest % n_gt;
  const size_t bh = size_t(rest / n_gt);

  const int32_t row = gtile * kRows + wave * 32 + l32;
  const bool rv = row < g.G;
  const size_t grow = (bh * g.G + (rv ? row : 0)) * size_t(D);
  bf16x8 kf[KS], vf[KS];
  load_key<D, T>(a.kg + grow, a.vg + grow, rv, a.c, kf, vf);

  const int32_t n0 = sp * kSplit, n1 = min(g.N, n0 + kSplit);
  const int32_t n_tiles = (n1 - n0 + kBT - 1) / kBT;
  auto row_of = [&](int32_t t, int r) -> int32_t {
    const int32_t n = n0 + t * kBT + r;
    return n < n1 ? n : kNone;
  };
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dk[db] = dv[db] = f32x16{};
  key_pass<D, T>(g, a, bh, kf, vf, n_tiles, row_of, qt, gt, lse2, dlt, dk, dv);

  if (!rv) return;
  float* dkr = a.dkg + grow;
  float* dvr = a.dvg + grow;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * db + 8 * gi + 4 * half + i;
        atomicAdd(dkr + d, dk[db][4 * gi + i] * a.scale);
        atomicAdd(dvr + d, dv[db][4 * gi + i]);
      }
    }
  }
}

// Inverse route table of one (batch*head): for every window w, the windows i
// whose routed list names w (once per naming, in order of i, then of list
// position), at r_list[r_off[w] .. r_off[w+1]).  Ids are clamped into
// [0, nW) as the forward clamps them.
__global__ __launch_bounds__(kNT) void routers_kernel(Geom g, const int32_t* route, int32_t* r_off,
                                                      int32_t* r_list) {
  const size_t bh = blockIdx.x;
  const int32_t nW = g.nW, K = g.topk;
  const int32_t* rt = route + bh * size_t(nW) * K;
  int32_t* off = r_off + bh * size_t(nW + 1);
  int32_t* lst = r_list + bh * size_t(nW) * K;
  for (int32_t w = threadIdx.x; w < nW; w += kNT) {
    int32_t cnt = 0;
    for (int32_t e = 0; e < nW * K; ++e) cnt += min(uint32_t(rt[e]), uint32_t(nW - 1)) == uint32_t(w);
    off[w + 1] = cnt;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    off[0] = 0;
    for (int32_t w = 0; w < nW; ++w) off[w + 1] += off[w];
  }
  __syncthreads();
  for (int32_t w = threadIdx.x; w < nW; w += kNT) {
    int32_t pos = off[w];
    for (int32_t e = 0; e < nW * K; ++e)
      if (min(uint32_t(rt[e]), uint32_t(nW - 1)) == uint32_t(w)) lst[pos++] = e / K;
  }
}

__global__ __launch_bounds__(kNT) void fill_zero_kernel(float* p, size_t n) {
  for (size_t i = size_t(blockIdx.x) * kNT + threadIdx.x; i < n; i += size_t(gridDim.x) * kNT)
    p[i] = 0.f;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

template <int D, typename T>
hipError_t run_bwd(const Geom& g, BwdArgs<T> a, hipStream_t s) {
  if (g.topk > 0)
    hipLaunchKernelGGL(routers_kernel, dim3(g.BH), dim3(kNT), 0, s, g, a.route, a.r_off, a.r_list);
  const int32_t n_rows = g.BH * g.nW * ((g.M + kRows - 1) / kRows);
  a.n_blocks = n_rows;
  hipLaunchKernelGGL((bwd_dq_kernel<D, T>), dim3(n_rows), dim3(kNT), 0, s, g, a);
  if (g.G > 0) {
    const size_t glob = size_t(g.BH) * g.G * D;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(kNT), 0, s, a.dkg, glob);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(kNT), 0, s, a.dvg, glob);
    const int32_t n_g = g.BH * ((g.G + kRows - 1) / kRows) * ((g.N + kSplit - 1) / kSplit);
    a.n_blocks = n_g;
    hipLaunchKernelGGL((bwd_dkv_global_kernel<D, T>), dim3(n_g), dim3(kNT), 0, s, g, a);
  }
  a.n_blocks = n_rows;
  hipLaunchKernelGGL((bwd_dkv_kernel<D, T>), dim3(n_rows), dim3(kNT), 0, s, g, a);
  return hipGetLastError();
}

}  // namespace

// Workspace: delta [B*H, N] floats, then the inverse route table.
size_t bwd_workspace_bytes(const Geom& g) {
  size_t b = align256(size_t(g.BH) * g.N * 4);
  if (g.topk > 0)
    b += align256(size_t(g.BH) * (g.nW + 1) * 4) + align256(size_t(g.BH) * g.nW * g.topk * 4);
  return b;
}

hipError_t launch_attn_bwd(const basa_plan_s& p, const void* q, const void* k, const void* v,
                           const void* kg, const void* vg, const int32_t* route, const void* out,
                           const float* lse, const void* dout, float* dq, float* dk, float* dv,
                           float* dkg, float* dvg, void* ws, hipStream_t s) {
  const Geom& g = p.g;
  char* wp = static_cast<char*>(ws);
  float* delta = reinterpret_cast<float*>(wp);
  wp += align256(size_t(g.BH) * g.N * 4);
  int32_t* r_off = nullptr;
  int32_t* r_list = nullptr;
  if (g.topk > 0) {
    r_off = reinterpret_cast<int32_t*>(wp);
    wp += align256(size_t(g.BH) * (g.nW + 1) * 4);
    r_list = reinterpret_cast<int32_t*>(wp);
  }
  const float scale = p.scale, c = p.scale * kLog2e;
  auto go = [&](auto dim, auto* tag) -> hipError_t {
    constexpr int D = decltype(dim)::value;
    using T = std::remove_pointer_t<decltype(tag)>;
    BwdArgs<T> a{static_cast<const T*>(q),    static_cast<const T*>(k),
                 static_cast<const T*>(v),    static_cast<const T*>(kg),
                 static_cast<const T*>(vg),   static_cast<const T*>(out),
                 static_cast<const T*>(dout), lse,
                 route,                       dq,
                 dk,                          dv,
                 dkg,                         dvg,
                 delta,                       r_off,
                 r_list,                      scale,
                 c,                           0};
    return run_bwd<D, T>(g, a, s);
  };
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  const bool f32 = p.params.dtype == BASA_F32;
  if (g.D == 64) return f32 ? go(D64{}, (float*)nullptr) : go(D64{}, (__bf16*)nullptr);
  return f32 ? go(D128{}, (float*)nullptr) : go(D128{}, (__bf16*)nullptr);
}

}  // namespace basa
