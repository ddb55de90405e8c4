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
//   dq      one workgroup per 256 queries of one (batch*head, window) -- per
//           128 queries with four waves when the key list is short -- walks
//           the window's key list in the forward's order (K, V tiles through
//           LDS) and accumulates dQ^T in registers.  It also writes delta for
//           the other two kernels.
//   dkv_g   one workgroup per 128 global rows and one range of queries:
//           every query attends every global row, so the range is plain
//           token order.  Each workgroup writes its partial dK^T, dV^T of
//           the range to the workspace; global_reduce_kernel then adds the
//           ranges' partials in range order (no atomics).
//   dkv     one workgroup per 128 keys of one window; walks every query that
//           has those keys in its list: the window's own queries, then the
//           queries of each window that routed to it (an inverse route table
//           is built first).  dK^T and dV^T stay in registers and each key
//           row is written once, with its pooled cell's share added: token n
//           of cell c gets dK_c / P through the mean (the global rows' sums
//           are complete by then).
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
// Tiles.  64 rows of bf16 in the forward's grouped layout, [8-row group][d/32
// block][8 rows][32 elements], the four 16-byte chunks of each 64-byte row
// segment XOR-swizzled by bits 2-3 of the row (the transposing reads follow
// the swizzle lane by lane).  They arrive by direct global -> LDS loads into
// a ring of four buffers, three tiles ahead of use; each buffer is its own
// LDS variable and the loop is unrolled by four, so every buffer index is a
// compile-time constant and the compiler need not wait for loads in flight
// into the other buffers.  Float inputs are first rounded to bf16 copies.
#include <type_traits>

#include "device_common.hpp"

namespace basa {

namespace {

constexpr int kBT = 64;           // rows per LDS tile
constexpr int kNB = 4;            // LDS buffers per tensor (3 tiles ahead)
constexpr int kMaxRoutes = 16;
constexpr int32_t kNone = INT32_MIN;
constexpr float kLog2e = 1.4426950408889634f;
// dq workgroups: 8 waves with a four-deep ring (one per compute unit), or,
// for short key lists, 4 waves with double buffering (two per compute unit,
// so that one's start overlaps the other's loop).
constexpr int kShortList = 32;    // key tiles below which dq takes 4 waves
constexpr int kNWk = 4;           // waves per dkv / dkv_g workgroup (two per compute unit)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
using I0 = std::integral_constant<int, 0>;
using I1 = std::integral_constant<int, 1>;
using I2 = std::integral_constant<int, 2>;
using I3 = std::integral_constant<int, 3>;

// s_waitcnt vmcnt(n) with the other counters left open (gfx9 encoding: vmcnt
// bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Waits until at most n tiles of PER loads each are in flight (n <= 2).
template <int PER>
__device__ __forceinline__ void wait_tiles(int n) {
  if (n <= 0) wait_vmcnt<0>();
  else if (n == 1) wait_vmcnt<PER>();
  else wait_vmcnt<2 * PER>();
}

// Workgroup barrier without a memory fence: LDS accesses of this wave are
// complete (lgkmcnt), tile loads are ordered by the explicit vmcnt waits.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// Element x of row r of a tile.
template <int D>
__device__ __forceinline__ int tile_off(int r, int x) {
  return (r >> 3) * (8 * D) + (x >> 5) * 256 + (r & 7) * 32 +
         8 * (((x >> 3) ^ (r >> 2)) & 3) + (x & 7);
}

// Per-lane element offsets of the fragment reads inside a tile; everything
// else in a fragment address is a compile-time immediate.
//   frag (A operand of rows 32 blk + l32, k step ks, 8 consecutive elements):
//     tile_off(32 blk + l32, 16 ks + 8 half) = f[ks & 1] + (ks / 2) 256 + blk 32 D
//     (the swizzle term depends on the lane and the parity of ks only);
//   tfrag (A operand of X^T for d block db and 16-row sub-tile st): lane
//     (g16, s16) reads 4 elements of row 16 st + 4 (g16 / 2) + s16 / 4 at
//     t_lo + st 16 D + db 256, and of that row + 8 at t_hi + st 16 D + db 256;
//     the transposing read hands each lane one d column of four rows, in the
//     row order in which the products' accumulator layout holds the B side.
template <int D>
struct FragBase {
  int f0, f1, t_lo, t_hi;
  __device__ __forceinline__ explicit FragBase(int lane) {
    const int l32 = lane & 31, half = lane >> 5, sw = (l32 >> 2) & 3;
    const int row = (l32 >> 3) * (8 * D) + (l32 & 7) * 32;
    f0 = row + 8 * (half ^ sw);
    f1 = row + 8 * ((2 + half) ^ sw);
    const int g16 = lane >> 4, s16 = lane & 15;
    const int rl = 4 * (g16 >> 1) + (s16 >> 2);          // row inside the 8-row group
    const int c = 2 * (g16 & 1) + ((s16 & 3) >> 1);      // 16-byte chunk of the segment
    const int e = 4 * (s16 & 1);                          // element inside the chunk
    t_lo = rl * 32 + 8 * (c ^ (g16 >> 1)) + e;
    t_hi = 8 * D + rl * 32 + 8 * (c ^ ((g16 >> 1) + 2)) + e;
  }
};

template <int D>
__device__ __forceinline__ bf16x8 frag(const uint16_t* t, const FragBase<D>& fb, int blk, int ks) {
  return *reinterpret_cast<const bf16x8*>(t + (ks & 1 ? fb.f1 : fb.f0) + (ks >> 1) * 256 +
                                          blk * (32 * D));
}

template <int D>
__device__ __forceinline__ bf16x8 tfrag(const uint16_t* t, const FragBase<D>& fb, int st, int db) {
  const uint16_t* at = t + st * (16 * D) + db * 256;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(at + fb.t_lo));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(at + fb.t_hi));
  return __builtin_bit_cast(
      bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                    __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
}

// Direct loads of a tile by NWV waves: load u (u = wave, wave + NWV, ...)
// fills 1 KB of the tile (two d blocks of one 8-row group) at a wave-uniform
// address, lane l writing bytes 16 l .. 16 l + 15, so each lane fetches the
// chunk that the swizzle puts in its slot.
template <int D, int NWV>
struct TileLoad {
  static constexpr int PER = D / 8 / NWV;  // 1 KB loads per wave, tile and tensor
  static constexpr int GPK = D / 64;       // 1 KB pieces per 8-row group
  static_assert(PER >= 1 && PER * NWV * 8 == D, "loads must cover the tile");
  // Row and first element of this lane's 16 bytes in load u.
  static __device__ __forceinline__ void slot(int u, int lane, int& r, int& x) {
    r = 8 * (u / GPK) + ((lane & 31) >> 2);
    x = 32 * (2 * (u % GPK) + (lane >> 5)) + 8 * ((lane & 3) ^ ((r >> 2) & 3));
  }
};

__device__ __forceinline__ void dma16(const void* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, float* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 4, 0, 0);
}
// The same loads issued from inline asm, for loops that pick their LDS
// buffer at run time: the compiler does not see these as LDS writes, so it
// adds no wait of its own before the loop's LDS reads (such a wait would
// take in every load in flight, the next tile's included).  Every read of
// their data follows an explicit s_waitcnt and a barrier.  M0 holds the
// wave's LDS destination (one wait state before the load); dma16_at takes a
// 32-bit byte offset from a wave-uniform base (the scalar-base form).
__device__ __forceinline__ void dma16_at(const void* base, uint32_t off, const void* dst) {
  const uint32_t m = uint32_t(reinterpret_cast<uintptr_t>(dst));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off),
               "s"(base), "s"(m)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_asm(const void* src, const void* dst) {
  const uint32_t m = uint32_t(reinterpret_cast<uintptr_t>(dst));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(m)
               : "memory", "m0");
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

// Tensors of one call.  q, k, v, kg, vg, dout are bf16 (the caller's, or
// rounded copies of float input); out keeps the caller's type TO.
template <typename TO>
struct BwdArgs {
  const __bf16 *q, *k, *v, *kg, *vg, *dout;
  const TO* out;
  const float* lse;
  const int32_t* route;
  float *dq, *dk, *dv, *dkg, *dvg;
  float* ndelta;            // [B*H, N] workspace: -(dO . O)
  float* nlse2;             // [B*H, N] workspace: -log2(e) * lse
  int32_t* r_off;           // [B*H, nW + 1] inverse route table offsets
  int32_t* r_list;          // [B*H, nW * topk] windows that routed to each window
  float scale, c;           // softmax scale; scale * log2(e)
  int32_t n_blocks;         // workgroups of the launch
  int32_t split;            // queries per dkv_g workgroup (a multiple of 64)
  float* part;              // dkv_g partial sums, one block per workgroup
  int32_t* order;           // [B*H * nW] (bh, window) pairs, most routed first
  const float* sentinel;    // {-inf, 0}: nlse2 and ndelta of a row that is no query
};

// Source of key j of window w's list, in the forward's order: token n >= 0,
// global row -1 - c, or kNone past the end.  rstart[r] = offset of routed
// window r inside the routed part, rstart[topk] = its length.
template <bool PAD>
__device__ __forceinline__ int32_t key_src(const Geom& g, uint32_t w, int32_t Mw,
                                           const int32_t* routes, const int32_t* rstart,
                                           int32_t j) {
  if (j < Mw) return window_token_t<PAD>(g, w, j);
  j -= Mw;
  if (j < g.G) return -1 - j;
  j -= g.G;
  if (j >= rstart[g.topk]) return kNone;
  int r = 0;
  while (r + 1 < g.topk && j >= rstart[r + 1]) ++r;
  return window_token_t<PAD>(g, uint32_t(routes[r]), j - rstart[r]);
}

// ------------------------------------------------------------------ dq

template <int D, typename TO, bool PAD, int NWV>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(Geom g, BwdArgs<TO> a) {
  constexpr int KS = D / 16, DB = D / 32, ROWS = 32 * NWV;
  constexpr int NB = NWV == 8 ? 4 : 2;  // ring depth: tiles NB - 1 ahead
  using TL = TileLoad<D, NWV>;
  constexpr int LPT = 2 * TL::PER;  // loads per tile and wave
  constexpr int T34 = NB > 2 ? kBT * D : 1;
  __shared__ __attribute__((aligned(1024))) uint16_t k_t0[kBT * D];
  __shared__ __attribute__((aligned(1024))) uint16_t k_t1[kBT * D];
  __shared__ __attribute__((aligned(1024))) uint16_t k_t2[T34];
  __shared__ __attribute__((aligned(1024))) uint16_t k_t3[T34];
  __shared__ __attribute__((aligned(1024))) uint16_t v_t0[kBT * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_t1[kBT * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_t2[T34];
  __shared__ __attribute__((aligned(1024))) uint16_t v_t3[T34];
  auto k_tile = [&](auto s) -> uint16_t* {
    constexpr int S = decltype(s)::value % NB;
    if constexpr (S == 0) return k_t0;
    else if constexpr (S == 1) return k_t1;
    else if constexpr (S == 2) return k_t2;
    else return k_t3;
  };
  auto v_tile = [&](auto s) -> uint16_t* {
    constexpr int S = decltype(s)::value % NB;
    if constexpr (S == 0) return v_t0;
    else if constexpr (S == 1) return v_t1;
    else if constexpr (S == 2) return v_t2;
    else return v_t3;
  };
  __shared__ int32_t routes[kMaxRoutes];
  __shared__ int32_t rstart[kMaxRoutes + 1];
  __shared__ int32_t routes_bad;     // a route id of this window is out of range
  __shared__ int32_t codes[2][kBT];  // row codes of tiles t + 3 and t + 4

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int32_t n_qt = (g.M + ROWS - 1) / ROWS;
  const int32_t blk = xcd_remap(blockIdx.x, a.n_blocks);
  const int32_t qt = blk % n_qt, rest = blk / n_qt;
  const uint32_t w = uint32_t(rest % g.nW);
  const size_t bh = size_t(rest / g.nW);
  const int32_t Mw = window_tokens(g, w);
  if (qt * ROWS >= Mw) return;

  // Routed window ids and the offsets of their segments.  As in the
  // forward, an id outside [0, nW) is never an address (window 0 stands in)
  // and makes the window's dq rows NaN.
  bool route_bad = false;
  if (tid < g.topk) {
    const int32_t r = a.route[(bh * g.nW + w) * g.topk + tid];
    route_bad = uint32_t(r) >= uint32_t(g.nW);
    routes[tid] = route_bad ? 0 : r;
  }
  if (tid < 64) {
    const bool any_bad = __any(route_bad);
    if (tid == 0) routes_bad = any_bad;
  }
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

  // Key tile t into a ring buffer: K and V rows of the key list (rows past
  // its end read token 0 and are masked).
  const __bf16* kh = a.k + bh * size_t(g.N) * D;
  const __bf16* vh = a.v + bh * size_t(g.N) * D;
  const __bf16* kgh = a.kg ? a.kg + bh * size_t(g.G) * D : kh;
  const __bf16* vgh = a.vg ? a.vg + bh * size_t(g.G) * D : vh;
  // Row codes of the key list (key_src) are computed one iteration before
  // their tile is requested, one row per lane of wave 0, into a two-slot LDS
  // table: the requests then need one LDS read per row instead of the index
  // arithmetic, which keeps the loop's registers (and so its waits) down.
  auto key_of = [&](int32_t j) { return j < L ? key_src<PAD>(g, w, Mw, routes, rstart, j) : kNone; };
  auto fill_codes = [&](int32_t t) {
    if (wave == 0) codes[t & 1][lane] = key_of(t * kBT + lane);
  };
  auto request = [&](int32_t src, int x, uint16_t* kb, uint16_t* vb, int u) {
    const bool glob = src != kNone && src < 0;
    const size_t row = src == kNone ? 0 : size_t(glob ? -1 - src : src);
    dma16((glob ? kgh : kh) + row * D + x, kb + u * 512);
    dma16((glob ? vgh : vh) + row * D + x, vb + u * 512);
  };
  // Tile t from the code table (filled during the previous iteration).
  auto issue = [&](int32_t t, auto slot) {
    uint16_t* kb = k_tile(slot);
    uint16_t* vb = v_tile(slot);
#pragma unroll
    for (int i = 0; i < TL::PER; ++i) {
      const int u = wave + NWV * i;
      int r, x;
      TL::slot(u, lane, r, x);
      request(codes[t & 1][r], x, kb, vb, u);
    }
  };
  auto exists = [&](int32_t t) { return int(t < n_tiles); };
  // The first NB - 1 tiles go out through the same table, two slots at a time.
  fill_codes(0);
  if (exists(1)) fill_codes(1);
  lds_barrier();
  issue(0, I0{});
  if constexpr (NB > 2) {
    if (exists(1)) issue(1, I1{});
    lds_barrier();
    if (exists(2)) fill_codes(2);
    lds_barrier();
    if (exists(2)) issue(2, I2{});
    if (exists(3)) fill_codes(3);
  }

  // This lane's query (lanes l32 and l32 + 32 share it, each holding half of
  // every 16-element k step), loaded while the first tiles are in flight.
  const int32_t qs = qt * ROWS + wave * 32 + l32;
  const bool qv = qs < Mw;
  const int32_t qn = qv ? window_token_t<PAD>(g, w, qs) : 0;
  const size_t qrow = (bh * g.N + qn) * size_t(D);
  bf16x8 qf[KS], gf[KS];
  float dsum = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float x[8] = {}, y[8] = {}, o[8] = {};
    if (qv) {
      load8_f32<__bf16>(a.q + qrow + 16 * ks + 8 * half, x);
      load8_f32<__bf16>(a.dout + qrow + 16 * ks + 8 * half, y);
      load8_f32<TO>(a.out + qrow + 16 * ks + 8 * half, o);
    }
    qf[ks] = scale8(x, a.c);
    gf[ks] = scale8(y, 1.f);
#pragma unroll
    for (int e = 0; e < 8; ++e) dsum += y[e] * o[e];
  }
  const float delta = pair_sum(dsum);
  // Accumulator inputs of the two products, splatted at each use (holding
  // the splats would take 32 registers across the loop).
  const float s_in = qv ? -kLog2e * a.lse[bh * g.N + qn] : -INFINITY;
  const float p_in = -delta;
  // The key passes take both as their products' accumulator inputs, stored
  // here already negated and scaled (every token is a query of one window).
  if (qv && half == 0) {
    a.ndelta[bh * g.N + qn] = p_in;
    a.nlse2[bh * g.N + qn] = s_in;
  }

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x16{};
  const FragBase<D> fb(lane);

  // masked: the tile may hold keys past the end of the list (their P is
  // set to 0); a full tile (every key < L) skips the per-key tests.
  auto compute = [&](const uint16_t* kt, const uint16_t* vt, int32_t t,
                     auto masked) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked)::value;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int32_t j0 = t * kBT + 32 * kb;
      if (kMasked && j0 >= L) break;
      f32x16 s = splat16(s_in), p = splat16(p_in);
      // One fragment pair ahead of the products (bounds the registers).
      bf16x8 ka = frag<D>(kt, fb, kb, 0), va = frag<D>(vt, fb, kb, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 kn = ka, vn = va;
        if (ks + 1 < KS) {
          kn = frag<D>(kt, fb, kb, ks + 1);
          vn = frag<D>(vt, fb, kb, ks + 1);
        }
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s, 0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, gf[ks], p, 0, 0, 0);
        ka = kn;
        va = vn;
        __builtin_amdgcn_sched_barrier(0);
      }
      // Lane (query, half) holds keys j0 + 8 gi + 4 half + 0..3 at 4 gi + 0..3.
      uint32_t dsw[8];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const int32_t key = j0 + 8 * (i >> 2) + 4 * half + (i & 3);
        const float p0 = !kMasked || key < L ? __builtin_amdgcn_exp2f(s[i]) : 0.f;
        const float p1 = !kMasked || key + 1 < L ? __builtin_amdgcn_exp2f(s[i + 1]) : 0.f;
        dsw[i / 2] = pack_bf16(p0 * p[i], p1 * p[i + 1]);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const bf16x8 bds = __builtin_bit_cast(
            bf16x8, u32x4{dsw[4 * jj], dsw[4 * jj + 1], dsw[4 * jj + 2], dsw[4 * jj + 3]});
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tfrag<D>(kt, fb, 2 * kb + jj, db),
                                                           bds, dq[db], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  // Iteration t (t % NB == S): tile t + NB - 1 is requested into the buffer
  // that iteration t - 1 read; tile t + 1 must have landed before the barrier.
  // deep: every tile the iteration requests or waits for exists (t + NB <
  // n_tiles), so the tests and the wait count are constants.
  auto iteration = [&](auto slot, int32_t t, auto masked,
                       auto deep) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    constexpr bool kDeep = decltype(deep)::value;
    if (kDeep || t + NB - 1 < n_tiles) issue(t + NB - 1, std::integral_constant<int, S + NB - 1>{});
    if (kDeep || t + NB < n_tiles) fill_codes(t + NB);
    compute(k_tile(slot), v_tile(slot), t, masked);
    if constexpr (NB > 2) {
      if constexpr (kDeep) wait_tiles<LPT>(2);
      else wait_tiles<LPT>(exists(t + 2) + exists(t + 3));
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
  };
  if constexpr (NB > 2) wait_tiles<LPT>(exists(1) + exists(2));
  else wait_vmcnt<0>();
  lds_barrier();
  // Trips of NB full tiles run unmasked (a slot index per iteration stays a
  // constant); the rest, up to NB - 1 full tiles and a partial one, masked.
  using NoMask = std::false_type;
  using Mask = std::true_type;
  using Deep = std::true_type;
  using Shallow = std::false_type;
  const int32_t n_full = L / kBT;
  int32_t t = 0;
  for (; t + NB <= n_full && t + 2 * NB - 1 < n_tiles; t += NB) {
    iteration(I0{}, t, NoMask{}, Deep{});
    iteration(I1{}, t + 1, NoMask{}, Deep{});
    if constexpr (NB > 2) {
      iteration(I2{}, t + 2, NoMask{}, Deep{});
      iteration(I3{}, t + 3, NoMask{}, Deep{});
    }
  }
  for (; t + NB <= n_full; t += NB) {
    iteration(I0{}, t, NoMask{}, Shallow{});
    iteration(I1{}, t + 1, NoMask{}, Shallow{});
    if constexpr (NB > 2) {
      iteration(I2{}, t + 2, NoMask{}, Shallow{});
      iteration(I3{}, t + 3, NoMask{}, Shallow{});
    }
  }
  for (; t < n_tiles; t += NB) {
    iteration(I0{}, t, Mask{}, Shallow{});
    if (t + 1 < n_tiles) iteration(I1{}, t + 1, Mask{}, Shallow{});
    if constexpr (NB > 2) {
      if (t + 2 < n_tiles) iteration(I2{}, t + 2, Mask{}, Shallow{});
      if (t + 3 < n_tiles) iteration(I3{}, t + 3, Mask{}, Shallow{});
    }
  }

  if (!qv) return;
  const float sc = routes_bad ? __uint_as_float(0x7fc00000u) : a.scale;
  // Lane (query, half) holds d = 32 db + 8 gi + 4 half + 0..3 of its row.
  float* dst = a.dq + qrow;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * gi + 4 * half) =
          f32x4{dq[db][4 * gi] * sc, dq[db][4 * gi + 1] * sc,
                dq[db][4 * gi + 2] * sc, dq[db][4 * gi + 3] * sc};
    }
  }
}

// ------------------------------------------------------------------ dkv

// LDS of one key pass: two buffers (one tile ahead) of Q and dO tiles and
// of the tile rows' lse2 and delta.  At 68 KB two workgroups share a compute
// unit, which hides more latency here than a deeper ring would.
template <int D>
struct KeyLds {
  uint16_t qt[2][kBT * D];
  uint16_t gt[2][kBT * D];
  float lse2[2][kBT];     // -log2(e) * lse of the tile's rows
  float dlt[2][kBT];      // -(dO . O) of the tile's rows
  int32_t codes[2][kBT];  // query tokens of tiles t + 1 and t + 2
};

// Waits for this wave's loads (the direct-to-LDS ones included), then for
// the whole workgroup.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// dK^T, dV^T of this lane's key (B operands kf = c*K, vf = V) over query
// tiles 0 .. n_tiles-1; row_of(t, r) gives the token of row r of tile t, or
// kNone, and is asked for tiles in increasing order.
template <int D, int NWV, typename TO, typename RowOf>
__device__ __forceinline__ void key_pass(const Geom& g, const BwdArgs<TO>& a, size_t bh,
                                         const bf16x8 (&kf)[D / 16], const bf16x8 (&vf)[D / 16],
                                         int32_t n_tiles, RowOf& row_of, KeyLds<D>& sm,
                                         f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32]) {
  constexpr int KS = D / 16, DB = D / 32;
  using TL = TileLoad<D, NWV>;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const FragBase<D> fb(lane);
  const __bf16* qh = a.q + bh * size_t(g.N) * D;
  const __bf16* gh = a.dout + bh * size_t(g.N) * D;
  // Rows that are no query read token 0's Q and dO, with -log2(e) lse =
  // -inf and -delta = 0 (the sentinel pair), so their P and dS are 0.  The rows'
  // tokens come from a two-slot LDS table that lane r of wave 0 fills one
  // iteration ahead (row_of runs there only, keeping the loop's registers
  // down).  lse and delta arrive by direct loads too: a plain load used in
  // the loop would have to wait for every tile load issued before it.
  auto fill = [&](int32_t t) {
    if (wave == 0) sm.codes[t & 1][lane] = row_of(t, lane);
  };
  auto fetch = [&](int32_t t, int buf) {
    const int32_t* code = sm.codes[t & 1];
#pragma unroll
    for (int i = 0; i < TL::PER; ++i) {
      const int u = wave + NWV * i;
      int r, x;
      TL::slot(u, lane, r, x);
      const int32_t n = code[r];
      // A 32-bit byte offset from the workgroup-uniform base (a head holds
      // at most 2^24 tokens of 256 bytes): the loads take the scalar-base
      // form and no per-lane 64-bit pointer lives across the loop.
      const uint32_t off = uint32_t(n != kNone ? n : 0) * uint32_t(2 * D) + uint32_t(2 * x);
      dma16_at(qh, off, &sm.qt[buf][u * 512]);
      dma16_at(gh, off, &sm.gt[buf][u * 512]);
    }
    if (wave == 0) {
      const int32_t n = code[lane];
      dma4_asm(n != kNone ? a.nlse2 + bh * g.N + n : a.sentinel, sm.lse2[buf]);
      dma4_asm(n != kNone ? a.ndelta + bh * g.N + n : a.sentinel + 1, sm.dlt[buf]);
    }
  };
  fill(0);
  if (n_tiles > 1) fill(1);
  __syncthreads();
  fetch(0, 0);
  tile_barrier();
  for (int32_t t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) fetch(t + 1, buf ^ 1);
    if (t + 2 < n_tiles) fill(t + 2);
    const uint16_t* qt = sm.qt[buf];
    const uint16_t* gt = sm.gt[buf];
#pragma unroll 1
    for (int qb = 0; qb < 2; ++qb) {
      // This lane's rows in the accumulator layout: 32 qb + 8 gi + 4 half + 0..3.
      f32x16 s, p;
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[buf][32 * qb + 8 * gi + 4 * half]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dlt[buf][32 * qb + 8 * gi + 4 * half]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[4 * gi + i] = l4[i];
          p[4 * gi + i] = d4[i];
        }
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag<D>(qt, fb, qb, ks), kf[ks], s, 0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag<D>(gt, fb, qb, ks), vf[ks], p, 0, 0, 0);
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
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tfrag<D>(gt, fb, 2 * qb + jj, db), bp,
                                                           dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tfrag<D>(qt, fb, 2 * qb + jj, db), bds,
                                                           dk[db], 0, 0, 0);
        }
      }
    }
    tile_barrier();
  }
}

// This lane's key: c*K and V rows as B operands (zero when invalid).
template <int D>
__device__ __forceinline__ void load_key(const __bf16* krow, const __bf16* vrow, bool valid,
                                         float c, bf16x8 (&kf)[D / 16], bf16x8 (&vf)[D / 16]) {
  const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    float x[8] = {}, y[8] = {};
    if (valid) {
      load8_f32<__bf16>(krow + 16 * ks + 8 * half, x);
      load8_f32<__bf16>(vrow + 16 * ks + 8 * half, y);
    }
    kf[ks] = scale8(x, c);
    vf[ks] = scale8(y, 1.f);
  }
}

template <int D, typename TO, bool PAD>
__global__ __launch_bounds__(64 * kNWk) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkv_kernel(Geom g, BwdArgs<TO> a) {
  constexpr int KS = D / 16, DB = D / 32, NWV = kNWk, ROWS = 32 * NWV;
  __shared__ __attribute__((aligned(1024))) KeyLds<D> sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int32_t n_kt = (g.M + ROWS - 1) / ROWS;
  // With routing, a window's work grows with the windows that routed to it:
  // the (bh, window) pairs run most routed first, so that the last round of
  // the launch holds the light ones.  Without, tiles of one window share an
  // XCD (and its L2).
  int32_t kt, rest;
  if (g.topk > 0) {
    kt = blockIdx.x % n_kt;
    rest = a.order[blockIdx.x / n_kt];
  } else {
    const int32_t blk = xcd_remap(blockIdx.x, a.n_blocks);
    kt = blk % n_kt;
    rest = blk / n_kt;
  }
  const uint32_t w = uint32_t(rest % g.nW);
  const size_t bh = size_t(rest / g.nW);
  const int32_t Mw = window_tokens(g, w);
  if (kt * ROWS >= Mw) return;

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
  // Tiles are asked for in increasing order (every lane asks for the same
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
    return slot < cur_m ? window_token_t<PAD>(g, cur_u, slot) : kNone;
  };

  const int32_t kslot = kt * ROWS + wave * 32 + l32;
  const bool kv = kslot < Mw;
  const int32_t kn = kv ? window_token_t<PAD>(g, w, kslot) : 0;
  const size_t krow = (bh * g.N + kn) * size_t(D);
  bf16x8 kf[KS], vf[KS];
  load_key<D>(a.k + krow, a.v + krow, kv, a.c, kf, vf);

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dk[db] = dv[db] = f32x16{};
  key_pass<D, NWV, TO>(g, a, bh, kf, vf, n_tiles, row_of, sm, dk, dv);

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

template <int D, typename TO>
__global__ __launch_bounds__(64 * kNWk) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkv_global_kernel(Geom g, BwdArgs<TO> a) {
  constexpr int KS = D / 16, DB = D / 32, NWV = kNWk, ROWS = 32 * NWV;
  __shared__ __attribute__((aligned(1024))) KeyLds<D> sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int32_t n_gt = (g.G + ROWS - 1) / ROWS;
  const int32_t n_sp = (g.N + a.split - 1) / a.split;
  const int32_t blk = blockIdx.x;
  const int32_t sp = blk % n_sp, rest = blk / n_sp;
  const int32_t gtile = rest % n_gt;
  const size_t bh = size_t(rest / n_gt);

  const int32_t row = gtile * ROWS + wave * 32 + l32;
  const bool rv = row < g.G;
  const size_t grow = (bh * g.G + (rv ? row : 0)) * size_t(D);
  bf16x8 kf[KS], vf[KS];
  load_key<D>(a.kg + grow, a.vg + grow, rv, a.c, kf, vf);

  const int32_t n0 = sp * a.split, n1 = min(g.N, n0 + a.split);
  const int32_t n_tiles = (n1 - n0 + kBT - 1) / kBT;
  auto row_of = [&](int32_t t, int r) -> int32_t {
    const int32_t n = n0 + t * kBT + r;
    return n < n1 ? n : kNone;
  };
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dk[db] = dv[db] = f32x16{};
  key_pass<D, NWV, TO>(g, a, bh, kf, vf, n_tiles, row_of, sm, dk, dv);

  // Partial sums leave in the accumulator layout, 1 KB per instruction:
  // block (workgroup, tensor, wave), then [db][gi][lane] x 4 floats.
  float* pb = a.part + (size_t(blk) * 2 * NWV + wave) * (DB * 4 * 64 * 4) + 4 * lane;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int at = (db * 4 + gi) * 256;
      *reinterpret_cast<f32x4*>(pb + at) =
          f32x4{dk[db][4 * gi] * a.scale, dk[db][4 * gi + 1] * a.scale,
                dk[db][4 * gi + 2] * a.scale, dk[db][4 * gi + 3] * a.scale};
      *reinterpret_cast<f32x4*>(pb + NWV * (DB * 4 * 64 * 4) + at) =
          f32x4{dv[db][4 * gi], dv[db][4 * gi + 1], dv[db][4 * gi + 2], dv[db][4 * gi + 3]};
    }
  }
}

// dK, dV of the global rows: the sum over query ranges of the dkv_g partial
// sums, in range order (one thread per 4 elements of [B*H, G, d]).
template <int D>
__global__ __launch_bounds__(256) void global_reduce_kernel(Geom g, const float* part, int32_t n_sp,
                                                            float* dkg, float* dvg) {
  constexpr int NWV = kNWk, ROWS = 32 * NWV, DB = D / 32, BLK = DB * 4 * 64 * 4;
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= size_t(g.BH) * g.G * (D / 4)) return;
  const int d = int(i % (D / 4)) * 4;
  const size_t rowi = i / (D / 4);
  const int32_t row = int32_t(rowi % g.G);
  const size_t bh = rowi / g.G;
  const int32_t n_gt = (g.G + ROWS - 1) / ROWS;
  const int32_t gtile = row / ROWS, wave = (row % ROWS) / 32, l32 = row % 32;
  const int db = d / 32, gi = (d % 32) / 8, half = (d % 8) / 4;
  const size_t within = size_t(wave) * BLK + ((db * 4 + gi) * 64 + l32 + 32 * half) * 4;
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  for (int32_t sp = 0; sp < n_sp; ++sp) {
    const size_t blk = (bh * n_gt + gtile) * n_sp + sp;
    const float* pb = part + blk * 2 * NWV * BLK + within;
    sk += *reinterpret_cast<const f32x4*>(pb);
    sv += *reinterpret_cast<const f32x4*>(pb + NWV * BLK);
  }
  *reinterpret_cast<f32x4*>(dkg + rowi * D + d) = sk;
  *reinterpret_cast<f32x4*>(dvg + rowi * D + d) = sv;
}

// Orders the (bh, window) pairs by the number of windows that routed to
// them, most first (counting sort; ties in no particular order, which only
// moves workgroups in time).  One workgroup.
constexpr int kOrderBuckets = 4096;
__global__ __launch_bounds__(256) void order_kernel(Geom g, const int32_t* r_off, int32_t* order) {
  __shared__ int32_t hist[kOrderBuckets];
  const int32_t n = g.BH * g.nW;
  for (int i = threadIdx.x; i < kOrderBuckets; i += 256) hist[i] = 0;
  __syncthreads();
  auto bucket = [&](int32_t i) {
    const int32_t bh = i / g.nW, w = i % g.nW;
    const int32_t* off = r_off + size_t(bh) * (g.nW + 1);
    return kOrderBuckets - 1 - min(off[w + 1] - off[w], kOrderBuckets - 1);
  };
  for (int32_t i = threadIdx.x; i < n; i += 256) atomicAdd(&hist[bucket(i)], 1);
  __syncthreads();
  // Exclusive scan of the histogram: thread t owns buckets [PER t, PER t + PER),
  // thread 0 scans the 256 chunk sums.
  constexpr int PER = kOrderBuckets / 256;
  __shared__ int32_t part[257];
  const int t = threadIdx.x;
  int32_t sum = 0;
  for (int b = 0; b < PER; ++b) sum += hist[t * PER + b];
  part[t + 1] = sum;
  __syncthreads();
  if (t == 0) {
    part[0] = 0;
    for (int i = 0; i < 256; ++i) part[i + 1] += part[i];
  }
  __syncthreads();
  int32_t acc = part[t];
  for (int b = 0; b < PER; ++b) {
    const int32_t c = hist[t * PER + b];
    hist[t * PER + b] = acc;
    acc += c;
  }
  __syncthreads();
  for (int32_t i = threadIdx.x; i < n; i += 256) order[atomicAdd(&hist[bucket(i)], 1)] = i;
}

// The nlse2 and ndelta of a row that is no query: -inf and 0 (its P and dS
// are then 0).
__global__ __launch_bounds__(64) void sentinel_kernel(float* p) {
  if (threadIdx.x == 0) {
    p[0] = -INFINITY;
    p[1] = 0.f;
  }
}

// Inverse route table of one head: r_off[w] .. r_off[w+1] index the windows
// that routed to w, listed in ascending window order (so the key passes add
// their queries in a fixed order).  The head's route table is staged in LDS
// when it fits (nW * topk <= kRouteStage), the per-window counts and offsets
// stay in LDS, and the offsets come from a chunked scan: thread t sums a
// contiguous chunk of windows, thread 0 scans the 256 chunk sums.
constexpr int kRouteStage = 16384;
constexpr int kMaxRouteWin = 8192;  // the plan's limit on routed windows
__global__ __launch_bounds__(256) void routers_kernel(Geom g, const int32_t* route, int32_t* r_off,
                                                      int32_t* r_list) {
  __shared__ int32_t rt_s[kRouteStage];
  __shared__ int32_t cnt_s[kMaxRouteWin];
  __shared__ int32_t off_s[kMaxRouteWin + 1];
  __shared__ int32_t part_s[257];
  const size_t bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t nW = g.nW, K = g.topk, n = nW * K;
  const int32_t* rt = route + bh * size_t(nW) * K;
  int32_t* off = r_off + bh * size_t(nW + 1);
  int32_t* lst = r_list + bh * size_t(nW) * K;
  const bool staged = n <= kRouteStage;
  // An id outside [0, nW) routes nothing: it maps to -1, which no window
  // matches (the forward and dq make that window's rows NaN).
  auto clamp = [&](int32_t x) { return uint32_t(x) < uint32_t(nW) ? x : -1; };
  if (staged)
    for (int32_t e = tid; e < n; e += 256) rt_s[e] = clamp(rt[e]);
  __syncthreads();
  // The scans read the table in batches (unrolled, the staged and the
  // global form as separate loops): one read at a time would wait out its
  // latency for every entry.
  auto count = [&](auto at) {
    for (int32_t w = tid; w < nW; w += 256) {
      int32_t cnt = 0;
#pragma unroll 16
      for (int32_t e = 0; e < n; ++e) cnt += at(e) == w;
      cnt_s[w] = cnt;
    }
  };
  auto fill = [&](auto at) {
    for (int32_t w = tid; w < nW; w += 256) {
      int32_t pos = off_s[w];
#pragma unroll 16
      for (int32_t e = 0; e < n; ++e)
        if (at(e) == w) lst[pos++] = e / K;
    }
  };
  auto from_lds = [&](int32_t e) { return rt_s[e]; };
  auto from_global = [&](int32_t e) { return clamp(rt[e]); };
  if (staged) count(from_lds); else count(from_global);
  __syncthreads();
  // Chunked exclusive scan of the counts into off_s[0 .. nW].
  const int32_t per = (nW + 255) / 256;
  const int32_t lo = min(nW, tid * per), hi = min(nW, lo + per);
  int32_t sum = 0;
  for (int32_t w = lo; w < hi; ++w) sum += cnt_s[w];
  part_s[tid + 1] = sum;
  __syncthreads();
  if (tid == 0) {
    part_s[0] = 0;
    for (int i = 0; i < 256; ++i) part_s[i + 1] += part_s[i];
  }
  __syncthreads();
  int32_t run = part_s[tid];
  for (int32_t w = lo; w < hi; ++w) {
    off_s[w] = run;
    run += cnt_s[w];
  }
  if (tid == 255) off_s[nW] = part_s[256];
  __syncthreads();
  for (int32_t w = tid; w <= nW; w += 256) off[w] = off_s[w];
  if (staged) fill(from_lds); else fill(from_global);
}

// float -> bf16 (round to nearest even), 8 elements per thread.
__global__ __launch_bounds__(256) void to_bf16_kernel(const float* x, __bf16* y, size_t n8) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n8; i += size_t(gridDim.x) * 256)
    *reinterpret_cast<u32x4*>(y + 8 * i) = load8_bf16<float>(x + 8 * i);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Queries per dkv_g workgroup (a multiple of 64).  The query ranges per row
// tile are chosen so that the workgroups fill whole rounds of the chip's
// 512 slots (256 compute units, two workgroups each): a partial last round
// costs more than the atomics of a few more ranges.  Ranges hold at least
// 1024 queries; without a count that fills 90% of its rounds, one range.
int32_t global_split(const Geom& g) {
  constexpr int64_t kSlots = 512;
  const int64_t tiles = int64_t(g.BH) * ((g.G + 32 * kNWk - 1) / (32 * kNWk));
  const int64_t most = std::max<int64_t>(1, (g.N + 1023) / 1024);
  // The fewest ranges whose workgroups fill at least 90% of their rounds.
  int64_t n_sp = 1;
  for (int64_t k = 1; k <= std::min<int64_t>(most, 64); ++k) {
    const int64_t wgs = tiles * k, rounds = (wgs + kSlots - 1) / kSlots;
    if (10 * wgs >= 9 * rounds * kSlots) {
      n_sp = k;
      break;
    }
  }
  const int64_t per = (g.N + n_sp - 1) / n_sp;
  return int32_t((per + kBT - 1) / kBT * kBT);
}

template <int D, typename TO, bool PAD>
hipError_t run_bwd(const Geom& g, BwdArgs<TO> a, hipStream_t s) {
  hipLaunchKernelGGL(sentinel_kernel, dim3(1), dim3(64), 0, s, const_cast<float*>(a.sentinel));
  if (g.topk > 0) {
    hipLaunchKernelGGL(routers_kernel, dim3(g.BH), dim3(256), 0, s, g, a.route, a.r_off, a.r_list);
    hipLaunchKernelGGL(order_kernel, dim3(1), dim3(256), 0, s, g, a.r_off, a.order);
  }
  if ((g.L + kBT - 1) / kBT < kShortList) {
    const int32_t n_q = g.BH * g.nW * ((g.M + 127) / 128);
    a.n_blocks = n_q;
    hipLaunchKernelGGL((bwd_dq_kernel<D, TO, PAD, 4>), dim3(n_q), dim3(256), 0, s, g, a);
  } else {
    const int32_t n_q = g.BH * g.nW * ((g.M + 255) / 256);
    a.n_blocks = n_q;
    hipLaunchKernelGGL((bwd_dq_kernel<D, TO, PAD, 8>), dim3(n_q), dim3(512), 0, s, g, a);
  }
  if (g.G > 0) {
    const size_t glob = size_t(g.BH) * g.G * D;
    a.split = global_split(g);
    const int32_t n_sp = (g.N + a.split - 1) / a.split;
    const int32_t n_g = g.BH * ((g.G + 32 * kNWk - 1) / (32 * kNWk)) * n_sp;
    a.n_blocks = n_g;
    hipLaunchKernelGGL((bwd_dkv_global_kernel<D, TO>), dim3(n_g), dim3(64 * kNWk), 0, s, g, a);
    hipLaunchKernelGGL(global_reduce_kernel<D>, dim3(uint32_t((glob / 4 + 255) / 256)), dim3(256), 0,
                       s, g, a.part, n_sp, a.dkg, a.dvg);
  }
  const int32_t n_k = g.BH * g.nW * ((g.M + 32 * kNWk - 1) / (32 * kNWk));
  a.n_blocks = n_k;
  hipLaunchKernelGGL((bwd_dkv_kernel<D, TO, PAD>), dim3(n_k), dim3(64 * kNWk), 0, s, g, a);
  return hipGetLastError();
}

// Workspace carve-up: -delta and -log2(e) lse, [B*H, N] floats each (the
// key passes' accumulator inputs, written by dq), the sentinel pair, the inverse
// route table and the order of the (bh, window) pairs, the dkv_g partial
// sums (two tensors x 128 rows x d floats per workgroup), and for float plans
// bf16 copies of q, k, v, d_out [B*H, N, d] and of the global rows
// [B*H, G, d].
struct WsLayout {
  size_t delta, nlse2, sentinel, r_off, r_list, order, part, copies, total;
};

WsLayout ws_layout(const basa_plan_s& p) {
  const Geom& g = p.g;
  WsLayout l{};
  size_t at = 0;
  l.delta = at;
  at += align256(size_t(g.BH) * g.N * 4);
  l.nlse2 = at;
  at += align256(size_t(g.BH) * g.N * 4);
  l.sentinel = at;
  at += 256;
  l.r_off = at;
  if (g.topk > 0) at += align256(size_t(g.BH) * (g.nW + 1) * 4);
  l.r_list = at;
  if (g.topk > 0) at += align256(size_t(g.BH) * g.nW * g.topk * 4);
  l.order = at;
  if (g.topk > 0) at += align256(size_t(g.BH) * g.nW * 4);
  l.part = at;
  if (g.G > 0) {
    const size_t n_sp = (g.N + global_split(g) - 1) / global_split(g);
    const size_t n_g = size_t(g.BH) * ((g.G + 32 * kNWk - 1) / (32 * kNWk)) * n_sp;
    at += align256(n_g * 2 * (32 * kNWk) * g.D * 4);
  }
  l.copies = at;
  if (p.params.dtype == BASA_F32)
    at += 4 * align256(size_t(g.BH) * g.N * g.D * 2) + 2 * align256(size_t(g.BH) * g.G * g.D * 2);
  l.total = at;
  return l;
}

}  // namespace

size_t bwd_workspace_bytes(const basa_plan_s& p) { return ws_layout(p).total; }

hipError_t launch_attn_bwd(const basa_plan_s& p, const void* q, const void* k, const void* v,
                           const void* kg, const void* vg, const int32_t* route, const void* out,
                           const float* lse, const void* dout, float* dq, float* dk, float* dv,
                           float* dkg, float* dvg, void* ws, hipStream_t s) {
  const Geom& g = p.g;
  const WsLayout l = ws_layout(p);
  char* base = static_cast<char*>(ws);
  float* delta = reinterpret_cast<float*>(base + l.delta);
  float* nlse2 = reinterpret_cast<float*>(base + l.nlse2);
  int32_t* r_off = g.topk > 0 ? reinterpret_cast<int32_t*>(base + l.r_off) : nullptr;
  int32_t* r_list = g.topk > 0 ? reinterpret_cast<int32_t*>(base + l.r_list) : nullptr;
  float* part = reinterpret_cast<float*>(base + l.part);
  int32_t* order = g.topk > 0 ? reinterpret_cast<int32_t*>(base + l.order) : nullptr;
  float* sentinel = reinterpret_cast<float*>(base + l.sentinel);
  const float scale = p.scale, c = p.scale * kLog2e;
  const bool f32 = p.params.dtype == BASA_F32;

  const __bf16 *qb, *kb, *vb, *kgb, *vgb, *gb;
  if (f32) {
    // Rounded copies: the products take bf16 operands either way.
    const size_t nt = size_t(g.BH) * g.N * g.D, ng = size_t(g.BH) * g.G * g.D;
    char* at = base + l.copies;
    auto take = [&](size_t n) {
      __bf16* r = reinterpret_cast<__bf16*>(at);
      at += align256(n * 2);
      return r;
    };
    __bf16* c0 = take(nt);
    __bf16* c1 = take(nt);
    __bf16* c2 = take(nt);
    __bf16* c3 = take(nt);
    __bf16* c4 = take(ng);
    __bf16* c5 = take(ng);
    auto conv = [&](const void* x, __bf16* y, size_t n) {
      if (n)
        hipLaunchKernelGGL(to_bf16_kernel, dim3(2048), dim3(256), 0, s,
                           static_cast<const float*>(x), y, n / 8);
    };
    conv(q, c0, nt);
    conv(k, c1, nt);
    conv(v, c2, nt);
    conv(dout, c3, nt);
    conv(kg, c4, ng);
    conv(vg, c5, ng);
    qb = c0;
    kb = c1;
    vb = c2;
    gb = c3;
    kgb = ng ? c4 : nullptr;
    vgb = ng ? c5 : nullptr;
  } else {
    qb = static_cast<const __bf16*>(q);
    kb = static_cast<const __bf16*>(k);
    vb = static_cast<const __bf16*>(v);
    kgb = static_cast<const __bf16*>(kg);
    vgb = static_cast<const __bf16*>(vg);
    gb = static_cast<const __bf16*>(dout);
  }
  auto go = [&](auto dim, auto* tag) -> hipError_t {
    constexpr int D = decltype(dim)::value;
    using TO = std::remove_pointer_t<decltype(tag)>;
    BwdArgs<TO> a{qb, kb, vb, kgb, vgb, gb, static_cast<const TO*>(out), lse, route,
                  dq, dk, dv, dkg, dvg, delta, nlse2, r_off, r_list, scale, c, 0, 0, part, order,
                  sentinel};
    // Plans without short windows take the plain window addressing.
    return g.padded ? run_bwd<D, TO, true>(g, a, s) : run_bwd<D, TO, false>(g, a, s);
  };
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  if (g.D == 64) return f32 ? go(D64{}, (float*)nullptr) : go(D64{}, (__bf16*)nullptr);
  return f32 ? go(D128{}, (float*)nullptr) : go(D128{}, (__bf16*)nullptr);
}

}  // namespace basa
