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
// Work decomposition.  One workgroup = 256 query slots of one (batch*head,
// window), split into eight 32-query blocks, one per wave (two waves per
// SIMD, so that one wave's vector work runs beside the other's matrix
// products); short key lists take four waves and 128 slots, two workgroups
// per CU.  The key list is staged through LDS in tiles of 64 rows; row codes
// of the key list (token n >= 0, global row -1 - c; token 0 past the end) are
// computed per workgroup into an LDS table.  bf16 queries of the eight-wave
// form come in the same way as the tiles (direct loads into LDS) and go to
// registers through the K fragment reads.
//
// Arithmetic per 32-key block j (bf16 matrix cores, v_mfma_f32_32x32x16_bf16):
//   S'^T[32 keys x 32 queries] = K_j (c Q)^T - m        c = scale * log2(e)
//     A = K rows (ds_read_b128), B = c*Q held in registers; the shift m
//     enters as the accumulator input (a constant splat), so the logits come
//     out already shifted, with no per-element vector work;
//   P = exp2(S'), rounded to bf16 for the P.V product; row sums of P in
//     float;
//   O^T[d x 32 queries] += V_j^T P^T      A = V^T fragments read with
//     ds_read_b64_tr_b16 from V rows, B = P straight from the S'^T layout.
// Each lane holds one query per block and 16 of its keys per 32-key block
// (the other 16 sit in lane ^ 32), so the row max needs one permlane swap.
// The transposing read hands each 16-lane group a 16 x 4 block turned on its
// side: source lane 4e + c reads 4 elements of key row e; lane i receives
// element i % 4 of source lanes 4e + i / 4, e = 0..3, i.e. four keys of one
// d column -- the A operand of the P.V product.
//
// Software pipeline.  Block j's step issues the P.V products of block j-1
// and the q.k products of block j+1; the exponentials, packing and row sums
// of S'_j are spread under both.  Tiles arrive by
// direct global -> LDS loads (global_load_lds_dwordx4, no staging
// registers), K four tiles and V three tiles ahead of use.
//
// Shift.  m is the exact maximum of key block 0 and stays fixed for the whole
// key list, so nothing is rescaled inside the loop: P = exp2(S') may exceed
// 1 where later keys score higher, which float represents exactly enough
// while S' <= 64 (P <= 2^64).  A workgroup whose queries see a larger S'
// finds each row's exact maximum with a q.k-only walk of the list and runs
// the list once more with m at that maximum.  The final
// normalisation divides by the sum of the same P, so the result does not
// depend on m.
//
// LDS layouts (bf16, no padding).  K and V tiles are grouped by 8 rows and
// d-blocked inside a group, [8 row groups][d/32 blocks][8 rows][32
// elements], so every fragment address is one per-lane base plus an
// immediate.  In K the four 16-byte chunks of a 64-byte row segment are
// XOR-swizzled by bits 2-3 of the row: the 16 rows one pass of a K fragment
// read touches then fill all banks once.  In V the 4 rows x 64 bytes a
// transposing read touches are 256 contiguous bytes.  A direct load writes
// 1 KB contiguously, two d blocks of one row group, so each of its rows is
// fetched as one 128-byte span (half as many memory requests per tile as
// 64-byte spans); each lane fetches whatever chunk belongs in its slot.
//
// Output.  The O^T accumulators give each lane 8-byte pieces of 32 rows; the
// rows are written through LDS instead (store_rows_bf16), 16 bytes per lane
// and whole rows per instruction.
#include <type_traits>

#include "device_common.hpp"

namespace basa {

namespace {

constexpr int kQB = 1;            // 32-query blocks per wave
constexpr int BQ = 256;           // query slots per workgroup of the eight-wave form
constexpr int BK = 64;            // key rows per LDS tile
static_assert(BQ == kAttnQueryTile, "the plan sizes text-query work by this tile");
constexpr int CE = 512;           // row codes per table chunk
constexpr int TPC = CE / BK;      // tiles per chunk
// Key lists of at most this many tiles run in the four-wave form (two
// workgroups per CU, so that one's start and end overlap the other's loop).
constexpr int kHalfFormMaxTiles = 12;
constexpr int kMaxTopk = 16;
constexpr float kSumLimit = 0x1p64f;  // largest row sum a pass accepts
constexpr int kMaxPasses = 2;  // a pass that overflows is followed by an exact one

// The direct global -> LDS loads of the tiles are issued from inline
// assembly, so the compiler does not track them.  Tracking them, it could not
// tell the ring buffers apart across the loop's back edge and waited for
// every load in flight before some LDS reads (two iterations in four),
// draining the prefetch ring.  Their ordering comes from the explicit waits
// below instead, each an asm statement with a memory clobber, so that no LDS
// access moves across a wait, a barrier or a load issue.

// s_waitcnt vmcnt(N): at most N vector-memory requests of this wave remain.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without a memory fence.  __syncthreads() also waits for
// every vector-memory request of the wave (vmcnt(0)), which would drain the
// global -> LDS loads in flight for later tiles; here LDS accesses of this
// wave (lgkmcnt) are completed and the tile loads are ordered by explicit
// vmcnt waits.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16 bytes per lane from global memory into LDS at lds + 16 * lane (M0 holds
// the wave's LDS base; one wait state between setting M0 and the load).
__device__ __forceinline__ void dma16(const void* src, const void* lds) {
  const uint32_t m = uint32_t(reinterpret_cast<uintptr_t>(lds));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src),
               "s"(m)
               : "memory", "m0");
}

// Waits until at most n * PER vector-memory requests of this wave remain.
template <int PER>
__device__ __forceinline__ void wait_vmcnt_tiles(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<PER>(); break;
    case 2: wait_vmcnt<2 * PER>(); break;
    case 3: wait_vmcnt<3 * PER>(); break;
    default: wait_vmcnt<4 * PER>(); break;
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

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
  int32_t branches;  // key-list segments attended: 1 local, 2 global rows, 4 routed
  int32_t n_split;   // text queries: passes over consecutive parts of the key list
  int32_t split_len; // keys per part (the last part may be shorter)
  // Workgroup id -> (query tile, window or text part, batch*head): division
  // by n_qt and by nW (text queries: n_split).
  FastDiv f_nqt, f_nw;
};

// The part of the slot -> token map of window w (window_token_t) that does
// not depend on the slot: the first position of the window (shift applied,
// not yet wrapped) and the divisors of its slot numbering.  The window of a
// workgroup is uniform, so this runs once on the scalar unit; each slot then
// costs two divisions by multiply-high and the wrap.
struct WinBase {
  int32_t t0, y0, x0;
  uint32_t slab, row;      // slots per time step, per row (short windows fewer)
  FastDiv f_slab, f_row;   // division by them
};

template <bool PAD>
__device__ __forceinline__ WinBase win_base(const Geom& g, uint32_t w) {
  const uint32_t wa = g.f_nwyx.div(w);
  const uint32_t wr = w - wa * uint32_t(g.nWy * g.nWx);
  const uint32_t wb = g.f_nwx.div(wr);
  const uint32_t wc = wr - wb * uint32_t(g.nWx);
  WinBase b;
  b.t0 = int32_t(wa) * g.wt + g.st;
  b.y0 = int32_t(wb) * g.wh + g.sy;
  b.x0 = int32_t(wc) * g.ww + g.sx;
  if constexpr (!PAD) {
    b.slab = uint32_t(g.wh * g.ww);
    b.row = uint32_t(g.ww);
    b.f_slab = g.f_whw;
    b.f_row = g.f_ww;
  } else {
    const bool sy = wb == uint32_t(g.nWy - 1), sx = wc == uint32_t(g.nWx - 1);
    b.row = uint32_t(sx ? g.rx : g.ww);
    b.slab = uint32_t(sy ? g.ry : g.wh) * b.row;
    b.f_slab = pick_div(sy, pick_div(sx, g.f_ryr, g.f_ryw), pick_div(sx, g.f_whr, g.f_whw));
    b.f_row = pick_div(sx, g.f_rx, g.f_ww);
  }
  return b;
}

// Token of slot s of the window with base b (the same map as window_token_t).
__device__ __forceinline__ int32_t win_token(const Geom& g, const WinBase& b, uint32_t s) {
  const uint32_t it = b.f_slab.div(s);
  const uint32_t sr = s - it * b.slab;
  const uint32_t iy = b.f_row.div(sr);
  const uint32_t ix = sr - iy * b.row;
  int32_t t = b.t0 + int32_t(it), y = b.y0 + int32_t(iy), x = b.x0 + int32_t(ix);
  t -= t >= g.T ? g.T : 0;
  y -= y >= g.Hg ? g.Hg : 0;
  x -= x >= g.Wg ? g.Wg : 0;
  return (t * g.Hg + y) * g.Wg + x;
}

// Row code of key j of window `win`'s key list (wb: its base), which holds L keys: the
// lenL slots of the window itself, the lenG global rows, then each routed
// window's slots (a branch-split pass keeps some of the three segments; the
// joint pass has lenL = the window's slots and lenG = G).  With short
// windows (PAD) routed window r starts at offset rstart[r] of the routed
// part; otherwise every window has M slots.  The text-query list (TEXT) is
// every image token in token order, then the text rows, which follow the Gp
// pooled cells among the global rows; a pass over one split of it starts at
// key `win` of that list.
template <bool PAD, bool TEXT = false>
__device__ __forceinline__ int32_t key_code(const Geom& g, uint32_t win, const WinBase& wb,
                                            int32_t lenL, int32_t lenG, int32_t L,
                                            const int32_t* routes, const int32_t* rstart,
                                            int32_t j) {
  // Past the end: token 0, a row in bounds whose keys the masking removes.
  if (j >= L) return 0;
  if constexpr (TEXT) {
    j += int32_t(win);
    return j < g.N ? j : -1 - (g.Gp + (j - g.N));
  }
  if (j < lenL) return win_token(g, wb, j);
  j -= lenL;
  if (j < lenG) return -1 - j;
  j -= lenG;
  if constexpr (!PAD) {
    const uint32_t r = g.f_M.div(j);
    return window_token_t<false>(g, routes[r], j - r * uint32_t(g.M));
  } else {
    int r = 0;
    while (r + 1 < g.topk && j >= rstart[r + 1]) ++r;
    return window_token_t<true>(g, routes[r], j - rstart[r]);
  }
}

// 8 consecutive query elements as loaded (QRaw) and scaled by c, rounded
// once to bf16 (4 packed words).
template <typename T>
struct QRawT;
template <>
struct QRawT<__bf16> { typedef u32x4 type; };
template <>
struct QRawT<float> { struct type { f32x4 lo, hi; }; };
template <typename T>
using QRaw = typename QRawT<T>::type;

__device__ __forceinline__ u32x4 load_q_raw(const __bf16* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ QRaw<float> load_q_raw(const float* p) {
  return QRaw<float>{*reinterpret_cast<const f32x4*>(p), *reinterpret_cast<const f32x4*>(p + 4)};
}

template <typename T>
__device__ __forceinline__ u32x4 scale_q(const QRaw<T>& r, float c);
template <>
__device__ __forceinline__ u32x4 scale_q<__bf16>(const u32x4& u, float c) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf16(bf16_lo(u[i]) * c, bf16_hi(u[i]) * c);
  return r;
}
template <>
__device__ __forceinline__ u32x4 scale_q<float>(const QRaw<float>& q, float c) {
  return u32x4{pack_bf16(q.lo[0] * c, q.lo[1] * c), pack_bf16(q.lo[2] * c, q.lo[3] * c),
               pack_bf16(q.hi[0] * c, q.hi[1] * c), pack_bf16(q.hi[2] * c, q.hi[3] * c)};
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

// Pins a value to this point of the instruction stream: the empty asm reads
// and writes the register, so the computation that produced it cannot sink
// past the scheduling barrier that follows (it would otherwise be moved next
// to its first use, into a later basic block, and lose its overlap with the
// matrix products).
__device__ __forceinline__ void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ f32x16 splat16(float x) {
  f32x16 r;
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = x;
  return r;
}

__device__ __forceinline__ float max16(const f32x16& s) {
  float m = fmaxf(s[0], s[1]);
#pragma unroll
  for (int i = 2; i < 16; i += 2) m = fmaxf(fmaxf(m, s[i]), s[i + 1]);
  return m;
}

// Writes one wave's 32-query output block (bf16) as whole rows.  In the
// O^T accumulators lane (q, h) holds, per d block db and group g4, the four
// values d = 32*db + 8*g4 + 4*h + 0..3 of query q: stored directly that is
// 8 bytes of each of 32 rows per instruction, which the memory pipeline
// takes a request per row for.  Instead the block is staged in stg (32 x D
// bf16 of LDS, private to the wave) and read back so that D/8 lanes cover one
// row with 16 bytes each.  Staging layout: 16-byte chunk c of row r sits at
// chunk c ^ ((r / RP) % CPR), its two 8-byte halves swapped for rows 16..31;
// both the 8-byte writes and the 16-byte reads are then free of bank
// conflicts.  o[db * QB + b] is the accumulator of d block db; qn is the
// token of query l32 (lane l32 and l32 + 32 hold the same); rows at or past
// rows_valid are not written.
template <int D, int QB>
__device__ __forceinline__ void store_rows_bf16(const f32x16* o, int b, float inv, uint16_t* stg,
                                                __bf16* out, int32_t qn, int32_t rows_valid,
                                                int lane) {
  constexpr int DB = D / 32, CPR = D / 8, RP = 128 / D, RPI = 64 / CPR, NI = 32 / RPI;
  const int l32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x16& acc = o[db * QB + b];
      const int pc = (4 * db + g4) ^ ((l32 / RP) % CPR);
      const int h = half ^ (l32 >> 4);
      *reinterpret_cast<u32x2*>(stg + l32 * D + 8 * pc + 4 * h) =
          u32x2{pack_bf16(acc[4 * g4] * inv, acc[4 * g4 + 1] * inv),
                pack_bf16(acc[4 * g4 + 2] * inv, acc[4 * g4 + 3] * inv)};
    }
  }
  // Every token and row piece is read back before the first store, so the
  // LDS round trips overlap instead of each store waiting for its own.
  const int c = lane % CPR;
  int32_t tok[NI];
  u32x4 v[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = RPI * i + lane / CPR;
    const int pc = c ^ ((row / RP) % CPR);
    tok[i] = __shfl(qn, row);
    v[i] = *reinterpret_cast<const u32x4*>(stg + row * D + 8 * pc);
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = RPI * i + lane / CPR;
    if (RPI * i >= 16) v[i] = u32x4{v[i][2], v[i][3], v[i][0], v[i][1]};
    // Streaming store: the rows are not read again by this kernel.
    if (row < rows_valid)
      __builtin_nontemporal_store(v[i], reinterpret_cast<u32x4*>(out + size_t(tok[i]) * D + 8 * c));
  }
}

}  // namespace

// TEXT: the text queries of a joint block.  Query slot s is text row s; its
// keys are every image token and every text row; rows of q, out and lse are
// text rows.  With n_split > 1 a workgroup takes part p of the key list and
// writes a partial result: rows of out and lse for part p follow p * B*H
// heads of text rows (merged afterwards by their log-sum-exps).
//
// NWG: waves per workgroup with QB = 1.  8: 256 query slots, four-deep K and
// V rings (135 KB of LDS, one workgroup per CU).  4: 128 query slots,
// two-deep rings (69 KB, two workgroups per CU); each tile is then requested
// one iteration before its use and every request of an iteration has
// landed by its end.
template <int D, typename T, int QB, bool PAD, bool TEXT = false, int NWG = 8>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NWG / QB, 64 * NWG / QB),
                          amdgpu_waves_per_eu(QB == 1 ? 2 : 1, QB == 1 ? 2 : 1)))
void window_attn_fwd_kernel(Geom g, AttnArgs<T> a) {
  constexpr int NW = NWG / QB;     // waves per workgroup, QB query blocks each
  constexpr int NT = 64 * NW;      // threads
  constexpr int BQW = 32 * QB * NW;  // query slots per workgroup
  constexpr int KS = D / 16;       // 16-wide k steps of q.k
  constexpr int DB = D / 32;       // 32-row blocks of O^T, 32-element blocks of a tile row
  static_assert(NW == 8 || NW == 4, "eight or four waves per workgroup");
  static_assert(!TEXT || BQW == BQ, "text-query work is sized by the eight-wave tile");
  constexpr int NBUF = NW == 8 ? 4 : 2;  // LDS tiles per tensor
  constexpr int kAheadK = NBUF;          // K tile t+NBUF is requested in iteration t
  constexpr int kAheadV = NBUF - 1;      // V tile t+NBUF-1 is requested in iteration t
  // The last fragments of an iteration are requested from the next V tile
  // before the barrier (the tile has landed one iteration earlier); in the
  // four-wave form that tile is still arriving, so an iteration requests its
  // own first fragments after the barrier.
  constexpr bool kCarry = NW == 8;
  constexpr int RG = 8 / NW;       // 8-row groups of a tile staged per wave
  constexpr int XPG = D / 64;      // 1 KB transfers per row group (two d blocks each)
  constexpr int TPW = RG * XPG;    // 1 KB transfers per wave, tile and tensor
  static_assert(TPW * NW * 1024 == BK * D * 2, "tile transfers must cover the tile");
  constexpr bool kDma = std::is_same<T, __bf16>::value;  // float input is rounded on the way

  // One variable per ring buffer: LDS lowering gives each its own alias
  // scope, and with the buffer of every access known at compile time the
  // compiler sees that the loads in flight into other buffers need no wait
  // before a buffer is read (ordering is by the explicit vmcnt waits below).
  __shared__ __attribute__((aligned(1024))) uint16_t k_t0[BK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t k_t1[BK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t k_t2[NBUF > 2 ? BK * D : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t k_t3[NBUF > 2 ? BK * D : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t v_t0[BK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_t1[BK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_t2[NBUF > 2 ? BK * D : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t v_t3[NBUF > 2 ? BK * D : 8];
  auto k_tile = [&](auto s) -> uint16_t* {
    constexpr int S = decltype(s)::value % NBUF;
    if constexpr (S == 0) return k_t0;
    else if constexpr (S == 1) return k_t1;
    else if constexpr (S == 2) return k_t2;
    else return k_t3;
  };
  auto v_tile = [&](auto s) -> uint16_t* {
    constexpr int S = decltype(s)::value % NBUF;
    if constexpr (S == 0) return v_t0;
    else if constexpr (S == 1) return v_t1;
    else if constexpr (S == 2) return v_t2;
    else return v_t3;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  __shared__ __attribute__((aligned(16))) int32_t code[2][CE];
  __shared__ int32_t routes[kMaxTopk];
  __shared__ int32_t rstart[kMaxTopk + 1];  // routed segment offsets (short windows)
  __shared__ int32_t overflow;
  __shared__ int32_t routes_bad;  // a route id of this window is out of range

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;

  const int32_t blk = xcd_remap(blockIdx.x, a.n_blocks);
  const int32_t rest = int32_t(a.f_nqt.div(uint32_t(blk)));
  const int32_t qt = blk - rest * a.n_qt;
  const int32_t bh_i = int32_t(a.f_nw.div(uint32_t(rest)));
  const int32_t sub = rest - bh_i * (TEXT ? a.n_split : g.nW);
  // Text queries: part `part` of the key list starts at key `key0`.
  const int32_t part = TEXT ? sub : 0;
  const int32_t key0 = TEXT ? part * a.split_len : 0;
  const uint32_t win = TEXT ? uint32_t(key0) : uint32_t(sub);
  const size_t bh = size_t(bh_i);
  // Output rows of this pass: text parts follow part * B*H heads.
  const size_t bh_out = TEXT ? size_t(part) * g.BH + bh : bh;
  // Query rows per head: image tokens, or text rows (the global rows after
  // the pooled cells).
  const int32_t n_text = g.G - g.Gp;
  const int32_t rows_q = TEXT ? n_text : g.N;
  // Slots of this window (fewer than M in a short window); a query tile with
  // none has nothing to do.
  const int32_t Mw = TEXT ? n_text : (PAD ? window_tokens(g, win) : g.M);
  const WinBase wbase = TEXT ? WinBase{} : win_base<PAD>(g, win);
  if ((PAD || TEXT) && qt * BQW >= Mw) return;

  const T* qh = a.q + bh * size_t(rows_q) * D;
  const T* kh = a.k + bh * size_t(g.N) * D;
  const T* vh = a.v + bh * size_t(g.N) * D;
  const T* kph = a.kp ? a.kp + bh * size_t(g.G) * D : kh;
  const T* vph = a.vp ? a.vp + bh * size_t(g.G) * D : vh;

  // The routed window ids go out first (the row codes wait for them), then
  // this wave's queries (lane l32 of block b holds slot q0 + 32b + l32),
  // which are scaled (and waited for) only after the first K/V requests, so
  // the latencies overlap.  An id outside [0, nW) is never used as an
  // address (window 0 stands in for it) and makes the window's output rows
  // and lse NaN, so that a corrupt table shows in the result.
  int32_t route_v = 0;
  bool route_bad = false;
  if (!TEXT && tid < g.topk) {
    const int32_t r = a.route[(bh * g.nW + win) * g.topk + tid];
    route_bad = uint32_t(r) >= uint32_t(g.nW);
    route_v = route_bad ? 0 : r;
  }
  const float c_l2 = a.scale_log2;
  const int32_t q0 = qt * BQW + wave * 32 * QB;
  const bool wave_active = q0 < Mw;
  int32_t qn[QB];
  bool q_valid[QB];
  QRaw<T> q_raw[QB][KS];
  bf16x8 qf[QB][KS];
  // bf16 queries of the eight-wave form come in by direct loads into LDS:
  // whole 128-byte row spans per request, issued at a fraction of the cost of
  // the 32-byte pieces each lane would load for itself.  The wave's 32 rows
  // take half of ring buffer K2, K3, V2 or V3 (wave / 2), which the first
  // tiles leave free, in the K tile layout, and come back as B-operand
  // fragments through the K fragment reads.  Otherwise each lane loads its own
  // pieces.  Either way every load is unconditional: a slot past the window
  // reads row 0, and its output is never written.
  constexpr bool kQLds = kDma && NBUF == 4 && QB == 1;
  uint16_t* const q_stage = (wave >> 1) == 0 ? k_t2 : (wave >> 1) == 1 ? k_t3
                            : (wave >> 1) == 2 ? v_t2 : v_t3;
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const int32_t qs = q0 + 32 * b + l32;
    q_valid[b] = qs < Mw;
    qn[b] = !q_valid[b] ? 0 : TEXT ? qs : win_token(g, wbase, qs);
    if constexpr (!kQLds) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        q_raw[b][ks] = load_q_raw(qh + size_t(qn[b]) * D + 16 * ks + 8 * half);
    }
  }
  // Stored before the direct query loads go out: the wait for the route ids
  // would otherwise wait for those loads as well.
  if (!TEXT && tid < g.topk) routes[tid] = route_v;
  if constexpr (kQLds) {
    // Row group rg of the wave is row group 4 * (wave & 1) + rg of the
    // buffer; lane l fetches row 8 rg + (l & 31) / 4, chunk swizzled as in K.
    const int x = (lane & 31) >> 2;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int32_t qs = q0 + 8 * rg + x;
      const int32_t row = qs < Mw ? (TEXT ? qs : win_token(g, wbase, qs)) : 0;
      const int trow = 32 * (wave & 1) + 8 * rg + x;
      const int qc = (lane & 3) ^ ((trow >> 2) & 3);
      const T* const src = qh + size_t(row) * D + 8 * qc + 32 * (lane >> 5);
#pragma unroll
      for (int u = 0; u < D / 64; ++u)
        dma16(src + 64 * u, q_stage + (4 * (wave & 1) + rg) * (8 * D) + u * 512);
    }
  }

  // Barriers here order LDS only: a fenced barrier would wait for the query
  // loads as well.
  if (!TEXT && g.topk > 0 && wave == 0) {
    const bool any_bad = __any(route_bad);
    if (tid == 0) routes_bad = any_bad;
  }
  if (!TEXT && g.topk > 0) lds_barrier();
  // Key list length: routed windows may be short when windows can be.
  int32_t routed_len = TEXT ? 0 : g.topk * g.M;
  if (PAD && !TEXT && g.topk > 0) {
    if (tid == 0) {
      int32_t acc = 0;
      for (int r = 0; r < g.topk; ++r) {
        rstart[r] = acc;
        acc += window_tokens(g, uint32_t(routes[r]));
      }
      rstart[g.topk] = acc;
    }
    lds_barrier();
    routed_len = rstart[g.topk];
  }
  // Segments of this pass (all three in the joint pass).
  // Text parts: image keys, then text rows, of keys [key0, key0 + part length).
  const int32_t text_len = min(a.split_len, g.N + n_text - key0);
  const int32_t lenL = TEXT ? max(0, min(text_len, g.N - key0)) : (a.branches & 1) ? Mw : 0;
  const int32_t lenG = TEXT ? text_len - lenL : (a.branches & 2) ? g.G : 0;
  if (!(a.branches & 4)) routed_len = 0;
  const int32_t L = lenL + lenG + routed_len;
  const int32_t n_tiles = (L + BK - 1) / BK;
  auto fill_chunk = [&](int32_t c) {
    int32_t* dst = code[c & 1];
    for (int e = tid; e < CE; e += NT)
      dst[e] = key_code<PAD, TEXT>(g, win, wbase, lenL, lenG, L, routes, rstart, c * CE + e);
  };
  fill_chunk(0);
  if (CE < L) fill_chunk(1);
  lds_barrier();

  // ---- staging: tile t of K or V into its LDS tile ---------------------
  // K and V tiles share one d-blocked layout and the same rows per lane: a
  // 1 KB transfer fills two d blocks of one 8-row group.  K chunks are
  // swizzled inside each 64-byte row segment (slot q holds chunk
  // q ^ ((row >> 2) & 3)).
  auto put = [&](const T* src, uint16_t* dst_wave) {
    if constexpr (kDma) {
      dma16(src, dst_wave);
    } else {
      *reinterpret_cast<u32x4*>(dst_wave + 8 * lane) = load8_bf16<T>(src);
    }
  };
  // Wave w stages row groups w, w + NW, ...: in row group rg lane l takes
  // row 8 rg + (l & 31) / 4 and, in transfer u, 16 bytes of d block
  // 2u + l / 32.
  auto srow = [&](int r) { return 8 * (wave + NW * r) + ((lane & 31) >> 2); };
  // Row codes of this lane's rows of tile t.
  struct Codes { int32_t c[RG]; };
  auto tile_code = [&](int32_t t) {
    Codes cs;
#pragma unroll
    for (int r = 0; r < RG; ++r) cs.c[r] = code[(t / TPC) & 1][(t % TPC) * BK + srow(r)];
    return cs;
  };
  // This lane's 16-byte chunk of a row (slot q of its 64-byte segment,
  // swizzled in K; d block 2u + lane / 32) is folded into per-lane bases of
  // the token rows and the global rows of K and V, once.  The chunk does not
  // depend on the row group: a lane's rows differ by multiples of 8 NW, which
  // leave bits 2-3 of the row unchanged for NW = 4 and 8.  A request then
  // takes the row from the code's sign (token n >= 0, global row -1 - code)
  // and one base of the two.
  const int lane_k = 8 * ((lane & 3) ^ ((srow(0) >> 2) & 3)) + 32 * (lane >> 5);
  const int lane_v = 8 * (lane & 3) + 32 * (lane >> 5);
  const T* const kt_b = kh + lane_k;
  const T* const kp_b = kph + lane_k;
  const T* const vt_b = vh + lane_v;
  const T* const vp_b = vph + lane_v;
  auto stage = [&](const Codes& cs, uint16_t* tile, const T* tok_b, const T* glob_b) {
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int32_t m = cs.c[r] >> 31;            // -1 for a global row
      const uint32_t row = uint32_t(cs.c[r] ^ m);  // token, or global row
      const T* const src = (m ? glob_b : tok_b) + size_t(row) * D;
#pragma unroll
      for (int u = 0; u < XPG; ++u) put(src + 64 * u, tile + (wave + NW * r) * (8 * D) + u * 512);
    }
  };
  auto stage_k = [&](int32_t, const Codes& cs, uint16_t* tile) { stage(cs, tile, kt_b, kp_b); };
  auto stage_v = [&](int32_t, const Codes& cs, uint16_t* tile) { stage(cs, tile, vt_b, vp_b); };

  // Requests for the first tiles go out while the queries are in flight.
  // Eight waves: K tiles 0..3 and V tiles 0..2, of which K0, K1, V0 and V1
  // must have landed before iteration 0 (which prefetches from V1).  Four
  // waves: K0, K1 and V0, all needed.
  auto exists = [&](int32_t t) { return int(t < n_tiles); };
  // Row codes of the next K and V tiles to request (read one iteration
  // ahead, so that issuing a request never waits for an LDS read).
  Codes k_code_next{}, v_code_next{};
  // In two parts: the first tiles (into buffers 0 and 1), then the rest
  // (buffers 2 and 3 may still hold queries in between).
  auto prologue_first = [&]() {
    stage_k(0, tile_code(0), k_tile(I0{}));
    if (exists(1)) stage_k(1, tile_code(1), k_tile(I1{}));
    stage_v(0, tile_code(0), v_tile(I0{}));
    if constexpr (NBUF == 4) {
      if (exists(1)) stage_v(1, tile_code(1), v_tile(I1{}));
    }
  };
  auto prologue_rest = [&]() {
    if constexpr (NBUF == 4) {
      if (exists(2)) stage_k(2, tile_code(2), k_tile(I2{}));
      if (exists(3)) stage_k(3, tile_code(3), k_tile(I3{}));
      if (exists(2)) stage_v(2, tile_code(2), v_tile(I2{}));
    }
    if (exists(kAheadK)) k_code_next = tile_code(kAheadK);
    if (exists(kAheadV)) v_code_next = tile_code(kAheadV);
  };
  auto prologue_requests = [&]() {
    prologue_first();
    prologue_rest();
  };
  // Waits until the tiles iteration 0 reads have landed.
  auto prologue_wait = [&]() {
    if constexpr (NBUF == 4) wait_vmcnt_tiles<TPW>(exists(2) + exists(3) + exists(2));
    else wait_vmcnt<0>();
  };
  // ---- fragment offsets inside a tile (elements) ----------------------
  // Element e of d block db in row r sits at (r/8)*8D + db*256 + (r%8)*32 + e.
  // K: row 32*kb + l32, chunk 2*ks + half: d block ks/2, slot
  // (2*(ks & 1) + half) ^ ((l32 >> 2) & 3); one base per parity of ks.
  const int ksw = (l32 >> 2) & 3;
  const int k_row = (l32 >> 3) * (8 * D) + (l32 & 7) * 32;
  const int k_base0 = k_row + 8 * (half ^ ksw);
  const int k_base1 = k_row + 8 * ((2 + half) ^ ksw);
  // V: row 16*st + 4*half + (s16 >> 2) (+8), elements 16*(g16 & 1) + 4*(s16 & 3).
  const int g16 = lane >> 4, s16 = lane & 15;
  const int v_base = (4 * half + (s16 >> 2)) * 32 + 16 * (g16 & 1) + 4 * (s16 & 3);

  auto kfrag = [&](const uint16_t* kt, int kb, int ks) {
    const int off = (ks & 1 ? k_base1 : k_base0) + (ks >> 1) * 256 + kb * (32 * D);
    return *reinterpret_cast<const bf16x8*>(kt + off);
  };
  auto vfrag = [&](const uint16_t* vt, int st, int db) {
    const uint16_t* at = vt + v_base + db * 256 + st * (16 * D);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)at);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(at + 8 * D));
    return __builtin_bit_cast(
        bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                      __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
  };

  // Scale the queries: qf = c * q, rounded once to bf16.
  if constexpr (kQLds) {
    // This wave's query rows were requested before the first tiles.
    prologue_first();
    wait_vmcnt_tiles<TPW>(2 + 2 * exists(1));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[0][ks] = __builtin_bit_cast(
          bf16x8, scale_q<T>(__builtin_bit_cast(u32x4, kfrag(q_stage, wave & 1, ks)), c_l2));
    lds_barrier();  // every wave has its queries before buffers 2 and 3 are refilled
    prologue_rest();
  } else {
    prologue_requests();
#pragma unroll
    for (int b = 0; b < QB; ++b) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[b][ks] = __builtin_bit_cast(bf16x8, scale_q<T>(q_raw[b][ks], c_l2));
    }
  }

  f32x16 sc[QB];          // S' of the current key block
  f32x16 o[DB][QB];       // O^T accumulators
  f32x16 cneg[QB];        // -m splat: accumulator input of the q.k products
  uint32_t pw[QB][8];     // P of the previous key block, packed bf16
  float m_i[QB];          // shift of this pass (log2 units)
  float l_i[QB];          // this lane's partial row sums

  // S'^T of 32-key block kb of tile kt (prologue), accumulator input cin[b];
  // `slice(ks)` runs under MFMA group ks.
  auto qk = [&](const uint16_t* kt, int kb, const f32x16* cin, f32x16* s,
                auto slice) __attribute__((always_inline)) {
    bf16x8 ka = kfrag(kt, kb, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 kn = ka;
      if (ks + 1 < KS) kn = kfrag(kt, kb, ks + 1);
#pragma unroll
      for (int b = 0; b < QB; ++b)
        s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[b][ks], ks == 0 ? cin[b] : s[b], 0,
                                                       0, 0);
      slice(ks);
      ka = kn;
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Keys of block j past the end of the list get -inf.
  auto mask_block = [&](int32_t j) {
    if ((j + 1) * 32 > L) {
      const int32_t base = j * 32 + 4 * half;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (base + (i >> 2) * 8 + (i & 3) >= L) {
#pragma unroll
          for (int b = 0; b < QB; ++b) sc[b][i] = -INFINITY;
        }
      }
    }
  };

  // exp2 of S'_j, packing into the B-operand words pn of the next P.V product
  // and the row sums: pair u (u = 0 .. 8*QB-1) covers elements 2w, 2w+1 of
  // query block b = u % QB, w = u / QB.  The pairs are spread over both halves
  // of a step, so the vector work sits under the P.V and the q.k products.
  uint32_t pn[QB][8];
  auto exp_pair = [&](int u) {
    const int b = u % QB, w = u / QB;
    const float p0 = __builtin_amdgcn_exp2f(sc[b][2 * w]), p1 = __builtin_amdgcn_exp2f(sc[b][2 * w + 1]);
    pn[b][w] = pack_bf16(p0, p1);
    l_i[b] += p0 + p1;
    pin(pn[b][w]);
    pin(l_i[b]);
  };
  constexpr int NG = 2 * DB + KS;   // MFMA groups per step
  constexpr int NP = 8 * QB;        // exponential pairs per step
  auto exp_slice = [&](int grp) {   // pairs under MFMA group grp of a step
#pragma unroll
    for (int u = (grp * NP) / NG; u < ((grp + 1) * NP) / NG; ++u) exp_pair(u);
  };

  // Fragment queue.  A step reads NF operand fragments in a fixed order --
  // V fragments (k step jj, d block db) for its P.V products, then K
  // fragments (k step ks) for its q.k products -- and each is requested PD
  // fragments ahead of use, across the two halves of a step and into the
  // V fragments of the next step.
  constexpr int NF = 2 * DB + KS, PD = 4;
  static_assert(NF % PD == 0 && PD <= 2 * DB, "fragment queue");
  bf16x8 fq[PD];
  auto fetch = [&](int f, const uint16_t* vt, int vst0, const uint16_t* kt, int kbn) {
    if (f < 2 * DB) return vfrag(vt, vst0 + f / DB, f % DB);
    return kfrag(kt, kbn, f - 2 * DB);
  };

  // One 32-key block step j: P.V of block j-1 (V tile vt, sub-tiles vst0 and
  // vst0 + 1), then q.k of block j+1 (K tile kt, block kbn), with the
  // exponentials, packing and row sums of S'_j spread under both.  The next step reads V
  // tile nvt from sub-tile nvst0.
  // With carry false the step's last PD groups request nothing (the next
  // step's first fragments are requested by the next iteration itself).
  auto step = [&](auto masked, int32_t j, const uint16_t* vt, int vst0, const uint16_t* kt,
                  int kbn, const uint16_t* nvt, int nvst0, auto carry)
                  __attribute__((always_inline)) {
    if constexpr (decltype(masked)::value) mask_block(j);
    auto refill = [&](int f) {
      const int gf = f + PD;
      if (gf < NF)
        fq[f % PD] = fetch(gf, vt, vst0, kt, kbn);
      else if (decltype(carry)::value)
        fq[f % PD] = fetch(gf - NF, nvt, nvst0, kt, kbn);
    };
#pragma unroll
    for (int f = 0; f < 2 * DB; ++f) {
      const int jj = f / DB, db = f % DB;
      const bf16x8 va = fq[f % PD];
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const bf16x8 pb = __builtin_bit_cast(
            bf16x8, u32x4{pw[b][4 * jj], pw[b][4 * jj + 1], pw[b][4 * jj + 2], pw[b][4 * jj + 3]});
        o[db][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[db][b], 0, 0, 0);
      }
      exp_slice(f);
      refill(f);
      __builtin_amdgcn_sched_barrier(0);
    }
    f32x16 sn[QB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int f = 2 * DB + ks;
      const bf16x8 ka = fq[f % PD];
#pragma unroll
      for (int b = 0; b < QB; ++b)
        sn[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[b][ks], ks == 0 ? cneg[b] : sn[b],
                                                        0, 0, 0);
      exp_slice(f);
      refill(f);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      sc[b] = sn[b];
#pragma unroll
      for (int w = 0; w < 8; ++w) pw[b][w] = pn[b][w];
    }
  };

  // Iteration t (t % NBUF == S, a compile-time constant): P.V of tile t's
  // two key blocks (2t, 2t+1) and q.k of tile t+1's (2t+2, 2t+3).  Requested
  // meanwhile: K tile t+kAheadK and V tile t+kAheadV.  On the final tile the
  // q.k products still run (on a stale buffer, results masked and unused).
  // deep: every tile this iteration requests or waits for exists (t +
  // kAheadK + 1 < n_tiles), so the guards and the wait count are constants.
  auto iteration = [&](auto masked, auto slot, int32_t t, auto deep) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    constexpr bool kDeep = decltype(deep)::value;
    // Code chunk c + 2 reuses chunk c's table once chunk c's last rows (V of
    // its last tile) were requested, one iteration before this one.
    if ((t + kAheadV) % TPC == 0 && t + kAheadV >= TPC) {
      const int32_t c = (t + kAheadV) / TPC + 1;
      if (c * CE < L) fill_chunk(c);
    }
    if (kDeep || t + kAheadK < n_tiles)
      stage_k(t + kAheadK, k_code_next, k_tile(std::integral_constant<int, S + kAheadK>{}));
    if (kDeep || t + kAheadV < n_tiles)
      stage_v(t + kAheadV, v_code_next, v_tile(std::integral_constant<int, S + kAheadV>{}));
    if (kDeep || t + kAheadK + 1 < n_tiles) k_code_next = tile_code(t + kAheadK + 1);
    if (kDeep || t + kAheadV + 1 < n_tiles) v_code_next = tile_code(t + kAheadV + 1);
    if (wave_active) {
      const uint16_t* vt = v_tile(std::integral_constant<int, S>{});
      const uint16_t* kt = k_tile(std::integral_constant<int, S + 1>{});
      const uint16_t* vnext = v_tile(std::integral_constant<int, S + 1>{});
      if constexpr (!kCarry) {
#pragma unroll
        for (int f = 0; f < PD; ++f) fq[f] = fetch(f, vt, 0, kt, 0);
      }
      step(masked, 2 * t + 1, vt, 0, kt, 0, vt, 2, std::true_type{});
      step(masked, 2 * t + 2, vt, 2, kt, 1, vnext, 0, std::integral_constant<bool, kCarry>{});
    }
    if constexpr (kCarry) {
      // K tile t+2 and V tiles t+1 (read next iteration) and t+2 (its first
      // fragments are requested at the end of the next iteration) must have
      // landed; the requests issued after them (K t+4, V t+3 this
      // iteration) may stay in flight.
      if constexpr (kDeep) wait_vmcnt<2 * TPW>();
      else wait_vmcnt_tiles<TPW>(exists(t + 4) + exists(t + 3));
    } else {
      // K tile t+2 and V tile t+1, both requested in this iteration.
      wait_vmcnt<0>();
    }
    lds_barrier();
  };

  // Exact row maxima of the logits, for a workgroup whose row sums left the
  // safe range: the key list is walked once more, q.k products only, one K
  // tile at a time through ring buffer 0, and each row's shift moves by the
  // largest S' = S - m it meets.  The ring is idle (every request of the pass
  // has landed and every wave is past the vote's barrier).
  auto max_scan = [&]() {
    float mx[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) mx[b] = -INFINITY;
    fill_chunk(0);
    if (CE < L) fill_chunk(1);
    lds_barrier();
    for (int32_t t = 0; t < n_tiles; ++t) {
      // Chunk c replaces chunk c - 2, whose tiles are all behind.
      if (t % TPC == 0 && t >= 2 * TPC) {
        fill_chunk(t / TPC);
        lds_barrier();
      }
      stage_k(t, tile_code(t), k_tile(I0{}));
      wait_vmcnt<0>();
      lds_barrier();
      if (wave_active) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          qk(k_tile(I0{}), kb, cneg, sc, [](int) {});
          mask_block(2 * t + kb);
#pragma unroll
          for (int b = 0; b < QB; ++b) mx[b] = fmaxf(mx[b], pair_max(max16(sc[b])));
        }
      }
      lds_barrier();  // every wave has read the tile before the next one lands
    }
#pragma unroll
    for (int b = 0; b < QB; ++b) m_i[b] += mx[b];
  };

  // Pass 0 fixes the shift m at the exact max of key block 0 and lets P grow
  // above 1 where later keys score higher; every P is at most the row sum, so
  // a row sum below 2^64 bounds them all.  A workgroup with a larger (or
  // non-finite) row sum finds each row's exact maximum (max_scan) and runs
  // the list again with it as the shift: then every P is at most 1 (up to
  // rounding) and every row sum at most the list length.
#pragma unroll
  for (int b = 0; b < QB; ++b) m_i[b] = 0.f;
  for (int pass = 0; pass < kMaxPasses; ++pass) {
    if (pass > 0) {
      fill_chunk(0);
      if (CE < L) fill_chunk(1);
      __syncthreads();
      prologue_requests();
    }
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      l_i[b] = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        o[db][b] = f32x16{};
        asm volatile("" : "+v"(o[db][b]));
      }
    }
    prologue_wait();
    lds_barrier();
    if (wave_active) {
      if (pass == 0) {
        f32x16 zero[QB];
#pragma unroll
        for (int b = 0; b < QB; ++b) zero[b] = f32x16{};
        qk(k_tile(I0{}), 0, zero, sc, [](int) {});
        mask_block(0);
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          m_i[b] = pair_max(max16(sc[b]));
          cneg[b] = splat16(-m_i[b]);
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[b][i] -= m_i[b];
        }
      } else {
#pragma unroll
        for (int b = 0; b < QB; ++b) cneg[b] = splat16(-m_i[b]);
        qk(k_tile(I0{}), 0, cneg, sc, [](int) {});
        mask_block(0);
      }
      f32x16 sn[QB];
      qk(k_tile(I0{}), 1, cneg, sn, [&](int ks) {
#pragma unroll
        for (int u = (ks * NP) / KS; u < ((ks + 1) * NP) / KS; ++u) exp_pair(u);
      });
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        sc[b] = sn[b];
#pragma unroll
        for (int w = 0; w < 8; ++w) pw[b][w] = pn[b][w];
      }
      if constexpr (kCarry) {
#pragma unroll
        for (int f = 0; f < PD; ++f) fq[f] = fetch(f, v_tile(I0{}), 0, k_tile(I1{}), 0);
      }
    }
    lds_barrier();  // every wave has read K tile 0 before iteration 0 refills its buffer

    // Four iterations per trip, so that every buffer index is a constant.
    // Iteration t meets keys past the end of the list only if block 2t+2
    // does ((2t + 3) * 32 > L): full trips before that run unmasked.
    using NoMask = std::false_type;
    using Mask = std::true_type;
    using Deep = std::true_type;
    using Shallow = std::false_type;
    int32_t t = 0;
    for (; t + 3 + kAheadK + 1 < n_tiles && (2 * (t + 3) + 3) * 32 <= L; t += 4) {
      iteration(NoMask{}, I0{}, t, Deep{});
      iteration(NoMask{}, I1{}, t + 1, Deep{});
      iteration(NoMask{}, I2{}, t + 2, Deep{});
      iteration(NoMask{}, I3{}, t + 3, Deep{});
    }
    for (; t + 3 < n_tiles && (2 * (t + 3) + 3) * 32 <= L; t += 4) {
      iteration(NoMask{}, I0{}, t, Shallow{});
      iteration(NoMask{}, I1{}, t + 1, Shallow{});
      iteration(NoMask{}, I2{}, t + 2, Shallow{});
      iteration(NoMask{}, I3{}, t + 3, Shallow{});
    }
    for (; t < n_tiles; t += 4) {
      iteration(Mask{}, I0{}, t, Shallow{});
      if (t + 1 < n_tiles) iteration(Mask{}, I1{}, t + 1, Shallow{});
      if (t + 2 < n_tiles) iteration(Mask{}, I2{}, t + 2, Shallow{});
      if (t + 3 < n_tiles) iteration(Mask{}, I3{}, t + 3, Shallow{});
    }

    // Workgroup vote: did any row sum of this pass leave the safe range?
    float l_tot[QB];
    bool bad = false;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      l_tot[b] = pair_sum(l_i[b]);
      // Tested on the bits: this file is built without NaN semantics.  A NaN
      // sum (NaN input) is left as it is.
      const uint32_t bits = __float_as_uint(l_tot[b]) & 0x7fffffffu;
      bad |= bits > __float_as_uint(kSumLimit) && bits <= 0x7f800000u;
    }
    if (tid == 0) overflow = 0;
    __syncthreads();
    if (wave_active && __any(bad) && lane == 0) overflow = 1;
    __syncthreads();
    if (!overflow || pass + 1 == kMaxPasses) break;
    max_scan();
  }

  if (!wave_active) return;
  const bool poison = !TEXT && g.topk > 0 && routes_bad;
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const float l_tot = poison ? __uint_as_float(0x7fc00000u) : pair_sum(l_i[b]);
    const float inv = 1.0f / l_tot;
    if constexpr (std::is_same<T, __bf16>::value) {
      // bf16 rows leave through the idle K ring (every wave is past the
      // last iteration's barrier, no request is in flight): block b of this
      // wave takes half of ring buffer (wave*QB + b) / 2.
      const int region = wave * QB + b;
      static_assert(2 * NBUF >= NW * QB, "the K ring holds every block's rows");
      uint16_t* kb = (region >> 1) == 0 ? k_t0 : k_t1;
      if constexpr (NBUF > 2) kb = (region >> 1) == 2 ? k_t2 : (region >> 1) == 3 ? k_t3 : kb;
      store_rows_bf16<D, QB>(&o[0][0], b, inv, kb + (region & 1) * 32 * D,
                             a.out + bh_out * size_t(rows_q) * D, qn[b], Mw - (q0 + 32 * b), lane);
    } else {
      if (q_valid[b]) {
        T* orow = a.out + (bh_out * rows_q + qn[b]) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float v4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = o[db][b][4 * g4 + e] * inv;
            store_out4<T>(orow + 32 * db + 8 * g4 + 4 * half, v4);
          }
        }
      }
    }
    if (a.lse && half == 0 && q_valid[b])
      a.lse[bh_out * rows_q + qn[b]] = (m_i[b] + log2f(l_tot)) * 0.69314718055994531f;
  }
}

hipError_t launch_attn(const basa_plan_s& p, const void* q, const void* k, const void* v,
                       const void* kp, const void* vp, const int32_t* route, void* out,
                       float* lse, hipStream_t s, int branches) {
  const Geom& g = p.g;
  // Short key lists take the four-wave form: two workgroups share a CU.
  const bool half = (int64_t(g.L) + BK - 1) / BK <= kHalfFormMaxTiles;
  const int32_t bq = half ? BQ / 2 : BQ;
  const int32_t n_qt = (g.M + bq - 1) / bq;
  const int64_t n_items = int64_t(n_qt) * g.nW * g.BH;
  if (n_items > INT32_MAX) return hipErrorInvalidValue;
  const float sl2 = float(double(p.scale) * 1.4426950408889634);
  const uint32_t grid = uint32_t(n_items);
#define BASA_ATTN_NW(D_, T_, PAD_, NWG_)                                                          \
  hipLaunchKernelGGL((window_attn_fwd_kernel<D_, T_, kQB, PAD_, false, NWG_>), dim3(grid),        \
                     dim3(64 * NWG_ / kQB), 0, s, g, a)
#define BASA_ATTN(D_, T_)                                                                         \
  do {                                                                                            \
    AttnArgs<T_> a{static_cast<const T_*>(q), static_cast<const T_*>(k), static_cast<const T_*>(v), \
                   static_cast<const T_*>(kp), static_cast<const T_*>(vp), route,                 \
                   static_cast<T_*>(out), lse, sl2, n_qt, int32_t(n_items), branches};            \
    a.f_nqt = make_fastdiv(uint32_t(n_qt));                                                      \
    a.f_nw = make_fastdiv(uint32_t(g.nW));                                                       \
    if (g.padded) {                                                                               \
      if (half) BASA_ATTN_NW(D_, T_, true, 4); else BASA_ATTN_NW(D_, T_, true, 8);                \
    } else {                                                                                      \
      if (half) BASA_ATTN_NW(D_, T_, false, 4); else BASA_ATTN_NW(D_, T_, false, 8);              \
    }                                                                                             \
  } while (0)
  const bool f32 = p.params.dtype == BASA_F32;
  if (g.D == 128) {
    if (f32) BASA_ATTN(128, float); else BASA_ATTN(128, __bf16);
  } else {
    if (f32) BASA_ATTN(64, float); else BASA_ATTN(64, __bf16);
  }
#undef BASA_ATTN
#undef BASA_ATTN_NW
  return hipGetLastError();
}

hipError_t launch_attn_text(const basa_plan_s& p, const void* q_text, const void* k,
                            const void* v, const void* kg, const void* vg, void* out_text,
                            float* lse_text, void* ws, hipStream_t s) {
  const Geom& g = p.g;
  const int32_t n_text = g.G - g.Gp;
  const int32_t n_qt = (n_text + BQ - 1) / BQ;
  const int32_t parts = p.text_split;
  const int64_t n_items = int64_t(n_qt) * parts * g.BH;
  if (n_text <= 0 || parts < 1 || n_items > INT32_MAX) return hipErrorInvalidValue;
  if (parts > 1 && !ws) return hipErrorInvalidValue;
  const float sl2 = float(double(p.scale) * 1.4426950408889634);
  const uint32_t grid = uint32_t(n_items);
  // With several parts each writes a partial result into the workspace:
  // outputs [parts][B*H][X][d] (plan dtype), then lse [parts][B*H][X].
  const size_t elem = p.params.dtype == BASA_F32 ? 4 : 2;
  const size_t rows = size_t(g.BH) * n_text;
  char* const wsb = static_cast<char*>(ws);
  void* const o_dst = parts > 1 ? static_cast<void*>(wsb) : out_text;
  float* const l_dst =
      parts > 1 ? reinterpret_cast<float*>(wsb + (parts * rows * g.D * elem + 255) / 256 * 256)
                : lse_text;
#define BASA_TEXT(D_, T_)                                                                        \
  do {                                                                                           \
    AttnArgs<T_> a{static_cast<const T_*>(q_text), static_cast<const T_*>(k),                   \
                   static_cast<const T_*>(v), static_cast<const T_*>(kg),                       \
                   static_cast<const T_*>(vg), nullptr, static_cast<T_*>(o_dst), l_dst,         \
                   sl2, n_qt, int32_t(n_items), 3, parts, p.text_split_len};                     \
    a.f_nqt = make_fastdiv(uint32_t(n_qt));                                                      \
    a.f_nw = make_fastdiv(uint32_t(parts));                                                      \
    hipLaunchKernelGGL((window_attn_fwd_kernel<D_, T_, kQB, false, true>), dim3(grid),          \
                       dim3(512 / kQB), 0, s, g, a);                                             \
  } while (0)
  const bool f32 = p.params.dtype == BASA_F32;
  if (g.D == 128) {
    if (f32) BASA_TEXT(128, float); else BASA_TEXT(128, __bf16);
  } else {
    if (f32) BASA_TEXT(64, float); else BASA_TEXT(64, __bf16);
  }
#undef BASA_TEXT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || parts == 1) return e;
  return launch_merge_parts(p, o_dst, l_dst, parts, rows, out_text, lse_text, s);
}

}  // namespace basa
