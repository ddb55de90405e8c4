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
// Work decomposition.  One workgroup = NW waves (4 or 8) = 32*NW query slots
// of one (batch*head, window); wave w owns slots [32w, 32w+32).  The key
// list is streamed through LDS in tiles of 64 rows.  Row codes of the key
// list (token n >= 0, pooled cell -1 - c, or past-the-end) are computed once
// per workgroup into an LDS table of two 512-entry chunks, refilled as the
// walk advances, so staging a row costs one LDS read of its code.
//
// Per wave and tile (bf16 matrix cores, v_mfma_f32_32x32x16_bf16):
//   S^T[64 keys x 32 queries] = K_tile . Q^T     A = K rows (ds_read_b128),
//                                                B = Q held in registers
//   online softmax in base 2, per query column: every lane holds one query
//     and 16 of its keys per 32-key block, so the row max / sum need one
//     cross-half exchange (v_permlane32_swap) and nothing else;
//   O^T[d x 32 queries] += V^T_tile . P^T        A = V^T fragments read with
//                                                ds_read_b64_tr_b16 from V
//                                                rows, B = P straight from
//                                                the S^T accumulator.
// The transposing read hands each 16-lane group a 16 x 4 block turned on its
// side: source lane 4e + c reads 4 elements of key row e; lane i receives
// element i % 4 of source lanes 4e + i / 4, e = 0..3, i.e. four keys of one
// d column -- the A operand of the P.V product.
//
// Software pipeline.  K runs one tile ahead of V: while the vector units turn
// S^T of tile t into P, the matrix cores already compute S^T of tile t+1, one
// 16-wide k step at a time with a slice of the exponentials under each pair
// of MFMAs; then O^T += V_t^T P^T.  Tiles arrive by direct global -> LDS
// loads (global_load_lds_dwordx4, no staging registers) issued one tile ahead.
//
// LDS layouts (bf16, no padding).  A K tile is [64 key rows][d] with the
// 16-byte chunks of row r stored at chunk index c ^ f(r): f spreads the 16
// consecutive rows of a K fragment read over all banks.  A V tile is d-blocked,
// [d/32 blocks][64 key rows][32 elements]: the 4 rows x 64 bytes a
// transposing read touches are then 256 contiguous bytes (no conflict), and
// every V fragment address is one per-lane base plus an immediate.  Either
// way a DMA wave writes 1 KB contiguously and each lane fetches whatever
// chunk belongs in its slot.
//
// The running maximum is only raised when a tile's maximum exceeds it by
// more than 8 (log2 units), so exp2 arguments stay <= 8 and O is rescaled
// rarely; the final normalisation uses the same maximum, so the result is
// unchanged.
#include <type_traits>

#include "device_common.hpp"

namespace basa {

namespace {

constexpr int BK = 64;            // key rows per tile
constexpr int CE = 512;           // row codes per table chunk
constexpr int TPC = CE / BK;      // tiles per chunk
constexpr int kMaxTopk = 16;
constexpr int32_t kNoRow = INT32_MIN;
constexpr float kRescaleSlack = 8.0f;  // log2 units
// Tiles in flight ahead of use: K tile t+1+kAhead and V tile t+kAhead are
// requested while tile t is processed; each tensor cycles through
// kAhead + 1 LDS tiles.
#ifdef BASA_ATTN_AHEAD
constexpr int kAhead = BASA_ATTN_AHEAD;
#else
constexpr int kAhead = 3;
#endif
constexpr int NBUF = kAhead + 1;

// s_waitcnt vmcnt(n) with the other counters left open (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

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

// Chunk swizzle of key row r (see the layout note above).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

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

template <int D, typename T, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2, 2)))
void window_attn_fwd_kernel(Geom g, AttnArgs<T> a) {
  constexpr int NT = 64 * NW;      // threads
  constexpr int BQ = 32 * NW;      // query slots per workgroup
  constexpr int KS = D / 16;       // 16-wide k steps of q.k
  constexpr int DB = D / 32;       // 32-row blocks of O^T
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;    // rows covered by one wave-wide 1 KB transfer
  constexpr int IPW = BK / RPI / NW;  // transfers per wave per tile and tensor
  static_assert(IPW >= 1 && IPW * RPI * NW == BK, "tile transfers must cover the tile");
  constexpr bool kDma = std::is_same<T, __bf16>::value;  // float input is rounded on the way

  __shared__ __attribute__((aligned(1024))) uint16_t k_tile[NBUF][BK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_tile[NBUF][BK * D];
  __shared__ int32_t code[2][CE];
  __shared__ int32_t routes[kMaxTopk];

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
  const T* kph = a.kp ? a.kp + bh * size_t(g.G) * D : kh;
  const T* vph = a.vp ? a.vp + bh * size_t(g.G) * D : vh;

  // Routed window ids are clamped into [0, nW) so that a corrupt table can
  // only give wrong keys, never an out-of-bounds read.
  if (tid < g.topk)
    routes[tid] = int32_t(min(uint32_t(a.route[(bh * g.nW + win) * g.topk + tid]),
                              uint32_t(g.nW - 1)));
  __syncthreads();
  const int32_t L = g.L;
  const int32_t n_tiles = (L + BK - 1) / BK;
  auto fill_chunk = [&](int32_t c) {
    int32_t* dst = code[c & 1];
    for (int e = tid; e < CE; e += NT) dst[e] = key_code(g, win, routes, c * CE + e);
  };
  fill_chunk(0);
  if (CE < L) fill_chunk(1);

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

  // ---- staging: tile t of K or V into its LDS tile ---------------------
  // A wave-wide transfer fills 1 KB: for K, RPI rows of d; for V, 16 rows of
  // one 32-wide d block.  Lane l fills the 16-byte slot l.
  const int32_t pool_lo = g.M, pool_hi = g.M + g.G;
  auto row_src = [&](const int32_t* cd, int r, int c, bool plain, const T* tokb,
                     const T* poolb) -> const T* {
    const int32_t cr = cd[r];
    if (plain) return tokb + size_t(cr) * D + 8 * c;
    const bool valid = cr != kNoRow;  // past the end: any finite row (masked later)
    const bool pooled = valid && cr < 0;
    const int32_t row = !valid ? 0 : (pooled ? -1 - cr : cr);
    return (pooled ? poolb : tokb) + size_t(row) * D + 8 * c;
  };
  auto put = [&](const T* src, uint16_t* dst_wave) {
    if constexpr (kDma) {
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)dst_wave, 16, 0, 0);
    } else {
      *reinterpret_cast<u32x4*>(dst_wave + 8 * lane) = load8_bf16<T>(src);
    }
  };
  auto stage_k = [&](int32_t t, uint16_t* tile) {
    const int32_t* cd = code[(t / TPC) & 1] + (t % TPC) * BK;
    const int32_t lo = t * BK, hi = lo + BK;
    const bool plain = hi <= L && (hi <= pool_lo || lo >= pool_hi);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int r0 = (wave * IPW + i) * RPI;
      const int r = r0 + lane / CPR;
      put(row_src(cd, r, (lane % CPR) ^ swz<D>(r), plain, kh, kph), tile + r0 * D);
    }
  };
  auto stage_v = [&](int32_t t, uint16_t* tile) {
    const int32_t* cd = code[(t / TPC) & 1] + (t % TPC) * BK;
    const int32_t lo = t * BK, hi = lo + BK;
    const bool plain = hi <= L && (hi <= pool_lo || lo >= pool_hi);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int ii = wave * IPW + i;           // 16 rows of d block ii / 4
      const int db = ii >> 2, r0 = 16 * (ii & 3);
      const int r = r0 + (lane >> 2);
      put(row_src(cd, r, 4 * db + (lane & 3), plain, vh, vph), tile + db * (BK * 32) + r0 * 32);
    }
  };

  // ---- fragment offsets inside a tile (elements) ----------------------
  // K: row l32 (+32 for the second block), logical chunk 2*kk + half.
  const int k_base = (l32 * D + 8 * swz<D>(l32)) ^ (8 * half);
  // V: row 16*st + 4*half + (s16 >> 2) (+8), elements 16*(g16 & 1) + 4*(s16 & 3).
  const int g16 = lane >> 4, s16 = lane & 15;
  const int v_base = (4 * half + (s16 >> 2)) * 32 + 16 * (g16 & 1) + 4 * (s16 & 3);

  // S^T of one tile: 64 keys (two 32-row blocks) x this wave's 32 queries,
  // one k step at a time; `slice(kk)` is issued under each pair of MFMAs.
  auto qk = [&](const uint16_t* kt, f32x16& s0, f32x16& s1, auto slice) {
    auto frag = [&](int rb, int kk) {
      return *reinterpret_cast<const bf16x8*>(kt + 32 * rb * D + (k_base ^ (16 * kk)));
    };
    bf16x8 a0 = frag(0, 0), a1 = frag(1, 0);
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      bf16x8 b0 = a0, b1 = a1;
      if (kk + 1 < KS) {
        b0 = frag(0, kk + 1);
        b1 = frag(1, kk + 1);
      }
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[kk], s1, 0, 0, 0);
      slice(kk);
      a0 = b0;
      a1 = b1;
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Prologue: K tiles 0 .. kAhead and V tiles 0 .. kAhead-1, and S^T of tile 0.
  for (int32_t j = 0; j <= kAhead && j < n_tiles; ++j) {
    stage_k(j, k_tile[j % NBUF]);
    if (j < kAhead) stage_v(j, v_tile[j % NBUF]);
  }
  wait_vmcnt<0>();
  __syncthreads();
  f32x16 s0, s1;
  if (wave_active) qk(k_tile[0], s0, s1, [](int) {});
  __syncthreads();  // every wave has read K tile 0 before it is overwritten

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_i = -INFINITY;  // running max of scaled logits (log2 units)
  float l_i = 0.f;        // this lane's partial sum of exp2 terms
  const float sl2 = a.scale_log2;

  // Iteration t: S^T of tile t+1 on the matrix cores while the vector units
  // turn S^T of tile t (s0, s1) into P; then O^T += V_t^T P^T.  Staged
  // meanwhile: K tile t+1+kAhead and V tile t+kAhead.  On the final
  // tile the q.k products still run (on a stale buffer, results unused) so
  // that every iteration is the same single basic block.
  for (int32_t t = 0; t < n_tiles; ++t) {
    const uint16_t* k_next_tile = k_tile[(t + 1) % NBUF];
    const uint16_t* v_cur = v_tile[t % NBUF];
    // Code chunk c + 2 reuses chunk c's table once chunk c's last rows (V of
    // its last tile) have been requested, one iteration before this one.
    if ((t + kAhead) % TPC == 0 && t + kAhead >= TPC) {
      const int32_t c = (t + kAhead) / TPC + 1;
      if (c * CE < L) fill_chunk(c);
    }
    const bool k_req = t + 1 + kAhead < n_tiles, v_req = t + kAhead < n_tiles;
    if (k_req) stage_k(t + 1 + kAhead, k_tile[t % NBUF]);              // held K tile t
    if (v_req) stage_v(t + kAhead, v_tile[(t + kAhead) % NBUF]);      // held V tile t-1
    if (wave_active) {
      if ((t + 1) * BK > L) {  // keys past the end of the list get -inf
        const int32_t base = t * BK + 4 * half;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int32_t kj = base + (i >> 2) * 8 + (i & 3);
          if (kj >= L) s0[i] = -INFINITY;
          if (kj + 32 >= L) s1[i] = -INFINITY;
        }
      }
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(fmaxf(mx, s0[i]), s1[i]);
      mx = pair_max(mx) * sl2;
      const float m_new = fmaxf(m_i, mx);
      if (__any(m_new > m_i + kRescaleSlack)) {
        const float alpha = m_i == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_i - m_new);
        l_i *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
        m_i = m_new;
      }
      // P = exp2(s * scale log2e - m) in slices of VPS values, packed two by
      // two into the B operand words of the P.V product; row sums in l_i.
      constexpr int VPS = 32 / KS;
      uint32_t pw[16];
      auto exp_slice = [&](int kk) {
        const int st = (kk * VPS) / 8;
        const f32x16& sv = st < 2 ? s0 : s1;
        const int i0 = 8 * (st & 1) + (kk * VPS) % 8;
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < VPS; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[i0 + e], sl2, -m_i));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[i0 + e + 1], sl2, -m_i));
          ps += p0 + p1;
          pw[(kk * VPS + e) / 2] = pack_bf16(p0, p1);
        }
        l_i += ps;
      };
      f32x16 n0, n1;
      qk(k_next_tile, n0, n1, exp_slice);
      // O^T += V_t^T P^T; the transposing V reads run one product ahead.
      auto read_va = [&](int st, int db) {
        const uint16_t* at = v_cur + v_base + db * (BK * 32) + st * 16 * 32;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)at);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(at + 8 * 32));
        return __builtin_bit_cast(
            bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                          __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
      };
      bf16x8 va = read_va(0, 0);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8 pb = __builtin_bit_cast(
            bf16x8, u32x4{pw[4 * st], pw[4 * st + 1], pw[4 * st + 2], pw[4 * st + 3]});
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int nst = db + 1 < DB ? st : st + 1, ndb = db + 1 < DB ? db + 1 : 0;
          bf16x8 vn = va;
          if (nst < 4) vn = read_va(nst, ndb);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[db], 0, 0, 0);
          va = vn;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      s0 = n0;
      s1 = n1;
    }
    // K tile t+2 and V tile t+1 (requested last iteration) must have landed;
    // this iteration's requests may stay in flight.
    if (k_req) wait_vmcnt<2 * IPW>();
    else if (v_req) wait_vmcnt<IPW>();
    else wait_vmcnt<0>();
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

template <int D, typename T, int NW>
static void launch_one(const Geom& g, const AttnArgs<T>& a, hipStream_t s) {
  hipLaunchKernelGGL((window_attn_fwd_kernel<D, T, NW>), dim3(uint32_t(a.n_blocks)),
                     dim3(64 * NW), 0, s, g, a);
}

hipError_t launch_attn(const basa_plan_s& p, const void* q, const void* k, const void* v,
                       const void* kp, const void* vp, const int32_t* route, void* out,
                       float* lse, hipStream_t s) {
  const Geom& g = p.g;
  // Eight waves (256 query slots) per workgroup once a window has that many
  // queries: the K/V list is staged once for twice the queries.
#ifdef BASA_ATTN_WAVES
  const int nw = BASA_ATTN_WAVES;
#else
  const int nw = g.M >= 256 ? 8 : 4;
#endif
  const int32_t bq = 32 * nw;
  const int32_t n_qt = (g.M + bq - 1) / bq;
  const int64_t n_blocks = int64_t(n_qt) * g.nW * g.BH;
  if (n_blocks > INT32_MAX) return hipErrorInvalidValue;
  const float sl2 = float(double(p.scale) * 1.4426950408889634);
#define BASA_ATTN(D_, T_)                                                                         \
  do {                                                                                            \
    AttnArgs<T_> a{static_cast<const T_*>(q), static_cast<const T_*>(k), static_cast<const T_*>(v), \
                   static_cast<const T_*>(kp), static_cast<const T_*>(vp), route,                 \
                   static_cast<T_*>(out), lse, sl2, n_qt, int32_t(n_blocks)};                     \
    if (nw == 8) launch_one<D_, T_, 8>(g, a, s); else launch_one<D_, T_, 4>(g, a, s);             \
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
