// k_probe.hip -- measurement hook: the bf16 matrix-core rate the chip
// sustains, and its clock under that load.
//
// The pages rate their kernels against the accelerator's nominal peak
// (thelatestinai.com card, Table 3, MFU column).  MI355X's nominal 2.5 PFLOP/s
// of dense bf16 assumes a 2.4 GHz clock; under sustained matrix-core load the
// clock sits lower.  This kernel measures what back-to-back
// v_mfma_f32_32x32x16_bf16 products reach: every wave runs four independent
// accumulator chains for a fixed number of steps (two waves per SIMD keep
// the matrix unit fed), on constant operands or on operands whose bits
// change from one product to the next (the chip's power, and so its clock
// under load, depends on how many operand bits switch), and wave 0 of every
// workgroup records the shader
// clock (s_memtime) and the 100 MHz constant clock (s_memrealtime) before
// and after, from which the host derives the clock under load.
#include "device_common.hpp"

namespace basa {

namespace {

constexpr int kProbeWaves = 4;  // waves per workgroup
constexpr int kProbeChains = 4; // independent accumulators per wave

typedef short s16x8 __attribute__((ext_vector_type(8)));

// Scrambles a 32-bit value (an integer hash: xor-shift and odd-multiply
// rounds), for operand bits that differ from lane to lane.
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Reverses the eight elements of a lane's fragment.
__device__ __forceinline__ s16x8 reversed(const s16x8& v) {
  return s16x8{v[7], v[6], v[5], v[4], v[3], v[2], v[1], v[0]};
}

// mode 0: every operand element is the bf16 value with bits `operand_bits`
// (the host passes 2^-6), so each product step adds 16 * 2^-12 = 2^-8 to
// every accumulator element, exactly in float32 while iters < 2^24.
// mode 1: operands whose bits change from one product to the next, as real
// data's do: step 2i multiplies A0 by B0 and step 2i + 1 multiplies A1 by B1,
// where A0, B0 hold per-lane pseudo-random bf16 values (random sign, 7
// mantissa bits, magnitude in [2^-6, 2^-4)) and A1, B1 are the same values
// with each lane's eight k elements in reverse order and A1 negated -- the
// same products in another order, negated.  Every product and every sum is
// exact in float32 (22 significant bits at most), so each pair of steps
// returns the accumulators to zero exactly: the sink reads 0 for even iters.
// sink[thread] receives the sum of element 0 of the four accumulators;
// clocks[4 * wg ..] the start and end readings of both clocks.
__global__ __launch_bounds__(64 * kProbeWaves) void mfma_probe_kernel(int32_t iters, int32_t mode,
                                                                      uint32_t operand_bits,
                                                                      float* sink,
                                                                      uint64_t* clocks) {
  s16x8 a0, b0;
  if (mode == 0) {
    const short e = short(operand_bits & 0xffffu);
    a0 = s16x8{e, e, e, e, e, e, e, e};
    b0 = a0;
  } else {
    const uint32_t seed = (blockIdx.x * blockDim.x + threadIdx.x) * 16u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t ha = probe_hash(seed + i), hb = probe_hash(seed + 8 + i);
      // sign | exponent 121 or 122 (2^-6 or 2^-5) | 7 mantissa bits
      a0[i] = short(((ha >> 31) << 15) | ((121u + ((ha >> 7) & 1u)) << 7) | (ha & 0x7fu));
      b0[i] = short(((hb >> 31) << 15) | ((121u + ((hb >> 7) & 1u)) << 7) | (hb & 0x7fu));
    }
  }
  const s16x8 a1 = reversed(a0) ^ s16x8{short(0x8000), short(0x8000), short(0x8000),
                                        short(0x8000), short(0x8000), short(0x8000),
                                        short(0x8000), short(0x8000)};
  const s16x8 b1 = reversed(b0);
  const bf16x8 fa0 = __builtin_bit_cast(bf16x8, a0), fb0 = __builtin_bit_cast(bf16x8, b0);
  const bf16x8 fa1 = __builtin_bit_cast(bf16x8, mode == 0 ? a0 : a1);
  const bf16x8 fb1 = __builtin_bit_cast(bf16x8, mode == 0 ? b0 : b1);
  f32x16 c[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) c[j] = f32x16{};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  // Two product steps per trip (iters is even in mode 1; an odd iters in
  // mode 0 takes one more step after the loop).
  for (int32_t i = 0; i + 1 < iters; i += 2) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j)
      c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0, fb0, c[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j)
      c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1, fb1, c[j], 0, 0, 0);
  }
  if (iters & 1) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j)
      c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0, fb0, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) s += c[j][0];
  // The end readings wait for the last products: the empty asm consumes s.
  asm volatile("" ::"v"(s));
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  sink[size_t(blockIdx.x) * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    uint64_t* out = clocks + 4 * size_t(blockIdx.x);
    out[0] = t0;
    out[1] = t1;
    out[2] = r0;
    out[3] = r1;
  }
}

}  // namespace

int probe_threads_per_workgroup() { return 64 * kProbeWaves; }

double probe_flops(int32_t iters, int32_t n_workgroups) {
  // 32 x 32 x 16 multiply-adds per product, two flops each.
  return 2.0 * 32 * 32 * 16 * double(kProbeChains) * kProbeWaves * double(iters) *
         double(n_workgroups);
}

hipError_t launch_probe_mfma(int32_t iters, int32_t mode, int32_t n_workgroups, float* sink,
                             uint64_t* clocks, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(uint32_t(n_workgroups)), dim3(64 * kProbeWaves), 0,
                     s, iters, mode, 0x3c80u, sink, clocks);
  return hipGetLastError();
}

}  // namespace basa
