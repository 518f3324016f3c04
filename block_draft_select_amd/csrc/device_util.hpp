// Device helpers shared by the gfx950 kernels: wave-64 reductions, ordered
// integer keys for floating-point values, packed 16-bit key arithmetic and
// the Philox4x32-10 counter-based generator.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfk {

constexpr int kWave = 64;

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- wave ops

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t w = __shfl_xor(v, o);
    v = w > v ? w : v;
  }
  return v;
}

__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ------------------------------------------------------- ordered keys
// An order-preserving map from IEEE bit patterns to unsigned integers:
// non-negative values get the sign bit set, negative values are inverted.
// Larger key <=> larger value.  -0.0 maps just below +0.0 unless
// canonicalised.  The all-ones NaN pattern maps to key 0, which the kernels
// use as "no element".

__device__ __forceinline__ uint32_t ord32(uint32_t bits) {
  return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

// ordered key with -0.0 folded onto +0.0
__device__ __forceinline__ uint32_t ord32_canon(uint32_t bits) {
  return ord32(bits == 0x80000000u ? 0u : bits);
}

__device__ __forceinline__ uint32_t unord32(uint32_t key) {
  return (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
}

// two bf16 patterns -> two 16-bit ordered keys (same lanes)
__device__ __forceinline__ uint32_t ord16x2(uint32_t x) {
  const s16x2 s = __builtin_bit_cast(s16x2, x) >> (s16x2)(15);
  return x ^ (__builtin_bit_cast(uint32_t, s) | 0x80008000u);
}

__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// per-lane saturating a - b on two 16-bit lanes
__device__ __forceinline__ uint32_t subsat_u16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, a),
                                                                    __builtin_bit_cast(u16x2, b)));
}

// ordered 32-bit key (canonical) of the fp32 widening of a bf16 whose
// 16-bit ordered key is k16
__device__ __forceinline__ uint32_t ord32_of_k16(uint32_t k16) {
  if (k16 == 0x7FFFu) return 0x80000000u;  // -0.0 -> +0.0
  return (k16 & 0x8000u) ? (k16 << 16) : ((k16 << 16) | 0xFFFFu);
}

// bf16 pattern of a 16-bit ordered key
__device__ __forceinline__ uint32_t bf16_of_k16(uint32_t k16) {
  return (k16 & 0x8000u) ? (k16 & 0x7FFFu) : (~k16 & 0xFFFFu);
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// ---------------------------------------------------------------- Philox
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): per round the 64-bit products of counter words
// 0 and 2 with the two multipliers are mixed into a permuted counter with
// the key; the key advances by the two Weyl constants between rounds.

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// the block of stream `seed` for (cycle, position, slot)
__device__ __forceinline__ uint4 stream_block(uint64_t seed, uint64_t cycle, uint32_t position,
                                              uint32_t slot) {
  return philox4x32_10(make_uint4((uint32_t)cycle, (uint32_t)(cycle >> 32), position, slot),
                       (uint32_t)seed, (uint32_t)(seed >> 32));
}

// (2k + 1) * 2^-24 with k the top 23 bits: exact in fp32, inside (0, 1)
__device__ __forceinline__ float u01_f32(uint32_t w) {
  return (float)((w >> 9) * 2u + 1u) * 0x1p-24f;
}

// (2k + 1) * 2^-53 with k the top 52 bits of hi:lo: exact in fp64
__device__ __forceinline__ double u01_f64(uint32_t hi, uint32_t lo) {
  const uint64_t v = ((uint64_t)hi << 32) | lo;
  return (double)((v >> 12) * 2ull + 1ull) * 0x1p-53;
}

__device__ __forceinline__ int clamp_idx(int v, int n) { return v < 0 ? 0 : (v >= n ? n - 1 : v); }

}  // namespace dfk
