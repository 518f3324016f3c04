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

// ---------------------------------------------------------------- DPP scans
// Cross-lane steps through the data-parallel-primitive (DPP) modifiers of
// GFX9: a lane reads another lane's register in the same instruction, with
// no LDS round trip.  Lanes whose source is outside their row, or whose row
// is masked off, receive `id` (the identity of the operation).

constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t id) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROW_MASK, 0xF, false);
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v, float id) {
  return __uint_as_float(dpp_u32<CTRL, ROW_MASK>(__float_as_uint(v), __float_as_uint(id)));
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double v, double id) {
  const uint64_t b = __double_as_longlong(v), i = __double_as_longlong(id);
  const uint32_t lo = dpp_u32<CTRL, ROW_MASK>((uint32_t)b, (uint32_t)i);
  const uint32_t hi = dpp_u32<CTRL, ROW_MASK>((uint32_t)(b >> 32), (uint32_t)(i >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// inclusive prefix sum over lanes 0..15 of each row (fp64)
__device__ __forceinline__ double row16_scan_f64(double v) {
  v += dpp_f64<kDppRowShr1>(v, 0.0);
  v += dpp_f64<kDppRowShr2>(v, 0.0);
  v += dpp_f64<kDppRowShr4>(v, 0.0);
  v += dpp_f64<kDppRowShr8>(v, 0.0);
  return v;
}

// inclusive prefix sum over the 64 lanes (fp64)
__device__ __forceinline__ double wave_scan_f64(double v) {
  v = row16_scan_f64(v);
  v += dpp_f64<kDppRowBcast15, 0xA>(v, 0.0);
  v += dpp_f64<kDppRowBcast31, 0xC>(v, 0.0);
  return v;
}

// running maximum over lanes 0..15 of each row (fp32); lane 15 holds the row max
__device__ __forceinline__ float row16_scan_max_f32(float v) {
  v = fmaxf(v, dpp_f32<kDppRowShr1>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<kDppRowShr2>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<kDppRowShr4>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<kDppRowShr8>(v, -INFINITY));
  return v;
}

// maximum over the 64 lanes (fp32), the same value in every lane
__device__ __forceinline__ float wave_max_dpp_f32(float v) {
  v = row16_scan_max_f32(v);
  v = fmaxf(v, dpp_f32<kDppRowBcast15, 0xA>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<kDppRowBcast31, 0xC>(v, -INFINITY));
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

// sum over the 64 lanes (fp64), the same value in every lane
__device__ __forceinline__ double wave_sum_dpp_f64(double v) {
  v = wave_scan_f64(v);
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)b, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(b >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)b, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(b >> 32), lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// lowest lane whose predicate holds (64 if none)
__device__ __forceinline__ int first_lane(bool pred) {
  const uint64_t m = __ballot(pred);
  return m ? __builtin_ctzll(m) : 64;
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

// ---------------------------------------------------------------- exp, x <= 0
// e^x for x <= 0 in fp64 (every exponent this library takes is a logit or
// score minus a maximum, so never positive).  Cody & Waite reduction:
// x = n ln2 + r with n = rint(x log2 e), |r| <= ln2 / 2, ln2 split into a
// head with 15 significant bits (22713 / 32768, so n * head is exact for
// every |n| < 2^38; here |n| <= 1443) and a tail; e^r from its Taylor series
// to degree 11 (truncation error below 1e-14 relative); scaled by 2^n.  The
// argument is clamped at -1000, where e^x is 0 in fp64.  Relative error
// below 1e-14 over [-708, 0]; a CPU test runs this same code on the host
// against the C library's exp.
__host__ __device__ inline double exp_nonpos(double x) {
  constexpr double kLog2E = 1.4426950408889634;
  constexpr double kLn2Head = 0.693145751953125;        // 22713 / 32768
  constexpr double kLn2Tail = 1.4286068203094173e-06;   // ln 2 - head
  x = fmax(x, -1000.0);
  const double n = __builtin_rint(x * kLog2E);
  double r = fma(-n, kLn2Head, x);
  r = fma(-n, kLn2Tail, r);
  double p = 2.505210838544172e-08;              // 1 / 11!
  p = fma(p, r, 2.755731922398589e-07);          // 1 / 10!
  p = fma(p, r, 2.7557319223985893e-06);         // 1 / 9!
  p = fma(p, r, 2.48015873015873e-05);           // 1 / 8!
  p = fma(p, r, 1.984126984126984e-04);          // 1 / 7!
  p = fma(p, r, 1.388888888888889e-03);          // 1 / 6!
  p = fma(p, r, 8.333333333333333e-03);          // 1 / 5!
  p = fma(p, r, 4.1666666666666664e-02);         // 1 / 4!
  p = fma(p, r, 1.6666666666666666e-01);         // 1 / 3!
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(p, (int)n);
}

// ---------------------------------------------------------------- hand-off inside a launch
// Values passed between blocks of one launch, which may run on different
// XCDs (each with its own L2), travel as device-scope atomic stores and
// loads: coherent across the XCDs without a release fence (which would
// write back a whole L2).  Nothing orders two such stores, so every entry
// validates itself against the launch's tag: a mix of the cycle epoch,
// which every cycle advances (so entries of earlier cycles do not match),
// forced odd (so a zero-filled buffer never matches).  A 64-bit value split
// over two words also carries a check word mixing value and tag (a reader
// that sees one word new and the other old finds a mismatch and reads
// again); a float travels in one word whose high half is the tag xor a mix
// of the value.  Memory holding anything else passes a check by chance only
// (about 2^-32 per entry).
__device__ __forceinline__ uint32_t handoff_tag(uint32_t epoch) { return (epoch * 0x9E3779B1u + 0x7F4A7C15u) | 1u; }
__device__ __forceinline__ uint32_t handoff_fmix(uint32_t bits) { return bits * 0x85EBCA77u; }
__device__ __forceinline__ uint32_t handoff_check(uint64_t v, uint32_t tag) {
  return ((uint32_t)v * 0x9E3779B1u) ^ ((uint32_t)(v >> 32) * 0x85EBCA77u) ^ tag;
}
__device__ __forceinline__ void handoff_store(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t handoff_load(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// a 64-bit value with its tag and check word: words p[0], p[1]
__device__ __forceinline__ void handoff_store_pair(uint64_t* p, uint64_t v, uint32_t tag) {
  handoff_store(p, v);
  handoff_store(p + 1, ((uint64_t)handoff_check(v, tag) << 32) | tag);
}
// a float with its tag in one word: (tag ^ fmix(value)) << 32 | value
__device__ __forceinline__ void handoff_store_f32(uint64_t* p, float v, uint32_t tag) {
  const uint32_t bits = __float_as_uint(v);
  handoff_store(p, ((uint64_t)(tag ^ handoff_fmix(bits)) << 32) | bits);
}

// ---------------------------------------------------------------- streaming loads
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load of data read once: the nontemporal hint keeps the stream
// from displacing reusable lines (measured ~10% faster than a plain load
// for one pass over a few hundred MB)
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// One step of the max-sum dynamic programme on a whole wave: lane
// g * 16 + j (g = 0..3) takes predecessors i = 4g .. 4g + 3 of successor j,
// so every lane must hold best(j) of its column j = lane % 16 on entry (the
// four groups are replicas).  On exit every lane holds, for its column, the
// maximum over i < K of best(i) + St[i * K + j] and the first i attaining
// it.  St is the step's K x K score block; rows and columns past K are read
// clamped and ignored.  The local pairs and the two cross-group rounds keep
// the lower index on ties, so the result equals a left-to-right scan with a
// strict compare.
__device__ __forceinline__ void maxplus_step(double best, const float* St, int K, int lane, double& m_out,
                                             int& arg_out) {
  const int j = min(lane & 15, K - 1), g = lane >> 4;
  double v[4];
  int a[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = 4 * g + u;
    const double pv = __shfl(best, (lane & 48) | i);  // best(i), from lane i of this group
    const float ev = St[min(i, K - 1) * K + j];
    v[u] = i < K ? pv + (double)ev : -INFINITY;
    a[u] = i;
  }
#pragma unroll
  for (int w = 1; w < 4; w *= 2)
#pragma unroll
    for (int u = 0; u < 4; u += 2 * w) {
      const bool right = v[u + w] > v[u];  // ties keep the lower index
      v[u] = right ? v[u + w] : v[u];
      a[u] = right ? a[u + w] : a[u];
    }
  double m = v[0];
  int arg = a[0];
#pragma unroll
  for (int off = 16; off <= 32; off *= 2) {
    const double mp = __shfl_xor(m, off);
    const int ap = __shfl_xor(arg, off);
    const bool take = mp > m || (mp == m && ap < arg);
    m = take ? mp : m;
    arg = take ? ap : arg;
  }
  m_out = m;
  arg_out = arg;
}

}  // namespace dfk
