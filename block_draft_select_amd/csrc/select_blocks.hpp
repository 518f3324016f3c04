// Device building blocks of S2..S4 (context gate, adjacent pair scores and
// the lattice trace; P3 "DFlash 2: Keep Drafting Parallel", section "What
// Comes Next", paragraph "A Lightweight Path Selector"; P1 "DFlash 2: Block
// diffusion, wearing a drafter's coat", sub-section "A path selector").
// The split entry points and the fused cycle call these same functions, so
// both give bit-identical results.
#pragma once

#include "device_util.hpp"
#include "internal.hpp"

namespace dfk {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef float v4f32 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- gate

constexpr int kGateWaves = 4;          // waves per gate block (split the hidden dimension)
constexpr int kGateRed = kGateWaves * 4 * 4 * 64;  // floats of LDS per gate block

// One 16-row x 64-column tile of g = sigmoid(h @ W_g^T), 4 waves splitting
// the hidden dimension, partial tiles summed through `red` (LDS) in wave
// order.  MFMA 16x16x16 bf16 operand layout: lane l holds
// A[l % 16][4 (l / 16) + 0..3] and B[4 (l / 16) + 0..3][l % 16]; the
// accumulator holds D[4 (l / 16) + i][l % 16].  Here A = h and
// B[k][n] = W_g[n][k]: both are contiguous along k, one 8-byte load each.
__device__ __forceinline__ void gate_tile_bf16(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int R,
                                               int H, int r, float* __restrict__ g, int tile_row, int tile_col,
                                               float* red) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row0 = tile_row * 16, col0 = tile_col * 64;
  const int ns = H / 16;
  const int s0 = wave * ns / kGateWaves, s1 = (wave + 1) * ns / kGateWaves;
  const int arow = row0 + (lane & 15);
  const int kq = (lane >> 4) * 4;
  const uint16_t* hp = h + (size_t)min(arow, R - 1) * H + kq;
  const uint16_t* wp[4];
  bool wok[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int col = col0 + ct * 16 + (lane & 15);
    wok[ct] = col < r;
    wp[ct] = W + (size_t)min(col, r - 1) * H + kq;
  }
  v4f32 acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = (v4f32){0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int s = s0; s < s1; ++s) {
    v4i16 a = *reinterpret_cast<const v4i16*>(hp + s * 16);
    if (arow >= R) a = (v4i16){0, 0, 0, 0};
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      v4i16 bv = *reinterpret_cast<const v4i16*>(wp[ct] + s * 16);
      if (!wok[ct]) bv = (v4i16){0, 0, 0, 0};
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bv, acc[ct], 0, 0, 0);
    }
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wave * 4 + ct) * 4 + i) * kWave + lane] = acc[ct][i];
  __syncthreads();
#pragma unroll
  for (int o4 = 0; o4 < 4; ++o4) {
    const int o = tid + o4 * 256;
    const int ct = o >> 8, i = (o >> 6) & 3, ln = o & 63;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kGateWaves; ++w) v += red[((w * 4 + ct) * 4 + i) * kWave + ln];
    const int row = row0 + (ln >> 4) * 4 + i;
    const int col = col0 + ct * 16 + (ln & 15);
    if (row < R && col < r) g[(size_t)row * r + col] = 1.0f / (1.0f + expf(-v));
  }
}

// fp32 operands: one row of g per 256-thread block, VALU
__device__ __forceinline__ void gate_row_f32(const float* __restrict__ h, const float* __restrict__ W, int H, int r,
                                             float* __restrict__ g, int row) {
  const int col = threadIdx.x;
  if (col >= r) return;
  const float* hr = h + (size_t)row * H;
  const float* wr = W + (size_t)col * H;
  float acc = 0.f;
  for (int k = 0; k < H; ++k) acc = fmaf(hr[k], wr[k], acc);
  g[(size_t)row * r + col] = 1.0f / (1.0f + expf(-acc));
}

// ---------------------------------------------------------------- edge scores

constexpr int kRowPad = DFLASH_R_MAX + 4;  // 16-byte aligned LDS rows

struct EdgeLds {
  float A[16][kRowPad];  // predecessor rows scaled by g_t
  float C[16][kRowPad];  // candidate rows
  int pidx[16], cidx[16];
  float cl[16];
};

// 16 embedding rows E[idx[i]] (zero rows where idx[i] < 0) of width r, one
// 256-thread block's share per thread: loaded into registers first, stored
// to LDS (fp32) afterwards, so that several row sets can be in flight.
template <int PT>
struct RowLoad {
  static constexpr int EPU = PT == DFLASH_BF16 ? 8 : 4;  // values per 16-byte load
  static constexpr int NU = PT == DFLASH_BF16 ? 2 : 4;   // loads per thread (16 rows x 256 values max)
  uint4 v[NU];

  __device__ __forceinline__ void load(const void* __restrict__ E, const int* idx, int r) {
    const int tid = threadIdx.x;
    const int upr = r / EPU;
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const int u = tid + k * 256;
      const int row = u / upr, col = (u - row * upr) * EPU;
      v[k] = make_uint4(0, 0, 0, 0);
      if (row < 16 && idx[row] >= 0) {
        if (PT == DFLASH_BF16)
          v[k] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(E) + (size_t)idx[row] * r + col);
        else
          v[k] = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(E) + (size_t)idx[row] * r + col);
      }
    }
  }

  // dst[row][col] = value, multiplied by g[col] when g is given
  __device__ __forceinline__ void store(int r, const float* g, float (*dst)[kRowPad]) const {
    const int tid = threadIdx.x;
    const int upr = r / EPU;
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const int u = tid + k * 256;
      const int row = u / upr, col = (u - row * upr) * EPU;
      if (row < 16) {
        float f[EPU];
        if (PT == DFLASH_BF16) {
          f[0] = bf16_lo(v[k].x); f[1] = bf16_hi(v[k].x);
          f[2] = bf16_lo(v[k].y); f[3] = bf16_hi(v[k].y);
          f[4] = bf16_lo(v[k].z); f[5] = bf16_hi(v[k].z);
          f[6] = bf16_lo(v[k].w); f[7] = bf16_hi(v[k].w);
        } else {
          f[0] = __uint_as_float(v[k].x); f[1] = __uint_as_float(v[k].y);
          f[2] = __uint_as_float(v[k].z); f[3] = __uint_as_float(v[k].w);
        }
#pragma unroll
        for (int e = 0; e < EPU; ++e) dst[row][col + e] = g ? f[e] * g[col + e] : f[e];
      }
    }
  }
};

// sum_k a[k] * c[k] in index order (one fused multiply-add per term);
// r is a multiple of 16, read 16 values of each operand per step
__device__ __forceinline__ float score_dot(const float* a, const float* c, int r) {
  float acc = 0.f;
  for (int k = 0; k < r; k += 16) {
    float4 av[4], cv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      av[u] = *reinterpret_cast<const float4*>(a + k + 4 * u);
      cv[u] = *reinterpret_cast<const float4*>(c + k + 4 * u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc = fmaf(av[u].x, cv[u].x, acc);
      acc = fmaf(av[u].y, cv[u].y, acc);
      acc = fmaf(av[u].z, cv[u].z, acc);
      acc = fmaf(av[u].w, cv[u].w, acc);
    }
  }
  return acc;
}

// Scores of edge (b, t) from the staged index lists in `e` (pidx, cidx, cl
// filled, barrier passed): S[i][j] = cl[j] + sum_k E[pidx_i,k] g_t[k] E[cidx_j,k].
template <int PT>
__device__ __forceinline__ void edge_scores(EdgeLds& e, const void* __restrict__ E, const float* __restrict__ gt,
                                            int K, int r, float* __restrict__ S_edge) {
  RowLoad<PT> a, c;
  a.load(E, e.pidx, r);
  c.load(E, e.cidx, r);
  a.store(r, gt, e.A);
  c.store(r, nullptr, e.C);
  __syncthreads();
  const int tid = threadIdx.x;
  const int i = tid >> 4, j = tid & 15;
  if (i < K && j < K) S_edge[i * K + j] = e.cl[j] + score_dot(e.A[i], e.C[j], r);
}

// ---------------------------------------------------------------- trace step

struct TraceLds {
  uint32_t u[DFLASH_L_MAX];  // word 0 of the (cycle, t + 1, 0) blocks
};

__device__ __forceinline__ void trace_setup(TraceLds& tl, float Tb, uint64_t seed, uint64_t cycle, int L, int lane) {
  if (Tb > 0.0f && lane < L) tl.u[lane] = stream_block(seed, cycle, (uint32_t)(lane + 1), 0u).x;
}

// One step of the walk by one wave; lane k < K holds the score of rank k
// in the predecessor's row `srow` (LDS).  Greedy: smallest rank attaining
// the maximum.  Sampling: w = exp((s - max) / T) in fp64, q = w / total,
// and the smallest rank whose inclusive prefix of w exceeds u * total.
// `ci` (LDS) holds the clamped candidate tokens of this position.  Writes
// q (global, and LDS when qs_lds is given), the rank and the token.
__device__ __forceinline__ int trace_step_dpp(const TraceLds& tl, const float* srow, float Tb, int t, int K, int lane,
                                              const int* ci, float* __restrict__ q_out, int32_t* __restrict__ rank_out,
                                              int32_t* __restrict__ tok_out, float* qs_lds) {
  const float s = lane < K ? srow[lane] : -INFINITY;
  const float m = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(row16_scan_max_f32(s)), 15));
  int j;
  float qv;
  if (!(Tb > 0.0f)) {
    j = first_lane(lane < K && s == m);
    if (j >= K) j = 0;
    qv = lane == j ? 1.0f : 0.0f;
  } else {
    const double w = lane < K ? exp(((double)s - (double)m) / (double)Tb) : 0.0;
    const double cum = row16_scan_f64(w);
    const double total = readlane_f64(cum, K - 1);
    const double target = (double)u01_f32(tl.u[t]) * total;
    j = first_lane(lane < K && cum > target);
    if (j >= K) j = K - 1;
    qv = (float)(w / total);
  }
  if (lane < K) {
    q_out[lane] = qv;
    if (qs_lds) qs_lds[lane] = qv;
  }
  if (lane == 0) {
    *rank_out = j;
    *tok_out = ci[j];
  }
  return j;
}

}  // namespace dfk
