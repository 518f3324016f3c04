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

constexpr int kGateWaves = 4;          // waves per gate block
constexpr int kGateCT = 2;             // 16-column tiles per gate block (32 columns)
constexpr int kGateCols = 16 * kGateCT;
constexpr int kGateRed = kGateWaves * kGateCT * 4 * 64;  // floats of LDS per gate block

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Partial pre-activation of one 16-row x 32-column tile of W_g h over
// hidden slice ks ([ks * 256, ks * 256 + 256) of the hidden dimension):
// part[ks][row][col] = sum over the slice of h[row][k] W_g[col][k].  Wave w
// takes the contiguous quarter [64 w, 64 w + 64) of the slice as two
// v_mfma_f32_16x16x32_bf16 steps per 16-column tile; every operand load is
// issued before the first MFMA, so a block waits on memory once, and each
// wave reads 128 contiguous bytes of every row it touches.  The four
// waves' tiles are summed through `red` (LDS) in wave order.  Operand
// layout: lane l holds A[l % 16][8 (l / 16) + 0..7] and
// B[8 (l / 16) + 0..7][l % 16] (one 16-byte load each, A = h and
// B[k][n] = W_g[n][k], both contiguous along k); the accumulator holds
// D[4 (l / 16) + i][l % 16].  A hidden slice shorter than 256 (hidden is a
// multiple of 16) zero-fills the 8-element groups past its end.
__device__ __forceinline__ void gate_partial_bf16(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W,
                                                  int R, int H, int r, float* __restrict__ part, int tile_row,
                                                  int tile_col, int ks, float* red) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row0 = tile_row * 16, col0 = tile_col * kGateCols;
  const int kend = min(H, ks * kGateSlice + kGateSlice);
  const int kw = ks * kGateSlice + wave * (kGateSlice / kGateWaves) + (lane >> 4) * 8;  // this lane's first k
  const int arow = row0 + (lane & 15);
  const uint16_t* hp = h + (size_t)min(arow, R - 1) * H + kw;
  const int col = col0 + (lane & 15);
  const uint16_t* wp = W + kw;
  constexpr int kSteps = kGateSlice / kGateWaves / 32;  // 32-wide k-steps per wave
  const bf16x8 zero = {};
  bf16x8 a[kSteps], bv[kSteps][kGateCT];
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const bool ok = kw + 32 * i < kend;
    a[i] = ok && arow < R ? *reinterpret_cast<const bf16x8*>(hp + 32 * i) : zero;
#pragma unroll
    for (int ct = 0; ct < kGateCT; ++ct) {
      const int c = col + ct * 16;
      bv[i][ct] = ok && c < r ? *reinterpret_cast<const bf16x8*>(wp + (size_t)c * H + 32 * i) : zero;
    }
  }
  v4f32 acc[kGateCT];
#pragma unroll
  for (int ct = 0; ct < kGateCT; ++ct) acc[ct] = (v4f32){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kSteps; ++i)
#pragma unroll
    for (int ct = 0; ct < kGateCT; ++ct)
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bv[i][ct], acc[ct], 0, 0, 0);
#pragma unroll
  for (int ct = 0; ct < kGateCT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wave * kGateCT + ct) * 4 + i) * kWave + lane] = acc[ct][i];
  __syncthreads();
  float* out = part + (size_t)ks * R * r;
#pragma unroll
  for (int o2 = 0; o2 < kGateCT; ++o2) {
    const int o = tid + o2 * 256;
    const int ct = o >> 8, i = (o >> 6) & 3, ln = o & 63;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kGateWaves; ++w) v += red[((w * kGateCT + ct) * 4 + i) * kWave + ln];
    const int row = row0 + (ln >> 4) * 4 + i;
    const int c = col0 + ct * 16 + (ln & 15);
    if (row < R && c < r) out[(size_t)row * r + c] = v;
  }
}

// fp32 operands: one row of pre-activations per 256-thread block, VALU
// (a single slice)
__device__ __forceinline__ void gate_row_f32(const float* __restrict__ h, const float* __restrict__ W, int H, int r,
                                             float* __restrict__ part, int row) {
  const int col = threadIdx.x;
  if (col >= r) return;
  const float* hr = h + (size_t)row * H;
  const float* wr = W + (size_t)col * H;
  float acc = 0.f;
  for (int k = 0; k < H; ++k) acc = fmaf(hr[k], wr[k], acc);
  part[(size_t)row * r + col] = acc;
}

// g = sigmoid(sum of the slice partials, in slice order) for one column of
// row `row`; `stride` = rows * r (the distance between slices)
__device__ __forceinline__ float gate_value(const float* __restrict__ part, int n_ks, size_t stride, int row, int r,
                                            int col) {
  const float* p = part + (size_t)row * r + col;
  float z = 0.f;
  for (int ks = 0; ks < n_ks; ++ks) z += p[ks * stride];
  return 1.0f / (1.0f + expf(-z));
}

// ---------------------------------------------------------------- edge scores

constexpr int kRowPad = DFLASH_R_MAX + 4;  // 16-byte aligned LDS rows

struct EdgeLds {
  float A[16][kRowPad];  // predecessor rows scaled by g_t
  float C[16][kRowPad];  // candidate rows
  float red[4][4][kWave];  // per-wave partial 16 x 16 products (MFMA accumulator layout)
  float g[DFLASH_R_MAX];   // gate of this edge
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

// Scores of edge (b, t) (drafter row `row`) from the staged index lists in
// `e` (pidx, cidx, cl filled, barrier passed):
// S[i][j] = cl[j] + sum_k E[pidx_i,k] g_t[k] E[cidx_j,k], with g_t summed
// from the gate slices (gpart, n_ks slices `gstride` apart).
// The 16 x r x 16 contraction runs on the matrix cores in fp32
// (v_mfma_f32_16x16x4_f32): wave w takes the k-range [w r/4, (w+1) r/4),
// A = g-scaled predecessor rows, B[k][j] = candidate row j; lane l feeds
// A[l % 16][k0 + l / 16] and B[k0 + l / 16][l % 16] (with the LDS row pitch
// of 260 floats the 64 lanes hit 64 distinct banks) and holds
// D[4 (l / 16) + v][l % 16].  The four partial products are summed in wave
// order.
template <int PT>
__device__ __forceinline__ void edge_scores(EdgeLds& e, const void* __restrict__ E, const float* __restrict__ gpart,
                                            int n_ks, size_t gstride, int row, int K, int r,
                                            float* __restrict__ S_edge) {
  RowLoad<PT> a, c;
  a.load(E, e.pidx, r);
  c.load(E, e.cidx, r);
  if ((int)threadIdx.x < r) e.g[threadIdx.x] = gate_value(gpart, n_ks, gstride, row, r, threadIdx.x);
  __syncthreads();
  a.store(r, e.g, e.A);
  c.store(r, nullptr, e.C);
  __syncthreads();
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int steps = r >> 4;  // k-steps of 4 per wave
  const int ka = wave * (r >> 2) + (lane >> 4);
  const float* ar = &e.A[lane & 15][ka];
  const float* cr = &e.C[lane & 15][ka];
  v4f32 acc = (v4f32){0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < steps; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ar[4 * s], cr[4 * s], acc, 0, 0, 0);
#pragma unroll
  for (int v = 0; v < 4; ++v) e.red[wave][v][lane] = acc[v];
  __syncthreads();
  const int i = tid >> 4, j = tid & 15;
  const int ln = ((i >> 2) << 4) + j, v = i & 3;
  const float d = ((e.red[0][v][ln] + e.red[1][v][ln]) + e.red[2][v][ln]) + e.red[3][v][ln];
  if (i < K && j < K) S_edge[i * K + j] = e.cl[j] + d;
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
// the maximum.  Sampling: w = exp((s - max) / T) in fp64 (the quotient
// taken as a product with invT = 1 / T), q = w / total, and the smallest
// rank whose inclusive prefix of w exceeds u * total.
// `ci` (LDS) holds the clamped candidate tokens of this position.  Writes
// q (global, and LDS when qs_lds is given), the rank and the token.
__device__ __forceinline__ int trace_step_dpp(const TraceLds& tl, const float* srow, float Tb, double invT, int t,
                                              int K, int lane,
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
    const double w = lane < K ? exp_nonpos(((double)s - (double)m) * invT) : 0.0;
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

// value of lane 16 g + 15 in every lane of 16-lane group g
__device__ __forceinline__ uint32_t group_last_u32(uint32_t v, int g) {
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 47), r3 = __builtin_amdgcn_readlane(v, 63);
  return g == 0 ? r0 : (g == 1 ? r1 : (g == 2 ? r2 : r3));
}

__device__ __forceinline__ double group_last_f64(double v, int g) {
  const uint64_t b = __double_as_longlong(v);
  const uint64_t lo = group_last_u32((uint32_t)b, g), hi = group_last_u32((uint32_t)(b >> 32), g);
  return __longlong_as_double((long long)((hi << 32) | lo));
}

// NQ x 4 rows of the trace table at once (16-lane group g of the wave takes
// rows row0 + 4 n + g, n < NQ; the NQ quads are independent, so their
// latency chains overlap): row (t, i) holds the scores S[t][i][.] of the
// successors of rank i at position t (LDS, K floats).  Each row gets the
// walk's decision -- the same arithmetic as trace_step_dpp -- written to
// jstar[row], and its q written over the scores in place.  With every row
// decided up front, the sequential walk is only L table look-ups.
// u[t] holds the trace uniform of position t (unused when greedy).
template <int NQ>
__device__ __forceinline__ void trace_rows(float* S, int row0, int n_rows, int K, float Tb, double invT,
                                           const uint4* u, int* jstar, int lane) {
  const int g = lane >> 4, j = lane & 15;
  int row[NQ];
  bool live[NQ];
  float s[NQ], m[NQ];
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    row[n] = row0 + 4 * n + g;
    live[n] = row[n] < n_rows && j < K;
    s[n] = live[n] ? S[(size_t)row[n] * K + j] : -INFINITY;
  }
#pragma unroll
  for (int n = 0; n < NQ; ++n) m[n] = __uint_as_float(group_last_u32(__float_as_uint(row16_scan_max_f32(s[n])), g));
  int jd[NQ];
  float qv[NQ];
  if (!(Tb > 0.0f)) {
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const uint32_t bits = (uint32_t)(__ballot(live[n] && s[n] == m[n]) >> (16 * g)) & 0xFFFFu;
      jd[n] = bits ? __builtin_ctz(bits) : 0;
      qv[n] = j == jd[n] ? 1.0f : 0.0f;
    }
  } else {
    double w[NQ], cum[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) w[n] = live[n] ? exp_nonpos(((double)s[n] - (double)m[n]) * invT) : 0.0;
#pragma unroll
    for (int n = 0; n < NQ; ++n) cum[n] = row16_scan_f64(w[n]);
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const double total = group_last_f64(cum[n], g);
      const double target = (double)u01_f32(u[row[n] < n_rows ? row[n] / K : 0].x) * total;
      const uint32_t bits = (uint32_t)(__ballot(live[n] && cum[n] > target) >> (16 * g)) & 0xFFFFu;
      jd[n] = bits ? __builtin_ctz(bits) : K - 1;
      qv[n] = (float)(w[n] / total);
    }
  }
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    if (live[n]) S[(size_t)row[n] * K + j] = qv[n];
    if (row[n] < n_rows && j == 0) jstar[row[n]] = jd[n];
  }
}

}  // namespace dfk
