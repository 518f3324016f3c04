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
static_assert(kGateCols == kGateTileCols, "the host counts gate tiles of kGateTileCols columns");
constexpr int kGateRed = kGateWaves * kGateCT * 4 * 64;  // floats of LDS per gate block

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Partial pre-activation of one 16-row x 32-column tile of W_g h over the
// hidden slices ks0 .. ks0 + n_sl - 1 (slice ks = [ks * 256, ks * 256 + 256)
// of the hidden dimension): part[grp][row][col] = sum over those slices of
// h[row][k] W_g[col][k], grp = ks0 / kGateGroup.  In each slice wave w takes
// the contiguous quarter [64 w, 64 w + 64) as two v_mfma_f32_16x16x32_bf16
// steps per 16-column tile, accumulating across the slices in slice order;
// a slice's operand loads are all issued before its first MFMA, and each
// wave reads 128 contiguous bytes of every row it touches.  The four
// waves' tiles are summed through `red` (LDS) in wave order.  Operand
// layout: lane l holds A[l % 16][8 (l / 16) + 0..7] and
// B[8 (l / 16) + 0..7][l % 16] (one 16-byte load each, A = h and
// B[k][n] = W_g[n][k], both contiguous along k); the accumulator holds
// D[4 (l / 16) + i][l % 16].  A slice shorter than 256 (hidden is a
// multiple of 16) zero-fills the 8-element groups past its end.
// PF slices have their operand loads issued together before their MFMAs
// (PF = 1 inside the streaming launch, whose occupancy a larger register
// set would cut).  The MFMAs run in the same order for every PF, so the
// results are identical; gate_quarter_bf16 below computes the same chains
// one wave per block for the standalone gate.
// With `tpart` set, the partials go to tpart (same indices) as hand-off
// words (tag | value) for readers in the same launch.
template <int PF>
__device__ __forceinline__ void gate_partial_bf16(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W,
                                                  int R, int H, int r, float* __restrict__ part, int tile_row,
                                                  int tile_col, int ks0, int n_sl, float* red,
                                                  uint64_t* __restrict__ tpart = nullptr, uint32_t tag = 0) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row0 = tile_row * 16, col0 = tile_col * kGateCols;
  const int arow = row0 + (lane & 15);
  const int col = col0 + (lane & 15);
  constexpr int kSteps = kGateSlice / kGateWaves / 32;  // 32-wide k-steps per wave and slice
  const bf16x8 zero = {};
  v4f32 acc[kGateCT];
#pragma unroll
  for (int ct = 0; ct < kGateCT; ++ct) acc[ct] = (v4f32){0.f, 0.f, 0.f, 0.f};
  for (int kb = ks0; kb < ks0 + n_sl; kb += PF) {
    bf16x8 a[PF][kSteps], bv[PF][kSteps][kGateCT];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int ks = kb + p;
      const int kend = ks < ks0 + n_sl ? min(H, ks * kGateSlice + kGateSlice) : 0;
      const int kw = ks * kGateSlice + wave * (kGateSlice / kGateWaves) + (lane >> 4) * 8;  // this lane's first k
      const uint16_t* hp = h + (size_t)min(arow, R - 1) * H + kw;
      const uint16_t* wp = W + kw;
#pragma unroll
      for (int i = 0; i < kSteps; ++i) {
        const bool ok = kw + 32 * i < kend;
        a[p][i] = ok && arow < R ? *reinterpret_cast<const bf16x8*>(hp + 32 * i) : zero;
#pragma unroll
        for (int ct = 0; ct < kGateCT; ++ct) {
          const int c = col + ct * 16;
          bv[p][i][ct] = ok && c < r ? *reinterpret_cast<const bf16x8*>(wp + (size_t)c * H + 32 * i) : zero;
        }
      }
    }
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      if (kb + p >= ks0 + n_sl) break;
#pragma unroll
      for (int i = 0; i < kSteps; ++i)
#pragma unroll
        for (int ct = 0; ct < kGateCT; ++ct)
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[p][i], bv[p][i][ct], acc[ct], 0, 0, 0);
    }
  }
#pragma unroll
  for (int ct = 0; ct < kGateCT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wave * kGateCT + ct) * 4 + i) * kWave + lane] = acc[ct][i];
  __syncthreads();
  const size_t obase = (size_t)(ks0 / kGateGroup) * R * r;
  float* out = part + obase;
#pragma unroll
  for (int o2 = 0; o2 < kGateCT; ++o2) {
    const int o = tid + o2 * 256;
    const int ct = o >> 8, i = (o >> 6) & 3, ln = o & 63;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kGateWaves; ++w) v += red[((w * kGateCT + ct) * 4 + i) * kWave + ln];
    const int row = row0 + (ln >> 4) * 4 + i;
    const int c = col0 + ct * 16 + (ln & 15);
    if (row < R && c < r) {
      if (tpart) handoff_store_f32(tpart + obase + (size_t)row * r + c, v, tag);
      else out[(size_t)row * r + c] = v;
    }
  }
}

// One quarter of gate_partial_bf16's tile in a block of one wave: the
// MFMA chain of quarter q (k in [64 q, 64 q + 64) of every slice of the
// group), written to qpart[grp][q][row][col] unsummed; the consumer adds the
// four quarters in order (0 + q0 + q1 + q2 + q3), which is the sum the
// four-wave tile forms in LDS, so the results are identical.
template <int PF>
__device__ __forceinline__ void gate_quarter_bf16(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W,
                                                  int R, int H, int r, float* __restrict__ qpart, int tile_row,
                                                  int tile_col, int ks0, int n_sl, int wave) {
  const int lane = threadIdx.x & 63;
  const int row0 = tile_row * 16, col0 = tile_col * kGateCols;
  const int arow = row0 + (lane & 15);
  const int col = col0 + (lane & 15);
  constexpr int kSteps = kGateSlice / kGateWaves / 32;
  const bf16x8 zero = {};
  v4f32 acc[kGateCT];
#pragma unroll
  for (int ct = 0; ct < kGateCT; ++ct) acc[ct] = (v4f32){0.f, 0.f, 0.f, 0.f};
  for (int kb = ks0; kb < ks0 + n_sl; kb += PF) {
    bf16x8 a[PF][kSteps], bv[PF][kSteps][kGateCT];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int ks = kb + p;
      const int kend = ks < ks0 + n_sl ? min(H, ks * kGateSlice + kGateSlice) : 0;
      const int kw = ks * kGateSlice + wave * (kGateSlice / kGateWaves) + (lane >> 4) * 8;
      const uint16_t* hp = h + (size_t)min(arow, R - 1) * H + kw;
      const uint16_t* wp = W + kw;
#pragma unroll
      for (int i = 0; i < kSteps; ++i) {
        const bool ok = kw + 32 * i < kend;
        a[p][i] = ok && arow < R ? *reinterpret_cast<const bf16x8*>(hp + 32 * i) : zero;
#pragma unroll
        for (int ct = 0; ct < kGateCT; ++ct) {
          const int c = col + ct * 16;
          bv[p][i][ct] = ok && c < r ? *reinterpret_cast<const bf16x8*>(wp + (size_t)c * H + 32 * i) : zero;
        }
      }
    }
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      if (kb + p >= ks0 + n_sl) break;
#pragma unroll
      for (int i = 0; i < kSteps; ++i)
#pragma unroll
        for (int ct = 0; ct < kGateCT; ++ct)
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[p][i], bv[p][i][ct], acc[ct], 0, 0, 0);
    }
  }
  float* out = qpart + ((size_t)(ks0 / kGateGroup) * kGateWaves + wave) * R * r;
#pragma unroll
  for (int ct = 0; ct < kGateCT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + (lane >> 4) * 4 + i;
      const int c = col0 + ct * 16 + (lane & 15);
      if (row < R && c < r) out[(size_t)row * r + c] = acc[ct][i];
    }
}

// g from the quarters: per group (0 + q0 + q1 + q2 + q3), the groups added
// in order, then the sigmoid (the same sums as gate_value over the tiles)
__device__ __forceinline__ float gate_value_quarters(const float* __restrict__ qpart, int n_grp, size_t stride, int row,
                                                     int r, int col) {
  const float* p = qpart + (size_t)row * r + col;
  float z = 0.f;
  for (int g = 0; g < n_grp; ++g) {
    float v[kGateWaves];
#pragma unroll
    for (int q = 0; q < kGateWaves; ++q) v[q] = p[((size_t)g * kGateWaves + q) * stride];
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < kGateWaves; ++q) s += v[q];
    z += s;
  }
  return 1.0f / (1.0f + expf(-z));
}

// fp32 operands: one row of pre-activations per 256-thread block, VALU
// (a single slice)
__device__ __forceinline__ void gate_row_f32(const float* __restrict__ h, const float* __restrict__ W, int H, int r,
                                             float* __restrict__ part, int row, uint64_t* __restrict__ tpart = nullptr,
                                             uint32_t tag = 0) {
  const int col = threadIdx.x;
  if (col >= r) return;
  const float* hr = h + (size_t)row * H;
  const float* wr = W + (size_t)col * H;
  // 16-byte loads (H % 16 == 0 and the rows are 16-byte aligned), sixteen
  // of the weight row in flight per round, four accumulators: one dependent
  // chain over H would pay a memory round trip every few values
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 64 <= H; k += 64) {
    float4 w[16], x[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      w[u] = *reinterpret_cast<const float4*>(wr + k + 4 * u);
      x[u] = *reinterpret_cast<const float4*>(hr + k + 4 * u);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      acc[0] = fmaf(x[u].x, w[u].x, acc[0]);
      acc[1] = fmaf(x[u].y, w[u].y, acc[1]);
      acc[2] = fmaf(x[u].z, w[u].z, acc[2]);
      acc[3] = fmaf(x[u].w, w[u].w, acc[3]);
    }
  }
  for (; k < H; k += 4) {
    const float4 w = *reinterpret_cast<const float4*>(wr + k);
    const float4 x = *reinterpret_cast<const float4*>(hr + k);
    acc[0] = fmaf(x.x, w.x, acc[0]);
    acc[1] = fmaf(x.y, w.y, acc[1]);
    acc[2] = fmaf(x.z, w.z, acc[2]);
    acc[3] = fmaf(x.w, w.w, acc[3]);
  }
  const float v = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  if (tpart) handoff_store_f32(tpart + (size_t)row * r + col, v, tag);
  else part[(size_t)row * r + col] = v;
}

// g = sigmoid(sum of the slice-group partials, in group order) for one
// column of row `row`; `stride` = rows * r (the distance between groups)
__device__ __forceinline__ float gate_value(const float* __restrict__ part, int n_ks, size_t stride, int row, int r,
                                            int col) {
  const float* p = part + (size_t)row * r + col;
  float z = 0.f;
  for (int k0 = 0; k0 < n_ks; k0 += 8) {  // eight slices' loads in flight at once
    // unconditional loads (slices past the last re-read it and are not
    // added): a masked load would be a branch that waits for the loads
    // issued before it
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[(size_t)min(k0 + i, n_ks - 1) * stride];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (k0 + i < n_ks) z += v[i];
  }
  return 1.0f / (1.0f + expf(-z));
}

// ---------------------------------------------------------------- edge scores

// LDS of one edge's scores in a 256-thread block (small enough to share a
// launch with the streaming blocks without costing them occupancy)
struct EdgeLds {
  float g[DFLASH_R_MAX];   // gate of this edge
  float red[4][4][kWave];  // per-wave partial 16 x 16 products (MFMA accumulator layout)
  int pidx[16], cidx[16];  // predecessor / candidate tokens (-1: zero row)
  float cl[16];            // candidate drafter logits U_t(b)
};

// g_t[k] for every k < r of drafter row `row` into e.g (threads k < r)
__device__ __forceinline__ void edge_gate(EdgeLds& e, const float* __restrict__ gpart, int n_ks, size_t gstride,
                                          int row, int r) {
  if ((int)threadIdx.x < r) e.g[threadIdx.x] = gate_value(gpart, n_ks, gstride, row, r, threadIdx.x);
}

// The n = r / 16 consecutive stored values E[idx][k0 .. k0 + n) (n <= 16;
// zeros when idx < 0), raw: 16-byte loads when the run allows them (the
// run then starts 16-byte aligned), single values otherwise.
template <int PT>
struct Run {
  static constexpr int NU = PT == DFLASH_BF16 ? 2 : 4;  // 16-byte units of 16 values
  uint4 u[NU];

  __device__ __forceinline__ void load(const void* __restrict__ E, int idx, int r, int k0, int n) {
#pragma unroll
    for (int h = 0; h < NU; ++h) u[h] = make_uint4(0, 0, 0, 0);
    if (idx < 0) return;
    constexpr int EPU = 16 / NU;  // values per unit
    if (PT == DFLASH_BF16) {
      const uint16_t* p = reinterpret_cast<const uint16_t*>(E) + (size_t)idx * r + k0;
      if (n % EPU == 0) {
#pragma unroll
        for (int h = 0; h < NU; ++h)
          if (EPU * h < n) u[h] = reinterpret_cast<const uint4*>(p)[h];
      } else {
        uint32_t w[8] = {};
#pragma unroll
        for (int s = 0; s < 16; ++s)
          if (s < n) w[s >> 1] |= (uint32_t)p[s] << (16 * (s & 1));
#pragma unroll
        for (int h = 0; h < NU; ++h) u[h] = make_uint4(w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]);
      }
    } else {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(E) + (size_t)idx * r + k0;
      if (n % EPU == 0) {
#pragma unroll
        for (int h = 0; h < NU; ++h)
          if (EPU * h < n) u[h] = reinterpret_cast<const uint4*>(p)[h];
      } else {
        uint32_t w[16] = {};
#pragma unroll
        for (int s = 0; s < 16; ++s)
          if (s < n) w[s] = p[s];
#pragma unroll
        for (int h = 0; h < NU; ++h) u[h] = make_uint4(w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]);
      }
    }
  }

  // value s of the run as fp32 (s a compile-time constant after unrolling)
  __device__ __forceinline__ float at(int s) const {
    const uint4 q = u[PT == DFLASH_BF16 ? s >> 3 : s >> 2];
    const int c = PT == DFLASH_BF16 ? (s >> 1) & 3 : s & 3;
    const uint32_t w = c == 0 ? q.x : c == 1 ? q.y : c == 2 ? q.z : q.w;
    if (PT == DFLASH_BF16) return (s & 1) ? bf16_hi(w) : bf16_lo(w);
    return __uint_as_float(w);
  }
};

// Scores of one edge, S[i][j] = cl[j] + sum_k E[pidx_i,k] g_t[k] E[cidx_j,k],
// with g_t staged in e.g (barrier passed) and, in registers, this lane's
// operand tokens (pidx_l = pidx_{l%16}, cidx_l = cidx_{l%16}) and this
// thread's candidate logit (cl_j = cl[tid % 16]).
// The 16 x r x 16 contraction runs on the matrix cores in fp32
// (v_mfma_f32_16x16x4_f32) with operands taken straight from the gathered
// embedding rows: wave w covers k in [w r/4, (w+1) r/4); lane group
// q = l / 16 owns the run of n = r/16 consecutive k starting at
// k(q) = (4 w + q) n and feeds its s-th value at step s, so lane l gives
// A[l % 16][k(q) + s] = E[pidx_{l%16}, k] g_t[k] and B[k(q) + s][l % 16] =
// E[cidx_{l%16}, k] (each lane reads one contiguous run per row: a wave
// reads whole 128-byte row pieces) and holds D[4 (l / 16) + v][l % 16].
// The four waves' products are summed in wave order.  The split entry
// point and the fused cycle both call this, so their scores are identical.
// Returns the score S[tid / 16][tid % 16] of the calling thread (meaningful
// where both indices are below K), so wave w holds rows 4 w .. 4 w + 3, one
// per 16-lane group.
template <int PT>
__device__ __forceinline__ float edge_contract_rows(EdgeLds& e, const void* __restrict__ E, int K, int r, int pidx_l,
                                                    int cidx_l, float cl_j, float* __restrict__ S_edge) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = r >> 4;
  const int k0 = ((wave << 2) + (lane >> 4)) * n;
  Run<PT> av, cv;
  av.load(E, pidx_l, r, k0, n);
  cv.load(E, cidx_l, r, k0, n);
  v4f32 acc = (v4f32){0.f, 0.f, 0.f, 0.f};
  if (n == 16) {  // r = 256: straight-line steps
#pragma unroll
    for (int s = 0; s < 16; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.at(s) * e.g[k0 + s], cv.at(s), acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if (s < n) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.at(s) * e.g[k0 + s], cv.at(s), acc, 0, 0, 0);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) e.red[wave][v][lane] = acc[v];
  __syncthreads();
  const int i = tid >> 4, j = tid & 15;
  const int ln = ((i >> 2) << 4) + j, v = i & 3;
  const float d = ((e.red[0][v][ln] + e.red[1][v][ln]) + e.red[2][v][ln]) + e.red[3][v][ln];
  const float sv = cl_j + d;
  if (i < K && j < K) S_edge[i * K + j] = sv;
  return sv;
}

// The same with the tokens and logits taken from the lists staged in `e`
// (pidx, cidx, cl and g filled, barrier passed).
template <int PT>
__device__ __forceinline__ float edge_contract(EdgeLds& e, const void* __restrict__ E, int K, int r,
                                               float* __restrict__ S_edge) {
  const int lane = threadIdx.x & 63;
  return edge_contract_rows<PT>(e, E, K, r, e.pidx[lane & 15], e.cidx[lane & 15], e.cl[threadIdx.x & 15], S_edge);
}

// ---------------------------------------------------------------- trace step

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

// Decision of one row (t, i) of the trace table, held by a 16-lane group
// g of the wave: lane j of the group holds s = S[t][i][j] (live: j < K),
// the scores of the successors of rank i at position t.  Greedy: the
// smallest rank attaining the maximum.  Sampling: w = exp((s - max) / T) in
// fp64 (as a product with invT = 1 / T), q = w / total, and the smallest
// rank whose inclusive prefix of w exceeds u * total, u the trace uniform
// (word 0 of the (cycle, t + 1, 0) block).  Returns the rank for every lane
// of the group and sets this lane's q.  Both trace entry points (the
// standalone trace and the fused cycle) decide every row of every position
// up front with this function; the walk itself is then L table look-ups.
__device__ __forceinline__ int trace_row_decide(float s, bool live, int g, int j, float Tb, double invT, uint32_t u,
                                                int K, float& qv) {
  s = live ? s : -INFINITY;
  const float m = __uint_as_float(group_last_u32(__float_as_uint(row16_scan_max_f32(s)), g));
  int jd;
  if (!(Tb > 0.0f)) {
    const uint32_t bits = (uint32_t)(__ballot(live && s == m) >> (16 * g)) & 0xFFFFu;
    jd = bits ? __builtin_ctz(bits) : 0;
    qv = j == jd ? 1.0f : 0.0f;
  } else {
    const double w = live ? exp_nonpos(((double)s - (double)m) * invT) : 0.0;
    const double cum = row16_scan_f64(w);
    const double total = group_last_f64(cum, g);
    const double target = (double)u01_f32(u) * total;
    const uint32_t bits = (uint32_t)(__ballot(live && cum > target) >> (16 * g)) & 0xFFFFu;
    jd = bits ? __builtin_ctz(bits) : K - 1;
    qv = (float)(w / total);
  }
  return jd;
}

}  // namespace dfk
