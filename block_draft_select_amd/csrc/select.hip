// S2..S4: context gate, adjacent pair scores and the lattice trace (P3
// "DFlash 2: Keep Drafting Parallel", section "What Comes Next", paragraph
// "A Lightweight Path Selector"; P1 "DFlash 2: Block diffusion, wearing a
// drafter's coat", sub-section "A path selector").
//
// gate:   g = sigmoid(h @ W_g), a [B*L, hidden] x [hidden, r] contraction.
//         bf16 operands run on MFMA (v_mfma_f32_16x16x16_bf16, fp32
//         accumulation; bf16 products are exact in fp32); a block owns a
//         16-row x 64-column tile and its four waves split the hidden
//         dimension, summed in a fixed order.  fp32 operands use VALU FMAs.
// scores: one block per edge (b, t): the 16 predecessor and 16 candidate
//         embedding rows are gathered into LDS in fp32 (predecessors already
//         scaled by g), then thread (i, j) forms the r-term dot product.
// trace:  one wave per stream walks the L edges; the softmax and inverse
//         CDF of a step run in fp64 over the K fp32 scores.
#include "device_util.hpp"
#include "internal.hpp"

namespace dfk {

namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef float v4f32 __attribute__((ext_vector_type(4)));

// MFMA 16x16x16 bf16 operand layout: lane l holds A[l % 16][4 (l / 16) + 0..3]
// and B[4 (l / 16) + 0..3][l % 16]; the accumulator holds D[4 (l / 16) + i][l % 16].
__global__ __launch_bounds__(256) void gate_mfma_bf16(const uint16_t* __restrict__ h,
                                                      const uint16_t* __restrict__ W, int R, int H,
                                                      int r, float* __restrict__ g) {
  __shared__ float red[4][4][4][kWave];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row0 = blockIdx.x * 16, col0 = blockIdx.y * 64;
  const int ns = H / 16;
  const int s0 = wave * ns / 4, s1 = (wave + 1) * ns / 4;
  const int arow = row0 + (lane & 15);
  const int kq = (lane >> 4) * 4;
  v4f32 acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = (v4f32){0.f, 0.f, 0.f, 0.f};
  for (int s = s0; s < s1; ++s) {
    const int k0 = s * 16 + kq;
    v4i16 a = (v4i16){0, 0, 0, 0};
    if (arow < R) a = *reinterpret_cast<const v4i16*>(h + (size_t)arow * H + k0);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int col = col0 + ct * 16 + (lane & 15);
      v4i16 bv = (v4i16){0, 0, 0, 0};
      if (col < r) {
        const uint16_t* wp = W + (size_t)k0 * r + col;
        bv = (v4i16){(short)wp[0], (short)wp[r], (short)wp[2 * r], (short)wp[3 * r]};
      }
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bv, acc[ct], 0, 0, 0);
    }
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][ct][i][lane] = acc[ct][i];
  __syncthreads();
  const int ct = wave;  // wave w finishes column tile w
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float v = ((red[0][ct][i][lane] + red[1][ct][i][lane]) + red[2][ct][i][lane]) + red[3][ct][i][lane];
    const int row = row0 + (lane >> 4) * 4 + i;
    const int col = col0 + ct * 16 + (lane & 15);
    if (row < R && col < r) g[(size_t)row * r + col] = 1.0f / (1.0f + expf(-v));
  }
}

__global__ __launch_bounds__(256) void gate_f32(const float* __restrict__ h, const float* __restrict__ W,
                                                int R, int H, int r, float* __restrict__ g) {
  const int row = blockIdx.x, col = threadIdx.x;
  if (col >= r) return;
  const float* hr = h + (size_t)row * H;
  float acc = 0.f;
  for (int k = 0; k < H; ++k) acc = fmaf(hr[k], W[(size_t)k * r + col], acc);
  g[(size_t)row * r + col] = 1.0f / (1.0f + expf(-acc));
}

template <int PT>
__device__ __forceinline__ void load8(const void* E, size_t off, float (&v)[8]) {
  if (PT == DFLASH_BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(E) + off);
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x);
    v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z);
    v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(E) + off);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(E) + off + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <int PT>
__global__ __launch_bounds__(256) void scores_kernel(const int32_t* __restrict__ x0,
                                                     const int32_t* __restrict__ cand_idx,
                                                     const float* __restrict__ cand_logit,
                                                     const void* __restrict__ E, const float* __restrict__ g,
                                                     int L, int V, int K, int r, float* __restrict__ S) {
  __shared__ float A[16][DFLASH_R_MAX + 1];  // predecessor rows scaled by g
  __shared__ float C[16][DFLASH_R_MAX + 1];  // candidate rows
  __shared__ int pidx[16], cidx[16];
  const int bt = blockIdx.x;
  const int b = bt / L, t = bt - b * L;
  const int tid = threadIdx.x;
  if (tid < 16) {
    int p = -1, c = -1;
    if (tid < K) {
      p = (t == 0) ? clamp_idx(x0[b], V) : clamp_idx(cand_idx[((size_t)b * L + t - 1) * K + tid], V);
      c = clamp_idx(cand_idx[((size_t)b * L + t) * K + tid], V);
    }
    pidx[tid] = p;
    cidx[tid] = c;
  }
  __syncthreads();
  const float* gr = g + (size_t)bt * r;
  const int cpr = r / 8;
  for (int i = tid; i < 32 * cpr; i += 256) {
    const int row = i / cpr, k0 = (i - row * cpr) * 8;
    const int idx = row < 16 ? pidx[row] : cidx[row - 16];
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (idx >= 0) load8<PT>(E, (size_t)idx * r + k0, v);
    if (row < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) A[row][k0 + e] = v[e] * gr[k0 + e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) C[row - 16][k0 + e] = v[e];
    }
  }
  __syncthreads();
  const int i = tid >> 4, j = tid & 15;
  if (i < K && j < K) {
    float acc = 0.f;
    for (int k = 0; k < r; ++k) acc = fmaf(A[i][k], C[j][k], acc);
    const size_t e0 = ((size_t)b * L + t) * K;
    S[(e0 + i) * K + j] = cand_logit[e0 + j] + acc;
  }
}

__global__ __launch_bounds__(64) void trace_kernel(const float* __restrict__ S, const int32_t* __restrict__ cand_idx,
                                                   const float* __restrict__ T, const uint64_t* __restrict__ seed,
                                                   uint64_t cycle, int L, int V, int K,
                                                   int32_t* __restrict__ path_rank, int32_t* __restrict__ draft_tok,
                                                   float* __restrict__ q) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const float Tb = T[b];
  const bool greedy = !(Tb > 0.0f);
  const uint64_t sd = seed[b];
  int prev = 0;
  for (int t = 0; t < L; ++t) {
    const size_t e0 = ((size_t)b * L + t) * K;
    const float s = lane < K ? S[(e0 + prev) * K + lane] : -INFINITY;
    const float m = wave_max_f32(s);
    int j;
    float qv;
    if (greedy) {
      j = wave_min_i32((lane < K && s == m) ? lane : 0x7FFFFFFF);
      if (j >= K) j = 0;
      qv = lane == j ? 1.0f : 0.0f;
    } else {
      const double w = lane < K ? exp(((double)s - (double)m) / (double)Tb) : 0.0;
      double cum = 0.0;  // inclusive prefix in rank order, summed sequentially
      for (int k = 0; k < K; ++k) {
        const double wk = __shfl(w, k);
        if (k <= lane) cum += wk;
      }
      const double total = __shfl(cum, K - 1);
      const uint4 rw = stream_block(sd, cycle, (uint32_t)(t + 1), 0u);
      const double target = (double)u01_f32(rw.x) * total;
      j = wave_min_i32((lane < K && cum > target) ? lane : 0x7FFFFFFF);
      if (j >= K) j = K - 1;
      qv = (float)(w / total);
    }
    if (lane < K) q[e0 + lane] = qv;
    if (lane == 0) {
      path_rank[(size_t)b * L + t] = j;
      draft_tok[(size_t)b * L + t] = clamp_idx(cand_idx[e0 + j], V);
    }
    prev = j;
  }
}

}  // namespace

hipError_t launch_gate(const dflash_dims& d, const void* h, const void* W_g, float* g, hipStream_t st) {
  const int R = d.B * d.L;
  if (d.param_dtype == DFLASH_BF16) {
    const dim3 grid((unsigned)((R + 15) / 16), (unsigned)((d.r + 63) / 64));
    hipLaunchKernelGGL(gate_mfma_bf16, grid, dim3(256), 0, st, reinterpret_cast<const uint16_t*>(h),
                       reinterpret_cast<const uint16_t*>(W_g), R, d.hidden, d.r, g);
  } else {
    hipLaunchKernelGGL(gate_f32, dim3((unsigned)R), dim3(256), 0, st, reinterpret_cast<const float*>(h),
                       reinterpret_cast<const float*>(W_g), R, d.hidden, d.r, g);
  }
  return hipGetLastError();
}

hipError_t launch_scores(const dflash_dims& d, const int32_t* x0, const int32_t* cand_idx,
                         const float* cand_logit, const void* E, const float* g, float* S,
                         hipStream_t st) {
  const dim3 grid((unsigned)(d.B * d.L));
  if (d.param_dtype == DFLASH_BF16)
    hipLaunchKernelGGL(scores_kernel<DFLASH_BF16>, grid, dim3(256), 0, st, x0, cand_idx, cand_logit, E, g,
                       d.L, d.V, d.K, d.r, S);
  else
    hipLaunchKernelGGL(scores_kernel<DFLASH_F32>, grid, dim3(256), 0, st, x0, cand_idx, cand_logit, E, g,
                       d.L, d.V, d.K, d.r, S);
  return hipGetLastError();
}

hipError_t launch_trace(const dflash_dims& d, const float* S, const int32_t* cand_idx, const float* T,
                        const uint64_t* seed, uint64_t cycle, int32_t* path_rank, int32_t* draft_tok,
                        float* q, hipStream_t st) {
  hipLaunchKernelGGL(trace_kernel, dim3((unsigned)d.B), dim3(64), 0, st, S, cand_idx, T, seed, cycle, d.L,
                     d.V, d.K, path_rank, draft_tok, q);
  return hipGetLastError();
}

}  // namespace dfk
