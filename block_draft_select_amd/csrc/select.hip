// dflash_pair_scores and dflash_trace: S2..S4 as standalone entry points
// (P3 "DFlash 2: Keep Drafting Parallel", section "What Comes Next",
// paragraph "A Lightweight Path Selector"; P1 "DFlash 2: Block diffusion,
// wearing a drafter's coat", sub-section "A path selector").  The device
// code lives in select_blocks.hpp, shared with the fused cycle.
#include "select_blocks.hpp"

namespace dfk {

namespace {

// grid (row tiles, column tiles, groups of hidden slices)
__global__ __launch_bounds__(256) void gate_mfma_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W,
                                                        int R, int H, int r, float* __restrict__ part) {
  __shared__ float red[kGateRed];
  const int n_ks = (H + kGateSlice - 1) / kGateSlice, ks0 = blockIdx.z * kGateGroup;
  gate_partial_bf16(h, W, R, H, r, part, blockIdx.x, blockIdx.y, ks0, min(kGateGroup, n_ks - ks0), red);
}

__global__ __launch_bounds__(256) void gate_f32_kernel(const float* __restrict__ h, const float* __restrict__ W,
                                                       int H, int r, float* __restrict__ part) {
  gate_row_f32(h, W, H, r, part, blockIdx.x);
}

// one block per edge (b, t), candidates read from the caller's arrays
template <int PT>
__global__ __launch_bounds__(256) void scores_kernel(const int32_t* __restrict__ x0,
                                                     const int32_t* __restrict__ cand_idx,
                                                     const float* __restrict__ cand_logit,
                                                     const void* __restrict__ E, const float* __restrict__ gpart,
                                                     int n_ks, int L, int V, int K, int r, float* __restrict__ S) {
  __shared__ EdgeLds e;
  const int bt = blockIdx.x;
  const int b = bt / L, t = bt - b * L;
  const int tid = threadIdx.x;
  if (tid < 16) {
    int p = -1, c = -1;
    float cl = 0.f;
    if (tid < K) {
      p = t == 0 ? clamp_idx(x0[b], V) : clamp_idx(cand_idx[((size_t)b * L + t - 1) * K + tid], V);
      c = clamp_idx(cand_idx[((size_t)b * L + t) * K + tid], V);
      cl = cand_logit[((size_t)b * L + t) * K + tid];
    } else if (t == 0) {
      p = clamp_idx(x0[b], V);  // edge 0: every predecessor row is x0
    }
    e.pidx[tid] = p;
    e.cidx[tid] = c;
    e.cl[tid] = cl;
  }
  edge_gate(e, gpart, n_ks, (size_t)gridDim.x * r, bt, r);
  __syncthreads();
  edge_contract<PT>(e, E, K, r, S + (size_t)bt * K * K);
}

// one wave per stream
__global__ __launch_bounds__(64) void trace_kernel(const float* __restrict__ S, const int32_t* __restrict__ cand_idx,
                                                   const float* __restrict__ T, const uint64_t* __restrict__ seed,
                                                   uint64_t cycle, int L, int V, int K,
                                                   int32_t* __restrict__ path_rank, int32_t* __restrict__ draft_tok,
                                                   float* __restrict__ q) {
  constexpr int NMAX = DFLASH_L_MAX * DFLASH_K_MAX * DFLASH_K_MAX;
  __shared__ TraceLds tl;
  __shared__ float Ss[NMAX];
  __shared__ int ci[DFLASH_L_MAX * DFLASH_K_MAX];
  const int b = blockIdx.x, lane = threadIdx.x;
  const float Tb = T[b];
  const size_t s0 = (size_t)b * L * K * K;
  const int n = L * K * K;
  // every load issued before the first store; indices past the stream's
  // arrays are clamped (a masked load would become a branch, and each
  // branch would wait for the loads before it)
  float sv[NMAX / 64];
#pragma unroll
  for (int s = 0; s < NMAX / 64; ++s) sv[s] = S[s0 + min(lane + s * 64, n - 1)];
  int cv[DFLASH_L_MAX * DFLASH_K_MAX / 64];
#pragma unroll
  for (int s = 0; s < DFLASH_L_MAX * DFLASH_K_MAX / 64; ++s)
    cv[s] = clamp_idx(cand_idx[(size_t)b * L * K + min(lane + s * 64, L * K - 1)], V);
#pragma unroll
  for (int s = 0; s < NMAX / 64; ++s)
    if (lane + s * 64 < n) Ss[lane + s * 64] = sv[s];
#pragma unroll
  for (int s = 0; s < DFLASH_L_MAX * DFLASH_K_MAX / 64; ++s)
    if (lane + s * 64 < L * K) ci[lane + s * 64] = cv[s];
  trace_setup(tl, Tb, seed[b], cycle, L, lane);
  __syncthreads();
  const double invT = Tb > 0.0f ? 1.0 / (double)Tb : 0.0;
  int prev = 0;
  for (int t = 0; t < L; ++t) {
    const size_t e0 = ((size_t)b * L + t) * K;
    prev = trace_step_dpp(tl, &Ss[(t * K + prev) * K], Tb, invT, t, K, lane, &ci[t * K], q + e0,
                          path_rank + (size_t)b * L + t, draft_tok + (size_t)b * L + t, nullptr);
  }
}

}  // namespace

hipError_t launch_gate(const dflash_dims& d, const void* h, const void* W_g, float* gpart, hipStream_t st) {
  const int R = d.B * d.L;
  if (d.param_dtype == DFLASH_BF16) {
    const dim3 grid((unsigned)((R + 15) / 16), (unsigned)((d.r + kGateCols - 1) / kGateCols), (unsigned)gate_groups(d));
    launch(gate_mfma_kernel, grid, dim3(256), st, reinterpret_cast<const uint16_t*>(h),
                       reinterpret_cast<const uint16_t*>(W_g), R, d.hidden, d.r, gpart);
  } else {
    launch(gate_f32_kernel, dim3((unsigned)R), dim3(256), st, reinterpret_cast<const float*>(h),
                       reinterpret_cast<const float*>(W_g), d.hidden, d.r, gpart);
  }
  return hipGetLastError();
}

hipError_t launch_scores(const dflash_dims& d, const int32_t* x0, const int32_t* cand_idx,
                         const float* cand_logit, const void* E, const float* gpart, float* S,
                         hipStream_t st) {
  const dim3 grid((unsigned)(d.B * d.L));
  const int n_ks = gate_groups(d);
  if (d.param_dtype == DFLASH_BF16)
    launch(scores_kernel<DFLASH_BF16>, grid, dim3(256), st, x0, cand_idx, cand_logit, E, gpart,
                       n_ks, d.L, d.V, d.K, d.r, S);
  else
    launch(scores_kernel<DFLASH_F32>, grid, dim3(256), st, x0, cand_idx, cand_logit, E, gpart,
                       n_ks, d.L, d.V, d.K, d.r, S);
  return hipGetLastError();
}

hipError_t launch_trace(const dflash_dims& d, const float* S, const int32_t* cand_idx, const float* T,
                        const uint64_t* seed, uint64_t cycle, int32_t* path_rank, int32_t* draft_tok,
                        float* q, hipStream_t st) {
  launch(trace_kernel, dim3((unsigned)d.B), dim3(64), st, S, cand_idx, T, seed, cycle, d.L,
                     d.V, d.K, path_rank, draft_tok, q);
  return hipGetLastError();
}

}  // namespace dfk
