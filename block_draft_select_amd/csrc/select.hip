// dflash_pair_scores and dflash_trace: S2..S4 as standalone entry points
// (P3 "DFlash 2: Keep Drafting Parallel", section "What Comes Next",
// paragraph "A Lightweight Path Selector"; P1 "DFlash 2: Block diffusion,
// wearing a drafter's coat", sub-section "A path selector").  The device
// code lives in select_blocks.hpp, shared with the fused cycle.
#include "select_blocks.hpp"

namespace dfk {

namespace {

// grid (row tiles, column tiles, groups of hidden slices)
// one wave per quarter of a tile (grid z = group * 4 + quarter): a tile's
// 192 KB of operands spread over four CUs instead of one, the whole group's
// loads of the quarter issued before its first MFMA; the consumer sums the
// quarters as the cycle's four-wave tiles do, so the scores are identical
__global__ __launch_bounds__(64) void gate_mfma_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W,
                                                       int R, int H, int r, float* __restrict__ qpart) {
  const int n_ks = (H + kGateSlice - 1) / kGateSlice, ks0 = (blockIdx.z / kGateWaves) * kGateGroup;
  gate_quarter_bf16<kGateGroup>(h, W, R, H, r, qpart, blockIdx.x, blockIdx.y, ks0, min(kGateGroup, n_ks - ks0),
                                blockIdx.z % kGateWaves);
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
  if (PT == DFLASH_BF16) {
    if (tid < r) e.g[tid] = gate_value_quarters(gpart, n_ks, (size_t)gridDim.x * r, bt, r, tid);
  } else {
    edge_gate(e, gpart, n_ks, (size_t)gridDim.x * r, bt, r);
  }
  __syncthreads();
  edge_contract<PT>(e, E, K, r, S + (size_t)bt * K * K);
}

// One 1024-thread block per stream.  Every row (t, i) of the trace table
// (position t reached from rank i) is decided up front, one 16-lane group
// per row, by the same arithmetic the fused cycle uses (trace_row_decide),
// so no step waits for the previous one; wave 0 then walks the table from
// rank 0 with lane reads of the decisions held in registers, and the block
// writes each position's rank, token and q (the row of its predecessor's
// rank).
constexpr int kTraceThreads = 1024;
constexpr int kTraceRows = kTraceThreads / 16;  // table rows decided per pass

__global__ __launch_bounds__(kTraceThreads) void trace_kernel(const float* __restrict__ S,
                                                              const int32_t* __restrict__ cand_idx,
                                                              const float* __restrict__ T,
                                                              const uint64_t* __restrict__ seed, uint64_t cycle, int L,
                                                              int V, int K, int32_t* __restrict__ path_rank,
                                                              int32_t* __restrict__ draft_tok, float* __restrict__ q) {
  constexpr int NP = DFLASH_L_MAX * DFLASH_K_MAX / kTraceRows;  // passes at most
  __shared__ float qtab[DFLASH_L_MAX * DFLASH_K_MAX * DFLASH_K_MAX];
  __shared__ int jst[DFLASH_L_MAX * DFLASH_K_MAX];
  __shared__ int rank[DFLASH_L_MAX];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int lk = L * K;
  const float Tb = T[b];
  const uint64_t sd = seed[b];
  const double invT = Tb > 0.0f ? 1.0 / (double)Tb : 0.0;
  const int g = tid >> 4, j = tid & 15;
  // every load first (clamped indices, masked afterwards)
  float sv[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = p * kTraceRows + g;
    sv[p] = S[(size_t)b * lk * K + (size_t)min(row, lk - 1) * K + min(j, K - 1)];
  }
  const int ci = clamp_idx(cand_idx[(size_t)b * lk + min(tid, lk - 1)], V);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = p * kTraceRows + g;
    if (p * kTraceRows >= lk) break;  // uniform
    const bool live = row < lk && j < K;
    const int t = min(row, lk - 1) / K;
    const uint32_t u = stream_block(sd, cycle, (uint32_t)(t + 1), 0u).x;
    float qv;
    const int jd = trace_row_decide(sv[p], live, (tid & 63) >> 4, j, Tb, invT, u, K, qv);
    if (live) qtab[row * K + j] = qv;
    if (row < lk && j == 0) jst[row] = jd;
  }
  __syncthreads();
  if (tid < kWave) {
    // the decisions in registers (lane l holds rows l, l + 64, ...): each
    // step of the walk is a lane read, not an LDS round trip
    constexpr int NJ = DFLASH_L_MAX * DFLASH_K_MAX / kWave;
    int jv[NJ];
#pragma unroll
    for (int c = 0; c < NJ; ++c) jv[c] = lane + c * kWave < lk ? jst[lane + c * kWave] : 0;
    int prev = 0, mine = 0;
    for (int t = 0; t < L; ++t) {
      const int row = t * K + prev;
      int next = 0;
#pragma unroll
      for (int c = 0; c < NJ; ++c) {
        const int v = __builtin_amdgcn_readlane(jv[c], row & 63);
        next = (row >> 6) == c ? v : next;
      }
      if (lane == t) mine = next;
      prev = next;
    }
    if (lane < L) rank[lane] = mine;
  }
  __syncthreads();
  if (tid < L) {
    path_rank[(size_t)b * L + tid] = rank[tid];
  }
  if (tid < lk) {
    const int t = tid / K, k = tid - t * K;
    const int pr = t > 0 ? rank[t - 1] : 0;
    q[(size_t)b * lk + tid] = qtab[(t * K + pr) * K + k];
    if (k == rank[t]) draft_tok[(size_t)b * L + t] = ci;
  }
}

}  // namespace

hipError_t launch_gate(const dflash_dims& d, const void* h, const void* W_g, float* gpart, hipStream_t st) {
  const int R = d.B * d.L;
  if (d.param_dtype == DFLASH_BF16) {
    const dim3 grid((unsigned)((R + 15) / 16), (unsigned)((d.r + kGateCols - 1) / kGateCols),
                    (unsigned)(gate_groups(d) * kGateWaves));
    launch(gate_mfma_kernel, grid, dim3(64), st, reinterpret_cast<const uint16_t*>(h),
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
  launch(trace_kernel, dim3((unsigned)d.B), dim3(kTraceThreads), st, S, cand_idx, T, seed, cycle, d.L,
                     d.V, d.K, path_rank, draft_tok, q);
  return hipGetLastError();
}

}  // namespace dfk
