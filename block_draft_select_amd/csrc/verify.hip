// dflash_verify: S5 + S6 as a standalone entry point (P1 "DFlash 2: Block
// diffusion, wearing a drafter's coat", section "Lossless, with conditions
// I did not used to state"; P2 "A 2B Drafter Made a 27B Model 3.4x Faster.
// Same Exact Output.", section "Caveats before you rebuild your serving
// stack").  The device code lives in stats_blocks.hpp, shared with the
// fused cycle.
#include "stats_blocks.hpp"

namespace dfk {

namespace {

// grid: x = group of 4 chunks (one per wave), y = target row b * (L + 1) + t
template <int DT>
__global__ __launch_bounds__(256) void stats_kernel(const void* __restrict__ Z, int L, int V, int n_chunk,
                                                    const float* __restrict__ T, ChunkStat* __restrict__ stats) {
  const int rowid = blockIdx.y;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (c >= n_chunk) return;
  const int lane = threadIdx.x & 63;
  const ChunkStat st = stats_chunk<DT>(Z, (size_t)rowid, V, c, T[rowid / (L + 1)], lane);
  if (lane == 0) stats[(size_t)rowid * n_chunk + c] = st;
}

template <int DT>
__global__ __launch_bounds__(kFinThreads) void finalize_kernel(
    const void* __restrict__ Z, int L, int V, int K, int n_chunk, const float* __restrict__ T,
    const uint64_t* __restrict__ seed, uint64_t cycle, const int32_t* __restrict__ cand_idx,
    const int32_t* __restrict__ path_rank, const float* __restrict__ q, const ChunkStat* __restrict__ stats,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tok) {
  __shared__ FinLds f;
  finalize_stream<DT, kFinVerify>(f, blockIdx.x, OneVocab{Z, V}, L, V, K, n_chunk, T, seed, cycle, cand_idx, nullptr, nullptr,
                             nullptr, const_cast<int32_t*>(path_rank), nullptr, const_cast<float*>(q), stats,
                             accept_len, out_tok);
}

}  // namespace

hipError_t launch_stats(const dflash_dims& d, const WsLayout& w, const void* Z, const float* T, ChunkStat* stats,
                        hipStream_t st) {
  const dim3 grid((unsigned)((w.n_chunk + 3) / 4), (unsigned)(d.B * (d.L + 1)));
  if (d.logit_dtype == DFLASH_BF16)
    launch(stats_kernel<DFLASH_BF16>, grid, dim3(256), st, Z, d.L, d.V, w.n_chunk, T, stats);
  else
    launch(stats_kernel<DFLASH_F32>, grid, dim3(256), st, Z, d.L, d.V, w.n_chunk, T, stats);
  return hipGetLastError();
}

hipError_t launch_finalize(const dflash_dims& d, const WsLayout& w, const void* Z,
                           const int32_t* cand_idx, const int32_t* path_rank, const float* q,
                           const float* T, const uint64_t* seed, uint64_t cycle,
                           const ChunkStat* stats, int32_t* accept_len, int32_t* out_tok,
                           hipStream_t st) {
  const dim3 grid((unsigned)d.B);
  if (d.logit_dtype == DFLASH_BF16)
    launch(finalize_kernel<DFLASH_BF16>, grid, dim3(kFinThreads), st, Z, d.L, d.V, d.K, w.n_chunk, T,
                       seed, cycle, cand_idx, path_rank, q, stats, accept_len, out_tok);
  else
    launch(finalize_kernel<DFLASH_F32>, grid, dim3(kFinThreads), st, Z, d.L, d.V, d.K, w.n_chunk, T,
                       seed, cycle, cand_idx, path_rank, q, stats, accept_len, out_tok);
  return hipGetLastError();
}

}  // namespace dfk
