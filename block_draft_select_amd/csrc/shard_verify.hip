// dflash_shard_stats and dflash_verify_shards: S5 + S6 when the target's
// vocabulary is split into shards (P1 "DFlash 2: Block diffusion, wearing a
// drafter's coat", "The architecture", "Lossless, with conditions I did not
// used to state"; the split itself follows a tensor-parallel LM head of the
// serving runtimes of P2 "A 2B Drafter Made a 27B Model 3.4x Faster. Same
// Exact Output.", "Running it").
//
// shard_stats_kernel: the chunk statistics of one shard's target rows
//   [B, L + 1, width], on a chunk grid that starts at the shard's first
//   token, written into that shard's columns of the statistics of the whole
//   vocabulary ([B, L + 1, total chunks]); greedy rows record global argmax
//   indices.  The device code is the unsplit statistics pass.
// finalize_shards_kernel: the unsplit finalize over that chunk grid; the
//   candidates' target logits and the drawn chunk are read from the shard
//   that holds them.
#include "stats_blocks.hpp"

namespace dfk {

namespace {

// grid: x = group of 4 chunks of the shard (one per wave), y = target row
template <int DT>
__global__ __launch_bounds__(256) void shard_stats_kernel(const void* __restrict__ Zs, int L, int width, int n_chunk_s,
                                                          int cbase, int n_chunk, int begin,
                                                          const float* __restrict__ T, ChunkStat* __restrict__ stats) {
  const int rowid = blockIdx.y;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (c >= n_chunk_s) return;
  const int lane = threadIdx.x & 63;
  ChunkStat st = stats_chunk<DT>(Zs, (size_t)rowid, width, c, T[rowid / (L + 1)], lane);
  if (st.arg >= 0) st.arg += begin;
  if (lane == 0) stats[(size_t)rowid * n_chunk + cbase + c] = st;
}

template <int DT>
__global__ __launch_bounds__(kFinThreads) void finalize_shards_kernel(
    const ShardMap map, int L, int V, int K, int n_chunk, const float* __restrict__ T,
    const uint64_t* __restrict__ seed, uint64_t cycle, const int32_t* __restrict__ cand_idx,
    const int32_t* __restrict__ path_rank, const float* __restrict__ q, const ChunkStat* __restrict__ stats,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tok) {
  __shared__ FinLds f;
  finalize_stream<DT, kFinVerify>(f, blockIdx.x, SplitVocab{map}, L, V, K, n_chunk, T, seed, cycle, cand_idx,
                                  nullptr, nullptr, nullptr, const_cast<int32_t*>(path_rank), nullptr,
                                  const_cast<float*>(q), stats, accept_len, out_tok);
}

}  // namespace

hipError_t launch_shard_stats(const dflash_dims& d, const ShardMap& m, int shard, const void* Zs, const float* T,
                              ChunkStat* stats, hipStream_t st) {
  const int width = m.begin[shard + 1] - m.begin[shard];
  const int n_chunk_s = m.cbase[shard + 1] - m.cbase[shard];
  const dim3 grid((unsigned)((n_chunk_s + 3) / 4), (unsigned)(d.B * (d.L + 1)));
  if (d.logit_dtype == DFLASH_BF16)
    launch(shard_stats_kernel<DFLASH_BF16>, grid, dim3(256), st, Zs, d.L, width, n_chunk_s, m.cbase[shard],
           m.cbase[m.n], m.begin[shard], T, stats);
  else
    launch(shard_stats_kernel<DFLASH_F32>, grid, dim3(256), st, Zs, d.L, width, n_chunk_s, m.cbase[shard],
           m.cbase[m.n], m.begin[shard], T, stats);
  return hipGetLastError();
}

hipError_t launch_finalize_shards(const dflash_dims& d, const ShardMap& m, const int32_t* cand_idx,
                                  const int32_t* path_rank, const float* q, const float* T, const uint64_t* seed,
                                  uint64_t cycle, const ChunkStat* stats, int32_t* accept_len, int32_t* out_tok,
                                  hipStream_t st) {
  const dim3 grid((unsigned)d.B);
  if (d.logit_dtype == DFLASH_BF16)
    launch(finalize_shards_kernel<DFLASH_BF16>, grid, dim3(kFinThreads), st, m, d.L, d.V, d.K, m.cbase[m.n], T,
           seed, cycle, cand_idx, path_rank, q, stats, accept_len, out_tok);
  else
    launch(finalize_shards_kernel<DFLASH_F32>, grid, dim3(kFinThreads), st, m, d.L, d.V, d.K, m.cbase[m.n], T,
           seed, cycle, cand_idx, path_rank, q, stats, accept_len, out_tok);
  return hipGetLastError();
}

}  // namespace dfk
