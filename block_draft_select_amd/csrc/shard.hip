// dflash_topk_merge: the exact top-K of a drafter row from the top-K lists
// of its vocabulary shards (P1 "DFlash 2: Block diffusion, wearing a
// drafter's coat", "Sixteen candidates per position": the K best tokens of
// each drafted position over the whole vocabulary).  When the vocabulary is
// split across devices, each shard keeps the K best of its own slice; the
// K best of the union of those lists are the K best of the row, ordered by
// value descending, then index ascending.
//
// One wave per row: the row's n_shards * K keys go to LDS as 64-bit ordered
// keys (canonical value above, inverted global index below, so a larger key
// is a better candidate and no two keys are equal), and each key's rank is
// the number of keys above it.
#include "device_util.hpp"
#include "internal.hpp"

namespace dfk {

namespace {

constexpr int kMergeWaves = 4;

__global__ __launch_bounds__(256) void topk_merge_kernel(int R, int K, int n_shards, ShardBegins sb,
                                                         const int32_t* __restrict__ idx_parts,
                                                         const float* __restrict__ val_parts,
                                                         int32_t* __restrict__ cand_idx,
                                                         float* __restrict__ cand_logit) {
  __shared__ uint64_t keys[kMergeWaves][DFLASH_MAX_SHARDS * DFLASH_K_MAX];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * kMergeWaves + wave;
  const bool live = row < R;  // every wave reaches the barrier
  const int n = n_shards * K;
  if (live) {
    for (int i = lane; i < n; i += kWave) {
      const int s = i / K, k = i - s * K;
      const size_t e = ((size_t)s * R + row) * K + k;
      const uint32_t gi = (uint32_t)(sb.begin[s] + idx_parts[e]);
      const uint32_t vk = ord32_canon(__float_as_uint(val_parts[e]));
      keys[wave][i] = ((uint64_t)vk << 32) | (uint32_t)~gi;
    }
  }
  __syncthreads();
  if (!live) return;
  for (int i = lane; i < n; i += kWave) {
    const uint64_t ki = keys[wave][i];
    int above = 0;
    for (int j = 0; j < n; ++j) above += keys[wave][j] > ki;
    if (above < K) {
      cand_idx[(size_t)row * K + above] = (int32_t)~(uint32_t)ki;
      cand_logit[(size_t)row * K + above] = __uint_as_float(unord32((uint32_t)(ki >> 32)));
    }
  }
}

}  // namespace

hipError_t launch_topk_merge(const dflash_dims& d, int n_shards, const ShardBegins& sb, const int32_t* idx_parts,
                             const float* val_parts, int32_t* cand_idx, float* cand_logit, hipStream_t st) {
  const int R = d.B * d.L;
  launch(topk_merge_kernel, dim3((unsigned)((R + kMergeWaves - 1) / kMergeWaves)), dim3(256), st, R, d.K, n_shards,
         sb, idx_parts, val_parts, cand_idx, cand_logit);
  return hipGetLastError();
}

}  // namespace dfk
