// dflash_topk: S1 as a standalone entry point (P1 "DFlash 2: Block
// diffusion, wearing a drafter's coat", section "Sixteen candidates per
// position").  topk_partial_kernel writes the sorted top list of every run
// of sub-segments (topk_blocks.hpp); topk_output_kernel merges the lists of
// each row and writes the candidates.
#include "topk_blocks.hpp"

namespace dfk {

namespace {

// grid: x = segment of the row (runs of `spb` sub-segments), y = row
template <int DT>
__global__ __launch_bounds__(kTopkThreads) void topk_partial_kernel(const void* __restrict__ U, int V, int K,
                                                                    int n_sub, int spb,
                                                                    uint64_t* __restrict__ partial) {
  __shared__ TkWave sw[4];
  __shared__ uint64_t block_top[16];
  __shared__ uint32_t bound;
  const int row = blockIdx.y, seg = blockIdx.x;
  topk_block<DT>(U, V, K, n_sub, spb, row, seg, sw, block_top, &bound,
                 partial + ((size_t)row * gridDim.x + seg) * 16);
}

// one block per row: merge the row's sorted lists and write its candidates
__global__ __launch_bounds__(256) void topk_output_kernel(const uint64_t* __restrict__ partial, int K, int n_seg,
                                                          int32_t* __restrict__ cand_idx,
                                                          float* __restrict__ cand_logit) {
  __shared__ uint64_t keys[kTopkMergeMax];
  __shared__ uint64_t out[16];
  const int row = blockIdx.x, tid = threadIdx.x;
  merge_row(partial + (size_t)row * n_seg * 16, n_seg, K, keys, out);
  if (tid < K) {
    cand_idx[(size_t)row * K + tid] = key_index(out[tid]);  // -1: an empty slot (no admissible value)
    cand_logit[(size_t)row * K + tid] = key_value(out[tid]);
  }
}

}  // namespace

hipError_t launch_topk_lists(const dflash_dims& d, const WsLayout& w, const void* U, char* ws, hipStream_t st) {
  const int rows = d.B * d.L;
  uint64_t* partial = reinterpret_cast<uint64_t*>(ws + w.topk_partial);
  const dim3 grid((unsigned)w.n_seg, (unsigned)rows);
  if (d.logit_dtype == DFLASH_BF16)
    launch(topk_partial_kernel<DFLASH_BF16>, grid, dim3(kTopkThreads), st, U, d.V, d.K, w.n_sub, w.spb, partial);
  else
    launch(topk_partial_kernel<DFLASH_F32>, grid, dim3(kTopkThreads), st, U, d.V, d.K, w.n_sub, w.spb, partial);
  return hipGetLastError();
}

hipError_t launch_topk(const dflash_dims& d, const WsLayout& w, const void* U, int32_t* cand_idx,
                       float* cand_logit, char* ws, hipStream_t st) {
  hipError_t e = launch_topk_lists(d, w, U, ws, st);
  if (e != hipSuccess) return e;
  launch(topk_output_kernel, dim3((unsigned)(d.B * d.L)), dim3(256), st,
         reinterpret_cast<const uint64_t*>(ws + w.topk_partial), d.K, w.n_seg, cand_idx, cand_logit);
  return hipGetLastError();
}

}  // namespace dfk
