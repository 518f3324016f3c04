// Host-side declarations shared by the ABI layer and the kernel files:
// geometry constants, the workspace layout and the kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dflash.h"

namespace dfk {

// top-K streaming geometry: a wave owns 8 16-byte loads per lane; a block of
// 4 waves owns one segment of a drafter row
constexpr int kTopkThreads = 256;
constexpr int kTopkLoads = 8;
constexpr int kTopkCap = 256;          // candidate buffer per wave
constexpr int kTopkMergeMax = 2048;    // keys the last block of a row merges in LDS

inline int topk_wave_elems(int logit_dtype) { return 64 * kTopkLoads * (logit_dtype == DFLASH_BF16 ? 8 : 4); }
inline int topk_block_elems(int logit_dtype) { return 4 * topk_wave_elems(logit_dtype); }
// blocks per drafter row stay <= 32 so that the partial lists of two rows
// fit the cycle's candidate/score block (kTopkCycleMerge keys of LDS)
constexpr int kTopkCycleMerge = 512;
constexpr int kTopkMaxSeg = kTopkCycleMerge / 16;

constexpr int kChunk = DFLASH_CHUNK;   // target-row chunk (one wave)

// 256-thread blocks of the streaming launch resident at once: eight per CU
// on the 256 CUs of an MI355X
constexpr int kResidentBlocks = 8 * 256;
// statistics blocks dispatched before the edge blocks, in percent of all
// statistics blocks (measured at concurrent-32: 41.3 to 41.9 us per cycle at
// 30 to 40, 42.2 at 0 and at 60, 42.8 at 80; the edges then start while
// the last top-K blocks finish)
constexpr int kEdgePrePct = 40;

// gate: the hidden dimension is cut into slices of kGateSlice; a gate block
// accumulates kGateGroup consecutive slices of one tile on the matrix
// cores, and consumers sum the groups' partial pre-activations W_g h in
// group order before the sigmoid
constexpr int kGateSlice = 256;
constexpr int kGateGroup = 8;
inline int gate_slices(const dflash_dims& d) {
  return d.param_dtype == DFLASH_BF16 ? (d.hidden + kGateSlice - 1) / kGateSlice : 1;
}
inline int gate_groups(const dflash_dims& d) { return (gate_slices(d) + kGateGroup - 1) / kGateGroup; }
// gate blocks of the streaming launch: bf16 tiles of 16 rows x 32 columns
// per slice group, or one fp32 row per block
constexpr int kGateTileRows = 16, kGateTileCols = 32;
inline long long stream_gate_blocks(const dflash_dims& d) {
  const long long R = (long long)d.B * d.L;
  return d.param_dtype == DFLASH_BF16
             ? ((R + kGateTileRows - 1) / kGateTileRows) * ((d.r + kGateTileCols - 1) / kGateTileCols) * gate_groups(d)
             : R;
}

struct ChunkStat {
  float m;      // chunk maximum logit
  float s;      // sum over the chunk of exp((z - m) / T)  (sampling rows)
  int32_t arg;  // first index of the maximum (greedy rows)
  int32_t pad;
};

struct WsLayout {
  int n_sub;    // top-K sub-segments (one wave's registers) per drafter row
  int spb;      // sub-segments per top-K block
  int n_seg;    // top-K blocks per drafter row (a merge kernel runs if > 1)
  int n_chunk;  // target chunks per row
  size_t topk_partial, gate, cand_idx, cand_logit, zc, S, path_rank, draft_tok, q, stats;
  size_t jstar, qtab;  // the fused cycle's trace table: decision and q of every row (t, i)
  // The fused cycle runs its edges inside the streaming launch when its
  // top-K, gate and edge blocks fit the GPU's resident blocks at once
  // (kResidentBlocks); it then hands over through: the cycle epoch (one
  // word, advanced by every cycle's last launch), the top-K lists as
  // (key, check | tag) pairs and the gate partials as (tag | value) words.
  bool edges;
  size_t epoch, tk_tag, gate_tag;
  size_t cycle_total;  // bytes the fused cycles use (the regions above)
  // the split path's gate partials, one per quarter of each tile (bf16
  // parameters) or one per row (fp32), after everything the cycles use
  size_t gate_q;
  size_t total;
};

WsLayout ws_layout(const dflash_dims& d);

// Events the next kernel launch on this thread records at the kernel's own
// start and end (hipExtLaunchKernel: the dispatch's timestamps, not the
// stream's), set by the per-kernel timer and consumed by that launch.
extern thread_local hipEvent_t g_launch_start, g_launch_stop;

template <typename F, typename... Args>
inline void launch(F kernel, dim3 grid, dim3 block, hipStream_t st, Args... args) {
  hipEvent_t a = g_launch_start, b = g_launch_stop;
  g_launch_start = g_launch_stop = nullptr;
  hipExtLaunchKernelGGL(kernel, grid, block, 0, st, a, b, 0, args...);
}

// ---- launchers (each enqueues on `st`; returns the launch status) ----

hipError_t launch_topk(const dflash_dims& d, const WsLayout& w, const void* U, int32_t* cand_idx,
                       float* cand_logit, char* ws, hipStream_t st);
hipError_t launch_gate(const dflash_dims& d, const void* h, const void* W_g, float* gpart, hipStream_t st);
hipError_t launch_scores(const dflash_dims& d, const int32_t* x0, const int32_t* cand_idx,
                         const float* cand_logit, const void* E, const float* gpart, float* S,
                         hipStream_t st);
// first global token index of each vocabulary shard
struct ShardBegins {
  int32_t begin[DFLASH_MAX_SHARDS];
};
// a vocabulary split for the verify: shard s covers tokens
// [begin[s], begin[s + 1]) (begin[n] = V), its residual-draw chunks are
// cbase[s] .. cbase[s + 1] - 1 (the grid restarts at each shard), and its
// target rows Z[s] are [B, L + 1, begin[s + 1] - begin[s]]
struct ShardMap {
  int32_t n;
  int32_t begin[DFLASH_MAX_SHARDS + 1];
  int32_t cbase[DFLASH_MAX_SHARDS + 1];
  const void* Z[DFLASH_MAX_SHARDS];
};
hipError_t launch_topk_merge(const dflash_dims& d, int n_shards, const ShardBegins& sb, const int32_t* idx_parts,
                             const float* val_parts, int32_t* cand_idx, float* cand_logit, hipStream_t st);
hipError_t launch_shard_stats(const dflash_dims& d, const ShardMap& m, int shard, const void* Zs, const float* T,
                              ChunkStat* stats, hipStream_t st);
hipError_t launch_finalize_shards(const dflash_dims& d, const ShardMap& m, const int32_t* cand_idx,
                                  const int32_t* path_rank, const float* q, const float* T, const uint64_t* seed,
                                  uint64_t cycle, const ChunkStat* stats, int32_t* accept_len, int32_t* out_tok,
                                  hipStream_t st);
hipError_t launch_trace_viterbi(const dflash_dims& d, const float* S, const int32_t* cand_idx, int32_t* path_rank,
                                int32_t* draft_tok, float* q, hipStream_t st);
hipError_t launch_trace(const dflash_dims& d, const float* S, const int32_t* cand_idx, const float* T,
                        const uint64_t* seed, uint64_t cycle, int32_t* path_rank, int32_t* draft_tok,
                        float* q, hipStream_t st);
hipError_t launch_stats(const dflash_dims& d, const WsLayout& w, const void* Z, const float* T, ChunkStat* stats,
                        hipStream_t st);
hipError_t launch_finalize(const dflash_dims& d, const WsLayout& w, const void* Z,
                           const int32_t* cand_idx, const int32_t* path_rank, const float* q,
                           const float* T, const uint64_t* seed, uint64_t cycle,
                           const ChunkStat* stats, int32_t* accept_len, int32_t* out_tok,
                           hipStream_t st);
// dflash_cycle: (1) top-K lists + chunk statistics + gate slices,
// (2) candidates + pair scores, (3) trace + verify
hipError_t launch_topk_lists(const dflash_dims& d, const WsLayout& w, const void* U, char* ws, hipStream_t st);
// the edge work folded into the streaming launch (its candidates, scores
// and trace-table rows; zc, jstar and qtab go to the workspace)
struct CycleEdges {
  int n_pre;  // statistics blocks dispatched before the edge blocks
  const int32_t* x0;
  const void* E;
  const uint64_t* seed;
  uint64_t cycle;
  int32_t* cand_idx;
  float* cand_logit;
  float* S;
};
hipError_t launch_cycle_stream(const dflash_dims& d, const WsLayout& w, const void* U, const void* Z, const void* h,
                               const void* W_g, const float* T, char* ws, hipStream_t st,
                               const CycleEdges* edges = nullptr);
hipError_t launch_cycle_scores(const dflash_dims& d, const WsLayout& w, const int32_t* x0, const void* E,
                               const void* Z, const float* T, const uint64_t* seed, uint64_t cycle, char* ws,
                               int32_t* cand_idx, float* cand_logit, float* S, hipStream_t st);
hipError_t launch_cycle_finalize(const dflash_dims& d, const WsLayout& w, const void* Z, const int32_t* cand_idx,
                                 const float* T, const uint64_t* seed, uint64_t cycle, char* ws, const float* S_maxsum,
                                 int32_t* path_rank, int32_t* draft_tok, float* q, int32_t* accept_len,
                                 int32_t* out_tok, hipStream_t st, bool advance_epoch = false);
hipError_t launch_conv2tap(const dflash_dims& d, const void* x, const void* x0, const void* Wt, float* y,
                           hipStream_t st);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
// device address and size of the library's static scratch on the current
// device (looked up once per device)
hipError_t static_scratch(void** out, size_t* bytes);
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st);
hipError_t launch_copy_probe(void* dst, const void* src, size_t bytes, hipStream_t st);

}  // namespace dfk
