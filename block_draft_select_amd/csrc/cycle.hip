// dflash_cycle: the whole draft -> select -> verify cycle in three launches
// on the caller's stream.
//   1. stream_kernel: one grid streams every logit once.  Its first blocks
//      compute the gate's pre-activation tiles (S2; they depend only on h
//      and W_g), the next ones fold the drafter rows into sorted top lists
//      (S1), the last ones reduce the target rows to chunk statistics (S5).
//      Nothing in the launch waits on anything else in it.
//   2. cand_scores_kernel: one block per edge (b, t) merges the top lists of
//      rows t-1 and t, writes row t's candidates (and their target logits),
//      computes the edge's pair scores (S2, S3), and decides the edge's K
//      rows of the trace table: for every predecessor rank i, the walk's
//      next rank and q (S4).
//   3. trace_finalize_kernel: one block per stream combines the chunk
//      statistics (one wave per target row), walks the decided table (L
//      look-ups) or, for the max-sum cycle, finds the max-sum path over the
//      pair scores, then runs the accept tests and the residual/bonus draw
//      (S6).
#include "stats_blocks.hpp"
#include "topk_blocks.hpp"

namespace dfk {

namespace {

union StreamLds {
  struct {
    TkWave sw[4];
    uint64_t block_top[16];
    uint32_t bound;
  } tk;
  float red[kGateRed];
};

constexpr bool kGateFirst = true;

// gate block gi -> (row tile, column tile, group of hidden slices), group fastest
template <int PT>
__device__ __forceinline__ void gate_block(const void* __restrict__ h, const void* __restrict__ W, int R, int H, int r,
                                           float* __restrict__ gpart, int gate_cols, int n_ks, int gi, float* red) {
  if (PT == DFLASH_BF16) {
    const int n_grp = (n_ks + kGateGroup - 1) / kGateGroup;
    const int g = gi % n_grp, tile = gi / n_grp;
    gate_partial_bf16<1>(reinterpret_cast<const uint16_t*>(h), reinterpret_cast<const uint16_t*>(W), R, H, r, gpart,
                      tile / gate_cols, tile - (tile / gate_cols) * gate_cols, g * kGateGroup,
                      min(kGateGroup, n_ks - g * kGateGroup), red);
  } else {
    gate_row_f32(reinterpret_cast<const float*>(h), reinterpret_cast<const float*>(W), H, r, gpart, gi);
  }
}

template <int DT, int PT>
__global__ __launch_bounds__(256) void stream_kernel(const void* __restrict__ U, const void* __restrict__ Z, int R,
                                                     int V, int K, int L, int n_sub, int spb, int n_seg,
                                                     uint64_t* __restrict__ partial, int n_chunk, int n_grp,
                                                     const float* __restrict__ T, ChunkStat* __restrict__ stats,
                                                     const void* __restrict__ h, const void* __restrict__ W, int H,
                                                     int r, float* __restrict__ gpart, int gate_cols, int n_ks,
                                                     int n_gate) {
  __shared__ StreamLds sh;
  // gate blocks first (few and long: each accumulates up to kGateGroup
  // hidden slices of its tile), then top-K blocks in drafter-row order, then
  // statistics blocks in target-row order: the grid sweeps U and then Z
  // front to back (measured ~10% faster than interleaving the two kinds,
  // which splits the reads between two distant regions)
  int id = blockIdx.x;
  if (kGateFirst) {
    if (id < n_gate) {
      gate_block<PT>(h, W, R, H, r, gpart, gate_cols, n_ks, id, sh.red);
      return;
    }
    id -= n_gate;
  }
  const int n_topk = R * n_seg;
  if (id < n_topk) {
    const int row = id / n_seg, seg = id - row * n_seg;
    topk_block<DT>(U, V, K, n_sub, spb, row, seg, sh.tk.sw, sh.tk.block_top, &sh.tk.bound,
                   partial + ((size_t)row * n_seg + seg) * 16);
    return;
  }
  id -= n_topk;
  const int n_stat = (R / L) * (L + 1) * n_grp;
  if (!kGateFirst && id >= n_stat) {
    gate_block<PT>(h, W, R, H, r, gpart, gate_cols, n_ks, id - n_stat, sh.red);
    return;
  }
  const int rowid = id / n_grp;
  const int c = (id - rowid * n_grp) * 4 + (threadIdx.x >> 6);
  if (c >= n_chunk) return;
  const int lane = threadIdx.x & 63;
  const ChunkStat st = stats_chunk<DT>(Z, (size_t)rowid, V, c, T[rowid / (L + 1)], lane);
  if (lane == 0) stats[(size_t)rowid * n_chunk + c] = st;
}

struct CandLds {
  EdgeLds e;
  uint64_t keys[2 * kTopkCycleMerge];
  uint64_t prev[16], cur[16];
};

template <int DT, int PT, bool WIDE>
__global__ __launch_bounds__(256) void cand_scores_kernel(const uint64_t* __restrict__ partial, int n_seg,
                                                          const int32_t* __restrict__ x0, const void* __restrict__ E,
                                                          const float* __restrict__ gpart, int n_ks,
                                                          const void* __restrict__ Z,
                                                          int L, int V, int K, int r, const float* __restrict__ T,
                                                          const uint64_t* __restrict__ seed, uint64_t cycle,
                                                          int32_t* __restrict__ cand_idx,
                                                          float* __restrict__ cand_logit, float* __restrict__ zc,
                                                          float* __restrict__ S, int32_t* __restrict__ jstar,
                                                          float* __restrict__ qtab) {
  __shared__ CandLds cl;
  const int bt = blockIdx.x;
  const int b = bt / L, t = bt - b * L;
  const int tid = threadIdx.x;
  if (tid < 16) cl.prev[tid] = cl.cur[tid] = 0ull;
  // every independent load first: the two rows' lists (registers), the
  // gate slices, the trace inputs; the trace uniform is computed while
  // they are in flight
  constexpr int KPT = 2 * kTopkCycleMerge / 256;  // list keys per thread
  const int nk = n_seg * 16;
  const uint64_t* l0 = partial + (size_t)(t > 0 ? bt - 1 : bt) * nk;
  const uint64_t* l1 = partial + (size_t)bt * nk;
  // unconditional loads from clamped slots, masked afterwards (a masked
  // load would be a branch that waits for the loads issued before it)
  uint64_t kv[KPT];
#pragma unroll
  for (int q = 0; q < KPT; ++q) {
    const int i = tid + q * 256;
    kv[q] = i < nk ? l0[i] : l1[min(i - nk, nk - 1)];
  }
  const float Tb = T[b];
  const uint64_t sd = seed[b];
  const uint32_t u = stream_block(sd, cycle, (uint32_t)(t + 1), 0u).x;  // the trace uniform of position t
  edge_gate(cl.e, gpart, n_ks, (size_t)gridDim.x * r, bt, r);
  // masked only here, after the gate's loads are in flight too: edge 0 has
  // no predecessor row (its keys read as empty)
#pragma unroll
  for (int q = 0; q < KPT; ++q) {
    const int i = tid + q * 256;
    if (i < 2 * nk) cl.keys[i] = i < nk && t == 0 ? 0ull : kv[q];
  }
  __syncthreads();
  merge_two_staged<WIDE>(cl.keys, n_seg, K, cl.prev, cl.cur);
  // every thread reads the merged lists itself (no second hand-off):
  // the tokens of row lane % 16 (its MFMA operands) and the logit of
  // candidate tid % 16 (its score's column)
  // (clamped: a row with fewer than K admissible values leaves empty list
  // slots, whose key decodes to -1; the gathers below must stay in range)
  const int rl = tid & 15;
  const int pl = rl < K ? clamp_idx(t == 0 ? x0[b] : key_index(cl.prev[rl]), V) : (t == 0 ? clamp_idx(x0[b], V) : -1);
  const int cidx_l = rl < K ? clamp_idx(key_index(cl.cur[rl]), V) : -1;
  const float cl_j = rl < K ? key_value(cl.cur[rl]) : 0.f;
  if (tid < K) {
    const size_t o = (size_t)bt * K + tid;
    cand_idx[o] = cidx_l;
    cand_logit[o] = cl_j;
  }
  // the candidates' target logits are gathered while the embedding rows load
  float zv = 0.f;
  if (tid < K) {
    const size_t zi = ((size_t)b * (L + 1) + t) * V + cidx_l;
    zv = DT == DFLASH_BF16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(Z)[zi] << 16)
                           : reinterpret_cast<const float*>(Z)[zi];
  }
  const float sv = edge_contract_rows<PT>(cl.e, E, K, r, pl, cidx_l, cl_j, S + (size_t)bt * K * K);
  if (tid < K) zc[(size_t)bt * K + tid] = zv;
  // S4's table rows (t, i) of this edge: the walk's decision and q from
  // every predecessor rank i (thread tid holds S[tid / 16][tid % 16])
  const double invT = Tb > 0.0f ? 1.0 / (double)Tb : 0.0;
  const int i = tid >> 4, j = tid & 15;
  float qv;
  const int jd = trace_row_decide(sv, i < K && j < K, (tid & 63) >> 4, j, Tb, invT, u, K, qv);
  if (i < K && j < K) qtab[((size_t)bt * K + i) * K + j] = qv;
  if (i < K && j == 0) jstar[(size_t)bt * K + i] = jd;
}

// MODE kFinTable: walk the decided table (jstar, qtab); kFinMaxSum: qtab is
// the pair scores S and the block finds the max-sum path (jstar unused)
template <int DT, int MODE>
__global__ __launch_bounds__(kFinThreads) void trace_finalize_kernel(
    const void* __restrict__ Z, int L, int V, int K, int n_chunk, const float* __restrict__ T,
    const uint64_t* __restrict__ seed, uint64_t cycle, const int32_t* __restrict__ cand_idx,
    const float* __restrict__ zc, const int32_t* __restrict__ jstar, const float* __restrict__ qtab,
    int32_t* __restrict__ path_rank,
    int32_t* __restrict__ draft_tok, float* __restrict__ q, const ChunkStat* __restrict__ stats,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tok) {
  __shared__ FinLds f;
  finalize_stream<DT, MODE>(f, blockIdx.x, OneVocab{Z, V}, L, V, K, n_chunk, T, seed, cycle, cand_idx, zc, jstar, qtab,
                            path_rank, draft_tok, q, stats, accept_len, out_tok);
}

}  // namespace

hipError_t launch_cycle_stream(const dflash_dims& d, const WsLayout& w, const void* U, const void* Z, const void* h,
                               const void* W_g, const float* T, char* ws, hipStream_t st) {
  const int R = d.B * d.L;
  const int n_grp = (w.n_chunk + 3) / 4;
  const int gate_cols = (d.r + kGateCols - 1) / kGateCols;
  const int n_ks = gate_slices(d);
  const int n_gate = d.param_dtype == DFLASH_BF16 ? ((R + 15) / 16) * gate_cols * gate_groups(d) : R;
  const long long blocks = (long long)R * w.n_seg + (long long)d.B * (d.L + 1) * n_grp + n_gate;
  uint64_t* partial = reinterpret_cast<uint64_t*>(ws + w.topk_partial);
  ChunkStat* stats = reinterpret_cast<ChunkStat*>(ws + w.stats);
  float* gpart = reinterpret_cast<float*>(ws + w.gate);
#define DF_STREAM(DT, PT)                                                                                     \
  launch((stream_kernel<DT, PT>), dim3((unsigned)blocks), dim3(256), st, U, Z, R, d.V, d.K,   \
                     d.L, w.n_sub, w.spb, w.n_seg, partial, w.n_chunk, n_grp, T, stats, h, W_g, d.hidden, d.r, \
                     gpart, gate_cols, n_ks, n_gate)
  if (d.logit_dtype == DFLASH_BF16) {
    if (d.param_dtype == DFLASH_BF16) DF_STREAM(DFLASH_BF16, DFLASH_BF16); else DF_STREAM(DFLASH_BF16, DFLASH_F32);
  } else {
    if (d.param_dtype == DFLASH_BF16) DF_STREAM(DFLASH_F32, DFLASH_BF16); else DF_STREAM(DFLASH_F32, DFLASH_F32);
  }
#undef DF_STREAM
  return hipGetLastError();
}

hipError_t launch_cycle_scores(const dflash_dims& d, const WsLayout& w, const int32_t* x0, const void* E,
                               const void* Z, const float* T, const uint64_t* seed, uint64_t cycle, char* ws,
                               int32_t* cand_idx, float* cand_logit, float* S, hipStream_t st) {
  const dim3 grid((unsigned)(d.B * d.L));
  const uint64_t* partial = reinterpret_cast<const uint64_t*>(ws + w.topk_partial);
  const float* g = reinterpret_cast<const float*>(ws + w.gate);
  float* zc = reinterpret_cast<float*>(ws + w.zc);
  int32_t* jstar = reinterpret_cast<int32_t*>(ws + w.jstar);
  float* qtab = reinterpret_cast<float*>(ws + w.qtab);
#define DF_SCORES_W(DT, PT, WIDE)                                                                           \
  launch((cand_scores_kernel<DT, PT, WIDE>), grid, dim3(256), st, partial, w.n_seg, x0, E, g, gate_groups(d), Z, \
         d.L, d.V, d.K, d.r, T, seed, cycle, cand_idx, cand_logit, zc, S, jstar, qtab)
#define DF_SCORES(DT, PT)                                                \
  do {                                                                   \
    if (merge_wide(w.n_seg)) DF_SCORES_W(DT, PT, true);                  \
    else DF_SCORES_W(DT, PT, false);                                     \
  } while (0)
  if (d.logit_dtype == DFLASH_BF16) {
    if (d.param_dtype == DFLASH_BF16) DF_SCORES(DFLASH_BF16, DFLASH_BF16); else DF_SCORES(DFLASH_BF16, DFLASH_F32);
  } else {
    if (d.param_dtype == DFLASH_BF16) DF_SCORES(DFLASH_F32, DFLASH_BF16); else DF_SCORES(DFLASH_F32, DFLASH_F32);
  }
#undef DF_SCORES
#undef DF_SCORES_W
  return hipGetLastError();
}

hipError_t launch_cycle_finalize(const dflash_dims& d, const WsLayout& w, const void* Z, const int32_t* cand_idx,
                                 const float* T, const uint64_t* seed, uint64_t cycle, char* ws, const float* S_maxsum,
                                 int32_t* path_rank, int32_t* draft_tok, float* q, int32_t* accept_len,
                                 int32_t* out_tok, hipStream_t st) {
  const dim3 grid((unsigned)d.B);
  const float* zc = reinterpret_cast<const float*>(ws + w.zc);
  const int32_t* jstar = reinterpret_cast<const int32_t*>(ws + w.jstar);
  const float* qtab = S_maxsum ? S_maxsum : reinterpret_cast<const float*>(ws + w.qtab);
  const ChunkStat* stats = reinterpret_cast<const ChunkStat*>(ws + w.stats);
#define DF_FIN(DT, MODE)                                                                                        \
  launch(trace_finalize_kernel<DT, MODE>, grid, dim3(kFinThreads), st, Z, d.L, d.V, d.K, w.n_chunk, T, seed,   \
         cycle, cand_idx, zc, jstar, qtab, path_rank, draft_tok, q, stats, accept_len, out_tok)
  if (S_maxsum) {
    if (d.logit_dtype == DFLASH_BF16) DF_FIN(DFLASH_BF16, kFinMaxSum); else DF_FIN(DFLASH_F32, kFinMaxSum);
  } else {
    if (d.logit_dtype == DFLASH_BF16) DF_FIN(DFLASH_BF16, kFinTable); else DF_FIN(DFLASH_F32, kFinTable);
  }
#undef DF_FIN
  return hipGetLastError();
}

}  // namespace dfk
