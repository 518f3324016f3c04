// dflash_cycle: the whole draft -> select -> verify cycle on the caller's
// stream, in two launches when the streaming launch's top-K, gate and edge
// blocks all fit the GPU at once, else in three.
//   1. stream_kernel: one grid streams every logit once.  Its first blocks
//      compute the gate's pre-activation tiles (S2; they depend only on h
//      and W_g), the next ones fold the drafter rows into sorted top lists
//      (S1), the last ones reduce the target rows to chunk statistics (S5).
//      In the two-launch form the grid also holds one block per edge
//      (b, t), dispatched after the first statistics blocks: it reads the
//      lists of rows t-1 and t and the gate partials as they are handed
//      over inside the launch (tagged entries, read until they carry this
//      cycle's tag), then does the edge's work (below).
//   2. cand_scores_kernel (three-launch form only): the same edge work as a
//      launch of its own: one block per edge merges the top lists of rows
//      t-1 and t, writes row t's candidates (and their target logits),
//      computes the edge's pair scores (S2, S3), and decides the edge's K
//      rows of the trace table: for every predecessor rank i, the walk's
//      next rank and q (S4).
//   3. trace_finalize_kernel: one block per stream combines the chunk
//      statistics (one wave per target row), walks the decided table (L
//      look-ups) or, for the max-sum cycle, finds the max-sum path over the
//      pair scores, then runs the accept tests and the residual/bonus draw
//      (S6); in the two-launch form it also advances the hand-off epoch.
#include <algorithm>

#include "stats_blocks.hpp"
#include "topk_blocks.hpp"

namespace dfk {

namespace {

struct CandLds {
  EdgeLds e;
  uint64_t keys[2 * kTopkCycleMerge];
  uint64_t prev[16], cur[16];
};

union StreamLds {
  struct {
    TkWave sw[4];
    uint64_t block_top[16];
    uint32_t bound;
  } tk;
  float red[kGateRed];
  CandLds cl;  // edge blocks of the launch that also runs the edges
};

// polls of a hand-off before an edge block gives up (a bound, never
// reached when every producer runs: producers precede their consumers in
// the grid and wait on nothing, so they are dispatched and finish)
constexpr int kHandoffTries = 1 << 16;

// gate block gi -> (row tile, column tile, group of hidden slices), group fastest
template <int PT>
__device__ __forceinline__ void gate_block(const void* __restrict__ h, const void* __restrict__ W, int R, int H, int r,
                                           float* __restrict__ gpart, int gate_cols, int n_ks, int gi, float* red,
                                           uint64_t* __restrict__ gtag, uint32_t tag) {
  if (PT == DFLASH_BF16) {
    const int n_grp = (n_ks + kGateGroup - 1) / kGateGroup;
    const int g = gi % n_grp, tile = gi / n_grp;
    gate_partial_bf16<1>(reinterpret_cast<const uint16_t*>(h), reinterpret_cast<const uint16_t*>(W), R, H, r, gpart,
                         tile / gate_cols, tile - (tile / gate_cols) * gate_cols, g * kGateGroup,
                         min(kGateGroup, n_ks - g * kGateGroup), red, gtag, tag);
  } else {
    gate_row_f32(reinterpret_cast<const float*>(h), reinterpret_cast<const float*>(W), H, r, gpart, gi, gtag, tag);
  }
}

// what the edge blocks of the streaming launch need beyond its own
// arguments (EDGE only)
struct EdgeArgs {
  const uint32_t* epoch;  // this cycle's epoch (advanced by the finalize)
  uint64_t* tk_tag;       // top-K lists as hand-off pairs [R, n_seg, 16, 2]
  uint64_t* gate_tag;     // gate partials as hand-off words [groups, R, r]
  int n_pre;              // statistics blocks placed before the edge blocks
  const int32_t* x0;
  const void* E;
  const uint64_t* seed;
  uint64_t cycle;
  int32_t* cand_idx;
  float* cand_logit;
  float* zc;
  float* S;
  int32_t* jstar;
  float* qtab;
};

// The edge (b, t)'s work once its inputs are staged: the two rows' lists in
// cl.keys (edge 0's predecessor list zeroed), its gate in cl.e.g, a barrier
// passed.  Merges the lists, writes row t's candidates and their target
// logits, computes the pair scores and decides the edge's K rows of the
// trace table.
template <int DT, int PT, bool WIDE>
__device__ __forceinline__ void edge_finish(CandLds& cl, int b, int t, int bt, int n_seg, const int32_t* __restrict__ x0,
                                            const void* __restrict__ E, const void* __restrict__ Z, int L, int V, int K,
                                            int r, float Tb, uint32_t u, int32_t* __restrict__ cand_idx,
                                            float* __restrict__ cand_logit, float* __restrict__ zc,
                                            float* __restrict__ S, int32_t* __restrict__ jstar,
                                            float* __restrict__ qtab) {
  const int tid = threadIdx.x;
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

// The edge (b, t) inside the streaming launch: its inputs are the hand-off
// entries of the same launch's top-K blocks (rows bt - 1 and bt) and gate
// blocks, read until every entry carries this launch's tag.  The gate is
// summed over the slice groups in group order, as gate_value does, so the
// scores equal the three-launch cycle's.
template <int DT, int PT>
__device__ __forceinline__ void edge_block(CandLds& cl, int bt, const uint64_t* __restrict__ tk_tag, int n_seg,
                                           const uint64_t* __restrict__ gtag, int n_ks, int R, uint32_t tag,
                                           const int32_t* __restrict__ x0, const void* __restrict__ E,
                                           const void* __restrict__ Z, int L, int V, int K, int r,
                                           const float* __restrict__ T, const uint64_t* __restrict__ seed,
                                           uint64_t cycle, int32_t* __restrict__ cand_idx,
                                           float* __restrict__ cand_logit, float* __restrict__ zc,
                                           float* __restrict__ S, int32_t* __restrict__ jstar,
                                           float* __restrict__ qtab) {
  const int b = bt / L, t = bt - b * L;
  const int tid = threadIdx.x;
  if (tid < 16) cl.prev[tid] = cl.cur[tid] = 0ull;
  // the temperature and the trace uniform of position t in vector
  // registers (opaque inputs): the launch's scalar registers, whose count is
  // the largest over every block kind, decide how many waves fit a SIMD
  // (eight need at most 100; in scalar registers these took 104)
  float Tb = T[b];
  uint64_t sd = seed[b];
  uint32_t pos = (uint32_t)(t + 1);
  asm volatile("" : "+v"(Tb), "+v"(sd), "+v"(pos));
  const uint32_t u = stream_block(sd, cycle, pos, 0u).x;
  constexpr int KPT = 2 * kTopkCycleMerge / 256;  // list keys per thread
  const int nk = n_seg * 16;
  const uint64_t* l0 = tk_tag + (size_t)(t > 0 ? bt - 1 : bt) * nk * 2;
  const uint64_t* l1 = tk_tag + (size_t)bt * nk * 2;
  uint64_t kv[KPT];
  float z = 0.f;
  for (int tries = 0;; ++tries) {
    // every entry of this thread in flight at once (slots past the lists
    // re-read the last entry and are not checked)
    bool ok = true;
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      const int i = tid + q * 256;
      const uint64_t* pe = i < nk ? l0 + 2 * i : l1 + 2 * min(i - nk, nk - 1);
      const uint64_t kw = handoff_load(pe), tw = handoff_load(pe + 1);
      kv[q] = kw;
      if (i < 2 * nk) ok = ok && (uint32_t)tw == tag && (uint32_t)(tw >> 32) == handoff_check(kw, tag);
    }
    if (tid < r) {
      z = 0.f;
      for (int g = 0; g < n_ks; ++g) {
        const uint64_t e = handoff_load(gtag + ((size_t)g * R + bt) * r + tid);
        ok = ok && ((uint32_t)(e >> 32) ^ handoff_fmix((uint32_t)e)) == tag;
        z += __uint_as_float((uint32_t)e);
      }
    }
    if (ok || tries >= kHandoffTries) break;
    __builtin_amdgcn_s_sleep(2);
  }
  if (tid < r) cl.e.g[tid] = 1.0f / (1.0f + expf(-z));
#pragma unroll
  for (int q = 0; q < KPT; ++q) {
    const int i = tid + q * 256;
    if (i < 2 * nk) cl.keys[i] = i < nk && t == 0 ? 0ull : kv[q];
  }
  __syncthreads();
  edge_finish<DT, PT, false>(cl, b, t, bt, n_seg, x0, E, Z, L, V, K, r, Tb, u, cand_idx, cand_logit, zc, S, jstar,
                             qtab);
}

// EDGE: the grid also holds the B * L edge blocks (after the first n_pre
// statistics blocks), the top-K and gate blocks hand their results to them
// through tagged entries, and the launch does the work of the separate
// candidate/score launch; otherwise the top-K lists and gate partials go to
// plain workspace arrays for that launch.
template <int DT, int PT, bool EDGE>
__global__ __launch_bounds__(256) void stream_kernel(const void* __restrict__ U, const void* __restrict__ Z, int R,
                                                     int V, int K, int L, int n_sub, int spb, int n_seg,
                                                     uint64_t* __restrict__ partial, int n_chunk, int n_grp,
                                                     const float* __restrict__ T, ChunkStat* __restrict__ stats,
                                                     const void* __restrict__ h, const void* __restrict__ W, int H,
                                                     int r, float* __restrict__ gpart, int gate_cols, int n_ks,
                                                     int n_gate, EdgeArgs ea) {
  __shared__ StreamLds sh;
  // gate blocks first (few and long: each accumulates up to kGateGroup
  // hidden slices of its tile), then top-K blocks in drafter-row order, then
  // statistics blocks in target-row order: the grid sweeps U and then Z
  // front to back (measured ~10% faster than interleaving the two kinds,
  // which splits the reads between two distant regions)
  int id = blockIdx.x;
  const uint32_t tag = EDGE ? handoff_tag(*ea.epoch) : 0u;
  uint64_t* const gtag = EDGE ? ea.gate_tag : nullptr;
  if (id < n_gate) {
    gate_block<PT>(h, W, R, H, r, gpart, gate_cols, n_ks, id, sh.red, gtag, tag);
    return;
  }
  id -= n_gate;
  const int n_topk = R * n_seg;
  if (id < n_topk) {
    const int row = id / n_seg, seg = id - row * n_seg;
    topk_block<DT>(U, V, K, n_sub, spb, row, seg, sh.tk.sw, sh.tk.block_top, &sh.tk.bound,
                   partial + ((size_t)row * n_seg + seg) * 16,
                   EDGE ? ea.tk_tag + ((size_t)row * n_seg + seg) * 32 : nullptr, tag);
    return;
  }
  id -= n_topk;
  if (EDGE && id >= ea.n_pre) {
    if (id < ea.n_pre + R) {
      edge_block<DT, PT>(sh.cl, id - ea.n_pre, ea.tk_tag, n_seg, ea.gate_tag, (n_ks + kGateGroup - 1) / kGateGroup,
                         R, tag, ea.x0, ea.E, Z, L, V, K, r, T, ea.seed, ea.cycle, ea.cand_idx, ea.cand_logit, ea.zc,
                         ea.S, ea.jstar, ea.qtab);
      return;
    }
    id -= R;
  }
  const int rowid = id / n_grp;
  const int c = (id - rowid * n_grp) * 4 + (threadIdx.x >> 6);
  if (c >= n_chunk) return;
  const int lane = threadIdx.x & 63;
  const ChunkStat st = stats_chunk<DT>(Z, (size_t)rowid, V, c, T[rowid / (L + 1)], lane);
  if (lane == 0) stats[(size_t)rowid * n_chunk + c] = st;
}

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
  edge_finish<DT, PT, WIDE>(cl, b, t, bt, n_seg, x0, E, Z, L, V, K, r, Tb, u, cand_idx, cand_logit, zc, S, jstar,
                            qtab);
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
    int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tok, uint32_t* __restrict__ epoch) {
  __shared__ FinLds f;
  // the cycle's last launch advances the epoch of the streaming launch's
  // hand-off tags (the streaming launch has finished reading it)
  if (epoch && blockIdx.x == 0 && threadIdx.x == 0) *epoch += 1u;
  finalize_stream<DT, MODE>(f, blockIdx.x, OneVocab{Z, V}, L, V, K, n_chunk, T, seed, cycle, cand_idx, zc, jstar, qtab,
                            path_rank, draft_tok, q, stats, accept_len, out_tok);
}

}  // namespace

hipError_t launch_cycle_stream(const dflash_dims& d, const WsLayout& w, const void* U, const void* Z, const void* h,
                               const void* W_g, const float* T, char* ws, hipStream_t st, const CycleEdges* ce) {
  const int R = d.B * d.L;
  const int n_grp = (w.n_chunk + 3) / 4;
  const int gate_cols = (d.r + kGateCols - 1) / kGateCols;
  const int n_ks = gate_slices(d);
  const int n_gate = (int)stream_gate_blocks(d);
  const int n_sblk = d.B * (d.L + 1) * n_grp;
  const long long blocks = (long long)R * w.n_seg + n_sblk + n_gate + (ce ? R : 0);
  uint64_t* partial = reinterpret_cast<uint64_t*>(ws + w.topk_partial);
  ChunkStat* stats = reinterpret_cast<ChunkStat*>(ws + w.stats);
  float* gpart = reinterpret_cast<float*>(ws + w.gate);
  EdgeArgs ea{};
  if (ce) {
    ea.epoch = reinterpret_cast<const uint32_t*>(ws + w.epoch);
    ea.tk_tag = reinterpret_cast<uint64_t*>(ws + w.tk_tag);
    ea.gate_tag = reinterpret_cast<uint64_t*>(ws + w.gate_tag);
    ea.n_pre = std::min(ce->n_pre, n_sblk);
    ea.x0 = ce->x0;
    ea.E = ce->E;
    ea.seed = ce->seed;
    ea.cycle = ce->cycle;
    ea.cand_idx = ce->cand_idx;
    ea.cand_logit = ce->cand_logit;
    ea.zc = reinterpret_cast<float*>(ws + w.zc);
    ea.S = ce->S;
    ea.jstar = reinterpret_cast<int32_t*>(ws + w.jstar);
    ea.qtab = reinterpret_cast<float*>(ws + w.qtab);
  }
#define DF_STREAM(DT, PT)                                                                                       \
  do {                                                                                                          \
    if (ce)                                                                                                     \
      launch((stream_kernel<DT, PT, true>), dim3((unsigned)blocks), dim3(256), st, U, Z, R, d.V, d.K, d.L,      \
             w.n_sub, w.spb, w.n_seg, partial, w.n_chunk, n_grp, T, stats, h, W_g, d.hidden, d.r, gpart,        \
             gate_cols, n_ks, n_gate, ea);                                                                      \
    else                                                                                                        \
      launch((stream_kernel<DT, PT, false>), dim3((unsigned)blocks), dim3(256), st, U, Z, R, d.V, d.K, d.L,     \
             w.n_sub, w.spb, w.n_seg, partial, w.n_chunk, n_grp, T, stats, h, W_g, d.hidden, d.r, gpart,        \
             gate_cols, n_ks, n_gate, ea);                                                                      \
  } while (0)
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
                                 int32_t* out_tok, hipStream_t st, bool advance_epoch) {
  uint32_t* epoch = advance_epoch ? reinterpret_cast<uint32_t*>(ws + w.epoch) : nullptr;
  const dim3 grid((unsigned)d.B);
  const float* zc = reinterpret_cast<const float*>(ws + w.zc);
  const int32_t* jstar = reinterpret_cast<const int32_t*>(ws + w.jstar);
  const float* qtab = S_maxsum ? S_maxsum : reinterpret_cast<const float*>(ws + w.qtab);
  const ChunkStat* stats = reinterpret_cast<const ChunkStat*>(ws + w.stats);
#define DF_FIN(DT, MODE)                                                                                        \
  launch(trace_finalize_kernel<DT, MODE>, grid, dim3(kFinThreads), st, Z, d.L, d.V, d.K, w.n_chunk, T, seed,   \
         cycle, cand_idx, zc, jstar, qtab, path_rank, draft_tok, q, stats, accept_len, out_tok, epoch)
  if (S_maxsum) {
    if (d.logit_dtype == DFLASH_BF16) DF_FIN(DFLASH_BF16, kFinMaxSum); else DF_FIN(DFLASH_F32, kFinMaxSum);
  } else {
    if (d.logit_dtype == DFLASH_BF16) DF_FIN(DFLASH_BF16, kFinTable); else DF_FIN(DFLASH_F32, kFinTable);
  }
#undef DF_FIN
  return hipGetLastError();
}

}  // namespace dfk
