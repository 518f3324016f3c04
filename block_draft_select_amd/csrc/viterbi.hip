// dflash_trace_viterbi: the global max-sum path through the candidate
// lattice, a variant of the greedy trace (P3 "DFlash 2: Keep Drafting
// Parallel", section "What Comes Next", paragraph "A Lightweight Path
// Selector": the pair scores of adjacent candidates and a walk from the
// verified token; the same section leaves better searches open).
//
// The value of a path is the sum of its L edge scores, edge 1 starting at
// the verified token (row 0 of its equal rows).  Dynamic programming in
// fp64 over the fp32 scores: best_1(j) = S[0, 0, j], best_t(j) = max_i
// best_{t-1}(i) + S[t-1, i, j] with back_t(j) the smallest i attaining it;
// the path ends at the smallest j attaining max best_L and is read back
// through the back pointers.  Smallest indices at every tie give the
// smallest optimal path in reverse lexicographic order.  The path is
// deterministic, so q is one-hot at each chosen rank.
//
// One wave per stream: the stream's scores go to LDS with coalesced loads,
// the four 16-lane groups each hold best_t(j) of every column j and its
// 4-bit back pointers in two registers, a DP step splits the predecessors
// four ways across the groups (lane shuffles, no barrier), and the backtrack
// is L lane reads of uniform indices.
#include "device_util.hpp"
#include "internal.hpp"

namespace dfk {

namespace {

__global__ __launch_bounds__(64) void viterbi_kernel(const float* __restrict__ S, const int32_t* __restrict__ cand_idx,
                                                     int L, int V, int K, int32_t* __restrict__ path_rank,
                                                     int32_t* __restrict__ draft_tok, float* __restrict__ q) {
  __shared__ float Ss[DFLASH_L_MAX * DFLASH_K_MAX * DFLASH_K_MAX];
  const int b = blockIdx.x, lane = threadIdx.x;
  const size_t s0 = (size_t)b * L * K * K;
  const int n = L * K * K;
  // stage the stream's scores in LDS: all 64 loads of a lane in flight at
  // once, indices clamped rather than masked (a masked load or store becomes
  // a branch that waits for the loads before it; slots past the scores get
  // copies of the last one and are never read)
  float v[DFLASH_L_MAX * DFLASH_K_MAX * DFLASH_K_MAX / 64];
#pragma unroll
  for (int u = 0; u < DFLASH_L_MAX * DFLASH_K_MAX * DFLASH_K_MAX / 64; ++u) v[u] = S[s0 + min(u * 64 + lane, n - 1)];
#pragma unroll
  for (int u = 0; u < DFLASH_L_MAX * DFLASH_K_MAX * DFLASH_K_MAX / 64; ++u) Ss[u * 64 + lane] = v[u];
  __syncthreads();

  // the step loops stay rolled (one wave issues every instruction of the
  // body itself, so a fully unrolled body measured slower).  Lane
  // g * 16 + j holds best_t(j) of column j = lane % 16 < K (four replicas);
  // its back pointers are 4-bit fields, steps 0..7 in bk0 and 8..15 in bk1
  const bool live = (lane & 15) < K;
  const int jr = min(lane & 15, K - 1);  // lanes past K read a valid column and discard it
  double best = live ? (double)Ss[jr] : -INFINITY;
  uint32_t bk0 = 0, bk1 = 0;
#pragma unroll 1
  for (int t = 1; t < L; ++t) {
    // the step over all 64 lanes (predecessor values by lane shuffles)
    double m;
    int arg;
    maxplus_step(best, &Ss[t * K * K], K, lane, m, arg);
    if (live) {
      best = m;
      if (t < 8) bk0 |= (uint32_t)arg << (4 * t);
      else bk1 |= (uint32_t)arg << (4 * (t - 8));
    }
  }

  // the path's last rank: the smallest j attaining max best_L
  double m = best;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off));
  const unsigned long long hit = __ballot(live && best == m);
  int jc = hit ? __ffsll((long long)hit) - 1 : 0;  // no hit only for non-finite scores
  int mine = lane == L - 1 ? jc : 0;
#pragma unroll 1
  for (int t = L - 1; t >= 1; --t) {
    const uint32_t w = __builtin_amdgcn_readlane(t < 8 ? bk0 : bk1, jc);
    jc = (int)((w >> (4 * (t & 7))) & 15u);
    if (lane == t - 1) mine = jc;
  }
  if (lane < L) {
    const size_t bt = (size_t)b * L + lane;
    path_rank[bt] = mine;
    draft_tok[bt] = clamp_idx(cand_idx[bt * K + mine], V);
  }
  for (int p = lane; p < L * K; p += 64) {
    const int t = p / K, k = p - t * K;
    q[(size_t)b * L * K + p] = k == __shfl(mine, t) ? 1.f : 0.f;
  }
}

}  // namespace

hipError_t launch_trace_viterbi(const dflash_dims& d, const float* S, const int32_t* cand_idx, int32_t* path_rank,
                                int32_t* draft_tok, float* q, hipStream_t st) {
  launch(viterbi_kernel, dim3((unsigned)d.B), dim3(64), st, S, cand_idx, d.L, d.V, d.K, path_rank, draft_tok, q);
  return hipGetLastError();
}

}  // namespace dfk
