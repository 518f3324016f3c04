// Device building blocks of S5 + S6 (verify against the target rows; P1
// "DFlash 2: Block diffusion, wearing a drafter's coat", section "Lossless,
// with conditions I did not used to state": a draft survives with chance
// min(1, p/q), a rejected one is replaced by a draw from the residual; P2 "A 2B Drafter
// Made a 27B Model 3.4x Faster. Same Exact Output.", section "Caveats before
// you rebuild your serving stack": greedy output equals the target's).
//
// stats_chunk: one wave reduces one chunk of DFLASH_CHUNK tokens of a target
//   row held in registers (64 values per lane, 16-byte loads):
//     greedy rows:   the chunk maximum and its first index;
//     sampling rows: the chunk maximum m and S = sum over all tokens of
//                    exp((z - m) / T), in fp32 with one v_exp_f32 per value
//                    (of the exactly formed difference z - m).
//   The statistics do not depend on the candidates, so they stream in the
//   same launch as the top-K; the candidates' own mass is taken out of their
//   chunk in fp64 by the finalize.  The bf16 maximum first tries a packed
//   signed 16-bit max of the raw patterns, exact whenever the maximum is
//   non-negative.
// finalize_stream: one block per stream combines the chunk statistics in
//   fp64, runs the accept tests, and draws the residual/bonus token in two
//   inverse-CDF levels (item = chunk or candidate, then the token inside a
//   drawn chunk, which is re-read).  Optionally the block first walks the
//   trace over a table whose rows were decided beforehand.
#pragma once

#include "device_util.hpp"
#include "internal.hpp"
#include "select_blocks.hpp"

namespace dfk {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint32_t smax_i16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, a),
                                                                __builtin_bit_cast(s16x2, b)));
}

// One chunk of a target row in a wave's registers: 64 raw values per lane
// (bf16 pairs or fp32 words), lane l holding 16-byte unit j * 64 + l.
template <int DT>
struct ChunkRegs {
  uint32_t x[DT == DFLASH_BF16 ? 32 : 64];
};

// Load chunk c of target row `rowid` (one wave; nontemporal 16-byte loads).
// 16-byte units past the row end hold -inf (weight 0, never the maximum).
template <int DT>
__device__ __forceinline__ void stats_load(const void* __restrict__ Z, size_t rowid, int V, int c, int lane,
                                           ChunkRegs<DT>& r) {
  const int lo = c * kChunk, hi = min(lo + kChunk, V);
  if (DT == DFLASH_BF16) {
    const uint16_t* row = reinterpret_cast<const uint16_t*>(Z) + rowid * V;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int base = lo + (j * kWave + lane) * 8;
      uint4 v = make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
      if (base < hi) v = load_stream16(row + base);
      r.x[4 * j + 0] = v.x;
      r.x[4 * j + 1] = v.y;
      r.x[4 * j + 2] = v.z;
      r.x[4 * j + 3] = v.w;
    }
  } else {
    const uint32_t* row = reinterpret_cast<const uint32_t*>(Z) + rowid * V;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int base = lo + (j * kWave + lane) * 4;
      uint4 v = make_uint4(0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u);
      if (base < hi) v = load_stream16(row + base);
      r.x[4 * j + 0] = v.x;
      r.x[4 * j + 1] = v.y;
      r.x[4 * j + 2] = v.z;
      r.x[4 * j + 3] = v.w;
    }
  }
}

// Statistics of the chunk held in r whose first token is lo (one wave).
template <int DT>
__device__ __forceinline__ ChunkStat stats_reduce(const ChunkRegs<DT>& r, int lo, float Tb, int lane) {
  const bool greedy = !(Tb > 0.0f);
  const uint32_t* x = r.x;
  ChunkStat st;
  st.pad = 0;
  if (DT == DFLASH_BF16) {
    if (greedy) {
      // composite key (canonical value, inverted chunk offset): the maximum
      // is the largest value at the smallest index
      uint32_t best = 0;
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        const uint32_t k2 = ord16x2(x[q]);
        const int off = ((q >> 2) * kWave + lane) * 8 + (q & 3) * 2;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t k = h ? (k2 >> 16) : (k2 & 0xFFFFu);
          k = (k == 0x7FFFu) ? 0x8000u : k;
          best = max(best, (k << 16) | (uint32_t)(0xFFFF - (off + h)));
        }
      }
      best = wave_max_u32(best);
      st.m = __uint_as_float(bf16_of_k16(best >> 16) << 16);
      st.s = 0.0f;
      st.arg = lo + (int)(0xFFFFu - (best & 0xFFFFu));
    } else {
      uint32_t mx = x[0];
#pragma unroll
      for (int q = 1; q < 32; ++q) mx = smax_i16x2(mx, x[q]);
      int top = max((int)(int16_t)(mx & 0xFFFFu), (int)(int16_t)(mx >> 16));
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) top = max(top, __shfl_xor(top, o));
      float m;
      if (top >= 0) {
        m = __uint_as_float((uint32_t)top << 16);  // non-negative pattern: the true maximum
      } else {
        uint32_t km = ord16x2(x[0]);
#pragma unroll
        for (int q = 1; q < 32; ++q) km = max_u16x2(km, ord16x2(x[q]));
        const uint32_t m16 = wave_max_u32(max(km & 0xFFFFu, km >> 16));
        m = __uint_as_float(bf16_of_k16(m16) << 16);
      }
      // exponent (z - m) * log2(e) / T: the difference of two bf16 values
      // is exact in fp32, so the terms near the maximum carry no error from
      // m (m * k2 rounded once would shift every term of the chunk by a
      // factor of relative size |m| / T * 2^-24, and overflow at tiny T)
      const float k2 = kLog2e / Tb;
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
      for (int q = 0; q < 32; q += 2) {
        s0 += __builtin_amdgcn_exp2f((bf16_lo(x[q]) - m) * k2);
        s1 += __builtin_amdgcn_exp2f((bf16_hi(x[q]) - m) * k2);
        s2 += __builtin_amdgcn_exp2f((bf16_lo(x[q + 1]) - m) * k2);
        s3 += __builtin_amdgcn_exp2f((bf16_hi(x[q + 1]) - m) * k2);
      }
      st.m = m;
      st.s = wave_sum_f32((s0 + s1) + (s2 + s3));
      st.arg = -1;
    }
  } else {
    if (greedy) {
      uint64_t best = 0;
#pragma unroll
      for (int q = 0; q < 64; ++q) {
        const int off = ((q >> 2) * kWave + lane) * 4 + (q & 3);
        const uint64_t key = ((uint64_t)ord32_canon(x[q]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)off);
        best = key > best ? key : best;
      }
      best = wave_max_u64(best);
      st.m = __uint_as_float(unord32((uint32_t)(best >> 32)));
      st.s = 0.0f;
      st.arg = lo + (int)(0xFFFFFFFFu - (uint32_t)best);
    } else {
      uint32_t mx = ord32(x[0]);
#pragma unroll
      for (int q = 1; q < 64; ++q) mx = max(mx, ord32(x[q]));
      const float m = __uint_as_float(unord32(wave_max_u32(mx)));
      const float k2 = kLog2e / Tb;
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
      for (int q = 0; q < 64; q += 4) {
        s0 += __builtin_amdgcn_exp2f((__uint_as_float(x[q + 0]) - m) * k2);
        s1 += __builtin_amdgcn_exp2f((__uint_as_float(x[q + 1]) - m) * k2);
        s2 += __builtin_amdgcn_exp2f((__uint_as_float(x[q + 2]) - m) * k2);
        s3 += __builtin_amdgcn_exp2f((__uint_as_float(x[q + 3]) - m) * k2);
      }
      st.m = m;
      st.s = wave_sum_f32((s0 + s1) + (s2 + s3));
      st.arg = -1;
    }
  }
  return st;
}

// Statistics of chunk c of target row `rowid` (one wave): load, then reduce.
template <int DT>
__device__ __forceinline__ ChunkStat stats_chunk(const void* __restrict__ Z, size_t rowid, int V, int c, float Tb,
                                                 int lane) {
  ChunkRegs<DT> r;
  stats_load<DT>(Z, rowid, V, c, lane, r);
  return stats_reduce<DT>(r, c * kChunk, Tb, lane);
}

template <int DT>
__device__ __forceinline__ double logit_at(const void* Z, size_t i) {
  if (DT == DFLASH_BF16) return (double)__uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(Z)[i] << 16);
  return (double)reinterpret_cast<const float*>(Z)[i];
}

// the TPT logits of tokens e0 .. e0 + TPT - 1 of the row starting at element
// zr, widened to fp64 (e0 counted from the row's first token).  Units of TPT
// tokens lie wholly inside or outside [0, hi) (row widths and chunk ends are
// multiples of 8 for bf16 and of 4 for fp32); units past hi read as -inf.
template <int DT, int TPT>
__device__ __forceinline__ void load_tokens(const void* __restrict__ Z, size_t zr, int e0, int hi, double (&zv)[TPT]) {
  static_assert(TPT == 4, "4 tokens per thread");
  const int V = hi;
  if (DT == DFLASH_BF16) {
    uint2 v = make_uint2(0xFF80FF80u, 0xFF80FF80u);
    if (e0 < V) v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(Z) + zr + e0);
    zv[0] = (double)bf16_lo(v.x);
    zv[1] = (double)bf16_hi(v.x);
    zv[2] = (double)bf16_lo(v.y);
    zv[3] = (double)bf16_hi(v.y);
  } else {
    uint4 v = make_uint4(0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u);
    if (e0 < V) v = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(Z) + zr + e0);
    zv[0] = (double)__uint_as_float(v.x);
    zv[1] = (double)__uint_as_float(v.y);
    zv[2] = (double)__uint_as_float(v.z);
    zv[3] = (double)__uint_as_float(v.w);
  }
}

// Where the residual draw's first-level chunks lie and where a token's
// target logit is stored.  OneVocab: one contiguous vocabulary [0, V), rows
// of V logits, chunks of kChunk tokens from token 0.  SplitVocab: a
// vocabulary split into shards, each with its own [B, L + 1, width] rows;
// the chunk grid restarts at every shard's first token.  Both give, for a
// chunk id, its token range [lo, hi) and where its logits live.
struct ChunkLoc {
  int lo, hi;        // global token range of the chunk
  const void* Zs;    // the rows holding it (the whole vocabulary or a shard)
  int base, width;   // first global token and width of those rows
};

struct OneVocab {
  const void* Z;
  int V;
  __device__ __forceinline__ int chunk_of(int tok) const { return tok / kChunk; }
  __device__ __forceinline__ ChunkLoc chunk(int c) const {
    const int lo = c * kChunk;
    return ChunkLoc{lo, min(lo + kChunk, V), Z, 0, V};
  }
  template <int DT>
  __device__ __forceinline__ double logit(size_t row, int tok) const {
    return logit_at<DT>(Z, row * (size_t)V + tok);
  }
};

struct SplitVocab {
  const ShardMap& m;
  __device__ __forceinline__ int shard_of(int tok) const {
    int lo = 0, hi = m.n - 1;  // the last shard whose first token is <= tok
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (m.begin[mid] <= tok) lo = mid; else hi = mid - 1;
    }
    return lo;
  }
  __device__ __forceinline__ int chunk_of(int tok) const {
    const int s = shard_of(tok);
    return m.cbase[s] + (tok - m.begin[s]) / kChunk;
  }
  __device__ __forceinline__ ChunkLoc chunk(int c) const {
    int lo = 0, hi = m.n - 1;  // the last shard whose first chunk is <= c
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (m.cbase[mid] <= c) lo = mid; else hi = mid - 1;
    }
    const int s = lo, b0 = m.begin[s], b1 = m.begin[s + 1];
    const int t0 = b0 + (c - m.cbase[s]) * kChunk;
    return ChunkLoc{t0, min(t0 + kChunk, b1), m.Z[s], b0, b1 - b0};
  }
  template <int DT>
  __device__ __forceinline__ double logit(size_t row, int tok) const {
    const int s = shard_of(tok), b0 = m.begin[s];
    return logit_at<DT>(m.Z[s], row * (size_t)(m.begin[s + 1] - b0) + (tok - b0));
  }
};

constexpr int kFinThreads = 1024;  // 16 waves: the parallel phases split 16 ways
constexpr int kFinWaves = kFinThreads / kWave;
constexpr int kFinTpt = kChunk / kFinThreads;  // tokens per thread in the in-chunk draw
constexpr int kTermCache = 2048;  // chunk terms of all rows kept in LDS when they fit

struct FinLds {
  float2 ms[kTermCache];                            // (m, s) of every chunk of every row
  double term[kTermCache];                          // s * exp((m - M_t) / T)
  float S[DFLASH_L_MAX * DFLASH_K_MAX * DFLASH_K_MAX];  // q of every trace-table row (t, i)
  int jstar[DFLASH_L_MAX * DFLASH_K_MAX];           // the walk's decision for every row
  float rowM[DFLASH_L_MAX + 1];
  double rowAll[DFLASH_L_MAX + 1];                  // sum over all tokens of exp((z - M) / T)
  int rowArg[DFLASH_L_MAX + 1];
  double pc[DFLASH_L_MAX][DFLASH_K_MAX];            // exp((z_cand - M) / T)
  double zc[DFLASH_L_MAX][DFLASH_K_MAX];            // candidate target logits
  float qs[DFLASH_L_MAX][DFLASH_K_MAX];
  int cand[DFLASH_L_MAX][DFLASH_K_MAX];
  int cchunk[DFLASH_L_MAX][DFLASH_K_MAX];           // the residual-draw chunk of each candidate
  int rank[DFLASH_L_MAX];
  uint4 rnd0[DFLASH_L_MAX];                         // (cycle, t + 1, 0) blocks
  uint4 rnd1[DFLASH_L_MAX + 1];                     // (cycle, t + 1, 1) blocks
  int pick_row[DFLASH_L_MAX + 1];                   // first-level draw of every row
  double wave_tot[kFinWaves];
  int s_n;
};

// Combine the statistics of row t (one wave): maximum, first argmax chunk,
// and for sampling rows every chunk term and the candidate weights.
template <int DT>
__device__ __forceinline__ void combine_row(FinLds& f, const ChunkStat* __restrict__ st_row, int t, int L, int K,
                                            int n_chunk, bool cached, bool greedy, double invT, int lane) {
  float M = -INFINITY;
  for (int c = lane; c < n_chunk; c += kWave) M = fmaxf(M, cached ? f.ms[t * n_chunk + c].x : st_row[c].m);
  M = wave_max_dpp_f32(M);
  if (greedy) {
    int first = 0x7FFFFFFF;
    for (int base = 0; base < n_chunk && first == 0x7FFFFFFF; base += kWave) {
      const int c = base + lane;
      const float m = c < n_chunk ? (cached ? f.ms[t * n_chunk + c].x : st_row[c].m) : -INFINITY;
      const int fl = first_lane(c < n_chunk && m == M);
      if (fl < 64) first = base + fl;
    }
    // no chunk maximum equals M only when every one is NaN (fmaxf skips
    // them): the row then has no defined argmax, and chunk 0's stays in range
    if (first == 0x7FFFFFFF) first = 0;
    if (lane == 0) {
      f.rowM[t] = M;
      f.rowArg[t] = st_row[first].arg;
    }
    return;
  }
  double s = 0.0;
  for (int c = lane; c < n_chunk; c += kWave) {
    const float2 v = cached ? f.ms[t * n_chunk + c] : make_float2(st_row[c].m, st_row[c].s);
    const double tm = (double)v.y * exp_nonpos(((double)v.x - (double)M) * invT);
    if (cached) f.term[t * n_chunk + c] = tm;
    s += tm;
  }
  s = wave_sum_dpp_f64(s);
  if (t < L && lane < K) f.pc[t][lane] = exp_nonpos((f.zc[t][lane] - (double)M) * invT);
  if (lane == 0) {
    f.rowM[t] = M;
    f.rowAll[t] = s;
  }
}

// First level of the residual/bonus draw of row t (one wave, registers
// only): the index of the drawn item among [chunk 0 .. n_chunk - 1 (the
// chunk's mass without the row's candidates), candidate 0 .. nk - 1
// (max(0, p - q))], nk = K for t < L and 0 for the bonus row.  If the
// residual has no mass the candidates keep mass p instead.  Items past the
// first 64 are recomputed in a second pass rather than stored.
__device__ __forceinline__ int pick_item(const FinLds& f, const ChunkStat* __restrict__ st, int t, int L, int K,
                                         int n_chunk, bool cached, double invT, const float* qrow, int lane) {
  const int nk = t < L ? K : 0;
  const double inv = 1.0 / f.rowAll[t];
  const uint4 w1 = f.rnd1[t];
  // the chunk of each of the row's candidates, in registers
  int cchunk[DFLASH_K_MAX];
#pragma unroll
  for (int k = 0; k < DFLASH_K_MAX; ++k) cchunk[k] = k < nk ? f.cchunk[t][k] : -1;
  const int n_item = n_chunk + nk;
  auto item = [&](int i, bool resid) -> double {
    if (i < n_chunk) {
      double tm;
      if (cached) {
        tm = f.term[t * n_chunk + i];
      } else {
        const ChunkStat cs = st[i];
        tm = (double)cs.s * exp_nonpos(((double)cs.m - (double)f.rowM[t]) * invT);
      }
      // the weights of the candidates inside chunk i, added in candidate
      // order (integer matching first: a chunk rarely holds more than one)
      uint32_t m = 0;
#pragma unroll
      for (int k = 0; k < DFLASH_K_MAX; ++k) m |= (cchunk[k] == i ? 1u : 0u) << k;
      double cm = 0.0;
      while (m) {
        cm += f.pc[t][__builtin_ctz(m)];
        m &= m - 1u;
      }
      return fmax(0.0, (tm - cm) * inv);
    }
    if (i < n_item) {
      const double p = f.pc[t][i - n_chunk] * inv;
      return resid ? fmax(0.0, p - (double)qrow[i - n_chunk]) : p;
    }
    return 0.0;
  };
  bool resid = true;
  double total = 0.0, cum0 = 0.0;
  for (int pass = 0; pass < 2; ++pass) {
    double carry = 0.0;
    for (int base = 0; base < n_item; base += kWave) {
      const double v = wave_scan_f64(item(base + lane, resid)) + carry;
      if (base == 0) cum0 = v;
      carry = readlane_f64(v, 63);
    }
    total = carry;
    if (total > 0.0 || nk == 0 || !resid) break;
    resid = false;  // the residual has no mass: draw from p itself
  }
  const double target = u01_f64(w1.x, w1.y) * total;
  const int fl0 = first_lane(lane < n_item && cum0 > target);
  if (fl0 < 64) return fl0;
  double carry = readlane_f64(cum0, 63);
  for (int base = kWave; base < n_item; base += kWave) {
    const double v = wave_scan_f64(item(base + lane, resid)) + carry;
    const int fl = first_lane(base + lane < n_item && v > target);
    if (fl < 64) return base + fl;
    carry = readlane_f64(v, 63);
  }
  return n_item - 1;
}

// What the finalize block does besides the verify: nothing (path_rank and q
// are inputs), the walk over the decided trace table, or the max-sum trace
// over the pair scores
enum { kFinVerify = 0, kFinTable = 1, kFinMaxSum = 2 };

// q of position t (t < L, K values in LDS): with the table walk, the table
// row of its predecessor's rank (rank 0 at t = 0); else the q in f.qs (the
// caller's, or one-hot at the max-sum path)
template <bool TABLE>
__device__ __forceinline__ const float* q_row_of(const FinLds& f, int t, int K) {
  if (TABLE) return &f.S[(t * K + (t > 0 ? f.rank[t - 1] : 0)) * K];
  return f.qs[t];
}

// One block per stream.  MODE kFinTable: the block also walks the trace
// over the decided trace table (jstar: decision of every row (t, i); qtab:
// the q of every row, [B, L, K, K]) and writes path_rank / draft_tok / q.
// kFinMaxSum: qtab holds the pair scores S [B, L, K, K]; wave 0 finds the
// max-sum path (the dynamic programme of dflash_trace_viterbi, the same
// arithmetic in the same order) and writes path_rank / draft_tok and a
// one-hot q.  kFinVerify: path_rank and q are inputs.  In the first two
// modes zc_pre holds the candidates' target logits [B, L, K] (fp32-exact
// values); otherwise it is not read and they are gathered here.
template <int DT, int MODE, class G>
__device__ void finalize_stream(FinLds& f, int b, const G& geo, int L, int V, int K, int n_chunk,
                                const float* __restrict__ T, const uint64_t* __restrict__ seed, uint64_t cycle,
                                const int32_t* __restrict__ cand_idx, const float* __restrict__ zc_pre,
                                const int32_t* __restrict__ jstar, const float* __restrict__ qtab,
                                int32_t* __restrict__ path_rank,
                                int32_t* __restrict__ draft_tok, float* __restrict__ q,
                                const ChunkStat* __restrict__ stats, int32_t* __restrict__ accept_len,
                                int32_t* __restrict__ out_tok) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float Tb = T[b];
  const bool greedy = !(Tb > 0.0f);
  const double invT = greedy ? 0.0 : 1.0 / (double)Tb;  // every exp((x - y) / T) is taken as exp_nonpos((x - y) * invT)
  const uint64_t sd = seed[b];
  const size_t zrow0 = (size_t)b * (L + 1);
  const ChunkStat* st_all = stats + zrow0 * n_chunk;
  const int n_terms = (L + 1) * n_chunk;
  const bool cached = n_terms <= kTermCache;

  // (0) every independent load at once, and all random blocks.  Loads are
  // unconditional, from clamped (in-range) indices, and land in registers
  // before any store: a masked load, or a store that needs a load's value
  // inside a branch, would be a branch that waits for the loads issued
  // before it
  const int lk = L * K;
  const size_t e0 = (size_t)b * lk;
  const int ei = min(tid, lk - 1);
  const int ci_raw = cand_idx[e0 + ei];
  // with the trace (the fused cycle) the scores launch has gathered the
  // candidates' target logits into zc_pre; the split verify reads them from Z
  const float zc_raw = MODE != kFinVerify ? zc_pre[e0 + ei] : 0.f;
  const float q_raw = MODE == kFinVerify ? q[e0 + ei] : 0.f;
  const int pr_raw = MODE == kFinVerify ? path_rank[(size_t)b * L + min(tid, L - 1)] : 0;
  constexpr int NS = DFLASH_L_MAX * DFLASH_K_MAX * DFLASH_K_MAX / kFinThreads;
  const size_t s0 = (size_t)b * lk * K;
  const int n = lk * K;
  float sv[NS];
  int js = 0;
  if (MODE != kFinVerify) {
#pragma unroll
    for (int k = 0; k < NS; ++k) sv[k] = qtab[s0 + min(tid + k * kFinThreads, n - 1)];
    if (MODE == kFinTable) js = jstar[e0 + ei];
  }
  constexpr int NC = kTermCache / kFinThreads;
  float2 mv[NC];
  if (cached) {
#pragma unroll
    for (int k = 0; k < NC; ++k)
      mv[k] = *reinterpret_cast<const float2*>(&st_all[min(tid + k * kFinThreads, n_terms - 1)]);
  }
  if (!greedy) {
    if (tid >= 64 && tid < 64 + L) f.rnd0[tid - 64] = stream_block(sd, cycle, (uint32_t)(tid - 63), 0u);
    if (tid >= 128 && tid <= 128 + L) f.rnd1[tid - 128] = stream_block(sd, cycle, (uint32_t)(tid - 127), 1u);
  }
  if (tid < lk) {
    const int t = tid / K, k = tid - (tid / K) * K;
    const int ci = clamp_idx(ci_raw, V);
    f.cand[t][k] = ci;
    f.cchunk[t][k] = geo.chunk_of(ci);
    if (MODE == kFinVerify) f.qs[t][k] = q_raw;
    if (!greedy) f.zc[t][k] = MODE != kFinVerify ? (double)zc_raw : geo.template logit<DT>(zrow0 + t, ci);
  }
  if (MODE == kFinVerify && tid < L) f.rank[tid] = clamp_idx(pr_raw, K);
  if (MODE != kFinVerify) {
#pragma unroll
    for (int k = 0; k < NS; ++k)
      if (tid + k * kFinThreads < n) f.S[tid + k * kFinThreads] = sv[k];
    if (MODE == kFinTable && tid < lk) f.jstar[tid] = min(max(js, 0), K - 1);
  }
  if (cached) {
#pragma unroll
    for (int k = 0; k < NC; ++k)
      if (tid + k * kFinThreads < n_terms) f.ms[tid + k * kFinThreads] = mv[k];
  }
  __syncthreads();

  // (1) the per-row combination of the chunk statistics, one wave per
  // target row; with the trace, wave 0 meanwhile walks the decided table
  // from rank 0 (L look-ups) and copies out each position's q (the row of
  // its predecessor's rank), rank and token
  if (MODE == kFinMaxSum && wave == 0) {
    // the max-sum path over the scores in f.S: lane g * 16 + j holds
    // best_t(j) (four replicas), a step splits the predecessors across the
    // groups, 4-bit back pointers of steps 0..7 and 8..15 in two registers;
    // first index at every tie
    const bool live = (lane & 15) < K;  // four 16-lane replicas of the columns
    const int jr = min(lane & 15, K - 1);
    double best = live ? (double)f.S[jr] : -INFINITY;
    uint32_t bk0 = 0, bk1 = 0;
#pragma unroll 1
    for (int t = 1; t < L; ++t) {
      double m;
      int arg;
      maxplus_step(best, &f.S[t * K * K], K, lane, m, arg);
      if (live) {
        best = m;
        if (t < 8) bk0 |= (uint32_t)arg << (4 * t);
        else bk1 |= (uint32_t)arg << (4 * (t - 8));
      }
    }
    double mx = best;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off));
    const unsigned long long hit = __ballot(live && best == mx);
    int jc = hit ? __ffsll((long long)hit) - 1 : 0;
    int mine = lane == L - 1 ? jc : 0;
#pragma unroll 1
    for (int t = L - 1; t >= 1; --t) {
      const uint32_t wv = __builtin_amdgcn_readlane(t < 8 ? bk0 : bk1, jc);
      jc = (int)((wv >> (4 * (t & 7))) & 15u);
      if (lane == t - 1) mine = jc;
    }
    if (lane < L) {
      f.rank[lane] = mine;
      path_rank[(size_t)b * L + lane] = mine;
      draft_tok[(size_t)b * L + lane] = f.cand[lane][mine];
    }
    for (int i = lane; i < L * K; i += kWave) {
      const int t = i / K;
      f.qs[t][i - t * K] = i - t * K == __shfl(mine, t) ? 1.f : 0.f;
    }
  } else if (MODE == kFinTable && wave == 0) {
    // the table's decisions in registers (lane l holds rows l, l + 64, ...)
    // so that each step of the chain is a lane read, not an LDS round trip
    constexpr int NJ = DFLASH_L_MAX * DFLASH_K_MAX / kWave;
    int jv[NJ];
#pragma unroll
    for (int c = 0; c < NJ; ++c) jv[c] = lane + c * kWave < L * K ? f.jstar[lane + c * kWave] : 0;
    int prev = 0, mine = 0;  // lane t keeps rank t
    for (int t = 0; t < L; ++t) {
      // every block's lane read, then a scalar select: no branch per step
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
    if (lane < L) {
      f.rank[lane] = mine;
      path_rank[(size_t)b * L + lane] = mine;
      draft_tok[(size_t)b * L + lane] = f.cand[lane][mine];
    }
  } else {
    constexpr int w0 = MODE != kFinVerify ? 1 : 0;
    for (int t = wave - w0; t <= L; t += kFinWaves - w0)
      combine_row<DT>(f, st_all + (size_t)t * n_chunk, t, L, K, n_chunk, cached, greedy, invT, lane);
  }
  __syncthreads();

  // the q output of the trace (the row of each position's predecessor's
  // rank, or one-hot at the max-sum path), written by the last wave (idle
  // or nearly so in the next phase)
  if (MODE != kFinVerify && wave == kFinWaves - 1) {
    for (int i = lane; i < L * K; i += kWave) {
      const int t = i / K;
      q[(size_t)b * L * K + i] = q_row_of<MODE == kFinTable>(f, t, K)[i - t * K];
    }
  }
  const size_t o = (size_t)b * (L + 1);
  if (greedy) {
    if (tid == 0) {
      int n = 0;
      while (n < L && f.cand[n][f.rank[n]] == f.rowArg[n]) ++n;
      accept_len[b] = n;
      for (int t = 0; t <= L; ++t) out_tok[o + t] = t < n ? f.cand[t][f.rank[t]] : (t == n ? f.rowArg[n] : -1);
    }
    return;
  }

  // (2) accept tests, all positions at once: u_t * q_t(d_t) < p_t(d_t)
  // (wave 0), beside the first level of the residual/bonus draw for every
  // row that could be the sampling row (the other waves, one row each)
  if (wave == 0) {
    bool rejected = false;
    if (lane < L) {
      const int j = f.rank[lane];
      const double u = (double)u01_f32(f.rnd0[lane].y);
      const double p = f.pc[lane][j] / f.rowAll[lane];
      rejected = !(u * (double)q_row_of<MODE == kFinTable>(f, lane, K)[j] < p);
    }
    const int fl = first_lane(rejected);
    if (lane == 0) f.s_n = fl < L ? fl : L;
  } else {
    for (int t = wave - 1; t <= L; t += kFinWaves - 1) {
      const int pk = pick_item(f, st_all + (size_t)t * n_chunk, t, L, K, n_chunk, cached, invT,
                               t < L ? q_row_of<MODE == kFinTable>(f, t, K) : f.qs[0], lane);
      if (lane == 0) f.pick_row[t] = pk;
    }
  }
  __syncthreads();
  const int ts = f.s_n;
  const int nk = ts < L ? K : 0;
  const uint4 w1 = f.rnd1[ts];
  const ChunkStat* st = st_all + (size_t)ts * n_chunk;
  const int pick = f.pick_row[ts];
  int tok;
  if (pick >= n_chunk) {
    tok = f.cand[ts][pick - n_chunk];
  } else {
    // (4) draw inside chunk `pick`: kFinTpt consecutive tokens per thread;
    // every weight is computed and masked afterwards (no branch per token)
    const ChunkLoc cl = geo.chunk(pick);
    const int c0 = cl.lo;
    const int e0 = c0 + tid * kFinTpt;
    const double mc = (double)(cached ? f.ms[ts * n_chunk + pick].x : st[pick].m);
    double zv[kFinTpt];
    load_tokens<DT, kFinTpt>(cl.Zs, (zrow0 + ts) * (size_t)cl.width, e0 - cl.base, cl.hi - cl.base, zv);
    // bit i set when token e0 + i is a candidate of row ts
    uint32_t cmask = 0;
#pragma unroll
    for (int k = 0; k < DFLASH_K_MAX; ++k) {
      const int off = (k < nk ? f.cand[ts][k] : -1) - e0;
      if (k < nk && off >= 0 && off < kFinTpt) cmask |= 1u << off;
    }
    // the weights exp2((z - m_c) * log2(e) / T) in fp32 (v_exp_f32) of the
    // exactly formed difference z - m_c (relative error about 2e-7),
    // accumulated in fp64
    const float k2 = kLog2e / Tb, mcf = (float)mc;
    double wv[kFinTpt];
    double run = 0.0;
    int last_pos = -1;
#pragma unroll
    for (int i = 0; i < kFinTpt; ++i) {
      const double ex = (double)__builtin_amdgcn_exp2f(((float)zv[i] - mcf) * k2);
      const double w = (e0 + i < cl.hi && !((cmask >> i) & 1u)) ? ex : 0.0;
      if (w > 0.0) last_pos = e0 + i;
      run += w;
      wv[i] = run;
    }
    const double incl = wave_scan_f64(run);
    if (lane == kWave - 1) f.wave_tot[wave] = incl;
    __syncthreads();
    // Every wave forms the same inclusive prefix sums P_w of the wave
    // totals (one lane per wave, a row scan) and so agrees on the owner:
    // the first wave with P_w > u2 * P_last.  Only the owner looks for the
    // token (the first of its values whose cumulative mass exceeds the
    // target; its last positive value if rounding leaves none) and writes
    // the outputs, so no second barrier is needed.  If no prefix exceeds
    // the target (rounding at the very end), the last wave with mass takes
    // its last positive value; with no mass at all, wave 0 takes the
    // chunk's first token.
    static_assert(kFinWaves == 16, "one row of lanes per wave total");
    const double tw = lane < kFinWaves ? f.wave_tot[lane] : 0.0;
    const double P = row16_scan_f64(tw);
    const double total = readlane_f64(P, kFinWaves - 1);
    const double target = u01_f64(w1.z, w1.w) * total;
    const uint64_t over = __ballot(lane < kFinWaves && P > target);
    const uint64_t mass = __ballot(lane < kFinWaves && tw > 0.0);
    const int owner = over ? __builtin_ctzll(over) : -1;
    const int lastw = mass ? 63 - __builtin_clzll(mass) : -1;
    const double before = owner > 0 ? readlane_f64(P, owner - 1) : 0.0;
    const int taker = owner >= 0 ? owner : (lastw >= 0 ? lastw : 0);
    if (wave != taker) return;
    int first = 0x7FFFFFFF;
    if (owner >= 0) {
      const double base = before + (incl - run);
#pragma unroll
      for (int i = kFinTpt - 1; i >= 0; --i)
        if (base + wv[i] > target) first = e0 + i;
    }
    // tokens follow the lane order: the wave's smallest hit is in its
    // lowest hitting lane, its last positive value in its highest lane
    const uint64_t hit = __ballot(first != 0x7FFFFFFF);
    const uint64_t pos = __ballot(last_pos >= 0);
    if (hit)
      tok = __builtin_amdgcn_readlane(first, __builtin_ctzll(hit));
    else if (pos)
      tok = __builtin_amdgcn_readlane(last_pos, 63 - __builtin_clzll(pos));
    else
      tok = c0;
    if (lane <= L) out_tok[o + lane] = lane < ts ? f.cand[lane][f.rank[lane]] : (lane == ts ? tok : -1);
    if (lane == 0) accept_len[b] = ts;
    return;
  }
  if (tid == 0) {
    accept_len[b] = ts;
    for (int t = 0; t <= L; ++t) out_tok[o + t] = t < ts ? f.cand[t][f.rank[t]] : (t == ts ? tok : -1);
  }
}

}  // namespace dfk
