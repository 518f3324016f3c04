// Device building blocks of S5 + S6 (verify against the target rows; P1
// "DFlash 2: Block diffusion, wearing a drafter's coat", section "Lossless,
// with conditions I did not used to state": accept with probability
// min(1, p/q), resample from the residual on rejection; P2 "A 2B Drafter
// Made a 27B Model 3.4x Faster. Same Exact Output.", section "Caveats before
// you rebuild your serving stack": greedy output equals the target's).
//
// stats_chunk: one wave reduces one chunk of DFLASH_CHUNK tokens of a target
//   row held in registers (64 values per lane, 16-byte loads):
//     greedy rows:   the chunk maximum and its first index;
//     sampling rows: the chunk maximum m and S = sum over all tokens of
//                    exp((z - m) / T), in fp32 with one v_exp_f32 per value.
//   The statistics do not depend on the candidates, so they stream in the
//   same launch as the top-K; the candidates' own mass is taken out of their
//   chunk in fp64 by the finalize.  The bf16 maximum first tries a packed
//   signed 16-bit max of the raw patterns, exact whenever the maximum is
//   non-negative.
// finalize_stream: one block per stream combines the chunk statistics in
//   fp64, runs the accept tests, and draws the residual/bonus token in two
//   inverse-CDF levels (item = chunk or candidate, then the token inside a
//   drawn chunk, which is re-read).  Optionally the block first walks the
//   trace (one wave) while the other waves combine the statistics.
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

// Statistics of chunk c of target row `rowid` (one wave).
template <int DT>
__device__ __forceinline__ ChunkStat stats_chunk(const void* __restrict__ Z, size_t rowid, int V, int c, float Tb,
                                                 int lane) {
  const bool greedy = !(Tb > 0.0f);
  const int lo = c * kChunk, hi = min(lo + kChunk, V);
  ChunkStat st;
  st.pad = 0;
  if (DT == DFLASH_BF16) {
    const uint16_t* row = reinterpret_cast<const uint16_t*>(Z) + rowid * V;
    uint32_t x[32];
    if (hi - lo == kChunk) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + lo + (j * kWave + lane) * 8);
        x[4 * j + 0] = v.x;
        x[4 * j + 1] = v.y;
        x[4 * j + 2] = v.z;
        x[4 * j + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int base = lo + (j * kWave + lane) * 8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t e0 = (base + 2 * q < hi) ? (uint32_t)row[base + 2 * q] : 0xFF80u;  // -inf
          const uint32_t e1 = (base + 2 * q + 1 < hi) ? (uint32_t)row[base + 2 * q + 1] : 0xFF80u;
          x[4 * j + q] = e0 | (e1 << 16);
        }
      }
    }
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
      const float k2 = kLog2e / Tb;
      const float mk = m * k2;
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
      for (int q = 0; q < 32; q += 2) {
        s0 += __builtin_amdgcn_exp2f(fmaf(bf16_lo(x[q]), k2, -mk));
        s1 += __builtin_amdgcn_exp2f(fmaf(bf16_hi(x[q]), k2, -mk));
        s2 += __builtin_amdgcn_exp2f(fmaf(bf16_lo(x[q + 1]), k2, -mk));
        s3 += __builtin_amdgcn_exp2f(fmaf(bf16_hi(x[q + 1]), k2, -mk));
      }
      st.m = m;
      st.s = wave_sum_f32((s0 + s1) + (s2 + s3));
      st.arg = -1;
    }
  } else {
    const uint32_t* row = reinterpret_cast<const uint32_t*>(Z) + rowid * V;
    uint32_t x[64];
    if (hi - lo == kChunk) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + lo + (j * kWave + lane) * 4);
        x[4 * j + 0] = v.x;
        x[4 * j + 1] = v.y;
        x[4 * j + 2] = v.z;
        x[4 * j + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int base = lo + (j * kWave + lane) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) x[4 * j + q] = (base + q < hi) ? row[base + q] : 0xFF800000u;
      }
    }
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
      const float mk = m * k2;
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
      for (int q = 0; q < 64; q += 4) {
        s0 += __builtin_amdgcn_exp2f(fmaf(__uint_as_float(x[q + 0]), k2, -mk));
        s1 += __builtin_amdgcn_exp2f(fmaf(__uint_as_float(x[q + 1]), k2, -mk));
        s2 += __builtin_amdgcn_exp2f(fmaf(__uint_as_float(x[q + 2]), k2, -mk));
        s3 += __builtin_amdgcn_exp2f(fmaf(__uint_as_float(x[q + 3]), k2, -mk));
      }
      st.m = m;
      st.s = wave_sum_f32((s0 + s1) + (s2 + s3));
      st.arg = -1;
    }
  }
  return st;
}

template <int DT>
__device__ __forceinline__ double logit_at(const void* Z, size_t i) {
  if (DT == DFLASH_BF16) return (double)__uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(Z)[i] << 16);
  return (double)reinterpret_cast<const float*>(Z)[i];
}

constexpr int kFinThreads = 256;
constexpr int kMaxChunks = DFLASH_V_MAX / kChunk;
constexpr int kTermCache = 2048;  // chunk terms of all rows kept in LDS when they fit

struct FinLds {
  float2 ms[kTermCache];                            // (m, s) of every chunk of every row
  double term[kTermCache];                          // s * exp((m - M_t) / T)
  float S[DFLASH_L_MAX * DFLASH_K_MAX * DFLASH_K_MAX];  // scores (when the trace runs here)
  TraceLds tl;
  float rowM[DFLASH_L_MAX + 1];
  double rowAll[DFLASH_L_MAX + 1];                  // sum over all tokens of exp((z - M) / T)
  int rowArg[DFLASH_L_MAX + 1];
  double pc[DFLASH_L_MAX][DFLASH_K_MAX];            // exp((z_cand - M) / T)
  double zc[DFLASH_L_MAX][DFLASH_K_MAX];            // candidate target logits
  float qs[DFLASH_L_MAX][DFLASH_K_MAX];
  int cand[DFLASH_L_MAX][DFLASH_K_MAX];
  int rank[DFLASH_L_MAX];
  uint4 rnd0[DFLASH_L_MAX];                         // (cycle, t + 1, 0) blocks
  uint4 rnd1[DFLASH_L_MAX + 1];                     // (cycle, t + 1, 1) blocks
  double item[kMaxChunks + DFLASH_K_MAX];
  double wave_tot[4];
  int s_n, s_pick, s_tok, s_last;
};

// Combine the statistics of row t (one wave): maximum, first argmax chunk,
// and for sampling rows every chunk term and the candidate weights.
template <int DT>
__device__ __forceinline__ void combine_row(FinLds& f, const ChunkStat* __restrict__ st_row, int t, int L, int K,
                                            int n_chunk, bool cached, bool greedy, double Td, int lane) {
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
    if (lane == 0) {
      f.rowM[t] = M;
      f.rowArg[t] = st_row[first].arg;
    }
    return;
  }
  double s = 0.0;
  for (int c = lane; c < n_chunk; c += kWave) {
    const float2 v = cached ? f.ms[t * n_chunk + c] : make_float2(st_row[c].m, st_row[c].s);
    const double tm = (double)v.y * exp(((double)v.x - (double)M) / Td);
    if (cached) f.term[t * n_chunk + c] = tm;
    s += tm;
  }
  s = wave_sum_dpp_f64(s);
  if (t < L && lane < K) f.pc[t][lane] = exp((f.zc[t][lane] - (double)M) / Td);
  if (lane == 0) {
    f.rowM[t] = M;
    f.rowAll[t] = s;
  }
}

// One block per stream.  WITH_TRACE: the block also walks the trace over
// scores S (wave 0) and writes path_rank / draft_tok / q; otherwise
// path_rank and q are inputs.  zc_pre, if given, holds the candidates'
// target logits [B, L, K] (fp32-exact values), else they are gathered here.
template <int DT, bool WITH_TRACE>
__device__ void finalize_stream(FinLds& f, int b, const void* __restrict__ Z, int L, int V, int K, int n_chunk,
                                const float* __restrict__ T, const uint64_t* __restrict__ seed, uint64_t cycle,
                                const int32_t* __restrict__ cand_idx, const float* __restrict__ zc_pre,
                                const float* __restrict__ S, int32_t* __restrict__ path_rank,
                                int32_t* __restrict__ draft_tok, float* __restrict__ q,
                                const ChunkStat* __restrict__ stats, int32_t* __restrict__ accept_len,
                                int32_t* __restrict__ out_tok) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float Tb = T[b];
  const bool greedy = !(Tb > 0.0f);
  const double Td = (double)Tb;
  const uint64_t sd = seed[b];
  const size_t Vs = (size_t)V;
  const size_t zrow0 = (size_t)b * (L + 1);
  const ChunkStat* st_all = stats + zrow0 * n_chunk;
  const int n_terms = (L + 1) * n_chunk;
  const bool cached = n_terms <= kTermCache;

  // (0) every independent load at once, and all random blocks
  if (tid < L * K) {
    const int t = tid / K, k = tid - (tid / K) * K;
    const size_t e = (size_t)b * L * K + tid;
    const int ci = clamp_idx(cand_idx[e], V);
    f.cand[t][k] = ci;
    if (!WITH_TRACE) f.qs[t][k] = q[e];
    if (!greedy) f.zc[t][k] = zc_pre ? (double)zc_pre[e] : logit_at<DT>(Z, (zrow0 + t) * Vs + ci);
  }
  if (!WITH_TRACE && tid < L) f.rank[tid] = clamp_idx(path_rank[(size_t)b * L + tid], K);
  if (WITH_TRACE) {
    // fixed trip counts so that every load is issued before the first store
    constexpr int NS = DFLASH_L_MAX * DFLASH_K_MAX * DFLASH_K_MAX / kFinThreads;
    const size_t s0 = (size_t)b * L * K * K;
    const int n = L * K * K;
    float sv[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) sv[k] = tid + k * kFinThreads < n ? S[s0 + tid + k * kFinThreads] : 0.f;
#pragma unroll
    for (int k = 0; k < NS; ++k)
      if (tid + k * kFinThreads < n) f.S[tid + k * kFinThreads] = sv[k];
    if (wave == 0) trace_setup(f.tl, Tb, sd, cycle, L, lane);
  }
  if (!greedy) {
    if (tid >= 64 && tid < 64 + L) f.rnd0[tid - 64] = stream_block(sd, cycle, (uint32_t)(tid - 63), 0u);
    if (tid >= 128 && tid <= 128 + L) f.rnd1[tid - 128] = stream_block(sd, cycle, (uint32_t)(tid - 127), 1u);
  }
  if (cached) {
    constexpr int NC = kTermCache / kFinThreads;
    float2 mv[NC];
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int i = tid + k * kFinThreads;
      mv[k] = i < n_terms ? *reinterpret_cast<const float2*>(&st_all[i]) : make_float2(0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < NC; ++k)
      if (tid + k * kFinThreads < n_terms) f.ms[tid + k * kFinThreads] = mv[k];
  }
  __syncthreads();

  // (1) the trace (wave 0) beside the per-row combination (the other waves)
  if (WITH_TRACE && wave == 0) {
    int prev = 0;
    for (int t = 0; t < L; ++t) {
      const size_t e0 = ((size_t)b * L + t) * K;
      const int j = trace_step_dpp(f.tl, &f.S[(t * K + prev) * K], Tb, t, K, lane, &f.cand[t][0], q + e0,
                                   path_rank + (size_t)b * L + t, draft_tok + (size_t)b * L + t, &f.qs[t][0]);
      if (lane == 0) f.rank[t] = j;
      prev = j;
    }
  }
  {
    const int w0 = WITH_TRACE ? 1 : 0, nw = WITH_TRACE ? 3 : 4;
    if (wave >= w0)
      for (int t = wave - w0; t <= L; t += nw)
        combine_row<DT>(f, st_all + (size_t)t * n_chunk, t, L, K, n_chunk, cached, greedy, Td, lane);
  }
  __syncthreads();

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
  if (wave == 0) {
    bool rejected = false;
    if (lane < L) {
      const int j = f.rank[lane];
      const double u = (double)u01_f32(f.rnd0[lane].y);
      const double p = f.pc[lane][j] / f.rowAll[lane];
      rejected = !(u * (double)f.qs[lane][j] < p);
    }
    const int fl = first_lane(rejected);
    if (lane == 0) f.s_n = fl < L ? fl : L;
  }
  __syncthreads();
  const int ts = f.s_n;
  const int nk = ts < L ? K : 0;
  const double inv = 1.0 / f.rowAll[ts];
  const uint4 w1 = f.rnd1[ts];
  const ChunkStat* st = st_all + (size_t)ts * n_chunk;

  // (3) residual items of row ts: chunk masses without the candidates, then
  // the candidates' max(0, p - q); drawn by one wave
  if (wave == 0) {
    // the row's candidates in registers: their chunk and weight
    int cchunk[DFLASH_K_MAX];
    double cpc[DFLASH_K_MAX];
#pragma unroll
    for (int k = 0; k < DFLASH_K_MAX; ++k) {
      cchunk[k] = k < nk ? f.cand[ts][k] / kChunk : -1;
      cpc[k] = k < nk ? f.pc[ts][k] : 0.0;
    }
    const int n_item = n_chunk + nk;
    bool resid = true;
    double total = 0.0;
    for (int pass = 0; pass < 2; ++pass) {
      double carry = 0.0;
      for (int base = 0; base < n_item; base += kWave) {
        const int i = base + lane;
        double v = 0.0;
        if (i < n_chunk) {
          double tm;
          if (cached) {
            tm = f.term[ts * n_chunk + i];
          } else {
            const ChunkStat cs = st[i];
            tm = (double)cs.s * exp(((double)cs.m - (double)f.rowM[ts]) / Td);
          }
          double cm = 0.0;
#pragma unroll
          for (int k = 0; k < DFLASH_K_MAX; ++k)
            if (k < nk && cchunk[k] == i) cm += cpc[k];
          v = fmax(0.0, (tm - cm) * inv);
        } else if (i < n_item) {
          const double p = f.pc[ts][i - n_chunk] * inv;
          v = resid ? fmax(0.0, p - (double)f.qs[ts][i - n_chunk]) : p;
        }
        v = wave_scan_f64(v) + carry;
        if (i < n_item) f.item[i] = v;
        carry = readlane_f64(v, 63);
      }
      total = carry;
      if (total > 0.0 || nk == 0 || !resid) break;
      resid = false;  // the residual has no mass: draw from p itself (candidates keep mass p)
    }
    const double target = u01_f64(w1.x, w1.y) * total;
    int pick = n_item - 1;
    for (int base = 0; base < n_item; base += kWave) {
      const int i = base + lane;
      const int fl = first_lane(i < n_item && f.item[i] > target);
      if (fl < 64) {
        pick = base + fl;
        break;
      }
    }
    if (lane == 0) {
      f.s_pick = pick;
      f.s_tok = 0x7FFFFFFF;
      f.s_last = -1;
    }
  }
  __syncthreads();
  const int pick = f.s_pick;
  int tok;
  if (pick >= n_chunk) {
    tok = f.cand[ts][pick - n_chunk];
  } else {
    // (4) draw inside chunk `pick`: 16 consecutive tokens per thread, fp64
    const int c0 = pick * kChunk;
    const double mc = (double)(cached ? f.ms[ts * n_chunk + pick].x : st[pick].m);
    const size_t zr = (zrow0 + ts) * Vs;
    double zv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = c0 + tid * 16 + i;
      zv[i] = e < V ? logit_at<DT>(Z, zr + e) : 0.0;
    }
    // bit i set when token c0 + tid * 16 + i is a candidate of row ts
    uint32_t cmask = 0;
#pragma unroll
    for (int k = 0; k < DFLASH_K_MAX; ++k) {
      const int off = (k < nk ? f.cand[ts][k] : -1) - (c0 + tid * 16);
      if (k < nk && off >= 0 && off < 16) cmask |= 1u << off;
    }
    double wv[16];
    double run = 0.0;
    int last_pos = -1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = c0 + tid * 16 + i;
      double w = 0.0;
      if (e < V && !((cmask >> i) & 1u)) w = exp((zv[i] - mc) / Td);
      if (w > 0.0) last_pos = e;
      run += w;
      wv[i] = run;
    }
    const double incl = wave_scan_f64(run);
    if (lane == kWave - 1) f.wave_tot[wave] = incl;
    __syncthreads();
    double base = incl - run;
    for (int w = 0; w < wave; ++w) base += f.wave_tot[w];
    const double total = f.wave_tot[0] + f.wave_tot[1] + f.wave_tot[2] + f.wave_tot[3];
    const double target = u01_f64(w1.z, w1.w) * total;
    int first = 0x7FFFFFFF;
#pragma unroll
    for (int i = 15; i >= 0; --i)
      if (base + wv[i] > target) first = c0 + tid * 16 + i;
    if (first != 0x7FFFFFFF) atomicMin(&f.s_tok, first);
    if (last_pos >= 0) atomicMax(&f.s_last, last_pos);
    __syncthreads();
    tok = f.s_tok;
    if (tok == 0x7FFFFFFF) tok = f.s_last >= 0 ? f.s_last : min(V - 1, c0);
  }
  if (tid == 0) {
    accept_len[b] = ts;
    for (int t = 0; t <= L; ++t) out_tok[o + t] = t < ts ? f.cand[t][f.rank[t]] : (t == ts ? tok : -1);
  }
}

}  // namespace dfk
