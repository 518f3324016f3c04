// S5 + S6: verify a drafted path against the target rows (P1 "DFlash 2:
// Block diffusion, wearing a drafter's coat", section "Lossless, with
// conditions I did not used to state": accept with probability min(1, p/q),
// resample from the residual on rejection; P2 "A 2B Drafter Made a 27B
// Model 3.4x Faster. Same Exact Output.", section "Caveats before you
// rebuild your serving stack": greedy output equals the target's).
//
// stats_kernel streams every target row once.  One wave owns one chunk of
// DFLASH_CHUNK tokens (64 values per lane, 16-byte loads) and writes
//   greedy rows:   the chunk maximum and its first index;
//   sampling rows: the chunk maximum m and S = sum over non-candidate
//                  tokens of exp((z - m) / T), in fp32 with one v_exp_f32
//                  per value (candidates of the row are masked by their
//                  owner lane).
// finalize_kernel (one block per stream) combines the chunk statistics in
// fp64, runs the accept tests, and for the residual draw picks an item
// among (chunks, candidates) and, if a chunk wins, re-reads that one chunk
// (8 KB) to draw the token inside it in fp64.
#include "device_util.hpp"
#include "internal.hpp"

namespace dfk {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// bf16 chunk: 8 loads of 16 bytes per lane; element of (load j, word c,
// half h) is at chunk offset ((j * 64 + lane) * 8 + 2c + h)
__device__ __forceinline__ void load_chunk_bf16(const uint16_t* __restrict__ row, int lo, int hi,
                                                int lane, uint32_t (&x)[32]) {
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
      for (int c = 0; c < 4; ++c) {
        const uint32_t e0 = (base + 2 * c < hi) ? (uint32_t)row[base + 2 * c] : 0xFF80u;  // -inf
        const uint32_t e1 = (base + 2 * c + 1 < hi) ? (uint32_t)row[base + 2 * c + 1] : 0xFF80u;
        x[4 * j + c] = e0 | (e1 << 16);
      }
    }
  }
}

// fp32 chunk: 16 loads of 16 bytes per lane; element of (load j, word c) is
// at chunk offset ((j * 64 + lane) * 4 + c)
__device__ __forceinline__ void load_chunk_f32(const uint32_t* __restrict__ row, int lo, int hi,
                                               int lane, uint32_t (&x)[64]) {
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
      for (int c = 0; c < 4; ++c) x[4 * j + c] = (base + c < hi) ? row[base + c] : 0xFF800000u;
    }
  }
}

template <int DT>
__global__ __launch_bounds__(256) void stats_kernel(const void* __restrict__ Z, int L, int V, int K,
                                                    int n_chunk, long total, const float* __restrict__ T,
                                                    const int32_t* __restrict__ cand_idx,
                                                    ChunkStat* __restrict__ stats) {
  const long g = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= total) return;
  const int lane = threadIdx.x & 63;
  const long rowid = g / n_chunk;  // b * (L + 1) + t
  const int c = (int)(g - rowid * n_chunk);
  const int b = (int)(rowid / (L + 1));
  const int t = (int)(rowid - (long)b * (L + 1));
  const float Tb = T[b];
  const bool greedy = !(Tb > 0.0f);
  const int lo = c * kChunk, hi = min(lo + kChunk, V);
  ChunkStat st;
  st.pad = 0;

  if (DT == DFLASH_BF16) {
    const uint16_t* row = reinterpret_cast<const uint16_t*>(Z) + (size_t)rowid * V;
    uint32_t x[32];
    load_chunk_bf16(row, lo, hi, lane, x);
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
      uint32_t mx = ord16x2(x[0]);
#pragma unroll
      for (int q = 1; q < 32; ++q) mx = max_u16x2(mx, ord16x2(x[q]));
      const uint32_t m16 = wave_max_u32(max(mx & 0xFFFFu, mx >> 16));
      const float m = __uint_as_float(bf16_of_k16(m16) << 16);
      if (t < L) {  // mask this position's candidates
        const int32_t* ci = cand_idx + ((size_t)b * L + t) * K;
        for (int k = 0; k < K; ++k) {
          const int v = ci[k];
          if (v >= lo && v < hi) {
            const int off = v - lo, unit = off >> 3;
            const int owner = unit & 63, q = (unit >> 6) * 4 + ((off & 7) >> 1), h = off & 1;
#pragma unroll
            for (int qq = 0; qq < 32; ++qq)
              if (qq == q && lane == owner)
                x[qq] = h ? ((x[qq] & 0x0000FFFFu) | 0xFF800000u) : ((x[qq] & 0xFFFF0000u) | 0x0000FF80u);
          }
        }
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
    const uint32_t* row = reinterpret_cast<const uint32_t*>(Z) + (size_t)rowid * V;
    uint32_t x[64];
    load_chunk_f32(row, lo, hi, lane, x);
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
      if (t < L) {
        const int32_t* ci = cand_idx + ((size_t)b * L + t) * K;
        for (int k = 0; k < K; ++k) {
          const int v = ci[k];
          if (v >= lo && v < hi) {
            const int off = v - lo, unit = off >> 2;
            const int owner = unit & 63, q = (unit >> 6) * 4 + (off & 3);
#pragma unroll
            for (int qq = 0; qq < 64; ++qq)
              if (qq == q && lane == owner) x[qq] = 0xFF800000u;
          }
        }
      }
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
  if (lane == 0) stats[g] = st;
}

template <int DT>
__device__ __forceinline__ double logit_at(const void* Z, size_t i) {
  if (DT == DFLASH_BF16) return (double)__uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(Z)[i] << 16);
  return (double)reinterpret_cast<const float*>(Z)[i];
}

constexpr int kFinThreads = 256;
constexpr int kMaxChunks = DFLASH_V_MAX / kChunk;

template <int DT>
__global__ __launch_bounds__(kFinThreads) void finalize_kernel(
    const void* __restrict__ Z, int L, int V, int K, int n_chunk, const float* __restrict__ T,
    const uint64_t* __restrict__ seed, uint64_t cycle, const int32_t* __restrict__ cand_idx,
    const int32_t* __restrict__ path_rank, const float* __restrict__ q, const ChunkStat* __restrict__ stats,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tok) {
  __shared__ float rowM[DFLASH_L_MAX + 1];
  __shared__ double rowNC[DFLASH_L_MAX + 1];
  __shared__ double rowSum[DFLASH_L_MAX + 1];
  __shared__ int rowArg[DFLASH_L_MAX + 1];
  __shared__ double pc[DFLASH_L_MAX][DFLASH_K_MAX];  // exp((z_cand - M) / T)
  __shared__ int rank_s[DFLASH_L_MAX];
  __shared__ int draft_s[DFLASH_L_MAX];
  __shared__ double item[kMaxChunks + DFLASH_K_MAX];
  __shared__ double wave_tot[4];
  __shared__ int s_n, s_pick, s_tok;
  __shared__ int cand_s[DFLASH_K_MAX];

  const int b = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float Tb = T[b];
  const bool greedy = !(Tb > 0.0f);
  const double Td = (double)Tb;
  const uint64_t sd = seed[b];
  const size_t Vs = (size_t)V;
  const size_t zrow0 = (size_t)b * (L + 1);

  if (tid < L) {
    const int j = clamp_idx(path_rank[(size_t)b * L + tid], K);
    rank_s[tid] = j;
    draft_s[tid] = clamp_idx(cand_idx[((size_t)b * L + tid) * K + j], V);
  }

  // per-row combination of the chunk statistics (one wave per row)
  for (int t = wave; t <= L; t += 4) {
    const ChunkStat* st = stats + (zrow0 + t) * n_chunk;
    float M = -INFINITY;
    for (int c = lane; c < n_chunk; c += kWave) M = fmaxf(M, st[c].m);
    M = wave_max_f32(M);
    int arg = 0x7FFFFFFF;
    double s = 0.0;
    if (greedy) {
      for (int c = lane; c < n_chunk; c += kWave)
        if (st[c].m == M) arg = min(arg, st[c].arg);
      arg = wave_min_i32(arg);
    } else {
      for (int c = lane; c < n_chunk; c += kWave)
        s += (double)st[c].s * exp(((double)st[c].m - (double)M) / Td);
      s = wave_sum_f64(s);
    }
    if (lane == 0) {
      rowM[t] = M;
      rowNC[t] = s;
      rowArg[t] = arg;
    }
  }
  __syncthreads();

  const size_t o = (size_t)b * (L + 1);
  if (greedy) {
    if (tid == 0) {
      int n = 0;
      while (n < L && draft_s[n] == rowArg[n]) ++n;
      accept_len[b] = n;
      for (int t = 0; t <= L; ++t) out_tok[o + t] = t < n ? draft_s[t] : (t == n ? rowArg[n] : -1);
    }
    return;
  }

  // candidate masses of rows 0..L-1 (unnormalised, relative to the row max)
  for (int i = tid; i < L * K; i += kFinThreads) {
    const int t = i / K, k = i - t * K;
    const int ci = clamp_idx(cand_idx[((size_t)b * L + t) * K + k], V);
    pc[t][k] = exp((logit_at<DT>(Z, (zrow0 + t) * Vs + ci) - (double)rowM[t]) / Td);
  }
  __syncthreads();
  if (tid <= L) {
    double s = rowNC[tid];
    if (tid < L)
      for (int k = 0; k < K; ++k) s += pc[tid][k];
    rowSum[tid] = s;
  }
  __syncthreads();

  // accept tests: u_t * q_t(d_t) < p_t(d_t)
  if (tid == 0) {
    int n = L;
    for (int t = 0; t < L; ++t) {
      const uint4 w = stream_block(sd, cycle, (uint32_t)(t + 1), 0u);
      const double u = (double)u01_f32(w.y);
      const double qd = (double)q[((size_t)b * L + t) * K + rank_s[t]];
      const double p = pc[t][rank_s[t]] / rowSum[t];
      if (!(u * qd < p)) {
        n = t;
        break;
      }
    }
    s_n = n;
  }
  __syncthreads();
  const int ts = s_n;
  const bool has_cand = ts < L;
  const int nk = has_cand ? K : 0;
  const double inv = 1.0 / rowSum[ts];
  const ChunkStat* st = stats + (zrow0 + ts) * n_chunk;
  const double Mts = (double)rowM[ts];

  // items: chunk masses, then candidate residuals
  for (int c = tid; c < n_chunk; c += kFinThreads)
    item[c] = (double)st[c].s * exp(((double)st[c].m - Mts) / Td) * inv;
  if (tid < nk) {
    const double p = pc[ts][tid] * inv;
    item[n_chunk + tid] = fmax(0.0, p - (double)q[((size_t)b * L + ts) * K + tid]);
    cand_s[tid] = clamp_idx(cand_idx[((size_t)b * L + ts) * K + tid], V);
  }
  __syncthreads();
  const int n_item = n_chunk + nk;
  const uint4 w1 = stream_block(sd, cycle, (uint32_t)(ts + 1), 1u);
  if (wave == 0) {
    // inclusive scan in item order (one wave, 64 items per step)
    double carry = 0.0;
    for (int base = 0; base < n_item; base += kWave) {
      double v = (base + lane < n_item) ? item[base + lane] : 0.0;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const double y = __shfl_up(v, off);
        if (lane >= off) v += y;
      }
      v += carry;
      if (base + lane < n_item) item[base + lane] = v;
      carry = __shfl(v, kWave - 1);
    }
    double total = carry;
    if (!(total > 0.0) && nk > 0) {
      // the residual has no mass: draw from p itself (candidates keep mass p)
      carry = 0.0;
      for (int base = 0; base < n_item; base += kWave) {
        const int i = base + lane;
        double v = 0.0;
        if (i < n_chunk) v = (double)st[i].s * exp(((double)st[i].m - Mts) / Td) * inv;
        else if (i < n_item) v = pc[ts][i - n_chunk] * inv;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const double y = __shfl_up(v, off);
          if (lane >= off) v += y;
        }
        v += carry;
        if (i < n_item) item[i] = v;
        carry = __shfl(v, kWave - 1);
      }
      total = carry;
    }
    const double target = u01_f64(w1.x, w1.y) * total;
    int pick = 0x7FFFFFFF;
    for (int base = 0; base < n_item; base += kWave) {
      const int i = base + lane;
      if (i < n_item && item[i] > target) pick = min(pick, i);
    }
    pick = wave_min_i32(pick);
    if (lane == 0) {
      s_pick = min(pick, n_item - 1);
      s_tok = 0x7FFFFFFF;
    }
  }
  __syncthreads();
  const int pick = s_pick;
  int tok;
  if (pick >= n_chunk) {
    tok = cand_s[pick - n_chunk];
  } else {
    // draw inside chunk `pick`: 16 consecutive tokens per thread, fp64
    const int c0 = pick * kChunk;
    const double mc = (double)st[pick].m;
    double wv[16];
    double run = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = c0 + tid * 16 + i;
      double w = 0.0;
      if (e < V) {
        bool is_c = false;
        for (int k = 0; k < nk; ++k) is_c |= (cand_s[k] == e);
        if (!is_c) w = exp((logit_at<DT>(Z, (zrow0 + ts) * Vs + e) - mc) / Td);
      }
      run += w;
      wv[i] = run;
    }
    // exclusive prefix of the thread totals across the block
    double incl = run;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const double y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    double base = incl - run;
    for (int w = 0; w < wave; ++w) base += wave_tot[w];
    const double total = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    const double target = u01_f64(w1.z, w1.w) * total;
    int first = 0x7FFFFFFF;
#pragma unroll
    for (int i = 15; i >= 0; --i)
      if (base + wv[i] > target) first = c0 + tid * 16 + i;
    if (first != 0x7FFFFFFF) atomicMin(&s_tok, first);
    __syncthreads();
    tok = s_tok;
    if (tok == 0x7FFFFFFF) tok = min(V - 1, c0 + kChunk - 1);
  }
  if (tid == 0) {
    accept_len[b] = ts;
    for (int t = 0; t <= L; ++t) out_tok[o + t] = t < ts ? draft_s[t] : (t == ts ? tok : -1);
  }
}

}  // namespace

hipError_t launch_stats(const dflash_dims& d, const WsLayout& w, const void* Z, const int32_t* cand_idx,
                        const float* T, ChunkStat* stats, hipStream_t st) {
  const long total = (long)d.B * (d.L + 1) * w.n_chunk;
  const dim3 grid((unsigned)((total + 3) / 4));
  if (d.logit_dtype == DFLASH_BF16)
    hipLaunchKernelGGL(stats_kernel<DFLASH_BF16>, grid, dim3(256), 0, st, Z, d.L, d.V, d.K, w.n_chunk,
                       total, T, cand_idx, stats);
  else
    hipLaunchKernelGGL(stats_kernel<DFLASH_F32>, grid, dim3(256), 0, st, Z, d.L, d.V, d.K, w.n_chunk,
                       total, T, cand_idx, stats);
  return hipGetLastError();
}

hipError_t launch_finalize(const dflash_dims& d, const WsLayout& w, const void* Z,
                           const int32_t* cand_idx, const int32_t* path_rank, const float* q,
                           const float* T, const uint64_t* seed, uint64_t cycle,
                           const ChunkStat* stats, int32_t* accept_len, int32_t* out_tok,
                           hipStream_t st) {
  const dim3 grid((unsigned)d.B);
  if (d.logit_dtype == DFLASH_BF16)
    hipLaunchKernelGGL(finalize_kernel<DFLASH_BF16>, grid, dim3(kFinThreads), 0, st, Z, d.L, d.V, d.K,
                       w.n_chunk, T, seed, cycle, cand_idx, path_rank, q, stats, accept_len, out_tok);
  else
    hipLaunchKernelGGL(finalize_kernel<DFLASH_F32>, grid, dim3(kFinThreads), 0, st, Z, d.L, d.V, d.K,
                       w.n_chunk, T, seed, cycle, cand_idx, path_rank, q, stats, accept_len, out_tok);
  return hipGetLastError();
}

}  // namespace dfk
