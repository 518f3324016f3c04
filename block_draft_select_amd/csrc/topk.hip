// S1: top-K candidates of every drafter row (P1 "DFlash 2: Block diffusion,
// wearing a drafter's coat", section "Sixteen candidates per position").
//
// Design for gfx950.  The drafter rows are streamed once from HBM with
// 16-byte loads; each wave keeps its whole sub-segment (4096 bf16 or 2048
// fp32 values) in registers and finds its exact top-K in two passes over
// those registers:
//   1. per-lane maximum of order-preserving 16-bit keys (packed u16 max on
//      two bf16 values at a time), then the K-th largest lane maximum by a
//      16-step ballot bisection: at least K elements are >= that threshold,
//      so every element below it is beaten by K others;
//   2. the (few) elements at or above the threshold are appended to an LDS
//      buffer and ranked exactly by (value desc, index asc).
// A tie-heavy sub-segment that overflows the buffer falls back to an exact
// bisection over (value, index) on the register-resident keys.  The 4 waves
// of a block merge their lists; the last block of a row (device-scope
// counter, reset by that block) merges the sorted segment lists by binary
// search and writes the row's K candidates.  Results are independent of
// the segmentation because the order is total.
#include "device_util.hpp"
#include "internal.hpp"

namespace dfk {

namespace {

struct TkWave {
  uint64_t buf[kTopkCap];
  uint64_t top[16];
  uint32_t cnt;
  uint32_t pad;
};

union TkShared {
  TkWave wave[4];
  uint64_t merge[kTopkMergeMax];
};

// 64-bit candidate key: ordered value in the high word, inverted index low
__device__ __forceinline__ uint64_t make_key(uint32_t ord_value, uint32_t idx) {
  return ((uint64_t)ord_value << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

// exact rank of the buffered candidates; writes the wave's sorted top list
__device__ void rank_buffer(TkWave& w, int K, int lane) {
  const uint32_t c = min(w.cnt, (uint32_t)kTopkCap);
  if (lane < 16) w.top[lane] = 0;
  for (uint32_t i = lane; i < c; i += kWave) {
    const uint64_t key = w.buf[i];
    uint32_t rank = 0;
    for (uint32_t j = 0; j < c; ++j) rank += (w.buf[j] > key) ? 1u : 0u;
    if (rank < (uint32_t)K) w.top[rank] = key;
  }
}

// Exact top-K selection over register-resident elements for sub-segments
// whose threshold admits more than kTopkCap candidates (many equal values).
// `cv(slot)` gives the canonical value key of a slot (0 = no element),
// `loc(slot)` its index inside the sub-segment, `key(slot)` its 64-bit key.
template <int NSLOT, int VBITS, int LBITS, class CV, class LOC, class KEY>
__device__ void fallback_select(TkWave& w, int K, int lane, CV cv, LOC loc, KEY key) {
  // K-th largest canonical value (with multiplicity)
  uint32_t tv = 0;
  for (int bit = VBITS - 1; bit >= 0; --bit) {
    const uint32_t c = tv | (1u << bit);
    uint32_t n = 0;
#pragma unroll
    for (int s = 0; s < NSLOT; ++s) n += (cv(s) >= c) ? 1u : 0u;
    if (wave_sum_u32(n) >= (uint32_t)K) tv = c;
  }
  uint32_t gt = 0;
#pragma unroll
  for (int s = 0; s < NSLOT; ++s) gt += (cv(s) > tv) ? 1u : 0u;
  gt = wave_sum_u32(gt);
  const uint32_t need = (uint32_t)K - gt;  // >= 1 because fewer than K exceed tv
  // smallest local index x with #(value == tv, index <= x) >= need
  uint32_t lo = 0, hi = (1u << LBITS) - 1;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    uint32_t n = 0;
#pragma unroll
    for (int s = 0; s < NSLOT; ++s) n += (cv(s) == tv && loc(s) <= mid) ? 1u : 0u;
    if (wave_sum_u32(n) >= need) hi = mid; else lo = mid + 1;
  }
  if (lane == 0) w.cnt = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
  for (int s = 0; s < NSLOT; ++s) {
    const uint32_t v = cv(s);
    if (v > tv || (v == tv && loc(s) <= lo)) {
      const uint32_t pos = atomicAdd(&w.cnt, 1u);
      if (pos < (uint32_t)kTopkCap) w.buf[pos] = key(s);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

// one wave: bf16 sub-segment [lo, hi) of `row`
__device__ void wave_topk_bf16(const uint16_t* __restrict__ row, int lo, int hi, int K, TkWave& w,
                               int lane) {
  constexpr int WS = 64 * kTopkLoads * 8;
  uint32_t kx[4 * kTopkLoads];
  if (hi - lo == WS) {
#pragma unroll
    for (int j = 0; j < kTopkLoads; ++j) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + lo + (j * kWave + lane) * 8);
      kx[4 * j + 0] = ord16x2(v.x);
      kx[4 * j + 1] = ord16x2(v.y);
      kx[4 * j + 2] = ord16x2(v.z);
      kx[4 * j + 3] = ord16x2(v.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kTopkLoads; ++j) {
      const int base = lo + (j * kWave + lane) * 8;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t e0 = (base + 2 * c < hi) ? (uint32_t)row[base + 2 * c] : 0xFFFFu;
        const uint32_t e1 = (base + 2 * c + 1 < hi) ? (uint32_t)row[base + 2 * c + 1] : 0xFFFFu;
        kx[4 * j + c] = ord16x2(e0 | (e1 << 16));  // 0xFFFF pads to key 0
      }
    }
  }
  uint32_t m = kx[0];
#pragma unroll
  for (int q = 1; q < 4 * kTopkLoads; ++q) m = max_u16x2(m, kx[q]);
  const uint32_t lanemax = max(m & 0xFFFFu, m >> 16);

  // K-th largest lane maximum
  uint32_t thr = 0;
  for (int bit = 15; bit >= 0; --bit) {
    const uint32_t c = thr | (1u << bit);
    if (__popcll(__ballot(lanemax >= c)) >= (unsigned)K) thr = c;
  }
  if (thr == 0x8000u) thr = 0x7FFFu;  // a +0.0 threshold also admits -0.0
  if (thr == 0u) thr = 1u;            // never admit padding

  if (lane == 0) w.cnt = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  const uint32_t tm1 = (thr - 1u) * 0x00010001u;
#pragma unroll
  for (int q = 0; q < 4 * kTopkLoads; ++q) {
    if (subsat_u16x2(kx[q], tm1) != 0u) {
      const int base = ((q >> 2) * kWave + lane) * 8 + (q & 3) * 2;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t k16 = h ? (kx[q] >> 16) : (kx[q] & 0xFFFFu);
        if (k16 >= thr) {
          const uint32_t pos = atomicAdd(&w.cnt, 1u);
          if (pos < (uint32_t)kTopkCap) w.buf[pos] = make_key(ord32_of_k16(k16), (uint32_t)(lo + base + h));
        }
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  if (w.cnt > (uint32_t)kTopkCap) {
    auto k16_of = [&](int s) -> uint32_t { return (s & 1) ? (kx[s >> 1] >> 16) : (kx[s >> 1] & 0xFFFFu); };
    auto cv = [&](int s) -> uint32_t {
      const uint32_t k = k16_of(s);
      return k == 0x7FFFu ? 0x8000u : k;
    };
    auto loc = [&](int s) -> uint32_t {
      const int q = s >> 1;
      return (uint32_t)((((q >> 2) * kWave + lane) * 8) + (q & 3) * 2 + (s & 1));
    };
    auto key = [&](int s) -> uint64_t { return make_key(ord32_of_k16(k16_of(s)), (uint32_t)lo + loc(s)); };
    fallback_select<8 * kTopkLoads, 16, 12>(w, K, lane, cv, loc, key);
  }
  rank_buffer(w, K, lane);
}

// one wave: fp32 sub-segment [lo, hi) of `row`
__device__ void wave_topk_f32(const uint32_t* __restrict__ row, int lo, int hi, int K, TkWave& w,
                              int lane) {
  constexpr int WS = 64 * kTopkLoads * 4;
  uint32_t kx[4 * kTopkLoads];
  if (hi - lo == WS) {
#pragma unroll
    for (int j = 0; j < kTopkLoads; ++j) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + lo + (j * kWave + lane) * 4);
      kx[4 * j + 0] = ord32(v.x);
      kx[4 * j + 1] = ord32(v.y);
      kx[4 * j + 2] = ord32(v.z);
      kx[4 * j + 3] = ord32(v.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kTopkLoads; ++j) {
      const int base = lo + (j * kWave + lane) * 4;
#pragma unroll
      for (int c = 0; c < 4; ++c) kx[4 * j + c] = (base + c < hi) ? ord32(row[base + c]) : 0u;
    }
  }
  uint32_t lanemax = kx[0];
#pragma unroll
  for (int q = 1; q < 4 * kTopkLoads; ++q) lanemax = max(lanemax, kx[q]);
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = thr | (1u << bit);
    if (__popcll(__ballot(lanemax >= c)) >= (unsigned)K) thr = c;
  }
  if (thr == 0x80000000u) thr = 0x7FFFFFFFu;
  if (thr == 0u) thr = 1u;

  if (lane == 0) w.cnt = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
  for (int q = 0; q < 4 * kTopkLoads; ++q) {
    if (kx[q] >= thr) {
      const uint32_t canon = kx[q] == 0x7FFFFFFFu ? 0x80000000u : kx[q];
      const int idx = lo + ((q >> 2) * kWave + lane) * 4 + (q & 3);
      const uint32_t pos = atomicAdd(&w.cnt, 1u);
      if (pos < (uint32_t)kTopkCap) w.buf[pos] = make_key(canon, (uint32_t)idx);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  if (w.cnt > (uint32_t)kTopkCap) {
    auto cv = [&](int s) -> uint32_t { return kx[s] == 0x7FFFFFFFu ? 0x80000000u : kx[s]; };
    auto loc = [&](int s) -> uint32_t { return (uint32_t)((((s >> 2) * kWave + lane) * 4) + (s & 3)); };
    auto key = [&](int s) -> uint64_t { return make_key(cv(s), (uint32_t)lo + loc(s)); };
    fallback_select<4 * kTopkLoads, 32, 11>(w, K, lane, cv, loc, key);
  }
  rank_buffer(w, K, lane);
}

__device__ __forceinline__ void write_candidate(int32_t* cand_idx, float* cand_logit, size_t o, uint64_t key) {
  cand_idx[o] = (int32_t)(0xFFFFFFFFu - (uint32_t)key);
  cand_logit[o] = __uint_as_float(unord32((uint32_t)(key >> 32)));
}

// number of entries of a descending list (zeros last) greater than key
__device__ __forceinline__ int count_greater(const uint64_t* list, int n, uint64_t key) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (list[mid] > key) lo = mid + 1; else hi = mid;
  }
  return lo;
}

template <int DT>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const void* __restrict__ U, int V, int K,
                                                            int n_seg, uint64_t* __restrict__ partial,
                                                            uint32_t* __restrict__ counter,
                                                            int32_t* __restrict__ cand_idx,
                                                            float* __restrict__ cand_logit) {
  __shared__ TkShared sh;
  __shared__ uint64_t block_top[16];
  __shared__ int s_last;
  const int row = blockIdx.x / n_seg;
  const int seg = blockIdx.x - row * n_seg;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int WS = 64 * kTopkLoads * (DT == DFLASH_BF16 ? 8 : 4);
  const int lo = seg * 4 * WS + wave * WS;
  const int hi = min(lo + WS, V);

  if (DT == DFLASH_BF16) {
    const uint16_t* r = reinterpret_cast<const uint16_t*>(U) + (size_t)row * V;
    wave_topk_bf16(r, lo, max(hi, lo), K, sh.wave[wave], lane);
  } else {
    const uint32_t* r = reinterpret_cast<const uint32_t*>(U) + (size_t)row * V;
    wave_topk_f32(r, lo, max(hi, lo), K, sh.wave[wave], lane);
  }
  __syncthreads();

  // merge the four wave lists of this segment (wave 0, one key per lane)
  if (wave == 0) {
    const int n = 4 * K;
    const uint64_t key = lane < n ? sh.wave[lane / K].top[lane % K] : 0ull;
    uint32_t rank = 0;
    for (int j = 0; j < n; ++j) rank += (sh.wave[j / K].top[j % K] > key) ? 1u : 0u;
    if (lane < 16) block_top[lane] = 0ull;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    if (key != 0ull && rank < (uint32_t)K) block_top[rank] = key;
  }
  __syncthreads();

  const size_t out0 = (size_t)row * K;
  if (n_seg == 1) {
    if (tid < K) write_candidate(cand_idx, cand_logit, out0 + tid, block_top[tid]);
    return;
  }
  if (tid < 16) {
    partial[((size_t)row * n_seg + seg) * 16 + tid] = block_top[tid];
    __threadfence();
  }
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&counter[row], 1u) == (uint32_t)(n_seg - 1)) ? 1 : 0;
  __syncthreads();
  if (!s_last) return;

  // last block of this row: merge the n_seg sorted lists
  __threadfence();
  const int nk = n_seg * 16;
  const uint64_t* src = partial + (size_t)row * n_seg * 16;
  for (int i = tid; i < nk; i += kTopkThreads) sh.merge[i] = __builtin_nontemporal_load(src + i);
  __syncthreads();
  for (int i = tid; i < nk; i += kTopkThreads) {
    const int s = i >> 4, k = i & 15;
    const uint64_t key = sh.merge[i];
    if (key == 0ull || k >= K) continue;
    int rank = k;
    for (int s2 = 0; s2 < n_seg && rank < K; ++s2)
      if (s2 != s) rank += count_greater(sh.merge + s2 * 16, K, key);
    if (rank < K) write_candidate(cand_idx, cand_logit, out0 + rank, key);
  }
  if (tid == 0) atomicExch(&counter[row], 0u);
}

}  // namespace

hipError_t launch_topk(const dflash_dims& d, const WsLayout& w, const void* U, int32_t* cand_idx,
                       float* cand_logit, char* ws, hipStream_t st) {
  const int rows = d.B * d.L;
  const dim3 grid((unsigned)(rows * w.n_seg));
  uint64_t* partial = reinterpret_cast<uint64_t*>(ws + w.topk_partial);
  uint32_t* counter = reinterpret_cast<uint32_t*>(ws + w.topk_counter);
  if (d.logit_dtype == DFLASH_BF16)
    hipLaunchKernelGGL(topk_kernel<DFLASH_BF16>, grid, dim3(kTopkThreads), 0, st, U, d.V, d.K, w.n_seg,
                       partial, counter, cand_idx, cand_logit);
  else
    hipLaunchKernelGGL(topk_kernel<DFLASH_F32>, grid, dim3(kTopkThreads), 0, st, U, d.V, d.K, w.n_seg,
                       partial, counter, cand_idx, cand_logit);
  return hipGetLastError();
}

}  // namespace dfk
