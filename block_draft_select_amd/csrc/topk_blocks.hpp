// Device building blocks of S1 (top-K candidates of every drafter row; P1
// "DFlash 2: Block diffusion, wearing a drafter's coat", section "Sixteen
// candidates per position").
//
// Drafter rows are streamed once from HBM with 16-byte loads.  A row is cut
// into sub-segments of 64 x 64 values (bf16; 64 x 32 fp32): one wave holds a
// whole sub-segment in registers and folds it into its running top list in
// two passes over those registers:
//   1. one value per lane (a packed signed 16-bit max of the raw bf16
//      patterns picks the lane maximum whenever the lane holds a
//      non-negative value, and some value of the lane otherwise), then the
//      K-th largest pick by a 16-step ballot bisection: at least K values
//      of the sub-segment are at or above it.  The running list's K-th key
//      (plus one: later indices lose ties) is a second lower bound; the
//      larger one is the threshold;
//   2. values at or above the threshold are appended to an LDS buffer next
//      to the running list (bf16: as 32-bit compact keys, widened to the
//      64-bit list keys only when they enter the list) and merged into it
//      by exact rank (value desc, index asc).
// Once a wave's running list is full, its K-th key + 1 replaces the
// per-sub-segment threshold (later sub-segments have larger indices and
// lose ties), and the bisection is skipped.  The four waves of a block also
// share a lower bound in LDS: any wave's K-th largest pick, and later any
// wave's K-th list value, bounds the block's K-th value from below, so
// smaller values cannot be in the block's list (equal values still can, by
// index).  For bf16 the first thresholds are shared before any wave scans.
// A tie-heavy sub-segment whose candidates overflow the buffer takes an
// out-of-line exact path that re-reads it.  A block (4 waves) owns a run of
// sub-segments and writes the sorted top list of that run; the lists of a
// row are merged by binary-search ranking.  Results do not depend on the
// segmentation because the order is total.
#pragma once

#include "device_util.hpp"
#include "internal.hpp"

namespace dfk {

struct TkWave {
  uint64_t buf[kTopkCap];
  uint64_t top[16];  // running list, sorted, zero = empty
  uint32_t cnt;
  uint32_t ntop;
};

// 64-bit candidate key: ordered value in the high word, inverted index low
__device__ __forceinline__ uint64_t make_key(uint32_t ord_value, uint32_t idx) {
  return ((uint64_t)ord_value << 32) | (uint64_t)(0xFFFFFFFFu - idx);
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

// number of entries of a 16-entry descending list (zeros last) greater
// than key: 16 independent loads and compares, no dependent chain
__device__ __forceinline__ int count_greater16(const uint64_t* list, uint64_t key) {
  int n = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) n += list[k] > key ? 1 : 0;
  return n;
}

// Merge the buffered keys into the running list.  buf[0, ntop) is the
// running list (sorted, descending); buf[ntop, cnt) holds new candidates in
// any order; all keys are distinct and non-zero.  A running key's new rank
// is its position plus the number of larger new keys; a new key's rank is
// the number of larger running keys (binary search) plus larger new keys.
__device__ void merge_buffer(TkWave& w, uint32_t cnt, int K, int lane) {
  const uint32_t ntop = w.ntop;
  const uint32_t c = min(cnt, (uint32_t)kTopkCap);
  if (c == ntop) return;  // nothing new
  if (c <= (uint32_t)kWave) {
    // one key per lane: its rank is the number of larger keys among all c,
    // read in batches of 16 independent loads
    const uint64_t mine = lane < (int)c ? w.buf[lane] : 0ull;
    uint32_t rank = 0;
    for (uint32_t j0 = 0; j0 < c; j0 += 16) {
      uint64_t o[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) o[u] = w.buf[j0 + u];
#pragma unroll
      for (int u = 0; u < 16; ++u) rank += (j0 + u < c && o[u] > mine) ? 1u : 0u;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (lane < (int)c && rank < (uint32_t)K) w.top[rank] = mine;
  } else {
    // rare (more than one key per lane): one slot of 64 keys at a time,
    // not unrolled, so that this path does not set the register count of
    // every launch that inlines it; ranks come from buf only, so each
    // slot's keys can be placed before the next slot is ranked
#pragma unroll 1
    for (uint32_t s0 = 0; s0 < c; s0 += kWave) {
      const uint32_t i = s0 + lane;
      const uint64_t mine = i < c ? w.buf[i] : 0ull;
      uint32_t rank = i < ntop ? i : (i < c ? (uint32_t)count_greater(w.buf, (int)ntop, mine) : 0xFFFFu);
      for (uint32_t j = ntop; j < c; ++j) rank += (w.buf[j] > mine) ? 1u : 0u;
      if (mine != 0ull && rank < (uint32_t)K) w.top[rank] = mine;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
  if (lane == 0) w.ntop = min(c, (uint32_t)K);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

// bf16 element of sub-segment [lo, hi) held by `lane` in slot s (0..63):
// load j = s / 8, position e = s % 8, index lo + (j * 64 + lane) * 8 + e
__device__ __forceinline__ int slot_index_bf16(int lo, int lane, int s) {
  return lo + ((s >> 3) * kWave + lane) * 8 + (s & 7);
}

// Exact top-K of one sub-segment whose threshold admits too many values
// (long runs of equal values).  Re-reads the sub-segment on every bisection
// step, one slot at a time (the slot loops stay rolled: unrolled, the
// compiler hoists every slot's load out of the bisection and this rare path
// would set the register count of the launches that call it); appends K
// keys to the buffer after its first `base` entries.
template <int DT>
__device__ __noinline__ void exact_subsegment(const void* row_ptr, int lo, int hi, int K, int lane,
                                              TkWave& w, uint32_t base) {
  constexpr int NS = DT == DFLASH_BF16 ? 64 : 32;
  constexpr int VBITS = DT == DFLASH_BF16 ? 16 : 32;
  // canonical value key (-0 folded onto +0) of slot s, 0 outside [lo, hi)
  auto cv = [&](int s, int& idx) -> uint32_t {
    if (DT == DFLASH_BF16) {
      idx = slot_index_bf16(lo, lane, s);
      if (idx >= hi) return 0u;
      const uint32_t b = reinterpret_cast<const uint16_t*>(row_ptr)[idx];
      const uint32_t k = ord16x2(b) & 0xFFFFu;
      return k == 0x7FFFu ? 0x8000u : k;
    } else {
      idx = lo + ((s >> 2) * kWave + lane) * 4 + (s & 3);
      if (idx >= hi) return 0u;
      return ord32_canon(reinterpret_cast<const uint32_t*>(row_ptr)[idx]);
    }
  };
  uint32_t tv = 0;
  for (int bit = VBITS - 1; bit >= 0; --bit) {
    const uint32_t c = tv | (1u << bit);
    uint32_t n = 0;
#pragma unroll 1
    for (int s = 0; s < NS; ++s) {
      int idx;
      n += (cv(s, idx) >= c) ? 1u : 0u;
    }
    if (wave_sum_u32(n) >= (uint32_t)K) tv = c;
  }
  uint32_t gt = 0;
#pragma unroll 1
  for (int s = 0; s < NS; ++s) {
    int idx;
    gt += (cv(s, idx) > tv) ? 1u : 0u;
  }
  gt = wave_sum_u32(gt);
  const uint32_t need = (uint32_t)K > gt ? (uint32_t)K - gt : 0u;
  // smallest index x with #(value == tv, index <= x) >= need
  int xlo = lo, xhi = hi - 1;
  while (xlo < xhi) {
    const int mid = (xlo + xhi) >> 1;
    uint32_t n = 0;
#pragma unroll 1
    for (int s = 0; s < NS; ++s) {
      int idx;
      n += (cv(s, idx) == tv && idx <= mid) ? 1u : 0u;
    }
    if (wave_sum_u32(n) >= need) xhi = mid; else xlo = mid + 1;
  }
  if (lane == 0) w.cnt = base;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll 1
  for (int s = 0; s < NS; ++s) {
    int idx;
    const uint32_t v = cv(s, idx);
    if (v != 0u && (v > tv || (v == tv && need > 0 && idx <= xlo))) {
      const uint32_t ord = DT == DFLASH_BF16 ? ord32_of_k16(v) : v;
      const uint32_t pos = atomicAdd(&w.cnt, 1u);
      if (pos < (uint32_t)kTopkCap) w.buf[pos] = make_key(ord, (uint32_t)idx);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

__device__ __forceinline__ uint32_t max_i16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, a),
                                                                __builtin_bit_cast(s16x2, b)));
}

// number of set bits of ballot b held by lanes below this one
__device__ __forceinline__ uint32_t lanes_below(uint64_t b) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
}

// Append `key` from every lane where `hit` holds, after the first `cnt`
// buffer entries (cnt is the same in every lane): a lane's slot is the
// number of hitting lanes below it, so no atomic and no round trip.
__device__ __forceinline__ void append_hits(bool hit, uint64_t key, TkWave& w, uint32_t& cnt) {
  const uint64_t b = __ballot(hit);
  if (hit) {
    const uint32_t pos = cnt + lanes_below(b);
    if (pos < (uint32_t)kTopkCap) w.buf[pos] = key;
  }
  cnt += (uint32_t)__popcll(b);
}

// bf16 candidates are buffered as 32-bit compact keys: the 16-bit ordered
// key (-0.0 folded onto +0.0) in the high half, 0xFFFE minus the value's
// offset in its sub-segment (< 4096) in the low half.  Within a sub-segment
// the compact order is the key order (value desc, index asc).  A running
// key (from an earlier sub-segment, so a smaller index) is written as its
// 16-bit head with low half 0xFFFF: it beats every compact key of equal
// value and no compact key equals it.

// Append the hits of one register (its low and high bf16 value) as compact
// keys after the first `cnt` entries of cb.  cnt is wave-uniform; a lane's
// slot is the number of hitting lanes below it.  Past the capacity nothing
// is written but cnt still counts, which sends the fold to the exact path.
__device__ __forceinline__ void append2_compact(bool hlo, bool hhi, uint32_t key_lo, uint32_t key_hi,
                                                uint32_t* cb, uint32_t& cnt) {
  const uint64_t blo = __ballot(hlo), bhi = __ballot(hhi);
  const uint32_t nlo = (uint32_t)__popcll(blo);
  const uint32_t n = nlo + (uint32_t)__popcll(bhi);
  if (cnt + n <= (uint32_t)kTopkCap) {
    if (hlo) cb[cnt + lanes_below(blo)] = key_lo;
    if (hhi) cb[cnt + nlo + lanes_below(bhi)] = key_hi;
  }
  cnt += n;
}

// Merge the compact buffer cb[0, c) (running heads, then new keys) into the
// running list; lo is the sub-segment's first index.  c > kWave (rare)
// widens the keys into the 64-bit buffer and takes the general merge.
__device__ void merge_compact_bf16(TkWave& w, uint32_t c, int K, int lane, int lo) {
  const uint32_t ntop = w.ntop;
  if (c == ntop) return;  // nothing new
  const uint32_t* cb = reinterpret_cast<const uint32_t*>(w.buf);
  auto widen = [&](uint32_t ck) -> uint64_t {
    return make_key(ord32_of_k16(ck >> 16), (uint32_t)lo + (0xFFFEu - (ck & 0xFFFFu)));
  };
  if (c <= (uint32_t)kWave) {
    const uint32_t mine = lane < (int)c ? cb[lane] : 0u;
    const uint64_t run = lane < (int)ntop ? w.top[lane] : 0ull;
    // a running key counts only the new keys above it (running heads of
    // equal value must not count each other); a new key counts all
    const uint32_t j_first = lane < (int)ntop ? ntop : 0u;
    uint32_t rank = lane < (int)ntop ? (uint32_t)lane : 0u;
    for (uint32_t j0 = 0; j0 < c; j0 += 16) {
      uint32_t o[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) o[u] = cb[j0 + u];
#pragma unroll
      for (int u = 0; u < 16; ++u) rank += (j0 + u >= j_first && j0 + u < c && o[u] > mine) ? 1u : 0u;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (lane < (int)c && rank < (uint32_t)K) w.top[rank] = lane < (int)ntop ? run : widen(mine);
    if (lane == 0) w.ntop = min(c, (uint32_t)K);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  } else {
    // every lane reads its (up to kTopkCap / kWave) keys before any lane
    // writes the widened ones over the same LDS
    constexpr int SL = kTopkCap / kWave;
    uint32_t ck[SL];
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const uint32_t i = lane + s * kWave;
      ck[s] = i < c ? cb[i] : 0u;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const uint32_t i = lane + s * kWave;
      if (i < c) w.buf[i] = i < ntop ? w.top[i] : widen(ck[s]);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    merge_buffer(w, c, K, lane);
  }
}

// Fold bf16 sub-segment [lo, hi) of `row` into the wave's running list.
// Registers keep the raw patterns.  A packed signed 16-bit max picks one
// actual value per lane (the lane maximum whenever the lane holds a
// non-negative value); the K-th largest of those picks is a valid
// threshold.  When the threshold is positive, a raw pattern passes exactly
// when it is >= the threshold's pattern as a signed 16-bit integer, and
// its ordered key is the pattern with the sign bit set, so neither the test
// nor the compact key needs a key transform.
//
// The fold runs in two steps so that a block can share its first
// thresholds before any wave scans: fold_bf16_load fills the registers and
// returns the wave's own threshold key (the running list's K-th key + 1, or
// the K-th largest pick); fold_bf16_scan raises it to the block bound, then
// buffers and merges the candidates.
__device__ __forceinline__ void load_sub_bf16(const uint16_t* __restrict__ row, int lo, int hi, int lane,
                                              uint32_t (&x)[4 * kTopkLoads]) {
  // 16-byte units lie wholly inside or outside [lo, hi) (row lengths are
  // multiples of 8 values); units past hi hold 0xFFFF pairs (key 0: never
  // admitted, and a lane whose pick is padding adds nothing to the count)
#pragma unroll
  for (int j = 0; j < kTopkLoads; ++j) {
    const int base = lo + (j * kWave + lane) * 8;
    uint4 v = make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu);
    if (base < hi) v = load_stream16(row + base);
    x[4 * j + 0] = v.x;
    x[4 * j + 1] = v.y;
    x[4 * j + 2] = v.z;
    x[4 * j + 3] = v.w;
  }
}

// the wave's threshold key for the sub-segment held in x (see above)
__device__ __forceinline__ uint32_t sub_threshold_bf16(int K, const TkWave& w, const uint32_t (&x)[4 * kTopkLoads]) {
  const uint32_t ntop = __builtin_amdgcn_readfirstlane(w.ntop);
  uint32_t thr;
  if (ntop == (uint32_t)K) {
    thr = (uint32_t)(w.top[K - 1] >> 48) + 1u;
  } else {
    uint32_t m = x[0];
#pragma unroll
    for (int q = 1; q < 4 * kTopkLoads; ++q) m = max_i16x2(m, x[q]);
    const int pick = max((int)(int16_t)(m & 0xFFFFu), (int)(int16_t)(m >> 16));
    const uint32_t pick_key = ord16x2((uint32_t)pick & 0xFFFFu) & 0xFFFFu;
    // K-th largest pick
    thr = 0;
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t c = thr | (1u << bit);
      if (__popcll(__ballot(pick_key >= c)) >= (unsigned)K) thr = c;
    }
    if (thr == 0x8000u) thr = 0x7FFFu;  // a +0.0 threshold also admits -0.0
    if (thr == 0u) thr = 1u;            // never admit padding
  }
  return thr;
}

__device__ __forceinline__ uint32_t fold_bf16_load(const uint16_t* __restrict__ row, int lo, int hi, int K,
                                                   const TkWave& w, int lane, uint32_t (&x)[4 * kTopkLoads]) {
  load_sub_bf16(row, lo, hi, lane, x);
  return sub_threshold_bf16(K, w, x);
}

__device__ __forceinline__ void fold_bf16_scan(const uint16_t* __restrict__ row, int lo, int hi, int K, TkWave& w,
                                               int lane, uint32_t* bbound, const uint32_t (&x)[4 * kTopkLoads],
                                               uint32_t thr) {
  const uint32_t ntop = __builtin_amdgcn_readfirstlane(w.ntop);
  uint32_t sb = *bbound;                // 16-bit key of the block bound
  if (sb == 0x8000u) sb = 0x7FFFu;      // a +0.0 bound also admits -0.0
  thr = __builtin_amdgcn_readfirstlane(max(thr, sb));

  // compact buffer = running heads, then the new candidates; a register is
  // looked at closely only when some lane's register passes the packed test
  uint32_t* cb = reinterpret_cast<uint32_t*>(w.buf);
  if (lane < (int)ntop) cb[lane] = ((uint32_t)(w.top[lane] >> 48) << 16) | 0xFFFFu;
  uint32_t cnt = ntop;
  // low half of the compact key of the lane's first value in each register
  // group: 0xFFFE - lane * 8, minus the register's constant offset below.
  // Opaque to the optimiser: otherwise the 32 per-register values are
  // hoisted out of the caller's sub-segment loop and held in registers
  uint32_t lane_lo = 0xFFFEu - (uint32_t)lane * 8u;
  asm volatile("" : "+v"(lane_lo));
  if (thr > 0x8000u && thr <= 0xFFFFu) {
    const int tp = (int)(thr & 0x7FFFu);  // positive threshold pattern
    const uint32_t tm1 = (uint32_t)(tp - 1) * 0x00010001u;
    const uint32_t pos_lo = 0x80000000u | lane_lo;  // sign bit of a positive key
#pragma unroll
    for (int q = 0; q < 4 * kTopkLoads; ++q) {
      if (__ballot(max_i16x2(x[q], tm1) != tm1)) {
        const uint32_t low = pos_lo - (uint32_t)((q >> 2) * kWave * 8 + (q & 3) * 2);
        append2_compact((int)(int16_t)(x[q] & 0xFFFFu) >= tp, (int)x[q] >> 16 >= tp, (x[q] << 16) | low,
                        (x[q] & 0xFFFF0000u) | (low - 1u), cb, cnt);
      }
    }
  } else if (thr <= 0xFFFFu) {
    const uint32_t tm1 = (thr - 1u) * 0x00010001u;
#pragma unroll
    for (int q = 0; q < 4 * kTopkLoads; ++q) {
      const uint32_t k2 = ord16x2(x[q]);
      if (__ballot(subsat_u16x2(k2, tm1) != 0u)) {
        uint32_t klo = k2 & 0xFFFFu, khi = k2 >> 16;
        klo = klo == 0x7FFFu ? 0x8000u : klo;
        khi = khi == 0x7FFFu ? 0x8000u : khi;
        const uint32_t low = lane_lo - (uint32_t)((q >> 2) * kWave * 8 + (q & 3) * 2);
        append2_compact(klo >= thr, khi >= thr, (klo << 16) | low, (khi << 16) | (low - 1u), cb, cnt);
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  if (cnt > (uint32_t)kTopkCap) {
    // too many candidates: the 64-bit buffer gets the running list back and
    // the exact path appends the sub-segment's own top K
    if (lane < (int)ntop) w.buf[lane] = w.top[lane];
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    exact_subsegment<DFLASH_BF16>(row, lo, hi, K, lane, w, ntop);
    merge_buffer(w, w.cnt, K, lane);
  } else {
    merge_compact_bf16(w, cnt, K, lane, lo);
  }
  if (lane == 0 && w.ntop == (uint32_t)K) atomicMax(bbound, (uint32_t)(w.top[K - 1] >> 48));
}

// fold fp32 sub-segment [lo, hi) of `row` into the wave's running list
__device__ void wave_fold_f32(const uint32_t* __restrict__ row, int lo, int hi, int K, TkWave& w, int lane,
                              uint32_t* bbound) {
  // units past hi hold key 0 (never admitted)
  uint32_t kx[4 * kTopkLoads];
#pragma unroll
  for (int j = 0; j < kTopkLoads; ++j) {
    const int base = lo + (j * kWave + lane) * 4;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (base < hi) {
      v = load_stream16(row + base);
      v = make_uint4(ord32(v.x), ord32(v.y), ord32(v.z), ord32(v.w));
    }
    kx[4 * j + 0] = v.x;
    kx[4 * j + 1] = v.y;
    kx[4 * j + 2] = v.z;
    kx[4 * j + 3] = v.w;
  }
  const uint32_t ntop = w.ntop;
  uint32_t thr;
  bool none = false;
  if (ntop == (uint32_t)K) {
    const uint32_t t = (uint32_t)(w.top[K - 1] >> 32);
    if (t == 0xFFFFFFFFu) none = true;
    thr = t + 1u;
  } else {
    uint32_t lanemax = kx[0];
#pragma unroll
    for (int q = 1; q < 4 * kTopkLoads; ++q) lanemax = max(lanemax, kx[q]);
    thr = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = thr | (1u << bit);
      if (__popcll(__ballot(lanemax >= c)) >= (unsigned)K) thr = c;
    }
    if (thr == 0x80000000u) thr = 0x7FFFFFFFu;
    if (thr == 0u) thr = 1u;
  }
  uint32_t sb = *bbound;                   // 32-bit key of the block bound
  if (sb == 0x80000000u) sb = 0x7FFFFFFFu;  // a +0.0 bound also admits -0.0
  thr = max(thr, sb);
  if (lane < (int)ntop) w.buf[lane] = w.top[lane];
  uint32_t cnt = ntop;
  if (!none) {
#pragma unroll
    for (int q = 0; q < 4 * kTopkLoads; ++q) {
      if (__ballot(kx[q] >= thr)) {
        const uint32_t canon = kx[q] == 0x7FFFFFFFu ? 0x80000000u : kx[q];
        const int idx = lo + ((q >> 2) * kWave + lane) * 4 + (q & 3);
        append_hits(kx[q] >= thr, make_key(canon, (uint32_t)idx), w, cnt);
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  if (cnt > (uint32_t)kTopkCap) {
    exact_subsegment<DFLASH_F32>(row, lo, hi, K, lane, w, ntop);
    cnt = w.cnt;
  }
  merge_buffer(w, cnt, K, lane);
  if (lane == 0 && w.ntop == (uint32_t)K) atomicMax(bbound, (uint32_t)(w.top[K - 1] >> 32));
}


// The sorted top list (16 keys, zero-padded) of sub-segments
// [seg * spb, min((seg + 1) * spb, n_sub)) of drafter row `row`, computed by
// a 256-thread block and written to `out16` (global), or, when `out_tag` is
// set, to out_tag as 16 hand-off pairs (key, check | tag) for readers in the
// same launch.  `sw` is LDS for 4 waves, `block_top` 16 LDS keys.
template <int DT>
__device__ __forceinline__ void topk_block(const void* __restrict__ U, int V, int K, int n_sub, int spb, int row,
                                           int seg, TkWave* sw, uint64_t* block_top, uint32_t* bbound,
                                           uint64_t* __restrict__ out16, uint64_t* __restrict__ out_tag = nullptr,
                                           uint32_t tag = 0) {
  constexpr int WS = 64 * kTopkLoads * (DT == DFLASH_BF16 ? 8 : 4);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  TkWave& w = sw[wave];
  if (lane < 16) w.top[lane] = 0ull;
  if (lane == 0) w.ntop = 0;
  if (tid == 0) *bbound = 0u;
  __syncthreads();
  const int s1 = min((seg + 1) * spb, n_sub);
  if (DT == DFLASH_BF16) {
    // first sub-segments: every wave publishes its own threshold before any
    // wave scans, so each scans against the largest of the four (any wave's
    // K-th largest pick bounds the block's K-th value from below)
    const uint16_t* rp = reinterpret_cast<const uint16_t*>(U) + (size_t)row * V;
    uint32_t x[4 * kTopkLoads];
    const int s0 = seg * spb + wave;
    uint32_t thr = 0;
    if (s0 < s1) {
      thr = fold_bf16_load(rp, s0 * WS, min(s0 * WS + WS, V), K, w, lane, x);
      if (lane == 0) atomicMax(bbound, thr);
    }
    __syncthreads();
    if (s0 < s1) fold_bf16_scan(rp, s0 * WS, min(s0 * WS + WS, V), K, w, lane, bbound, x, thr);
    for (int s = s0 + 4; s < s1; s += 4) {
      const int lo = s * WS, hi = min(lo + WS, V);
      thr = fold_bf16_load(rp, lo, hi, K, w, lane, x);
      fold_bf16_scan(rp, lo, hi, K, w, lane, bbound, x, thr);
    }
  } else {
    for (int s = seg * spb + wave; s < s1; s += 4) {
      const int lo = s * WS, hi = min(lo + WS, V);
      wave_fold_f32(reinterpret_cast<const uint32_t*>(U) + (size_t)row * V, lo, hi, K, w, lane, bbound);
    }
  }
  if (tid < 16) block_top[tid] = 0ull;
  __syncthreads();
  // merge the four sorted wave lists: one key per thread of the first 64
  if (tid < 64) {
    const int lw = tid >> 4, k = tid & 15;
    const uint64_t key = sw[lw].top[k];
    if (key != 0ull && k < K) {
      int rank = k;
#pragma unroll
      for (int o = 0; o < 4; ++o)
        if (o != lw) rank += count_greater16(sw[o].top, key);
      if (rank < K) block_top[rank] = key;
    }
  }
  __syncthreads();
  if (tid < 16) {
    if (out_tag) handoff_store_pair(out_tag + 2 * tid, block_top[tid], tag);
    else out16[tid] = block_top[tid];
  }
}

// Merge the n_seg sorted lists of one row (global, 16 keys each) into the
// row's sorted top-K keys `out` (LDS, K entries), using `keys` (LDS, at
// least n_seg * 16 entries) as staging.  Every thread of the block takes
// part; ends with a barrier.
__device__ __forceinline__ void merge_row(const uint64_t* __restrict__ lists, int n_seg, int K, uint64_t* keys,
                                          uint64_t* out) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int nk = n_seg * 16;
  for (int i = tid; i < nk; i += nt) keys[i] = lists[i];
  __syncthreads();
  for (int i = tid; i < nk; i += nt) {
    const int s = i >> 4, k = i & 15;
    const uint64_t key = keys[i];
    if (key == 0ull || k >= K) continue;
    int rank = k;
    for (int s2 = 0; s2 < n_seg && rank < K; ++s2)
      if (s2 != s) rank += count_greater16(keys + s2 * 16, key);
    if (rank < K) out[rank] = key;
  }
  __syncthreads();
}

// Merge the sorted lists of two rows, staged in `keys` (LDS, barrier
// passed: n_seg lists of 16 keys of row r0, then n_seg lists of row r1;
// zeros for an absent row), into out0 / out1 (LDS, K entries each) in one
// pass: each key's rank is its position in its own list plus the count of
// greater keys in the row's other lists.  Every thread of the block takes
// part; ends with a barrier.
// The other lists are searched G at a time (G = 8, or 16 when a row has
// more than 8 lists: merge_wide), each group's searches advanced level by
// level so that a level's G loads are in flight together.
__host__ __device__ constexpr bool merge_wide(int n_seg) { return n_seg > 8; }

template <bool WIDE>
__device__ __forceinline__ void merge_two_staged(const uint64_t* keys, int n_seg, int K, uint64_t* out0,
                                                 uint64_t* out1) {
  constexpr int G = WIDE ? 16 : 8;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int nk = n_seg * 16;
  for (int i = tid; i < 2 * nk; i += nt) {
    const int half = i >= nk, j = i - half * nk;
    const int s = j >> 4, k = j & 15;
    const uint64_t key = keys[i];
    if (key == 0ull || k >= K) continue;
    const uint64_t* base = keys + half * nk;
    int rank = k;
    for (int g0 = 0; g0 < n_seg; g0 += G) {
      const uint64_t* lp[G];
      int lo[G];
      bool l15[G];
#pragma unroll
      for (int q = 0; q < G; ++q) {
        lp[q] = base + min(g0 + q, n_seg - 1) * 16;
        l15[q] = lp[q][15] > key;
        lo[q] = lp[q][7] > key ? 8 : 0;
      }
#pragma unroll
      for (int q = 0; q < G; ++q) lo[q] += lp[q][lo[q] + 3] > key ? 4 : 0;
#pragma unroll
      for (int q = 0; q < G; ++q) lo[q] += lp[q][lo[q] + 1] > key ? 2 : 0;
#pragma unroll
      for (int q = 0; q < G; ++q) lo[q] += lp[q][lo[q]] > key ? 1 : 0;
#pragma unroll
      for (int q = 0; q < G; ++q) {
        const int s2 = g0 + q;
        if (s2 < n_seg && s2 != s) rank += lo[q] == 15 && l15[q] ? 16 : lo[q];
      }
    }
    if (rank < K) (half ? out1 : out0)[rank] = key;
  }
  __syncthreads();
}

__device__ __forceinline__ int key_index(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }
__device__ __forceinline__ float key_value(uint64_t key) { return __uint_as_float(unord32((uint32_t)(key >> 32))); }

}  // namespace dfk
