// C ABI of libdflash.so: host-side validation, workspace layout and the
// launch sequence of every entry point declared in include/dflash.h.
// Nothing here allocates device memory; all work goes to the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "dflash.h"
#include "internal.hpp"

namespace {

thread_local std::string g_err;

dflash_status fail(dflash_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t logit_bytes(int32_t dt) { return dt == DFLASH_BF16 ? 2 : 4; }

dflash_status check_dims(const dflash_dims* d) {
  if (!d) return fail(DFLASH_ERR_INVALID_ARG, "dims is NULL");
  if (d->B < 1) return fail(DFLASH_ERR_INVALID_ARG, "B must be >= 1");
  if (d->L < 1 || d->L > DFLASH_L_MAX) return fail(DFLASH_ERR_INVALID_ARG, "L must be in [1, 16]");
  if (d->K < 1 || d->K > DFLASH_K_MAX) return fail(DFLASH_ERR_INVALID_ARG, "K must be in [1, 16]");
  if (d->V < d->K) return fail(DFLASH_ERR_INVALID_ARG, "V must be >= K");
  if (d->V > DFLASH_V_MAX) return fail(DFLASH_ERR_UNSUPPORTED, "V above DFLASH_V_MAX");
  if (d->r < 16 || d->r > DFLASH_R_MAX || d->r % 16) return fail(DFLASH_ERR_INVALID_ARG, "r must be a multiple of 16 in [16, 256]");
  if (d->hidden < 16 || d->hidden % 16) return fail(DFLASH_ERR_INVALID_ARG, "hidden must be a positive multiple of 16");
  if (d->logit_dtype != DFLASH_F32 && d->logit_dtype != DFLASH_BF16) return fail(DFLASH_ERR_INVALID_ARG, "unknown logit_dtype");
  if (d->param_dtype != DFLASH_F32 && d->param_dtype != DFLASH_BF16) return fail(DFLASH_ERR_INVALID_ARG, "unknown param_dtype");
  if (((size_t)d->V * logit_bytes(d->logit_dtype)) % 16)
    return fail(DFLASH_ERR_UNSUPPORTED, "a logit row must span a multiple of 16 bytes (V % 8 for bf16, V % 4 for fp32)");
  const long long rows = (long long)d->B * (d->L + 1);
  if (rows > 65535) return fail(DFLASH_ERR_UNSUPPORTED, "B * (L + 1) must not exceed 65535");
  return DFLASH_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Ptr {
  const void* p;
  const char* name;
  bool need16;
};

dflash_status check_ptrs(std::initializer_list<Ptr> ps) {
  for (const Ptr& p : ps) {
    if (!p.p) return fail(DFLASH_ERR_INVALID_ARG, std::string(p.name) + " is NULL");
    if (p.need16 && !aligned16(p.p)) return fail(DFLASH_ERR_INVALID_ARG, std::string(p.name) + " is not 16-byte aligned");
  }
  return DFLASH_OK;
}

dflash_status check_ws(const dfk::WsLayout& w, void* ws, size_t ws_bytes) {
  if (!ws) return fail(DFLASH_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(ws)) return fail(DFLASH_ERR_WORKSPACE, "workspace is not 16-byte aligned");
  if (ws_bytes < w.total)
    return fail(DFLASH_ERR_WORKSPACE, "workspace too small: need " + std::to_string(w.total) + " bytes");
  return DFLASH_OK;
}

// ---------------------------------------------------------------- timer

struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending[DFLASH_KERNEL_COUNT];
  std::vector<hipEvent_t> pool;

  hipEvent_t take() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

Profiler& prof() {
  static Profiler* p = new Profiler();
  return *p;
}

// Run `f` (which enqueues on `st`), timed when the timer is on.  Entry
// points of a single launch hand the events to that launch, which records
// them at the kernel's own start and end; the two-launch top-K entry point
// brackets its launches with events on the stream.
template <class F>
hipError_t timed(int kernel, hipStream_t st, F f) {
  Profiler& P = prof();
  hipEvent_t a = nullptr, b = nullptr;
  {
    std::lock_guard<std::mutex> lk(P.mu);
    if (P.on) {
      a = P.take();
      b = P.take();
    }
  }
  const bool on_stream = kernel == DFLASH_KERNEL_TOPK;
  if (a && b) {
    if (on_stream) {
      hipEventRecord(a, st);
    } else {
      dfk::g_launch_start = a;
      dfk::g_launch_stop = b;
    }
  }
  const hipError_t e = f();
  const bool launched = !(dfk::g_launch_start || dfk::g_launch_stop);
  dfk::g_launch_start = dfk::g_launch_stop = nullptr;
  if (a && b) {
    if (on_stream) hipEventRecord(b, st);
    std::lock_guard<std::mutex> lk(P.mu);
    if (e == hipSuccess && launched) {
      P.pending[kernel].push_back({a, b});
    } else {
      P.pool.push_back(a);
      P.pool.push_back(b);
    }
  }
  return e;
}

dflash_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DFLASH_OK;
  return fail(DFLASH_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

namespace dfk {

thread_local hipEvent_t g_launch_start = nullptr, g_launch_stop = nullptr;

// Sub-segments per top-K block: by default the smallest multiple of 4 that
// keeps the top-K part of the grid at or below 2048 blocks; raised so that
// a row has at most 8 partial lists when the top-K part still has 512 or
// more blocks (the scores launch searches more than 8 lists 16 at a time,
// about 2.5 us more at 151936 tokens, which outweighs the longer top-K
// blocks once the grid is that large: +5% cycles/s at 4 and 5 drafted
// positions of 32 streams, -6% at one stream); at least enough that a row
// has at most kTopkMaxSeg blocks.  DFLASH_TOPK_SPB overrides the default
// for tuning sweeps.
static int topk_spb(size_t rows, int n_sub) {
  static const int env = [] {
    const char* s = std::getenv("DFLASH_TOPK_SPB");
    return s ? std::atoi(s) : 0;
  }();
  int spb = 4;
  if (env > 0) {
    spb = env;
  } else {
    while (spb < n_sub && rows * (size_t)((n_sub + spb - 1) / spb) > 2048) spb += 4;
    const int spb8 = ((n_sub + 7) / 8 + 3) / 4 * 4;
    if (spb < spb8 && rows * (size_t)((n_sub + spb8 - 1) / spb8) >= 512) spb = spb8;
  }
  const int min_spb = (n_sub + kTopkMaxSeg - 1) / kTopkMaxSeg;
  return spb < min_spb ? min_spb : spb;
}

WsLayout ws_layout(const dflash_dims& d) {
  WsLayout w{};
  const size_t R = (size_t)d.B * d.L;
  const int we = topk_wave_elems(d.logit_dtype);
  w.n_sub = (d.V + we - 1) / we;
  w.spb = topk_spb(R, w.n_sub);
  w.n_seg = (w.n_sub + w.spb - 1) / w.spb;
  w.n_chunk = (d.V + kChunk - 1) / kChunk;
  size_t o = 0;
  w.epoch = o;        o = align256(o + sizeof(uint32_t));
  w.topk_partial = o; o = align256(o + R * w.n_seg * 16 * sizeof(uint64_t));
  w.gate = o;         o = align256(o + (size_t)gate_groups(d) * R * d.r * sizeof(float));
  w.cand_idx = o;     o = align256(o + R * d.K * sizeof(int32_t));
  w.cand_logit = o;   o = align256(o + R * d.K * sizeof(float));
  w.zc = o;           o = align256(o + R * d.K * sizeof(float));
  w.S = o;            o = align256(o + R * d.K * d.K * sizeof(float));
  w.path_rank = o;    o = align256(o + R * sizeof(int32_t));
  w.draft_tok = o;    o = align256(o + R * sizeof(int32_t));
  w.q = o;            o = align256(o + R * d.K * sizeof(float));
  w.stats = o;        o = align256(o + (size_t)d.B * (d.L + 1) * w.n_chunk * sizeof(ChunkStat));
  w.jstar = o;        o = align256(o + R * d.K * sizeof(int32_t));
  w.qtab = o;         o = align256(o + R * d.K * d.K * sizeof(float));
  w.edges = (long long)R * w.n_seg + stream_gate_blocks(d) + (long long)R <= kResidentBlocks;
  if (w.edges) {
    w.tk_tag = o;     o = align256(o + R * w.n_seg * 16 * 2 * sizeof(uint64_t));
    w.gate_tag = o;   o = align256(o + (size_t)gate_groups(d) * R * d.r * sizeof(uint64_t));
  }
  w.cycle_total = o;
  w.gate_q = o;       o = align256(o + (size_t)gate_groups(d) * (d.param_dtype == DFLASH_BF16 ? 4 : 1) * R * d.r *
                                         sizeof(float));
  w.total = o;
  return w;
}

}  // namespace dfk

extern "C" {

int32_t dflash_abi_version(void) { return DFLASH_ABI_VERSION; }

const char* dflash_status_string(dflash_status s) {
  switch (s) {
    case DFLASH_OK: return "DFLASH_OK";
    case DFLASH_ERR_INVALID_ARG: return "DFLASH_ERR_INVALID_ARG";
    case DFLASH_ERR_UNSUPPORTED: return "DFLASH_ERR_UNSUPPORTED";
    case DFLASH_ERR_WORKSPACE: return "DFLASH_ERR_WORKSPACE";
    case DFLASH_ERR_HIP: return "DFLASH_ERR_HIP";
    default: return "DFLASH_ERR_UNKNOWN";
  }
}

const char* dflash_last_error(void) { return g_err.c_str(); }

dflash_status dflash_workspace_bytes(const dflash_dims* d, size_t* bytes) {
  try {
    g_err.clear();
    if (dflash_status s = check_dims(d)) return s;
    if (!bytes) return fail(DFLASH_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = dfk::ws_layout(*d).total;
    return DFLASH_OK;
  } catch (...) {
    return fail(DFLASH_ERR_INVALID_ARG, "internal error");
  }
}

dflash_status dflash_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  try {
    g_err.clear();
    if (!ws) return fail(DFLASH_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned16(ws)) return fail(DFLASH_ERR_WORKSPACE, "workspace is not 16-byte aligned");
    if (ws_bytes == 0) return DFLASH_OK;
    return hip_status(dfk::launch_fill_zero(ws, ws_bytes, (hipStream_t)stream), "workspace fill");
  } catch (...) {
    return fail(DFLASH_ERR_HIP, "internal error");
  }
}

dflash_status dflash_topk(const dflash_dims* d, const void* U, int32_t* cand_idx, float* cand_logit,
                          void* ws, size_t ws_bytes, void* stream) {
  try {
    g_err.clear();
    if (dflash_status s = check_dims(d)) return s;
    if (dflash_status s = check_ptrs({{U, "U", true}, {cand_idx, "cand_idx", false}, {cand_logit, "cand_logit", false}})) return s;
    const dfk::WsLayout w = dfk::ws_layout(*d);
    if (dflash_status s = check_ws(w, ws, ws_bytes)) return s;
    hipStream_t st = (hipStream_t)stream;
    return hip_status(timed(DFLASH_KERNEL_TOPK, st, [&] {
      return dfk::launch_topk(*d, w, U, cand_idx, cand_logit, static_cast<char*>(ws), st);
    }), "topk launch");
  } catch (...) {
    return fail(DFLASH_ERR_HIP, "internal error");
  }
}

dflash_status dflash_pair_scores(const dflash_dims* d, const int32_t* x0, const int32_t* cand_idx,
                                 const float* cand_logit, const void* E, const void* W_g, const void* h,
                                 float* S, void* ws, size_t ws_bytes, void* stream) {
  try {
    g_err.clear();
    if (dflash_status s = check_dims(d)) return s;
    if (dflash_status s = check_ptrs({{x0, "x0", false}, {cand_idx, "cand_idx", false}, {cand_logit, "cand_logit", false},
                                      {E, "E", true}, {W_g, "W_g", true}, {h, "h", true}, {S, "S", false}})) return s;
    const dfk::WsLayout w = dfk::ws_layout(*d);
    if (dflash_status s = check_ws(w, ws, ws_bytes)) return s;
    hipStream_t st = (hipStream_t)stream;
    float* g = reinterpret_cast<float*>(static_cast<char*>(ws) + w.gate_q);
    if (dflash_status s = hip_status(timed(DFLASH_KERNEL_GATE, st, [&] { return dfk::launch_gate(*d, h, W_g, g, st); }), "gate launch")) return s;
    return hip_status(timed(DFLASH_KERNEL_SCORES, st, [&] {
      return dfk::launch_scores(*d, x0, cand_idx, cand_logit, E, g, S, st);
    }), "scores launch");
  } catch (...) {
    return fail(DFLASH_ERR_HIP, "internal error");
  }
}

dflash_status dflash_trace(const dflash_dims* d, const float* S, const int32_t* cand_idx, const float* T,
                           const uint64_t* seed, uint64_t cycle, int32_t* path_rank, int32_t* draft_tok,
                           float* q, void* stream) {
  try {
    g_err.clear();
    if (dflash_status s = check_dims(d)) return s;
    if (dflash_status s = check_ptrs({{S, "S", false}, {cand_idx, "cand_idx", false}, {T, "T", false}, {seed, "seed", false},
                                      {path_rank, "path_rank", false}, {draft_tok, "draft_tok", false}, {q, "q", false}})) return s;
    hipStream_t st = (hipStream_t)stream;
    return hip_status(timed(DFLASH_KERNEL_TRACE, st, [&] {
      return dfk::launch_trace(*d, S, cand_idx, T, seed, cycle, path_rank, draft_tok, q, st);
    }), "trace launch");
  } catch (...) {
    return fail(DFLASH_ERR_HIP, "internal error");
  }
}

dflash_status dflash_topk_merge(const dflash_dims* d, int32_t n_shards, const int32_t* shard_begin,
                                const int32_t* cand_idx_parts, const float* cand_logit_parts, int32_t* cand_idx,
                                float* cand_logit, void* stream) {
  try {
    g_err.clear();
    if (dflash_status s = check_dims(d)) return s;
    if (n_shards < 1 || n_shards > DFLASH_MAX_SHARDS)
      return fail(DFLASH_ERR_INVALID_ARG, "n_shards must be in 1 .. DFLASH_MAX_SHARDS");
    if (!shard_begin) return fail(DFLASH_ERR_INVALID_ARG, "shard_begin is NULL");
    if (dflash_status s = check_ptrs({{cand_idx_parts, "cand_idx_parts", false},
                                      {cand_logit_parts, "cand_logit_parts", false},
                                      {cand_idx, "cand_idx", false}, {cand_logit, "cand_logit", false}})) return s;
    dfk::ShardBegins sb{};
    for (int s = 0; s < n_shards; ++s) {
      const int64_t lo = shard_begin[s], hi = s + 1 < n_shards ? shard_begin[s + 1] : d->V;
      if ((s == 0 && lo != 0) || hi - lo < d->K || hi > d->V)
        return fail(DFLASH_ERR_INVALID_ARG, "shards must start at 0, increase, and be at least K tokens wide");
      sb.begin[s] = (int32_t)lo;
    }
    hipStream_t st = (hipStream_t)stream;
    return hip_status(timed(DFLASH_KERNEL_TOPK_MERGE, st, [&] {
      return dfk::launch_topk_merge(*d, n_shards, sb, cand_idx_parts, cand_logit_parts, cand_idx, cand_logit, st);
    }), "top-K merge launch");
  } catch (...) {
    return fail(DFLASH_ERR_HIP, "internal error");
  }
}

// the vocabulary split of the verify: shard boundaries, chunk bases and
// (when Z_shards is given) each shard's rows
static dflash_status make_shard_map(const dflash_dims* d, int32_t n_shards, const int32_t* shard_begin,
                                    const void* const* Z_shards, dfk::ShardMap& m) {
  if (n_shards < 1 || n_shards > DFLASH_MAX_SHARDS)
    return fail(DFLASH_ERR_INVALID_ARG, "n_shards must be in 1 .. DFLASH_MAX_SHARDS");
  if (!shard_begin) return fail(DFLASH_ERR_INVALID_ARG, "shard_begin is NULL");
  const int unit = d->logit_dtype == DFLASH_BF16 ? 8 : 4;
  m.n = n_shards;
  m.cbase[0] = 0;
  for (int s = 0; s < n_shards; ++s) {
    const int64_t lo = shard_begin[s], hi = s + 1 < n_shards ? shard_begin[s + 1] : d->V;
    if ((s == 0 && lo != 0) || hi <= lo || hi > d->V || lo % unit)
      return fail(DFLASH_ERR_INVALID_ARG, "shards must start at 0, increase, end by V, and begin at multiples of "
                                          "8 tokens (bf16) or 4 (fp32)");
    m.begin[s] = (int32_t)lo;
    m.cbase[s + 1] = m.cbase[s] + (int32_t)((hi - lo + dfk::kChunk - 1) / dfk::kChunk);
    m.Z[s] = nullptr;
    if (Z_shards) {
      if (!Z_shards[s]) return fail(DFLASH_ERR_INVALID_ARG, "a shard's Z is NULL");
      if (!aligned16(Z_shards[s])) return fail(DFLASH_ERR_INVALID_ARG, "a shard's Z is not 16-byte aligned");
      m.Z[s] = Z_shards[s];
    }
  }
  m.begin[n_shards] = d->V;
  return DFLASH_OK;
}

dflash_status dflash_shard_stats_bytes(const dflash_dims* d, int32_t n_shards, const int32_t* shard_begin,
                                       size_t* bytes) {
  try {
    g_err.clear();
    if (dflash_status s = check_dims(d)) return s;
    if (!bytes) return fail(DFLASH_ERR_INVALID_ARG, "bytes is NULL");
    dfk::ShardMap m{};
    if (dflash_status s = make_shard_map(d, n_shards, shard_begin, nullptr, m)) return s;
    *bytes = (size_t)d->B * (d->L + 1) * m.cbase[m.n] * sizeof(dfk::ChunkStat);
    return DFLASH_OK;
  } catch (...) {
    return fail(DFLASH_ERR_INVALID_ARG, "internal error");
  }
}

dflash_status dflash_shard_stats(const dflash_dims* d, int32_t n_shards, const int32_t* shard_begin, int32_t shard,
                                 const void* Z_shard, const float* T, void* stats, void* stream) {
  try {
    g_err.clear();
    if (dflash_status s = check_dims(d)) return s;
    dfk::ShardMap m{};
    if (dflash_status s = make_shard_map(d, n_shards, shard_begin, nullptr, m)) return s;
    if (shard < 0 || shard >= n_shards) return fail(DFLASH_ERR_INVALID_ARG, "shard must be in 0 .. n_shards - 1");
    if (dflash_status s = check_ptrs({{Z_shard, "Z_shard", true}, {T, "T", false}, {stats, "stats", true}})) return s;
    hipStream_t st = (hipStream_t)stream;
    return hip_status(timed(DFLASH_KERNEL_SHARD_STATS, st, [&] {
      return dfk::launch_shard_stats(*d, m, shard, Z_shard, T, static_cast<dfk::ChunkStat*>(stats), st);
    }), "shard stats launch");
  } catch (...) {
    return fail(DFLASH_ERR_HIP, "internal error");
  }
}

dflash_status dflash_verify_shards(const dflash_dims* d, int32_t n_shards, const int32_t* shard_begin,
                                   const void* const* Z_shards, const void* stats, const int32_t* cand_idx,
                                   const int32_t* path_rank, const float* q, const float* T, const uint64_t* seed,
                                   uint64_t cycle, int32_t* accept_len, int32_t* out_tok, void* stream) {
  try {
    g_err.clear();
    if (dflash_status s = check_dims(d)) return s;
    if (!Z_shards) return fail(DFLASH_ERR_INVALID_ARG, "Z_shards is NULL");
    dfk::ShardMap m{};
    if (dflash_status s = make_shard_map(d, n_shards, shard_begin, Z_shards, m)) return s;
    if (dflash_status s = check_ptrs({{stats, "stats", true}, {cand_idx, "cand_idx", false},
                                      {path_rank, "path_rank", false}, {q, "q", false}, {T, "T", false},
                                      {seed, "seed", false}, {accept_len, "accept_len", false},
                                      {out_tok, "out_tok", false}})) return s;
    hipStream_t st = (hipStream_t)stream;
    return hip_status(timed(DFLASH_KERNEL_SHARD_FINALIZE, st, [&] {
      return dfk::launch_finalize_shards(*d, m, cand_idx, path_rank, q, T, seed, cycle,
                                         static_cast<const dfk::ChunkStat*>(stats), accept_len, out_tok, st);
    }), "shard finalize launch");
  } catch (...) {
    return fail(DFLASH_ERR_HIP, "internal error");
  }
}

dflash_status dflash_trace_viterbi(const dflash_dims* d, const float* S, const int32_t* cand_idx, int32_t* path_rank,
                                   int32_t* draft_tok, float* q, void* stream) {
  try {
    g_err.clear();
    if (dflash_status s = check_dims(d)) return s;
    if (dflash_status s = check_ptrs({{S, "S", false}, {cand_idx, "cand_idx", false}, {path_rank, "path_rank", false},
                                      {draft_tok, "draft_tok", false}, {q, "q", false}})) return s;
    hipStream_t st = (hipStream_t)stream;
    return hip_status(timed(DFLASH_KERNEL_TRACE_VITERBI, st, [&] {
      return dfk::launch_trace_viterbi(*d, S, cand_idx, path_rank, draft_tok, q, st);
    }), "viterbi trace launch");
  } catch (...) {
    return fail(DFLASH_ERR_HIP, "internal error");
  }
}

dflash_status dflash_verify(const dflash_dims* d, const void* Z, const int32_t* cand_idx, const int32_t* path_rank,
                            const float* q, const float* T, const uint64_t* seed, uint64_t cycle,
                            int32_t* accept_len, int32_t* out_tok, void* ws, size_t ws_bytes, void* stream) {
  try {
    g_err.clear();
    if (dflash_status s = check_dims(d)) return s;
    if (dflash_status s = check_ptrs({{Z, "Z", true}, {cand_idx, "cand_idx", false}, {path_rank, "path_rank", false},
                                      {q, "q", false}, {T, "T", false}, {seed, "seed", false},
                                      {accept_len, "accept_len", false}, {out_tok, "out_tok", false}})) return s;
    const dfk::WsLayout w = dfk::ws_layout(*d);
    if (dflash_status s = check_ws(w, ws, ws_bytes)) return s;
    hipStream_t st = (hipStream_t)stream;
    dfk::ChunkStat* stats = reinterpret_cast<dfk::ChunkStat*>(static_cast<char*>(ws) + w.stats);
    if (dflash_status s = hip_status(timed(DFLASH_KERNEL_STATS, st, [&] {
          return dfk::launch_stats(*d, w, Z, T, stats, st);
        }), "stats launch")) return s;
    return hip_status(timed(DFLASH_KERNEL_FINALIZE, st, [&] {
      return dfk::launch_finalize(*d, w, Z, cand_idx, path_rank, q, T, seed, cycle, stats, accept_len, out_tok, st);
    }), "finalize launch");
  } catch (...) {
    return fail(DFLASH_ERR_HIP, "internal error");
  }
}

// dflash_cycle and dflash_cycle_maxsum: the streaming launch, the
// candidate/score launch, then the trace + verify launch (walking the greedy
// or sampled table, or finding the max-sum path over the scores)
static dflash_status cycle_impl(bool maxsum, const dflash_dims* d, const void* U, const void* Z, const int32_t* x0,
                                const void* E, const void* W_g, const void* h, const float* T, const uint64_t* seed,
                                uint64_t cycle, int32_t* accept_len, int32_t* out_tok, int32_t* cand_idx_opt,
                                float* cand_logit_opt, float* S_opt, int32_t* path_rank_opt, int32_t* draft_tok_opt,
                                float* q_opt, void* ws, size_t ws_bytes, void* stream) {
  try {
    g_err.clear();
    if (dflash_status s = check_dims(d)) return s;
    if (dflash_status s = check_ptrs({{U, "U", true}, {Z, "Z", true}, {x0, "x0", false}, {E, "E", true},
                                      {W_g, "W_g", true}, {h, "h", true}, {T, "T", false}, {seed, "seed", false},
                                      {accept_len, "accept_len", false}, {out_tok, "out_tok", false}})) return s;
    const dfk::WsLayout w = dfk::ws_layout(*d);
    if (dflash_status s = check_ws(w, ws, ws_bytes)) return s;
    char* base = static_cast<char*>(ws);
    int32_t* cand_idx = cand_idx_opt ? cand_idx_opt : reinterpret_cast<int32_t*>(base + w.cand_idx);
    float* cand_logit = cand_logit_opt ? cand_logit_opt : reinterpret_cast<float*>(base + w.cand_logit);
    float* S = S_opt ? S_opt : reinterpret_cast<float*>(base + w.S);
    int32_t* path_rank = path_rank_opt ? path_rank_opt : reinterpret_cast<int32_t*>(base + w.path_rank);
    int32_t* draft_tok = draft_tok_opt ? draft_tok_opt : reinterpret_cast<int32_t*>(base + w.draft_tok);
    float* q = q_opt ? q_opt : reinterpret_cast<float*>(base + w.q);
    hipStream_t st = (hipStream_t)stream;
    if (w.edges) {
      // the edges run inside the streaming launch: two launches
      const int n_sblk = d->B * (d->L + 1) * ((w.n_chunk + 3) / 4);
      const dfk::CycleEdges ce{(int)((long long)n_sblk * dfk::kEdgePrePct / 100), x0, E, seed, cycle, cand_idx,
                               cand_logit, S};
      if (dflash_status s = hip_status(timed(DFLASH_KERNEL_CYCLE_STREAM, st, [&] {
            return dfk::launch_cycle_stream(*d, w, U, Z, h, W_g, T, base, st, &ce);
          }), "stream launch")) return s;
    } else {
      if (dflash_status s = hip_status(timed(DFLASH_KERNEL_CYCLE_STREAM, st, [&] {
            return dfk::launch_cycle_stream(*d, w, U, Z, h, W_g, T, base, st);
          }), "stream launch")) return s;
      if (dflash_status s = hip_status(timed(DFLASH_KERNEL_CYCLE_SCORES, st, [&] {
            return dfk::launch_cycle_scores(*d, w, x0, E, Z, T, seed, cycle, base, cand_idx, cand_logit, S, st);
          }), "scores launch")) return s;
    }
    return hip_status(timed(DFLASH_KERNEL_CYCLE_FINALIZE, st, [&] {
      return dfk::launch_cycle_finalize(*d, w, Z, cand_idx, T, seed, cycle, base, maxsum ? S : nullptr, path_rank,
                                        draft_tok, q, accept_len, out_tok, st, w.edges);
    }), "finalize launch");
  } catch (...) {
    return fail(DFLASH_ERR_HIP, "internal error");
  }
}

dflash_status dflash_cycle(const dflash_dims* d, const void* U, const void* Z, const int32_t* x0, const void* E,
                           const void* W_g, const void* h, const float* T, const uint64_t* seed, uint64_t cycle,
                           int32_t* accept_len, int32_t* out_tok, int32_t* cand_idx_opt, float* cand_logit_opt,
                           float* S_opt, int32_t* path_rank_opt, int32_t* draft_tok_opt, float* q_opt, void* ws,
                           size_t ws_bytes, void* stream) {
  return cycle_impl(false, d, U, Z, x0, E, W_g, h, T, seed, cycle, accept_len, out_tok, cand_idx_opt,
                    cand_logit_opt, S_opt, path_rank_opt, draft_tok_opt, q_opt, ws, ws_bytes, stream);
}

dflash_status dflash_cycle_static(const dflash_dims* d, const void* U, const void* Z, const int32_t* x0,
                                  const void* E, const void* W_g, const void* h, const float* T,
                                  const uint64_t* seed, uint64_t cycle, int32_t* accept_len, int32_t* out_tok,
                                  int32_t* cand_idx_opt, float* cand_logit_opt, float* S_opt,
                                  int32_t* path_rank_opt, int32_t* draft_tok_opt, float* q_opt, void* stream) {
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  try {
    g_err.clear();
    if (dflash_status s = check_dims(d)) return s;
    // the cycle's own regions (the split path's tail is not touched)
    const size_t need = dfk::ws_layout(*d).cycle_total;
    if (need > DFLASH_STATIC_SCRATCH_BYTES)
      return fail(DFLASH_ERR_WORKSPACE, "these sizes need " + std::to_string(need) +
                                            " bytes of scratch, above the static maximum of " +
                                            std::to_string((size_t)DFLASH_STATIC_SCRATCH_BYTES) +
                                            " (use dflash_cycle with a workspace)");
    if (dflash_status s = hip_status(dfk::static_scratch(&scratch, &scratch_bytes), "static scratch lookup"))
      return s;
  } catch (...) {
    return fail(DFLASH_ERR_HIP, "internal error");
  }
  // the library's own array stands in for the caller's workspace
  return cycle_impl(false, d, U, Z, x0, E, W_g, h, T, seed, cycle, accept_len, out_tok, cand_idx_opt,
                    cand_logit_opt, S_opt, path_rank_opt, draft_tok_opt, q_opt, scratch, scratch_bytes, stream);
}

dflash_status dflash_cycle_maxsum(const dflash_dims* d, const void* U, const void* Z, const int32_t* x0,
                                  const void* E, const void* W_g, const void* h, const float* T,
                                  const uint64_t* seed, uint64_t cycle, int32_t* accept_len, int32_t* out_tok,
                                  int32_t* cand_idx_opt, float* cand_logit_opt, float* S_opt,
                                  int32_t* path_rank_opt, int32_t* draft_tok_opt, float* q_opt, void* ws,
                                  size_t ws_bytes, void* stream) {
  return cycle_impl(true, d, U, Z, x0, E, W_g, h, T, seed, cycle, accept_len, out_tok, cand_idx_opt,
                    cand_logit_opt, S_opt, path_rank_opt, draft_tok_opt, q_opt, ws, ws_bytes, stream);
}

dflash_status dflash_conv2tap(const dflash_dims* d, const void* x, const void* x0, const void* Wt, float* y,
                              void* stream) {
  try {
    g_err.clear();
    if (dflash_status s = check_dims(d)) return s;
    if (dflash_status s = check_ptrs({{x, "x", true}, {x0, "x0", false}, {Wt, "Wt", true}, {y, "y", false}})) return s;
    hipStream_t st = (hipStream_t)stream;
    return hip_status(timed(DFLASH_KERNEL_CONV2TAP, st, [&] { return dfk::launch_conv2tap(*d, x, x0, Wt, y, st); }),
                      "conv2tap launch");
  } catch (...) {
    return fail(DFLASH_ERR_HIP, "internal error");
  }
}

dflash_status dflash_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  try {
    g_err.clear();
    if (dflash_status s = check_ptrs({{buf, "buf", true}, {sink, "sink", false}})) return s;
    if (bytes % 16) return fail(DFLASH_ERR_INVALID_ARG, "bytes must be a multiple of 16");
    return hip_status(dfk::launch_read_probe(buf, bytes, sink, (hipStream_t)stream), "read probe");
  } catch (...) {
    return fail(DFLASH_ERR_HIP, "internal error");
  }
}

dflash_status dflash_copy_probe(void* dst, const void* src, size_t bytes, void* stream) {
  try {
    g_err.clear();
    if (dflash_status s = check_ptrs({{dst, "dst", true}, {src, "src", true}})) return s;
    if (bytes % 16) return fail(DFLASH_ERR_INVALID_ARG, "bytes must be a multiple of 16");
    return hip_status(dfk::launch_copy_probe(dst, src, bytes, (hipStream_t)stream), "copy probe");
  } catch (...) {
    return fail(DFLASH_ERR_HIP, "internal error");
  }
}

const char* dflash_kernel_name(int32_t kernel) {
  static const char* names[DFLASH_KERNEL_COUNT] = {"topk", "gate", "scores", "trace", "stats", "finalize",
                                                   "cycle_stream", "cycle_scores", "cycle_finalize", "conv2tap",
                                                   "trace_viterbi", "topk_merge", "shard_stats",
                                                   "shard_finalize"};
  return (kernel >= 0 && kernel < DFLASH_KERNEL_COUNT) ? names[kernel] : "";
}

dflash_status dflash_profile_enable(int32_t on) {
  try {
    g_err.clear();
    Profiler& P = prof();
    std::lock_guard<std::mutex> lk(P.mu);
    for (auto& v : P.pending) {
      for (auto& pr : v) {
        hipEventSynchronize(pr.second);
        P.pool.push_back(pr.first);
        P.pool.push_back(pr.second);
      }
      v.clear();
    }
    P.on = on != 0;
    return DFLASH_OK;
  } catch (...) {
    return fail(DFLASH_ERR_HIP, "internal error");
  }
}

dflash_status dflash_profile_collect(int32_t kernel, int64_t* launches, double* total_ms) {
  try {
    g_err.clear();
    if (kernel < 0 || kernel >= DFLASH_KERNEL_COUNT) return fail(DFLASH_ERR_INVALID_ARG, "unknown kernel id");
    if (!launches || !total_ms) return fail(DFLASH_ERR_INVALID_ARG, "output pointer is NULL");
    Profiler& P = prof();
    std::lock_guard<std::mutex> lk(P.mu);
    double sum = 0.0;
    int64_t n = 0;
    for (auto& pr : P.pending[kernel]) {
      if (hipEventSynchronize(pr.second) != hipSuccess) return fail(DFLASH_ERR_HIP, "event synchronize failed");
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess) return fail(DFLASH_ERR_HIP, "event timing failed");
      sum += ms;
      ++n;
      P.pool.push_back(pr.first);
      P.pool.push_back(pr.second);
    }
    P.pending[kernel].clear();
    *launches = n;
    *total_ms = sum;
    return DFLASH_OK;
  } catch (...) {
    return fail(DFLASH_ERR_HIP, "internal error");
  }
}

}  // extern "C"
