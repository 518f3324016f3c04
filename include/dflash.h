/*
 * dflash.h -- C ABI of the MI355X (gfx950) DFlash 2 draft -> select -> verify
 * hot path.  Library: block_draft_select_amd/libdflash.so.
 *
 * The method (four web pages on DFlash 2, cited by title and section):
 *   P1 "DFlash 2: Block diffusion, wearing a drafter's coat", section
 *      "The architecture" (sub-sections "Sixteen candidates per position",
 *      "A path selector", "Suffix-decay convolution", "Lossless, with
 *      conditions I did not used to state").
 *   P2 "A 2B Drafter Made a 27B Model 3.4x Faster. Same Exact Output.",
 *      sections "What a block-diffusion drafter is, and why it kept
 *      breaking", "The two fixes", "Caveats before you rebuild your serving
 *      stack".
 *   P3 "DFlash 2: Keep Drafting Parallel" (news text), section "What Comes
 *      Next", paragraph "A Lightweight Path Selector".
 *
 * One cycle of B independent streams: the drafter gives L logit rows U
 * (one per drafted position) and L context vectors h; the library keeps the
 * K best candidates per position, scores every adjacent candidate pair with
 * the drafter logit plus a gated bilinear embedding match, walks one path
 * through the candidate lattice, and verifies it against L+1 target logit
 * rows Z by rejection sampling (accept with min(1, p/q), resample from the
 * normalised residual max(0, p - q), bonus token when all L are accepted).
 * dflash_cycle does the whole cycle in two or three launches; dflash_topk,
 * dflash_pair_scores, dflash_trace and dflash_verify are its steps one by
 * one.  Beside them: dflash_trace_viterbi and dflash_cycle_maxsum take the
 * path of largest summed score instead of the greedy/sampled walk, and
 * dflash_conv2tap is the drafter's two-tap dynamic convolution, upstream of
 * the context vectors h.
 *
 * Conventions for every entry point:
 *   - Every array argument is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or retains caller memory.  Arrays are
 *     dense row-major with the shapes given in brackets.  U, Z, E, W_g and h
 *     must be 16-byte aligned.
 *   - Scratch lives in a caller-provided device workspace of at least
 *     dflash_workspace_bytes() bytes; its contents need no initialisation
 *     (dflash_workspace_init zero-fills one for callers who want defined
 *     contents).  The fused cycles keep one word of state in it between
 *     calls (the epoch of the hand-off entries passed between blocks of
 *     one launch, which validate themselves against it): memory that holds
 *     anything other than zeros or this workspace's own earlier cycles'
 *     entries passes that check by chance only (about 2^-32 per entry), so
 *     zero-filling a workspace before its first fused cycle, and after it
 *     served other sizes, rules that out.
 *     Calls that overlap in time must not share a workspace.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL is the default stream).  Outputs are valid once the caller
 *     synchronises with that stream.
 *   - Arguments are validated on the host before anything is enqueued: an
 *     invalid call returns an error status, launches nothing and leaves
 *     every output untouched.  dflash_last_error() then gives a message
 *     (thread-local).  No C++ exception crosses this boundary.
 *   - Outputs are a pure function of the inputs (including seed[] and
 *     cycle); they do not depend on launch shapes, split factors or timing.
 *   - Device-side index inputs (x0, cand_idx, path_rank) that lie outside
 *     their range are clamped into it, so no out-of-bounds access occurs;
 *     the outputs of such a stream are then unspecified.
 *   - Logits must be finite; NaN or infinite logits give unspecified
 *     results, but every token id the library writes still lies in [0, V)
 *     (or is the -1 padding) and no access leaves its array.
 *   - A finite temperature T[b] > 0 selects sampling for stream b; 0, a
 *     negative value or NaN selects greedy decoding (the defined behaviour,
 *     not an error: temperatures are device data, read only by the
 *     kernels); +inf gives unspecified results.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH_ABI_VERSION 1
#define DFLASH_K_MAX 16      /* candidates kept per position */
#define DFLASH_L_MAX 16      /* drafted positions per block */
#define DFLASH_MAX_SHARDS 64 /* vocabulary shards dflash_topk_merge combines */
#define DFLASH_R_MAX 256     /* embedding rank */
#define DFLASH_V_MAX 2097152 /* vocabulary size */
#define DFLASH_CHUNK 4096    /* tokens per first-level item of the residual draw */
#define DFLASH_STATIC_SCRATCH_BYTES (8u << 20) /* the library's own scratch per GPU (dflash_cycle_static) */

typedef int32_t dflash_status;
enum {
  DFLASH_OK = 0,
  DFLASH_ERR_INVALID_ARG = 1, /* bad dimension, null or misaligned pointer */
  DFLASH_ERR_UNSUPPORTED = 2, /* valid request the library does not handle */
  DFLASH_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  DFLASH_ERR_HIP = 4          /* the HIP runtime refused a launch */
};

/* element type of U and Z (logit_dtype) and of E, W_g and h (param_dtype) */
enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 };

typedef struct dflash_dims {
  int32_t B;           /* streams, >= 1, B * (L + 1) <= 65535 */
  int32_t L;           /* drafted positions, 1..DFLASH_L_MAX */
  int32_t V;           /* vocabulary, K..DFLASH_V_MAX; V * sizeof(logit) % 16 == 0 */
  int32_t K;           /* candidates per position, 1..DFLASH_K_MAX */
  int32_t r;           /* embedding rank, 16..DFLASH_R_MAX, multiple of 16 */
  int32_t hidden;      /* context width, >= 16, multiple of 16 */
  int32_t logit_dtype; /* DFLASH_F32 | DFLASH_BF16 */
  int32_t param_dtype; /* DFLASH_F32 | DFLASH_BF16 */
} dflash_dims;

/* Version of this ABI (DFLASH_ABI_VERSION). */
int32_t dflash_abi_version(void);

/* Static name of a status code. */
const char* dflash_status_string(dflash_status s);

/* Detail of the last error on the calling thread ("" if none). */
const char* dflash_last_error(void);

/* Bytes of workspace every entry point needs for `d` (host only, pure).
 * Returns DFLASH_ERR_INVALID_ARG / DFLASH_ERR_UNSUPPORTED for bad dims. */
dflash_status dflash_workspace_bytes(const dflash_dims* d, size_t* bytes);

/* Zero-fill `ws_bytes` bytes of a workspace on `stream` (a fill kernel). */
dflash_status dflash_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* S1 -- top-K candidates per drafted position (P1 "Sixteen candidates per
 * position"; P2 "What a block-diffusion drafter is ...").
 *   U          [B, L, V] logits (logit_dtype)
 *   cand_idx   [B, L, K] int32 out: token ids, ordered by logit descending,
 *              equal logits by token id ascending (-0.0 equals +0.0)
 *   cand_logit [B, L, K] float out: those logits, widened exactly to fp32 */
dflash_status dflash_topk(const dflash_dims* d, const void* U, int32_t* cand_idx,
                          float* cand_logit, void* ws, size_t ws_bytes, void* stream);

/* S1 over a vocabulary split -- the exact top-K of every drafter row from
 * the top-K lists of its vocabulary shards (P1 "Sixteen candidates per
 * position": the K best tokens over the whole vocabulary).  Shard s covers
 * tokens [shard_begin[s], shard_begin[s+1]) (the last one up to V); its list
 * is what dflash_topk returns for the shard's own [B, L, width] slice of U
 * (indices local to the shard).  The result equals dflash_topk over the whole
 * of U: the K best of the union, value descending, then global index
 * ascending, -0 equal to +0.
 *   d                  B, L, V, K of the whole problem (validated as usual)
 *   n_shards           1 .. DFLASH_MAX_SHARDS
 *   shard_begin        HOST array [n_shards]: shard_begin[0] = 0, increasing,
 *                      every shard at least K tokens wide
 *   cand_idx_parts     [n_shards, B, L, K] int32, local indices in [0, width)
 *   cand_logit_parts   [n_shards, B, L, K] float
 *   cand_idx, cand_logit  [B, L, K] out (global indices)
 * One launch on `stream` (one wave per row); no workspace.  Invalid
 * arguments launch nothing and leave the outputs untouched. */
dflash_status dflash_topk_merge(const dflash_dims* d, int32_t n_shards, const int32_t* shard_begin,
                                const int32_t* cand_idx_parts, const float* cand_logit_parts,
                                int32_t* cand_idx, float* cand_logit, void* stream);

/* S5 over a vocabulary split -- the chunk statistics of one shard's target
 * rows (P1 "Lossless, with conditions I did not used to state"; the split
 * follows a tensor-parallel LM head, P2 "Running it").  Shard s covers
 * tokens [shard_begin[s], shard_begin[s+1]) (the last one up to V) and holds
 * its own rows Z_shard [B, L + 1, width].  The residual draw's chunks
 * restart at every shard's first token (DFLASH_CHUNK tokens each, the last
 * one of a shard shorter), so each shard's statistics depend only on its
 * own logits.  This call writes shard `shard`'s columns of `stats`, the
 * statistics of the whole vocabulary: [B, L + 1, C] records of 16 bytes,
 * C = sum over shards of ceil(width / DFLASH_CHUNK) (its size in bytes:
 * dflash_shard_stats_bytes).  With one shard per device, the columns of
 * the other shards arrive by an exchange of these records (an all-gather,
 * or a sum over zero-filled buffers) before dflash_verify_shards.
 *   d            the whole problem (V = the whole vocabulary)
 *   n_shards     1 .. DFLASH_MAX_SHARDS
 *   shard_begin  HOST array [n_shards]: shard_begin[0] = 0, increasing, each
 *                a multiple of 8 (bf16 logits) or 4 (fp32), below V
 *   shard        which shard's statistics to compute, 0 .. n_shards - 1
 *   Z_shard      [B, L + 1, width] logits of the shard (logit_dtype),
 *                16-byte aligned
 *   T            [B] temperatures
 *   stats        [B, L + 1, C] x 16 bytes, written in this shard's columns
 * One launch on `stream`; no workspace.  Invalid arguments launch nothing. */
dflash_status dflash_shard_stats_bytes(const dflash_dims* d, int32_t n_shards, const int32_t* shard_begin,
                                       size_t* bytes);
dflash_status dflash_shard_stats(const dflash_dims* d, int32_t n_shards, const int32_t* shard_begin, int32_t shard,
                                 const void* Z_shard, const float* T, void* stats, void* stream);

/* S6 over a vocabulary split -- dflash_verify from the statistics of every
 * shard (dflash_shard_stats), with the residual draw's chunks restarting at
 * every shard boundary; without a split (one shard) the outputs equal
 * dflash_verify's, and so do they when every boundary is a multiple of
 * DFLASH_CHUNK.  The candidates' target logits and the drawn chunk are read
 * from the shard that holds them (one device here; across devices, only
 * the owner of the drawn chunk would re-read it).
 *   Z_shards     HOST array [n_shards] of device pointers, shard s's rows
 *                [B, L + 1, width_s] (16-byte aligned)
 *   stats        [B, L + 1, C] x 16 bytes, every shard's columns filled
 *   the rest as dflash_verify
 * One launch on `stream` (one block per stream); no workspace. */
dflash_status dflash_verify_shards(const dflash_dims* d, int32_t n_shards, const int32_t* shard_begin,
                                   const void* const* Z_shards, const void* stats, const int32_t* cand_idx,
                                   const int32_t* path_rank, const float* q, const float* T, const uint64_t* seed,
                                   uint64_t cycle, int32_t* accept_len, int32_t* out_tok, void* stream);

/* S2 + S3 -- context gate and adjacent pair scores (P3 "A Lightweight Path
 * Selector"; P1 "A path selector").  With g_t[k] = sigmoid(sum_j
 * W_g[k,j] * h_t[j]):
 *   S[b,t,i,j] = cand_logit[b,t,j] + sum_k E[a_i,k] * g_t[k] * E[c_j,k]
 * where c_j = cand_idx[b,t,j] and a_i = cand_idx[b,t-1,i] for t >= 1, and
 * a_i = x0[b] (the last verified token) for every row i of edge t = 0.
 *   x0         [B] int32, the last verified token of each stream
 *   cand_idx   [B, L, K] int32, cand_logit [B, L, K] float (from dflash_topk)
 *   E          [V, r] candidate embeddings (param_dtype)
 *   W_g        [r, hidden] gate weights (param_dtype), one row per
 *              embedding dimension (the layout of a linear layer's weight)
 *   h          [B, L, hidden] drafter context (param_dtype)
 *   S          [B, L, K, K] float out (rows: predecessor rank, cols: rank) */
dflash_status dflash_pair_scores(const dflash_dims* d, const int32_t* x0,
                                 const int32_t* cand_idx, const float* cand_logit,
                                 const void* E, const void* W_g, const void* h, float* S,
                                 void* ws, size_t ws_bytes, void* stream);

/* S4 -- walk one path through the lattice (P3 "A Lightweight Path Selector").
 * Starting at rank 0 of edge 0, position t picks rank j_t from row j_{t-1}
 * of S[b,t]: greedy (smallest rank attaining the maximum) when T[b] <= 0,
 * otherwise a draw from q_t = softmax(S[b,t,j_{t-1},:] / T[b]) by inverse
 * CDF with the fp32 uniform u = ((w >> 9) * 2 + 1) * 2^-24 of word 0 of
 * Philox4x32-10(key = seed[b], counter = (cycle lo, cycle hi, t + 1, 0)).
 *   T          [B] float temperatures;  seed [B] uint64 Philox keys
 *   path_rank  [B, L] int32 out;  draft_tok [B, L] int32 out (the tokens)
 *   q          [B, L, K] float out: q_t (one-hot at T <= 0) */
dflash_status dflash_trace(const dflash_dims* d, const float* S, const int32_t* cand_idx,
                           const float* T, const uint64_t* seed, uint64_t cycle,
                           int32_t* path_rank, int32_t* draft_tok, float* q, void* stream);

/* S5 + S6 -- verify against the target (P1 "Lossless, with conditions I did
 * not used to state"; P2 "Caveats before you rebuild your serving stack").
 * Greedy streams accept the longest prefix whose drafts equal the target
 * argmax (smallest index on ties) and emit the argmax of the next row.
 * Sampling streams accept position t while u_t * q_t(d_t) < p_t(d_t), with
 * p_t = softmax(Z[b,t,:] / T[b]) and u_t the fp32 uniform of word 1 of the
 * (cycle, t + 1, 0) block; at the first rejection (or after L accepts, on
 * row L with no candidates) one token is drawn from the normalised residual
 * (max(0, p - q) on the candidates of that position, p elsewhere; p itself
 * if that residual has no mass) in two inverse-CDF levels: fp64 uniform u1
 * (words 0,1 of the (cycle, row + 1, 1) block) picks an item among
 * [DFLASH_CHUNK-token chunks carrying their non-candidate mass, then the K
 * candidates]; u2 (words 2,3) picks the token inside a picked chunk; each
 * fp64 uniform is ((hi:lo >> 12) * 2 + 1) * 2^-53.
 *   Z          [B, L + 1, V] target logits (logit_dtype)
 *   cand_idx   [B, L, K], path_rank [B, L], q [B, L, K] (from dflash_trace)
 *   accept_len [B] int32 out: accepted drafts n in 0..L
 *   out_tok    [B, L + 1] int32 out: the n accepted drafts, then the
 *              resampled or bonus token, then -1 padding */
dflash_status dflash_verify(const dflash_dims* d, const void* Z, const int32_t* cand_idx,
                            const int32_t* path_rank, const float* q, const float* T,
                            const uint64_t* seed, uint64_t cycle, int32_t* accept_len,
                            int32_t* out_tok, void* ws, size_t ws_bytes, void* stream);

/* One whole cycle: dflash_topk, dflash_pair_scores, dflash_trace and
 * dflash_verify on one stream, with identical results, in two launches
 * when the candidate and score work fits inside the streaming launch (its
 * top-K, gate and edge blocks all resident at once on the GPU: 2048
 * 256-thread blocks on an MI355X), else in three.
 * The intermediate outputs (cand_idx [B,L,K], cand_logit [B,L,K],
 * S [B,L,K,K], path_rank [B,L], draft_tok [B,L], q [B,L,K]) are written
 * where the caller passes non-NULL pointers and kept in the workspace
 * otherwise.
 * The call enqueues kernels only (no allocation, copy or memset), so it may
 * be captured into a HIP graph: a replay repeats the captured arguments,
 * the cycle number included, while the workspace's hand-off epoch, device
 * state that every cycle advances, keeps successive replays apart. */
dflash_status dflash_cycle(const dflash_dims* d, const void* U, const void* Z,
                           const int32_t* x0, const void* E, const void* W_g, const void* h,
                           const float* T, const uint64_t* seed, uint64_t cycle,
                           int32_t* accept_len, int32_t* out_tok,
                           int32_t* cand_idx_opt, float* cand_logit_opt, float* S_opt,
                           int32_t* path_rank_opt, int32_t* draft_tok_opt, float* q_opt,
                           void* ws, size_t ws_bytes, void* stream);

/* dflash_cycle without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The scratch is the library's
 * own file-scope device array of DFLASH_STATIC_SCRATCH_BYTES (8 MiB) per
 * GPU, held until the process ends; no call allocates or frees anything.
 * Same arguments, results and launches as dflash_cycle otherwise.
 *   - Sizes whose cycle workspace (dflash_workspace_bytes less the split
 *     path's gate partials, which the layout keeps last and the cycle does
 *     not touch) exceeds DFLASH_STATIC_SCRATCH_BYTES are rejected with
 *     DFLASH_ERR_WORKSPACE before anything is enqueued (the five benchmark
 *     shapes, up to B = 128, L = 8, V = 262144, need at most 5.7 MiB).
 *   - The first call on a device looks up the array's device address with
 *     hipGetSymbolAddress (a host-side query, no allocation) while that
 *     device is current; make that first call outside graph capture.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (the cycle needs none cleared): calls that overlap in
 *     time on one GPU (concurrent streams, threads) race and must not. */
dflash_status dflash_cycle_static(const dflash_dims* d, const void* U, const void* Z,
                                  const int32_t* x0, const void* E, const void* W_g, const void* h,
                                  const float* T, const uint64_t* seed, uint64_t cycle,
                                  int32_t* accept_len, int32_t* out_tok,
                                  int32_t* cand_idx_opt, float* cand_logit_opt, float* S_opt,
                                  int32_t* path_rank_opt, int32_t* draft_tok_opt, float* q_opt,
                                  void* stream);

/* The whole cycle with the max-sum trace (dflash_trace_viterbi) in place of
 * the greedy/sampled walk, in two or three launches like dflash_cycle: its
 * streaming launch (with the candidate/score work inside when it fits, else
 * a candidate/score launch after it), then one block per stream that finds
 * the max-sum path over the pair scores and runs the verify.  Same
 * arguments, layouts and workspace as dflash_cycle; q is one-hot.  Outputs
 * equal those of dflash_topk, dflash_pair_scores, dflash_trace_viterbi and
 * dflash_verify called in turn. */
dflash_status dflash_cycle_maxsum(const dflash_dims* d, const void* U, const void* Z,
                                  const int32_t* x0, const void* E, const void* W_g, const void* h,
                                  const float* T, const uint64_t* seed, uint64_t cycle,
                                  int32_t* accept_len, int32_t* out_tok,
                                  int32_t* cand_idx_opt, float* cand_logit_opt, float* S_opt,
                                  int32_t* path_rank_opt, int32_t* draft_tok_opt, float* q_opt,
                                  void* ws, size_t ws_bytes, void* stream);

/* Max-sum (Viterbi) variant of the trace (P3 "DFlash 2: Keep Drafting
 * Parallel", "What Comes Next", paragraph "A Lightweight Path Selector": the
 * pair scores and a walk from the verified token; better searches are left
 * open there).  Instead of the greedy walk, the path of largest summed edge
 * score S[0, 0, j_1] + S[1, j_1, j_2] + ... + S[L-1, j_{L-1}, j_L] over all
 * K^L paths; among equal values the smallest in reverse lexicographic order
 * (j_L first).  Sums are formed in fp64 from the fp32 scores.  The path is
 * deterministic, so q is one-hot at each chosen rank and dflash_verify keeps
 * the target distribution exact at any temperature.
 *   d          uses B, L, V, K (the whole struct is validated)
 *   S          [B, L, K, K] fp32, as written by dflash_pair_scores
 *   cand_idx   [B, L, K] i32 (indices outside [0, V) are clamped for draft_tok)
 *   path_rank  [B, L] i32, written: the chosen rank per position
 *   draft_tok  [B, L] i32, written: cand_idx at that rank
 *   q          [B, L, K] fp32, written: one-hot at path_rank
 * Caller-owned device buffers; one launch on `stream` (one wave per stream);
 * no workspace; no random numbers.  Scores must be finite.  Invalid
 * arguments launch nothing and leave the outputs untouched. */
dflash_status dflash_trace_viterbi(const dflash_dims* d, const float* S, const int32_t* cand_idx, int32_t* path_rank,
                                   int32_t* draft_tok, float* q, void* stream);

/* The two-tap dynamic depthwise convolution of the drafter's block
 * representations (P1 "DFlash 2: Block diffusion, wearing a drafter's coat",
 * "The architecture", "Suffix-decay convolution"; P2 "A 2B Drafter Made a
 * 27B Model 3.4x Faster. Same Exact Output.", "The two fixes"):
 *   [w0_t | w1_t] = Wt x_t,  y_t = w0_t * x_t + w1_t * x_{t-1},
 * with x_0 = x0 (the representation of the last verified position).  The
 * tap generator is not on the pages; this linear map is a reading.
 *   d   uses B, L, hidden and param_dtype (the whole struct is validated)
 *   x   [B, L, hidden]   param_dtype, 16-byte aligned
 *   x0  [B, hidden]      param_dtype
 *   Wt  [2*hidden, hidden] param_dtype, 16-byte aligned: row c generates
 *       w0[c], row hidden + c generates w1[c] (k contiguous per tap)
 *   y   [B, L, hidden]   fp32, written
 * Caller-owned device buffers; one launch on `stream` (kernels only, so the
 * call may be captured into a HIP graph); no workspace.  fp32 accumulation
 * (bf16 products are exact in fp32) in a fixed order, so repeated calls give
 * identical y.  Invalid arguments launch nothing and leave y untouched. */
dflash_status dflash_conv2tap(const dflash_dims* d, const void* x, const void* x0, const void* Wt, float* y,
                              void* stream);

/* ---- measurement helpers (not part of the method) ---------------------- */

/* Stream-read `bytes` (multiple of 16, 16-byte aligned) of `buf` once: the
 * achievable HBM read ceiling for the streaming launch's access shape (each
 * wave one contiguous 8 KB piece, nontemporal 16-byte loads, all in flight
 * together).  Each lane folds its words with XOR and stores to *sink only if
 * the fold equals one fixed constant, so the loads cannot be elided; *sink
 * is normally left untouched. */
dflash_status dflash_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Plain copy of `bytes` (multiple of 16, both 16-byte aligned): the
 * reference kernel for scaling hardware byte counters. */
dflash_status dflash_copy_probe(void* dst, const void* src, size_t bytes, void* stream);

/* Kernel identifiers for the per-kernel timer. */
enum {
  DFLASH_KERNEL_TOPK = 0,
  DFLASH_KERNEL_GATE = 1,
  DFLASH_KERNEL_SCORES = 2,
  DFLASH_KERNEL_TRACE = 3,
  DFLASH_KERNEL_STATS = 4,
  DFLASH_KERNEL_FINALIZE = 5,
  DFLASH_KERNEL_CYCLE_STREAM = 6,   /* dflash_cycle: gate + top-K lists + target chunk statistics
                                       (+ candidates and pair scores in the two-launch form) */
  DFLASH_KERNEL_CYCLE_SCORES = 7,   /* dflash_cycle, three-launch form: candidates + pair scores */
  DFLASH_KERNEL_CYCLE_FINALIZE = 8, /* dflash_cycle: trace + verify */
  DFLASH_KERNEL_CONV2TAP = 9,       /* dflash_conv2tap */
  DFLASH_KERNEL_TRACE_VITERBI = 10, /* dflash_trace_viterbi */
  DFLASH_KERNEL_TOPK_MERGE = 11,    /* dflash_topk_merge */
  DFLASH_KERNEL_SHARD_STATS = 12,   /* dflash_shard_stats */
  DFLASH_KERNEL_SHARD_FINALIZE = 13, /* dflash_verify_shards */
  DFLASH_KERNEL_COUNT = 14
};

/* Name of a kernel identifier ("" if out of range). */
const char* dflash_kernel_name(int32_t kernel);

/* Enable (on != 0) or disable the per-kernel timer: while enabled, every
 * launch is bracketed by hipEvents recorded on its own stream.  Enabling
 * discards earlier samples.  Host-side state shared by all threads. */
dflash_status dflash_profile_enable(int32_t on);

/* Wait for recorded launches of `kernel` and return their count and summed
 * duration in milliseconds; the samples are then discarded. */
dflash_status dflash_profile_collect(int32_t kernel, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
