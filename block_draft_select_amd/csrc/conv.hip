// The two-tap dynamic depthwise convolution of the drafter's block
// representations (P1 "DFlash 2: Block diffusion, wearing a drafter's coat",
// "The architecture", sub-section "Suffix-decay convolution"; P2 "A 2B
// Drafter Made a 27B Model 3.4x Faster. Same Exact Output.", "The two
// fixes").  Reading of the unstated tap generator: one linear map per
// position, [w0_t | w1_t] = Wt x_t with Wt [2H, H] (row c generates w0[c],
// row H + c generates w1[c]), and y_t = w0_t * x_t + w1_t * x_{t-1}, x0 the
// first position's predecessor.
//
// bf16 operands: the taps are a GEMM [B*L, H] x [H, 2H] on the matrix cores
// (v_mfma_f32_16x16x32_bf16) with the mixing fused into its epilogue, so
// neither the taps nor a transposed copy ever reach HBM.  A block of WM x WN
// waves owns BM rows and BC channels of both taps; every 64-wide k
// stage of its x rows and generator rows lands in LDS as whole 128-byte row
// pieces (16-byte chunks XOR-swizzled by row, so that neither the stores
// nor the fragment reads conflict in the banks), either straight from
// global memory into a ring of stage buffers (global_load_lds_dwordx4) or
// through registers into a double buffer with P stages of loads in flight,
// while the MFMAs read the current stage.  A wave owns MT row tiles and CT channel tiles of both taps,
// so the two taps of each output sit in the same lane and the epilogue
// mixes them from registers.  The row tiles of one channel tile share an XCD (block id mod 8), so that
// tile's generator rows come from HBM once and from that XCD's L2 after.
// fp32 operands: one thread per output, two dot products on the VALU.
#include "device_util.hpp"
#include "internal.hpp"
#include "select_blocks.hpp"


namespace dfk {

namespace {

constexpr int kConvBK = 64;                // k per LDS stage (two MFMA k-steps)

// MT 16-row tiles and CT 16-channel tiles (each with both taps) per wave;
// the block's WM x WN waves cover BM rows and BC channels
template <int MT, int CT, int WM, int WN>
struct ConvTile {
  static constexpr int THREADS = 64 * WM * WN;
  static constexpr int BM = 16 * MT * WM;
  static constexpr int BC = 16 * CT * WN;
  static constexpr int ROWS = BM + 2 * BC;  // staged rows: x rows, then tap-0 and tap-1 generator rows
  static constexpr int RPI = THREADS / 8;   // rows one load instruction covers (eight lanes per row)
  static constexpr int LOADS = ROWS / RPI;  // 16-byte loads per thread per stage (register-staged ring)
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// block id -> (row tile, channel tile): ids with the same value mod 8 run on
// one XCD; the n_rt row tiles of channel tile ct take ids
// (ct / 8) * 8 * n_rt + rt * 8 + ct % 8
__device__ __forceinline__ bool conv_tile(int id, int n_rt, int n_ct, int& rt, int& ct) {
  const int grp = id / (8 * n_rt), rem = id - grp * 8 * n_rt;
  rt = rem >> 3;
  ct = grp * 8 + (rem & 7);
  return ct < n_ct;
}

// Workgroup barrier for LDS hand-offs only: this wave's LDS reads and
// writes complete (lgkmcnt 0), then s_barrier.  __syncthreads() would also
// wait for every global load in flight (vmcnt 0), which drains the prefetch
// ring at every stage.  The empty asm keeps the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63 (no wait), expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// MFMA fragment offsets inside a stage: lane row lane % 16 (tile rows start
// at multiples of 16, so the row's swizzle key is lane % 8), 16-byte chunk
// 4 * ks + lane / 16 of the 64-wide stage
struct ConvFrag {
  int fo[kConvBK / 32];
  __device__ __forceinline__ explicit ConvFrag(int lane) {
#pragma unroll
    for (int ks = 0; ks < kConvBK / 32; ++ks) {
      const int c = 4 * ks + (lane >> 4);
      fo[ks] = (lane & 15) * (kConvBK * 2) + (c ^ (lane & 7)) * 16;
    }
  }
};

// one stage's MFMAs of a wave: every fragment first, then the products
template <int MT, int CT, int BC>
__device__ __forceinline__ void conv_stage(const unsigned char* st, const ConvFrag& f, int a_row, int b_row,
                                           v4f32 (&acc)[MT][CT][2]) {
  constexpr int PITCH = kConvBK * 2;
  bf16x8 a[kConvBK / 32][MT], b[kConvBK / 32][CT][2];
#pragma unroll
  for (int ks = 0; ks < kConvBK / 32; ++ks) {
#pragma unroll
    for (int m = 0; m < MT; ++m) a[ks][m] = *reinterpret_cast<const bf16x8*>(st + (a_row + m * 16) * PITCH + f.fo[ks]);
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int tap = 0; tap < 2; ++tap)
        b[ks][c][tap] = *reinterpret_cast<const bf16x8*>(st + (b_row + tap * BC + c * 16) * PITCH + f.fo[ks]);
  }
  // one-tile waves: left to itself the scheduler hangs each MFMA behind its
  // own fragment read's LDS round trip; the scheduling barrier keeps the
  // stage's reads together ahead of the MFMAs (16.0 to 16.3 against 17.1 to
  // 17.7 us at 256 x 2048; the larger tiles interleave well by themselves)
  if constexpr (MT == 1 && CT == 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < kConvBK / 32; ++ks)
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int tap = 0; tap < 2; ++tap)
          acc[m][c][tap] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks][m], b[ks][c][tap], acc[m][c][tap], 0, 0, 0);
}

// epilogue: element e of the lane holds (row 4 * (lane / 16) + e, channel
// lane % 16) of each tile; both taps of that output are in this lane
template <int MT, int CT>
__device__ __forceinline__ void conv_mix_store(const v4f32 (&acc)[MT][CT][2], const uint16_t* __restrict__ x,
                                               const uint16_t* __restrict__ x0, int R, int L, int H, int rbase,
                                               int cbase, int lane, float* __restrict__ y) {
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int ch = cbase + c * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = rbase + m * 16 + 4 * (lane >> 4) + e;
        if (row >= R || ch >= H) continue;
        const int t = row % L;
        const float xv = bf16_to_f32(x[(size_t)row * H + ch]);
        const float xp = bf16_to_f32(t > 0 ? x[(size_t)(row - 1) * H + ch] : x0[(size_t)(row / L) * H + ch]);
        y[(size_t)row * H + ch] = fmaf(acc[m][c][1][e], xp, acc[m][c][0][e] * xv);
      }
    }
}

// Register-staged ring: each thread loads its LOADS row pieces of a stage
// into registers (P stages in flight) and stores them to a double-buffered
// LDS.  Used for the 128 x 64 tiles, whose 64 KB of LDS lets two blocks
// share a CU.
template <int MT, int CT, int P, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void conv_mfma_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ x0,
                                                                 const uint16_t* __restrict__ Wt, int R, int L, int H,
                                                                 int n_rt, int n_ct, float* __restrict__ y) {
  using Tl = ConvTile<MT, CT, WM, WN>;
  constexpr int PITCH = kConvBK * 2;  // 128-byte rows, 16-byte chunks XOR-swizzled by row % 8
  static_assert(Tl::BM % Tl::RPI == 0 && (2 * Tl::BC) % Tl::RPI == 0, "a load instruction covers rows of one operand");
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][Tl::ROWS * PITCH];
  int rt, ct;
  if (!conv_tile(blockIdx.x, n_rt, n_ct, rt, ct)) return;  // padding ids of the last channel group
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave % WM, wn = wave / WM;
  const int row0 = rt * Tl::BM, ch0 = ct * Tl::BC;
  const int n_st = (H + kConvBK - 1) / kConvBK;

  // this thread's share of a stage: LOADS row pieces of 16 bytes; staged row
  // rho = p / 8 holds x row row0 + rho, then the tap-0 generator rows
  // ch0 + j and the tap-1 rows H + ch0 + j
  const uint16_t* src[Tl::LOADS];
  unsigned rmask[Tl::LOADS];  // all ones for a row inside the operand, else zero
  int dst[Tl::LOADS];
  const int c8 = (tid & 7) * 8;
#pragma unroll
  for (int i = 0; i < Tl::LOADS; ++i) {
    const int rho = (tid >> 3) + Tl::RPI * i;
    dst[i] = rho * PITCH + ((tid & 7) ^ (rho & 7)) * 16;
    if (rho < Tl::BM) {
      const int row = row0 + rho;
      rmask[i] = row < R ? 0xFFFFFFFFu : 0u;
      src[i] = x + (size_t)min(row, R - 1) * H + c8;
    } else {
      const int j = rho - Tl::BM, tap = j / Tl::BC, c = ch0 + j - tap * Tl::BC;
      rmask[i] = c < H ? 0xFFFFFFFFu : 0u;
      src[i] = Wt + ((size_t)tap * H + min(c, H - 1)) * H + c8;
    }
  }
  // P stages of loads in flight: register slot u % P holds stage u until
  // it is stored to LDS, then takes stage u + P
  uint4 pre[P][Tl::LOADS];
  // loads are unconditional (a masked load would become a branch, and the
  // compiler would then wait for every load in flight before each store):
  // a k run past the row end reads the row's last eight values instead,
  // and the store writes zeros for it and for rows past the edge
  auto load_stage = [&](int s, uint4(&r)[Tl::LOADS]) {
    const int k0 = s * kConvBK;
    const int ko = k0 + c8 < H ? k0 : H - 8 - c8;
#pragma unroll
    for (int i = 0; i < Tl::LOADS; ++i) r[i] = *reinterpret_cast<const uint4*>(src[i] + ko);
  };
  auto store_stage = [&](const uint4(&r)[Tl::LOADS], int s, int buf) {
    const unsigned kok = s * kConvBK + c8 < H ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int i = 0; i < Tl::LOADS; ++i) {
      const unsigned m = kok & rmask[i];
      *reinterpret_cast<uint4*>(&lds[buf][dst[i]]) = make_uint4(r[i].x & m, r[i].y & m, r[i].z & m, r[i].w & m);
    }
  };

  v4f32 acc[MT][CT][2];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[m][c][0] = acc[m][c][1] = (v4f32){0.f, 0.f, 0.f, 0.f};
  const ConvFrag f(lane);
  const int a_row = wm * 16 * MT, b_row = Tl::BM + wn * 16 * CT;

  // straight-line ring (P divides the stage count, so no stage test inside
  // the unrolled body): the last P stages reload the final stage into slots
  // that are never stored, and the last store fills a buffer nobody reads
#pragma unroll
  for (int u = 0; u < P; ++u) load_stage(u, pre[u]);
  store_stage(pre[0], 0, 0);
  lds_barrier();
  for (int s0 = 0; s0 < n_st; s0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int s = s0 + u;
      load_stage(min(s + P, n_st - 1), pre[u]);  // stage s is in LDS already
      conv_stage<MT, CT, Tl::BC>(lds[s & 1], f, a_row, b_row, acc);
      store_stage(pre[(u + 1) % P], min(s + 1, n_st - 1), (s + 1) & 1);
      lds_barrier();
    }
  }
  conv_mix_store<MT, CT>(acc, x, x0, R, L, H, row0 + wm * 16 * MT, ch0 + wn * 16 * CT, lane, y);
}

// One 16-byte piece per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane l's piece lands at l * 16 bytes past the
// wave-uniform LDS address.  The data never passes through registers, and
// the wave's vmcnt counts the transfer.  The host pass of the kernel
// templates does not know the builtin, so it is compiled in the device pass
// only.
__device__ __forceinline__ void load_to_lds16(const uint16_t* g, unsigned char* l) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
#endif
}

// Direct-to-LDS ring: NB stage buffers, one barrier per stage; while stage
// s is multiplied, stages s + 1 .. s + NB - 2 are in flight, and stage
// s + NB - 1 is issued after its MFMAs into the buffer stage s - 1 used.  A wave instruction
// fills one 8-row group of a stage (8 x 128 bytes, contiguous in LDS): lane
// l writes row 8g + l / 8 at position l % 8, which holds the row's chunk
// (l % 8) ^ (l / 8), so the swizzle is applied on the global side.  Rows
// past the edge read a clamped row: they only feed outputs that are never
// stored.  A k run past the row end reads the row's last eight values, and
// the stage holding it is cleared there before it is used.
template <int MT, int CT, int NB, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void conv_lds_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ x0,
                                                                const uint16_t* __restrict__ Wt, int R, int L, int H,
                                                                int n_rt, int n_ct, float* __restrict__ y) {
  using Tl = ConvTile<MT, CT, WM, WN>;
  constexpr int NW = WM * WN;
  constexpr int PITCH = kConvBK * 2;
  constexpr int GROUPS = Tl::ROWS / 8;  // 8-row groups per stage
  // load instructions per wave per stage: group g = wave + NW * i is the
  // wave's instruction i, so the first GROUPS % NW waves take one more
  constexpr int LPW = (GROUPS + NW - 1) / NW, LPW_LO = GROUPS / NW, NHI = GROUPS % NW;
  constexpr int INFLIGHT = LPW * (NB - 2), INFLIGHT_LO = LPW_LO * (NB - 2);
  static_assert(NB >= 3 && INFLIGHT <= 63, "a stage multiplied, one refilling, one landing; the vmcnt field");
  constexpr int SBYTES = Tl::ROWS * PITCH;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[NB * SBYTES];
  int rt, ct;
  if (!conv_tile(blockIdx.x, n_rt, n_ct, rt, ct)) return;  // padding ids of the last channel group
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave % WM, wn = wave / WM;
  const int row0 = rt * Tl::BM, ch0 = ct * Tl::BC;
  const int n_st = (H + kConvBK - 1) / kConvBK;

  // group g = wave + NW * i of every stage is this wave's instruction i
  const uint16_t* rowp[LPW];
  const int cc = ((lane & 7) ^ (lane >> 3)) * 8;  // element column of the lane's chunk
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int rho = min(8 * (wave + NW * i) + (lane >> 3), Tl::ROWS - 1);  // past the groups: unused
    if (rho < Tl::BM) {
      rowp[i] = x + (size_t)min(row0 + rho, R - 1) * H;
    } else {
      const int j = rho - Tl::BM, tap = j / Tl::BC, c = ch0 + j - tap * Tl::BC;
      rowp[i] = Wt + ((size_t)tap * H + min(c, H - 1)) * H;
    }
  }
  // stage t into buffer t % NB; past the last stage the last one is loaded
  // again into a buffer no later stage uses, so that every wave issues the
  // same count and the waits below hold at the tail too
  auto issue = [&](int t) {
    const int col = min(min(t, n_st - 1) * kConvBK + cc, H - 8);
    unsigned char* base = lds + (t % NB) * SBYTES;
#pragma unroll
    for (int i = 0; i < LPW; ++i)
      if (wave + NW * i < GROUPS) load_to_lds16(rowp[i] + col, base + (wave + NW * i) * (8 * PITCH));
  };

  v4f32 acc[MT][CT][2];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[m][c][0] = acc[m][c][1] = (v4f32){0.f, 0.f, 0.f, 0.f};
  const ConvFrag f(lane);
  const int a_row = wm * 16 * MT, b_row = Tl::BM + wn * 16 * CT;

#pragma unroll
  for (int u = 0; u < NB - 1; ++u) issue(u);
  for (int s = 0; s < n_st; ++s) {
    // this wave's transfers of stage s are done when only its transfers of
    // the NB - 2 stages issued after it remain, and its LDS reads are done; the
    // barrier then makes the whole stage visible and tells every wave that
    // all have finished reading the buffer that stage s - 1 used
    asm volatile("" ::: "memory");
    if (NHI == 0 || wave < NHI)
      __builtin_amdgcn_s_waitcnt(0x0070 | (INFLIGHT & 15) | ((INFLIGHT >> 4) << 14));  // vmcnt(INFLIGHT) lgkmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt(0x0070 | (INFLIGHT_LO & 15) | ((INFLIGHT_LO >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    unsigned char* st = lds + (s % NB) * SBYTES;
    if (s * kConvBK + kConvBK > H) {
      const int valid = (H - s * kConvBK) / 8;  // whole chunks inside the row (hidden % 16 == 0)
      for (int q = tid; q < Tl::ROWS * 8; q += 64 * NW) {
        const int r = q >> 3, pos = q & 7;
        if ((pos ^ (r & 7)) >= valid) *reinterpret_cast<uint4*>(st + r * PITCH + pos * 16) = make_uint4(0u, 0u, 0u, 0u);
      }
      lds_barrier();
    }
    conv_stage<MT, CT, Tl::BC>(st, f, a_row, b_row, acc);
    // stage s + NB - 1 into the buffer stage s - 1 used, issued after this
    // stage's fragment reads so that the wave's MFMAs are not queued behind
    // the transfers (50 against 55 us at 1024 x 3072 issued before them)
    issue(s + NB - 1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no transfer outlives the loop
  conv_mix_store<MT, CT>(acc, x, x0, R, L, H, row0 + wm * 16 * MT, ch0 + wn * 16 * CT, lane, y);
}

template <int MT, int CT, int P, int WM, int WN>
hipError_t launch_conv_mfma(const void* x, const void* x0, const void* Wt, int R, int L, int H, float* y,
                            hipStream_t st) {
  using Tl = ConvTile<MT, CT, WM, WN>;
  const int n_rt = (R + Tl::BM - 1) / Tl::BM;
  const int n_ct = (H + Tl::BC - 1) / Tl::BC;
  const long long blocks = (long long)((n_ct + 7) / 8) * 8 * n_rt;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  launch(conv_mfma_kernel<MT, CT, P, WM, WN>, dim3((unsigned)blocks), dim3(Tl::THREADS), st,
         reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(x0),
         reinterpret_cast<const uint16_t*>(Wt), R, L, H, n_rt, n_ct, y);
  return hipSuccess;
}

template <int MT, int CT, int NB, int WM, int WN>
hipError_t launch_conv_lds(const void* x, const void* x0, const void* Wt, int R, int L, int H, float* y,
                           hipStream_t st) {
  using Tl = ConvTile<MT, CT, WM, WN>;
  const int n_rt = (R + Tl::BM - 1) / Tl::BM;
  const int n_ct = (H + Tl::BC - 1) / Tl::BC;
  const long long blocks = (long long)((n_ct + 7) / 8) * 8 * n_rt;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  launch(conv_lds_kernel<MT, CT, NB, WM, WN>, dim3((unsigned)blocks), dim3(Tl::THREADS), st,
         reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(x0),
         reinterpret_cast<const uint16_t*>(Wt), R, L, H, n_rt, n_ct, y);
  return hipSuccess;
}

__global__ __launch_bounds__(256) void conv_f32_kernel(const float* __restrict__ x, const float* __restrict__ x0,
                                                       const float* __restrict__ Wt, int L, int H,
                                                       float* __restrict__ y) {
  const int row = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
  if (c >= H) return;
  const float* xr = x + (size_t)row * H;
  const float* g0 = Wt + (size_t)c * H;
  const float* g1 = Wt + (size_t)(H + c) * H;
  // 16-byte loads (H % 16 == 0, rows 16-byte aligned), eight of each row in
  // flight per round, four accumulators per tap: one dependent chain over H
  // would pay a memory round trip every few values
  float a0[4] = {0.f, 0.f, 0.f, 0.f}, a1[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < H; k += 32) {
    float4 xv[8], v0[8], v1[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kk = min(k + 4 * u, H - 4);  // past the row end: re-read, not added
      xv[u] = *reinterpret_cast<const float4*>(xr + kk);
      v0[u] = *reinterpret_cast<const float4*>(g0 + kk);
      v1[u] = *reinterpret_cast<const float4*>(g1 + kk);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (k + 4 * u >= H) break;
      a0[0] = fmaf(xv[u].x, v0[u].x, a0[0]);
      a0[1] = fmaf(xv[u].y, v0[u].y, a0[1]);
      a0[2] = fmaf(xv[u].z, v0[u].z, a0[2]);
      a0[3] = fmaf(xv[u].w, v0[u].w, a0[3]);
      a1[0] = fmaf(xv[u].x, v1[u].x, a1[0]);
      a1[1] = fmaf(xv[u].y, v1[u].y, a1[1]);
      a1[2] = fmaf(xv[u].z, v1[u].z, a1[2]);
      a1[3] = fmaf(xv[u].w, v1[u].w, a1[3]);
    }
  }
  const float w0 = (a0[0] + a0[1]) + (a0[2] + a0[3]);
  const float w1 = (a1[0] + a1[1]) + (a1[2] + a1[3]);
  const int t = row % L;
  const float xp = t > 0 ? x[(size_t)(row - 1) * H + c] : x0[(size_t)(row / L) * H + c];
  y[(size_t)row * H + c] = fmaf(w1, xp, w0 * xr[c]);
}

}  // namespace

hipError_t launch_conv2tap(const dflash_dims& d, const void* x, const void* x0, const void* Wt, float* y,
                           hipStream_t st) {
  const int R = d.B * d.L, H = d.hidden;
  if (d.param_dtype == DFLASH_BF16) {
    const long long big = (long long)((R + 127) / 128) * ((H + 63) / 64);
    const long long wide = (long long)((R + 127) / 128) * ((H + 95) / 96);
    const int n_st = (H + kConvBK - 1) / kConvBK;
    // 128 x 96 tiles when they give 7/8 to all of the CUs one block each
    // (they stage the fewest bytes per CU), twelve waves (4 x 3) direct to
    // LDS with three stage buffers (120 KB).  Else 128 x 64 tiles when
    // they alone give every CU a block, eight waves (4 x 2) register-staged
    // with P = 2 stages in flight (P divides the stage count), so that two
    // blocks fit a CU.  Else 64 x 32 tiles, eight waves direct to LDS with
    // four buffers (64 KB).  Measured at 1024 x 3072: 50.4 us for the
    // 128 x 96 tiles direct to LDS (51.8 with eight waves), 56 to 57
    // register-staged (P = 4), 62 to 63 for 128 x 64; at 256 x 2048: 14.5
    // to 15.0 us for the 64 x 32 tiles direct to LDS, 15.6 to 16.3
    // register-staged.
    hipError_t e;
    if (wide >= 224 && wide <= 256) {
      e = launch_conv_lds<2, 2, 3, 4, 3>(x, x0, Wt, R, d.L, H, y, st);
    } else if (big >= 256) {
      e = n_st % 2 == 0 ? launch_conv_mfma<2, 2, 2, 4, 2>(x, x0, Wt, R, d.L, H, y, st)
                        : launch_conv_mfma<2, 2, 1, 4, 2>(x, x0, Wt, R, d.L, H, y, st);
    } else {
      e = launch_conv_lds<1, 1, 4, 4, 2>(x, x0, Wt, R, d.L, H, y, st);
    }
    if (e != hipSuccess) return e;
  } else {
    launch(conv_f32_kernel, dim3((unsigned)((H + 255) / 256), (unsigned)R), dim3(256), st,
           reinterpret_cast<const float*>(x), reinterpret_cast<const float*>(x0), reinterpret_cast<const float*>(Wt),
           d.L, H, y);
  }
  return hipGetLastError();
}

}  // namespace dfk
