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
// neither the taps nor a transposed copy ever reach HBM.  A block owns 64
// rows (four 16-row MFMA tiles) and 16 channels of both taps (two 16-column
// tiles, rows c and H + c of Wt); its four waves split the k range
// (interleaved 32-wide steps) and their partial tiles are summed through
// LDS in wave order.  Both operands are k-contiguous, so every fragment is
// one 16-byte load per lane.  The row tiles of one channel tile are placed
// on one XCD (block id mod 8), so that tile's Wt rows come from HBM once and
// from that XCD's L2 after.
// fp32 operands: one thread per output, two dot products on the VALU.
#include "device_util.hpp"
#include "internal.hpp"
#include "select_blocks.hpp"

namespace dfk {

namespace {

constexpr int kConvRowTiles = 4;              // 16-row MFMA tiles per block
constexpr int kConvRows = 16 * kConvRowTiles;  // rows per block
constexpr int kConvCh = 16;                    // channels per block (each tap)
constexpr int kConvWaves = 4;

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

__global__ __launch_bounds__(256) void conv_mfma_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ x0,
                                                        const uint16_t* __restrict__ Wt, int R, int L, int H, int n_rt,
                                                        int n_ct, float* __restrict__ y) {
  __shared__ float red[kConvWaves][kConvRowTiles * 2][4][kWave];  // 32 KB
  int rt, ct;
  if (!conv_tile(blockIdx.x, n_rt, n_ct, rt, ct)) return;  // padding ids of the last channel group
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row0 = rt * kConvRows, ch0 = ct * kConvCh;
  const int kl = (lane >> 4) * 8;  // this lane's k offset inside a 32-wide step
  // operand rows of this lane: four x rows (one per row tile) and the two
  // generator rows of channel ch0 + lane % 16 (clamped in range; masked below)
  const uint16_t* ap[kConvRowTiles];
  bool aok[kConvRowTiles];
#pragma unroll
  for (int i = 0; i < kConvRowTiles; ++i) {
    const int row = row0 + i * 16 + (lane & 15);
    aok[i] = row < R;
    ap[i] = x + (size_t)min(row, R - 1) * H + kl;
  }
  const int ch = ch0 + (lane & 15);
  const bool bok = ch < H;
  const uint16_t* bp0 = Wt + (size_t)min(ch, H - 1) * H + kl;
  const uint16_t* bp1 = bp0 + (size_t)H * H;
  const bf16x8 zero = {};
  v4f32 acc[kConvRowTiles][2];
#pragma unroll
  for (int i = 0; i < kConvRowTiles; ++i) acc[i][0] = acc[i][1] = (v4f32){0.f, 0.f, 0.f, 0.f};
  const int n_steps = (H + 31) / 32;
  // two k-steps per iteration: every operand of both loaded before the
  // first MFMA
  for (int s0 = wave; s0 < n_steps; s0 += 2 * kConvWaves) {
    bf16x8 a[2][kConvRowTiles], b[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int s = s0 + u * kConvWaves;
      const int k = s * 32;
      const bool kok = s < n_steps && k + kl < H;
#pragma unroll
      for (int i = 0; i < kConvRowTiles; ++i)
        a[u][i] = kok && aok[i] ? *reinterpret_cast<const bf16x8*>(ap[i] + k) : zero;
      b[u][0] = kok && bok ? *reinterpret_cast<const bf16x8*>(bp0 + k) : zero;
      b[u][1] = kok && bok ? *reinterpret_cast<const bf16x8*>(bp1 + k) : zero;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < kConvRowTiles; ++i)
#pragma unroll
        for (int tap = 0; tap < 2; ++tap)
          acc[i][tap] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][i], b[u][tap], acc[i][tap], 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < kConvRowTiles; ++i)
#pragma unroll
    for (int tap = 0; tap < 2; ++tap)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][i * 2 + tap][e][lane] = acc[i][tap][e];
  __syncthreads();
  // epilogue: 64 rows x 16 channels, four outputs per thread; the MFMA
  // tile holds (row 4 * (lane / 16) + e, column lane % 16) in element e
#pragma unroll
  for (int o = 0; o < kConvRows * kConvCh / 256; ++o) {
    const int p = tid + o * 256;
    const int rl = p / kConvCh, cl = p - (p / kConvCh) * kConvCh;
    const int row = row0 + rl, c = ch0 + cl;
    if (row >= R || c >= H) continue;
    const int i = rl >> 4, rr = rl & 15;
    const int ln = (rr >> 2) * 16 + cl, e = rr & 3;
    float w0 = 0.f, w1 = 0.f;
#pragma unroll
    for (int w = 0; w < kConvWaves; ++w) {
      w0 += red[w][i * 2][e][ln];
      w1 += red[w][i * 2 + 1][e][ln];
    }
    const int t = row % L;
    const float xv = bf16_to_f32(x[(size_t)row * H + c]);
    const float xp = bf16_to_f32(t > 0 ? x[(size_t)(row - 1) * H + c] : x0[(size_t)(row / L) * H + c]);
    y[(size_t)row * H + c] = fmaf(w1, xp, w0 * xv);
  }
}

__global__ __launch_bounds__(256) void conv_f32_kernel(const float* __restrict__ x, const float* __restrict__ x0,
                                                       const float* __restrict__ Wt, int L, int H,
                                                       float* __restrict__ y) {
  const int row = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
  if (c >= H) return;
  const float* xr = x + (size_t)row * H;
  const float* g0 = Wt + (size_t)c * H;
  const float* g1 = Wt + (size_t)(H + c) * H;
  float w0 = 0.f, w1 = 0.f;
  for (int k = 0; k < H; ++k) {
    w0 = fmaf(xr[k], g0[k], w0);
    w1 = fmaf(xr[k], g1[k], w1);
  }
  const int t = row % L;
  const float xp = t > 0 ? x[(size_t)(row - 1) * H + c] : x0[(size_t)(row / L) * H + c];
  y[(size_t)row * H + c] = fmaf(w1, xp, w0 * xr[c]);
}

}  // namespace

hipError_t launch_conv2tap(const dflash_dims& d, const void* x, const void* x0, const void* Wt, float* y,
                           hipStream_t st) {
  const int R = d.B * d.L, H = d.hidden;
  if (d.param_dtype == DFLASH_BF16) {
    const int n_rt = (R + kConvRows - 1) / kConvRows;
    const int n_ct = (H + kConvCh - 1) / kConvCh;
    const long long blocks = (long long)((n_ct + 7) / 8) * 8 * n_rt;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    launch(conv_mfma_kernel, dim3((unsigned)blocks), dim3(256), st, reinterpret_cast<const uint16_t*>(x),
           reinterpret_cast<const uint16_t*>(x0), reinterpret_cast<const uint16_t*>(Wt), R, d.L, H, n_rt, n_ct, y);
  } else {
    launch(conv_f32_kernel, dim3((unsigned)((H + 255) / 256), (unsigned)R), dim3(256), st,
           reinterpret_cast<const float*>(x), reinterpret_cast<const float*>(x0), reinterpret_cast<const float*>(Wt),
           d.L, H, y);
  }
  return hipGetLastError();
}

}  // namespace dfk
