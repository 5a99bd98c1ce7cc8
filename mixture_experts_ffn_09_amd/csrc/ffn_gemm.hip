// Grouped expert FFN as a tiled MFMA GEMM (bf16 weights, bf16 activations):
// the form for many rows per expert (prefill, and the shared expert).
//
// Per group g (routed expert, or the shared expert) with rows X_g:
//   pass 1: H = silu(X_g Wg^T) * (X_g Wu^T)   (SwiGLU in the epilogue)
//   pass 2: Y = H Wd^T
// ("Mixture of Experts for LLM Inference", "The MoE change is surprisingly
// local": each expert is a full FFN; "Mixture of Experts Explained", "The
// slot it replaces": three matrices.)
//
// Tiling for gfx950: a 256-thread workgroup computes BM rows x 128 weight
// rows (pass 1: 64 gate/up pairs) with 2 x 2 waves, each wave (BM/2) x 64
// with v_mfma_f32_16x16x32_bf16.  Activation tiles go through LDS, written in
// MFMA-fragment order (every 1 KB is one A operand: lane l holds row l % 16,
// k = 8 * (l / 16) + j), so both the LDS writes and the operand reads are
// contiguous 16-byte accesses.  Weights are pre-packed in the same fragment
// order, so each wave loads its B operands straight from global memory into
// registers, one fully coalesced 1 KB per fragment.  Two LDS stages of 64 K
// each; the next stage's activations and weights are loaded while the
// current one is multiplied.
//
// Tile order: workgroup ids are spread over the 8 XCDs round-robin, so the
// linear tile index is remapped to give each XCD a contiguous range, and the
// range is walked in groups of 8 weight tiles x all row tiles: workgroups
// that run together on one XCD share their weight and activation slices in
// that XCD's L2.  Row tiles are counted on the device (a one-workgroup scan
// of ceil(rows_g / BM)), so no host synchronisation on the counts is needed.

#include "common.h"
#include "kernels.h"

namespace {

constexpr int GM_BN = 128;    // weight rows per workgroup tile
constexpr int GM_BK = 64;     // K per LDS stage
constexpr int GM_GN = 8;      // weight tiles per tile-order group
constexpr int NXCD = 8;

struct GemmParams {
  const uint16_t* a;          // routed activations (row r, or row perm[r])
  const int32_t* perm;        // null: a is expert-contiguous
  const uint16_t* a_sh;       // shared-expert activations (row t)
  const int32_t* offsets;     // [N+1]
  const int32_t* tiles;       // [g1-g0+1] first row tile of each group
  int T, N, g0, g1;
  int K;                      // reduction length
  int n_out;                  // output width (pass 1: d_ff, pass 2: d)
  int NT;                     // weight tiles (GM_BN weight rows each)
  const uint8_t* w;           // packed routed weights
  const uint8_t* w_sh;        // packed shared weights
  const float* s;             // FP8 block scales (routed)
  const float* s_sh;          // FP8 block scales (shared)
  uint16_t* out;
  uint16_t* out_sh;
};

__device__ __forceinline__ void fp8_half_to_bf16(const u32x4_t& q, int half, u32x4_t& o) {
  const uint32_t w0 = half ? q[2] : q[0];
  const uint32_t w1 = half ? q[3] : q[1];
  o[0] = e4m3x2_to_bf16x2<false>(w0);
  o[1] = e4m3x2_to_bf16x2<true>(w0);
  o[2] = e4m3x2_to_bf16x2<false>(w1);
  o[3] = e4m3x2_to_bf16x2<true>(w1);
}

__device__ __forceinline__ void group_rows(const GemmParams& p, int g, int& base, int& rows) {
  if (g < p.N) {
    base = p.offsets[g];
    rows = p.offsets[g + 1] - base;
  } else {
    base = 0;
    rows = p.T;
  }
}

// tiles[i] = sum over groups g0 .. g0+i-1 of ceil(rows_g / bm)
__global__ __launch_bounds__(1024) void tile_schedule_kernel(GemmParams p, int bm,
                                                             int32_t* tiles) {
  __shared__ int32_t sc[1024];
  const int n = p.g1 - p.g0;
  const int i = threadIdx.x;
  int v = 0;
  if (i < n) {
    int base, rows;
    group_rows(p, p.g0 + i, base, rows);
    v = rows > 0 ? (rows + bm - 1) / bm : 0;
  }
  sc[i] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int t = i >= off ? sc[i - off] : 0;
    __syncthreads();
    sc[i] += t;
    __syncthreads();
  }
  if (i < n) tiles[i + 1] = sc[i];
  if (i == 0) tiles[0] = 0;
}

template <int BM, bool GATED, bool FP8>
__global__ __launch_bounds__(256, 1) void ffn_gemm_kernel(GemmParams p) {
  constexpr int MBW = BM / 32;        // 16-row blocks per wave (wave tile BM/2 rows)
  constexpr int NBW = 4;              // 16-row weight blocks per wave
  constexpr int AFR = BM / 16;        // A fragments per 32-K step
  constexpr int ACH = AFR * 64 / 256; // 16-byte A chunks per thread per 32-K step
  constexpr int NH = GATED ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][AFR * 1024];  // [buf][kstep]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile index: XCD remap, then groups of GM_GN weight tiles
  const int ngroups = p.g1 - p.g0;
  const int MT = p.tiles[ngroups];
  const int per = gridDim.x / NXCD;
  const int L = (blockIdx.x % NXCD) * per + blockIdx.x / NXCD;
  if (L >= MT * p.NT) return;
  const int blk = L / (MT * GM_GN);
  const int gw = min(GM_GN, p.NT - blk * GM_GN);
  const int rr = L - blk * MT * GM_GN;
  const int mt = rr / gw;
  const int nt = blk * GM_GN + rr % gw;
  // group of row tile mt (binary search over the tile starts)
  int lo = 0, hi = ngroups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.tiles[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  const int g = p.g0 + lo;
  const int m0 = (mt - p.tiles[lo]) * BM;
  int row_base, rows;
  group_rows(p, g, row_base, rows);
  const bool shared = g >= p.N;
  uint16_t* out = shared ? p.out_sh : p.out;

  const int KT = p.K / GM_BK;    // LDS stages
  // packed weight K steps: 32 wide (bf16) or 64 wide (FP8, two MFMA steps)
  const int KS = FP8 ? p.K / 64 : p.K / 32;
  // weights: this wave's 4 blocks per K step
  const size_t wbytes = (size_t)NH * p.n_out * p.K * (FP8 ? 1 : 2);
  const uint8_t* W = shared ? p.w_sh : p.w + (size_t)g * wbytes;
  const uint8_t* wptr[NBW];
  int srow[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    if (GATED) {
      const int pb = nt * 4 + wn * 2 + (j >> 1);   // gate/up pair block
      wptr[j] = W + (((size_t)pb * KS) * 2 + (j & 1)) * 1024 + lane * 16;
      srow[j] = (j & 1) * (p.n_out / MOE_FP8_BLOCK) + (pb * 16) / MOE_FP8_BLOCK;
    } else {
      const int nb = nt * 8 + wn * 4 + j;
      wptr[j] = W + ((size_t)nb * KS) * 1024 + lane * 16;
      srow[j] = (nb * 16) / MOE_FP8_BLOCK;
    }
  }
  const size_t wstep = (size_t)NH * 1024;  // bytes between K steps of one block
  const int SK = p.K / MOE_FP8_BLOCK;
  const float* S = nullptr;
  if (FP8) S = shared ? p.s_sh : p.s + (size_t)g * NH * (p.n_out / MOE_FP8_BLOCK) * SK;

  // activations: this thread's ACH 16-byte chunks per 32-K step
  const uint16_t* arow[ACH];
#pragma unroll
  for (int c = 0; c < ACH; ++c) {
    const int chunk = tid + 256 * c;
    const int fr = chunk >> 6, l = chunk & 63;
    int r = m0 + fr * 16 + (l & 15);
    r = min(r, rows - 1);  // rows past the end only feed rows that are not stored
    const uint16_t* ptr;
    if (shared)
      ptr = p.a_sh + (size_t)r * p.K;
    else if (p.perm)
      ptr = p.a + (size_t)p.perm[row_base + r] * p.K;
    else
      ptr = p.a + (size_t)(row_base + r) * p.K;
    arow[c] = ptr + (l >> 4) * 8;
  }

  floatx4_t acc[MBW][NBW];
  floatx4_t part[FP8 ? MBW : 1][NBW];  // FP8: sum over the current 128-K scale block
#pragma unroll
  for (int i = 0; i < MBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < (FP8 ? MBW : 1); ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) part[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t ga[2][ACH];      // staged activations of the next stage (2 K steps)
  u32x4_t gb[2][2][NBW];   // weights: [stage parity][K step][block]

  auto load_a = [&](int kt) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c = 0; c < ACH; ++c)
        ga[s][c] = *reinterpret_cast<const u32x4_t*>(arow[c] + kt * GM_BK + s * 32);
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c = 0; c < ACH; ++c)
        *reinterpret_cast<u32x4_t*>(&lds[buf][s][(tid + 256 * c) * 16]) = ga[s][c];
  };
  auto load_b = [&](int par, int kt) {
#pragma unroll
    for (int s = 0; s < (FP8 ? 1 : 2); ++s)
#pragma unroll
      for (int j = 0; j < NBW; ++j)
        gb[par][s][j] = *reinterpret_cast<const u32x4_t*>(
            wptr[j] + (size_t)(FP8 ? kt : kt * 2 + s) * wstep);
  };
  auto compute = [&](int buf, int par) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4_t af[MBW];
#pragma unroll
      for (int i = 0; i < MBW; ++i)
        af[i] = *reinterpret_cast<const u32x4_t*>(&lds[buf][s][((wm * MBW + i) * 64 + lane) * 16]);
      if (!FP8) {
#pragma unroll
        for (int i = 0; i < MBW; ++i)
#pragma unroll
          for (int j = 0; j < NBW; ++j) acc[i][j] = mfma16x16x32(af[i], gb[par][s][j], acc[i][j]);
      } else {
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          u32x4_t bf;
          fp8_half_to_bf16(gb[par][0][j], s, bf);
#pragma unroll
          for (int i = 0; i < (FP8 ? MBW : 1); ++i) part[i][j] = mfma16x16x32(af[i], bf, part[i][j]);
        }
      }
    }
  };
  // FP8: after every second stage a 128-K scale block is complete
  auto close_scale_block = [&](int kt) {
    if (!FP8) return;
    const int kc = kt >> 1;
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const float sc = S[(size_t)srow[j] * SK + kc];
#pragma unroll
      for (int i = 0; i < (FP8 ? MBW : 1); ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] += sc * part[i][j][e];
        part[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  // prologue
  load_a(0);
  load_b(0, 0);
  store_a(0);
  if (KT > 1) load_a(1);
  __syncthreads();

  for (int kt = 0; kt < KT; kt += 2) {
    // even stage: data in lds[0], weights in gb[0]
    if (kt + 1 < KT) load_b(1, kt + 1);
    compute(0, 0);
    if (kt + 1 < KT) {
      store_a(1);
      if (kt + 2 < KT) load_a(kt + 2);
    }
    __syncthreads();
    if (kt + 1 >= KT) break;
    // odd stage: lds[1], gb[1]
    if (kt + 2 < KT) load_b(0, kt + 2);
    compute(1, 1);
    close_scale_block(kt + 1);
    if (kt + 2 < KT) {
      store_a(0);
      if (kt + 3 < KT) load_a(kt + 3);
    }
    __syncthreads();
  }

  // epilogue: acc[i][j] lane holds rows 4*(lane/16)+e of column lane%16
#pragma unroll
  for (int i = 0; i < MBW; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = m0 + (wm * MBW + i) * 16 + (lane >> 4) * 4 + e;
      if (r >= rows) continue;
      uint16_t* orow = out + (size_t)(row_base + r) * p.n_out;
      if (GATED) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int col = (nt * 4 + wn * 2 + q) * 16 + (lane & 15);
          const float v = silu_f32(acc[i][2 * q][e]) * acc[i][2 * q + 1][e];
          orow[col] = (uint16_t)f32_to_bf16(v);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          const int col = (nt * 8 + wn * 4 + j) * 16 + (lane & 15);
          orow[col] = (uint16_t)f32_to_bf16(acc[i][j][e]);
        }
      }
    }
  }
}

}  // namespace

int gemm_row_tile(int avg_rows, bool fp8) { return (!fp8 && avg_rows >= 192) ? 256 : 128; }

bool gemm_shape_ok(int d, int d_ff) { return d % 128 == 0 && d_ff % 64 == 0; }

template <int BM, bool FP8>
static void launch_gemm_kernel(bool gated, long long nwg, const GemmParams& p, hipStream_t st) {
  if (gated)
    ffn_gemm_kernel<BM, true, FP8><<<dim3((unsigned)nwg), 256, 0, st>>>(p);
  else
    ffn_gemm_kernel<BM, false, FP8><<<dim3((unsigned)nwg), 256, 0, st>>>(p);
}

hipError_t launch_ffn_gemm(const FfnArgs& a, int pass, int g0, int g1, int bm, int max_rows,
                           int32_t* sched, hipStream_t st) {
  if (g1 <= g0) return hipSuccess;
  for (int ps = 1; ps <= 2; ++ps) {
    if (!(pass & ps)) continue;
    const bool gated = ps == 1;
    GemmParams p{};
    p.a = gated ? a.x_rows : a.H;
    p.perm = gated ? a.perm_token : nullptr;
    p.a_sh = gated ? a.x_sh : a.H_sh;
    p.offsets = a.offsets;
    p.tiles = sched + (gated ? 0 : 1024);
    p.T = a.T;
    p.N = a.N;
    p.g0 = g0;
    p.g1 = g1;
    p.K = gated ? a.d : a.d_ff;
    p.n_out = gated ? a.d_ff : a.d;
    p.NT = gated ? (2 * a.d_ff) / GM_BN : a.d / GM_BN;
    p.w = static_cast<const uint8_t*>(gated ? a.w13 : a.w2);
    p.w_sh = static_cast<const uint8_t*>(gated ? a.w13_sh : a.w2_sh);
    p.s = gated ? a.s13 : a.s2;
    p.s_sh = gated ? a.s13_sh : a.s2_sh;
    p.out = gated ? a.H : a.Y;
    p.out_sh = gated ? a.H_sh : a.Y_sh;
    tile_schedule_kernel<<<1, 1024, 0, st>>>(p, bm, const_cast<int32_t*>(p.tiles));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // upper bound of row tiles: every group's rows / bm, rounded up per group
    const long long mt_max = (long long)max_rows / bm + (g1 - g0);
    long long nwg = mt_max * p.NT;
    nwg = (nwg + NXCD - 1) / NXCD * NXCD;
    if (a.fp8)
      launch_gemm_kernel<128, true>(gated, nwg, p, st);
    else if (bm == 256)
      launch_gemm_kernel<256, false>(gated, nwg, p, st);
    else
      launch_gemm_kernel<128, false>(gated, nwg, p, st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
