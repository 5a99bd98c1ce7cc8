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
// Two tilings for gfx950, both on v_mfma_f32_16x16x32_bf16:
//  * bf16 weights: 4 waves, one per SIMD, accumulators in AGPRs; tiles of
//    256 weight rows x 256 activation rows, the last tile of a group cut to
//    64 or 128 rows when that holds its remaining rows
//    (ffn_gemm_big_kernel below).
//  * FP8 weights (and shapes past 32-bit operand offsets): 128-row tiles in a
//    512-thread workgroup (8 waves, two per SIMD, so one wave's LDS or
//    barrier wait is covered by the other's MFMAs), 2 x 4 waves of 64 x 64.
// Both operands reach LDS through direct global-to-LDS loads (each lane's 16
// bytes land at lane * 16 of a 1 KB block), so no registers are spent on
// staging.  Every 1 KB in LDS is one MFMA operand (lane l holds row l % 16,
// k = 8 * (l / 16) + j): the activation copy picks its global addresses to
// produce that order and the weights are pre-packed in it, so operand reads
// are contiguous ds_read_b128.  A ring of stages (32 K each; 64 for FP8)
// keeps the copies of the next stages in flight while one is multiplied.
//
// Tile order: workgroup ids are spread over the 8 XCDs round-robin, so the
// linear tile index is remapped to give each XCD a contiguous range, and the
// range is walked in groups of a few weight tiles x all row tiles (4, or 8
// on the four-wave kernel's down pass): workgroups that run together on one
// XCD share their weight and activation slices in that XCD's L2.  Row tiles
// are counted on the device (a one-workgroup scan of ceil(rows_g / BM)), so
// no host synchronisation on the counts is needed.  On the four-wave kernel
// a short last round of tiles on an XCD runs as parts of the tiles' weight
// rows (xcd_unit), so that round does not leave most CUs idle.

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int GM_BN = 256;    // weight rows per workgroup tile
constexpr int GM_GN = 4;      // weight tiles per tile-order group
constexpr int NXCD = 8;
constexpr int FW_LDS = 160 * 1024;  // LDS of the four-wave kernel

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
  const uint8_t* s4;          // MXFP4 E8M0 scales, packed (routed)
  const uint8_t* s4_sh;       // MXFP4 E8M0 scales, packed (shared)
  uint16_t* out;
  uint16_t* out_sh;
};

// Linear tile index of this workgroup, or -1 if it has none.  Workgroups are
// dealt to the XCDs round-robin (XCD = blockIdx % 8) and dispatched in
// blockIdx order; the grid is an upper bound of the tile count, so the real
// count (known only on the device) is cut into 8 equal contiguous ranges, one
// per XCD, and the workgroups past a range exit.  Every XCD gets the same
// share of the work, and the live workgroups are the first ones dispatched.
// Needs gridDim.x to be a multiple of 8 and at least the tile count.
__device__ __forceinline__ int xcd_tile(int total) {
  const int per = (total + NXCD - 1) / NXCD;
  const int slot = blockIdx.x / NXCD;
  const int L = (blockIdx.x % NXCD) * per + slot;
  return (slot < per && L < total) ? L : -1;
}

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

// Wait until at most `later` stages of LPS copies each are still in flight
// (later <= MAXL, a run-time value turned into an immediate).
template <int LPS, int MAXL>
__device__ __forceinline__ void wait_stages(int later) {
  static_assert(MAXL >= 0 && MAXL <= 6, "ring depth");
  if (MAXL >= 6 && later >= 6) wait_vmcnt<(MAXL >= 6 ? 6 : 0) * LPS>();
  else if (MAXL >= 5 && later == 5) wait_vmcnt<(MAXL >= 5 ? 5 : 0) * LPS>();
  else if (MAXL >= 4 && later == 4) wait_vmcnt<(MAXL >= 4 ? 4 : 0) * LPS>();
  else if (MAXL >= 3 && later == 3) wait_vmcnt<(MAXL >= 3 ? 3 : 0) * LPS>();
  else if (MAXL >= 2 && later == 2) wait_vmcnt<(MAXL >= 2 ? 2 : 0) * LPS>();
  else if (MAXL >= 1 && later == 1) wait_vmcnt<LPS>();
  else wait_vmcnt<0>();
}

template <int BM, bool GATED, bool FP8>
__global__ __launch_bounds__(512, 1) void ffn_gemm_kernel(GemmParams p) {
  constexpr int NWN = 4;              // wave grid 2 x 4 (8 waves, two per SIMD)
  constexpr int MBW = BM / 32;        // 16-row blocks per wave (wave tile BM/2 rows)
  constexpr int NBW = 4;              // 16-row weight blocks per wave (wave tile 64 wide)
  constexpr int AFR = BM / 16;        // activation fragments per 32-K step
  constexpr int WBL = NWN * NBW;      // weight blocks per tile (GM_BN / 16)
  constexpr int NH = GATED ? 2 : 1;
  // One stage = SK 32-K steps (FP8: 2, the width of one packed block).
  constexpr int SK = FP8 ? 2 : 1;
  constexpr int A_BYTES = SK * AFR * 1024;
  constexpr int B_FRAGS = WBL * (FP8 ? 1 : SK);
  constexpr int STAGE = A_BYTES + B_FRAGS * 1024;
  // ring depth: bf16 keeps three 24 KB stages so that two workgroups share a
  // CU (their barriers interleave; measured faster than one workgroup with
  // four to six stages); fp8 keeps up to four 32 KB stages
  constexpr int NS = FP8 ? ((160 * 1024 / STAGE) < 4 ? (160 * 1024 / STAGE) : 4) : 3;
  constexpr int A_PER_WAVE = SK * AFR / 8;
  constexpr int B_PER_WAVE = B_FRAGS / 8;
  constexpr int LPS = A_PER_WAVE + B_PER_WAVE;  // copies per wave per stage
  constexpr int KSTAGE = 32 * SK;
  static_assert(GM_BN == WBL * 16, "tile width");
  static_assert(NS >= 2 && (NS - 2) * LPS < 64, "ring");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;

  // ---- tile index: XCD remap, then groups of GM_GN weight tiles
  const int ngroups = p.g1 - p.g0;
  const int MT = p.tiles[ngroups];
  const int L = xcd_tile(MT * p.NT);
  if (L < 0) return;
  const int blk = L / (MT * GM_GN);
  const int gw = min(GM_GN, p.NT - blk * GM_GN);
  const int rr = L - blk * MT * GM_GN;
  const int mt = rr / gw;
  const int nt = blk * GM_GN + rr % gw;
  int lo = 0, hi = ngroups - 1;  // group of row tile mt
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

  const int KT = p.K / KSTAGE;                // stages over K
  const int KS = FP8 ? p.K / 64 : p.K / 32;   // packed weight K steps
  const size_t wbytes = (size_t)NH * p.n_out * p.K * (FP8 ? 1 : 2);
  const uint8_t* W = shared ? p.w_sh : p.w + (size_t)g * wbytes;
  const size_t wstep = (size_t)NH * 1024;     // bytes between K steps of one block

  // Weight block jb of the tile: gated -> pair nt*8 + jb/2, gate (even) or
  // up (odd); down -> row block nt*16 + jb.
  auto block_offset = [&](int jb) -> size_t {
    if (GATED) {
      const int pb = nt * (WBL / 2) + (jb >> 1);
      return (((size_t)pb * KS) * 2 + (jb & 1)) * 1024;
    }
    return ((size_t)(nt * WBL + jb) * KS) * 1024;
  };
  const uint8_t* bsrc[B_PER_WAVE];
  int bdst[B_PER_WAVE], bks[B_PER_WAVE];
#pragma unroll
  for (int i = 0; i < B_PER_WAVE; ++i) {
    const int q = wave * B_PER_WAVE + i;
    const int jb = FP8 ? q : (q % WBL);
    const int sb = FP8 ? 0 : (q / WBL);
    bsrc[i] = W + block_offset(jb) + lane * 16;
    bks[i] = sb;
    bdst[i] = A_BYTES + (FP8 ? jb : (sb * WBL + jb)) * 1024;
  }
  const uint16_t* asrc[A_PER_WAVE];
  int adst[A_PER_WAVE];
#pragma unroll
  for (int i = 0; i < A_PER_WAVE; ++i) {
    const int q = wave * A_PER_WAVE + i;
    const int mb = q % AFR, sa = q / AFR;
    const int r = min(m0 + mb * 16 + (lane & 15), rows - 1);  // rows past the end are not stored
    const uint16_t* ptr;
    if (shared)
      ptr = p.a_sh + (size_t)r * p.K;
    else if (p.perm)
      ptr = p.a + (size_t)p.perm[row_base + r] * p.K;
    else
      ptr = p.a + (size_t)(row_base + r) * p.K;
    asrc[i] = ptr + (lane >> 4) * 8 + sa * 32;
    adst[i] = (sa * AFR + mb) * 1024;
  }
  auto issue_stage = [&](int kt) {
    uint8_t* base = lds + (kt % NS) * STAGE;
#pragma unroll
    for (int i = 0; i < A_PER_WAVE; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(asrc[i] + kt * KSTAGE),
                                       (void*)(base + adst[i]), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < B_PER_WAVE; ++i)
      __builtin_amdgcn_global_load_lds(
          (const void*)(bsrc[i] + (size_t)(FP8 ? kt : kt * SK + bks[i]) * wstep),
          (void*)(base + bdst[i]), 16, 0, 0);
  };

  // FP8 scales of this wave's blocks
  int srow[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const int jb = wn * NBW + j;
    if (GATED)
      srow[j] = (jb & 1) * (p.n_out / MOE_FP8_BLOCK) + ((nt * (WBL / 2) + (jb >> 1)) * 16) / MOE_FP8_BLOCK;
    else
      srow[j] = ((nt * WBL + jb) * 16) / MOE_FP8_BLOCK;
  }
  const int SKB = p.K / MOE_FP8_BLOCK;
  const float* S = nullptr;
  if (FP8) S = shared ? p.s_sh : p.s + (size_t)g * NH * (p.n_out / MOE_FP8_BLOCK) * SKB;

  floatx4_t acc[MBW][NBW];
  floatx4_t part[FP8 ? MBW : 1][NBW];
#pragma unroll
  for (int i = 0; i < MBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < (FP8 ? MBW : 1); ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) part[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // prologue: NS-1 stages in flight
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < KT) issue_stage(st);

  for (int kt = 0; kt < KT; ++kt) {
    // stage kt has landed (this wave's copies): later stages may still fly
    wait_stages<LPS, NS - 2>(min(NS - 2, KT - 1 - kt));
    // everyone's copies of stage kt are visible, and stage kt-1 is no
    // longer read: its buffer takes stage kt+NS-1
    barrier_no_fence();
    if (kt + NS - 1 < KT) issue_stage(kt + NS - 1);
    const uint8_t* base = lds + (kt % NS) * STAGE;
    u32x4_t bq[NBW];
    if (FP8) {
#pragma unroll
      for (int j = 0; j < NBW; ++j)
        bq[j] = *reinterpret_cast<const u32x4_t*>(base + A_BYTES + (wn * NBW + j) * 1024 + lane * 16);
    }
#pragma unroll
    for (int s2 = 0; s2 < SK; ++s2) {
      u32x4_t af[MBW], bf[NBW];
#pragma unroll
      for (int i = 0; i < MBW; ++i)
        af[i] = *reinterpret_cast<const u32x4_t*>(base + (s2 * AFR + wm * MBW + i) * 1024 + lane * 16);
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        if (!FP8)
          bf[j] = *reinterpret_cast<const u32x4_t*>(base + A_BYTES + (s2 * WBL + wn * NBW + j) * 1024 +
                                                    lane * 16);
        else
          fp8_half_to_bf16(bq[j], s2, bf[j]);
      }
      __builtin_amdgcn_sched_barrier(0);  // all operand reads issued before the MFMAs
#pragma unroll
      for (int i = 0; i < MBW; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          if (!FP8)
            acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
          else
            part[i < (FP8 ? MBW : 1) ? i : 0][j] =
                mfma16x16x32(af[i], bf[j], part[i < (FP8 ? MBW : 1) ? i : 0][j]);
        }
    }
    if (FP8 && (kt & 1)) {  // a 128-K scale block is complete
      const int kc = kt >> 1;
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const float sc = S[(size_t)srow[j] * SKB + kc];
#pragma unroll
        for (int i = 0; i < (FP8 ? MBW : 1); ++i) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] += sc * part[i][j][e];
          part[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    // this wave's operand reads of stage kt are complete before the next
    // barrier lets its buffer be refilled
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
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
        for (int q = 0; q < NBW / 2; ++q) {
          const int col = (nt * (WBL / 2) + wn * (NBW / 2) + q) * 16 + (lane & 15);
          const float v = silu_f32(acc[i][2 * q][e]) * acc[i][2 * q + 1][e];
          orow[col] = (uint16_t)f32_to_bf16(v);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          const int col = (nt * WBL + wn * NBW + j) * 16 + (lane & 15);
          orow[col] = (uint16_t)f32_to_bf16(acc[i][j][e]);
        }
      }
    }
  }
}

// Four-wave form for bf16 weights (one wave per SIMD, one workgroup per CU):
// a tile is 256 weight rows wide and 64, 128 or 256 rows tall.  A group of r
// rows takes ceil(r / 256) tiles; all are 256 rows tall except the last,
// which is the smallest of 64, 128, 256 that holds the rows left.  So a group
// never streams its weights more often than ceil(r / 256) times, and a small
// group (most of them, with many experts) costs MFMA work in proportion to
// its rows.  Tall and short tiles share one launch: short tiles are bound by
// the weight stream, tall ones by the MFMAs, and running them side by side
// lets the two limits overlap.
//
// Wave layout and work per 32-K step (per wave):
//   256 rows: 2 x 2 waves of 128 x 128; 16 fragment reads, 64 MFMAs
//             (MXFP4: 1 x 4 waves of 256 x 64, 16 activation fragments and
//             4 weight fragments, so each weight fragment is decoded by one
//             wave instead of two: half the decode work per MFMA)
//   128 rows: 1 x 4 waves of 128 x  64; 12 fragment reads, 32 MFMAs
//    64 rows: 1 x 4 waves of  64 x  64;  8 fragment reads, 16 MFMAs
// The accumulators live in AGPRs.  With a single wave per SIMD nothing hides
// a stall, so each step spreads its copies and fragment reads evenly between
// its MFMAs instead of issuing them in bursts.
//
// Operand copies.  The copy path is limited by the cache lines each copy
// instruction touches more than by bytes: a 1 KB weight block touches 8 lines,
// while a 16-row x 32-K activation fragment (64 bytes of each of 16 gathered
// rows) touches 16.  So the activation rows are copied two K steps at a time,
// 8 rows x 128 bytes (8 whole lines) per instruction, into a ring of "pair"
// buffers holding steps 2p and 2p+1; the weights keep a ring of NS one-step
// buffers.  Inside a fragment's 2 KB of a pair buffer, row r (of 16), K group
// g (8 inputs) and step parity s sit at
//   (r / 8) * 1024 + (r % 8) * 128 + ((4 s + g) ^ ((r / 2) % 8)) * 16,
// so each row's 128 bytes of the pair are one 128-byte LDS line, filled by 8
// consecutive lanes of a copy instruction (lane i writes offset 16 i and
// fetches the piece that belongs there: 8 rows per instruction, one whole
// cache line each), while the XOR spreads an MFMA operand read (lane l: row
// l % 16, group l / 16) over all banks.
//
// Schedule: the copies issued at step kt are those of step j = kt + NS - 1
// (clamped to the last step): its weight blocks and one half of an
// activation pair (rows 0-7 of pair (j + 1) / 2 when j is odd, rows 8-15
// when j is even), so every step issues the same number of copies.  At the
// top of step kt a wave waits until the copies of steps up to kt + 1 have
// landed, then a barrier makes every wave's copies visible; the fragments of
// step kt + 1 are read during step kt.  A pair buffer is rewritten only after
// the barrier that follows its last read (2 NPA >= NS + 1).

// MXFP4 weights (FP4): the packed 1 KB blocks hold 16 weight rows x 128
// inputs (four 32-K steps; lane l's 16 bytes are four words of 8 E2M1 codes,
// word s the B operand of step s), so the weight ring holds NQ "quads" of
// four steps each, WBL blocks per quad, plus each block's E8M0 scales of the
// quad (16 rows x 4 bytes, one byte per 32 inputs, in a 256-byte slot).  Copy step j carries,
// besides its activation half-pair, one weight block and its scale bytes of
// quad j / 4 + 1 per wave (block (4 (j % 4) + wave) % WBL, so the four
// waves and four steps cover all WBL blocks); so every step still issues the
// same number of copies, quad 0 comes in copy steps -4 .. -1 of the prologue,
// and quad q is read during steps 4 q - 1 .. 4 q + 2.  A quad buffer is
// rewritten only after the barrier that follows its last read
// (4 NQ >= NS + 6).  The operand reads of a step are one code word and one
// scale byte per block; they are decoded exactly to bf16 (a power of two
// times an E2M1 value) at the end of the step before, in the shadow of the
// step's last MFMAs.
//
// One tile: WM x (4 / WM) waves, each MBW x NBW blocks of 16 x 16; NS weight
// steps (bf16) and NPA activation pairs in LDS.  The tile's weight rows are
// the WN * NBW 16-row blocks from block nb0 on (gate/up: interleaved pairs,
// nb0 even): a whole 256-row weight tile, or a part of one.
template <bool GATED, int WM, int MBW, int NBW, int NS, int NPA, bool FP4 = false>
__device__ __forceinline__ void four_wave_tile(const GemmParams& p, uint8_t* lds, int g,
                                               int row_base, int rows, int m0, int nb0) {
  constexpr int WN = 4 / WM;
  constexpr int BM = WM * MBW * 16;
  constexpr int AFR = BM / 16;        // activation fragments per step
  constexpr int WBL = WN * NBW;       // weight blocks per step
  static_assert(WBL % 4 == 0 && (!GATED || NBW % 2 == 0), "tile width");
  static_assert(AFR % 4 == 0, "activation fragments are copied four waves at a time");
  constexpr int NH = GATED ? 2 : 1;
  constexpr int NQ = 3;                        // FP4: quad buffers
  constexpr int B_STEP = WBL * 1024;           // one weight step (FP4: quad) in LDS
  constexpr int B_BUFS = FP4 ? NQ : NS;
  constexpr int S_QUAD = WBL * 256;            // FP4: scales of one quad (64 of 256 bytes used)
  constexpr int S_RING = FP4 ? NQ * S_QUAD : 0;
  constexpr int A_PAIR = AFR * 2048;           // one activation pair in LDS
  constexpr int B_PER_WAVE = FP4 ? 2 : WBL / 4;  // weight (FP4: block + scale) copies
  constexpr int A_HALF = AFR / 4;              // activation copies per wave per step
  constexpr int LPS = B_PER_WAVE + A_HALF;     // copies per wave per step
  constexpr int NRD = MBW + (FP4 ? 2 : 1) * NBW;  // operand reads per wave per step
  constexpr int NMF = MBW * NBW;               // MFMAs per wave per step
  static_assert(B_BUFS * B_STEP + S_RING + NPA * A_PAIR <= FW_LDS, "LDS");
  static_assert(NS >= 3 && 2 * NPA >= NS + 1 && (NS - 2) * LPS < 64, "ring");
  static_assert(!FP4 || 4 * NQ >= NS + 6, "quad ring");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const bool shared = g >= p.N;
  uint16_t* out = shared ? p.out_sh : p.out;
  uint8_t* const bring = lds;
  uint8_t* const sring = lds + B_BUFS * B_STEP;
  uint8_t* const aring = sring + S_RING;

  const int KT = p.K / 32;
  const int KQ4 = p.K / 128;                   // FP4: quads (packed K steps)
  const int KQ = (KT + 15) / 16;               // FP4: 256-byte scale chunks per row block
  const size_t wbytes = FP4 ? (size_t)NH * p.n_out * p.K / 2 : (size_t)NH * p.n_out * p.K * 2;
  const uint8_t* W = shared ? p.w_sh : p.w + (size_t)g * wbytes;
  const size_t wstep = (size_t)NH * 1024;

  // Copies are buffer loads straight into LDS: the per-lane byte offsets stay
  // in VGPRs for the whole loop and the K advance is a scalar offset.  Reads
  // past a resource's size return zero.
  const __amdgpu_buffer_rsrc_t wres =
      __builtin_amdgcn_make_buffer_rsrc((void*)W, 0, (int)(uint32_t)wbytes, BUF_DWORD3);
  // weight block jb of the tile: its 16-row block and gate/up half
  auto block_rh = [&](int jb, int& rb, int& h) {
    if (GATED) {
      rb = nb0 / 2 + (jb >> 1);
      h = jb & 1;
    } else {
      rb = nb0 + jb;
      h = 0;
    }
  };
  // bf16: block jb = wave * B_PER_WAVE + i; FP4: the block of sub-step i
  constexpr int NBO = FP4 ? 4 : B_PER_WAVE;
  uint32_t boff[NBO];
  int bdst[NBO];
#pragma unroll
  for (int i = 0; i < NBO; ++i) {
    const int jb = FP4 ? (4 * i + wave) % WBL : wave * B_PER_WAVE + i;
    int rb, h;
    block_rh(jb, rb, h);
    const uint32_t ksteps = FP4 ? (uint32_t)KQ4 : (uint32_t)KT;
    boff[i] = (((uint32_t)rb * ksteps) * NH + h) * 1024 + lane * 16;
    bdst[i] = jb * 1024;
  }
  // FP4 scales: chunk (row block, 4 quads, gate/up) of 16 rows x 16 bytes;
  // lane i < 16 copies row i's 4 bytes of a quad
  const uint8_t* S4 = nullptr;
  uint32_t sbytes = 0;
  if (FP4) {
    sbytes = (uint32_t)((size_t)NH * p.n_out * KQ * 16);
    S4 = shared ? p.s4_sh : p.s4 + (size_t)g * sbytes;
  }
  const __amdgpu_buffer_rsrc_t sres =
      __builtin_amdgcn_make_buffer_rsrc((void*)S4, 0, (int)sbytes, BUF_DWORD3);
  uint32_t soff[FP4 ? 4 : 1];
#pragma unroll
  for (int i = 0; i < (FP4 ? 4 : 0); ++i) {
    int rb, h;
    block_rh((4 * i + wave) % WBL, rb, h);
    soff[i] = (((uint32_t)rb * KQ) * NH + h) * 256 + (lane & 15) * 16;
  }
  const uint16_t* abase = shared ? p.a_sh : p.a;
  const uint32_t abytes = (uint32_t)((size_t)(shared ? rows : (p.perm ? p.T : row_base + rows)) * p.K * 2);
  const __amdgpu_buffer_rsrc_t ares =
      __builtin_amdgcn_make_buffer_rsrc((void*)abase, 0, (int)abytes, BUF_DWORD3);
  // activation copy (q, h) of this wave: fragment f = wave * A_HALF + q,
  // rows 8 h .. 8 h + 7 of it, both steps of a pair; lane i fetches row
  // r = 8 h + i / 8 and the 16 bytes (4 s + g) = (i % 8) ^ ((r / 2) % 8) of its
  // 128 bytes
  uint32_t aoff[A_HALF][2];
  int adst[A_HALF][2];
#pragma unroll
  for (int c = 0; c < 2 * A_HALF; ++c) {
    const int q = c >> 1, h = c & 1;
    const int f = wave * A_HALF + q;
    const int rf = 8 * h + (lane >> 3);         // row within the fragment
    const int r = min(m0 + f * 16 + rf, rows - 1);  // rows past the end are not stored
    int src;
    if (shared)
      src = r;
    else if (p.perm)
      src = p.perm[row_base + r];
    else
      src = row_base + r;
    const int piece = (lane & 7) ^ ((rf >> 1) & 7);  // 4 s + g
    aoff[q][h] = (uint32_t)src * (uint32_t)p.K * 2 + piece * 16;
    adst[q][h] = f * 2048 + h * 1024;
  }
  // operand read of lane l: row l % 16, K group l / 16 (activations: offset
  // within a fragment's 2 KB for an even and an odd step)
  const int rl = lane & 15, gl = lane >> 4;
  const int a_rd0 = (rl >> 3) * 1024 + (rl & 7) * 128 + (gl ^ ((rl >> 1) & 7)) * 16;
  const int a_rd1 = (rl >> 3) * 1024 + (rl & 7) * 128 + ((4 + gl) ^ ((rl >> 1) & 7)) * 16;

  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  // copy number q of step j (weights first, then half (j + 1) % 2 of the
  // activation pair (j + 1) / 2; j = -1 has only the latter in bf16)
  auto copy_one = [&](int q, int j) {
    if (FP4 && q < B_PER_WAVE) {
      // block (4 (j % 4) + wave) % WBL of quad j / 4 + 1 (source clamped to
      // the last quad; the buffer index is not)
      const int qd = (j >> 2) + 1, sub = j & 3;
      const int qc = min(qd, KQ4 - 1);
      if (q == 0) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wres, (lds_ptr_t)(bring + (qd % NQ) * B_STEP + bdst[sub]), 16, boff[sub],
            qc * (int)wstep, 0, 0);
      } else {
        // every lane copies 4 bytes to slot offset 4 * lane: lanes 16..63 repeat
        // rows 0..15 into the unused 192 bytes of the block's 256-byte slot
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            sres, (lds_ptr_t)(sring + (qd % NQ) * S_QUAD + (bdst[sub] >> 2)), 4, soff[sub],
            ((qc >> 2) * NH) * 256 + (qc & 3) * 4, 0, 0);
      }
    } else if (q < B_PER_WAVE) {
      const int kl = min(j, KT - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wres, (lds_ptr_t)(bring + (j % NS) * B_STEP + bdst[q]), 16, boff[q],
          kl * (int)wstep, 0, 0);
    } else {
      const int pr = (j + 1) >> 1, h = (j + 1) & 1;
      const int pl = min(pr, KT / 2 - 1);
      const int qa = q - B_PER_WAVE;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ares, (lds_ptr_t)(aring + (pr % NPA) * A_PAIR + adst[qa][h]), 16, aoff[qa][h],
          pl * 128, 0, 0);
    }
  };

  floatx4_t acc[MBW][NBW];
#pragma unroll
  for (int i = 0; i < MBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t ca[MBW], cb[NBW], na[MBW], nb[NBW];
  uint32_t rc[FP4 ? NBW : 1], rs[FP4 ? NBW : 1];  // FP4: code words and scale bytes
  // fragment f of step kt: f < MBW are activation blocks, the rest weight blocks
  // (FP4: NBW code words, then NBW scale bytes) (odd: the parity of kt, known
  // where it is called)
  // The ring slots are uniform values passed through readfirstlane: opaque to
  // loop strength reduction, which would otherwise keep one address register
  // per fragment and correct each of them every step (on the MXFP4 gate/up
  // pass 54 of its 138 vector instructions per two steps); so a read is a
  // lane base plus the slot plus a constant that the instruction carries.
  // The bf16 down pass keeps the plain arithmetic for its weight reads: with
  // those opaque too it runs out of registers.
  constexpr bool OPAQUE_B = FP4 || GATED;
  auto read_one = [&](u32x4_t (&fa)[MBW], u32x4_t (&fb)[NBW], int f, int kt, bool odd) {
    if (f < MBW) {
      const int slot = __builtin_amdgcn_readfirstlane(((kt >> 1) % NPA) * A_PAIR);
      fa[f] = *reinterpret_cast<const u32x4_t*>(aring + slot + (odd ? a_rd1 : a_rd0) +
                                                (wm * MBW + f) * 2048);
    } else if (FP4) {
      const int qd = kt >> 2, sub = kt & 3;
      const int j = (f - MBW) % NBW;
      if (f < MBW + NBW) {
        const int slot = __builtin_amdgcn_readfirstlane((qd % NQ) * B_STEP + sub * 4);
        rc[FP4 ? j : 0] = *reinterpret_cast<const uint32_t*>(bring + slot + lane * 16 +
                                                             (wn * NBW + j) * 1024);
      } else {
        const int slot = __builtin_amdgcn_readfirstlane((qd % NQ) * S_QUAD + sub);
        rs[FP4 ? j : 0] = *(sring + slot + (lane & 15) * 4 + (wn * NBW + j) * 256);
      }
    } else if constexpr (OPAQUE_B) {
      const int slot = __builtin_amdgcn_readfirstlane((kt % NS) * B_STEP);
      fb[f - MBW] = *reinterpret_cast<const u32x4_t*>(bring + slot + lane * 16 +
                                                      (wn * NBW + f - MBW) * 1024);
    } else {
      fb[f - MBW] = *reinterpret_cast<const u32x4_t*>(
          bring + (kt % NS) * B_STEP + ((wn * NBW + f - MBW) * 64 + lane) * 16);
    }
  };
  // FP4: the weight operands of the step just read
  auto decode = [&](u32x4_t (&fb)[NBW]) {
#pragma unroll
    for (int j = 0; j < (FP4 ? NBW : 0); ++j) fb[j] = fp4_word_to_bf16(rc[FP4 ? j : 0], rs[FP4 ? j : 0]);
  };
  // Step kt (PAR = kt & 1): wait until the copies of step kt+1 have landed for
  // every wave, then run step kt's MFMAs with two streams interleaved: the
  // copies of step kt+NS-1 and the fragment reads of step kt+1.  The clamped
  // copies near the end only land in buffers no later step reads, and the
  // reads past the last step land in registers that are never used.
  auto stage = [&](auto par, const u32x4_t (&fa)[MBW], const u32x4_t (&fb)[NBW],
                   u32x4_t (&ga)[MBW], u32x4_t (&gb)[NBW], int kt) {
    constexpr int PAR = decltype(par)::value;
    // copies still allowed in flight: those of steps kt+2 .. kt+NS-2
    wait_vmcnt<(NS - 3) * LPS>();
    barrier_no_fence();
    __builtin_amdgcn_sched_barrier(0);
    // program order already alternates copies and reads, as the compiler may
    // not move an LDS read past a copy into LDS
#pragma unroll
    for (int q = 0; q < LPS; ++q) {
      copy_one(q, kt + NS - 1);
#pragma unroll
      for (int f = q * NRD / LPS; f < (q + 1) * NRD / LPS; ++f)
        read_one(ga, gb, f, kt + 1, PAR == 0);
    }
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j) acc[i][j] = mfma16x16x32(fa[i], fb[j], acc[i][j]);
    if constexpr (FP4 && GATED) {
      // copies and operand reads between the first half of the MFMAs, the
      // decode of the next step's weight operands (5 vector instructions per
      // block: 4 conversions and the scale shift) between the second half
      decode(gb);
      stage_pattern<0, LPS, NRD, NMF / 2>();
      decode_pattern<0, NBW, 5, NMF - NMF / 2>();
      __builtin_amdgcn_sched_barrier(0);
    } else {
      stage_pattern<0, LPS, NRD, NMF>();
      __builtin_amdgcn_sched_barrier(0);
      if (FP4) {
        // the down pass decodes after the MFMAs (interleaving them would
        // spill registers there)
        decode(gb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // K/32 is even (and at least 4) for every accepted shape
  if (FP4) {
    // quad 0: weight blocks and scales of copy steps -4 .. -1
#pragma unroll
    for (int j = -4; j < -1; ++j)
#pragma unroll
      for (int q = 0; q < B_PER_WAVE; ++q) copy_one(q, j);
#pragma unroll
    for (int q = 0; q < LPS; ++q) copy_one(q, -1);
  } else {
#pragma unroll
    for (int q = B_PER_WAVE; q < LPS; ++q) copy_one(q, -1);
  }
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
#pragma unroll
    for (int q = 0; q < LPS; ++q) copy_one(q, j);
  wait_vmcnt<(NS - 2) * LPS>();  // the copies of steps -1 and 0 have landed
  barrier_no_fence();
#pragma unroll
  for (int f = 0; f < NRD; ++f) read_one(ca, cb, f, 0, false);
  if (FP4) decode(cb);

  for (int kt = 0; kt < KT; kt += 2) {
    stage(std::integral_constant<int, 0>{}, ca, cb, na, nb, kt);
    stage(std::integral_constant<int, 1>{}, na, nb, ca, cb, kt + 1);
  }
  wait_vmcnt<0>();  // the clamped copies of the last steps
  // Pin every accumulator to its AGPRs at the end of the loop (an empty asm
  // statement, no instruction).  Without it the register allocator gives the
  // down pass's MFMAs of the smaller tiles destinations other than their
  // accumulator inputs and copies the accumulators back at every loop latch
  // (three moves per MFMA on the 128-row down tile), apparently to suit the
  // epilogue's read order.  The 256-accumulator tile needs no pin (and with
  // one it spills a register).
  if constexpr (MBW * NBW < 64) {
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
      for (int j = 0; j < NBW; ++j) asm volatile("" : "+a"(acc[i][j]));
  }

  // Epilogue through LDS.  A lane holds 4 rows of one column of each 16 x 16
  // block; neighbouring lanes hold neighbouring columns.  Lanes 2c and 2c+1
  // swap two values (one DPP move each), so that each holds two rows of the
  // column pair (2c, 2c+1), packs each pair into one dword (hardware RNE
  // conversion) and writes it to the wave's staging rows in LDS; then every
  // lane reads 16 contiguous bytes of a row back and the wave stores whole
  // rows with 16-byte stores (a 128-byte line per 8 or 16 lanes) instead of
  // one 2-byte store per value.
  constexpr int WC = GATED ? NBW * 8 : NBW * 16;  // output columns of a wave
  constexpr int WR = MBW * 16;                    // output rows of a wave
  constexpr int RS = WC * 2 + 16;                 // staging row stride (bytes)
  static_assert(4 * WR * RS <= FW_LDS, "epilogue staging");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's last ring reads
  barrier_no_fence();                  // no wave reads the rings any more
  uint8_t* const stg = lds + wave * (WR * RS);
  const bool odd = lane & 1;
#pragma unroll
  for (int i = 0; i < MBW; ++i) {
#pragma unroll
    for (int q = 0; q < (GATED ? NBW / 2 : NBW); ++q) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = GATED ? silu_f32(acc[i][2 * q][e]) * acc[i][2 * q + 1][e] : acc[i][q][e];
      // even lanes keep rows 0, 2 and take the neighbour's; odd lanes rows 1, 3
      const float s0 = odd ? v[0] : v[1], s1 = odd ? v[2] : v[3];
      const float r0 = __int_as_float(
          __builtin_amdgcn_update_dpp(0, __float_as_int(s0), 0xB1, 0xf, 0xf, false));
      const float r1 = __int_as_float(
          __builtin_amdgcn_update_dpp(0, __float_as_int(s1), 0xB1, 0xf, 0xf, false));
      const uint32_t w0 = odd ? pack_bf16x2_rne(r0, v[1]) : pack_bf16x2_rne(v[0], r0);
      const uint32_t w1 = odd ? pack_bf16x2_rne(r1, v[3]) : pack_bf16x2_rne(v[2], r1);
      const int row = i * 16 + (lane >> 4) * 4 + (odd ? 1 : 0);
      const int col = q * 16 + (lane & 14);
      *reinterpret_cast<uint32_t*>(stg + row * RS + col * 2) = w0;
      *reinterpret_cast<uint32_t*>(stg + (row + 2) * RS + col * 2) = w1;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // the wave's staging writes are done
  __builtin_amdgcn_wave_barrier();
  constexpr int LPR = WC * 2 / 16;     // lanes per output row
  constexpr int RPI = 64 / LPR;        // rows per read
  const int col0 = GATED ? (nb0 / 2 + wn * (NBW / 2)) * 16 : (nb0 + wn * NBW) * 16;
#pragma unroll
  for (int it = 0; it < WR / RPI; ++it) {
    const int rr = it * RPI + lane / LPR;
    const int c8 = (lane % LPR) * 8;
    const u32x4_t val = *reinterpret_cast<const u32x4_t*>(stg + rr * RS + c8 * 2);
    const int r = m0 + wm * WR + rr;
    if (r < rows)
      __builtin_nontemporal_store(
          val, reinterpret_cast<u32x4_t*>(out + (size_t)(row_base + r) * p.n_out + col0 + c8));
  }
}

constexpr int XCD_CUS = 32;  // CUs per XCD

// Work unit of this workgroup for the four-wave kernel: tile L, whole
// (nsub = 1) or its weight rows cut into nsub parts (part sub).  As in
// xcd_tile each XCD walks a contiguous eighth of the tiles, one workgroup
// per CU, in about cnt / XCD_CUS rounds.  When the last round would hold at
// most half of the XCD's CUs, each of its tiles is cut into 2 (at most 16
// tiles) or 4 (at most 8) parts of the weight rows, each over the whole K, so
// that round keeps most CUs busy and takes a fraction of a tile's time (on
// the mixtral-prefill down pass a last round of 6 tiles on 32 CUs took 18% of
// the pass).  Each output element is still summed by one workgroup in K
// order, as in a whole tile.  Returns -1 for no work.  Needs gridDim.x >=
// 8 * (ceil(total / 8) + XCD_CUS).
__device__ __forceinline__ int xcd_unit(int total, int& nsub, int& sub) {
  const int per = (total + NXCD - 1) / NXCD;
  const int x = blockIdx.x % NXCD, slot = blockIdx.x / NXCD;
  const int cnt = max(0, min(per, total - x * per));
  const int tail = cnt % XCD_CUS;
  const int ns = tail == 0 ? 1 : (tail <= XCD_CUS / 4 ? 4 : (tail <= XCD_CUS / 2 ? 2 : 1));
  const int whole = ns > 1 ? cnt - tail : cnt;
  nsub = 1;
  sub = 0;
  if (slot < whole) return x * per + slot;
  const int j = slot - whole;
  if (ns == 1 || j >= tail * ns) return -1;
  nsub = ns;
  sub = j % ns;
  return x * per + whole + j / ns;
}

template <bool GATED, bool FP4>
__global__ __launch_bounds__(256, 1) void ffn_gemm_big_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[FW_LDS];
  const int ngroups = p.g1 - p.g0;
  const int MT = p.tiles[ngroups];
  int nsub, sub;
  const int L = xcd_unit(MT * p.NT, nsub, sub);
  if (L < 0) return;
  // tile-order groups: 4 weight tiles on the gate/up pass, 8 on the down
  // pass, where sharing each activation tile among more weight tiles
  // measured faster on both prefill shapes
  constexpr int GN = GATED ? GM_GN : 2 * GM_GN;
  const int blk = L / (MT * GN);
  const int gw = min(GN, p.NT - blk * GN);
  const int rr = L - blk * MT * GN;
  const int mt = rr / gw;
  const int nt = blk * GN + rr % gw;
  int lo = 0, hi = ngroups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.tiles[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  const int g = p.g0 + lo;
  const int m0 = (mt - p.tiles[lo]) * 256;
  int row_base, rows;
  group_rows(p, g, row_base, rows);
  const int left = rows - m0;   // rows from this tile on (> 0)
  const int nb0 = nt * (GM_BN / 16);  // first 16-row weight block of the tile
  if (nsub > 1) {
    // a part of a tail tile: 4 parts of 64 weight rows or 2 of 128 (short
    // tiles stream as many weight bytes as tall ones, so they are cut too)
    if (nsub == 4) {
      const int nb = nb0 + sub * 4;
      if (left > 128)
        four_wave_tile<GATED, 2, 8, 2, 5, 3, FP4>(p, lds, g, row_base, rows, m0, nb);
      else if (left > 64)
        four_wave_tile<GATED, 2, 4, 2, 6, 4, FP4>(p, lds, g, row_base, rows, m0, nb);
      else
        four_wave_tile<GATED, 2, 2, 2, 6, 4, FP4>(p, lds, g, row_base, rows, m0, nb);
    } else {
      const int nb = nb0 + sub * 8;
      if (left > 128)
        four_wave_tile<GATED, 2, 8, 4, 5, 3, FP4>(p, lds, g, row_base, rows, m0, nb);
      else if (left > 64)
        four_wave_tile<GATED, 1, 8, 2, 6, 4, FP4>(p, lds, g, row_base, rows, m0, nb);
      else
        four_wave_tile<GATED, 1, 4, 2, 6, 4, FP4>(p, lds, g, row_base, rows, m0, nb);
    }
    return;
  }
  if (left > 128) {
    // MXFP4: the 1 x 4 layout decodes each weight fragment once per tile
    // (mixtral-prefill-mxfp4 down pass 2.01 -> 1.83 ms, gate/up 3.29 -> 3.24)
    if constexpr (FP4)
      four_wave_tile<GATED, 1, 16, 4, 4, 3, FP4>(p, lds, g, row_base, rows, m0, nb0);
    else
      four_wave_tile<GATED, 2, 8, 8, 4, 3, FP4>(p, lds, g, row_base, rows, m0, nb0);
  } else if (left > 64)
    four_wave_tile<GATED, 1, 8, 4, 5, 3, FP4>(p, lds, g, row_base, rows, m0, nb0);
  else
    four_wave_tile<GATED, 1, 4, 4, 6, 4, FP4>(p, lds, g, row_base, rows, m0, nb0);
}

template <int BM, bool FP8>
void launch_gemm_kernel(bool gated, long long nwg, const GemmParams& p, hipStream_t st) {
  if (gated)
    ffn_gemm_kernel<BM, true, FP8><<<dim3((unsigned)nwg), 512, 0, st>>>(p);
  else
    ffn_gemm_kernel<BM, false, FP8><<<dim3((unsigned)nwg), 512, 0, st>>>(p);
}

}  // namespace

bool gemm_shape_ok(int d, int d_ff) { return d % 256 == 0 && d_ff % 128 == 0; }

// The four-wave kernel addresses operands through 32-bit buffer offsets.
bool gemm_four_wave_ok(const FfnArgs& a) {
  const long long lim = 0x7fffffffLL;
  return !a.fp8 && (long long)a.T * a.d * 2 <= lim && (long long)a.T * a.k * a.d_ff * 2 <= lim &&
         4LL * a.d * a.d_ff <= lim;
}

hipError_t launch_ffn_gemm(const FfnArgs& a, int pass, int g0, int g1, int max_rows,
                           int32_t* sched, hipStream_t st) {
  if (g1 <= g0) return hipSuccess;
  // bf16 and MXFP4 weights take the four-wave kernel (tiles of 64..256 rows);
  // FP8 weights, or bf16 shapes past 32-bit operand offsets, take the
  // eight-wave kernel with 128-row tiles (MXFP4 there is the caller's error:
  // it runs through the streaming kernel instead)
  const bool four_wave = gemm_four_wave_ok(a);
  if (a.mxfp4 && !four_wave) return hipErrorInvalidValue;
  const int bm = four_wave ? 256 : 128;
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
    if (a.mxfp4) {
      p.s4 = static_cast<const uint8_t*>(gated ? a.s13 : a.s2);
      p.s4_sh = static_cast<const uint8_t*>(gated ? a.s13_sh : a.s2_sh);
    } else {
      p.s = static_cast<const float*>(gated ? a.s13 : a.s2);
      p.s_sh = static_cast<const float*>(gated ? a.s13_sh : a.s2_sh);
    }
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
    else if (four_wave) {
      // room for the parts of the last round's tiles (xcd_unit)
      const unsigned nwg_fw = (unsigned)(nwg + (long long)NXCD * XCD_CUS);
      if (a.mxfp4) {
        if (gated)
          ffn_gemm_big_kernel<true, true><<<dim3(nwg_fw), 256, 0, st>>>(p);
        else
          ffn_gemm_big_kernel<false, true><<<dim3(nwg_fw), 256, 0, st>>>(p);
      } else if (gated) {
        ffn_gemm_big_kernel<true, false><<<dim3(nwg_fw), 256, 0, st>>>(p);
      } else {
        ffn_gemm_big_kernel<false, false><<<dim3(nwg_fw), 256, 0, st>>>(p);
      }
    } else
      launch_gemm_kernel<128, false>(gated, nwg, p, st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
