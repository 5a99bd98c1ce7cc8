// Grouped expert FFN for bfloat16 activations with bfloat16 or FP8 (OCP
// E4M3, one float32 scale per 128x128 block) weights: the weight-streaming
// form, for few rows per expert (decode).
//
// An expert is a complete SwiGLU FFN with its own three matrices ("Mixture of
// Experts for LLM Inference", "The MoE change is surprisingly local";
// "Mixture of Experts Explained", "The slot it replaces, and what an expert
// is").  Pass 1 computes H = silu(X Wg^T) * (X Wu^T) with the SwiGLU in the
// epilogue; pass 2 computes Y = H Wd^T.  Only experts that received rows
// touch their weights.
//
// Work split: grid.y = group (routed expert, then the shared expert), grid.x
// over 16-row blocks of the weight matrix.  Each wave owns P such blocks
// (pairs of gate/up blocks in pass 1) and streams them along K exactly once
// per 16*MB rows of activations, so the weight stream is read once for up to
// 16*MB rows.  Weights are pre-packed so that one K step of one block is a
// contiguous 1 KB: each lane's 16-byte load is its v_mfma_f32_16x16x32_bf16
// B operand (bf16) or two of them (fp8, converted exactly to bf16 in
// registers), and a wave's loads are fully coalesced.  Activations come from
// L2 (they are re-read by every wave of the group).
//
// MFMA 16x16x32 operand mapping used on both sides: lane l holds row (A) /
// column (B) l % 16 and k = 8 * (l / 16) + j, j < 8; the accumulator lane l
// holds rows 4 * (l / 16) + i, i < 4, of column l % 16.

#include "common.h"
#include "kernels.h"

namespace {

constexpr int SW_WAVES = 4;  // waves per workgroup

struct StreamParams {
  const uint16_t* a;          // routed activations (row r, or row perm[r])
  const int32_t* perm;        // null: a is already expert-contiguous
  const uint16_t* a_sh;       // shared-expert activations, row t
  const int32_t* offsets;     // [N+1]
  int T, N;
  int K;       // reduction length
  int n_out;   // output width
  const uint8_t* w;           // packed routed weights
  const uint8_t* w_sh;        // packed shared weights
  const float* s;             // fp8 scales (routed)
  const float* s_sh;          // fp8 scales (shared)
  uint16_t* out;              // routed output rows
  uint16_t* out_sh;           // shared output rows
};

__device__ __forceinline__ void fp8_block_to_bf16(const u32x4_t& q, u32x4_t& lo, u32x4_t& hi) {
  lo[0] = e4m3x2_to_bf16x2<false>(q[0]);
  lo[1] = e4m3x2_to_bf16x2<true>(q[0]);
  lo[2] = e4m3x2_to_bf16x2<false>(q[1]);
  lo[3] = e4m3x2_to_bf16x2<true>(q[1]);
  hi[0] = e4m3x2_to_bf16x2<false>(q[2]);
  hi[1] = e4m3x2_to_bf16x2<true>(q[2]);
  hi[2] = e4m3x2_to_bf16x2<false>(q[3]);
  hi[3] = e4m3x2_to_bf16x2<true>(q[3]);
}

// GATED: pass 1 (gate+up, SwiGLU) else pass 2 (down).
template <int P, int MB, bool FP8, bool GATED>
__global__ __launch_bounds__(256) void ffn_stream_kernel(StreamParams p) {
  constexpr int NH = GATED ? 2 : 1;  // weight blocks per output block
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.y;
  const int NB = p.n_out / 16;
  const int nb0 = (blockIdx.x * SW_WAVES + wave) * P;
  if (nb0 >= NB) return;

  const bool shared = g >= p.N;
  int row_base, rows;
  if (!shared) {
    row_base = p.offsets[g];
    rows = p.offsets[g + 1] - row_base;
  } else {
    row_base = 0;
    rows = p.T;
  }
  if (rows <= 0) return;
  uint16_t* out = shared ? p.out_sh : p.out;

  // per-expert packed bytes and scale counts
  const size_t wbytes = (size_t)NH * p.n_out * p.K * (FP8 ? 1 : 2);
  const uint8_t* W = shared ? p.w_sh : p.w + (size_t)g * wbytes;
  const int KS = FP8 ? p.K / 64 : p.K / 32;     // K steps of one 1 KB block
  const int SK = p.K / MOE_FP8_BLOCK;           // scale columns
  const int SR = p.n_out / MOE_FP8_BLOCK;       // scale rows per matrix
  const float* S = nullptr;
  if (FP8) S = shared ? p.s_sh : p.s + (size_t)g * NH * SR * SK;

  const int lrow = lane & 15;   // A row / B column within a block
  const int lk = (lane >> 4) * 8;

  for (int m0 = 0; m0 < rows; m0 += 16 * MB) {
    // activation row pointers of this lane, one per 16-row block
    const uint16_t* arow[MB];
    bool av[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      int r = m0 + mb * 16 + lrow;
      av[mb] = r < rows;
      const uint16_t* ptr = p.a;
      if (av[mb]) {
        if (shared)
          ptr = p.a_sh + (size_t)r * p.K;
        else if (p.perm)
          ptr = p.a + (size_t)p.perm[row_base + r] * p.K;
        else
          ptr = p.a + (size_t)(row_base + r) * p.K;
      }
      arow[mb] = ptr + lk;
    }

    floatx4_t acc[P][NH][MB];
#pragma unroll
    for (int i = 0; i < P; ++i)
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[i][h][mb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    const u32x4_t zero4 = {0u, 0u, 0u, 0u};

    if (!FP8) {
#pragma unroll 4
      for (int ks = 0; ks < KS; ++ks) {
        u32x4_t b[P][NH];
#pragma unroll
        for (int i = 0; i < P; ++i)
#pragma unroll
          for (int h = 0; h < NH; ++h) {
            const size_t blk = ((size_t)(nb0 + i) * KS + ks) * NH + h;
            b[i][h] = (nb0 + i < NB)
                          ? *reinterpret_cast<const u32x4_t*>(W + blk * 1024 + lane * 16)
                          : zero4;
          }
        u32x4_t a[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          a[mb] = av[mb] ? *reinterpret_cast<const u32x4_t*>(arow[mb] + ks * 32) : zero4;
#pragma unroll
        for (int i = 0; i < P; ++i)
#pragma unroll
          for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              acc[i][h][mb] = mfma16x16x32(a[mb], b[i][h], acc[i][h][mb]);
      }
    } else {
      // FP8: K in chunks of 128 (two 1 KB steps of 64); per chunk a fresh
      // partial sum is scaled by its block scale and added.
      for (int kc = 0; kc < SK; ++kc) {
        floatx4_t part[P][NH][MB];
#pragma unroll
        for (int i = 0; i < P; ++i)
#pragma unroll
          for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) part[i][h][mb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int ks = kc * 2 + half;
          u32x4_t b[P][NH];
#pragma unroll
          for (int i = 0; i < P; ++i)
#pragma unroll
            for (int h = 0; h < NH; ++h) {
              const size_t blk = ((size_t)(nb0 + i) * KS + ks) * NH + h;
              b[i][h] = (nb0 + i < NB)
                            ? *reinterpret_cast<const u32x4_t*>(W + blk * 1024 + lane * 16)
                            : zero4;
            }
          u32x4_t a0[MB], a1[MB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            a0[mb] = av[mb] ? *reinterpret_cast<const u32x4_t*>(arow[mb] + ks * 64) : zero4;
            a1[mb] = av[mb] ? *reinterpret_cast<const u32x4_t*>(arow[mb] + ks * 64 + 32) : zero4;
          }
#pragma unroll
          for (int i = 0; i < P; ++i)
#pragma unroll
            for (int h = 0; h < NH; ++h) {
              u32x4_t blo, bhi;
              fp8_block_to_bf16(b[i][h], blo, bhi);
#pragma unroll
              for (int mb = 0; mb < MB; ++mb) {
                part[i][h][mb] = mfma16x16x32(a0[mb], blo, part[i][h][mb]);
                part[i][h][mb] = mfma16x16x32(a1[mb], bhi, part[i][h][mb]);
              }
            }
        }
#pragma unroll
        for (int i = 0; i < P; ++i)
#pragma unroll
          for (int h = 0; h < NH; ++h) {
            const int srow = ((nb0 + i) * 16) / MOE_FP8_BLOCK;
            const float sc = (nb0 + i < NB) ? S[((size_t)h * SR + srow) * SK + kc] : 0.f;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[i][h][mb][e] += sc * part[i][h][mb][e];
          }
      }
    }

    // epilogue: lane holds rows 4*(lane/16)+e of column lane%16
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int n = (nb0 + i) * 16 + lrow;
      if (nb0 + i >= NB) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = m0 + mb * 16 + (lane >> 4) * 4 + e;
          if (r >= rows) continue;
          float v;
          if (GATED)
            v = silu_f32(acc[i][0][mb][e]) * acc[i][NH - 1][mb][e];
          else
            v = acc[i][0][mb][e];
          out[(size_t)(row_base + r) * p.n_out + n] = (uint16_t)f32_to_bf16(v);
        }
    }
  }
}

template <int P, int MB, bool FP8, bool GATED>
hipError_t launch_stream(const StreamParams& sp, int groups, hipStream_t st) {
  const int NB = sp.n_out / 16;
  dim3 grid(ceil_div(NB, SW_WAVES * P), groups);
  ffn_stream_kernel<P, MB, FP8, GATED><<<grid, SW_WAVES * 64, 0, st>>>(sp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_lowp(const FfnArgs& a, int pass, hipStream_t st) {
  const int groups = a.N + a.n_shared;
  StreamParams up{};
  up.a = a.x_rows;
  up.perm = a.perm_token;
  up.a_sh = a.x_sh;
  up.offsets = a.offsets;
  up.T = a.T;
  up.N = a.N;
  up.K = a.d;
  up.n_out = a.d_ff;
  up.w = static_cast<const uint8_t*>(a.w13);
  up.w_sh = static_cast<const uint8_t*>(a.w13_sh);
  up.s = a.s13;
  up.s_sh = a.s13_sh;
  up.out = a.H;
  up.out_sh = a.H_sh;

  StreamParams dn = up;
  dn.a = a.H;
  dn.perm = nullptr;
  dn.a_sh = a.H_sh;
  dn.K = a.d_ff;
  dn.n_out = a.d;
  dn.w = static_cast<const uint8_t*>(a.w2);
  dn.w_sh = static_cast<const uint8_t*>(a.w2_sh);
  dn.s = a.s2;
  dn.s_sh = a.s2_sh;
  dn.out = a.Y;
  dn.out_sh = a.Y_sh;

  hipError_t e = hipSuccess;
  if (pass & 1) {
    e = a.fp8 ? launch_stream<2, 2, true, true>(up, groups, st)
              : launch_stream<2, 2, false, true>(up, groups, st);
    if (e != hipSuccess) return e;
  }
  if (pass & 2)
    e = a.fp8 ? launch_stream<2, 2, true, false>(dn, groups, st)
              : launch_stream<2, 2, false, false>(dn, groups, st);
  return e;
}
