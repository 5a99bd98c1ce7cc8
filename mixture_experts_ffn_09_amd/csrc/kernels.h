// Host-side launchers of the gfx950 kernels (each returns the launch
// status; none synchronises).  Pointers are device pointers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Router logits x[T][d] @ W[d][N] in float32 as router_splits() partial
// sums over K: partial[S][T][N].  act_bf16: x is bfloat16 (else float32).
int router_splits(int T, int N, int d, bool act_bf16);
// bytes of router scratch: the partial logits, and with bf16 x when N > 8 or
// T >= 1024 the router weight split into three bf16 planes (after the
// logits, 256-aligned)
size_t router_scratch_bytes(int T, int N, int d, bool act_bf16);
hipError_t launch_router_logits(const void* x, bool act_bf16, const float* w_router,
                                float* partial, int T, int d, int N, hipStream_t st);

// Sums the S partials (+ offset[N]), selects the top k and writes the gates
// (one wave per token).
// per-16-token-block probability sums [stats_blocks(T)][N], then P, f, the
// balancing term and the bias step
int stats_blocks(int T);
hipError_t launch_load_stats(const float* partial, int S, const float* offset, int sigmoid, int T,
                             int N, int k, const int32_t* counts, float alpha, float step,
                             float* bp, float* frac, float* prob, float* aux, float* bias,
                             hipStream_t st);
// gsize > 0: at most max_groups groups of gsize consecutive experts per token
// Logits and selection in one launch for T <= 64 tokens and N <= 8 experts.
bool router_fused_small(int T, int N);
hipError_t launch_router_fused_small(const void* x, bool act_bf16, const float* w_router,
                                     const float* offset, const float* select_bias, int sigmoid,
                                     int T, int d, int N, int k, int gsize, int max_groups,
                                     int32_t* topk_idx, float* topk_w, hipStream_t st);
hipError_t launch_router_topk(const float* partial, int S, const float* offset,
                              const float* select_bias, int sigmoid, int T, int N, int k,
                              int gsize, int max_groups, int32_t* topk_idx, float* topk_w,
                              hipStream_t st);

// Counts, offsets and the stable (expert, token) permutation.  hist is
// scratch of permute_blocks(T) * N int32 (unused when that is 1).
int permute_blocks(int T);
hipError_t launch_permute(const int32_t* topk_idx, int T, int k, int N, int32_t* hist,
                          int32_t* counts, int32_t* offsets, int32_t* perm_token,
                          int32_t* inv_perm, hipStream_t st);

// x_perm[r] = x[perm_token[r]] for r < rows (row_bytes per row).
// capacity-limited routing from the dropless one (counts_f/offsets_f/inv_f)
hipError_t launch_capacity(const int32_t* topk_idx, int T, int k, int N, int cap,
                           const int32_t* counts_f, const int32_t* offsets_f, const int32_t* inv_f,
                           int32_t* counts, int32_t* offsets, int32_t* perm_token,
                           int32_t* inv_perm, hipStream_t st);
hipError_t launch_gather_rows(const void* x, const int32_t* perm_token, void* x_perm,
                              int rows, int row_bytes, hipStream_t st);

// Expert FFN.  Routed expert e owns rows [offsets[e], offsets[e+1]); its
// input row r is x_rows[perm_token[r]] (perm_token given) or x_rows[r]
// (x_rows already expert-contiguous).  The shared expert (n_shared == 1)
// reads x_sh[t] for t < T.  Outputs: H / Y (routed, row r), H_sh / Y_sh
// (shared, row t).
struct FfnArgs {
  const uint16_t* x_rows;
  const int32_t* perm_token;
  const uint16_t* x_sh;
  const int32_t* offsets;
  int T, k, N, n_shared, d, d_ff;
  bool fp8;                   // OCP E4M3 weights, float32 scale per 128x128 block
  bool mxfp4;                 // E2M1 weights, E8M0 scale byte per 32 inputs
  int32_t* sched;             // 2048 int32 of scratch for the GEMM tile schedule
  const void* w13;
  const void* w2;
  const void* s13;
  const void* s2;
  const void* w13_sh;
  const void* w2_sh;
  const void* s13_sh;
  const void* s2_sh;
  uint16_t* H;
  uint16_t* H_sh;
  uint16_t* Y;
  uint16_t* Y_sh;
};
// pass: 1 = gate/up + SwiGLU only, 2 = down only, 3 = both.  Picks, per group
// range, the weight-streaming kernel (few rows per expert) or the tiled
// GEMM (many rows).
hipError_t launch_ffn_lowp(const FfnArgs& a, int pass, hipStream_t st);

// Streaming kernel over groups [g0, g1).
hipError_t launch_ffn_stream(const FfnArgs& a, int pass, int g0, int g1, int rows_hint,
                             hipStream_t st);
// Tiled GEMM over groups [g0, g1) with row tile bm; max_rows bounds the total
// rows of those groups.
bool gemm_shape_ok(int d, int d_ff);
// the four-wave GEMM (bf16 and MXFP4 weights) fits this call's sizes
bool gemm_four_wave_ok(const FfnArgs& a);
hipError_t launch_ffn_gemm(const FfnArgs& a, int pass, int g0, int g1, int max_rows,
                           int32_t* sched, hipStream_t st);

// Float32 expert FFN (float32 activations and weights), same row scheme.
struct FfnF32Args {
  const float* x_rows;
  const int32_t* perm_token;
  const float* x_sh;
  const int32_t* offsets;
  int T, N, n_shared, d, d_ff, max_rows;
  const float* w13;           // [N][2][d_ff][d]
  const float* w2;            // [N][d][d_ff]
  const float* w13_sh;
  const float* w2_sh;
  float* H;
  float* H_sh;
  float* Y;
  float* Y_sh;
};
hipError_t launch_ffn_f32(const FfnF32Args& a, int pass, hipStream_t st);

// out[t] = sum_i g[t,i] * Y[inv[t,i]] (+ Ys[t]).
hipError_t launch_combine(const void* y_perm, const void* y_shared, const int32_t* inv_perm,
                          const float* topk_w, void* out, int T, int k, int d, bool act_bf16,
                          hipStream_t st);

// Weight repack (see moe_pack_weights).  esize: 4 (f32), 2 (bf16), 1 (fp8).
// MXFP4 scales: natural [n_mats][nh][rows][cols/32] bytes -> the packed
// layout the streaming kernel reads (16 rows x 16 bytes per 256-byte chunk)
size_t packed_scale_bytes(int n_mats, int rows, int cols, int nh);
hipError_t launch_pack_scales(const void* src, void* dst, int n_mats, int rows, int cols, int nh,
                              hipStream_t st);
hipError_t launch_pack(const void* src_a, const void* src_b, void* dst, int n_mats, int rows,
                       int cols, int esize, hipStream_t st);
