// Router: logits (a small linear layer, one score per expert) and top-k
// selection with renormalised gates.
//
// "Mixture of Experts for LLM Inference", "Opening the router": linear layer
// -> scores -> keep the K best -> renormalise; "Chapter 19", 19.3.2:
// gate_logits = hidden_state @ W_router, top-k, softmax over the selected;
// "AI Infrastructure series - Part 12", worked example: DeepSeek-V3 scores
// each expert with a sigmoid, picks the top 8, normalises the chosen 8;
// "Chapter 19", 19.3.4: the balancing bias affects selection only.

#include "common.h"
#include "kernels.h"

namespace {

// ---------------------------------------------------------------------------
// Logits: float32 GEMM, 32 tokens x 64 experts per 256-thread workgroup,
// K staged through LDS 32 at a time; each thread owns 2 tokens x 4 experts.
// ---------------------------------------------------------------------------
constexpr int RL_TM = 32, RL_TN = 64, RL_TK = 32;

template <bool BF16>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ xv,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ offset,
                                                            float* __restrict__ logits, int T,
                                                            int d, int N) {
  __shared__ float xs[RL_TK][RL_TM + 1];
  __shared__ float ws[RL_TK][RL_TN];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * RL_TM;
  const int e0 = blockIdx.y * RL_TN;
  const int ty = tid / 16, tx = tid % 16;
  float acc[2][4] = {};
  for (int k0 = 0; k0 < d; k0 += RL_TK) {
    // x tile: 32 tokens x 32 k, 4 elements per thread
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int li = tid + r * 256;
      int tt = li / RL_TK, kk = li % RL_TK;
      int t = t0 + tt, kg = k0 + kk;
      float v = 0.f;
      if (t < T && kg < d) {
        if (BF16)
          v = bf16_to_f32(static_cast<const uint16_t*>(xv)[(size_t)t * d + kg]);
        else
          v = static_cast<const float*>(xv)[(size_t)t * d + kg];
      }
      xs[kk][tt] = v;
    }
    // W tile: 32 k x 64 experts, 8 elements per thread
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      int li = tid + r * 256;
      int kk = li / RL_TN, ee = li % RL_TN;
      int kg = k0 + kk, e = e0 + ee;
      ws[kk][ee] = (kg < d && e < N) ? w[(size_t)kg * N + e] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < RL_TK; ++kk) {
      float a0 = xs[kk][ty * 2], a1 = xs[kk][ty * 2 + 1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float b = ws[kk][tx * 4 + j];
        acc[0][j] = fmaf(a0, b, acc[0][j]);
        acc[1][j] = fmaf(a1, b, acc[1][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int t = t0 + ty * 2 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = e0 + tx * 4 + j;
      if (e < N) logits[(size_t)t * N + e] = acc[i][j] + (offset ? offset[e] : 0.f);
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token.  Lane l holds experts l, l+64, ...; k rounds of
// a wave-wide arg-max on (score desc, index asc).
// ---------------------------------------------------------------------------
struct Cand {
  float s;
  int i;
};

__device__ __forceinline__ bool better(float s1, int i1, float s2, int i2) {
  return s1 > s2 || (s1 == s2 && i1 < i2);
}

template <int NJ>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits,
                                                          const float* __restrict__ bias,
                                                          int sigmoid, int T, int N, int k,
                                                          int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float lg[NJ], sc[NJ];
  bool live[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    int e = lane + 64 * j;
    live[j] = e < N;
    float l = live[j] ? logits[(size_t)t * N + e] : 0.f;
    lg[j] = l;
    float s = l;
    if (sigmoid) {
      s = sigmoid_f32(l);
      if (bias && live[j]) s += bias[e];
    }
    sc[j] = s;
  }
  // selected logits, kept in lane i (i < k <= 64) or replicated via loop
  float my_logit = 0.f;
  int my_idx = 0;
  float sel_logit0 = 0.f;
  for (int r = 0; r < k; ++r) {
    float bs = -INFINITY;
    int bi = 0x7fffffff;
    float bl = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      int e = lane + 64 * j;
      if (live[j] && better(sc[j], e, bs, bi)) {
        bs = sc[j];
        bi = e;
        bl = lg[j];
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float os = __shfl_xor(bs, off);
      int oi = __shfl_xor(bi, off);
      float ol = __shfl_xor(bl, off);
      if (better(os, oi, bs, bi)) {
        bs = os;
        bi = oi;
        bl = ol;
      }
    }
    // every lane now holds the winner; retire it
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (lane + 64 * j == bi) live[j] = false;
    if (r == 0) sel_logit0 = bl;
    if ((r & 63) == lane) {
      my_logit = bl;
      my_idx = bi;
    }
  }
  // gates over the k selected (k <= 64 handled by lanes; k > 64 loops)
  float v = 0.f;
  if (lane < k) v = sigmoid ? sigmoid_f32(my_logit) : __expf(my_logit - sel_logit0);
  float sum = v;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = my_idx;
    topk_w[(size_t)t * k + lane] = v / sum;
  }
}

}  // namespace

hipError_t launch_router_logits(const void* x, bool act_bf16, const float* w_router,
                                const float* offset, float* logits, int T, int d, int N,
                                hipStream_t st) {
  dim3 grid(ceil_div(T, RL_TM), ceil_div(N, RL_TN));
  if (act_bf16)
    router_logits_kernel<true><<<grid, 256, 0, st>>>(x, w_router, offset, logits, T, d, N);
  else
    router_logits_kernel<false><<<grid, 256, 0, st>>>(x, w_router, offset, logits, T, d, N);
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* logits, const float* select_bias, int sigmoid,
                              int T, int N, int k, int32_t* topk_idx, float* topk_w,
                              hipStream_t st) {
  dim3 grid(ceil_div(T, 4));
  int nj = ceil_div(N, 64);
#define RT_CASE(NJ)                                                                       \
  router_topk_kernel<NJ><<<grid, 256, 0, st>>>(logits, select_bias, sigmoid, T, N, k, \
                                               topk_idx, topk_w)
  if (nj <= 1) RT_CASE(1);
  else if (nj <= 2) RT_CASE(2);
  else if (nj <= 4) RT_CASE(4);
  else if (nj <= 8) RT_CASE(8);
  else RT_CASE(16);
#undef RT_CASE
  return hipGetLastError();
}
