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
// Logits: float32 dot products, split over K into S partial sums
// partial[s][t][e] (summed in a fixed order by the top-k kernel, so the
// result does not depend on scheduling).  Two shapes:
//  * N <= 8: one thread per token owning all experts; the W slice is staged
//    in LDS and read as a broadcast.
//  * N > 8: 32 tokens x 64 experts per workgroup, each thread 2 x 4,
//    K staged through LDS 32 at a time.
// ---------------------------------------------------------------------------
constexpr int RL_TM = 32, RL_TN = 64, RL_TK = 32;
constexpr int RS_TM = 256, RS_KT = 256;

template <bool BF16>
__global__ __launch_bounds__(256) void router_logits_small_n(const void* __restrict__ xv,
                                                             const float* __restrict__ w,
                                                             float* __restrict__ partial, int T,
                                                             int d, int N, int KC) {
  __shared__ float ws[RS_KT][8];
  const int tid = threadIdx.x;
  const int t = blockIdx.x * RS_TM + tid;
  const int s = blockIdx.z;
  const int k_begin = s * KC, k_end = min(d, k_begin + KC);
  float acc[8] = {};
  for (int kt = k_begin; kt < k_end; kt += RS_KT) {
    for (int i = tid; i < RS_KT * 8; i += 256) {
      const int kk = i >> 3, e = i & 7;
      ws[kk][e] = (kt + kk < k_end && e < N) ? w[(size_t)(kt + kk) * N + e] : 0.f;
    }
    __syncthreads();
    const int kn = min(RS_KT, k_end - kt);
    if (t < T) {
      if (BF16) {
        const uint16_t* xr = static_cast<const uint16_t*>(xv) + (size_t)t * d + kt;
        for (int kk = 0; kk < kn; kk += 8) {  // bf16 K ranges are multiples of 8
          const u32x4_t q = *reinterpret_cast<const u32x4_t*>(xr + kk);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x0 = bf16_to_f32(q[j] & 0xffffu), x1 = bf16_to_f32(q[j] >> 16);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              acc[e] = fmaf(x0, ws[kk + 2 * j][e], acc[e]);
              acc[e] = fmaf(x1, ws[kk + 2 * j + 1][e], acc[e]);
            }
          }
        }
      } else {
        const float* xr = static_cast<const float*>(xv) + (size_t)t * d + kt;
        for (int kk = 0; kk < kn; ++kk) {
          const float xk = xr[kk];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(xk, ws[kk][e], acc[e]);
        }
      }
    }
    __syncthreads();
  }
  if (t < T)
    for (int e = 0; e < N; ++e) partial[((size_t)s * T + t) * N + e] = acc[e];
}

template <bool BF16>
__global__ __launch_bounds__(256) void router_logits_tiled(const void* __restrict__ xv,
                                                           const float* __restrict__ w,
                                                           float* __restrict__ partial, int T,
                                                           int d, int N, int KC) {
  __shared__ float xs[RL_TK][RL_TM + 1];
  __shared__ float ws[RL_TK][RL_TN];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * RL_TM;
  const int e0 = blockIdx.y * RL_TN;
  const int s = blockIdx.z;
  const int k_begin = s * KC, k_end = min(d, k_begin + KC);
  const int ty = tid / 16, tx = tid % 16;
  float acc[2][4] = {};
  for (int k0 = k_begin; k0 < k_end; k0 += RL_TK) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int li = tid + r * 256;
      const int tt = li / RL_TK, kk = li % RL_TK;
      const int t = t0 + tt, kg = k0 + kk;
      float v = 0.f;
      if (t < T && kg < k_end) {
        if (BF16)
          v = bf16_to_f32(static_cast<const uint16_t*>(xv)[(size_t)t * d + kg]);
        else
          v = static_cast<const float*>(xv)[(size_t)t * d + kg];
      }
      xs[kk][tt] = v;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int li = tid + r * 256;
      const int kk = li / RL_TN, ee = li % RL_TN;
      const int kg = k0 + kk, e = e0 + ee;
      ws[kk][ee] = (kg < k_end && e < N) ? w[(size_t)kg * N + e] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < RL_TK; ++kk) {
      const float a0 = xs[kk][ty * 2], a1 = xs[kk][ty * 2 + 1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float b = ws[kk][tx * 4 + j];
        acc[0][j] = fmaf(a0, b, acc[0][j]);
        acc[1][j] = fmaf(a1, b, acc[1][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + ty * 2 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < N) partial[((size_t)s * T + t) * N + e] = acc[i][j];
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token.  Lane l holds experts l, l+64, ...; k rounds of
// a wave-wide arg-max on (score desc, index asc).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better(float s1, int i1, float s2, int i2) {
  return s1 > s2 || (s1 == s2 && i1 < i2);
}

template <int NJ>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ partial,
                                                          int S, const float* __restrict__ offset,
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
    float l = 0.f;
    if (live[j]) {
#pragma unroll 4
      for (int sp = 0; sp < S; ++sp) l += partial[((size_t)sp * T + t) * N + e];
      if (offset) l += offset[e];
    }
    lg[j] = l;
    float s = l;
    if (sigmoid) {
      s = sigmoid_f32(l);
      if (bias && live[j]) s += bias[e];
    }
    sc[j] = s;
  }
  // lane i keeps the i-th selected expert (k <= 64)
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

int router_splits(int T, int N, int d) {
  if (T <= 0) return 1;
  const int tiles = N <= 8 ? ceil_div(T, RS_TM) : ceil_div(T, RL_TM) * ceil_div(N, RL_TN);
  // enough workgroups to fill the chip, but at least 256 of K per split
  int S = 1024 / tiles;
  S = S < 1 ? 1 : S;
  const int smax = ceil_div(d, 256);
  S = S > smax ? smax : S;
  const int KC = ceil_div(ceil_div(d, S), 32) * 32;
  return ceil_div(d, KC);
}

static int router_chunk(int T, int N, int d) {
  const int S = router_splits(T, N, d);
  return ceil_div(ceil_div(d, S), 32) * 32;
}

hipError_t launch_router_logits(const void* x, bool act_bf16, const float* w_router,
                                float* partial, int T, int d, int N, hipStream_t st) {
  const int S = router_splits(T, N, d);
  const int KC = router_chunk(T, N, d);
  if (N <= 8) {
    dim3 grid(ceil_div(T, RS_TM), 1, S);
    if (act_bf16)
      router_logits_small_n<true><<<grid, 256, 0, st>>>(x, w_router, partial, T, d, N, KC);
    else
      router_logits_small_n<false><<<grid, 256, 0, st>>>(x, w_router, partial, T, d, N, KC);
  } else {
    dim3 grid(ceil_div(T, RL_TM), ceil_div(N, RL_TN), S);
    if (act_bf16)
      router_logits_tiled<true><<<grid, 256, 0, st>>>(x, w_router, partial, T, d, N, KC);
    else
      router_logits_tiled<false><<<grid, 256, 0, st>>>(x, w_router, partial, T, d, N, KC);
  }
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* partial, int S, const float* offset,
                              const float* select_bias, int sigmoid, int T, int N, int k,
                              int32_t* topk_idx, float* topk_w, hipStream_t st) {
  dim3 grid(ceil_div(T, 4));
  int nj = ceil_div(N, 64);
#define RT_CASE(NJ)                                                                  \
  router_topk_kernel<NJ><<<grid, 256, 0, st>>>(partial, S, offset, select_bias, sigmoid, T, N, \
                                               k, topk_idx, topk_w)
  if (nj <= 1) RT_CASE(1);
  else if (nj <= 2) RT_CASE(2);
  else if (nj <= 4) RT_CASE(4);
  else RT_CASE(8);
#undef RT_CASE
  return hipGetLastError();
}
