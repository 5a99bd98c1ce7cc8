// Weighted combine and un-permute: out[t] = sum_{i<k} g[t,i] *
// Y[inv_perm[t,i]] (+ Y_shared[t]).  The output is the gate-weighted sum of
// the selected experts ("Mixture of Experts for LLM Inference", "The MoE
// change is surprisingly local"; "Chapter 19", 19.3.2) plus the always-on
// shared expert with weight 1 ("Shared experts: stop relearning the
// basics").  Slots are added in a fixed order with float32 accumulation and
// each output element is written once: the result does not depend on
// scheduling.

#include "common.h"
#include "kernels.h"

namespace {

// bf16: each thread owns 8 consecutive columns (16-byte loads and stores).
__global__ __launch_bounds__(256) void combine_bf16_kernel(const uint16_t* __restrict__ y,
                                                           const uint16_t* __restrict__ ys,
                                                           const int32_t* __restrict__ inv,
                                                           const float* __restrict__ gw,
                                                           uint16_t* __restrict__ out, int k,
                                                           int d, int chunks) {
  const int t = blockIdx.x / chunks;
  const int c0 = ((blockIdx.x % chunks) * 256 + threadIdx.x) * 8;
  if (c0 >= d) return;
  float acc[8] = {};
  // slots in ascending order, 8 at a time: the rows and gates of a batch are
  // loaded together, then added in slot order (a dropped slot, row -1, adds
  // nothing)
  for (int i0 = 0; i0 < k; i0 += 8) {
    int r[8];
    float g[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool in = i0 + u < k;
      r[u] = in ? inv[(size_t)t * k + i0 + u] : -1;
      g[u] = in ? gw[(size_t)t * k + i0 + u] : 0.f;
    }
    // expert output rows are read once: non-temporal loads
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = r[u] >= 0 ? __builtin_nontemporal_load(
                             reinterpret_cast<const u32x4_t*>(y + (size_t)r[u] * d + c0))
                       : u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (r[u] < 0) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] = fmaf(g[u], bf16_to_f32(v[u][j] & 0xffffu), acc[2 * j]);
        acc[2 * j + 1] = fmaf(g[u], bf16_to_f32(v[u][j] >> 16), acc[2 * j + 1]);
      }
    }
  }
  if (ys) {
    const u32x4_t v =
        __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(ys + (size_t)t * d + c0));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += bf16_to_f32(v[j] & 0xffffu);
      acc[2 * j + 1] += bf16_to_f32(v[j] >> 16);
    }
  }
  u32x4_t o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
  *reinterpret_cast<u32x4_t*>(out + (size_t)t * d + c0) = o;
}

__global__ __launch_bounds__(256) void combine_f32_kernel(const float* __restrict__ y,
                                                          const float* __restrict__ ys,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ gw,
                                                          float* __restrict__ out, int k, int d,
                                                          int chunks) {
  const int t = blockIdx.x / chunks;
  const int c = (blockIdx.x % chunks) * 256 + threadIdx.x;
  if (c >= d) return;
  float acc = 0.f;
  for (int i0 = 0; i0 < k; i0 += 8) {  // as in the bf16 kernel
    int r[8];
    float g[8], v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool in = i0 + u < k;
      r[u] = in ? inv[(size_t)t * k + i0 + u] : -1;
      g[u] = in ? gw[(size_t)t * k + i0 + u] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = r[u] >= 0 ? y[(size_t)r[u] * d + c] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (r[u] >= 0) acc = fmaf(g[u], v[u], acc);
  }
  if (ys) acc += ys[(size_t)t * d + c];
  out[(size_t)t * d + c] = acc;
}

}  // namespace

hipError_t launch_combine(const void* y_perm, const void* y_shared, const int32_t* inv_perm,
                          const float* topk_w, void* out, int T, int k, int d, bool act_bf16,
                          hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (act_bf16) {
    const int chunks = ceil_div(d, 256 * 8);
    combine_bf16_kernel<<<dim3(chunks * T), 256, 0, st>>>(
        static_cast<const uint16_t*>(y_perm), static_cast<const uint16_t*>(y_shared), inv_perm,
        topk_w, static_cast<uint16_t*>(out), k, d, chunks);
  } else {
    const int chunks = ceil_div(d, 256);
    combine_f32_kernel<<<dim3(chunks * T), 256, 0, st>>>(
        static_cast<const float*>(y_perm), static_cast<const float*>(y_shared), inv_perm, topk_w,
        static_cast<float*>(out), k, d, chunks);
  }
  return hipGetLastError();
}
