// Load statistics of a routed batch and one step of the selection-bias
// controller.
//
// "Chapter 19", 19.3.3: the Switch balancing term alpha * N * sum_i f_i P_i,
// with f_i the share of the batch routed to expert i and P_i the batch's
// average routing probability of expert i ("Mixture of Experts for LLM
// Inference", "Classic fix: auxiliary loss": weight 0.01).  19.3.4 and
// "DeepSeek-style bias controller": a per-expert bias used only for
// selection, lowered for overloaded experts and raised for underloaded ones
// after each batch ("AI Infrastructure series - Part 12", "How are experts
// kept evenly busy?": by 0.001).
//
// The routing probability of a token is the softmax of its N logits, or in
// sigmoid mode its affinities sigmoid(s) divided by their sum over all N
// (the selection bias never enters).  Every sum runs in a fixed order: the
// logits' K-split partials in split order (as the top-k kernel sums them),
// tokens within a wave in token order, waves within a 16-token block in wave
// order, blocks in block order, and the final N-term sum as a fixed tree.

#include "common.h"
#include "kernels.h"

namespace {

constexpr int ST_WAVES = 4;
constexpr int ST_TOK = 16;  // tokens per block (enough blocks to fill the chip at T = 256)
constexpr int ST_TPW = ST_TOK / ST_WAVES;

// bp[b][e] = sum over block b's tokens of p[t][e]
template <int NJ>
__global__ __launch_bounds__(256) void router_prob_block_kernel(
    const float* __restrict__ partial, int S, const float* __restrict__ offset, int sigmoid,
    int T, int N, float* __restrict__ bp) {
  __shared__ float wp[ST_WAVES][NJ * 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = 0.f;
  for (int i = 0; i < ST_TPW; ++i) {
    const int t = blockIdx.x * ST_TOK + w * ST_TPW + i;
    if (t >= T) break;  // uniform across the wave
    // split sums in ascending split order (as the top-k kernel forms them);
    // the loads of 8 splits x NJ columns are issued together
    float lg[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) lg[j] = 0.f;
    const float* prow = partial + (size_t)t * N + lane;
    const size_t sstride = (size_t)T * N;
    for (int sp0 = 0; sp0 < S; sp0 += 8) {
      float v[8][NJ];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          v[u][j] = (sp0 + u < S && lane + 64 * j < N) ? prow[(sp0 + u) * sstride + 64 * j] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int j = 0; j < NJ; ++j) lg[j] += v[u][j];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      if (e < N) {
        if (offset) lg[j] += offset[e];
      } else {
        lg[j] = -INFINITY;
      }
      mx = fmaxf(mx, lg[j]);
    }
    float z[NJ];
    float sum = 0.f;
    if (!sigmoid) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const bool live = lane + 64 * j < N;
      z[j] = !live ? 0.f : (sigmoid ? sigmoid_f32(lg[j]) : __expf(lg[j] - mx));
      sum += z[j];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    const float inv = 1.f / sum;
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] += z[j] * inv;
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) wp[w][lane + 64 * j] = acc[j];
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += 256) {
    float v = wp[0][e];
#pragma unroll
    for (int ww = 1; ww < ST_WAVES; ++ww) v += wp[ww][e];
    bp[(size_t)blockIdx.x * N + e] = v;
  }
}

// One workgroup of 512 threads (N <= 512): P, f, the balancing term and the
// bias step.
__global__ __launch_bounds__(512) void load_stats_finish_kernel(
    const float* __restrict__ bp, int nblk, const int32_t* __restrict__ counts, int T, int k,
    int N, float alpha, float step, float* __restrict__ frac, float* __restrict__ prob,
    float* __restrict__ aux, float* __restrict__ bias) {
  __shared__ float term[512];
  const int e = threadIdx.x;
  float t = 0.f;
  if (e < N) {
    // ascending block order; the loads of 8 blocks are issued together
    float s = 0.f;
    for (int b0 = 0; b0 < nblk; b0 += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = b0 + u < nblk ? bp[(size_t)(b0 + u) * N + e] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    const float P = s / (float)T;
    const int c = counts[e];
    const float f = (float)c / (float)((long long)T * k);
    if (prob) prob[e] = P;
    if (frac) frac[e] = f;
    t = f * P;
    if (bias) {
      // compare the load with the mean T*k/N exactly: c * N against T * k
      const long long lhs = (long long)c * N, rhs = (long long)T * k;
      const float sg = lhs < rhs ? 1.f : (lhs > rhs ? -1.f : 0.f);
      bias[e] = bias[e] + step * sg;
    }
  }
  term[e] = t;
  __syncthreads();
#pragma unroll
  for (int h = 256; h >= 1; h >>= 1) {
    if (e < h) term[e] += term[e + h];
    __syncthreads();
  }
  if (e == 0 && aux) aux[0] = alpha * (float)N * term[0];
}

}  // namespace

int stats_blocks(int T) { return T <= 0 ? 1 : ceil_div(T, ST_TOK); }

hipError_t launch_load_stats(const float* partial, int S, const float* offset, int sigmoid, int T,
                             int N, int k, const int32_t* counts, float alpha, float step,
                             float* bp, float* frac, float* prob, float* aux, float* bias,
                             hipStream_t st) {
  const int nblk = stats_blocks(T);
  const int nj = ceil_div(N, 64);
#define ST_CASE(NJ) router_prob_block_kernel<NJ><<<nblk, 256, 0, st>>>(partial, S, offset, sigmoid, T, N, bp)
  if (nj <= 1) ST_CASE(1);
  else if (nj <= 2) ST_CASE(2);
  else if (nj <= 4) ST_CASE(4);
  else ST_CASE(8);
#undef ST_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  load_stats_finish_kernel<<<1, 512, 0, st>>>(bp, nblk, counts, T, k, N, alpha, step, frac, prob,
                                              aux, bias);
  return hipGetLastError();
}
