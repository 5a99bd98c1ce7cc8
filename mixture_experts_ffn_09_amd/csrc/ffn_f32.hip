// Grouped SwiGLU expert FFN in float32 (float32 activations and weights).
// Same grouping and row numbering as the low-precision path; 16x16 output
// tiles with K staged through LDS.  Weights in natural [out][in] layout:
// w13 = [N][2][d_ff][d] (gate, then up), w2 = [N][d][d_ff].

#include "common.h"
#include "kernels.h"

namespace {

constexpr int FT = 16;

__device__ __forceinline__ bool group_rows(const FfnF32Args& p, int g, int& base, int& rows) {
  if (g < p.N) {
    base = p.offsets[g];
    rows = p.offsets[g + 1] - base;
  } else {
    base = 0;
    rows = p.T;
  }
  return rows > 0;
}

// H[r][n] = silu(a_r . Wg[n]) * (a_r . Wu[n])
__global__ __launch_bounds__(256) void ffn_up_f32_kernel(FfnF32Args p) {
  __shared__ float as[FT][FT + 1];
  __shared__ float gs[FT][FT + 1];
  __shared__ float us[FT][FT + 1];
  const int g = blockIdx.z;
  int base, rows;
  if (!group_rows(p, g, base, rows)) return;
  const int m0 = blockIdx.y * FT;
  if (m0 >= rows) return;
  const int n0 = blockIdx.x * FT;
  const int tx = threadIdx.x % FT, ty = threadIdx.x / FT;
  const bool shared = g >= p.N;
  const float* Wg = shared ? p.w13_sh : p.w13 + (size_t)g * 2 * p.d_ff * p.d;
  const float* Wu = Wg + (size_t)p.d_ff * p.d;
  // the row this thread loads for the A tile
  const int lr = m0 + ty;
  const float* arow = nullptr;
  if (lr < rows) {
    if (shared)
      arow = p.x_sh + (size_t)lr * p.d;
    else if (p.perm_token)
      arow = p.x_rows + (size_t)p.perm_token[base + lr] * p.d;
    else
      arow = p.x_rows + (size_t)(base + lr) * p.d;
  }
  float sg = 0.f, su = 0.f;
  for (int k0 = 0; k0 < p.d; k0 += FT) {
    const int kk = k0 + tx;
    as[ty][tx] = (arow && kk < p.d) ? arow[kk] : 0.f;
    const int wn = n0 + ty;
    gs[ty][tx] = (wn < p.d_ff && kk < p.d) ? Wg[(size_t)wn * p.d + kk] : 0.f;
    us[ty][tx] = (wn < p.d_ff && kk < p.d) ? Wu[(size_t)wn * p.d + kk] : 0.f;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      sg = fmaf(as[ty][j], gs[tx][j], sg);
      su = fmaf(as[ty][j], us[tx][j], su);
    }
    __syncthreads();
  }
  const int r = m0 + ty, n = n0 + tx;
  float* H = shared ? p.H_sh : p.H;
  if (r < rows && n < p.d_ff) H[(size_t)(base + r) * p.d_ff + n] = silu_f32(sg) * su;
}

// Y[r][n] = h_r . Wd[n]
__global__ __launch_bounds__(256) void ffn_down_f32_kernel(FfnF32Args p) {
  __shared__ float hs[FT][FT + 1];
  __shared__ float ws[FT][FT + 1];
  const int g = blockIdx.z;
  int base, rows;
  if (!group_rows(p, g, base, rows)) return;
  const int m0 = blockIdx.y * FT;
  if (m0 >= rows) return;
  const int n0 = blockIdx.x * FT;
  const int tx = threadIdx.x % FT, ty = threadIdx.x / FT;
  const bool shared = g >= p.N;
  const float* Wd = shared ? p.w2_sh : p.w2 + (size_t)g * p.d * p.d_ff;
  const float* Hin = shared ? p.H_sh : p.H;
  float s = 0.f;
  for (int k0 = 0; k0 < p.d_ff; k0 += FT) {
    const int kk = k0 + tx;
    const int lr = m0 + ty;
    hs[ty][tx] = (lr < rows && kk < p.d_ff) ? Hin[(size_t)(base + lr) * p.d_ff + kk] : 0.f;
    const int wn = n0 + ty;
    ws[ty][tx] = (wn < p.d && kk < p.d_ff) ? Wd[(size_t)wn * p.d_ff + kk] : 0.f;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < FT; ++j) s = fmaf(hs[ty][j], ws[tx][j], s);
    __syncthreads();
  }
  const int r = m0 + ty, n = n0 + tx;
  float* Y = shared ? p.Y_sh : p.Y;
  if (r < rows && n < p.d) Y[(size_t)(base + r) * p.d + n] = s;
}

}  // namespace

hipError_t launch_ffn_f32(const FfnF32Args& a, int pass, hipStream_t st) {
  const int groups = a.N + a.n_shared;
  // a group holds at most max_rows rows
  const int mt = ceil_div(a.max_rows, FT);
  if (pass & 1) {
    dim3 g1(ceil_div(a.d_ff, FT), mt, groups);
    ffn_up_f32_kernel<<<g1, 256, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (pass & 2) {
    dim3 g2(ceil_div(a.d, FT), mt, groups);
    ffn_down_f32_kernel<<<g2, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  return hipSuccess;
}
