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
// result does not depend on scheduling).  Shapes:
//  * N <= 8 (float32 x, or bfloat16 x below 1024 tokens): one thread per
//    token owning all experts; the W slice is staged in LDS and read as a
//    broadcast (router_logits_small_n).  With T <= 64
//    the layer instead runs logits and selection in one kernel
//    (router_fused_small_kernel, below the top-k kernel).
//  * N > 8, or N <= 8 from 1024 tokens, bfloat16 x: MFMA on three bfloat16
//    planes of W (at large batches the one-token-per-lane form reads 64 rows
//    per load instruction, and the copy path, not the arithmetic, set its
//    time: 45 us for the 8192 x 4096 mixtral-prefill batch)
//    (router_logits_mfma; router_logits_ring for large batches).
//  * N > 8, float32 x: 32 tokens x 64 experts per workgroup, each thread
//    2 x 4, K staged through LDS 32 at a time (router_logits_tiled).
// ---------------------------------------------------------------------------
constexpr int RL_TM = 32, RL_TN = 64, RL_TK = 32;
constexpr int RS_TM = 256, RS_KT = 256;

template <bool BF16, int TPB>
__global__ __launch_bounds__(256) void router_logits_small_n(const void* __restrict__ xv,
                                                             const float* __restrict__ w,
                                                             float* __restrict__ partial, int T,
                                                             int d, int N, int KC) {
  // TPB tokens per workgroup, 256 / TPB lanes split each token's K range
  constexpr int KL = 256 / TPB;
  __shared__ float ws[RS_KT][8];
  __shared__ float red[KL > 1 ? KL : 1][TPB][8];
  const int tid = threadIdx.x;
  const int tl = tid % TPB, kl = tid / TPB;
  const int t = blockIdx.x * TPB + tl;
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
#pragma unroll 4
        for (int kk = kl * 8; kk < kn; kk += 8 * KL) {  // bf16 K ranges are multiples of 8
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
        for (int kk = kl; kk < kn; kk += KL) {
          const float xk = xr[kk];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(xk, ws[kk][e], acc[e]);
        }
      }
    }
    __syncthreads();
  }
  if (KL > 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[kl][tl][e] = acc[e];
    __syncthreads();
    if (kl == 0) {
      for (int l = 1; l < KL; ++l)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += red[l][tl][e];
    }
  }
  if (kl == 0 && t < T)
    for (int e = 0; e < N; ++e) partial[((size_t)s * T + t) * N + e] = acc[e];
}

// ---------------------------------------------------------------------------
// bf16 activations, N > 8: the float32 router weight is split exactly into
// three bfloat16 planes (w = hi + mid + lo, 8 significand bits each), so each
// product x * plane is exact in float32 (x is bf16) and three
// v_mfma_f32_16x16x32_bf16 per step give the float32 dot product.  The split
// runs once per call (router_split_kernel) into scratch, already in B-operand
// order ([32-K step][16-expert block][plane][64 lanes][8 bf16], zero-padded),
// instead of once per token tile.  64 tokens x 64 experts per workgroup
// (2 x 2 waves of 32 x 32); the planes of the slice are staged in LDS;
// activations load straight into A operands.  Optional split over K.
// ---------------------------------------------------------------------------
constexpr int RM_TM = 64, RM_TN = 64, RM_BK = 64;

__device__ __forceinline__ void split3_bf16(float w, uint32_t& h, uint32_t& m, uint32_t& l) {
  h = f32_to_bf16(w);
  const float r1 = w - bf16_to_f32(h);   // exact
  m = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(m);  // exact
  l = f32_to_bf16(r2);
}

// one thread per (32-K step, 16-expert block, lane): its 8 weights in the
// three planes
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ w,
                                                           uint16_t* __restrict__ planes, int d,
                                                           int N, int NB, size_t total) {
  const size_t c = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= total) return;
  const int l = (int)(c & 63);
  const int nb = (int)((c >> 6) % NB);
  const int ks = (int)((c >> 6) / NB);
  const int e = nb * 16 + (l & 15);
  const int kb = ks * 32 + (l >> 4) * 8;
  uint32_t hh[4], mm[4], ll[4];
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const float w0 = (e < N && kb + j < d) ? w[(size_t)(kb + j) * N + e] : 0.f;
    const float w1 = (e < N && kb + j + 1 < d) ? w[(size_t)(kb + j + 1) * N + e] : 0.f;
    uint32_t h0, m0, l0, h1, m1, l1;
    split3_bf16(w0, h0, m0, l0);
    split3_bf16(w1, h1, m1, l1);
    hh[j / 2] = h0 | (h1 << 16);
    mm[j / 2] = m0 | (m1 << 16);
    ll[j / 2] = l0 | (l1 << 16);
  }
  uint16_t* out = planes + (((size_t)ks * NB + nb) * 3 * 64 + l) * 8;
  *reinterpret_cast<u32x4_t*>(out) = u32x4_t{hh[0], hh[1], hh[2], hh[3]};
  *reinterpret_cast<u32x4_t*>(out + 64 * 8) = u32x4_t{mm[0], mm[1], mm[2], mm[3]};
  *reinterpret_cast<u32x4_t*>(out + 2 * 64 * 8) = u32x4_t{ll[0], ll[1], ll[2], ll[3]};
}

__global__ __launch_bounds__(256) void router_logits_mfma(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ planes,
                                                          float* __restrict__ partial, int T,
                                                          int d, int N, int NB, int KC) {
  // [plane][k step][n block][64 lanes][8 bf16]
  __shared__ __attribute__((aligned(16))) uint16_t wl[3][RM_BK / 32][RM_TN / 16][64 * 8];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.x * RM_TM, e0 = blockIdx.y * RM_TN, s = blockIdx.z;
  const int k_begin = s * KC, k_end = min(d, k_begin + KC);
  // A rows of this lane for its two 16-token blocks (clamped; not stored)
  const uint16_t* arow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = min(t0 + (wm * 2 + i) * 16 + (lane & 15), T - 1);
    arow[i] = x + (size_t)t * d + (lane >> 4) * 8;
  }
  floatx4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // Operands of one 64-K chunk in registers: this lane's A fragments (2 K
  // steps x its 2 token blocks; d is a multiple of 8, so a lane's 8 inputs
  // are all in range or all out) and its two B-operand lane slots of all
  // three planes (steps past this split's end and expert blocks past the last
  // are zero).  The next chunk's are loaded while this one is multiplied.
  auto load_chunk = [&](int k0, u32x4_t (&a)[2][2], u32x4_t (&b)[2][3]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kk = k0 + ks * 32;
      const bool ain = kk + (lane >> 4) * 8 < k_end;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[ks][i] = ain ? *reinterpret_cast<const u32x4_t*>(arow[i] + kk) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int slot = tid + 256 * r;          // 0 .. 511
      const int frag = slot >> 6, l = slot & 63;
      const int ks = frag / (RM_TN / 16), nb = frag % (RM_TN / 16);
      const int gks = k0 / 32 + ks, gnb = e0 / 16 + nb;
      const bool in = gks * 32 < k_end && gnb < NB;
      const uint16_t* src = planes + (((size_t)gks * NB + gnb) * 3 * 64 + l) * 8;
#pragma unroll
      for (int pl = 0; pl < 3; ++pl)
        b[r][pl] = in ? *reinterpret_cast<const u32x4_t*>(src + pl * 64 * 8) : u32x4_t{0, 0, 0, 0};
    }
  };
  u32x4_t ac[2][2], bc[2][3], an[2][2], bn[2][3];
  load_chunk(k_begin, ac, bc);
  for (int k0 = k_begin; k0 < k_end; k0 += RM_BK) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int slot = tid + 256 * r;
      const int frag = slot >> 6, l = slot & 63;
      const int ks = frag / (RM_TN / 16), nb = frag % (RM_TN / 16);
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) *reinterpret_cast<u32x4_t*>(&wl[pl][ks][nb][l * 8]) = bc[r][pl];
    }
    // the next chunk (clamped: the last one is loaded again and not used)
    load_chunk(min(k0 + RM_BK, k_end - 1) / 32 * 32, an, bn);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < RM_BK / 32; ++ks) {
      if (k0 + ks * 32 >= k_end) break;  // K chunks are multiples of 32
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int nb = wn * 2 + j;
#pragma unroll
        for (int pl = 0; pl < 3; ++pl) {
          const u32x4_t b = *reinterpret_cast<const u32x4_t*>(&wl[pl][ks][nb][lane * 8]);
#pragma unroll
          for (int i = 0; i < 2; ++i) acc[i][j] = mfma16x16x32(ac[ks][i], b, acc[i][j]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i) ac[ks][i] = an[ks][i];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) bc[r][pl] = bn[r][pl];
  }
  // lane holds rows 4*(lane/16)+q of column lane%16
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + (wm * 2 + i) * 16 + (lane >> 4) * 4 + q;
        const int e = e0 + (wn * 2 + j) * 16 + (lane & 15);
        if (t < T && e < N) partial[((size_t)s * T + t) * N + e] = acc[i][j][q];
      }
}

// Large batches: 128 tokens x 128 experts per workgroup, one wave per SIMD
// (2 x 2 waves of 64 x 64), both operands moved global -> LDS by buffer
// loads into a ring of RR_NS stages of 32 K, so several stages are in flight
// while one is multiplied (the register-prefetch kernel above keeps one).
// A stage holds 8 activation fragments and 8 expert blocks x 3 weight planes,
// each 1 KB in MFMA operand order (lane l's 16 bytes at l * 16), read back
// conflict-free.  Wave 0 copies the activations, waves 1-3 the planes: eight
// 1 KB copies per wave per stage.  Needs N % 128 == 0, d % 32 == 0 and
// T * d * 2 < 2^31; rows past T are loaded clamped and not stored.
constexpr int RR_TM = 128, RR_TN = 128, RR_NS = 5;
constexpr int RR_STAGE = 32 * 1024;
constexpr int RR_CPW = 8;  // copies per wave per stage

__global__ __launch_bounds__(256, 1) void router_logits_ring(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ planes,
                                                             float* __restrict__ partial, int T,
                                                             int d, int N, int NB, int KC) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[RR_NS * RR_STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.x * RR_TM, e0 = blockIdx.y * RR_TN, s = blockIdx.z;
  const int k_begin = s * KC, k_end = min(d, k_begin + KC);
  const int nst = (k_end - k_begin) / 32;  // >= 1: d and KC are multiples of 32
  const int ks0 = k_begin / 32;

  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)x, 0, (int)((size_t)T * d * 2), BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t pres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)planes, 0, (int)((size_t)(d / 32) * NB * 3 * 1024), BUF_DWORD3);
  // this wave's eight copies: byte offset (lane part), LDS slot offset, and
  // the per-stage advance of the scalar offset
  uint32_t voff[RR_CPW];
  int ldst[RR_CPW];
#pragma unroll
  for (int i = 0; i < RR_CPW; ++i) {
    if (wave == 0) {  // activation fragment i: tokens t0 + 16 i + l % 16
      const int t = min(t0 + 16 * i + (lane & 15), T - 1);
      voff[i] = (uint32_t)t * (uint32_t)d * 2 + (lane >> 4) * 16;
      ldst[i] = i * 1024;
    } else {          // plane fragment c = (wave - 1) * 8 + i: block c / 3, plane c % 3
      const int c = (wave - 1) * RR_CPW + i;
      const int gnb = e0 / 16 + c / 3;
      voff[i] = (uint32_t)((gnb * 3 + c % 3) * 1024 + lane * 16);
      ldst[i] = 8192 + c * 1024;
    }
  }
  const int sadv = wave == 0 ? 64 : NB * 3 * 1024;  // bytes per 32-K stage
  const int sbase = wave == 0 ? k_begin * 2 : ks0 * NB * 3 * 1024;

  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  // copy i of stage j into slot j % RR_NS (stages past the last load the
  // last one again, into a slot no later stage reads)
  auto copy_one = [&](int i, int j) {
    const int jl = min(j, nst - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        wave == 0 ? xres : pres, (lds_ptr_t)(lds + (j % RR_NS) * RR_STAGE + ldst[i]), 16,
        voff[i], sbase + jl * sadv, 0, 0);
  };
  // operand read f of stage j: f < 4 activation fragment wm * 4 + f, else
  // expert block wn * 4 + (f - 4) / 3 in plane (f - 4) % 3
  auto read_one = [&](int f, int j, u32x4_t (&a)[4], u32x4_t (&b)[4][3]) {
    const uint8_t* slot = lds + (j % RR_NS) * RR_STAGE + lane * 16;
    if (f < 4)
      a[f] = *reinterpret_cast<const u32x4_t*>(slot + (wm * 4 + f) * 1024);
    else
      b[(f - 4) / 3][(f - 4) % 3] = *reinterpret_cast<const u32x4_t*>(
          slot + 8192 + (wn * 12 + f - 4) * 1024);
  };

  floatx4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[i][n] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t ca[4], cb[4][3], na[4], nb[4][3];

#pragma unroll
  for (int j = 0; j < RR_NS - 1; ++j)
#pragma unroll
    for (int i = 0; i < RR_CPW; ++i) copy_one(i, j);
  wait_vmcnt<(RR_NS - 2) * RR_CPW>();  // stage 0 has landed (this wave's copies)
  barrier_no_fence();
#pragma unroll
  for (int f = 0; f < 16; ++f) read_one(f, 0, ca, cb);
  // Step j: stage j + 1 has landed for every wave and every wave is past
  // stage j - 1; stage j's 48 MFMAs run interleaved with the copies of stage
  // j + RR_NS - 1 and the operand reads of stage j + 1 (program order
  // alternates the two, since an LDS read may not move past a copy into LDS).
  auto step = [&](int j, const u32x4_t (&a)[4], const u32x4_t (&b)[4][3], u32x4_t (&ga)[4],
                  u32x4_t (&gb)[4][3]) {
    wait_vmcnt<(RR_NS - 3) * RR_CPW>();
    barrier_no_fence();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < RR_CPW; ++i) {
      copy_one(i, j + RR_NS - 1);
      read_one(2 * i, j + 1, ga, gb);
      read_one(2 * i + 1, j + 1, ga, gb);
    }
#pragma unroll
    for (int pl = 0; pl < 3; ++pl)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[i][n] = mfma16x16x32(a[i], b[n][pl], acc[i][n]);
    stage_pattern<0, RR_CPW, 16, 48>();
    __builtin_amdgcn_sched_barrier(0);
  };
  int j = 0;
  for (; j + 1 < nst; j += 2) {
    step(j, ca, cb, na, nb);
    step(j + 1, na, nb, ca, cb);
  }
  if (j < nst) step(j, ca, cb, na, nb);
  wait_vmcnt<0>();  // the clamped copies of the last stages

  // lane holds rows 4 * (lane / 16) + q of column lane % 16 of each block
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = t0 + (wm * 4 + i) * 16 + (lane >> 4) * 4 + q;
      if (t >= T) continue;
      float* prow = partial + ((size_t)s * T + t) * N + e0 + wn * 64 + (lane & 15);
#pragma unroll
      for (int n = 0; n < 4; ++n) prow[n * 16] = acc[i][n][q];
    }
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
// Candidate (score s, index i) as one integer whose order is that of (s desc,
// i asc): the float's bits made monotone (-0 taken as +0) above the inverted
// index.  0 is below every candidate and marks "none".  A NaN score ranks
// below every other score, -inf included (its upper half is 0, below the
// monotone bits of -inf), and among NaN scores the lower index wins, so k
// experts are always chosen and every id lies in [0, N).
__device__ __forceinline__ uint64_t order_key(float s, int idx) {
  if (s != s) return 0xFFFFFFFFull - (uint32_t)idx;
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (0xFFFFFFFFu - (uint32_t)idx);
}

__device__ __forceinline__ int key_index(uint64_t key) {
  return (int)(0xFFFFFFFFu - (uint32_t)key);
}

// one DPP step of the wave maximum: each lane takes the larger of its value
// and the one the DPP control routes to it (lanes with no source keep theirs)
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xf, false);
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xf, false);
  const uint64_t o = ((uint64_t)ohi << 32) | olo;
  return o > v ? o : v;
}

// Maximum over the 64 lanes, returned to every lane (as a wave-uniform
// value): shifts right by 1, 2, 4, 8 within each row of 16 leave the row's
// maximum in its lane 15; broadcasting lane 15 into the next row and then
// lane 31 into rows 2 and 3 leaves the wave's maximum in lane 63.  No LDS.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0x111, 0xf>(v);  // row_shr:1
  v = dpp_max_step<0x112, 0xf>(v);  // row_shr:2
  v = dpp_max_step<0x114, 0xf>(v);  // row_shr:4
  v = dpp_max_step<0x118, 0xf>(v);  // row_shr:8
  v = dpp_max_step<0x142, 0xa>(v);  // row_bcast:15 into rows 1, 3
  v = dpp_max_step<0x143, 0xc>(v);  // row_bcast:31 into rows 2, 3
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// One wave scores and selects for one token.  Lane l holds the logits of
// experts l + 64 j (j < NJ) in lg; on return lanes i < k hold the i-th
// selected expert (best first, the lower index winning ties) and its gate.
// With gsize > 0 the experts form N / gsize groups of gsize consecutive ids
// (at most 64 groups) and a token may use at most max_groups of them: a
// group's score is its best expert's selection score, the max_groups best
// groups are kept (exact ties to the lower group index), and the selection
// runs over their experts only ("Mixture of Experts for LLM Inference",
// "Three tricks that tame the all-to-alls": node-limited routing).  gscr is
// this wave's LDS scratch of N floats.
template <int NJ>
__device__ __forceinline__ void select_topk(const float (&lg)[NJ], int N, int k, int sigmoid,
                                            const float* __restrict__ bias, int lane, int gsize,
                                            int max_groups, float* gscr, int& my_idx,
                                            float& my_w) {
  float sc[NJ];
  bool live[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    live[j] = e < N;
    float s = lg[j];
    if (sigmoid) {
      s = sigmoid_f32(lg[j]);
      if (bias && live[j]) s += bias[e];
    }
    sc[j] = s;
  }
  if (gsize > 0) {
    const int G = N / gsize;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (live[j]) gscr[lane + 64 * j] = sc[j];
    __builtin_amdgcn_wave_barrier();
    // the group's best score: fmaxf skips NaN, so the maximum is NaN only
    // when every score of the group is NaN (and then ranks lowest)
    float gm = -INFINITY;
    if (lane < G) {
      gm = gscr[lane * gsize];
      for (int e = lane * gsize + 1; e < (lane + 1) * gsize; ++e) gm = fmaxf(gm, gscr[e]);
    }
    uint64_t gk = lane < G ? order_key(gm, lane) : 0;
    uint64_t allowed = 0;
    for (int r = 0; r < max_groups; ++r) {
      const uint64_t b = wave_max_u64(gk);
      if (b == 0) break;
      const int bi = key_index(b);
      allowed |= 1ull << bi;
      if (lane == bi) gk = 0;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      live[j] = live[j] && ((allowed >> ((lane + 64 * j) / gsize)) & 1ull);
  }
  float my_logit = 0.f;
  float sel_logit0 = 0.f;
  my_idx = 0;
  uint64_t key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) key[j] = live[j] ? order_key(sc[j], lane + 64 * j) : 0;
  for (int r = 0; r < k; ++r) {
    uint64_t b = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) b = key[j] > b ? key[j] : b;
    b = wave_max_u64(b);
    int bi = 0x7fffffff;
    float bl = 0.f;
    if (b != 0) {
      // the winner's logit, from its lane; retire the winner
      bi = key_index(b);
      const int bj = bi >> 6;
      float lsel = lg[0];
#pragma unroll
      for (int j = 1; j < NJ; ++j)
        if (j == bj) lsel = lg[j];
      bl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lsel), bi & 63));
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (lane + 64 * j == bi) key[j] = 0;
    }
    if (r == 0) sel_logit0 = bl;
    if ((r & 63) == lane) {
      my_logit = bl;
      my_idx = bi;
    }
  }
  // gates over the k selected: softmax of their logits, or their unbiased
  // sigmoid scores divided by the sum
  float v = 0.f;
  if (lane < k) v = sigmoid ? sigmoid_f32(my_logit) : __expf(my_logit - sel_logit0);
  float sum = v;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  my_w = v / sum;
}

template <int NJ>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ partial,
                                                          int S, const float* __restrict__ offset,
                                                          const float* __restrict__ bias,
                                                          int sigmoid, int T, int N, int k,
                                                          int gsize, int max_groups,
                                                          int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w) {
  __shared__ float gscr[4][NJ * 64];
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  // split sums in ascending split order; the loads of 8 splits x NJ columns
  // are issued together, so the latency is paid once per 8 splits
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
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    if (offset && lane + 64 * j < N) lg[j] += offset[lane + 64 * j];
  int my_idx;
  float my_w;
  select_topk<NJ>(lg, N, k, sigmoid, bias, lane, gsize, max_groups, gscr[threadIdx.x >> 6],
                  my_idx, my_w);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = my_idx;
    topk_w[(size_t)t * k + lane] = my_w;
  }
}

// Few tokens and experts (T <= 64, N <= 8): logits and selection in one
// kernel, one workgroup per token.  Each thread dots 8-input chunks of the
// token against the N weight columns (float32 FMAs), the 256 partial sums are
// reduced in a fixed order (a butterfly within each wave, then the four wave
// totals in order), and wave 0 selects and gates as the top-k kernel does.
// Saves the split-K partial buffer and a second launch at decode sizes.
template <bool BF16>
__global__ __launch_bounds__(256) void router_fused_small_kernel(
    const void* __restrict__ xv, const float* __restrict__ w, const float* __restrict__ offset,
    const float* __restrict__ bias, int sigmoid, int d, int N, int k, int gsize,
    int max_groups, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  __shared__ float wsum[4][8];
  __shared__ float gscr[64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int t = blockIdx.x;
  // thread tid takes inputs tid, tid + 256, ...: a wave's x loads and its
  // weight-row loads (N floats each) are contiguous across its lanes
  // (the loads of 8 inputs are issued together)
  float acc[8] = {};
  for (int k0 = tid; k0 < d; k0 += 8 * 256) {
    float xk[8];
    u32x4_t w0[8], w1[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kk = min(k0 + u * 256, d - 1);  // past the end: loaded, weighted 0
      const float xv_ = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(xv)[(size_t)t * d + kk])
                             : static_cast<const float*>(xv)[(size_t)t * d + kk];
      xk[u] = k0 + u * 256 < d ? xv_ : 0.f;
      const float* wr = w + (size_t)kk * N;
      if (N == 8) {  // one 32-byte row: two 16-byte loads
        w0[u] = *reinterpret_cast<const u32x4_t*>(wr);
        w1[u] = *reinterpret_cast<const u32x4_t*>(wr + 4);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w0[u][e] = e < N ? __float_as_uint(wr[e]) : 0u;
          w1[u][e] = e + 4 < N ? __float_as_uint(wr[e + 4]) : 0u;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = fmaf(xk[u], __uint_as_float(w0[u][e]), acc[e]);
        acc[e + 4] = fmaf(xk[u], __uint_as_float(w1[u][e]), acc[e + 4]);
      }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float v = acc[e];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
    acc[e] = v;
  }
  if (lane == 0)
#pragma unroll
    for (int e = 0; e < 8; ++e) wsum[wv][e] = acc[e];
  __syncthreads();
  if (wv != 0) return;
  float lg[1] = {0.f};
  if (lane < N) {
    lg[0] = ((wsum[0][lane] + wsum[1][lane]) + wsum[2][lane]) + wsum[3][lane];
    if (offset) lg[0] += offset[lane];
  }
  int my_idx;
  float my_w;
  select_topk<1>(lg, N, k, sigmoid, bias, lane, gsize, max_groups, gscr, my_idx, my_w);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = my_idx;
    topk_w[(size_t)t * k + lane] = my_w;
  }
}

}  // namespace

// Router kernel choice: bf16 x with N > 8 or T >= 1024 -> MFMA (the LDS-ring
// form for large batches with N % 128 == 0); else N <= 8 -> small_n; else
// tiled fp32.
static bool router_mfma(int T, int N, bool act_bf16) { return act_bf16 && (N > 8 || T >= 1024); }

static bool router_ring(int T, int N, int d, bool act_bf16) {
  return act_bf16 && N % RR_TN == 0 && d % 32 == 0 && T >= 1024 &&
         (long long)T * d * 2 <= 0x7fffffffLL;
}

static int router_tiles(int T, int N, bool mfma) {
  if (mfma) return ceil_div(T, RM_TM) * ceil_div(N, RM_TN);
  if (N <= 8) return ceil_div(T, RS_TM);
  return ceil_div(T, RL_TM) * ceil_div(N, RL_TN);
}

int router_splits(int T, int N, int d, bool act_bf16) {
  if (T <= 0) return 1;
  if (router_ring(T, N, d, act_bf16)) {
    // one workgroup per CU, at least 256 of K per split
    const int tiles = ceil_div(T, RR_TM) * (N / RR_TN);
    int S = 256 / tiles;
    S = S < 1 ? 1 : S;
    const int smax = ceil_div(d, 256);
    S = S > smax ? smax : S;
    const int KC = ceil_div(ceil_div(d, S), 64) * 64;
    return ceil_div(d, KC);
  }
  const int tiles = router_tiles(T, N, router_mfma(T, N, act_bf16));
  // enough workgroups to fill the chip, but at least 256 of K per split
  int S = 1024 / tiles;
  S = S < 1 ? 1 : S;
  const int smax = ceil_div(d, 256);
  S = S > smax ? smax : S;
  const int KC = ceil_div(ceil_div(d, S), 64) * 64;
  return ceil_div(d, KC);
}

// bytes of the pre-split weight planes (MFMA path only)
static size_t router_plane_bytes(int N, int d) {
  return (size_t)ceil_div(d, 32) * ceil_div(N, 16) * 3 * 1024;
}

static size_t align256_sz(size_t v) { return (v + 255) / 256 * 256; }

size_t router_scratch_bytes(int T, int N, int d, bool act_bf16) {
  const size_t logits = (size_t)router_splits(T, N, d, act_bf16) * T * N * 4;
  return router_mfma(T, N, act_bf16) ? align256_sz(logits) + router_plane_bytes(N, d) : logits;
}

static int router_chunk(int T, int N, int d, bool act_bf16) {
  const int S = router_splits(T, N, d, act_bf16);
  return ceil_div(ceil_div(d, S), 64) * 64;
}

hipError_t launch_router_logits(const void* x, bool act_bf16, const float* w_router,
                                float* partial, int T, int d, int N, hipStream_t st) {
  const int S = router_splits(T, N, d, act_bf16);
  const int KC = router_chunk(T, N, d, act_bf16);
  if (!router_mfma(T, N, act_bf16) && N <= 8) {
    // few tokens: spread each token's K over lanes of the workgroup
    if (T <= 16) {
      dim3 grid(ceil_div(T, 16), 1, S);
      if (act_bf16)
        router_logits_small_n<true, 16><<<grid, 256, 0, st>>>(x, w_router, partial, T, d, N, KC);
      else
        router_logits_small_n<false, 16><<<grid, 256, 0, st>>>(x, w_router, partial, T, d, N, KC);
    } else {
      dim3 grid(ceil_div(T, RS_TM), 1, S);
      if (act_bf16)
        router_logits_small_n<true, RS_TM><<<grid, 256, 0, st>>>(x, w_router, partial, T, d, N, KC);
      else
        router_logits_small_n<false, RS_TM><<<grid, 256, 0, st>>>(x, w_router, partial, T, d, N, KC);
    }
  } else if (act_bf16) {
    dim3 grid(ceil_div(T, RM_TM), ceil_div(N, RM_TN), S);
    // planes live after the partial logits in the router's scratch
    const int NB = ceil_div(N, 16);
    uint16_t* planes = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(partial) +
                                                   align256_sz((size_t)S * T * N * 4));
    const size_t total = (size_t)ceil_div(d, 32) * NB * 64;
    router_split_kernel<<<dim3((unsigned)ceil_div((int)total, 256)), 256, 0, st>>>(
        w_router, planes, d, N, NB, total);
    if (router_ring(T, N, d, act_bf16))
      router_logits_ring<<<dim3(ceil_div(T, RR_TM), N / RR_TN, S), 256, 0, st>>>(
          static_cast<const uint16_t*>(x), planes, partial, T, d, N, NB, KC);
    else
      router_logits_mfma<<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(x), planes, partial,
                                               T, d, N, NB, KC);
  } else {
    dim3 grid(ceil_div(T, RL_TM), ceil_div(N, RL_TN), S);
    router_logits_tiled<false><<<grid, 256, 0, st>>>(x, w_router, partial, T, d, N, KC);
  }
  return hipGetLastError();
}

bool router_fused_small(int T, int N) { return T >= 1 && T <= 64 && N <= 8; }

hipError_t launch_router_fused_small(const void* x, bool act_bf16, const float* w_router,
                                     const float* offset, const float* select_bias, int sigmoid,
                                     int T, int d, int N, int k, int gsize, int max_groups,
                                     int32_t* topk_idx, float* topk_w, hipStream_t st) {
  if (act_bf16)
    router_fused_small_kernel<true><<<T, 256, 0, st>>>(x, w_router, offset, select_bias, sigmoid,
                                                       d, N, k, gsize, max_groups, topk_idx,
                                                       topk_w);
  else
    router_fused_small_kernel<false><<<T, 256, 0, st>>>(x, w_router, offset, select_bias,
                                                        sigmoid, d, N, k, gsize, max_groups,
                                                        topk_idx, topk_w);
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* partial, int S, const float* offset,
                              const float* select_bias, int sigmoid, int T, int N, int k,
                              int gsize, int max_groups, int32_t* topk_idx, float* topk_w,
                              hipStream_t st) {
  dim3 grid(ceil_div(T, 4));
  int nj = ceil_div(N, 64);
#define RT_CASE(NJ)                                                                  \
  router_topk_kernel<NJ><<<grid, 256, 0, st>>>(partial, S, offset, select_bias, sigmoid, T, N, \
                                               k, gsize, max_groups, topk_idx, topk_w)
  if (nj <= 1) RT_CASE(1);
  else if (nj <= 2) RT_CASE(2);
  else if (nj <= 4) RT_CASE(4);
  else RT_CASE(8);
#undef RT_CASE
  return hipGetLastError();
}
