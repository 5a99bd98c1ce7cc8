// Route and pack ("Chapter 19", 19.6.3): per-expert counts, exclusive
// offsets, and the stable expert-contiguous order of (token, slot)
// assignments, by (expert ascending, token ascending).
//
// One 1024-thread workgroup.  Wave w owns a contiguous token range.  Pass 1
// counts its assignments into a wave-private LDS histogram (order-free
// adds).  The histograms are scanned over (expert, wave) into global row
// bases.  Pass 2 revisits the range 64 tokens at a time; the rank of an
// assignment among earlier same-expert assignments of the 64 is found with
// ballots over the bits of the expert id, so positions never depend on the
// order in which atomics land.

#include "common.h"
#include "kernels.h"

namespace {

constexpr int PW = 16;  // waves

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__global__ __launch_bounds__(1024) void permute_kernel(const int32_t* __restrict__ idx, int T,
                                                       int k, int N, int nbits,
                                                       int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ perm_token,
                                                       int32_t* __restrict__ inv_perm) {
  extern __shared__ int32_t hist[];  // [PW][N] then scan[N]
  int32_t* scan = hist + PW * N;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int chunk = ceil_div(T, PW);
  const int t_begin = min(T, w * chunk), t_end = min(T, t_begin + chunk);
  const uint32_t sentinel = (1u << nbits) - 1u;  // >= N, never a valid id

  for (int i = tid; i < PW * N; i += 1024) hist[i] = 0;
  __syncthreads();

  // pass 1: wave-private counts
  for (int t = t_begin + lane; t < t_end; t += 64)
    for (int i = 0; i < k; ++i) {
      int e = idx[(size_t)t * k + i];
      if (e >= 0 && e < N) atomicAdd(&hist[w * N + e], 1);
    }
  __syncthreads();

  // per-expert totals (N <= 1024 = one expert per thread); hist becomes the
  // wave's base within the expert
  if (tid < N) {
    int run = 0;
    for (int ww = 0; ww < PW; ++ww) {
      int v = hist[ww * N + tid];
      hist[ww * N + tid] = run;
      run += v;
    }
    scan[tid] = run;
  }
  __syncthreads();
  // inclusive scan of the N totals (Hillis-Steele)
  for (int off = 1; off < N; off <<= 1) {
    int v = (tid < N && tid >= off) ? scan[tid - off] : 0;
    __syncthreads();
    if (tid < N) scan[tid] += v;
    __syncthreads();
  }
  if (tid < N) {
    const int excl = tid ? scan[tid - 1] : 0;
    offsets[tid] = excl;
    counts[tid] = scan[tid] - excl;
    if (tid == N - 1) offsets[N] = scan[tid];
    for (int ww = 0; ww < PW; ++ww) hist[ww * N + tid] += excl;
  }
  __syncthreads();

  // pass 2: stable positions
  const uint64_t lt = lanemask_lt();
  for (int tb = t_begin; tb < t_end; tb += 64) {
    const int t = tb + lane;
    const bool tv = t < t_end;
    // my k expert ids (sentinel when absent)
    for (int i = 0; i < k; ++i) {
      int e = tv ? idx[(size_t)t * k + i] : -1;
      bool ok = e >= 0 && e < N;
      uint32_t my = ok ? (uint32_t)e : sentinel;
      int rank = 0;
      for (int i2 = 0; i2 < k; ++i2) {
        int e2 = tv ? idx[(size_t)t * k + i2] : -1;
        uint32_t other = (e2 >= 0 && e2 < N) ? (uint32_t)e2 : sentinel;
        uint64_t m = ~0ull;
        for (int b = 0; b < nbits; ++b) {
          uint64_t bal = __ballot((other >> b) & 1u);
          m &= ((my >> b) & 1u) ? bal : ~bal;
        }
        rank += __popcll(m & lt);
        // the same token listing the expert in an earlier slot comes first
        if (i2 < i && other == my && ok) ++rank;
      }
      if (ok) {
        int pos = hist[w * N + (int)my] + rank;
        perm_token[pos] = t;
        inv_perm[(size_t)t * k + i] = pos;
      } else if (tv) {
        inv_perm[(size_t)t * k + i] = -1;
      }
    }
    // advance the wave's bases by this group's counts (after all reads)
    __builtin_amdgcn_wave_barrier();
    for (int i = 0; i < k; ++i) {
      int e = tv ? idx[(size_t)t * k + i] : -1;
      if (e >= 0 && e < N) atomicAdd(&hist[w * N + e], 1);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ x,
                                                          const int32_t* __restrict__ perm,
                                                          uint8_t* __restrict__ xp, int rows,
                                                          int row_bytes) {
  const int r = blockIdx.x;
  if (r >= rows) return;
  const int t = perm[r];
  const uint8_t* src = x + (size_t)t * row_bytes;
  uint8_t* dst = xp + (size_t)r * row_bytes;
  if ((row_bytes & 15) == 0) {
    for (int c = threadIdx.x * 16; c < row_bytes; c += 256 * 16)
      *reinterpret_cast<uint4*>(dst + c) = *reinterpret_cast<const uint4*>(src + c);
  } else {
    for (int c = threadIdx.x * 4; c < row_bytes; c += 256 * 4)
      *reinterpret_cast<uint32_t*>(dst + c) = *reinterpret_cast<const uint32_t*>(src + c);
  }
}

}  // namespace

hipError_t launch_permute(const int32_t* topk_idx, int T, int k, int N, int32_t* counts,
                          int32_t* offsets, int32_t* perm_token, int32_t* inv_perm,
                          hipStream_t st) {
  int nbits = 1;
  while ((1 << nbits) <= N) ++nbits;  // 2^nbits > N: room for the sentinel
  size_t lds = (size_t)(PW + 1) * N * sizeof(int32_t);
  permute_kernel<<<1, 1024, lds, st>>>(topk_idx, T, k, N, nbits, counts, offsets, perm_token,
                                       inv_perm);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* perm_token, void* x_perm, int rows,
                              int row_bytes, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  gather_rows_kernel<<<rows, 256, 0, st>>>(static_cast<const uint8_t*>(x), perm_token,
                                           static_cast<uint8_t*>(x_perm), rows, row_bytes);
  return hipGetLastError();
}
