// Route and pack ("Chapter 19", 19.6.3): per-expert counts, exclusive
// offsets, and the stable expert-contiguous order of (token, slot)
// assignments, by (expert ascending, token ascending, slot ascending).
//
// Tokens are cut into blocks of 256 (one workgroup, 4 waves of 64 tokens).
// A first kernel writes each block's per-expert counts (order-free LDS adds).
// The second kernel gives every block its row bases - expert offset plus the
// counts of earlier blocks plus those of earlier waves in the block - and
// ranks each assignment among earlier same-expert assignments of its wave:
// from per-expert masks of the wave's lanes (OR-ed in LDS), or, when a token
// lists an expert twice, with ballots over the bits of the expert id.  Every
// position follows from counts, masks and ballots alone, never from the
// order in which atomics land.
// With a single block the first kernel is skipped.

#include "common.h"
#include "kernels.h"

namespace {

constexpr int PB_WAVES = 4;
constexpr int PB_TOK = PB_WAVES * 64;  // tokens per block

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// hist[b][e]: assignments of block b's tokens to expert e
__global__ __launch_bounds__(256) void block_hist_kernel(const int32_t* __restrict__ idx, int T,
                                                         int k, int N,
                                                         int32_t* __restrict__ hist) {
  extern __shared__ int32_t h[];
  for (int e = threadIdx.x; e < N; e += 256) h[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * PB_TOK + threadIdx.x;
  if (t < T)
    for (int i = 0; i < k; ++i) {
      const int e = idx[(size_t)t * k + i];
      if (e >= 0 && e < N) atomicAdd(&h[e], 1);
    }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += 256) hist[(size_t)blockIdx.x * N + e] = h[e];
}

// Exclusive scan of v[0..n) in place (n <= 2 * 256), by all 256 threads of
// the workgroup: each thread sums two neighbours, the waves scan with
// shuffles, the wave totals are scanned in LDS.  Returns the grand total.
__device__ int block_exclusive_scan(int32_t* v, int n, int32_t* wtot) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i0 = 2 * tid;
  const int a = i0 < n ? v[i0] : 0, b = i0 + 1 < n ? v[i0 + 1] : 0;
  int incl = a + b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int up = __shfl_up(incl, o);
    if (lane >= o) incl += up;
  }
  if (lane == 63) wtot[w] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int ww = 0; ww < PB_WAVES; ++ww) {
    const int t = wtot[ww];
    if (ww < w) before += t;
    total += t;
  }
  const int excl = before + incl - (a + b);
  __syncthreads();  // every thread has read its inputs and wtot
  if (i0 < n) v[i0] = excl;
  if (i0 + 1 < n) v[i0 + 1] = excl + a;
  __syncthreads();
  return total;
}

// hist == nullptr: a single block (T <= 256) counts for itself.
__global__ __launch_bounds__(256) void permute_kernel(const int32_t* __restrict__ idx, int T,
                                                      int k, int N, int nbits,
                                                      const int32_t* __restrict__ hist, int nblk,
                                                      int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ perm_token,
                                                      int32_t* __restrict__ inv_perm) {
  extern __shared__ __attribute__((aligned(8))) int32_t sm[];
  uint64_t* msk = reinterpret_cast<uint64_t*>(sm);  // [PB_WAVES][N] lane masks per expert
  int32_t* wh = sm + 2 * PB_WAVES * N;    // [PB_WAVES][N] wave counts, then wave bases
  int32_t* tot = wh + PB_WAVES * N;       // [N] totals, then exclusive offsets
  int32_t* bef = tot + N;                 // [N] counts of earlier blocks
  int32_t* wtot = bef + N;                // [PB_WAVES] scan scratch
  int32_t* sid = wtot + PB_WAVES;         // [PB_TOK][k] the block's expert ids
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int b = blockIdx.x;
  const int t = b * PB_TOK + w * 64 + lane;
  const bool tv = t < T;
  const uint32_t sentinel = (1u << nbits) - 1u;  // >= N, never a valid id

  for (int i = tid; i < PB_WAVES * N; i += 256) wh[i] = 0;
  // the block's ids, read once (coalesced) and kept in LDS
  {
    const int first = b * PB_TOK * k;
    const int cnt = min(PB_TOK, T - b * PB_TOK) * k;
    for (int i = tid; i < cnt; i += 256) sid[i] = idx[(size_t)first + i];
  }
  __syncthreads();
  int32_t* my = sid + (w * 64 + lane) * k;
  if (tv)
    for (int i = 0; i < k; ++i) {
      const int e = my[i];
      if (e >= 0 && e < N) atomicAdd(&wh[w * N + e], 1);
    }
  __syncthreads();

  // totals and the counts of earlier blocks
  for (int e = tid; e < N; e += 256) {
    int before = 0, total = 0;
    if (hist) {
      // the loads of 8 blocks' counts are issued together
      for (int bb0 = 0; bb0 < nblk; bb0 += 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = bb0 + u < nblk ? hist[(size_t)(bb0 + u) * N + e] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          total += v[u];
          if (bb0 + u < b) before += v[u];
        }
      }
    } else {
      for (int ww = 0; ww < PB_WAVES; ++ww) total += wh[ww * N + e];
    }
    tot[e] = total;
    bef[e] = before;
  }
  __syncthreads();
  const int grand = block_exclusive_scan(tot, N, wtot);
  if (b == 0 && tid == 0) offsets[N] = grand;
  for (int e = tid; e < N; e += 256) {
    if (b == 0) {
      const int next = (e + 1 < N) ? tot[e + 1] : grand;
      offsets[e] = tot[e];
      counts[e] = next - tot[e];
    }
    int run = tot[e] + bef[e];
    for (int ww = 0; ww < PB_WAVES; ++ww) {
      const int v = wh[ww * N + e];
      wh[ww * N + e] = run;
      run += v;
    }
  }
  __syncthreads();

  // ranks within the wave's 64 tokens
  const uint64_t lt = lanemask_lt();
  // Usual case, no token listing an expert twice: the rank of (t, i) is the
  // number of earlier lanes whose token lists the same expert, read from a
  // per-expert mask of lanes (LDS OR of each lane's bit; the result does not
  // depend on the order the ORs land in).
  bool dup = false;
  if (tv)
    for (int i = 1; i < k; ++i)
      for (int i2 = 0; i2 < i; ++i2) dup |= my[i] == my[i2];
  if (__ballot(dup) == 0) {
    uint64_t* wm = msk + (size_t)w * N;
    for (int e = lane; e < N; e += 64) wm[e] = 0ull;
    __builtin_amdgcn_wave_barrier();
    if (tv)
      for (int i = 0; i < k; ++i) {
        const int e = my[i];
        if (e >= 0 && e < N) atomicOr(reinterpret_cast<unsigned long long*>(&wm[e]), 1ull << lane);
      }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): every lane's OR has landed
    __builtin_amdgcn_wave_barrier();
    if (tv)
      for (int i = 0; i < k; ++i) {
        const int e = my[i];
        if (e >= 0 && e < N) {
          const int pos = wh[w * N + e] + __popcll(wm[e] & lt);
          perm_token[pos] = t;
          inv_perm[(size_t)t * k + i] = pos;
        } else {
          inv_perm[(size_t)t * k + i] = -1;
        }
      }
    return;
  }
  // a token lists an expert twice: ranks from ballots over the bits of the
  // expert ids, slot by slot
  for (int i = 0; i < k; ++i) {
    const int e = tv ? my[i] : -1;
    const bool ok = e >= 0 && e < N;
    const uint32_t mine = ok ? (uint32_t)e : sentinel;
    int rank = 0;
    for (int i2 = 0; i2 < k; ++i2) {
      const int e2 = tv ? my[i2] : -1;
      const uint32_t other = (e2 >= 0 && e2 < N) ? (uint32_t)e2 : sentinel;
      uint64_t m = ~0ull;
      for (int bit = 0; bit < nbits; ++bit) {
        const uint64_t bal = __ballot((other >> bit) & 1u);
        m &= ((mine >> bit) & 1u) ? bal : ~bal;
      }
      rank += __popcll(m & lt);
      // the same token listing the expert in an earlier slot comes first
      if (i2 < i && other == mine && ok) ++rank;
    }
    if (ok) {
      const int pos = wh[w * N + (int)mine] + rank;
      perm_token[pos] = t;
      inv_perm[(size_t)t * k + i] = pos;
    } else if (tv) {
      inv_perm[(size_t)t * k + i] = -1;
    }
  }
}

// Capacity-limited dispatch ("Chapter 19", 19.6.1): from the dropless
// routing (counts_f, offsets_f, inv_f as written by permute_kernel), each
// expert keeps the first `cap` rows of its segment - its first cap
// assignments in token order, then slot order - and the kept rows are packed
// in the same order.  Dropped assignments get inv_perm = -1.  Every block
// recomputes the capped offsets (N <= 512); block 0 writes counts/offsets.
__global__ __launch_bounds__(256) void capacity_kernel(
    const int32_t* __restrict__ idx, int A, int k, int N, int cap,
    const int32_t* __restrict__ counts_f, const int32_t* __restrict__ offsets_f,
    const int32_t* __restrict__ inv_f, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_token,
    int32_t* __restrict__ inv_perm) {
  extern __shared__ int32_t sm[];
  int32_t* oc = sm;           // [N] capped counts, then their exclusive offsets
  int32_t* wtot = sm + N;     // [PB_WAVES]
  const int tid = threadIdx.x;
  for (int e = tid; e < N; e += 256) oc[e] = min(counts_f[e], cap);
  __syncthreads();
  if (blockIdx.x == 0)
    for (int e = tid; e < N; e += 256) counts[e] = oc[e];
  __syncthreads();
  const int total = block_exclusive_scan(oc, N, wtot);
  if (blockIdx.x == 0) {
    for (int e = tid; e < N; e += 256) offsets[e] = oc[e];
    if (tid == 0) offsets[N] = total;
  }
  for (int a = blockIdx.x * 256 + tid; a < A; a += gridDim.x * 256) {
    const int e = idx[a];
    const int pos = inv_f[a];
    int r = -1;
    if (pos >= 0 && e >= 0 && e < N) {
      const int rank = pos - offsets_f[e];
      if (rank < cap) {
        r = oc[e] + rank;
        perm_token[r] = a / k;
      }
    }
    inv_perm[a] = r;
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

int permute_blocks(int T) { return T <= 0 ? 1 : ceil_div(T, PB_TOK); }

hipError_t launch_permute(const int32_t* topk_idx, int T, int k, int N, int32_t* hist,
                          int32_t* counts, int32_t* offsets, int32_t* perm_token,
                          int32_t* inv_perm, hipStream_t st) {
  int nbits = 1;
  while ((1 << nbits) <= N) ++nbits;  // 2^nbits > N: room for the sentinel
  const int nblk = permute_blocks(T);
  if (nblk > 1) {
    block_hist_kernel<<<nblk, 256, N * sizeof(int32_t), st>>>(topk_idx, T, k, N, hist);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t lds =
      ((size_t)(3 * PB_WAVES + 2) * N + PB_WAVES + (size_t)PB_TOK * k) * sizeof(int32_t);
  permute_kernel<<<nblk, 256, lds, st>>>(topk_idx, T, k, N, nbits, nblk > 1 ? hist : nullptr,
                                         nblk, counts, offsets, perm_token, inv_perm);
  return hipGetLastError();
}

hipError_t launch_capacity(const int32_t* topk_idx, int T, int k, int N, int cap,
                           const int32_t* counts_f, const int32_t* offsets_f, const int32_t* inv_f,
                           int32_t* counts, int32_t* offsets, int32_t* perm_token,
                           int32_t* inv_perm, hipStream_t st) {
  const int A = T * k;
  int grid = ceil_div(A, 256);
  grid = grid < 1 ? 1 : (grid > 1024 ? 1024 : grid);
  const size_t lds = ((size_t)N + PB_WAVES) * sizeof(int32_t);
  capacity_kernel<<<grid, 256, lds, st>>>(topk_idx, A, k, N, cap, counts_f, offsets_f, inv_f,
                                          counts, offsets, perm_token, inv_perm);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* perm_token, void* x_perm, int rows,
                              int row_bytes, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  gather_rows_kernel<<<rows, 256, 0, st>>>(static_cast<const uint8_t*>(x), perm_token,
                                           static_cast<uint8_t*>(x_perm), rows, row_bytes);
  return hipGetLastError();
}
