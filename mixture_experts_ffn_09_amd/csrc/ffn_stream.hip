// Grouped expert FFN for bfloat16 activations with bfloat16, FP8 (OCP E4M3,
// one float32 scale per 128x128 block) or MXFP4 (E2M1 codes, one E8M0 scale
// per 32 inputs) weights: the weight-streaming form, for few rows per expert
// (decode).
//
// An expert is a complete SwiGLU FFN with its own three matrices ("Mixture of
// Experts for LLM Inference", "The MoE change is surprisingly local";
// "Mixture of Experts Explained", "The slot it replaces, and what an expert
// is").  Pass 1 computes H = silu(X Wg^T) * (X Wu^T) with the SwiGLU in the
// epilogue; pass 2 computes Y = H Wd^T.  Only experts that received rows
// touch their weights.
//
// Work split: grid.y = group (routed expert, then the shared expert), grid.x
// over 16-row blocks of the weight matrix.  Each wave owns NP such blocks
// (pairs of gate/up blocks in pass 1) and streams them along K exactly once
// per 16*MB rows of activations, so the weight stream is read once for up to
// 16*MB rows.  Weights are pre-packed so that one K step of one block is a
// contiguous 1 KB: each lane's 16-byte load is its v_mfma_f32_16x16x32_bf16
// B operand (bf16) or two of them (fp8, converted exactly to bf16 in
// registers; MXFP4 words decoded with their scales), and a wave's loads are
// fully coalesced.  The activation fragments of a chunk of K steps, the same
// for all of a workgroup's waves, are copied once per workgroup into LDS
// (double-buffered) where the K steps allow it; otherwise each wave reads
// them from L2.
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
  int T, N, g0;
  int a_rows;    // rows of `a` (T with perm, else the assignments)
  int n_routed;  // routed groups in this launch (g0 .. g0+n_routed-1)
  int sh_rows;   // rows per shared-expert slice (grid rows past the routed ones)
  int K;       // reduction length
  int n_out;   // output width
  const uint8_t* w;           // packed routed weights
  const uint8_t* w_sh;        // packed shared weights
  const void* s;              // fp8 (float32) or MXFP4 (E8M0 byte) scales, routed
  const void* s_sh;           // the same, shared expert
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

// Weight formats of the streaming kernel
constexpr int WF_BF16 = 0, WF_FP8 = 1, WF_MXFP4 = 2;

// GATED: pass 1 (gate+up, SwiGLU) else pass 2 (down).  One wave owns NP
// consecutive 16-row output blocks and walks K with a ring of D K-steps of
// loads in flight (each step: NP * NH weight blocks of 1 KB plus MB
// activation fragments, which serve all NP blocks).  Activation rows past
// the group's end are clamped to its last row: row m of an MFMA result
// depends only on row m of A, and those rows are not stored.
// SQ4 (MXFP4 with K % 512 == 0): a lane's E8M0 scales of four consecutive
// K steps are 16 contiguous bytes of its row, fetched with one load per four
// steps instead of one per step; the loop then advances four steps at a time.
// LDSA: the activation fragments, the same for the workgroup's four waves,
// are copied once per workgroup into LDS (global-to-LDS copies in fragment
// order, a double buffer of CH K steps, each wave copying a quarter) and
// read from there, instead of once per wave from L2: a quarter of the
// activation load instructions, which otherwise outnumber the weight loads'
// cache-line requests.  One barrier per chunk: after it every wave's copies
// of this chunk have landed and every wave has finished reading the previous
// one, whose buffer the next chunk's copies then reuse.  `store` is false for
// a wave past the last weight block: it mirrors a valid block to take part in
// the copies and barriers, and stores nothing.
template <int MB, int NP, int D, int FMT, bool GATED, bool SQ4 = false, bool LDSA = false>
__device__ __forceinline__ void stream_body(const StreamParams& p, int nb0, int g, bool shared,
                                            int row_base, int rows, int m_first, uint8_t* alds,
                                            bool store) {
  constexpr bool FP8 = FMT == WF_FP8, FP4 = FMT == WF_MXFP4;
  constexpr int NH = GATED ? 2 : 1;
  constexpr int AF = FP4 ? 4 : (FP8 ? 2 : 1);  // 32-wide activation fragments per K step
  static_assert(!FP8 || D % 2 == 0, "FP8 needs an even ring depth");
  static_assert(8 % NP == 0, "the NP blocks of a wave share one 128-row scale block");
  const int lane = threadIdx.x & 63;
  uint16_t* out = shared ? p.out_sh : p.out;

  // bytes of one group's weights: bf16 2, fp8 1, MXFP4 1/2 per element
  const size_t wbytes = (size_t)NH * p.n_out * p.K * (FP8 ? 2 : (FP4 ? 1 : 4)) / 2;
  const uint8_t* W = shared ? p.w_sh : p.w + (size_t)g * wbytes;
  const int KS = p.K / (32 * AF);                 // K steps of one 1 KB block
  const size_t bstride = (size_t)KS * NH * 1024;  // one 16-row block, all K
  const uint8_t* Wnb = W + (size_t)nb0 * bstride + lane * 16;
  const int SK = p.K / MOE_FP8_BLOCK;
  const int SR = p.n_out / MOE_FP8_BLOCK;
  const float* S = nullptr;
  if (FP8)
    S = (shared ? static_cast<const float*>(p.s_sh)
                : static_cast<const float*>(p.s) + (size_t)g * NH * SR * SK) +
        (size_t)((nb0 * 16) / MOE_FP8_BLOCK) * SK;
  // MXFP4: one E8M0 byte per 32 inputs of a row, packed per group as
  // [row block][group of 4 K steps][NH][16 rows][16 bytes]; a lane's scales
  // of four steps are one 16-byte chunk, of one step 4 bytes of it
  const int KQ = (p.K / 32 + 15) / 16;
  const uint8_t* S4 = nullptr;
  if (FP4)
    S4 = (shared ? static_cast<const uint8_t*>(p.s_sh)
                 : static_cast<const uint8_t*>(p.s) + (size_t)g * NH * p.n_out * KQ * 16) +
         (size_t)nb0 * KQ * NH * 256 + (lane & 15) * 16;
  // chunk of block nb0 + j, matrix h, K steps 4 kq .. 4 kq + 3
  auto s4_chunk = [&](int j, int h, int kq) {
    return S4 + ((size_t)(j * KQ + kq) * NH + h) * 256;
  };

  const int lrow = lane & 15;
  const int lk = (lane >> 4) * 8;
  // LDSA copies are buffer loads: a uniform resource over the activation
  // rows and per-lane 32-bit byte offsets (the launch checks they fit); the
  // buffer form keeps the compiler's own vmcnt waits exact
  const uint16_t* abase = shared ? p.a_sh : p.a;
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      (void*)abase, 0,
      (int)(uint32_t)((size_t)(shared || p.perm ? p.T : row_base + rows) * p.K * 2),
      BUF_DWORD3);

  for (int m0 = m_first; m0 < rows; m0 += 16 * MB) {
    const uint16_t* arow[MB];
    uint32_t aoff[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = min(m0 + mb * 16 + lrow, rows - 1);
      int src;
      if (shared)
        src = r;
      else if (p.perm)
        src = p.perm[row_base + r];
      else
        src = row_base + r;
      arow[mb] = abase + (size_t)src * p.K + lk;
      aoff[mb] = ((uint32_t)src * (uint32_t)p.K + lk) * 2;
    }

    floatx4_t acc[NP][NH][MB];
    floatx4_t part[NP][NH][MB];
#pragma unroll
    for (int j = 0; j < NP; ++j)
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          acc[j][h][mb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
          part[j][h][mb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        }

    // steps per inner iteration: the ring depth, or four for the scale quads;
    // with LDSA, steps per LDS chunk (at least 8 KB of fragments)
    constexpr int G = SQ4 ? (D > 4 ? D : 4) : D;
    constexpr int CH = LDSA ? (G > 8 / (MB * AF) ? G : 8 / (MB * AF)) : G;
    constexpr int NF = CH * MB * AF;            // 1 KB fragments per chunk
    constexpr int NPH = NP * NH;                // weight loads per step
    static_assert(!LDSA || (NF % SW_WAVES == 0 && NF <= 16), "LDS chunk");
    static_assert(!LDSA || !FP4 || SQ4, "per-step scale loads are not counted");
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // issue this wave's share of the copies of chunk c into buffer c & 1
    auto copy_chunk = [&](int c) {
#pragma unroll
      for (int t = 0; t < (LDSA ? NF / SW_WAVES : 0); ++t) {
        const int fi = t * SW_WAVES + wave;     // fragment (step, row block, part)
        const int cs = fi / (MB * AF), mb = (fi / AF) % MB, f = fi % AF;
        uint32_t ro = aoff[0];
#pragma unroll
        for (int q = 1; q < MB; ++q)
          if (mb == q) ro = aoff[q];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ares, (lds_ptr_t)(alds + (c & 1) * (NF * 1024) + fi * 1024), 16, ro,
            ((c * CH + cs) * (32 * AF) + f * 32) * 2, 0, 0);
      }
    };
    if (LDSA) {
      barrier_no_fence();  // the previous pass has finished reading both buffers
      copy_chunk(0);
      __builtin_amdgcn_sched_barrier(0);
    }

    u32x4_t bq[D][NP][NH];
    u32x4_t aq[D][MB][AF];
    u32x4_t ach[LDSA ? CH : 1][MB][AF];   // the current chunk's fragments
    // FP8 block scales ride in the ring with the weights (an odd slot holds
    // an odd step, which closes a 128-wide block): loaded right before use,
    // the wait for them would drain the whole ring every second step
    float sfq[FP8 ? D : 1][NH];
    uint32_t sq[FP4 && !SQ4 ? D : 1][NP][NH];
    u32x4_t sqc[SQ4 ? NP : 1][SQ4 ? NH : 1], sqn[SQ4 ? NP : 1][SQ4 ? NH : 1];
    // scales of K steps ks .. ks+3, all NP blocks and both halves
    auto load_sq4 = [&](u32x4_t (&q)[SQ4 ? NP : 1][SQ4 ? NH : 1], int ks) {
#pragma unroll
      for (int j = 0; j < (SQ4 ? NP : 0); ++j)
#pragma unroll
        for (int h = 0; h < NH; ++h)
          q[j][h] = *reinterpret_cast<const u32x4_t*>(s4_chunk(j, h, ks >> 2));
    };
    if (SQ4) load_sq4(sqn, 0);
    auto load_step = [&](int u, int ks) {
#pragma unroll
      for (int j = 0; j < NP; ++j)
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          // non-temporal: each weight byte is read once per pass, and the
          // streaming cache policy sustains more read bandwidth (a plain
          // stream of this shape: 6.1 TB/s with ordinary loads, 6.8 with
          // non-temporal ones)
          bq[u][j][h] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4_t*>(Wnb + j * bstride + ((size_t)ks * NH + h) * 1024));
          if (FP4 && !SQ4)
            sq[FP4 && !SQ4 ? u : 0][j][h] =
                *reinterpret_cast<const uint32_t*>(s4_chunk(j, h, ks >> 2) + (ks & 3) * 4);
        }
      if (FP8 && (u & 1)) {
#pragma unroll
        for (int h = 0; h < NH; ++h) sfq[FP8 ? u : 0][h] = S[(size_t)h * SR * SK + (ks >> 1)];
      }
#pragma unroll
      for (int mb = 0; mb < (LDSA ? 0 : MB); ++mb)
#pragma unroll
        for (int f = 0; f < AF; ++f)
          aq[u][mb][f] = *reinterpret_cast<const u32x4_t*>(arow[mb] + ks * (32 * AF) + f * 32);
    };
#pragma unroll
    for (int u = 0; u < D; ++u) load_step(u, min(u, KS - 1));
    // keep the ring: the scheduler must not sink loads next to their use
    __builtin_amdgcn_sched_barrier(0);

    for (int ks0 = 0; ks0 < KS; ks0 += CH) {
      if (LDSA) {
        // this wave's copies of the chunk have landed once at most the loads
        // issued after them are outstanding: the ring's prologue for the
        // first chunk, the previous chunk's refills (and scale quads) later
        // (a lower bound of the count: the weight loads and scale quads;
        // any other vector load after the copies only makes the wait longer)
        if (ks0 == 0)
          wait_vmcnt<(SQ4 ? NPH : 0) + D * NPH>();
        else
          wait_vmcnt<CH * NPH + (SQ4 ? (CH / 4) * NPH : 0)>();
        barrier_no_fence();
        // read the whole chunk before the next chunk's copies are issued, so
        // no LDS read has to wait for copies still in flight
        const uint8_t* abuf = alds + ((ks0 / CH) & 1) * (NF * 1024) + lane * 16;
#pragma unroll
        for (int i = 0; i < CH; ++i)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int f = 0; f < AF; ++f)
              ach[LDSA ? i : 0][mb][f] =
                  *reinterpret_cast<const u32x4_t*>(abuf + ((i * MB + mb) * AF + f) * 1024);
        __builtin_amdgcn_sched_barrier(0);
        // the last chunk copies itself again into the idle buffer: with no
        // branch, the compiler's own waits stay exact across iterations; a
        // fragment is always copied by the same wave, so its copies land in
        // issue order
        copy_chunk(min(ks0 / CH + 1, KS / CH - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int u = i % D;      // ring slot
        const int ks = ks0 + i;   // KS is a multiple of CH: no bounds branch
        if (LDSA) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int f = 0; f < AF; ++f) aq[u][mb][f] = ach[LDSA ? i : 0][mb][f];
        }
        if (SQ4 && (i & 3) == 0) {
#pragma unroll
          for (int j = 0; j < (SQ4 ? NP : 0); ++j)
#pragma unroll
            for (int h = 0; h < NH; ++h) sqc[j][h] = sqn[j][h];
          load_sq4(sqn, min(ks + 4, KS - 4));
        }
        if (FP4) {
          // four 32-wide K steps per block: word s4 of a lane's 16 bytes holds
          // its 8 codes of step s4, decoded with the step's scale straight to
          // bf16 (a power of two times an E2M1 value is exact in bf16)
#pragma unroll
          for (int j = 0; j < NP; ++j)
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
              for (int s4 = 0; s4 < 4; ++s4) {
                const uint32_t sw = SQ4 ? sqc[SQ4 ? j : 0][SQ4 ? h : 0][i & 3]
                                        : sq[FP4 && !SQ4 ? u : 0][j][h];
                const u32x4_t b = fp4_word_to_bf16(bq[u][j][h][s4], (sw >> (8 * s4)) & 0xffu);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                  acc[j][h][mb] = mfma16x16x32(aq[u][mb][s4], b, acc[j][h][mb]);
              }
        } else if (!FP8) {
#pragma unroll
          for (int j = 0; j < NP; ++j)
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
              for (int mb = 0; mb < MB; ++mb)
                acc[j][h][mb] = mfma16x16x32(aq[u][mb][0], bq[u][j][h], acc[j][h][mb]);
        } else {
#pragma unroll
          for (int j = 0; j < NP; ++j)
#pragma unroll
            for (int h = 0; h < NH; ++h) {
              u32x4_t blo, bhi;
              fp8_block_to_bf16(bq[u][j][h], blo, bhi);
#pragma unroll
              for (int mb = 0; mb < MB; ++mb) {
                part[j][h][mb] = mfma16x16x32(aq[u][mb][0], blo, part[j][h][mb]);
                part[j][h][mb] = mfma16x16x32(aq[u][mb][AF - 1], bhi, part[j][h][mb]);
              }
            }
          // every second 64-wide step closes a 128-wide scale block (D is
          // even and ks0 a multiple of D, so ks and u have the same parity)
          if (u & 1) {
#pragma unroll
            for (int h = 0; h < NH; ++h) {
              const float sc = sfq[FP8 ? u : 0][h];
#pragma unroll
              for (int j = 0; j < NP; ++j)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
                  for (int e = 0; e < 4; ++e) acc[j][h][mb][e] += sc * part[j][h][mb][e];
                  part[j][h][mb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
                }
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        load_step(u, min(ks + D, KS - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    if (LDSA) wait_vmcnt<0>();  // no copy outlives the pass
    // epilogue: lane holds rows 4*(lane/16)+e of column lane%16
    if (LDSA && !store) continue;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int n = (nb0 + j) * 16 + lrow;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = m0 + mb * 16 + (lane >> 4) * 4 + e;
          if (r >= rows) continue;
          float v;
          if (GATED)
            v = silu_f32(acc[j][0][mb][e]) * acc[j][NH - 1][mb][e];
          else
            v = acc[j][0][mb][e];
          out[(size_t)(row_base + r) * p.n_out + n] = (uint16_t)f32_to_bf16(v);
        }
    }
  }
}

// HOT: a routed group (or a slice of the shared expert) with more than 16
// rows takes passes of 32 rows (MB = 2, half the ring depth) and one with
// more than 32 rows passes of 64 (MB = 4, a quarter of it, but 2 at most and
// never more than D), so the registers stay within the 16-row form's,
// instead of streaming its weights once per 16 rows: with skewed routing a
// few hot experts hold many of the rows (on the skewed fp8 decode workload
// this cut the gate/up time by 12%).  Each ring
// depth used here divides D, and D divides the K steps, so the K loop never
// runs past the last step.
template <int MB, int NP, int D, int FMT, bool GATED, bool HOT, bool LDSA>
__global__ __launch_bounds__(256) void ffn_stream_kernel(StreamParams p) {
  // activation chunks: two buffers of up to 8 KB (bf16) or 16 KB (FP8, MXFP4)
  __shared__ __attribute__((aligned(1024))) uint8_t alds[LDSA ? (FMT == WF_BF16 ? 16384 : 32768) : 1024];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NB = p.n_out / 16;  // a multiple of NP
  int nb0 = (blockIdx.x * SW_WAVES + wave) * NP;
  const bool store = nb0 < NB;
  if (!store) {
    if (!LDSA) return;
    nb0 = NB - NP;  // mirror a valid block for the copies and barriers
  }

  // grid rows: routed groups, then slices of the shared expert's T rows
  const bool shared = (int)blockIdx.y >= p.n_routed;
  const int g = shared ? p.N : p.g0 + blockIdx.y;
  int row_base, rows, m_first = 0;
  if (!shared) {
    row_base = p.offsets[g];
    rows = p.offsets[g + 1] - row_base;
  } else {
    row_base = 0;
    m_first = (blockIdx.y - p.n_routed) * p.sh_rows;
    rows = min(p.T, m_first + p.sh_rows);
  }
  if (rows <= m_first) return;
  // rows of this grid row: a routed group, or one slice of the shared expert
  const int nrows = rows - m_first;
  if (HOT && nrows > 32)
    stream_body<4, NP, (D >= 8 ? D / 4 : (D >= 2 ? 2 : 1)), FMT, GATED, false, LDSA && HOT>(
        p, nb0, g, shared, row_base, rows, m_first, alds, store);
  else if (HOT && nrows > 16)
    stream_body<2, NP, (D >= 4 ? D / 2 : D), FMT, GATED, false, LDSA && HOT>(
        p, nb0, g, shared, row_base, rows, m_first, alds, store);
  else if (FMT == WF_MXFP4 && p.K % 512 == 0 &&
           ((uintptr_t)(shared ? p.s_sh : p.s) & 15) == 0)
    stream_body<MB, NP, D, FMT, GATED, FMT == WF_MXFP4, LDSA>(p, nb0, g, shared, row_base, rows,
                                                              m_first, alds, store);
  else
    stream_body<MB, NP, D, FMT, GATED, false, LDSA && FMT != WF_MXFP4>(
        p, nb0, g, shared, row_base, rows, m_first, alds, store);
}

template <int MB, int NP, int D, int FMT, bool GATED>
hipError_t launch_stream_d(const StreamParams& sp, int groups, hipStream_t st) {
  // groups = grid rows (routed groups + shared slices)
  const int NW = sp.n_out / 16 / NP;  // waves per group
  dim3 grid(ceil_div(NW, SW_WAVES), groups);
  // the per-group 32- and 64-row passes need the 16-row form's register room;
  // the MXFP4 form (four activation fragments per step) has none to spare
  constexpr bool HOT = MB == 1 && FMT != WF_MXFP4;
  // activations through LDS where every pass width's chunk divides the K
  // steps (chunks are at most 8 steps); MXFP4 only with 16-row passes
  const int KS = sp.K / (FMT == WF_MXFP4 ? 128 : (FMT == WF_FP8 ? 64 : 32));
  constexpr bool LOK = FMT != WF_MXFP4 || MB == 1;
  const bool fits = (long long)(sp.a_rows > sp.T ? sp.a_rows : sp.T) * sp.K * 2 <= 0x7fffffffLL;
  if (LOK && KS % 8 == 0 && fits)
    ffn_stream_kernel<MB, NP, D, FMT, GATED, HOT, LOK><<<grid, SW_WAVES * 64, 0, st>>>(sp);
  else
    ffn_stream_kernel<MB, NP, D, FMT, GATED, HOT, false><<<grid, SW_WAVES * 64, 0, st>>>(sp);
  return hipGetLastError();
}

// The ring depth must divide the number of K steps; it shrinks as NP or MB
// grow (down to 2) so that the registers of the ring stay within an
// occupancy of two or more waves per SIMD.  An MXFP4 step carries four
// activation fragments and its LDS chunk holds at most 16, so its ring is at
// most 4 deep (4 rather than 2 with two blocks per wave: the same two waves
// per SIMD, and the 4096 x 14336 down pass 57% -> 66% of HBM peak).
template <int MB, int NP, int FMT, bool GATED>
hipError_t launch_stream(const StreamParams& sp, int groups, hipStream_t st) {
  constexpr int DF = 8 / (NP * MB);
  constexpr int DR = FMT == WF_MXFP4 && DF > 4 ? 4 : DF;
  constexpr int DMAX = DR < 2 ? 2 : DR;
  const int KS = sp.K / (FMT == WF_MXFP4 ? 128 : (FMT == WF_FP8 ? 64 : 32));
  if (DMAX >= 8 && KS % 8 == 0) return launch_stream_d<MB, NP, (DMAX >= 8 ? 8 : 2), FMT, GATED>(sp, groups, st);
  if (DMAX >= 4 && KS % 4 == 0) return launch_stream_d<MB, NP, (DMAX >= 4 ? 4 : 2), FMT, GATED>(sp, groups, st);
  if (KS % 2 == 0) return launch_stream_d<MB, NP, 2, FMT, GATED>(sp, groups, st);
  // FP8 K is a multiple of 128, so KS is even there
  return launch_stream_d<MB, NP, (FMT == WF_FP8 ? 2 : 1), FMT, GATED>(sp, groups, st);
}

// Weight blocks per wave.  The activation fragments of a K step are loaded
// once per workgroup into LDS where the K steps allow it (else once per
// wave) and used for all of a wave's blocks.  MXFP4 steps carry
// four activation fragments per 1 KB weight block; on its down pass two
// blocks per wave measured faster (34% -> 42% of HBM peak with a ring of 2),
// on its gate/up pass one block with a ring of 4 (60% -> 68%).  Everywhere
// else one block per wave with the deepest ring measured fastest (the fp8
// 7168 x 2048 down projection once took two blocks, when every wave read its
// own activation fragments; with the fragments in LDS one block is 2.5%
// faster on that pass).
int stream_np(int fmt, bool gated, int n_out) {
  const int NB = n_out / 16;
  int np = (fmt == WF_MXFP4 && !gated) ? 2 : 1;
  while (np > 1 && NB % np) np >>= 1;
  return np;
}

}  // namespace

template <int MB, int FMT>
static hipError_t stream_pass_fmt(bool gated, const StreamParams& sp, int groups,
                                  hipStream_t st) {
  const int np = stream_np(FMT, gated, sp.n_out);
  if (np == 2)
    return gated ? launch_stream<MB, 2, FMT, true>(sp, groups, st)
                 : launch_stream<MB, 2, FMT, false>(sp, groups, st);
  return gated ? launch_stream<MB, 1, FMT, true>(sp, groups, st)
               : launch_stream<MB, 1, FMT, false>(sp, groups, st);
}

template <int MB>
static hipError_t stream_pass(int fmt, bool gated, const StreamParams& sp, int groups,
                              hipStream_t st) {
  if (fmt == WF_FP8) return stream_pass_fmt<MB, WF_FP8>(gated, sp, groups, st);
  if (fmt == WF_MXFP4) return stream_pass_fmt<MB, WF_MXFP4>(gated, sp, groups, st);
  return stream_pass_fmt<MB, WF_BF16>(gated, sp, groups, st);
}

hipError_t launch_ffn_stream(const FfnArgs& a, int pass, int g0, int g1, int rows_hint,
                             hipStream_t st) {
  if (g1 <= g0) return hipSuccess;
  const int mb = rows_hint <= 16 ? 1 : (rows_hint <= 32 ? 2 : 4);
  const int fmt = a.fp8 ? WF_FP8 : (a.mxfp4 ? WF_MXFP4 : WF_BF16);

  const bool with_shared = g1 > a.N;
  const int n_routed = (g1 > a.N ? a.N : g1) - g0;
  // the shared expert's rows are cut into slices of one pass each, run side
  // by side; where the 64-row passes exist (16-row launches, not MXFP4)
  // each slice is 64 rows, so the shared weights are streamed once per 64
  // tokens rather than per 16 (dsv3-decode-fp8: 4 slices instead of 16)
  const bool hot = mb == 1 && fmt != WF_MXFP4;
  const int sh_rows = hot ? 64 : 16 * mb;
  const int sh_slices = with_shared ? ceil_div(a.T, sh_rows) : 0;
  StreamParams up{};
  up.a = a.x_rows;
  up.perm = a.perm_token;
  up.a_sh = a.x_sh;
  up.offsets = a.offsets;
  up.T = a.T;
  up.a_rows = a.perm_token ? a.T : a.T * a.k;
  up.N = a.N;
  up.g0 = g0;
  up.n_routed = n_routed;
  up.sh_rows = sh_rows;
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
  dn.a_rows = a.T * a.k;
  dn.a_sh = a.H_sh;
  dn.K = a.d_ff;
  dn.n_out = a.d;
  dn.w = static_cast<const uint8_t*>(a.w2);
  dn.w_sh = static_cast<const uint8_t*>(a.w2_sh);
  dn.s = a.s2;
  dn.s_sh = a.s2_sh;
  dn.out = a.Y;
  dn.out_sh = a.Y_sh;

  const int groups = n_routed + sh_slices;
  // rows held per pass: 16 * MB (a group with more rows takes more passes)
  hipError_t e = hipSuccess;
  for (int ps = 1; ps <= 2 && e == hipSuccess; ++ps) {
    if (!(pass & ps)) continue;
    const StreamParams& sp = ps == 1 ? up : dn;
    if (mb == 1)
      e = stream_pass<1>(fmt, ps == 1, sp, groups, st);
    else if (mb == 2)
      e = stream_pass<2>(fmt, ps == 1, sp, groups, st);
    else
      e = stream_pass<4>(fmt, ps == 1, sp, groups, st);
  }
  return e;
}

hipError_t launch_ffn_lowp(const FfnArgs& a, int pass, hipStream_t st) {
  // MXFP4 weights take the tiled GEMM only in its four-wave form (the one
  // with an E2M1 operand path)
  const bool gemm_ok = gemm_shape_ok(a.d, a.d_ff) && (!a.mxfp4 || gemm_four_wave_ok(a));
  const int avg = (int)(((long long)a.T * a.k + a.N - 1) / a.N);  // rows per routed expert
  const bool routed_gemm = gemm_ok && avg >= 64;
  // the shared expert joins a routed streaming launch up to a few hundred
  // tokens; beyond that, or next to a routed GEMM, it is a GEMM too
  const bool shared_gemm = gemm_ok && a.n_shared && (routed_gemm ? a.T >= 64 : a.T > 512);
  hipError_t e = hipSuccess;
  // Run pass by pass so the down projection always sees complete H rows.
  for (int ps = 1; ps <= 2; ++ps) {
    if (!(pass & ps)) continue;
    if (routed_gemm && shared_gemm) {
      // one launch over routed + shared groups: their tiles share the machine
      e = launch_ffn_gemm(a, ps, 0, a.N + 1, a.T * a.k + a.T, a.sched, st);
      if (e != hipSuccess) return e;
      continue;
    }
    if (routed_gemm) {
      e = launch_ffn_gemm(a, ps, 0, a.N, a.T * a.k, a.sched, st);
      if (e != hipSuccess) return e;
      if (a.n_shared)  // shared_gemm is false only below 64 tokens
        e = launch_ffn_stream(a, ps, a.N, a.N + 1, a.T, st);
    } else if (a.n_shared && !shared_gemm) {
      e = launch_ffn_stream(a, ps, 0, a.N + 1, avg, st);  // routed + shared slices
    } else {
      e = launch_ffn_stream(a, ps, 0, a.N, avg, st);
      if (e == hipSuccess && a.n_shared)
        e = launch_ffn_gemm(a, ps, a.N, a.N + 1, a.T, a.sched, st);
    }
    if (e != hipSuccess) return e;
  }
  return e;
}
