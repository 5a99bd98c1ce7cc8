// One-time repack of expert weights from [out][in] row-major into the
// streaming kernels' block layout.
//
// A block covers 16 output rows and one K step (32 inputs for bf16, 64 for
// FP8, 128 for MXFP4) and is 1 KB: 64 lanes x 16 bytes, lane l holding row
// l % 16 and the 8 (bf16), 2 x 8 (FP8: k-steps 2s and 2s+1 of 32) or 4 x 8
// (MXFP4: k-steps 4s .. 4s+3, 4 bytes each) consecutive inputs starting at
// 8 * (l / 16) - exactly its MFMA B operand(s).  Blocks are ordered
// (expert, row block, K step, matrix) with matrix = gate, up for the fused
// gate/up weight, so one row block's stream along K is contiguous.
//
// MXFP4 scales (one E8M0 byte per 32 inputs of a row) are repacked so that
// the scales a wave needs together are contiguous: for each expert, 16-row
// block, group of four 128-wide K steps (16 scale bytes of a row) and matrix
// (gate, up), 16 rows x 16 bytes = 256 bytes, rows in order; a last, partial
// group is padded with zero bytes.  A lane's scales for four K steps are then
// one 16-byte chunk, and the 16 rows of a block two cache lines.

#include "common.h"
#include "kernels.h"

namespace {

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ a,
                                                   const uint8_t* __restrict__ b,
                                                   uint8_t* __restrict__ dst, int rows,
                                                   int cols, int esize, int nh,
                                                   size_t total_chunks) {
  const size_t c = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= total_chunks) return;
  const int lane = (int)(c & 63);
  size_t blk = c >> 6;
  const int ksteps = esize == 2 ? cols / 32 : (esize == 1 ? cols / 64 : cols / 128);
  const int h = (int)(blk % nh);
  blk /= nh;
  const int ks = (int)(blk % ksteps);
  blk /= ksteps;
  const int nb = (int)(blk % (rows / 16));
  const size_t e = blk / (rows / 16);
  // bytes per matrix: esize 0 marks MXFP4 (two codes per byte)
  const size_t mat_bytes = esize ? (size_t)rows * cols * esize : (size_t)rows * cols / 2;
  const uint8_t* src = (h ? b : a) + e * mat_bytes;
  const int row = nb * 16 + (lane & 15);
  uint8_t* out = dst + c * 16;
  if (esize == 0) {
    // 4 steps of 32 inputs: word s holds the lane's 8 codes of step s
    const int col = ks * 128 + (lane >> 4) * 8;
    const uint8_t* s = src + (size_t)row * (cols / 2) + col / 2;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint32_t*>(out + 4 * q) = *reinterpret_cast<const uint32_t*>(s + 16 * q);
  } else if (esize == 2) {
    const int col = ks * 32 + (lane >> 4) * 8;
    *reinterpret_cast<uint4*>(out) =
        *reinterpret_cast<const uint4*>(src + ((size_t)row * cols + col) * 2);
  } else {
    const int col = ks * 64 + (lane >> 4) * 8;
    const uint8_t* s = src + (size_t)row * cols + col;
    *reinterpret_cast<uint2*>(out) = *reinterpret_cast<const uint2*>(s);
    *reinterpret_cast<uint2*>(out + 8) = *reinterpret_cast<const uint2*>(s + 32);
  }
}

// One 16-byte chunk of packed MXFP4 scales per thread: chunk c = ((((e * RB
// + rb) * KQ + kq) * nh + h) * 16 + r), from row rb * 16 + r of matrix h of
// expert e in the natural [e][h][rows][cols / 32] layout.
__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t* __restrict__ src,
                                                          uint8_t* __restrict__ dst, int rows,
                                                          int sbytes, int kq_n, int nh,
                                                          size_t total_chunks) {
  const size_t c = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= total_chunks) return;
  size_t t = c;
  const int r = (int)(t % 16);
  t /= 16;
  const int h = (int)(t % nh);
  t /= nh;
  const int kq = (int)(t % kq_n);
  t /= kq_n;
  const int rb = (int)(t % (rows / 16));
  const size_t e = t / (rows / 16);
  const uint8_t* row = src + ((e * nh + h) * rows + rb * 16 + r) * (size_t)sbytes;
  uint8_t* out = dst + c * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int col = kq * 16 + i;
    out[i] = col < sbytes ? row[col] : 0;
  }
}

}  // namespace

size_t packed_scale_bytes(int n_mats, int rows, int cols, int nh) {
  const int kq_n = (cols / 32 + 15) / 16;
  return (size_t)n_mats * nh * rows * kq_n * 16;
}

hipError_t launch_pack_scales(const void* src, void* dst, int n_mats, int rows, int cols, int nh,
                              hipStream_t st) {
  const int sbytes = cols / 32;
  const int kq_n = (sbytes + 15) / 16;
  const size_t chunks = packed_scale_bytes(n_mats, rows, cols, nh) / 16;
  const size_t grid = (chunks + 255) / 256;
  pack_scales_kernel<<<dim3((unsigned)grid), 256, 0, st>>>(
      static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), rows, sbytes, kq_n, nh,
      chunks);
  return hipGetLastError();
}

hipError_t launch_pack(const void* src_a, const void* src_b, void* dst, int n_mats, int rows,
                       int cols, int esize, hipStream_t st) {
  const int nh = src_b ? 2 : 1;
  const size_t bytes = esize ? (size_t)n_mats * nh * rows * cols * esize
                             : (size_t)n_mats * nh * rows * cols / 2;
  if (esize == 4) {
    // float32 weights keep the natural layout: gate block then up block
    const size_t one = (size_t)rows * cols * 4;
    for (int e = 0; e < n_mats; ++e) {
      hipError_t r = hipMemcpyAsync(static_cast<uint8_t*>(dst) + (size_t)e * nh * one,
                                    static_cast<const uint8_t*>(src_a) + (size_t)e * one, one,
                                    hipMemcpyDeviceToDevice, st);
      if (r != hipSuccess) return r;
      if (nh == 2) {
        r = hipMemcpyAsync(static_cast<uint8_t*>(dst) + (size_t)e * nh * one + one,
                           static_cast<const uint8_t*>(src_b) + (size_t)e * one, one,
                           hipMemcpyDeviceToDevice, st);
        if (r != hipSuccess) return r;
      }
    }
    return hipSuccess;
  }
  const size_t chunks = bytes / 16;
  const size_t grid = (chunks + 255) / 256;
  pack_kernel<<<dim3((unsigned)grid), 256, 0, st>>>(static_cast<const uint8_t*>(src_a),
                                                    static_cast<const uint8_t*>(src_b),
                                                    static_cast<uint8_t*>(dst), rows, cols,
                                                    esize, nh, chunks);
  return hipGetLastError();
}
