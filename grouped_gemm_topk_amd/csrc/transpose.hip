// Layout kernels of the grouped GEMM's backward pass.
//
// The MFMA grouped GEMM reduces along the contiguous dimension of both of its
// operands.  The gradients of the indexed grouped GEMM (axolotl page,
// cg_backward.py) reduce along other dimensions: the input gradient along the
// weights' output dimension N, the weight gradient along the rows of each
// expert.  These kernels move the operands into reduction-contiguous form:
//
//  transpose_kernel:        bf16 [B, R, C] -> [B, C, R] (the weights, per expert)
//  gather_transpose_kernel: the rows of the aligned (sorted, padded) order,
//                           gathered and written column-wise: dst[c][j] =
//                           src[row(j)][c], zero for a pad position
//  seg_table_kernel:        the padded-position window of every expert
//
// All three are HBM-bound: 64 x 128 tiles through LDS (four 16-byte loads in
// flight per thread), 16-byte global loads and stores along the contiguous
// dimension of each side (eight lanes cover one 128-byte line), rows of the
// LDS tile padded by one 32-bit word so that the column-wise reads of eight
// consecutive rows fall into distinct banks.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kTR = 64;         // tile rows of the source (positions for the gather)
constexpr int kTC = 128;        // tile columns of the source
constexpr int kPad = 2;         // bf16 elements of padding per LDS row
constexpr int kLoads = kTR * (kTC / 8) / 256;    // 16-byte loads per thread (4)
constexpr int kStores = kTC * (kTR / 8) / 256;   // 16-byte stores per thread (4)
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t Tile[kTR][kTC + kPad];

// 256 threads: kTR tile rows x kTC / 8 chunks of 8 elements, all loads issued
// before any LDS write.  src_row(r) gives the global row pointer of tile row r
// (or nullptr: zeros); a chunk is in range when col0 + 8 * ch < ncols.
template <typename SrcRow>
__device__ __forceinline__ void load_tile(Tile& tile, SrcRow src_row, int col0, int ncols) {
  const int tid = threadIdx.x;
  u32x4 v[kLoads];
#pragma unroll
  for (int q = 0; q < kLoads; ++q) {
    const int w = tid + 256 * q;
    const int r = w / (kTC / 8), ch = w % (kTC / 8);
    const uint16_t* row = src_row(r);
    v[q] = u32x4{0u, 0u, 0u, 0u};
    if (row && col0 + ch * 8 < ncols) v[q] = *(const u32x4*)(row + col0 + ch * 8);
  }
#pragma unroll
  for (int q = 0; q < kLoads; ++q) {
    const int w = tid + 256 * q;
    const int r = w / (kTC / 8), ch = w % (kTC / 8);
    unsigned* d = (unsigned*)&tile[r][ch * 8];   // 4-byte aligned (row stride 260 B)
    d[0] = v[q].x;
    d[1] = v[q].y;
    d[2] = v[q].z;
    d[3] = v[q].w;
  }
}

// writes the transposed tile: dst row (col0 + cc) gets tile column cc, 8
// consecutive tile rows per 16-byte store (eight lanes cover one 128-byte
// line); dst_row(cc) gives the output row pointer (already offset to the
// tile's first element) or nullptr; a chunk is written when row0 + 8 * ch < nrows
template <typename DstRow>
__device__ __forceinline__ void store_tile_t(Tile& tile, DstRow dst_row, int row0, int nrows) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < kStores; ++q) {
    const int w = tid + 256 * q;
    const int cc = w / (kTR / 8), ch = w % (kTR / 8);
    uint16_t* out = dst_row(cc);
    if (!out || row0 + ch * 8 >= nrows) continue;
    unsigned pk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pk[i] = (unsigned)tile[ch * 8 + 2 * i][cc] | ((unsigned)tile[ch * 8 + 2 * i + 1][cc] << 16);
    *(u32x4*)(out + ch * 8) = u32x4{pk[0], pk[1], pk[2], pk[3]};
  }
}

__global__ void __launch_bounds__(256) transpose_kernel(const uint16_t* __restrict__ src,
                                                        uint16_t* __restrict__ dst, int R, int C) {
  __shared__ Tile tile;
  const int c0 = blockIdx.x * kTC, r0 = blockIdx.y * kTR;
  const int64_t mat = (int64_t)R * C;
  const uint16_t* s = src + blockIdx.z * mat;
  uint16_t* d = dst + blockIdx.z * mat;
  load_tile(tile, [&](int r) { return r0 + r < R ? s + (int64_t)(r0 + r) * C : nullptr; }, c0, C);
  __syncthreads();
  store_tile_t(tile, [&](int cc) { return c0 + cc < C ? d + (int64_t)(c0 + cc) * R + r0 : nullptr; },
               r0, R);
}

__global__ void __launch_bounds__(256) gather_transpose_kernel(
    const uint16_t* __restrict__ src, int C, const int* __restrict__ sorted,
    const int* __restrict__ ntpp, int num_valid, int div, int cap, uint16_t* __restrict__ dst,
    int ld) {
  __shared__ Tile tile;
  const int c0 = blockIdx.x * kTC, j0 = blockIdx.y * kTR;
  const int total = *ntpp;
  if (j0 >= total) return;   // positions past the padded total are never read
  load_tile(tile, [&](int r) -> const uint16_t* {
    const int j = j0 + r;
    if (j >= total) return nullptr;
    const int sid = sorted[j];
    if (sid < 0 || sid >= num_valid) return nullptr;   // a pad: zeros
    return src + (int64_t)(div > 0 ? sid / div : sid) * C;
  }, c0, C);
  __syncthreads();
  store_tile_t(tile, [&](int cc) { return c0 + cc < C ? dst + (int64_t)(c0 + cc) * ld + j0 : nullptr; },
               j0, cap);
}

__global__ void __launch_bounds__(1024) seg_table_kernel(const int* __restrict__ expert_ids,
                                                         const int* __restrict__ ntpp, int bm, int E,
                                                         int* __restrict__ seg_beg,
                                                         int* __restrict__ seg_end) {
  __shared__ int s_beg[kMaxExperts], s_end[kMaxExperts];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) s_beg[e] = s_end[e] = 0;
  __syncthreads();
  const int nblk = *ntpp / bm;
  for (int b = tid; b < nblk; b += blockDim.x) {
    const int e = expert_ids[b];
    if (e < 0 || e >= E) continue;
    if (b == 0 || expert_ids[b - 1] != e) s_beg[e] = b * bm;
    if (b == nblk - 1 || expert_ids[b + 1] != e) s_end[e] = (b + 1) * bm;
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    seg_beg[e] = s_beg[e];
    seg_end[e] = s_end[e];
  }
}

}  // namespace

hipError_t launch_transpose(const uint16_t* src, uint16_t* dst, int B, int R, int C, hipStream_t s) {
  if (B == 0 || R == 0 || C == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_kernel, dim3((C + kTC - 1) / kTC, (R + kTR - 1) / kTR, B), dim3(256),
                     0, s, src, dst, R, C);
  return hipGetLastError();
}

hipError_t launch_gather_transpose(const uint16_t* src, int C, const int* sorted, const int* ntpp,
                                   int num_valid, int div, int cap, uint16_t* dst, int ld,
                                   hipStream_t s) {
  if (C == 0 || cap == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_transpose_kernel, dim3((C + kTC - 1) / kTC, (cap + kTR - 1) / kTR),
                     dim3(256), 0, s, src, C, sorted, ntpp, num_valid, div, cap, dst, ld);
  return hipGetLastError();
}

hipError_t launch_seg_table(const int* expert_ids, const int* ntpp, int block_m, int E,
                            int* seg_beg, int* seg_end, hipStream_t s) {
  hipLaunchKernelGGL(seg_table_kernel, dim3(1), dim3(1024), 0, s, expert_ids, ntpp, block_m, E,
                     seg_beg, seg_end);
  return hipGetLastError();
}

}  // namespace moe
