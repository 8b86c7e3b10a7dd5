// Decode path (T <= 16 tokens): expert GEMVs that stream every touched
// expert's weights from HBM once and apply them to all tokens routed to it.
//
// The aligned layout already groups the slots of one expert into one block
// (each expert has at most T <= 16 slots), which is the dedupe of duplicate
// experts across tokens of the B70 grouped multi-token experiment (*Intent*):
// one read of the expert's rows serves every token that picked it.  The
// activation is fused into the first GEMV (SwiGLU of the axolotl DeepSeek-V3
// MoE forward, relu^2 of the mlxcel fc1 kernel) and the routed weight plus the
// sum over the k slots into the second (skill card *Common Pitfalls* 4).
//
// gfx950 mapping.  The work is HBM-bound, so the kernels are shaped for bytes
// in flight, not for MFMA rate: one v_mfma_f32_16x16x32_bf16 tile covers 16
// weight rows x up to 16 tokens.  K is permuted inside each 256-wide round so
// that every lane reads 128 contiguous bytes of one weight row (8 x 16-byte
// loads) and the token operand is read with the same permutation; a sum over
// k is indifferent to the order of its terms.  GEMV1 splits K across the 4
// waves of a workgroup and reduces in LDS before the activation; GEMV2 gives
// each wave its own 16 output rows and adds the weighted results into `out`
// with fp32 atomics (the k slots of a token land in any order).
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRound = 256;   // K elements per round: 4 lane groups x 64

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Token rows of block b: for column j < 16 returns the token (or -1) and slot.
struct BlockRows {
  bool shared;
  int base;      // first padded position of the block
};

__device__ __forceinline__ int block_token(const GemvParams& p, const BlockRows& br, int j,
                                           int* slot) {
  if (br.shared) {
    *slot = -1;
    return j < p.T ? j : -1;
  }
  int sid = p.sorted_ids[br.base + j];
  if (sid < 0 || sid >= p.T * p.k) return -1;
  *slot = sid;
  return sid / p.k;
}

// One 256-wide K round of a 16-row weight tile against 16 token rows.
// w: this lane's weight row (null = zero row), b: this lane's token row (null =
// zero), k0 = round start + 64 * lane group.
__device__ __forceinline__ f32x4 round16(const uint16_t* w, const uint16_t* b, int k0, int K,
                                         f32x4 acc) {
  u32x4 wa[8], xb[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    int kc = k0 + 8 * q;
    wa[q] = (w && kc < K) ? *(const u32x4*)(w + kc) : u32x4{0u, 0u, 0u, 0u};
    xb[q] = (b && kc < K) ? *(const u32x4*)(b + kc) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) acc = mfma16(wa[q], xb[q], acc);
  return acc;
}

__device__ __forceinline__ void round16x2(const uint16_t* w0, const uint16_t* w1,
                                          const uint16_t* b, int k0, int K, f32x4& a0,
                                          f32x4& a1) {
  u32x4 wa[8], wb[8], xb[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    int kc = k0 + 8 * q;
    wa[q] = (w0 && kc < K) ? *(const u32x4*)(w0 + kc) : u32x4{0u, 0u, 0u, 0u};
    wb[q] = (w1 && kc < K) ? *(const u32x4*)(w1 + kc) : u32x4{0u, 0u, 0u, 0u};
    xb[q] = (b && kc < K) ? *(const u32x4*)(b + kc) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    a0 = mfma16(wa[q], xb[q], a0);
    a1 = mfma16(wb[q], xb[q], a1);
  }
}

// GEMV1: act[row j of block b][c0 + 0..15] = act(x[token j] . w13[e] rows).
// Grid (ceil(I/16), nblk + shared); 4 waves split K; also zeroes `out`.
template <bool SW>
__global__ void __launch_bounds__(256) gemv1_kernel(GemvParams p) {
  __shared__ f32x4 s_red[4][2][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // zero the output that GEMV2 accumulates into
  {
    const int64_t n4 = (int64_t)p.T * p.H / 4;
    const int64_t nwg = (int64_t)gridDim.x * gridDim.y;
    const int64_t wg = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    for (int64_t i = wg * 256 + tid; i < n4; i += nwg * 256)
      ((float4*)p.out)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  const int b = blockIdx.y;
  BlockRows br;
  br.shared = b == p.nblk;
  br.base = b * p.bm;
  const uint16_t* W;
  if (br.shared) {
    W = p.sw13;
  } else {
    if (br.base >= *p.ntpp) return;
    int e = p.expert_ids[b];
    if (e < 0 || e >= p.E) return;
    W = p.w13 + (int64_t)e * (SW ? 2 * p.I : p.I) * p.H;
  }
  const int c0 = blockIdx.x * 16;
  const int r = lane & 15;   // weight row in the tile / token column
  const int g = lane >> 4;   // lane group along K
  int slot;
  const int tok = block_token(p, br, r, &slot);
  const uint16_t* xrow = tok >= 0 ? p.x + (int64_t)tok * p.H : nullptr;
  const bool rowok = c0 + r < p.I;
  const uint16_t* wg_row = rowok ? W + (int64_t)(c0 + r) * p.H : nullptr;
  const uint16_t* wu_row = (SW && rowok) ? W + (int64_t)(p.I + c0 + r) * p.H : nullptr;

  f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
  const int rounds = (p.H + kRound - 1) / kRound;
  for (int rd = wave; rd < rounds; rd += 4) {
    const int k0 = rd * kRound + 64 * g;
    if (SW)
      round16x2(wg_row, wu_row, xrow, k0, p.H, ag, au);
    else
      ag = round16(wg_row, xrow, k0, p.H, ag);
  }
  s_red[wave][0][lane] = ag;
  if (SW) s_red[wave][1][lane] = au;
  __syncthreads();
  if (wave != 0) return;
  f32x4 hg = s_red[0][0][lane], hu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 1; w < 4; ++w) hg += s_red[w][0][lane];
  if (SW) {
    hu = s_red[0][1][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) hu += s_red[w][1][lane];
  }
  // lane holds rows (act cols) c0 + 4g + v of token column j = lane & 15
  const int j = lane & 15;
  int slot_j;
  const int tok_j = block_token(p, br, j, &slot_j);
  if (tok_j < 0) return;
  const int col = c0 + 4 * g;
  if (col >= p.I) return;
  float o[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    if (SW) {
      o[v] = silu(hg[v]) * hu[v];
    } else {
      float t = fmaxf(hg[v], 0.f);
      o[v] = t * t;
    }
  }
  uint16_t* dst = br.shared ? p.act_sh + (int64_t)j * p.I : p.act + (int64_t)(br.base + j) * p.I;
  uint2 pk;
  pk.x = (unsigned)f32_to_bf16(o[0]) | ((unsigned)f32_to_bf16(o[1]) << 16);
  pk.y = (unsigned)f32_to_bf16(o[2]) | ((unsigned)f32_to_bf16(o[3]) << 16);
  *(uint2*)(dst + col) = pk;
}

// GEMV2: out[token j][h] += w_slot * (act[row j] . w2[e][h]) for 16 rows h per
// wave.  Grid (ceil(H/64), nblk + shared).
__global__ void __launch_bounds__(256) gemv2_kernel(GemvParams p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.y;
  BlockRows br;
  br.shared = b == p.nblk;
  br.base = b * p.bm;
  const uint16_t* W;
  if (br.shared) {
    W = p.sw2;
  } else {
    if (br.base >= *p.ntpp) return;
    int e = p.expert_ids[b];
    if (e < 0 || e >= p.E) return;
    W = p.w2 + (int64_t)e * p.H * p.I;
  }
  const int h0 = (blockIdx.x * 4 + wave) * 16;
  if (h0 >= p.H) return;
  const int r = lane & 15;
  const int g = lane >> 4;
  int slot;
  const int tok = block_token(p, br, r, &slot);
  const uint16_t* arow = nullptr;
  if (tok >= 0)
    arow = br.shared ? p.act_sh + (int64_t)r * p.I : p.act + (int64_t)(br.base + r) * p.I;
  const uint16_t* wrow = h0 + r < p.H ? W + (int64_t)(h0 + r) * p.I : nullptr;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int rounds = (p.I + kRound - 1) / kRound;
  for (int rd = 0; rd < rounds; ++rd) acc = round16(wrow, arow, rd * kRound + 64 * g, p.I, acc);
  // lane holds rows h0 + 4g + v of token column j = lane & 15
  const int j = lane & 15;
  int slot_j;
  const int tok_j = block_token(p, br, j, &slot_j);
  if (tok_j < 0) return;
  const float wgt = br.shared ? 1.f : p.topk_w[slot_j];
  float* dst = p.out + (int64_t)tok_j * p.H + h0 + 4 * g;
#pragma unroll
  for (int v = 0; v < 4; ++v)
    if (h0 + 4 * g + v < p.H) unsafeAtomicAdd(dst + v, wgt * acc[v]);
}

}  // namespace

hipError_t launch_gemv(const GemvParams& p, bool swiglu, hipStream_t s) {
  const unsigned nb = (unsigned)(p.nblk + (p.sw13 ? 1 : 0));
  if (nb == 0) return hipSuccess;
  dim3 g1((p.I + 15) / 16, nb);
  if (swiglu)
    hipLaunchKernelGGL(gemv1_kernel<true>, g1, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(gemv1_kernel<false>, g1, dim3(256), 0, s, p);
  dim3 g2((p.H + 63) / 64, nb);
  hipLaunchKernelGGL(gemv2_kernel, g2, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
