// Grouped GEMM over the aligned (sorted + padded) token layout, bf16 MFMA on
// gfx950, with fused epilogues.
//
// The structure is the one of the skill card "Fused Moe Kernel", *Grouped
// GEMM Structure*: a tiled GEMM whose M-blocks reach their token rows through
// sorted_token_ids (token = id / top_k, *Common Pitfalls* 1), whose weight
// matrix is chosen per M-block by expert_ids (weights stacked [E, N, K],
// *Common Pitfalls* 3), and whose blocks at or beyond num_tokens_post_padded
// exit at once.  Epilogues: SwiGLU act_fn(gate) * up (axolotl DeepSeek-V3 MoE
// forward), squared ReLU (mlxcel fc1 -> relu^2), plain store, and the routed
// weight times the row scattered to its slot (*Common Pitfalls* 4).
//
// gfx950 mapping.  One workgroup = 4 wave64s computes a BM x BNW tile of
// C^T = W_e . X^T: the weight rows play the MFMA "A" role and the gathered
// token rows the "B" role, so each lane ends up owning 4 consecutive output
// features of one token row and stores them as one 8- or 16-byte write.
// Operands are staged global -> registers -> LDS (double buffered, one barrier
// per 64-wide K step).  LDS rows are 128 bytes with the 16-byte chunk index
// XOR-swizzled by the row so that the MFMA operand reads spread over banks.
// v_mfma_f32_32x32x16_bf16 is used when a wave owns >= 32 token rows,
// v_mfma_f32_16x16x32_bf16 for BLOCK_M = 16.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 64;

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

template <int MT>
struct Mfma;

template <>
struct Mfma<32> {
  typedef f32x16 acc_t;
  static constexpr int kSteps = BK / 16;  // k per instruction: 16
  static constexpr int kVals = 16;
  __device__ static __forceinline__ acc_t run(bf16x8 a, bf16x8 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // operand chunk (16-byte unit along K) and row read by a lane at k-step kk
  __device__ static __forceinline__ int chunk(int kk, int lane) { return 2 * kk + (lane >> 5); }
  __device__ static __forceinline__ int row(int lane) { return lane & 31; }
  // output: column (token) and the first of 4 consecutive rows (features) of group g
  __device__ static __forceinline__ int out_col(int lane) { return lane & 31; }
  __device__ static __forceinline__ int out_row(int g, int lane) { return 8 * g + 4 * (lane >> 5); }
  static constexpr int kGroups = 4;
};

template <>
struct Mfma<16> {
  typedef f32x4 acc_t;
  static constexpr int kSteps = BK / 32;  // k per instruction: 32
  static constexpr int kVals = 4;
  __device__ static __forceinline__ acc_t run(bf16x8 a, bf16x8 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ int chunk(int kk, int lane) { return 4 * kk + (lane >> 4); }
  __device__ static __forceinline__ int row(int lane) { return lane & 15; }
  __device__ static __forceinline__ int out_col(int lane) { return lane & 15; }
  __device__ static __forceinline__ int out_row(int g, int lane) { return 4 * (lane >> 4); }
  static constexpr int kGroups = 1;
};

__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ (r & 7)); }

// BM token rows x BNW weight rows per workgroup tile; WAVES_M x WAVES_N waves.
// SW: the tile's first BNW/2 weight rows are gate rows n0.., the rest the up
// rows I+n0.. of the same act columns, and the epilogue is SwiGLU.
template <int BM, int BNW, int WAVES_M, int WAVES_N, bool SW>
__global__ void __launch_bounds__(256) grouped_gemm_kernel(GemmParams p) {
  constexpr int WM = BM / WAVES_M;
  constexpr int MT = WM >= 32 ? 32 : 16;
  typedef Mfma<MT> M;
  constexpr int WNW = BNW / WAVES_N;
  constexpr int FM = WM / MT;
  constexpr int FN = WNW / MT;
  constexpr int XL = (BM * 8 + 255) / 256;
  constexpr int WL = BNW * 8 / 256;
  static_assert(WAVES_M * WAVES_N == 4, "4 waves");
  static_assert(!SW || FN % 2 == 0, "SwiGLU pairs gate and up subtiles");
  static_assert(BNW * 8 % 256 == 0, "weight tile load");

  __shared__ u32x4 sX[2][BM * 8];
  __shared__ u32x4 sW[2][BNW * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave % WAVES_N;
  const int wm = wave / WAVES_N;

  const int mb = blockIdx.y;
  const int m0 = mb * BM;
  const int total_rows = p.ntpp ? *p.ntpp : p.M;
  if (m0 >= total_rows) return;
  const int e = p.expert_ids ? p.expert_ids[mb] : 0;
  if (e < 0 || e >= p.E) return;
  const uint16_t* We = p.W + (int64_t)e * p.N * p.K;
  const int ncols = SW ? p.I : p.N;           // output columns
  const int n0 = blockIdx.x * (SW ? BNW / 2 : BNW);

  // ---- per-thread global source rows (null = zero row)
  const uint16_t* xsrc[XL];
  int xch[XL], xrow[XL];
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    int idx = tid + 256 * j;
    xrow[j] = idx >> 3;
    xch[j] = idx & 7;
    xsrc[j] = nullptr;
    if (idx < BM * 8) {
      int i = m0 + xrow[j];
      if (p.sorted_ids) {
        int sid = p.sorted_ids[i];
        if (sid >= 0 && sid < p.num_valid) {
          int arow = p.a_row_div ? sid / p.a_row_div : i;
          xsrc[j] = p.A + (int64_t)arow * p.K;
        }
      } else if (i < p.M) {
        xsrc[j] = p.A + (int64_t)i * p.K;
      }
    }
  }
  const uint16_t* wsrc[WL];
  int wch[WL], wrow[WL];
#pragma unroll
  for (int j = 0; j < WL; ++j) {
    int idx = tid + 256 * j;
    int r = idx >> 3;
    wrow[j] = r;
    wch[j] = idx & 7;
    int g;
    bool ok;
    if (SW) {
      int c = r < BNW / 2 ? n0 + r : n0 + r - BNW / 2;
      ok = c < p.I;
      g = r < BNW / 2 ? c : p.I + c;
    } else {
      g = n0 + r;
      ok = g < p.N;
    }
    wsrc[j] = ok ? We + (int64_t)g * p.K : nullptr;
  }

  typename M::acc_t acc[FN][FM];
#pragma unroll
  for (int f = 0; f < FN; ++f)
#pragma unroll
    for (int q = 0; q < FM; ++q)
#pragma unroll
      for (int v = 0; v < M::kVals; ++v) acc[f][q][v] = 0.f;

  u32x4 xr[XL], wr[WL];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int j = 0; j < XL; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      int kc = k0 + xch[j] * 8;
      if (xsrc[j] && kc < p.K) v = *(const u32x4*)(xsrc[j] + kc);
      xr[j] = v;
    }
#pragma unroll
    for (int j = 0; j < WL; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      int kc = k0 + wch[j] * 8;
      if (wsrc[j] && kc < p.K) v = *(const u32x4*)(wsrc[j] + kc);
      wr[j] = v;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < XL; ++j)
      if (tid + 256 * j < BM * 8) sX[buf][swz(xrow[j], xch[j])] = xr[j];
#pragma unroll
    for (int j = 0; j < WL; ++j) sW[buf][swz(wrow[j], wch[j])] = wr[j];
  };
  // local weight row of subtile f of this wave
  auto wsub = [&](int f) {
    if (SW) {
      constexpr int WNA = BNW / 2 / WAVES_N;
      return f < FN / 2 ? wn * WNA + f * MT : BNW / 2 + wn * WNA + (f - FN / 2) * MT;
    }
    return wn * WNW + f * MT;
  };

  const int nk = (p.K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < M::kSteps; ++kk) {
      const int c = M::chunk(kk, lane);
      bf16x8 bx[FM];
#pragma unroll
      for (int q = 0; q < FM; ++q) {
        int r = wm * WM + q * MT + M::row(lane);
        u32x4 t = sX[buf][swz(r, c)];
        bx[q] = __builtin_bit_cast(bf16x8, t);
      }
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        int r = wsub(f) + M::row(lane);
        u32x4 t = sW[buf][swz(r, c)];
        bf16x8 aw = __builtin_bit_cast(bf16x8, t);
#pragma unroll
        for (int q = 0; q < FM; ++q) acc[f][q] = M::run(aw, bx[q], acc[f][q]);
      }
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  const int epi = p.epi;
#pragma unroll
  for (int q = 0; q < FM; ++q) {
    const int mloc = wm * WM + q * MT + M::out_col(lane);
    const int i = m0 + mloc;
    int64_t orow;
    float scale = 1.f;
    bool ok;
    if (epi == 3) {
      int sid;
      if (p.sorted_ids) {
        sid = p.sorted_ids[i];
        ok = sid >= 0 && sid < p.num_valid;
      } else {
        sid = i;
        ok = i < p.M;
      }
      if (ok && p.topk_w) scale = p.topk_w[sid];
      orow = p.c_row_offset + sid;
    } else {
      ok = p.sorted_ids ? true : i < p.M;
      orow = i;
    }
    if (!ok) continue;
    constexpr int FO = SW ? FN / 2 : FN;
#pragma unroll
    for (int f = 0; f < FO; ++f) {
      const int colbase = SW ? n0 + wn * (BNW / 2 / WAVES_N) + f * MT : n0 + wn * WNW + f * MT;
#pragma unroll
      for (int g = 0; g < M::kGroups; ++g) {
        const int col = colbase + M::out_row(g, lane);
        if (col >= ncols) continue;
        float o[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float h = acc[f][q][4 * g + v];
          if (SW) {
            float u = acc[f + FN / 2][q][4 * g + v];
            o[v] = silu(h) * u;
          } else if (epi == 2) {
            float r = fmaxf(h, 0.f);
            o[v] = r * r;
          } else {
            o[v] = h * scale;
          }
        }
        if (p.c_fp32) {
          float4* dst = (float4*)((float*)p.C + orow * p.ldc + col);
          *dst = make_float4(o[0], o[1], o[2], o[3]);
        } else {
          uint2 pk;
          pk.x = (unsigned)f32_to_bf16(o[0]) | ((unsigned)f32_to_bf16(o[1]) << 16);
          pk.y = (unsigned)f32_to_bf16(o[2]) | ((unsigned)f32_to_bf16(o[3]) << 16);
          *(uint2*)((uint16_t*)p.C + orow * p.ldc + col) = pk;
        }
      }
    }
  }
}

template <int BM, int BNW, int WAVES_M, int WAVES_N>
hipError_t launch_bm(const GemmParams& p, hipStream_t s) {
  const bool sw = p.epi == 1;
  const int ncols = sw ? p.I : p.N;
  const int tile_n = sw ? BNW / 2 : BNW;
  const int mblocks = (p.M + BM - 1) / BM;
  dim3 grid((ncols + tile_n - 1) / tile_n, mblocks);
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  if (sw)
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BNW, WAVES_M, WAVES_N, true>), grid, dim3(256), 0,
                       s, p);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BNW, WAVES_M, WAVES_N, false>), grid, dim3(256),
                       0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmParams& p, int block_m, hipStream_t s) {
  switch (block_m) {
    case 128: return launch_bm<128, 256, 2, 2>(p, s);
    case 64: return launch_bm<64, 256, 1, 4>(p, s);
    case 32: return launch_bm<32, 256, 1, 4>(p, s);
    case 16: return launch_bm<16, 128, 1, 4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// out[t] = sum_j yslot[t*k + j] (+ yslot[T*k + t] for the shared expert), in j order.
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ yslot, int T, int k,
                                                      int H, int has_shared, float* __restrict__ out) {
  const int h4 = H / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * h4) return;
  const int t = (int)(idx / h4);
  const int c = (int)(idx % h4) * 4;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    float4 y = *(const float4*)(yslot + ((int64_t)t * k + j) * H + c);
    a.x += y.x; a.y += y.y; a.z += y.z; a.w += y.w;
  }
  if (has_shared) {
    float4 y = *(const float4*)(yslot + ((int64_t)T * k + t) * H + c);
    a.x += y.x; a.y += y.y; a.z += y.z; a.w += y.w;
  }
  *(float4*)(out + (int64_t)t * H + c) = a;
}

hipError_t launch_combine(const float* yslot, int T, int k, int H, int has_shared, float* out,
                          hipStream_t s) {
  int64_t n = (int64_t)T * (H / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, yslot, T, k,
                     H, has_shared, out);
  return hipGetLastError();
}

}  // namespace moe
