// Routing kernels: top-k gating and the sort-and-pad ("align") pass.
//
// Gating follows the skill card "Fused Moe Kernel", *Token-Expert Routing*
// step 1, with the DeepSeek-V3 grouped variant (n_group / topk_group of the
// axolotl DeepSeek-V3 benchmark config).  Align is steps 2-3 of the same
// section: slots grouped by expert, each expert padded to a multiple of
// BLOCK_M, pads marked with a value >= num_valid (*Common Pitfalls* 2).
//
// gfx950 design: one wave64 per token for gating (logits of up to 256 experts
// live in four registers per lane; k rounds of a butterfly arg-max).  Align
// ranks slots inside a wave with ballots (the lanes holding the same expert
// are found by AND-ing one ballot per bit of the expert id), combines waves
// with a per-expert prefix in LDS, and is stable: slots of one expert keep
// ascending order.
#include <hip/hip_runtime.h>
#include <limits.h>

#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kWave = 64;

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  // key order: larger logit first, lower expert index on ties; ib == INT_MAX is "none"
  if (ib == INT_MAX) return ia != INT_MAX;
  if (ia == INT_MAX) return false;
  return va > vb || (va == vb && ia < ib);
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ double sigmoid64(double l) { return 1.0 / (1.0 + exp(-l)); }

// Gating of token t by the calling wave.  `s_sig` is per-wave LDS scratch of
// MOE_MAX_EXPERTS doubles, `s_keep` per-wave scratch of 64 ints (group flags).
// Returns through lane j < k: *out_id, *out_w.
__device__ void gate_token(const GateParams& p, int t, double* s_sig, int* s_keep,
                           int* out_id, float* out_w) {
  const int lane = threadIdx.x & (kWave - 1);
  const float* row = p.logits + (int64_t)t * p.E;
  float v[4];
  bool avail[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = lane + kWave * i;
    avail[i] = e < p.E;
    v[i] = avail[i] ? row[e] : 0.f;
  }

  if (p.n_group > 1) {
    // group restriction: groups of gsize contiguous experts ranked by the sum
    // of their two largest fp64 sigmoids; keep the best topk_group groups
    const int gsize = p.E / p.n_group;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (avail[i]) s_sig[lane + kWave * i] = sigmoid64((double)v[i]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    double score = -1.0;
    if (lane < p.n_group) {
      double b1 = -1.0, b2 = -1.0;
      for (int q = 0; q < gsize; ++q) {
        double s = s_sig[lane * gsize + q];
        if (s > b1) { b2 = b1; b1 = s; }
        else if (s > b2) { b2 = s; }
      }
      score = b1 + (gsize > 1 ? b2 : 0.0);
    }
    // rank of my group: groups with a larger score, or an equal score and a lower index
    int rank = 0;
    for (int g = 0; g < p.n_group; ++g) {
      double o = __shfl(score, g, kWave);
      rank += (o > score || (o == score && g < lane)) ? 1 : 0;
    }
    if (lane < p.n_group) s_keep[lane] = rank < p.topk_group ? 1 : 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (avail[i]) avail[i] = s_keep[(lane + kWave * i) / gsize] != 0;
  }

  // softmax without renormalisation needs the full denominator
  double full_den = 0.0;
  double vmax_all = 0.0;

  int my_id = INT_MAX;
  float my_v = 0.f;
  float first_v = 0.f;
  for (int j = 0; j < p.k; ++j) {
    float bv = 0.f;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = lane + kWave * i;
      if (avail[i] && better(v[i], e, bv, bi)) { bv = v[i]; bi = e; }
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
      float ov = __shfl_xor(bv, off, kWave);
      int oi = __shfl_xor(bi, off, kWave);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (j == 0) first_v = bv;
    if (lane == j) { my_id = bi; my_v = bv; }
    if (bi != INT_MAX && (bi & (kWave - 1)) == lane) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (bi == lane + kWave * i) avail[i] = false;
    }
  }

  double wj;
  if (p.scoring == 0) {
    if (p.renorm) {
      double ex = lane < p.k ? exp((double)my_v - (double)first_v) : 0.0;
      wj = ex / wave_sum(ex);
    } else {
      // max over all experts: the first selection when nothing is masked
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + kWave * i < p.E) m = fmaxf(m, v[i]);
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
      vmax_all = (double)m;
      double part = 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + kWave * i < p.E) part += exp((double)v[i] - vmax_all);
      full_den = wave_sum(part);
      wj = exp((double)my_v - vmax_all) / full_den;
    }
  } else {
    double sg = lane < p.k ? sigmoid64((double)my_v) : 0.0;
    wj = p.renorm ? sg / wave_sum(sg) : sg;
  }
  *out_id = my_id;
  *out_w = (float)(wj * (double)p.scale);
}

// ------------------------------------------------------------------ align helpers
// Exclusive scan of the padded expert sizes by wave 0 of the block.  Fills
// s_off[e] (start) and returns nothing; s_cnt holds the counts.  Then writes
// expert_ids, the pads and num_tokens_post_padded.
__device__ void align_layout(const int* s_cnt, int* s_off, int* s_cursor, int E, int bm, int n,
                             int* sorted_ids, int* expert_ids, int* ntpp, int* s_total) {
  const int tid = threadIdx.x;
  if (tid < kWave) {
    // each lane owns 4 consecutive experts
    int base = tid * 4;
    int pc[4];
    int local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = base + i;
      int c = e < E ? s_cnt[e] : 0;
      pc[i] = (c + bm - 1) / bm * bm;
      local += pc[i];
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      int o = __shfl_up(incl, off, kWave);
      if (tid >= off) incl += o;
    }
    int run = incl - local;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = base + i;
      if (e < E) { s_off[e] = run; s_cursor[e] = run; }
      run += pc[i];
    }
    if (tid == kWave - 1) {
      *s_total = incl;
      *ntpp = incl;
    }
  }
  __syncthreads();
  const int total = *s_total;
  // expert of every block: the last expert whose offset is <= block start
  for (int b = tid; b * bm < total; b += blockDim.x) {
    int pos = b * bm;
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= pos) lo = mid; else hi = mid - 1;
    }
    // skip empty experts that share the offset: take the first non-empty one at pos
    // (an empty expert has the same offset as the next one; the binary search
    // returned the last e with off <= pos, which is non-empty because pos < total)
    expert_ids[b] = lo;
  }
  // pads of each expert
  for (int e = tid; e < E; e += blockDim.x) {
    int c = s_cnt[e];
    int pcount = (c + bm - 1) / bm * bm;
    for (int r = c; r < pcount; ++r) sorted_ids[s_off[e] + r] = n;
  }
}

// Stable scatter of `cnt` slots starting at `slot0`, whose experts are read by
// `get_id(i)` (i in [0, cnt)).  s_cursor[e] holds the next write position of
// expert e and is advanced.  s_wcnt is LDS scratch [2][16][MOE_MAX_EXPERTS].
template <typename GetId>
__device__ void stable_scatter(GetId get_id, int slot0, int cnt, int E, int* s_cursor,
                               int* s_wcnt, int* sorted_ids) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int nwaves = blockDim.x / kWave;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  // clear both buffers
  for (int i = tid; i < 2 * 16 * 256; i += blockDim.x) s_wcnt[i] = 0;
  __syncthreads();
  int it = 0;
  for (int base = 0; base < cnt; base += blockDim.x, ++it) {
    int* buf = s_wcnt + (it & 1) * (16 * 256);
    int* other = s_wcnt + ((it + 1) & 1) * (16 * 256);
    int i = base + tid;
    int e = -1;
    if (i < cnt) {
      e = get_id(i);
      if (e < 0 || e >= E) e = -1;
    }
    uint64_t match = __ballot(e >= 0);
    for (int b = 0; b < nbits; ++b) {
      uint64_t bal = __ballot(e >= 0 && ((e >> b) & 1));
      match &= ((e >> b) & 1) ? bal : ~bal;
    }
    int rank = __popcll(match & lt_mask);
    if (e >= 0 && rank == 0) buf[wave * 256 + e] = __popcll(match);
    __syncthreads();
    // per-expert exclusive prefix over the waves, plus the running cursor
    for (int x = tid; x < E; x += blockDim.x) {
      int run = s_cursor[x];
      for (int w = 0; w < nwaves; ++w) {
        int c = buf[w * 256 + x];
        buf[w * 256 + x] = run;
        run += c;
        other[w * 256 + x] = 0;
      }
      s_cursor[x] = run;
    }
    __syncthreads();
    if (e >= 0) sorted_ids[buf[wave * 256 + e] + rank] = slot0 + i;
  }
}

// ------------------------------------------------------------------ kernels
__global__ void __launch_bounds__(256) gate_kernel(GateParams p) {
  __shared__ double s_sig[4][256];
  __shared__ int s_keep[4][64];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * 4 + wave;
  if (t >= p.T) return;  // uniform per wave; gate_token synchronises only within the wave
  int id;
  float w;
  gate_token(p, t, s_sig[wave], s_keep[wave], &id, &w);
  if (lane < p.k) {
    p.topk_ids[(int64_t)t * p.k + lane] = id;
    p.topk_w[(int64_t)t * p.k + lane] = w;
  }
}

// One workgroup: all n <= kSingleBlockSlots slots.  When `g` is given, gating
// runs first inside the same workgroup (one wave per token).
__global__ void __launch_bounds__(1024) align_single_kernel(AlignParams a, GateParams g,
                                                            int do_gate) {
  __shared__ int s_ids[kSingleBlockSlots];
  __shared__ int s_cnt[256], s_off[256], s_cursor[256];
  __shared__ int s_wcnt[2 * 16 * 256];
  __shared__ int s_total;
  __shared__ double s_sig[16][256];
  __shared__ int s_keep[16][64];
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);

  if (do_gate) {
    for (int t = wave; t < g.T; t += 16) {
      int id;
      float w;
      gate_token(g, t, s_sig[wave], s_keep[wave], &id, &w);
      if (lane < g.k) {
        g.topk_ids[t * g.k + lane] = id;
        g.topk_w[t * g.k + lane] = w;
        s_ids[t * g.k + lane] = id;
      }
    }
  } else {
    for (int i = tid; i < a.n; i += blockDim.x) s_ids[i] = a.topk_ids[i];
  }
  for (int e = tid; e < 256; e += blockDim.x) s_cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < a.n; i += blockDim.x) {
    int e = s_ids[i];
    if (e >= 0 && e < a.E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  align_layout(s_cnt, s_off, s_cursor, a.E, a.block_m, a.n, a.sorted_ids, a.expert_ids, a.ntpp,
               &s_total);
  __syncthreads();
  stable_scatter([&](int i) { return s_ids[i]; }, 0, a.n, a.E, s_cursor, s_wcnt, a.sorted_ids);
}

// Multi-block path, step 1: per-chunk expert histogram.
__global__ void __launch_bounds__(1024) align_count_kernel(AlignParams a) {
  __shared__ int s_cnt[256];
  const int tid = threadIdx.x;
  for (int e = tid; e < 256; e += blockDim.x) s_cnt[e] = 0;
  __syncthreads();
  const int s0 = blockIdx.x * kAlignChunk;
  const int s1 = min(a.n, s0 + kAlignChunk);
  for (int s = s0 + tid; s < s1; s += blockDim.x) {
    int e = a.topk_ids[s];
    if (e >= 0 && e < a.E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += blockDim.x) a.block_counts[blockIdx.x * a.E + e] = s_cnt[e];
}

// Step 2: one workgroup turns chunk histograms into per-chunk bases, pads the
// experts and writes expert_ids and the padded total.
__global__ void __launch_bounds__(1024) align_scan_kernel(AlignParams a) {
  __shared__ int s_cnt[256], s_off[256], s_cursor[256];
  __shared__ int s_total;
  const int tid = threadIdx.x;
  for (int e = tid; e < a.E; e += blockDim.x) {
    int run = 0;
    for (int b = 0; b < a.nblocks; ++b) {
      int c = a.block_counts[b * a.E + e];
      a.block_counts[b * a.E + e] = run;
      run += c;
    }
    s_cnt[e] = run;
  }
  __syncthreads();
  align_layout(s_cnt, s_off, s_cursor, a.E, a.block_m, a.n, a.sorted_ids, a.expert_ids, a.ntpp,
               &s_total);
  for (int e = tid; e < a.E; e += blockDim.x) a.expert_off[e] = s_off[e];
}

// Step 3: each chunk scatters its slots at expert offset + chunk base.
__global__ void __launch_bounds__(1024) align_scatter_kernel(AlignParams a) {
  __shared__ int s_cursor[256];
  __shared__ int s_wcnt[2 * 16 * 256];
  const int tid = threadIdx.x;
  for (int e = tid; e < a.E; e += blockDim.x)
    s_cursor[e] = a.expert_off[e] + a.block_counts[blockIdx.x * a.E + e];
  __syncthreads();
  const int s0 = blockIdx.x * kAlignChunk;
  const int cnt = min(a.n, s0 + kAlignChunk) - s0;
  const int* ids = a.topk_ids + s0;
  stable_scatter([&](int i) { return ids[i]; }, s0, cnt, a.E, s_cursor, s_wcnt, a.sorted_ids);
}

}  // namespace

hipError_t launch_gate(const GateParams& p, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  dim3 grid((p.T + 3) / 4);
  hipLaunchKernelGGL(gate_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_route_fused(const GateParams& g, const AlignParams& a, hipStream_t s) {
  hipLaunchKernelGGL(align_single_kernel, dim3(1), dim3(1024), 0, s, a, g, 1);
  return hipGetLastError();
}

hipError_t launch_align(const AlignParams& p, hipStream_t s) {
  if (p.n <= kSingleBlockSlots) {
    GateParams none{};
    hipLaunchKernelGGL(align_single_kernel, dim3(1), dim3(1024), 0, s, p, none, 0);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(align_count_kernel, dim3(p.nblocks), dim3(1024), 0, s, p);
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(1024), 0, s, p);
  hipLaunchKernelGGL(align_scatter_kernel, dim3(p.nblocks), dim3(1024), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
