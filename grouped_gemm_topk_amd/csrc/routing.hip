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
// Padded exclusive scan of the expert counts by wave 0 (four experts per
// lane): s_off[e] = start of expert e in the padded order, *s_total = padded
// length.  The caller synchronises before reading them.
__device__ void align_offsets(const int* s_cnt, int* s_off, int E, int bm, int* s_total) {
  const int tid = threadIdx.x;
  if (tid >= kWave) return;
  const int base = tid * 4;
  int pc[4];
  int local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = base + i;
    const int c = e < E ? s_cnt[e] : 0;
    pc[i] = (c + bm - 1) / bm * bm;   // an empty expert takes no block
    local += pc[i];
  }
  int incl = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (tid >= off) incl += o;
  }
  int run = incl - local;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = base + i;
    if (e < E) s_off[e] = run;
    run += pc[i];
  }
  if (tid == kWave - 1) *s_total = incl;
}

// expert_ids of every block, the pad entries of sorted_ids (value n) and the
// padded total, all threads of the workgroup in parallel.
__device__ void write_layout(const int* s_cnt, const int* s_off, int E, int bm, int n, int total,
                             int* sorted_ids, int* expert_ids, int* ntpp) {
  const int tid = threadIdx.x;
  if (tid == 0) *ntpp = total;
  // expert of a block: the last expert whose offset is <= the block start (an
  // empty expert shares its offset with the next one, so the last such expert
  // is the non-empty one that owns the block)
  for (int b = tid; b * bm < total; b += blockDim.x) {
    const int pos = b * bm;
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= pos) lo = mid; else hi = mid - 1;
    }
    expert_ids[b] = lo;
  }
  // pads: expert e owns padded positions [off + c, off + round_up(c, bm))
  for (int idx = tid; idx < E * bm; idx += blockDim.x) {
    const int e = idx / bm, r = idx - e * bm;
    const int c = s_cnt[e];
    const int pc = (c + bm - 1) / bm * bm;
    if (c + r < pc) sorted_ids[s_off[e] + c + r] = n;
  }
}

// Lanes of this wave whose expert equals e (one ballot per bit of the id);
// lanes with e < 0 are excluded.
__device__ __forceinline__ uint64_t same_expert(int e, int nbits) {
  uint64_t match = __ballot(e >= 0);
  for (int b = 0; b < nbits; ++b) {
    const uint64_t bal = __ballot(e >= 0 && ((e >> b) & 1));
    match &= ((e >> b) & 1) ? bal : ~bal;
  }
  return e >= 0 ? match : 0ull;
}

__device__ __forceinline__ int id_bits(int E) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  return nbits;
}

// Stable scatter of `cnt` slots starting at `slot0`, whose experts are read by
// `get_id(i)` (i in [0, cnt)), by a 1024-thread workgroup.  s_cursor[e] holds
// the next write position of expert e and is advanced.  LDS scratch: s_wcnt
// and s_base, [16 waves][256 experts] each; s_wcnt must be zero on entry and
// is left zero.
template <typename GetId>
__device__ void stable_scatter(GetId get_id, int slot0, int cnt, int E, int* s_cursor,
                               int* s_wcnt, int* s_base, int* sorted_ids) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int nbits = id_bits(E);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int base = 0; base < cnt; base += 1024) {
    const int i = base + tid;
    int e = -1;
    if (i < cnt) {
      e = get_id(i);
      if (e < 0 || e >= E) e = -1;
    }
    const uint64_t match = same_expert(e, nbits);
    const int rank = __popcll(match & lt_mask);
    if (e >= 0 && rank == 0) s_wcnt[wave * 256 + e] = __popcll(match);
    __syncthreads();
    // per expert: exclusive prefix over the 16 waves (16 lanes per expert, a
    // width-16 shuffle scan), plus the running cursor; counts are cleared
    for (int e0 = wave * 4; e0 < E; e0 += 64) {
      const int ee = e0 + (lane >> 4), ww = lane & 15;
      const int v = ee < E ? s_wcnt[ww * 256 + ee] : 0;
      int incl = v;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const int o = __shfl_up(incl, off, 16);
        if (ww >= off) incl += o;
      }
      if (ee < E) {
        const int cur = s_cursor[ee];
        s_base[ww * 256 + ee] = cur + incl - v;
        s_wcnt[ww * 256 + ee] = 0;
        if (ww == 15) s_cursor[ee] = cur + incl;
      }
    }
    __syncthreads();
    if (e >= 0) sorted_ids[s_base[wave * 256 + e] + rank] = slot0 + i;
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

// One workgroup: all n <= kSingleBlockSlots slots.  When `do_gate` is set,
// gating runs first inside the same workgroup (one wave per token).
__global__ void __launch_bounds__(1024) align_single_kernel(AlignParams a, GateParams g,
                                                            int do_gate) {
  __shared__ int s_ids[kSingleBlockSlots];
  __shared__ int s_cnt[256], s_off[256], s_cursor[256];
  __shared__ int s_wcnt[16 * 256], s_base[16 * 256];
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
  for (int i = tid; i < 16 * 256; i += blockDim.x) s_wcnt[i] = 0;
  __syncthreads();
  for (int i = tid; i < a.n; i += blockDim.x) {
    const int e = s_ids[i];
    if (e >= 0 && e < a.E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  align_offsets(s_cnt, s_off, a.E, a.block_m, &s_total);
  __syncthreads();
  write_layout(s_cnt, s_off, a.E, a.block_m, a.n, s_total, a.sorted_ids, a.expert_ids, a.ntpp);
  for (int e = tid; e < a.E; e += blockDim.x) s_cursor[e] = s_off[e];
  __syncthreads();
  stable_scatter([&](int i) { return s_ids[i]; }, 0, a.n, a.E, s_cursor, s_wcnt, s_base,
                 a.sorted_ids);
}

// Two-kernel path, step 1: expert histogram of each chunk of a.chunk slots
// (one leader per expert and wave adds the wave's count).
__global__ void __launch_bounds__(1024) align_count_kernel(AlignParams a) {
  __shared__ int s_cnt[256];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int nbits = id_bits(a.E);
  for (int e = tid; e < 256; e += blockDim.x) s_cnt[e] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)blockIdx.x * a.chunk;
  const int64_t s1 = min((int64_t)a.n, s0 + a.chunk);
  for (int64_t base = s0; base < s1; base += 1024) {
    const int64_t s = base + tid;
    int e = s < s1 ? a.topk_ids[s] : -1;
    if (e >= a.E) e = -1;
    const uint64_t match = same_expert(e, nbits);
    if (e >= 0 && __popcll(match & lt_mask) == 0) atomicAdd(&s_cnt[e], __popcll(match));
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += blockDim.x) a.block_counts[blockIdx.x * a.E + e] = s_cnt[e];
}

// Step 2: every workgroup derives the expert offsets and its chunk's base per
// expert from all chunk histograms (a few KB from L2), workgroup 0 writes the
// layout (expert_ids, pads, padded total), and each workgroup scatters its
// chunk's slots stably.
__global__ void __launch_bounds__(1024) align_place_kernel(AlignParams a) {
  __shared__ int s_tot[4][256], s_pre[4][256];
  __shared__ int s_cnt[256], s_off[256], s_cursor[256];
  __shared__ int s_wcnt[16 * 256], s_base[16 * 256];
  __shared__ int s_total;
  const int tid = threadIdx.x;
  const int q = tid >> 8, e = tid & 255;
  for (int i = tid; i < 16 * 256; i += blockDim.x) s_wcnt[i] = 0;
  {
    int tot = 0, pre = 0;
    if (e < a.E) {
      for (int b = q; b < a.nblocks; b += 4) {
        const int c = a.block_counts[b * a.E + e];
        tot += c;
        if (b < (int)blockIdx.x) pre += c;
      }
    }
    s_tot[q][e] = tot;
    s_pre[q][e] = pre;
  }
  __syncthreads();
  if (tid < 256) {
    s_cnt[tid] = s_tot[0][tid] + s_tot[1][tid] + s_tot[2][tid] + s_tot[3][tid];
    s_pre[0][tid] += s_pre[1][tid] + s_pre[2][tid] + s_pre[3][tid];
  }
  __syncthreads();
  align_offsets(s_cnt, s_off, a.E, a.block_m, &s_total);
  __syncthreads();
  if (blockIdx.x == 0)
    write_layout(s_cnt, s_off, a.E, a.block_m, a.n, s_total, a.sorted_ids, a.expert_ids, a.ntpp);
  for (int x = tid; x < a.E; x += blockDim.x) s_cursor[x] = s_off[x] + s_pre[0][x];
  __syncthreads();
  const int64_t s0 = (int64_t)blockIdx.x * a.chunk;
  const int cnt = (int)(min((int64_t)a.n, s0 + a.chunk) - s0);
  const int* ids = a.topk_ids + s0;
  stable_scatter([&](int i) { return ids[i]; }, (int)s0, cnt, a.E, s_cursor, s_wcnt, s_base,
                 a.sorted_ids);
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
  hipLaunchKernelGGL(align_place_kernel, dim3(p.nblocks), dim3(1024), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
