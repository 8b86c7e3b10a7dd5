// Routing kernels: top-k gating and the sort-and-pad ("align") pass.
//
// Gating follows the skill card "Fused Moe Kernel", *Token-Expert Routing*
// step 1, with the DeepSeek-V3 grouped variant (n_group / topk_group of the
// axolotl DeepSeek-V3 benchmark config).  Align is steps 2-3 of the same
// section: slots grouped by expert, each expert padded to a multiple of
// BLOCK_M, pads marked with a value >= num_valid (*Common Pitfalls* 2).
//
// gfx950 design: one wave64 per token for gating (logits of up to 256 experts
// live in four registers per lane; the top-k is a two-level rank of 64-bit
// order keys through LDS).  Align
// ranks slots inside a wave with ballots (the lanes holding the same expert
// are found by AND-ing one ballot per bit of the expert id), combines waves
// with a per-expert prefix in LDS, and is stable: slots of one expert keep
// ascending order.
#include <hip/hip_runtime.h>
#include <limits.h>

#include "moe_internal.h"
#include "wave_topk.h"

namespace moe {

namespace {

constexpr int kWave = 64;

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ double sigmoid64(double l) { return 1.0 / (1.0 + exp(-l)); }

// Gating of token t by the calling wave.  `s_sig` is per-wave LDS scratch of
// MOE_MAX_EXPERTS doubles, `s_keep` per-wave scratch of 64 ints.  Returns
// through lane j < k: *out_id, *out_w.  Ranks and sums go through LDS (one
// broadcast read per value) rather than chains of cross-lane shuffles; the
// top-k is the two-level wave_topk.
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
    wave_sync_lds();
    double score = -1.0;
    if (lane < p.n_group) {
      double b1 = -1.0, b2 = -1.0;
      for (int q = 0; q < gsize; ++q) {
        double sg = s_sig[lane * gsize + q];
        if (sg > b1) { b2 = b1; b1 = sg; }
        else if (sg > b2) { b2 = sg; }
      }
      score = b1 + (gsize > 1 ? b2 : 0.0);
    }
    wave_sync_lds();   // every lane is done with the sigmoids
    if (lane < p.n_group) s_sig[lane] = score;
    wave_sync_lds();
    // rank of my group: groups with a larger score, or an equal score and a lower index
    int rank = 0;
    if (lane < p.n_group)
      for (int g = 0; g < p.n_group; ++g) {
        const double o = s_sig[g];
        rank += (o > score || (o == score && g < lane)) ? 1 : 0;
      }
    const uint64_t keep = __ballot(lane < p.n_group && rank < p.topk_group);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (avail[i]) avail[i] = (keep >> ((lane + kWave * i) / gsize)) & 1ull;
    wave_sync_lds();   // the group scores are read; s_sig is free
  }

  // the k largest keys (masked and absent experts have key 0); selection j's
  // expert and value go to LDS slot j
  int* s_id = s_keep;
  float* s_val = (float*)(s_keep + 16);
  uint64_t kown[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kown[i] = avail[i] ? order_key(v[i], lane + kWave * i) : 0ull;
  wave_topk_n((p.E + kWave - 1) / kWave, (uint64_t*)s_sig, kown, lane, p.k, [&](int i, int r) {
    s_id[r] = lane + kWave * i;
    s_val[r] = v[i];
  });
  wave_sync_lds();
  int my_id = INT_MAX;
  float my_v = 0.f;
  if (lane < p.k) {
    my_id = s_id[lane];
    my_v = s_val[lane];
  }
  const float first_v = s_val[0];

  // weights in fp64; the k terms of a renormalisation are added in selection
  // order
  double* s_term = s_sig;
  auto sum_k = [&](double term) {
    if (lane < p.k) s_term[lane] = term;
    wave_sync_lds();
    double den = 0.0;
    for (int j = 0; j < p.k; ++j) den += s_term[j];
    return den;
  };
  double wj;
  if (p.scoring == 0) {
    if (p.renorm) {
      const double ex = lane < p.k ? exp((double)my_v - (double)first_v) : 0.0;
      wj = ex / sum_k(ex);
    } else {
      // nothing is masked (grouping needs sigmoid scoring): the first
      // selection is the maximum over all experts
      const double vmax_all = (double)first_v;
      double part = 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + kWave * i < p.E) part += exp((double)v[i] - vmax_all);
      const double full_den = wave_sum(part);
      wj = exp((double)my_v - vmax_all) / full_den;
    }
  } else {
    const double sg = lane < p.k ? sigmoid64((double)my_v) : 0.0;
    wj = p.renorm ? sg / sum_k(sg) : sg;
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
// padded total.  Worker w of nw (a thread index over every workgroup that
// takes part) writes entries w, w + nw, ...; worker 0 writes the total.
__device__ void write_layout(const int* s_cnt, const int* s_off, int E, int bm, int n, int total,
                             int* sorted_ids, int* expert_ids, int* ntpp, int w, int nw) {
  const int tid = w;
  if (tid == 0) *ntpp = total;
  // expert of a block: the last expert whose offset is <= the block start (an
  // empty expert shares its offset with the next one, so the last such expert
  // is the non-empty one that owns the block)
  for (int b = tid; b * bm < total; b += nw) {
    const int pos = b * bm;
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= pos) lo = mid; else hi = mid - 1;
    }
    expert_ids[b] = lo;
  }
  // pads: expert e owns padded positions [off + c, off + round_up(c, bm))
  for (int idx = tid; idx < E * bm; idx += nw) {
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

// Router logits x[t] . W_router[e] (fp32 accumulation, v_mfma_f32_16x16x32_bf16
// with operands straight from L2, 16 experts x 16 tokens per tile).  Each
// workgroup (16 waves) takes kRouterTokens tokens and either every expert
// (GATE: the logits stay in LDS and each wave gates one token there) or one
// tile of 16 experts (grid y; logits only, for decode, whose GEMV path
// gates).  A wave accumulates up to kTiles expert tiles at once, so each
// token fragment it loads serves all of them; the waves split H in 32-element
// steps as many ways (ksplit) as the tile groups leave room for, and the
// partial tiles are added in LDS in a fixed order.  LDS (dynamic, sized by E
// on the host): region A = the partial tiles [ksplit][16][E16], reused after
// the sum as per-wave gating scratch; then, for GATE, the logits [16][E].
// The static allocation covers the largest E.
constexpr int kRouterTokens = 16;
typedef __bf16 rbf16x8 __attribute__((ext_vector_type(8)));
typedef float rf32x4 __attribute__((ext_vector_type(4)));
typedef unsigned ru32x4 __attribute__((ext_vector_type(4)));

template <bool GATE>
struct RouterShape {
  static constexpr int kWaves = 16;
  static constexpr int kTiles = GATE ? 4 : 1;   // expert tiles one wave accumulates
  static constexpr int kSteps = GATE ? 4 : 2;   // K steps whose loads are issued together
  static constexpr int kLds = GATE ? 81920 : 16384;   // >= router_lds_bytes(E) for every E <= 256
};

struct RouterSplit {
  int ntiles, ksplit, e16;
};

__host__ __device__ inline RouterSplit router_split(int E, bool gate) {
  const int nw = gate ? RouterShape<true>::kWaves : RouterShape<false>::kWaves;
  const int tpw = gate ? RouterShape<true>::kTiles : RouterShape<false>::kTiles;
  RouterSplit r;
  r.ntiles = gate ? (E + 15) / 16 : 1;
  const int ngroups = (r.ntiles + tpw - 1) / tpw;
  r.ksplit = nw / ngroups > 1 ? nw / ngroups : 1;
  r.e16 = 16 * r.ntiles;
  return r;
}

__host__ __device__ inline size_t router_region_a(int E, bool gate) {
  const RouterSplit sp = router_split(E, gate);
  size_t a = (size_t)sp.ksplit * kRouterTokens * sp.e16 * sizeof(float);
  if (gate) {
    const size_t scratch =
        (size_t)RouterShape<true>::kWaves * (kMaxExperts * sizeof(double) + 64 * sizeof(int));
    a = a > scratch ? a : scratch;
  }
  return (a + 15) / 16 * 16;
}

__host__ __device__ inline size_t router_lds_bytes(int E, bool gate) {
  return router_region_a(E, gate) + (gate ? (size_t)kRouterTokens * E * sizeof(float) : 0);
}

template <bool GATE>
__global__ void __launch_bounds__(RouterShape<GATE>::kWaves * 64) router_kernel(
    GateParams g, const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int H,
    float* __restrict__ logits) {
  constexpr int NW = RouterShape<GATE>::kWaves;
  constexpr int TPW = RouterShape<GATE>::kTiles;
  constexpr int U = RouterShape<GATE>::kSteps;
  __shared__ __attribute__((aligned(16))) unsigned char router_lds[RouterShape<GATE>::kLds];
  const RouterSplit sp = router_split(g.E, GATE);
  float* s_part = (float*)router_lds;                                        // [ksplit][16][e16]
  float* s_log = (float*)(router_lds + router_region_a(g.E, GATE));          // [16][E]
  double* s_sig = (double*)router_lds;                                       // [NW][256] after the sum
  int* s_keep = (int*)(s_sig + NW * kMaxExperts);                            // [NW][64]

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int t0 = blockIdx.x * kRouterTokens;
  const int nt = min(kRouterTokens, g.T - t0);
  const int e_base = GATE ? 0 : blockIdx.y * 16;
  const int kp = wave % sp.ksplit, tg = wave / sp.ksplit;
  const int r = lane & 15, gq = lane >> 4;   // operand row / column r, K group gq
  const uint16_t* xr = r < nt ? x + (int64_t)(t0 + r) * H : nullptr;
  const ru32x4 zero = {0u, 0u, 0u, 0u};
  auto ld = [&](const uint16_t* row, int kc) -> ru32x4 {
    return (row && kc < H) ? *(const ru32x4*)(row + kc) : zero;
  };
  auto mma = [&](ru32x4 a, ru32x4 b, rf32x4 c) -> rf32x4 {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(rbf16x8, a),
                                                   __builtin_bit_cast(rbf16x8, b), c, 0, 0, 0);
  };
  // tile group tg: tiles tg * TPW + j that exist.  The loop runs over
  // groups of U K steps (32 elements each), every load of a group issued
  // before its MFMAs; the trip count is wave-uniform (the MFMAs need the whole
  // wave); each lane reads its 8 K elements from kb (H is a multiple of 8;
  // zeros past H, so steps past the end add nothing)
  const int tile0 = tg * TPW;
  if (tile0 < sp.ntiles) {
    const uint16_t* wrow[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int e = e_base + (tile0 + j) * 16 + r;
      wrow[j] = (tile0 + j < sp.ntiles && e < g.E) ? wr + (int64_t)e * H : nullptr;
    }
    rf32x4 acc[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) acc[j] = rf32x4{0.f, 0.f, 0.f, 0.f};
    const int KS = 32 * sp.ksplit;
    for (int kb = 32 * kp + 8 * gq; kb - 8 * gq < H; kb += U * KS) {
      ru32x4 b[U], a[U][TPW];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        b[u] = ld(xr, kb + u * KS);
#pragma unroll
        for (int j = 0; j < TPW; ++j) a[u][j] = ld(wrow[j], kb + u * KS);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < TPW; ++j) acc[j] = mma(a[u][j], b[u], acc[j]);
    }
    // lane (r, gq) holds experts 16 i + 4 gq + v of token r
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      if (tile0 + j >= sp.ntiles) break;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        s_part[(kp * kRouterTokens + r) * sp.e16 + (tile0 + j) * 16 + 4 * gq + v] = acc[j][v];
    }
  }
  __syncthreads();
  const int ne = GATE ? g.E : min(16, g.E - e_base);
  for (int idx = tid; idx < nt * ne; idx += blockDim.x) {
    const int t = idx / ne, j = idx - t * ne;
    float v = 0.f;
    for (int q = 0; q < sp.ksplit; ++q) v += s_part[(q * kRouterTokens + t) * sp.e16 + j];
    logits[(int64_t)(t0 + t) * g.E + e_base + j] = v;
    if (GATE) s_log[t * g.E + j] = v;
  }
  if (!GATE) return;
  __syncthreads();   // region A becomes the gating scratch
  GateParams lg = g;
  lg.logits = s_log;   // the tile's logits, row stride E, in LDS
  for (int t = wave; t < nt; t += NW) {
    int id;
    float w;
    gate_token(lg, t, s_sig + wave * kMaxExperts, s_keep + wave * 64, &id, &w);
    if (lane < g.k) {
      g.topk_ids[(int64_t)(t0 + t) * g.k + lane] = id;
      g.topk_w[(int64_t)(t0 + t) * g.k + lane] = w;
    }
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
  write_layout(s_cnt, s_off, a.E, a.block_m, a.n, s_total, a.sorted_ids, a.expert_ids, a.ntpp,
               tid, blockDim.x);
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
// expert from all chunk histograms (a few KB from L2), the workgroups write
// the layout (expert_ids, pads, padded total) together, and each workgroup
// scatters its chunk's slots stably.
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
      // (unrolled so that the loads, from L2, are in flight together: at
      // 64 chunks each thread reads 16)
#pragma unroll 16
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
  // every workgroup has the layout: they write its block ids and pads together
  write_layout(s_cnt, s_off, a.E, a.block_m, a.n, s_total, a.sorted_ids, a.expert_ids, a.ntpp,
               (int)(blockIdx.x * blockDim.x + tid), (int)(gridDim.x * blockDim.x));
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

hipError_t launch_router(const GateParams& g, const uint16_t* x, const uint16_t* router_w, int H,
                         float* logits, bool gate, hipStream_t s) {
  if (g.T == 0) return hipSuccess;
  const unsigned nb = (unsigned)((g.T + kRouterTokens - 1) / kRouterTokens);
  if (g.E < 1 || g.E > kMaxExperts ||
      router_lds_bytes(g.E, gate) > (size_t)(gate ? RouterShape<true>::kLds : RouterShape<false>::kLds))
    return hipErrorInvalidValue;
  if (gate)
    hipLaunchKernelGGL(router_kernel<true>, dim3(nb), dim3(RouterShape<true>::kWaves * 64), 0, s, g,
                       x, router_w, H, logits);
  else
    hipLaunchKernelGGL(router_kernel<false>, dim3(nb, (g.E + 15) / 16),
                       dim3(RouterShape<false>::kWaves * 64), 0, s, g, x, router_w, H, logits);
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
