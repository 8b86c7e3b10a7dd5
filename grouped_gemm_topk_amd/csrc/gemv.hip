// Decode path (T <= 16 tokens): routing plus two expert GEMVs in two launches.
//
// The aligned layout groups the slots of one expert into one block (each
// expert has at most T <= 16 slots), which is the dedupe of duplicate experts
// across tokens of the B70 grouped multi-token experiment (*Intent*): one
// read of an expert's rows serves every token that picked it.  The activation
// is fused into the first GEMV (SwiGLU of the axolotl DeepSeek-V3 MoE forward,
// relu^2 of the mlxcel fc1 kernel) and the routed weight plus the sum over the
// k slots into the second (skill card *Common Pitfalls* 4).  That B70
// experiment lost to a per-slot path because its grouping added scans,
// scatters and register pressure; here the grouping costs nothing extra
// because the routing itself produces it.
//
// gfx950 mapping.  At decode the layer is HBM-bound and latency-bound:
// * Routing (top-k gating and align for at most 256 slots) runs as a prologue
//   of EVERY workgroup of GEMV1 from the router logits in LDS, so no separate
//   routing launch sits on the critical path; workgroup (0,0) also writes the
//   routing outputs that GEMV2 and the caller read.  Top-k uses ranks: each
//   lane counts the experts that beat its own (logit, then lower index) with
//   broadcast LDS reads, so there is no chain of cross-lane reductions.
// * Weights are read once with coalesced nontemporal loads and staged through
//   LDS into the operand layout of v_mfma_f32_16x16x32_bf16, whose tile covers
//   16 weight rows x up to 16 tokens.  K is split across the waves of a
//   workgroup and reduced in LDS.
// * GEMV2 adds weight * result into `out` with fp32 atomics (the k slots of a
//   token arrive in any order); GEMV1 zeroes `out` first.
// * From kFusedMinSlots slots on, a second path: a one-workgroup route kernel
//   (routing, zeroing `out`, resetting per-block counters), then one launch in
//   which the first workgroups do the W13 GEMV and count themselves done per
//   block, and the rest request their W2 weights at once, wait for their
//   block's count and finish.  The activation rows cross between them with
//   device-coherent 8-byte stores and loads, which need no cache maintenance
//   (an acquire per poll invalidated the L2 and was seven times slower; one
//   shared counter serialised every workgroup's atomic).  The W2 stream then
//   overlaps the W13 one, which pays once the W13 phase is long (larger T);
//   for a handful of slots the separate, prologue-carrying GEMV1 is faster.
#include <hip/hip_runtime.h>
#include <limits.h>

#include "moe_internal.h"
#include "wave_topk.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRound = 256;       // K elements per round: 8 MFMAs x 32
constexpr int kMaxSlots = kGemvMaxTokens * 16;

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

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ------------------------------------------------------------------ routing prologue
constexpr int kRow = kMaxExperts;   // LDS row of one token's logits, padded with -inf

constexpr int kPrologueWaves = 4;     // waves of GEMV1, which carries the prologue
constexpr int kRouteWaves = 16;       // waves of the route kernel: one per token

template <int NW>
struct RouteLdsT {
  float wlog[NW][kRow];     // per-wave copy of one token's logits
  uint64_t key[NW][kRow];   // per-wave order keys of one token
  double gscore[NW][64];
  double ex[kMaxSlots];        // per-slot exp / sigmoid terms of the weights
  int ids[kMaxSlots];
  float val[kMaxSlots];
  float wts[kMaxSlots];
  unsigned tokmask[kMaxExperts];  // bit t: token t picked the expert
  int off[kMaxExperts];
  int blk_expert[kMaxSlots];   // expert of each block (<= min(E, n) blocks)
  int rowslot[16];             // slot of each of this workgroup's 16 rows (-1: none)
  int ntpp;
  int my_expert;               // expert of this workgroup's block, -1 if none
};
typedef RouteLdsT<kPrologueWaves> RouteLds;

// Gating + align for all T <= 16 tokens by one workgroup of NW waves (one
// token per wave at a time)
// waves.  Fills `L` and, when `write_out`, the routing outputs in global
// memory.  `blk` is the block whose rows this workgroup needs (or -1).
template <int NW>
__device__ void route_prologue(const GemvParams& p, RouteLdsT<NW>& L, int blk, bool write_out) {
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int T = p.T, E = p.E, k = p.k;
  const int n = T * k;

  for (int e = tid; e < E; e += nthr) L.tokmask[e] = 0u;
  if (tid < 16) L.rowslot[tid] = -1;
  __syncthreads();

  // ---- gating: one wave per token
  float* wl = L.wlog[wave];
  uint64_t* wk = L.key[wave];
  for (int t = wave; t < T; t += NW) {
    float v[4];
    bool avail[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = lane + 64 * i;
      avail[i] = e < E;
      v[i] = avail[i] ? p.logits[t * E + e] : 0.f;
    }
    if (p.n_group > 1) {
      // groups of gsize contiguous experts ranked by the sum of their two
      // largest fp64 sigmoids (ties to the lower group index); experts of the
      // other groups are masked
      const int gsize = E / p.n_group;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i < E) wl[lane + 64 * i] = v[i];
      wave_sync_lds();
      double score = -1.0;
      if (lane < p.n_group) {
        double b1 = -1.0, b2 = -1.0;
        for (int q = 0; q < gsize; ++q) {
          double s = 1.0 / (1.0 + exp(-(double)wl[lane * gsize + q]));
          if (s > b1) { b2 = b1; b1 = s; }
          else if (s > b2) { b2 = s; }
        }
        score = b1 + (gsize > 1 ? b2 : 0.0);
        L.gscore[wave][lane] = score;
      }
      wave_sync_lds();
      int keep = 0;
      if (lane < p.n_group) {
        int rank = 0;
        for (int g = 0; g < p.n_group; ++g) {
          double o = L.gscore[wave][g];
          rank += (o > score || (o == score && g < lane)) ? 1 : 0;
        }
        keep = rank < p.topk_group;
      }
      const uint64_t keep_mask = __ballot(keep);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int e = lane + 64 * i;
        if (e < E && !((keep_mask >> (e / gsize)) & 1ull)) avail[i] = false;
      }
    }
    // the k largest keys: keys order by logit, then by lower expert index;
    // absent and group-masked experts have key 0 and are never selected (a
    // logit of -inf still has a non-zero key)
    uint64_t kown[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kown[i] = avail[i] ? order_key(v[i], lane + 64 * i) : 0ull;
    auto sel = [&](int i, int r) {
      L.ids[t * k + r] = lane + 64 * i;
      L.val[t * k + r] = v[i];
    };
    wave_topk_n((E + 63) >> 6, wk, kown, lane, k, sel);
    wave_sync_lds();
    // weights in fp64 (only where the routing outputs are written: the GEMV
    // reads them from there): each selected lane forms its term, then sums
    // the k terms of the token in selection order
    if (write_out) {
      double full = 0.0;
      if (p.scoring == 0 && !p.renorm) {
        const double m = (double)L.val[t * k];   // nothing is masked: the global max
        double part = 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (lane + 64 * i < E) part += exp((double)v[i] - m);
        full = wave_sum(part);
      }
      double term = 0.0;
      if (lane < k) {
        const double mine = (double)L.val[t * k + lane];
        term = p.scoring == 0 ? exp(mine - (double)L.val[t * k]) : 1.0 / (1.0 + exp(-mine));
        L.ex[t * k + lane] = term;
      }
      wave_sync_lds();
      if (lane < k) {
        double den;
        if (!p.renorm) {
          den = p.scoring == 0 ? full : 1.0;
        } else {
          den = 0.0;
          for (int j = 0; j < k; ++j) den += L.ex[t * k + j];
        }
        L.wts[t * k + lane] = (float)(term / den * (double)p.scale);
      }
    }
    if (lane < k) {
      atomicOr(&L.tokmask[L.ids[t * k + lane]], 1u << t);
    }
  }
  __syncthreads();

  // ---- align: count of expert e = popcount(tokmask[e]); the rank of token t's
  // slot inside expert e = tokens below t that picked e (slots ascend with t).
  // An expert holds at most T <= 16 <= bm slots, so its padded count is 0 or
  // bm: its offset is bm times the number of non-empty experts below it (one
  // ballot per 64 experts), and it owns at most one block.
  if (tid < 64) {
    int before = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 64 * i;
      const bool ne = e < E && L.tokmask[e] != 0u;
      const uint64_t m = __ballot(ne);
      const int idx = before + __popcll(m & ((1ull << tid) - 1ull));
      if (e < E) {
        L.off[e] = idx * p.bm;
        if (ne) L.blk_expert[idx] = e;
      }
      before += __popcll(m);
    }
    if (tid == 0) L.ntpp = before * p.bm;
  }
  __syncthreads();
  const int ntpp = L.ntpp;
  const int b0 = blk >= 0 ? blk * p.bm : -1;
  for (int s = tid; s < n; s += nthr) {
    const int e = L.ids[s];
    const int t = s / k;
    const int pos = L.off[e] + __popc(L.tokmask[e] & ((1u << t) - 1u));
    if (b0 >= 0 && pos >= b0 && pos < b0 + 16) L.rowslot[pos - b0] = s;
    if (write_out) {
      p.sorted_ids[pos] = s;
      p.topk_ids[s] = e;
      p.topk_w[s] = L.wts[s];
    }
  }
  if (write_out) {
    for (int e = tid; e < E; e += nthr) {
      int c = __popc(L.tokmask[e]);
      int pc = (c + p.bm - 1) / p.bm * p.bm;
      for (int r = c; r < pc; ++r) p.sorted_ids[L.off[e] + r] = n;
      if (pc > 0) p.expert_ids[L.off[e] / p.bm] = e;
    }
    if (tid == 0) *p.ntpp = ntpp;
  }
  if (tid == 0) L.my_expert = (blk >= 0 && blk * p.bm < ntpp) ? L.blk_expert[blk] : -1;
  __syncthreads();
}

// ------------------------------------------------------------------ GEMV tiles
// A weight tile is 16 rows x 256 elements (one 512-byte K round per row).  It
// is loaded with fully coalesced 1 KB wave loads (load j covers tile rows 2j
// and 2j+1, 32 lanes x 16 bytes each), parked in the wave's own LDS buffer with
// the 16-byte chunk index XOR-ed by the row, and read back in the MFMA operand
// layout (lane r + 16 g: row r, chunk 4 q + g for MFMA q), which is then
// free of bank conflicts.  The token operand uses the same K order:
// MFMA q covers K elements k0 + 32 q + 8 g + 0..7 for lane group g.
constexpr int kTileU4 = 16 * 32;   // 16-byte chunks of one tile

// One tile's weight rows: bf16, or MXFP8 (Q: FP8 E4M3 bytes, one E8M0 scale
// byte per 32 elements of a row, OCP Microscaling), which is decoded exactly
// to bf16 on its way into LDS.  The buffer descriptor covers the tile's valid
// rows (at most 16), so loads past them return zero.  DWORD3 0x00020000 =
// raw 32-bit data format for gfx9 buffers.
struct WSrc {
  __amdgpu_buffer_rsrc_t rs;
  int ld;                  // row stride in elements
  const uint8_t* sc;       // MXFP8: scale row of the tile's first row
  int rows;                // valid rows (<= 16)
};

template <bool Q>
__device__ __forceinline__ WSrc make_wsrc(const void* mat, const uint8_t* scales, int64_t row0,
                                          int ld, int rows_valid) {
  WSrc w;
  w.rows = rows_valid < 16 ? rows_valid : 16;
  w.ld = ld;
  constexpr int eb = Q ? 1 : 2;   // bytes per element
  const char* first = (const char*)mat + row0 * ld * eb;
  w.rs = __builtin_amdgcn_make_buffer_rsrc((void*)first, (short)0, (int)(w.rows * ld * eb),
                                           0x00020000);
  w.sc = Q ? scales + row0 * (ld / 32) : nullptr;
  return w;
}

// bf16: eight 1 KB wave loads (load j covers tile rows 2j and 2j+1, 32 lanes x
// 16 bytes).  MXFP8: four 1 KB wave loads (load j covers rows 4j .. 4j+3, 16
// lanes x 16 elements each) plus each lane's four scale bytes in v[4].
template <bool Q>
__device__ __forceinline__ void tile_load(const WSrc& w, int k0, int K, u32x4 (&v)[8]) {
  const int lane = threadIdx.x & 63;
  if (!Q) {
    const int kc = k0 + 8 * (lane & 31);
    const int base = (lane >> 5) * w.ld * 2 + kc * 2;   // byte offset of row (lane >> 5)
    const int step = 4 * w.ld;                          // two rows
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int off = kc < K ? base + j * step : -1;     // -1: beyond the descriptor -> zero
      v[j] = __builtin_amdgcn_raw_buffer_load_b128(w.rs, off, 0, 2 /* nontemporal */);
    }
  } else {
    const int kc = k0 + 16 * (lane & 15);
    const int r0 = lane >> 4;
    unsigned sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 4 * j + r0;
      const int off = kc < K ? row * w.ld + kc : -1;
      v[j] = __builtin_amdgcn_raw_buffer_load_b128(w.rs, off, 0, 2 /* nontemporal */);
      sc[j] = (kc < K && row < w.rows) ? w.sc[row * (w.ld / 32) + kc / 32] : 0u;
    }
    v[4] = u32x4{sc[0], sc[1], sc[2], sc[3]};
  }
}

// two E4M3 bytes of `four` (the low or the high pair) times the E8M0 scale
// `s` -> two bf16 (exact: three mantissa bits times a power of two)
template <bool HI>
__device__ __forceinline__ unsigned e4m3x2_to_bf16x2(unsigned four, float s) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(four, s, HI));
}

// The tile in the wave's own LDS buffer, 16-byte chunks of 8 bf16 with the
// chunk index XOR-ed by the row (row r, chunk c at r * 32 + (c ^ r)).
template <bool Q>
__device__ __forceinline__ void tile_store(u32x4* lds, const u32x4 (&v)[8]) {
  const int lane = threadIdx.x & 63;
  if (!Q) {
    const int ch = lane & 31;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 2 * j + (lane >> 5);
      lds[row * 32 + (ch ^ row)] = v[j];
    }
  } else {
    const int c8 = lane & 15;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 4 * j + (lane >> 4);
      // the E8M0 byte is the exponent field of the float scale operand
      const float s = __builtin_bit_cast(float, v[4][j] << 23);
      const u32x4 x = v[j];
      const u32x4 lo = {e4m3x2_to_bf16x2<false>(x.x, s), e4m3x2_to_bf16x2<true>(x.x, s),
                        e4m3x2_to_bf16x2<false>(x.y, s), e4m3x2_to_bf16x2<true>(x.y, s)};
      const u32x4 hi = {e4m3x2_to_bf16x2<false>(x.z, s), e4m3x2_to_bf16x2<true>(x.z, s),
                        e4m3x2_to_bf16x2<false>(x.w, s), e4m3x2_to_bf16x2<true>(x.w, s)};
      lds[row * 32 + ((2 * c8) ^ row)] = lo;
      lds[row * 32 + ((2 * c8 + 1) ^ row)] = hi;
    }
  }
}

__device__ __forceinline__ u32x4 tile_operand(const u32x4* lds, int q) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int c = 4 * q + (lane >> 4);
  return lds[r * 32 + (c ^ r)];
}

__device__ __forceinline__ void token_operands(const uint16_t* row, int k0, int K, u32x4 (&xb)[8]) {
  const int kg = k0 + 8 * ((threadIdx.x & 63) >> 4);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int kc = kg + 32 * q;
    xb[q] = (row && kc < K) ? *(const u32x4*)(row + kc) : u32x4{0u, 0u, 0u, 0u};
  }
}

// token_operands for rows another workgroup of the same launch wrote: 8-byte
// device-coherent loads, which never return a stale L2 copy (the writer used
// device-coherent stores and counted itself done after they completed)
__device__ __forceinline__ void token_operands_coherent(const uint16_t* row, int k0, int K,
                                                        u32x4 (&xb)[8]) {
  const int kg = k0 + 8 * ((threadIdx.x & 63) >> 4);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int kc = kg + 32 * q;
    if (row && kc < K) {
      const uint64_t* p8 = (const uint64_t*)(row + kc);
      const uint64_t lo = __hip_atomic_load(p8, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t hi = __hip_atomic_load(p8 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      xb[q] = u32x4{(unsigned)lo, (unsigned)(lo >> 32), (unsigned)hi, (unsigned)(hi >> 32)};
    } else {
      xb[q] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

__device__ __forceinline__ f32x4 tile_mfma(const u32x4* lds, const u32x4 (&xb)[8], f32x4 acc) {
#pragma unroll
  for (int q = 0; q < 8; ++q) acc = mfma16(tile_operand(lds, q), xb[q], acc);
  return acc;
}

// K rounds kp, kp + S, ... of one tile against one token row, with the
// next round's weight tile requested before the current one is consumed, so
// that every wave keeps a tile of loads in flight.
template <bool Q>
__device__ __forceinline__ f32x4 stream_rounds(const WSrc& ws, int K, const uint16_t* brow, int kp,
                                               int S, int rounds, u32x4* tl, f32x4 acc) {
  u32x4 cur[8], nxt[8], xb[8];
  int rd = kp;
  if (rd < rounds) tile_load<Q>(ws, rd * kRound, K, cur);
  while (rd < rounds) {
    const int nrd = rd + S;
    if (nrd < rounds) tile_load<Q>(ws, nrd * kRound, K, nxt);
    token_operands(brow, rd * kRound, K, xb);
    tile_store<Q>(tl, cur);
    wave_sync_lds();
    acc = tile_mfma(tl, xb, acc);
    wave_sync_lds();
    rd = nrd;
    if (rd >= rounds) break;
    const int nrd2 = rd + S;
    if (nrd2 < rounds) tile_load<Q>(ws, nrd2 * kRound, K, cur);
    token_operands(brow, rd * kRound, K, xb);
    tile_store<Q>(tl, nxt);
    wave_sync_lds();
    acc = tile_mfma(tl, xb, acc);
    wave_sync_lds();
    rd = nrd2;
  }
  return acc;
}

// K rounds kp, kp + S, ... of one tile against one token row.  The caller
// has issued the loads of the first two rounds (stream_begin) into cur / nxt;
// each round's weight tile is consumed while the round two steps later is in
// flight, so every wave keeps two tiles of loads outstanding.
template <bool Q>
__device__ __forceinline__ void stream_begin(const WSrc& ws, int K, int kp, int S, int rounds,
                                             u32x4 (&cur)[8], u32x4 (&nxt)[8]) {
  if (kp < rounds) tile_load<Q>(ws, kp * kRound, K, cur);
  if (kp + S < rounds) tile_load<Q>(ws, (kp + S) * kRound, K, nxt);
}

template <bool Q, bool COHERENT>
__device__ __forceinline__ f32x4 stream_finish(const WSrc& ws, int K, const uint16_t* brow, int kp,
                                               int S, int rounds, u32x4* tl, f32x4 acc,
                                               u32x4 (&cur)[8], u32x4 (&nxt)[8]) {
  u32x4 xb[8];
  int rd = kp;
  while (rd < rounds) {
    if (COHERENT) token_operands_coherent(brow, rd * kRound, K, xb);
    else token_operands(brow, rd * kRound, K, xb);
    tile_store<Q>(tl, cur);
    wave_sync_lds();
    acc = tile_mfma(tl, xb, acc);
    wave_sync_lds();
    if (rd + 2 * S < rounds) tile_load<Q>(ws, (rd + 2 * S) * kRound, K, cur);
    rd += S;
    if (rd >= rounds) break;
    if (COHERENT) token_operands_coherent(brow, rd * kRound, K, xb);
    else token_operands(brow, rd * kRound, K, xb);
    tile_store<Q>(tl, nxt);
    wave_sync_lds();
    acc = tile_mfma(tl, xb, acc);
    wave_sync_lds();
    if (rd + 2 * S < rounds) tile_load<Q>(ws, (rd + 2 * S) * kRound, K, nxt);
    rd += S;
  }
  return acc;
}

// The expert matrices of a block: W13 rows [M1, H] or W2 rows [H, I] of expert
// e (or the shared expert), and with MXFP8 their scale rows.
template <bool Q>
__device__ __forceinline__ const void* w13_mat(const GemvParams& p, bool shared, int e, int M1,
                                               const uint8_t** sc) {
  if (shared) {
    *sc = p.sw13_s;
    return p.sw13;
  }
  *sc = Q ? p.w13_s + (int64_t)e * M1 * (p.H / 32) : nullptr;
  return (const char*)p.w13 + (int64_t)e * M1 * p.H * (Q ? 1 : 2);
}

template <bool Q>
__device__ __forceinline__ const void* w2_mat(const GemvParams& p, bool shared, int e,
                                              const uint8_t** sc) {
  if (shared) {
    *sc = p.sw2_s;
    return p.sw2;
  }
  *sc = Q ? p.w2_s + (int64_t)e * p.H * (p.I / 32) : nullptr;
  return (const char*)p.w2 + (int64_t)e * p.H * p.I * (Q ? 1 : 2);
}

constexpr int kG1Waves = kPrologueWaves;
constexpr int kG2Waves = 4;

// GEMV1: routing prologue, then the workgroup's p.nt1 tiles of 16 act columns
// at once, each tile on 8 / p.nt1 waves (SwiGLU: half on the gate rows, half
// on the up rows) that split K.  act[row j of block b][c0 + 0..15] =
// act(x[token of row j] . w13[e] rows).  Also zeroes `out`.
// Grid (ceil(ceil(I/16) / nt1), nblk + shared).
template <bool SW, bool Q>
__global__ void __launch_bounds__(kG1Waves * 64) gemv1_kernel(GemvParams p) {
  __shared__ union {
    RouteLds L;
    u32x4 tile[kG1Waves][kTileU4];
  } sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  {  // zero the output that GEMV2 accumulates into
    const int64_t n4 = (int64_t)p.T * p.H / 4;
    const int64_t nwg = (int64_t)gridDim.x * gridDim.y;
    const int64_t wg = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    for (int64_t i = wg * blockDim.x + tid; i < n4; i += nwg * blockDim.x)
      ((float4*)p.out)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  const int b = blockIdx.y;
  const bool shared = b == p.nblk;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *p.status = 0;   // no waits here
  route_prologue(p, sm.L, shared ? -1 : b, blockIdx.x == 0 && blockIdx.y == 0);
  const int e = sm.L.my_expert;
  const int r = lane & 15;   // token column of this lane (operand and result)
  const int g = lane >> 4;
  const int slot = shared ? (r < p.T ? r : -1) : sm.L.rowslot[r];
  __syncthreads();           // the LDS union is reused below
  if (!shared && e < 0) return;
  const int M1 = SW ? 2 * p.I : p.I;
  const uint8_t* Wsc;
  const void* W = w13_mat<Q>(p, shared, e, M1, &Wsc);
  const int tok = slot < 0 ? -1 : (shared ? slot : slot / p.k);
  const uint16_t* xrow = tok >= 0 ? p.x + (int64_t)tok * p.H : nullptr;
  u32x4* tl = sm.tile[wave];
  const int rounds = (p.H + kRound - 1) / kRound;

  // tile ti of the workgroup is handled by `per` waves: SwiGLU gives half of
  // them the gate rows and half the up rows, each half splitting K S ways
  const int per = kG1Waves / p.nt1;
  const int S = SW ? per / 2 : per;
  const int ti = wave / per;
  const int wi = wave % per;
  const bool up = SW && wi >= S;
  const int kp = wi % S;
  const int c0 = (blockIdx.x * p.nt1 + ti) * 16;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (c0 < p.I) {
    const WSrc ws = make_wsrc<Q>(W, Wsc, (up ? p.I : 0) + c0, p.H, p.I - c0);
    acc = stream_rounds<Q>(ws, p.H, xrow, kp, S, rounds, tl, acc);
  }
  ((f32x4*)tl)[lane] = acc;   // partial sums reuse the wave's own tile buffer
  __syncthreads();
  if (wi != 0 || c0 >= p.I || slot < 0 || c0 + 4 * g >= p.I) return;
  f32x4 hg = acc, hu = {0.f, 0.f, 0.f, 0.f};
  for (int w = 1; w < per; ++w) {
    const f32x4 o = ((const f32x4*)sm.tile[wave + w])[lane];
    if (SW && w >= S) hu += o; else hg += o;
  }
  // lane holds act columns c0 + 4 g + v of token column r
  float o4[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    if (SW) {
      o4[v] = silu(hg[v]) * hu[v];
    } else {
      float t = fmaxf(hg[v], 0.f);
      o4[v] = t * t;
    }
  }
  uint16_t* dst = shared ? p.act_sh + (int64_t)r * p.I : p.act + (int64_t)(b * p.bm + r) * p.I;
  uint2 pk;
  pk.x = (unsigned)f32_to_bf16(o4[0]) | ((unsigned)f32_to_bf16(o4[1]) << 16);
  pk.y = (unsigned)f32_to_bf16(o4[2]) | ((unsigned)f32_to_bf16(o4[3]) << 16);
  *(uint2*)(dst + c0 + 4 * g) = pk;
}

// GEMV2: the workgroup's p.nt2 tiles of 16 output rows at once, each on
// p.s2 = 4 / p.nt2 waves that split K; out[token of row j][h0 + ..] +=
// w_slot * (act[row j] . w2[e][h]).  Grid (ceil(ceil(H/16) / nt2), nblk + shared).
template <bool Q>
__global__ void __launch_bounds__(kG2Waves * 64) gemv2_kernel(GemvParams p) {
  __shared__ u32x4 s_tile[kG2Waves][kTileU4];
  __shared__ int s_slot[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.y;
  const bool shared = b == p.nblk;
  const int base = b * p.bm;
  const uint8_t* Wsc;
  const void* W;
  if (shared) {
    W = w2_mat<Q>(p, true, 0, &Wsc);
  } else {
    if (base >= *p.ntpp) return;
    const int e = p.expert_ids[b];
    if (e < 0 || e >= p.E) return;
    W = w2_mat<Q>(p, false, e, &Wsc);
  }
  if (tid < 16) {
    int s = -1;
    if (shared) {
      s = tid < p.T ? tid : -1;
    } else {
      int sid = p.sorted_ids[base + tid];
      s = (sid >= 0 && sid < p.T * p.k) ? sid : -1;
    }
    s_slot[tid] = s;
  }
  __syncthreads();
  const int r = lane & 15;
  const int g = lane >> 4;
  const int slot = s_slot[r];
  const uint16_t* arow = nullptr;
  if (slot >= 0) arow = shared ? p.act_sh + (int64_t)r * p.I : p.act + (int64_t)(base + r) * p.I;
  u32x4* tl = s_tile[wave];
  const int rounds = (p.I + kRound - 1) / kRound;

  const int S = kG2Waves / p.nt2;
  const int ti = wave / S;
  const int kp = wave % S;
  const int h0 = (blockIdx.x * p.nt2 + ti) * 16;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (h0 < p.H) {
    const WSrc ws = make_wsrc<Q>(W, Wsc, h0, p.I, p.H - h0);
    acc = stream_rounds<Q>(ws, p.I, arow, kp, S, rounds, tl, acc);
  }
  ((f32x4*)tl)[lane] = acc;
  __syncthreads();
  if (kp != 0 || h0 >= p.H || slot < 0) return;
  for (int w = wave + 1; w < wave + S; ++w) acc += ((const f32x4*)s_tile[w])[lane];
  const int tok = shared ? slot : slot / p.k;
  const float wgt = shared ? 1.f : p.topk_w[slot];
  // lane holds rows h0 + 4 g + v of token column r
  float* dst = p.out + (int64_t)tok * p.H + h0 + 4 * g;
#pragma unroll
  for (int v = 0; v < 4; ++v)
    if (h0 + 4 * g + v < p.H) unsafeAtomicAdd(dst + v, wgt * acc[v]);
}

// ------------------------------------------------------------------ fused path (larger T)
constexpr int kWaves = kPrologueWaves;   // waves of every decode workgroup
// the launcher sizes the tiles per workgroup of both decode forms with the
// GEMV wave counts, so the fused kernel must have the same waves (each tile's
// waves split K: kWaves / tiles per workgroup >= 1)
static_assert(kWaves == kG1Waves && kWaves == kG2Waves, "decode wave counts must agree");
// slots (T * top_k) from which the fused path runs: measured on MI355X, the
// separate W2 launch is cheaper at 8 and 24 slots (128 experts top-8, T = 1, 3
// and top-6, T = 1), the fused launch at 64 and 96 (T = 8 top-8, T = 16 top-6)
constexpr int kFusedMinSlots = 48;

// Control block in the layer workspace, reset by route_kernel before every
// decode_kernel launch: per block b (routed blocks, then the shared expert),
// the number of W13 workgroups of b that are done, each counter on its own
// 128-byte line so that the blocks' atomics do not queue behind each other.
constexpr int kCtlStride = 32;
// bound of the W2 workgroups' wait (polls about half a microsecond apart,
// about a second in all): far above any W13 phase, so a stuck counter ends
// the wait instead of the process.  The output is then wrong, and the
// workgroup records it in the layer's status word (the word after the
// counters, cleared by every call) for the caller to read.
constexpr int kMaxSpin = 1 << 21;
constexpr int kSpinSleep = 16;   // s_sleep units of 64 cycles between polls

// Routing for all T <= 16 tokens by one workgroup (gating + align, the
// outputs the decode kernel and the caller read), then zero `out` (the W2
// phase accumulates into it) and reset the control block.
__global__ void __launch_bounds__(kRouteWaves * 64) route_kernel(GemvParams p) {
  __shared__ RouteLdsT<kRouteWaves> L;
  route_prologue(p, L, -1, true);
  const int64_t n4 = (int64_t)p.T * p.H / 4;
  for (int64_t i = threadIdx.x; i < n4; i += blockDim.x)
    ((float4*)p.out)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  const int nb = p.nblk + (p.sw13 ? 1 : 0);
  for (int b = threadIdx.x; b < nb; b += blockDim.x) p.ctl[b * kCtlStride] = 0;
  if (threadIdx.x == 0) *p.status = 0;
}

// The slot of row r of block b, or -1 (a pad or no block); the shared expert's
// rows are the tokens.
__device__ __forceinline__ int block_row_slot(const GemvParams& p, int b, bool shared, int r, int ntpp) {
  if (shared) return r < p.T ? r : -1;
  if (b * p.bm >= ntpp) return -1;
  const int sid = p.sorted_ids[b * p.bm + r];
  return (sid >= 0 && sid < p.T * p.k) ? sid : -1;
}

// W13 phase, one workgroup: p.nt1 tiles of 16 act columns at once, each tile
// on kWaves / p.nt1 waves (SwiGLU: half on the gate rows, half on the up
// rows) that split K.  act[row j of block b][c0 + 0..15] = act(x[token of row
// j] . w13[e] rows).
template <bool SW, bool Q>
__device__ void w13_phase(const GemvParams& p, int bx, int b, u32x4 (*s_tile)[kTileU4], int* s_slot) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool shared = b == p.nblk;
  const int ntpp = *p.ntpp;
  if (tid < 16) s_slot[tid] = block_row_slot(p, b, shared, tid, ntpp);
  const int e = shared ? 0 : (b * p.bm < ntpp ? p.expert_ids[b] : -1);
  __syncthreads();
  if (!shared && (e < 0 || e >= p.E)) return;
  const int r = lane & 15;   // token column of this lane (operand and result)
  const int g = lane >> 4;
  const int slot = s_slot[r];
  const int M1 = SW ? 2 * p.I : p.I;
  const uint8_t* Wsc;
  const void* W = w13_mat<Q>(p, shared, e, M1, &Wsc);
  const int tok = slot < 0 ? -1 : (shared ? slot : slot / p.k);
  const uint16_t* xrow = tok >= 0 ? p.x + (int64_t)tok * p.H : nullptr;
  u32x4* tl = s_tile[wave];
  const int rounds = (p.H + kRound - 1) / kRound;
  const int per = kWaves / p.nt1;
  const int S = SW ? per / 2 : per;
  const int ti = wave / per;
  const int wi = wave % per;
  const bool up = SW && wi >= S;
  const int kp = wi % S;
  const int c0 = (bx * p.nt1 + ti) * 16;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (c0 < p.I) {
    const WSrc ws = make_wsrc<Q>(W, Wsc, (up ? p.I : 0) + c0, p.H, p.I - c0);
    u32x4 cur[8], nxt[8];
    stream_begin<Q>(ws, p.H, kp, S, rounds, cur, nxt);
    acc = stream_finish<Q, false>(ws, p.H, xrow, kp, S, rounds, tl, acc, cur, nxt);
  }
  ((f32x4*)tl)[lane] = acc;   // partial sums reuse the wave's own tile buffer
  __syncthreads();
  if (wi != 0 || c0 >= p.I || slot < 0 || c0 + 4 * g >= p.I) return;
  f32x4 hg = acc, hu = {0.f, 0.f, 0.f, 0.f};
  for (int w = 1; w < per; ++w) {
    const f32x4 o = ((const f32x4*)s_tile[wave + w])[lane];
    if (SW && w >= S) hu += o; else hg += o;
  }
  // lane holds act columns c0 + 4 g + v of token column r
  float o4[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    if (SW) {
      o4[v] = silu(hg[v]) * hu[v];
    } else {
      float t = fmaxf(hg[v], 0.f);
      o4[v] = t * t;
    }
  }
  uint16_t* dst = shared ? p.act_sh + (int64_t)r * p.I : p.act + (int64_t)(b * p.bm + r) * p.I;
  const uint64_t lo = (uint64_t)f32_to_bf16(o4[0]) | ((uint64_t)f32_to_bf16(o4[1]) << 16);
  const uint64_t hi = (uint64_t)f32_to_bf16(o4[2]) | ((uint64_t)f32_to_bf16(o4[3]) << 16);
  // device-coherent store: the W2 phase of this launch reads it from another CU
  __hip_atomic_store((uint64_t*)(dst + c0 + 4 * g), lo | (hi << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// W2 phase, one workgroup: p.nt2 tiles of 16 output rows at once, each on
// kWaves / p.nt2 waves that split K; out[token of row j][h0 + ..] +=
// w_slot * (act[row j] . w2[e][h]).  The first two rounds of weights are
// requested before the wait for the W13 phase, so they arrive while it runs.
template <bool Q>
__device__ void w2_phase(const GemvParams& p, int bx, int b, int g1x, u32x4 (*s_tile)[kTileU4],
                         int* s_slot) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool shared = b == p.nblk;
  const int ntpp = *p.ntpp;
  if (tid < 16) s_slot[tid] = block_row_slot(p, b, shared, tid, ntpp);
  const int e = shared ? 0 : (b * p.bm < ntpp ? p.expert_ids[b] : -1);
  const bool active = shared || (e >= 0 && e < p.E);
  const uint8_t* Wsc;
  const void* W = w2_mat<Q>(p, shared, active ? e : 0, &Wsc);
  const int rounds = (p.I + kRound - 1) / kRound;
  const int S = kWaves / p.nt2;
  const int ti = wave / S;
  const int kp = wave % S;
  const int h0 = (bx * p.nt2 + ti) * 16;
  const bool work = active && h0 < p.H;
  const WSrc ws = make_wsrc<Q>(W, Wsc, work ? h0 : 0, p.I, work ? p.H - h0 : 0);
  u32x4 cur[8], nxt[8];
  if (work) stream_begin<Q>(ws, p.I, kp, S, rounds, cur, nxt);
  // wait until the g1x W13 workgroups of this block have published its act rows
  if (tid == 0 && active) {
    int spins = 0;
    while (__hip_atomic_load(&p.ctl[b * kCtlStride], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
               g1x &&
           ++spins < kMaxSpin)
      __builtin_amdgcn_s_sleep(kSpinSleep);
    if (spins >= kMaxSpin)   // the wait expired: this call's output is invalid
      __hip_atomic_store(p.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();   // the act rows are then read with device-coherent loads
  if (!active) return;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int slot = s_slot[r];
  const uint16_t* arow = nullptr;
  if (slot >= 0) arow = shared ? p.act_sh + (int64_t)r * p.I : p.act + (int64_t)(b * p.bm + r) * p.I;
  u32x4* tl = s_tile[wave];
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (work) acc = stream_finish<Q, true>(ws, p.I, arow, kp, S, rounds, tl, acc, cur, nxt);
  ((f32x4*)tl)[lane] = acc;
  __syncthreads();
  if (kp != 0 || !work || slot < 0) return;
  for (int w = wave + 1; w < wave + S; ++w) acc += ((const f32x4*)s_tile[w])[lane];
  const int tok = shared ? slot : slot / p.k;
  const float wgt = shared ? 1.f : p.topk_w[slot];
  // lane holds rows h0 + 4 g + v of token column r
  float* dst = p.out + (int64_t)tok * p.H + h0 + 4 * g;
#pragma unroll
  for (int v = 0; v < 4; ++v)
    if (h0 + 4 * g + v < p.H) unsafeAtomicAdd(dst + v, wgt * acc[v]);
}

// Both GEMVs in one launch.  Workgroups [0, n1 = g1x * nb) do the W13 phase
// (tile bx, block b) and count themselves done in their block's counter; the
// rest do the W2 phase of a block, which waits for that block's count.
// Workgroups are dispatched in index order, so every W13 workgroup is running
// or finished before a W2 workgroup waits (and the wait is bounded).
template <bool SW, bool Q>
__global__ void __launch_bounds__(kWaves * 64) decode_kernel(GemvParams p, int g1x, int g2x) {
  __shared__ u32x4 s_tile[kWaves][kTileU4];
  __shared__ int s_slot[16];
  const int nb = p.nblk + (p.sw13 ? 1 : 0);
  const int n1 = g1x * nb;
  const int t = blockIdx.x;
  if (t < n1) {
    const int b = t / g1x;
    w13_phase<SW, Q>(p, t % g1x, b, s_tile, s_slot);
    // every thread's device-coherent act stores have completed before the count
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(&p.ctl[b * kCtlStride], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    const int t2 = t - n1;
    w2_phase<Q>(p, t2 % g2x, t2 / g2x, g1x, s_tile, s_slot);
  }
}

}  // namespace

// Tiles per workgroup: the largest power of two (up to the wave count) that
// still leaves at least `target` workgroups; the remaining waves split K.
// Measured targets: 768 for the W13 GEMV (about three workgroups per CU),
// 384 for W2 (fatter workgroups: decode T = 1 27.4 -> 26.8 us, relu2 T = 1
// 35.0 -> 33.8 us; 192 was slower again).
constexpr int64_t kTilesTargetW13 = 768;
constexpr int64_t kTilesTargetW2 = 384;
static int pick_tiles(int64_t tiles, int waves, int64_t target) {
  int nt = 1;
  while (nt < waves && tiles / (2 * nt) >= target) nt *= 2;
  return nt;
}

template <bool Q>
static hipError_t launch_gemv_fmt(GemvParams p, bool swiglu, hipStream_t s) {
  const int nb = p.nblk + (p.sw13 ? 1 : 0);
  const int tiles1 = (p.I + 15) / 16;
  const int tiles2 = (p.H + 15) / 16;
  p.nt1 = pick_tiles((int64_t)tiles1 * nb, swiglu ? kG1Waves / 2 : kG1Waves, kTilesTargetW13);
  p.nt2 = pick_tiles((int64_t)tiles2 * nb, kG2Waves, kTilesTargetW2);
  const int g1x = (tiles1 + p.nt1 - 1) / p.nt1;
  const int g2x = (tiles2 + p.nt2 - 1) / p.nt2;
  if (p.T * p.k >= kFusedMinSlots) {
    // route once, then both GEMVs in one launch with the W2 weights requested
    // while the W13 phase runs
    hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteWaves * 64), 0, s, p);
    const unsigned nwg = (unsigned)((g1x + g2x) * nb);
    if (swiglu)
      hipLaunchKernelGGL((decode_kernel<true, Q>), dim3(nwg), dim3(kWaves * 64), 0, s, p, g1x, g2x);
    else
      hipLaunchKernelGGL((decode_kernel<false, Q>), dim3(nwg), dim3(kWaves * 64), 0, s, p, g1x, g2x);
    return hipGetLastError();
  }
  dim3 g1(g1x, nb);
  if (swiglu)
    hipLaunchKernelGGL((gemv1_kernel<true, Q>), g1, dim3(kG1Waves * 64), 0, s, p);
  else
    hipLaunchKernelGGL((gemv1_kernel<false, Q>), g1, dim3(kG1Waves * 64), 0, s, p);
  dim3 g2(g2x, nb);
  hipLaunchKernelGGL((gemv2_kernel<Q>), g2, dim3(kG2Waves * 64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvParams& p, bool swiglu, hipStream_t s) {
  return p.mx ? launch_gemv_fmt<true>(p, swiglu, s) : launch_gemv_fmt<false>(p, swiglu, s);
}

}  // namespace moe
