// Grouped GEMM over the aligned (sorted + padded) token layout, bf16 MFMA on
// gfx950, with fused epilogues.
//
// The structure is the one of the skill card "Fused Moe Kernel", *Grouped
// GEMM Structure*: a tiled GEMM whose M-blocks reach their token rows through
// sorted_token_ids (token = id / top_k, *Common Pitfalls* 1), whose weight
// matrix is chosen per M-block by expert_ids (weights stacked [E, N, K],
// *Common Pitfalls* 3), and whose blocks at or beyond num_tokens_post_padded
// exit at once.  Epilogues: SwiGLU, silu(gate) times up (axolotl DeepSeek-V3 MoE
// forward), squared ReLU (mlxcel fc1 -> relu^2), plain store, and the routed
// weight times the row scattered to its slot (*Common Pitfalls* 4).
//
// gfx950 mapping.  One workgroup of 4 or 8 wave64s computes a BM x BNW tile
// of C^T = W_e . X^T: the weight rows play the MFMA "A" role and the gathered
// token rows the "B" role, so each lane ends up owning 4 consecutive output
// features of one token row and stores them as one 8- or 16-byte write.
// Operands go global -> LDS directly (buffer loads with the LDS destination
// bit) through an NS-stage ring of LDS buffers, NS - 1 K steps ahead of the
// MFMAs, with one barrier per K step.  A K step is 64 elements wide so each
// row chunk is one full 128-byte line (64-byte chunks halve what the
// load path delivers per CU).  Each thread's loads of a later step are spread
// between the MFMAs of the current one instead of being issued as a burst,
// which kept the address queue full and stalled the issuing waves.  The LDS
// chunk order is XOR-swizzled so the MFMA operand reads are free of bank
// conflicts.  Workgroups are mapped to tiles XCD by XCD (each XCD gets an
// equal, contiguous range of the tiles whose m-blocks hold rows; the grid is
// sized for the align capacity and the rest exit) and, inside a range, the
// tiles of one expert's run
// of M-blocks are consecutive, in chunks of 8 M-blocks per N-tile, so that a
// weight tile and the token rows are reused from that XCD's L2 (the L2
// grouping / cache-aware scheduling of the skill card's *Optimization
// Patterns*).
// v_mfma_f32_32x32x16_bf16 is used when a wave owns >= 32 token rows,
// v_mfma_f32_16x16x32_bf16 for BLOCK_M = 16.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));



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

// Operand tiles live in LDS as rows of BK bf16 (CPR = BK / 8 chunks of 16
// bytes).  16 / CPR rows fill the 64 banks once; XOR-ing the chunk with
// (row / (16 / CPR)) mod CPR gives any 16 consecutive rows read at one chunk
// 16 distinct bank groups, and 16 consecutive threads writing consecutive
// chunks hit distinct ones too.
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  return r * CPR + (c ^ ((r / (16 / CPR)) % CPR));
}

#ifndef MOE_GM
#define MOE_GM 8   // m-blocks per tile chunk
#endif

__device__ __forceinline__ int xcd_tile(int L, int n) {
  // workgroups are handed to the 8 XCDs round-robin by linear id: give XCD x
  // the contiguous tile range [start(x), start(x + 1))
  const int q = n >> 3, r = n & 7, x = L & 7;
  return x * q + (x < r ? x : r) + (L >> 3);
}

// [rs, re): the maximal run of m-blocks around mb0 (below vb) that hold the
// same expert id; wave-uniform, 64 ids per probe.
__device__ __forceinline__ void expert_run(const int* __restrict__ expert_ids, int mb0, int vb,
                                           int lane, int& rs, int& re) {
  const int e0 = expert_ids[mb0];
  for (int base = mb0 - 1;; base -= 64) {
    const int idx = base - lane;
    const bool stop = idx < 0 || expert_ids[idx < 0 ? 0 : idx] != e0;
    const uint64_t b = __ballot(stop);
    if (b) { rs = base - (int)__builtin_ctzll(b) + 1; break; }
  }
  for (int base = mb0 + 1;; base += 64) {
    const int idx = base + lane;
    const bool stop = idx >= vb || expert_ids[idx >= vb ? mb0 : idx] != e0;
    const uint64_t b = __ballot(stop);
    if (b) { re = base + (int)__builtin_ctzll(b); break; }
  }
}

// BM token rows x BNW weight rows per workgroup tile, WAVES_M x WAVES_N waves,
// BK-wide K steps, NS LDS stages (direct path: loads for step kt + NS - 1 are
// issued while step kt is computed), MINW waves per SIMD requested (the launch bound).
// SW: the tile's first BNW/2 weight rows are gate rows n0.., the rest the up
// rows I+n0.. of the same act columns, and the epilogue is SwiGLU.
template <int BM, int BNW, int WAVES_M, int WAVES_N, bool SW, int BK, int NS, int MINW>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, MINW) grouped_gemm_kernel(GemmParams pin) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;   // threads of the workgroup
  constexpr int CPR = BK / 8;
  constexpr int WM = BM / WAVES_M;
  constexpr int MT = WM >= 32 ? 32 : 16;
  typedef Mfma<MT> M;
  constexpr int KSTEPS = BK / (MT == 32 ? 16 : 32);
  constexpr int WNW = BNW / WAVES_N;
  constexpr int FM = WM / MT;
  constexpr int FN = WNW / MT;
  constexpr int XL = (BM * CPR + NT - 1) / NT;
  constexpr int WL = BNW * CPR / NT;
  static_assert(WAVES_M * WAVES_N >= 4 && WAVES_M * WAVES_N <= 8, "4 to 8 waves");
  static_assert(!SW || FN % 2 == 0, "SwiGLU pairs gate and up subtiles");
  static_assert(BNW * CPR % NT == 0, "weight tile load");
  static_assert(KSTEPS >= 1, "K step");

  // LDS stages (loads run NS - 1 K steps ahead)
  constexpr int NBUF = NS;
  static_assert(NS >= 2, "the load pipeline needs two or more stages");
  __shared__ u32x4 sX[NBUF][BM * CPR];
  __shared__ u32x4 sW[NBUF][BNW * CPR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int wn = wave % WAVES_N;
  const int wm = wave / WAVES_N;

  // ---- tile of this workgroup: XCD-contiguous; the tiles of each expert's
  // run of m-blocks are consecutive, in chunks of GM m-blocks with the n-tile
  // outer, so that neighbouring workgroups share weight tiles and token rows
  const int ntn = pin.ntiles_n;
  GemmParams p = pin;
  int mb, nt;
  const uint16_t* We;
  int64_t a_bytes, w_bytes;   // bytes the A / W descriptors may reach
  if (pin.nseg > 0) {
    // segmented reduction: segment s is a dense product over its own columns
    const int per = ntn * pin.mblocks;
    const int tg = xcd_tile(blockIdx.x, per * pin.nseg);
    const int sg = tg / per, r = tg - sg * per;
    mb = r % pin.mblocks;
    nt = r / pin.mblocks;
    const int beg = pin.seg_beg[sg];
    p.K = pin.seg_end[sg] - beg;
    p.A = pin.A + beg;
    We = pin.W + beg;
    p.C = (char*)pin.C + sg * pin.seg_c_stride * (pin.c_fp32 ? 4 : 2);
    a_bytes = ((int64_t)p.a_rows * p.lda - beg) * 2;
    w_bytes = ((int64_t)p.N * p.ldw - beg) * 2;
  } else {
    // only the tiles of m-blocks that hold rows are mapped (the grid is sized
    // for the align capacity): workgroups past them exit, and since the
    // workgroups go to the XCDs round-robin, every XCD gets an equal share
    const int vbr = min(pin.mblocks, ((pin.ntpp ? *pin.ntpp : pin.M) + BM - 1) / BM);
    const int nvalid = ntn * (vbr + pin.nsb);
    if ((int)blockIdx.x >= nvalid) return;
    const int tg = xcd_tile(blockIdx.x, nvalid);
    // tiles past the routed ones belong to the dense second part
    const bool second = tg >= ntn * vbr;
    if (second) {
      p.A = pin.A2;
      p.W = pin.W2;
      p.E = 1;
      p.a_row_div = 0;
      p.sorted_ids = nullptr;
      p.expert_ids = nullptr;
      p.ntpp = nullptr;
      p.M = pin.M2;
      p.a_rows = pin.M2;
      p.C = pin.C2;
      p.c_row_offset = pin.c2_row_offset;
      p.topk_w = nullptr;
    }
    const int nmb = second ? pin.nsb : vbr;
    const int t = second ? tg - ntn * vbr : tg;
    const int total_rows = p.ntpp ? *p.ntpp : p.M;
    const int vb = min(nmb, (total_rows + BM - 1) / BM);   // m-blocks holding rows
    const int mb0 = t / ntn;
    if (mb0 >= vb) return;
    int rs = 0, re = vb;
    if (p.expert_ids) expert_run(p.expert_ids, mb0, vb, lane, rs, re);
    constexpr int GM = MOE_GM;
    const int jr = t - rs * ntn;
    const int grp = jr / (GM * ntn);
    const int gsz = min(GM, re - rs - grp * GM);
    const int j = jr - grp * GM * ntn;
    mb = rs + grp * GM + j % gsz;
    nt = j / gsz;
    const int e = p.expert_ids ? p.expert_ids[mb] : 0;
    if (e < 0 || e >= p.E) return;
    We = p.W + (int64_t)e * p.N * p.ldw;
    a_bytes = (int64_t)p.a_rows * p.lda * 2;
    w_bytes = (int64_t)p.N * p.ldw * 2;
  }
  const int m0 = mb * BM;
  const int ncols = SW ? p.I : p.N;           // output columns
  const int n0 = nt * (SW ? BNW / 2 : BNW);

  // kNoRow: an offset beyond every descriptor even after the K advance is
  // added, so the load reads zeros
  constexpr int kNoRow = 0x7fff0000;

  // ---- direct-to-LDS: lane l of a wave load fills LDS unit (base + l); the
  // unit at (row r, position pos) holds global chunk pos ^ mask(r), so the
  // source offsets carry the swizzle and each row's lanes still read one line
  int xdo[XL], wdo[WL];
  {
#pragma unroll
    for (int q = 0; q < XL; ++q) {
      const int u = tid + NT * q;
      const int r = u / CPR;
      const int c = (u % CPR) ^ ((r / (16 / CPR)) % CPR);
      xdo[q] = kNoRow;
      if (u < BM * CPR) {
        const int i = m0 + r;
        int arow = -1;
        if (p.sorted_ids) {
          const int sid = p.sorted_ids[i];
          if (sid >= 0 && sid < p.num_valid) arow = p.a_row_div ? sid / p.a_row_div : i;
        } else if (i < p.M) {
          arow = i;
        }
        if (arow >= 0) xdo[q] = arow * p.lda * 2 + c * 16;
      }
    }
#pragma unroll
    for (int q = 0; q < WL; ++q) {
      const int u = tid + NT * q;
      const int r = u / CPR;
      const int c = (u % CPR) ^ ((r / (16 / CPR)) % CPR);
      int g;
      bool ok;
      if (SW) {
        const int cc = r < BNW / 2 ? n0 + r : n0 + r - BNW / 2;
        ok = cc < p.I;
        g = r < BNW / 2 ? cc : p.I + cc;
      } else {
        g = n0 + r;
        ok = g < p.N;
      }
      wdo[q] = ok ? g * p.ldw * 2 + c * 16 : kNoRow;
    }
  }

  // ---- LDS read addresses: every operand row a lane reads is row(lane) plus
  // a multiple of 16, which keeps the swizzle mask of row(lane); so per
  // k-substep one base index per operand and compile-time subtile offsets
  constexpr int WNA = SW ? BNW / 2 / WAVES_N : WNW;
  int xb[KSTEPS], wb[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    const int lr = M::row(lane);
    const int lb = swz<CPR>(lr, M::chunk(kk, lane));
    xb[kk] = lb + wm * WM * CPR;
    wb[kk] = lb + wn * WNA * CPR;
  }
  // weight subtile f starts this many rows after the wave's first weight row
  auto wsub_off = [&](int f) {
    if (SW) return f < FN / 2 ? f * MT : BNW / 2 + (f - FN / 2) * MT;
    return f * MT;
  };

  typename M::acc_t acc[FN][FM];
#pragma unroll
  for (int f = 0; f < FN; ++f)
#pragma unroll
    for (int q = 0; q < FM; ++q)
#pragma unroll
      for (int v = 0; v < M::kVals; ++v) acc[f][q][v] = 0.f;

  // direct-to-LDS loads of K step kt into LDS buffer b.  Issued from inline
  // asm (buffer_load_dwordx4 ... lds; M0 holds the wave's LDS destination and
  // is restored) so that the compiler, which cannot tell the in-flight
  // transfers from the LDS reads of other buffers, does not wait for all of
  // them before every read; completion is awaited explicitly (vmcnt) before
  // the barrier that publishes a step.  The asm writes no register.
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  auto rsrc4 = [](const void* base, int64_t bytes) {
    const uint64_t a = (uint64_t)base;
    return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
  };
  const i32x4 xr4 = rsrc4(p.A, a_bytes);
  const i32x4 wr4 = rsrc4(We, w_bytes);
  auto dma1 = [](const i32x4& rs, const void* lds, int voff, int soff) {
    const unsigned la = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
    int m0save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(m0save)
        : "s"(la), "v"(voff), "s"(rs), "s"(soff)
        : "memory");
  };
  // this wave issues the last of the XL token-row loads (waves past the end of
  // the token tile skip it)
  const bool x_wave = NT * (XL - 1) + 64 * wave < BM * CPR;
  // load i (of XL + WL per thread) of K step kt into LDS buffer b: the first
  // XL are token-row chunks, the rest weight-row chunks; the ragged last K
  // step (tail) masks the 16-byte chunks beyond K
  auto dma_one = [&](auto tail_c, int kt, int b, int i) {
    constexpr bool tail = decltype(tail_c)::value;
    const int k0 = kt * BK;
    const bool is_x = i < XL;
    const int q = is_x ? i : i - XL;
    if (is_x && NT * q + 64 * wave >= BM * CPR) return;   // wave-uniform
    const int u = tid + NT * q;
    int off = is_x ? xdo[is_x ? q : 0] : wdo[is_x ? 0 : q], soff = k0 * 2;
    if constexpr (tail) {
      const int c = (u % CPR) ^ ((u / CPR / (16 / CPR)) % CPR);
      off = (k0 + c * 8 < p.K && off != kNoRow) ? off + k0 * 2 : kNoRow;
      soff = 0;
    }
    if (is_x) dma1(xr4, sX[b] + NT * q + 64 * wave, off, soff);
    else dma1(wr4, sW[b] + NT * q + 64 * wave, off, soff);
  };
  // one whole K step of direct loads into LDS buffer b
  auto dma_step = [&](auto tail_c, int kt, int b) {
#pragma unroll
    for (int i = 0; i < XL + WL; ++i) dma_one(tail_c, kt, b, i);
  };
  auto dma = [&](int kt, int b) {
    if ((kt + 1) * BK > p.K) dma_step(std::true_type{}, kt, b);
    else dma_step(std::false_type{}, kt, b);
  };
  // operand registers of one k-substep
  struct Ops {
    bf16x8 b[FM], a[FN];
  };
  auto read_ops = [&](const u32x4* sx, const u32x4* sw, int kk, Ops& o) {
#pragma unroll
    for (int q = 0; q < FM; ++q) o.b[q] = __builtin_bit_cast(bf16x8, sx[xb[kk] + q * MT * CPR]);
#pragma unroll
    for (int f = 0; f < FN; ++f) o.a[f] = __builtin_bit_cast(bf16x8, sw[wb[kk] + wsub_off(f) * CPR]);
  };
  // the MFMAs of substep kk with this thread's loads of a later K step spread
  // between them: load i follows MFMA i * TM / ND of the step, so the address
  // queue drains while the matrix cores work
  auto mfmas_spread = [&](const Ops& o, int kk, auto&& load_i) {
    constexpr int TM = KSTEPS * FN * FM;
    constexpr int ND = XL + WL;
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int q = 0; q < FM; ++q) {
        acc[f][q] = M::run(o.a[f], o.b[q], acc[f][q]);
        const int m = (kk * FN + f) * FM + q;
#pragma unroll
        for (int i = 0; i < ND; ++i)
          if (i * TM / ND == m) load_i(i);
      }
  };

  // ---- pipeline over K steps, one barrier per step.
  // NBUF = NS buffers, D = NS - 1: step kt computes from buffer
  // kt % NBUF while its MFMAs interleave the loads of step kt + D into the
  // buffer that step kt - 1 used (every wave is past the barrier that ended
  // step kt - 1); then each thread waits for its own loads of step kt + 1 and
  // the barrier makes them visible to all waves.
  const int nk = (p.K + BK - 1) / BK;
  {
    // vmcnt(n) with the other counters left alone; n = loads one thread
    // issues per K step (a compile-time count per kind of wave)
    constexpr int NXW = XL + WL;
    constexpr int NW = WL + XL - 1;
    static_assert((BM * CPR - NT * (XL - 1)) % 64 == 0, "the last token-row load is whole waves");
    constexpr int D = NBUF - 1;   // prefetch distance in K steps
    static_assert((D - 1) * NXW <= 63, "vmcnt range");
    // wait until this thread's loads of the oldest pending step have landed;
    // in steady state D - 1 later steps stay in flight (a compile-time count
    // per kind of wave), near the end of K everything is waited for
#define MOE_VMW(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
    auto wait_steady = [&]() {
      if (x_wave) MOE_VMW((D - 1) * NXW); else MOE_VMW((D - 1) * NW);
    };
    auto wait_all = [&]() { MOE_VMW(0); };
#undef MOE_VMW
    for (int st = 0; st < D; ++st)
      if (st < nk) dma(st, st);
    if (nk > D - 1) wait_steady(); else wait_all();
    __builtin_amdgcn_s_barrier();
    int b0 = 0;
    for (int kt = 0; kt < nk; ++kt) {
      const int bd = b0 == 0 ? NBUF - 1 : b0 - 1;   // (kt + D) % NBUF
      // 0: no load this step, 1: a full K step, 2: the ragged last K step
      const int dmode = kt + D < nk ? ((kt + D + 1) * BK > p.K ? 2 : 1) : 0;
      auto load_i = [&](int i) {
        if (dmode == 1) dma_one(std::false_type{}, kt + D, bd, i);
        else if (dmode == 2) dma_one(std::true_type{}, kt + D, bd, i);
      };
      const u32x4* const rx = sX[b0];
      const u32x4* const rw = sW[b0];
      Ops sa, sb;
      read_ops(rx, rw, 0, sa);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; kk += 2) {
        if (kk + 1 < KSTEPS) read_ops(rx, rw, kk + 1, sb);
        mfmas_spread(sa, kk, load_i);
        if (kk + 2 < KSTEPS) read_ops(rx, rw, kk + 2, sa);
        if (kk + 1 < KSTEPS) mfmas_spread(sb, kk + 1, load_i);
      }
      if (kt + 1 < nk) {
        // this thread's part of step kt + 1 has landed; steps kt + 2 .. kt + D
        // (those issued) may still be in flight
        if (kt + D <= nk - 1) wait_steady(); else wait_all();
        __builtin_amdgcn_s_barrier();
      }
      b0 = b0 == NBUF - 1 ? 0 : b0 + 1;
    }
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
          const float h = acc[f][q][4 * g + v];
          if (SW) {
            const float u = acc[f + FN / 2][q][4 * g + v];
            o[v] = silu(h) * u;
          } else if (epi == 2) {
            const float r = fmaxf(h, 0.f);
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

template <int BM, int BNW, int WAVES_M, int WAVES_N, int BK, int NS, int MINW>
hipError_t launch_bm(GemmParams p, hipStream_t s) {
  const bool sw = p.epi == 1;
  const int ncols = sw ? p.I : p.N;
  const int tile_n = sw ? BNW / 2 : BNW;
  p.mblocks = (p.M + BM - 1) / BM;
  p.nsb = p.M2 > 0 ? (p.M2 + BM - 1) / BM : 0;
  p.ntiles_n = (ncols + tile_n - 1) / tile_n;
  if (p.nseg > 0) p.nsb = 0;
  const int64_t nwg = (int64_t)(p.mblocks + p.nsb) * p.ntiles_n * (p.nseg > 0 ? p.nseg : 1);
  if (nwg == 0) return hipSuccess;
  if (sw)
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BNW, WAVES_M, WAVES_N, true, BK, NS, MINW>),
                       dim3((unsigned)nwg), dim3(64 * WAVES_M * WAVES_N), 0, s, p);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BNW, WAVES_M, WAVES_N, false, BK, NS, MINW>),
                       dim3((unsigned)nwg), dim3(64 * WAVES_M * WAVES_N), 0, s, p);
  return hipGetLastError();
}

}  // namespace

// Tile configurations per BLOCK_M (compile-time knobs, defaults tuned on MI355X):
// BM, BNW, WAVES_M, WAVES_N, BK, NS, MINW.
#ifndef MOE_G128
#define MOE_G128 128, 256, 2, 4, 64, 3, 1
#endif
#ifndef MOE_G64
#define MOE_G64 64, 256, 2, 4, 64, 2, 4
#endif
#ifndef MOE_G32
#define MOE_G32 32, 256, 2, 4, 64, 2, 4
#endif
#ifndef MOE_G16
#define MOE_G16 16, 128, 1, 4, 64, 3, 2
#endif

hipError_t launch_grouped_gemm(const GemmParams& p, int block_m, hipStream_t s) {
  switch (block_m) {
    case 128: return launch_bm<MOE_G128>(p, s);
    case 64: return launch_bm<MOE_G64>(p, s);
    case 32: return launch_bm<MOE_G32>(p, s);
    case 16: return launch_bm<MOE_G16>(p, s);
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
