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
// conflicts.  Tiles are numbered XCD by XCD (each XCD gets an equal,
// contiguous range of the tiles whose m-blocks hold rows) and, inside a
// range, the tiles of one expert's run of M-blocks are consecutive, in chunks
// of 8 M-blocks per N-tile, so that a weight tile and the token rows are
// reused from that XCD's L2 (the L2 grouping / cache-aware scheduling of the
// skill card's *Optimization Patterns*).  With the 128- and 256-row tiles
// the grid is one workgroup per CU and each workgroup runs a sequence of
// tiles; the expert ids of the m-blocks sit in LDS for the tile mapping.  The
// 128-row tile (three LDS stages) splits its waves: eight compute waves
// multiply out of LDS and write the tiles, eight loader waves issue every
// direct load, two K steps ahead, in one sequence across the tile boundaries,
// so the compute waves' stores never wait in a load counter.  The 256-row
// tile (two stages, no room for loader waves' registers) has every wave load
// and compute: between two tiles it requests the next tile's first K step
// and then writes the finished tile while it is in flight, and the global
// reads a tile's set-up needs (sorted token ids, routed weights) are issued a
// tile ahead.  v_mfma_f32_32x32x16_bf16 is used when a wave owns >= 32 token
// rows, v_mfma_f32_16x16x32_bf16 for BLOCK_M = 16.
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));



// silu(z) = z * sigmoid(z) with the hardware reciprocal (the result is rounded
// to bf16 next)
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

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

// m-blocks per tile chunk of the tile order (4: zipf128 1 % faster than 8,
// the other layers the same; 2 and 16 slower)
#ifndef MOE_GM
#define MOE_GM 4
#endif
#ifndef MOE_PC
#define MOE_PC 1   // loader / compute split for persistent 128-row tiles
#endif
#ifndef MOE_NLW
#define MOE_NLW 8   // loader waves of the split
#endif

__device__ __forceinline__ int xcd_tile(int L, int n) {
  // workgroups are handed to the 8 XCDs round-robin by linear id: give XCD x
  // the contiguous tile range [start(x), start(x + 1))
  const int q = n >> 3, r = n & 7, x = L & 7;
  return x * q + (x < r ? x : r) + (L >> 3);
}

// [rs, re): the maximal run of m-blocks around mb0 (below vb) that hold the
// expert e0 = id(mb0); wave-uniform, 64 ids per probe (both directions'
// first probes read together); id(i) gives the expert id of m-block i.
template <typename Id>
__device__ __forceinline__ void expert_run(Id id, int mb0, int vb, int lane, int e0, int& rs,
                                           int& re) {
  auto probe_lo = [&](int base, int v) { const int i = base - lane; return i < 0 || v != e0; };
  auto probe_hi = [&](int base, int v) { const int i = base + lane; return i >= vb || v != e0; };
  auto at = [&](int i) { return id(i < 0 ? 0 : (i >= vb ? mb0 : i)); };
  int lo = mb0 - 1, hi = mb0 + 1;
  const int vlo = at(lo - lane), vhi = at(hi + lane);
  uint64_t b = __ballot(probe_lo(lo, vlo));
  while (!b) {
    lo -= 64;
    b = __ballot(probe_lo(lo, at(lo - lane)));
  }
  rs = lo - (int)__builtin_ctzll(b) + 1;
  b = __ballot(probe_hi(hi, vhi));
  while (!b) {
    hi += 64;
    b = __ballot(probe_hi(hi, at(hi + lane)));
  }
  re = hi + (int)__builtin_ctzll(b);
}

// expert ids kept in LDS by the 128-row tile (its three stages leave 16 KB of
// the 160 KB; the smaller tiles run two workgroups per CU and keep none)
template <int BM>
constexpr int kEidsLds = BM >= 128 ? 2048 : 0;

// BM token rows x BNW weight rows per workgroup tile, WAVES_M x WAVES_N waves,
// BK-wide K steps, NS LDS stages (direct path: loads for step kt + NS - 1 are
// issued while step kt is computed), MINW waves per SIMD requested (the launch bound).
// SW: the tile's first BNW/2 weight rows are gate rows n0.., the rest the up
// rows I+n0.. of the same act columns, and the epilogue is SwiGLU.
// WNT: weight rows are loaded with the non-temporal hint (see launch_bm).
// PC: MOE_NLW more waves (loader waves) issue every direct load and the
// WAVES_M x WAVES_N waves only compute and store (see the PC branch below).
// LDS bytes of one tile configuration's body: its stages, the expert-id copy
// and (loader / compute split) the sorted-id buffers of the loader waves
template <int BM, int BNW, int BK, int NS, bool PC>
constexpr int kBodyLds = NS * (BM + BNW) * (BK / 8) * 16 + kEidsLds<BM> * 4 + (PC ? 4 * BM * 4 : 0);

// One tile configuration's work in a launch; the kernel below runs it once,
// or (the 256 x 256 tile) twice.  tail_mode: 0 all tiles of the launch, 1 its
// full rounds, 2 the slices of its last round (see nrun); lds: the
// workgroup's LDS, kBodyLds bytes of it used.
template <int BM, int BNW, int WAVES_M, int WAVES_N, bool SW, int BK, int NS, bool WNT, bool PC>
__device__ __forceinline__ void gemm_body(const GemmParams& pin, const int tail_mode,
                                          unsigned char* lds) {
  constexpr int NCW = WAVES_M * WAVES_N;        // compute waves
  constexpr int NT = 64 * (NCW + (PC ? MOE_NLW : 0));   // threads of the workgroup
  constexpr int LT = PC ? 64 * MOE_NLW : NT;            // threads that issue direct loads
  constexpr int CPR = BK / 8;
  constexpr int WM = BM / WAVES_M;
  constexpr int MT = WM >= 32 ? 32 : 16;
  typedef Mfma<MT> M;
  constexpr int KSTEPS = BK / (MT == 32 ? 16 : 32);
  constexpr int WNW = BNW / WAVES_N;
  constexpr int FM = WM / MT;
  constexpr int FN = WNW / MT;
  constexpr int XL = (BM * CPR + LT - 1) / LT;
  constexpr int WL = BNW * CPR / LT;
  static_assert(NCW >= 4 && NCW <= 8, "4 to 8 compute waves");
  static_assert(!SW || FN % 2 == 0, "SwiGLU pairs gate and up subtiles");
  static_assert(BNW * CPR % LT == 0, "weight tile load");
  static_assert(KSTEPS >= 1, "K step");

  // LDS stages (loads run NS - 1 K steps ahead)
  constexpr int NBUF = NS;
  static_assert(NS >= 2, "the load pipeline needs two or more stages");
  typedef u32x4 XStage[BM * CPR];
  typedef u32x4 WStage[BNW * CPR];
  XStage* const sX = reinterpret_cast<XStage*>(lds);
  WStage* const sW = reinterpret_cast<WStage*>(lds + NBUF * BM * CPR * 16);
  unsigned char* const lds_rest = lds + NBUF * (BM + BNW) * CPR * 16;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int wn = wave % WAVES_N;
  const int wm = wave / WAVES_N;
  // the loader threads: all of them, or the loader waves after the compute waves
  const int ltid = PC ? tid - 64 * NCW : tid;
  const int lwave = PC ? wave - NCW : wave;

  // ---- the tiles of this launch.  Tiles are numbered XCD by XCD: tile L of
  // the launch's sequence goes to XCD L mod 8 (the order in which workgroups
  // are handed to the XCDs), and each XCD owns an equal, contiguous range of
  // tile indices.  Inside a range the tiles of each expert's run of m-blocks
  // are consecutive, in chunks of GM m-blocks with the n-tile outer, so that
  // the workgroups running at the same time on one XCD share weight tiles and
  // token rows in its L2.  Only the tiles of m-blocks that hold rows are
  // numbered (the grid is sized for the align capacity).  A workgroup runs
  // tiles blockIdx.x, blockIdx.x + gridDim.x, ... (the grid is one workgroup
  // per CU when it has more tiles than that).  Between two tiles it requests
  // the next tile's first K steps and writes the finished tile while they are
  // in flight; the global reads a tile's set-up needs (sorted token ids,
  // routed weights) are issued one tile ahead, so they land with those loads.
  const int ntn = pin.ntiles_n;
  int vbr = 0, nvalid;
  if (pin.nseg > 0) {
    nvalid = ntn * pin.mblocks * pin.nseg;
  } else {
    vbr = min(pin.mblocks, ((pin.ntpp ? *pin.ntpp : pin.M) + BM - 1) / BM);
    nvalid = ntn * (vbr + pin.nsb);
  }
  // nrun: the launch-sequence indices this pass runs.  In a persistent
  // launch whose last round would fill at most a quarter of the grid, the
  // pass over the full tiles stops after its full rounds (tail mode 1), and
  // a second pass (tail mode 2, see grouped_gemm_kernel) runs the tiles of
  // that round cut into tail_s slices of its own, narrower tile width, one
  // per workgroup, so that the last round's few tiles are spread over the CUs.
  // (A quarter: the slices then fit in one round.  On the dsv3 layer's W2, a
  // last round of 44 tiles took 72 us and its 176 slices take 43 us; two
  // rounds of slices would cost about what a half-full last round does.)
  int nrun = nvalid, tail_base = 0;
  if (tail_mode) {
    const int gm = pin.main_grid;
    const int rem = nvalid % gm;
    const bool split = nvalid > gm && rem > 0 && 4 * rem <= gm;
    if (tail_mode == 1) {
      if (split) nrun = nvalid - rem;
    } else {
      if (!split) return;
      tail_base = nvalid - rem;
      // one slice per workgroup (see resolve): this workgroup's slice exists
      // when its tile does
      const int i = ((int)blockIdx.x >> 3) / pin.tail_s;
      if ((((int)blockIdx.x - tail_base) & 7) + 8 * i >= rem) return;
      nrun = (int)blockIdx.x + 1;
    }
  }
  if ((int)blockIdx.x >= nrun) return;
  const int G = gridDim.x;
  const int ncols = SW ? pin.I : pin.N;   // output columns
  constexpr int GM = MOE_GM;
  // kNoRow: an offset beyond every descriptor (the host keeps operand buffers
  // below it) even after the K advance is added, so the load reads zeros
  constexpr int kNoRow = kNoRowOffset;

  // the expert ids of the routed m-blocks, copied to LDS once per workgroup
  // (every tile's mapping reads them) when the tile's LDS leaves room
  typedef __attribute__((address_space(3))) int lds_int;
  lds_int* s_eids = nullptr;
  if constexpr (kEidsLds<BM> > 0) s_eids = (lds_int*)lds_rest;
  const bool eids_lds = kEidsLds<BM> > 0 && pin.nseg == 0 && pin.expert_ids && vbr <= kEidsLds<BM>;
  if (eids_lds) {
    for (int i = tid; i < vbr; i += NT) s_eids[i] = pin.expert_ids[i];
    __syncthreads();
  }
  auto eid = [&](int i) -> int {
    if (eids_lds) return s_eids[i];
    return pin.expert_ids[i];
  };

  // a tile's place: m-block, n-tile, expert (the segment in segmented launches)
  struct Map {
    int mb, nt, e;
    int slice;            // slice of the n-tile (tail mode 2)
    bool second, store;   // dense second part; false only for an invalid expert id
  };
  auto resolve = [&](int Lt) -> Map {
    Map m;
    m.store = true;
    m.second = false;
    m.slice = 0;
    if (tail_mode == 2) {
      // a slice of a tile of the last round.  Workgroup Lt runs
      // on XCD Lt mod 8: it takes a tile whose launch index is numbered for
      // that XCD (index tail_base + j with j = Lt - tail_base mod 8), so that
      // the slices of one tile, which read the same token rows, and the
      // neighbouring tiles of that XCD's range share its L2
      const int r = Lt >> 3, i = r / pin.tail_s;
      m.slice = r - i * pin.tail_s;
      Lt = tail_base + ((Lt - tail_base) & 7) + 8 * i;
    }
    const int tg = xcd_tile(Lt, nvalid);
    if (pin.nseg > 0) {
      // segmented reduction: segment s is a dense product over its own columns
      const int per = ntn * pin.mblocks;
      const int sg = tg / per, r = tg - sg * per;
      m.mb = r % pin.mblocks;
      m.nt = r / pin.mblocks;
      m.e = sg;
      return m;
    }
    // tiles past the routed ones belong to the dense second part
    m.second = tg >= ntn * vbr;
    const int vb = m.second ? pin.nsb : vbr;
    const int tl = m.second ? tg - ntn * vbr : tg;
    const int mb0 = tl / ntn;   // < vb for every numbered tile
    int rs = 0, re = vb, e = 0;
    if (!m.second && pin.expert_ids) {
      e = eid(mb0);   // the expert of the whole run
      expert_run(eid, mb0, vb, lane, e, rs, re);
    }
    const int jr = tl - rs * ntn;
    const int grp = jr / (GM * ntn);
    const int gsz = min(GM, re - rs - grp * GM);
    const int j = jr - grp * GM * ntn;
    m.mb = rs + grp * GM + j % gsz;
    m.nt = j / gsz;
    if (!m.second && (e < 0 || e >= pin.E)) {   // computed, not written
      m.store = false;
      e = 0;
    }
    m.e = e;
    return m;
  };

  // what a tile's loads and stores use
  struct Tile {
    const uint16_t* A;        // token rows (at the segment's first column)
    const uint16_t* W;        // this tile's expert weights
    char* C;                  // output base
    const int* sorted;        // sorted token ids (nullptr: rows in order)
    const float* topk_w;      // routed weights of the scatter epilogue
    int64_t c_row_offset, a_bytes, w_bytes;
    int a_row_div, M, K, m0, n0;
    bool store;
  };
  auto tile_of = [&](const Map& m) -> Tile {
    Tile t;
    t.store = m.store;
    t.m0 = m.mb * BM;
    t.n0 = tail_mode == 2 ? m.nt * pin.main_tile_n + m.slice * (SW ? BNW / 2 : BNW)
                          : m.nt * (SW ? BNW / 2 : BNW);
    t.K = pin.K;
    if (pin.nseg > 0) {
      const int beg = pin.seg_beg[m.e];
      t.K = pin.seg_end[m.e] - beg;
      t.A = pin.A + beg;
      t.W = pin.W + beg;
      t.C = (char*)pin.C + m.e * pin.seg_c_stride * (pin.c_fp32 ? 4 : 2);
      t.sorted = pin.sorted_ids;
      t.topk_w = pin.topk_w;
      t.c_row_offset = pin.c_row_offset;
      t.a_row_div = pin.a_row_div;
      t.M = pin.M;
      t.a_bytes = ((int64_t)pin.a_rows * pin.lda - beg) * 2;
      t.w_bytes = ((int64_t)pin.N * pin.ldw - beg) * 2;
    } else if (m.second) {
      t.A = pin.A2;
      t.W = pin.W2;
      t.C = (char*)pin.C2;
      t.sorted = nullptr;
      t.topk_w = nullptr;
      t.c_row_offset = pin.c2_row_offset;
      t.a_row_div = 0;
      t.M = pin.M2;
      t.a_bytes = (int64_t)pin.M2 * pin.lda * 2;
      t.w_bytes = (int64_t)pin.N * pin.ldw * 2;
    } else {
      t.A = pin.A;
      t.W = pin.W + (int64_t)m.e * pin.N * pin.ldw;
      t.C = (char*)pin.C;
      t.sorted = pin.sorted_ids;
      t.topk_w = pin.topk_w;
      t.c_row_offset = pin.c_row_offset;
      t.a_row_div = pin.a_row_div;
      t.M = pin.M;
      t.a_bytes = (int64_t)pin.a_rows * pin.lda * 2;
      t.w_bytes = (int64_t)pin.N * pin.ldw * 2;
    }
    return t;
  };

  // sorted ids of the token rows this thread loads (XL) and of the rows its
  // lane writes (FM): global reads, issued a tile ahead
  auto load_ids = [&](const Tile& t, int* xs, int* es) {
#pragma unroll
    for (int q = 0; q < XL; ++q) {
      const int u = ltid + LT * q;
      const int i = t.m0 + u / CPR;
      xs[q] = (u < BM * CPR && t.sorted) ? t.sorted[i] : i;
    }
#pragma unroll
    for (int q = 0; q < FM; ++q) {
      const int i = t.m0 + wm * WM + q * MT + M::out_col(lane);
      es[q] = t.sorted ? t.sorted[i] : i;
    }
  };

  // direct-to-LDS source offsets: lane l of a wave load fills LDS unit
  // (base + l); the unit at (row r, position pos) holds global chunk
  // pos ^ mask(r), so the offsets carry the swizzle and each row's lanes still
  // read one line
  auto offsets = [&](const Tile& t, const int* xs, int* xdo, int* wdo) {
#pragma unroll
    for (int q = 0; q < XL; ++q) {
      const int u = ltid + LT * q;
      const int r = u / CPR;
      const int c = (u % CPR) ^ ((r / (16 / CPR)) % CPR);
      xdo[q] = kNoRow;
      if (u < BM * CPR) {
        const int i = t.m0 + r;
        int arow = -1;
        if (t.sorted) {
          const int sid = xs[q];
          if (sid >= 0 && sid < pin.num_valid) arow = t.a_row_div ? sid / t.a_row_div : i;
        } else if (i < t.M) {
          arow = i;
        }
        if (arow >= 0) xdo[q] = arow * pin.lda * 2 + c * 16;
      }
    }
#pragma unroll
    for (int q = 0; q < WL; ++q) {
      const int u = ltid + LT * q;
      const int r = u / CPR;
      const int c = (u % CPR) ^ ((r / (16 / CPR)) % CPR);
      int g;
      bool ok;
      if (SW) {
        const int cc = r < BNW / 2 ? t.n0 + r : t.n0 + r - BNW / 2;
        ok = cc < pin.I;
        g = r < BNW / 2 ? cc : pin.I + cc;
      } else {
        g = t.n0 + r;
        ok = g < pin.N;
      }
      wdo[q] = ok ? g * pin.ldw * 2 + c * 16 : kNoRow;
    }
  };

  // epilogue rows of this lane (the q-th MFMA column block): output row,
  // whether it is written, and its routed weight (read a tile ahead)
  const int epi = pin.epi;
  struct EpiRows {
    int64_t orow[FM];
    int sid[FM];
    bool ok[FM];
  };
  auto epi_rows = [&](const Tile& t, const int* es, EpiRows& er) {
#pragma unroll
    for (int q = 0; q < FM; ++q) {
      const int i = t.m0 + wm * WM + q * MT + M::out_col(lane);
      if (epi == 3) {
        const int sid = es[q];
        const bool ok = t.sorted ? (sid >= 0 && sid < pin.num_valid) : i < t.M;
        er.sid[q] = sid;
        er.orow[q] = t.c_row_offset + sid;
        er.ok[q] = ok && t.store;
      } else {
        er.sid[q] = i;
        er.ok[q] = (t.sorted ? true : i < t.M) && t.store;
        er.orow[q] = i;
      }
    }
  };
  auto load_scale = [&](const Tile& t, const EpiRows& er, float* sc) {
#pragma unroll
    for (int q = 0; q < FM; ++q)
      sc[q] = (epi == 3 && t.topk_w && er.ok[q]) ? t.topk_w[er.sid[q]] : 1.f;
  };

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

  // direct-to-LDS loads of K step kt into LDS buffer b.  Issued from inline
  // asm (buffer_load_dwordx4 ... lds; M0 holds the wave's LDS destination and
  // is restored) so that the compiler, which cannot tell the in-flight
  // transfers from the LDS reads of other buffers, does not wait for all of
  // them before every read; completion is awaited explicitly (vmcnt) before
  // the barrier that publishes a step.  The asm writes no register.  Ordinary
  // loads (tile setup, epilogue rows) are waited for explicitly before the
  // next direct loads are issued, so that no wait the compiler places for
  // them falls inside the pipeline.
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  // (the words are made wave-uniform explicitly: the asm takes them in SGPRs)
  auto rsrc4 = [](const void* base, int64_t bytes) {
    const uint64_t a = (uint64_t)base;
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
                 __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
  };
  // la: LDS byte address of the wave's 64 destination units (wave-uniform:
  // each wave fills its own block of units)
  auto dma1 = [](const i32x4& rs, unsigned la, int voff, int soff) {
    const unsigned l = la;
    const int so = soff;
    int m0save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(m0save)
        : "s"(l), "v"(voff), "s"(rs), "s"(so)
        : "memory");
  };
  // weight rows with the non-temporal hint (WNT launches: every expert holds
  // about one m-block, so each weight tile is read by one tile only and
  // should not displace the token rows from the caches)
  auto dma1_nt = [](const i32x4& rs, unsigned la, int voff, int soff) {
    const unsigned l = la;
    const int so = soff;
    int m0save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen nt lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(m0save)
        : "s"(l), "v"(voff), "s"(rs), "s"(so)
        : "memory");
  };
  typedef const __attribute__((address_space(3))) void* lds_cptr;
  const unsigned lds_x = (unsigned)(uintptr_t)(lds_cptr)&sX[0][0];
  const unsigned lds_w = (unsigned)(uintptr_t)(lds_cptr)&sW[0][0];
  // vmcnt(n) with the other counters left alone
#define MOE_VMW(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

  // the loader thread's direct-load offsets and buffer descriptors for the
  // tile it is loading
  int xdo[XL], wdo[WL];
  i32x4 xr4, wr4;
  int K = pin.K;

  // this wave issues the last of the XL token-row loads (waves past the end of
  // the token tile skip it)
  const bool x_wave = LT * (XL - 1) + 64 * lwave < BM * CPR;
  // load i (of XL + WL per thread) of K step kt into LDS buffer b: the first
  // XL are token-row chunks, the rest weight-row chunks; the ragged last K
  // step (tail) masks the 16-byte chunks beyond K
  auto dma_one = [&](auto tail_c, int kt, int b, int i) {
    constexpr bool tail = decltype(tail_c)::value;
    const int k0 = kt * BK;
    const bool is_x = i < XL;
    const int q = is_x ? i : i - XL;
    if (is_x && LT * q + 64 * lwave >= BM * CPR) return;   // wave-uniform
    const int u = ltid + LT * q;
    int off = is_x ? xdo[is_x ? q : 0] : wdo[is_x ? 0 : q], soff = k0 * 2;
    if constexpr (tail) {
      const int c = (u % CPR) ^ ((u / CPR / (16 / CPR)) % CPR);
      off = (k0 + c * 8 < K && off != kNoRow) ? off + k0 * 2 : kNoRow;
      soff = 0;
    }
    const unsigned unit = (unsigned)(LT * q + 64 * lwave);
    if (is_x) dma1(xr4, lds_x + (unsigned)((b * BM * CPR + unit) * 16), off, soff);
    else if constexpr (WNT) dma1_nt(wr4, lds_w + (unsigned)((b * BNW * CPR + unit) * 16), off, soff);
    else dma1(wr4, lds_w + (unsigned)((b * BNW * CPR + unit) * 16), off, soff);
  };
  // the direct loads [i0, i1) of K step kt into LDS buffer b (all of them:
  // [0, XL + WL); the weight chunks alone: [XL, XL + WL))
  auto dma_part = [&](int kt, int b, int i0, int i1) {
    const bool tail = (kt + 1) * BK > K;
#pragma unroll
    for (int i = 0; i < XL + WL; ++i) {
      if (i < i0 || i >= i1) continue;
      if (tail) dma_one(std::true_type{}, kt, b, i);
      else dma_one(std::false_type{}, kt, b, i);
    }
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
  // queue drains while the matrix cores work (the 256-row tile, one step
  // ahead only, issues them within the first quarter of the step's MFMAs:
  // 2-4 % faster than across the whole step)
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
          if (i * TM / (BM == 256 ? 4 * ND : ND) == m) load_i(i);
      }
  };

  // ---- pipeline over K steps, one barrier per step.
  // NBUF = NS buffers, D = NS - 1: step kt computes from buffer b0 while its
  // MFMAs interleave the loads of step kt + D into the buffer that step
  // kt - 1 used (every wave is past the barrier that ended step kt - 1); then
  // each thread waits for its own loads of step kt + 1 and the barrier makes
  // them visible to all waves.  The ring continues from tile to tile: the next
  // tile's first D steps go to the D buffers the last step did not read.
  constexpr int NXW = XL + WL;
  constexpr int NW = WL + XL - 1;
  static_assert((BM * CPR - LT * (XL - 1)) % 64 == 0, "the last token-row load is whole waves");
  constexpr int D = NBUF - 1;   // prefetch distance in K steps
  static_assert((D - 1) * NXW <= 63, "vmcnt range");
  // wait until this thread's loads of the oldest pending step have landed;
  // in steady state D - 1 later steps stay in flight (a compile-time count
  // per kind of wave), near the end of K everything is waited for
  auto wait_steady = [&]() {
    if (x_wave) MOE_VMW((D - 1) * NXW); else MOE_VMW((D - 1) * NW);
  };
  auto wait_all = [&]() { MOE_VMW(0); };
  // the first D steps of the current tile into buffers b, b + 1, ...: the
  // weight chunks first (they need no token index)
  auto first_steps = [&](int b, int nk) {
    for (int st = 0; st < D; ++st)
      if (st < nk) dma_part(st, (b + st) % NBUF, XL, XL + WL);
    for (int st = 0; st < D; ++st)
      if (st < nk) dma_part(st, (b + st) % NBUF, 0, XL);
  };

  // the epilogue of a finished tile: activation or routed-weight scale, then
  // the stores of this lane's outputs
  auto epilogue = [&](const Tile& done, const EpiRows& der, const float* dsc) {
#pragma unroll
    for (int q = 0; q < FM; ++q) {
      if (!der.ok[q]) continue;
      const int64_t orow = der.orow[q];
      const float scale = dsc[q];
      constexpr int FO = SW ? FN / 2 : FN;
#pragma unroll
      for (int f = 0; f < FO; ++f) {
        const int colbase = SW ? done.n0 + wn * (BNW / 2 / WAVES_N) + f * MT : done.n0 + wn * WNW + f * MT;
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
          if (pin.c_fp32) {
            float4* dst = (float4*)((float*)done.C + orow * pin.ldc + col);
            *dst = make_float4(o[0], o[1], o[2], o[3]);
          } else {
            const bf16x2 lo = {(__bf16)o[0], (__bf16)o[1]}, hi = {(__bf16)o[2], (__bf16)o[3]};
            uint2 pk;
            pk.x = __builtin_bit_cast(unsigned, lo);
            pk.y = __builtin_bit_cast(unsigned, hi);
            *(uint2*)((uint16_t*)done.C + orow * pin.ldc + col) = pk;
          }
        }
      }
    }
  };
  auto zero_acc = [&]() {
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int q = 0; q < FM; ++q)
#pragma unroll
        for (int v = 0; v < M::kVals; ++v) acc[f][q][v] = 0.f;
  };

  if constexpr (PC) {
    // ---- loader / compute split.  Every tile of the launch has the same K,
    // so the workgroup's work is C = (its tiles) x nk K steps in one sequence,
    // and cycle c ends with barrier c.  In cycle c the compute waves multiply
    // step c out of LDS buffer c mod 3; the loader waves issue all loads of
    // step c + 2 at once into the buffer step c - 1 used (every compute wave
    // is past barrier c - 1, so done reading it), wait until their loads of
    // step c + 1 have landed and meet the compute waves at barrier c.  The
    // sequence runs on across tile boundaries: the loads of the next tile's
    // first steps are in flight while the compute waves finish a tile and
    // write it.  The compute waves issue no direct loads and wait for no
    // load counter in the K loop, so their stores never hold up the pipeline;
    // the loader waves' counter holds their direct loads only, so the waits
    // are compile-time counts.
    static_assert(D == 2 && XL * LT == BM * CPR, "loader split: three stages, whole loads");
    constexpr int NL = XL + WL;   // direct loads per loader thread and K step
    // the sorted token ids of tile j, which the loader threads need for their
    // row offsets, are read by the compute waves with ordinary loads and put
    // in s_ids[j mod R] during the epilogue of tile j - J, and read by the
    // loader waves in cycle j * nk - 2; J keeps that at least one barrier
    // after the write, and R >= J keeps a buffer from being rewritten before
    // it was read
    constexpr int R = 4;
    int (*const s_ids)[BM] = reinterpret_cast<int (*)[BM]>(lds_rest + kEidsLds<BM> * 4);
    const int L0 = blockIdx.x;
    const int ntl = (nrun - L0 + G - 1) / G;   // tiles of this workgroup (>= 1)
    const int nk = (K + BK - 1) / BK;
    const int C = ntl * nk;
    const int J = nk >= 3 ? 2 : (nk == 2 ? 3 : 4);   // (J - 1) * nk >= 3, J <= R
    auto tile_at = [&](int i) { return tile_of(resolve(L0 + i * G)); };
    // a barrier the compiler moves no memory access across; the compute
    // waves' LDS writes (the ids) have completed before they reach it
    auto bar = [] {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    auto bar_c = [&] {
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), the other counters left alone
      bar();
    };

    if (wave >= NCW) {
      // ---- loader waves
      auto setup = [&](int i) {
        const Tile t = tile_at(i);
        int xs[XL];
#pragma unroll
        for (int q = 0; q < XL; ++q) xs[q] = t.sorted ? s_ids[i % R][(ltid + LT * q) / CPR] : 0;
        offsets(t, xs, xdo, wdo);
        xr4 = rsrc4(t.A, t.a_bytes);
        wr4 = rsrc4(t.W, t.w_bytes);
      };
      // (the descriptors are wave-uniform, but carried around the loop the
      // compiler no longer knows it: made uniform again before each step)
      auto unif = [](i32x4& v) {
#pragma unroll
        for (int w = 0; w < 4; ++w) v[w] = __builtin_amdgcn_readfirstlane(v[w]);
      };
      auto issue = [&](int st) {   // all loads of step st of the sequence
        const int i = st / nk, kt = st - i * nk;
        if (kt == 0) setup(i);
        unif(xr4);
        unif(wr4);
        dma_part(kt, st % NBUF, 0, NL);
      };
      bar();   // the first tiles' ids are in LDS
      const int np = C < 2 ? C : 2;
      for (int st = 0; st < np; ++st) issue(st);
      if (np == 2) MOE_VMW(NL); else MOE_VMW(0);
      bar();
      for (int c = 0; c < C; ++c) {
        if (c + 2 < C) {
          issue(c + 2);
          MOE_VMW(NL);   // step c + 1 has landed; step c + 2 may be in flight
        } else if (c + 1 < C) {
          MOE_VMW(0);
        }
        bar();
      }
    } else {
      // ---- compute waves
      auto load_es = [&](const Tile& t, int* es) {
#pragma unroll
        for (int q = 0; q < FM; ++q) {
          const int i = t.m0 + wm * WM + q * MT + M::out_col(lane);
          es[q] = t.sorted ? t.sorted[i] : i;
        }
      };
      auto load_ids_of = [&](int j) -> int {   // thread tid < BM: tile j's row tid
        const Tile t = tile_at(j);
        return (tid < BM && t.sorted) ? t.sorted[t.m0 + tid] : 0;
      };
      Tile tc = tile_at(0), tn = tc;
      int es[FM];
      EpiRows er;
      float sc[FM];
      load_es(tc, es);
      epi_rows(tc, es, er);
      load_scale(tc, er, sc);
      if (ntl > 1) {
        tn = tile_at(1);
        load_es(tn, es);
      }
      for (int j = 0; j < J && j < ntl; ++j) {
        const int v = load_ids_of(j);
        if (tid < BM) s_ids[j % R][tid] = v;
      }
      int pid = J < ntl ? load_ids_of(J) : 0;
      bar_c();   // the first tiles' ids are in LDS
      bar();     // the first step has landed
      auto noload = [](int) {};
      int b0 = 0;
      for (int i = 0; i < ntl; ++i) {
        zero_acc();
        for (int kt = 0; kt < nk; ++kt) {
          const u32x4* const rx = sX[b0];
          const u32x4* const rw = sW[b0];
          Ops sa, sb;
          read_ops(rx, rw, 0, sa);
#pragma unroll
          for (int kk = 0; kk < KSTEPS; kk += 2) {
            if (kk + 1 < KSTEPS) read_ops(rx, rw, kk + 1, sb);
            mfmas_spread(sa, kk, noload);
            if (kk + 2 < KSTEPS) read_ops(rx, rw, kk + 2, sa);
            if (kk + 1 < KSTEPS) mfmas_spread(sb, kk + 1, noload);
          }
          bar_c();
          b0 = b0 == NBUF - 1 ? 0 : b0 + 1;
        }
        epilogue(tc, er, sc);
        if (i + 1 < ntl) {
          // tile i + 1's epilogue rows and routed weights, tile i + 2's rows,
          // and the sorted ids the loader waves need J tiles ahead
          tc = tn;
          epi_rows(tc, es, er);
          load_scale(tc, er, sc);
          if (i + 2 < ntl) {
            tn = tile_at(i + 2);
            load_es(tn, es);
          }
          if (i + J < ntl) {
            if (tid < BM) s_ids[(i + J) % R][tid] = pid;
            if (i + J + 1 < ntl) pid = load_ids_of(i + J + 1);
          }
        }
      }
    }
  } else {
    // the first tile, set up in full
    int L = blockIdx.x;
    Tile cur = tile_of(resolve(L));
    int xs[XL], es[FM];
    load_ids(cur, xs, es);
    MOE_VMW(0);
    EpiRows er;
    float sc[FM];
    offsets(cur, xs, xdo, wdo);
    epi_rows(cur, es, er);
    load_scale(cur, er, sc);
    xr4 = rsrc4(cur.A, cur.a_bytes);
    wr4 = rsrc4(cur.W, cur.w_bytes);
    K = cur.K;

    int b0 = 0;
    first_steps(0, (K + BK - 1) / BK);
    // the second tile: mapping and row ids
    int Ln = L + G;
    Tile nxt = cur;
    if (Ln < nrun) {
      nxt = tile_of(resolve(Ln));
      load_ids(nxt, xs, es);
    }
    wait_all();
    __builtin_amdgcn_s_barrier();
    for (;;) {
      const int nk = (K + BK - 1) / BK;
      zero_acc();
      for (int kt = 0; kt < nk; ++kt) {
        const int bd = b0 == 0 ? NBUF - 1 : b0 - 1;   // the buffer of step kt + D
        // 0: no load this step, 1: a full K step, 2: the ragged last K step
        const int dmode = kt + D < nk ? ((kt + D + 1) * BK > K ? 2 : 1) : 0;
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

      // ---- between tiles (the same K: segmented launches run one tile per
      // workgroup).  No direct load is in flight here, so waiting for the reads
      // issued a tile ago costs nothing.
      MOE_VMW(0);
      const Tile done = cur;
      const EpiRows der = er;
      float dsc[FM];
  #pragma unroll
      for (int q = 0; q < FM; ++q) dsc[q] = sc[q];
      const bool more = Ln < nrun;
      if (more) {
        // the next tile: its first D steps, then its routed weights
        cur = nxt;
        offsets(cur, xs, xdo, wdo);
        epi_rows(cur, es, er);
        xr4 = rsrc4(cur.A, cur.a_bytes);
        wr4 = rsrc4(cur.W, cur.w_bytes);
        K = cur.K;
        first_steps(b0, (K + BK - 1) / BK);
        load_scale(cur, er, sc);
        // the tile after it: mapping and row ids
        Ln += G;
        if (Ln < nrun) {
          nxt = tile_of(resolve(Ln));
          load_ids(nxt, xs, es);
        }
      }

      // ---- epilogue of the finished tile
      epilogue(done, der, dsc);
      if (!more) break;
      // the next tile's first steps (and this tile's stores) have landed
      wait_all();
      __builtin_amdgcn_s_barrier();
    }
  }
#undef MOE_VMW
}

// The grouped GEMM kernel: one tile configuration's work (gemm_body).  A
// persistent 256 x 256 launch whose last round would fill at most a quarter
// of the grid runs its full rounds and then, in the same launch, the tiles of
// that round cut into slices of 64 weight rows (32 act columns with SwiGLU)
// on eight waves of 32-row MFMA blocks, so every output is the same bit for
// bit as with the whole tiles; a workgroup takes its slice as soon as its
// full rounds are done.
template <int BM, int BNW, int WAVES_M, int WAVES_N, bool SW, int BK, int NS, int MINW,
          bool WNT = false, bool PC = false>
__global__ void __launch_bounds__(64 * (WAVES_M * WAVES_N + (PC ? MOE_NLW : 0)), MINW)
    grouped_gemm_kernel(GemmParams pin) {
  constexpr bool SLICES = BM == 256 && BNW == 256 && !PC && WAVES_M * WAVES_N == 8;
  constexpr int MAIN_LDS = kBodyLds<BM, BNW, BK, NS, PC>;
  constexpr int SLICE_LDS = SLICES ? kBodyLds<BM, 64, BK, 3, false> : 0;
  __shared__ __attribute__((aligned(16))) unsigned char lds[MAIN_LDS > SLICE_LDS ? MAIN_LDS : SLICE_LDS];
  gemm_body<BM, BNW, WAVES_M, WAVES_N, SW, BK, NS, WNT, PC>(pin, pin.tail, lds);
  if constexpr (SLICES) {
    if (pin.tail == 1) {
      __syncthreads();   // every wave is done with the stages of its last tile
      gemm_body<BM, 64, BM / 32, 1, SW, BK, 3, false, false>(pin, 2, lds);
    }
  }
}

// compute units of the current device (cached per device, safe to call from
// several host threads; 0 if unknown)
int cu_count() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// the main launch of launch_bm: the kernel instantiation for the tile and
// its epilogue, non-temporal weights and the loader / compute split
template <int BM, int BNW, int WAVES_M, int WAVES_N, int BK, int NS, int MINW>
hipError_t launch_main(const GemmParams& p, dim3 grid, dim3 block, bool sw, bool wnt, hipStream_t s) {
  if constexpr (BM == 128 && NS == 3) {
    // persistent 128-row tiles with one K: the loader / compute split
    if (p.nseg == 0 && MOE_PC && !p.per_tile) {
      const dim3 block_pc(64 * (WAVES_M * WAVES_N + MOE_NLW));
      if (wnt && sw)
        hipLaunchKernelGGL((grouped_gemm_kernel<BM, BNW, WAVES_M, WAVES_N, true, BK, NS, MINW, true, true>),
                           grid, block_pc, 0, s, p);
      else if (wnt)
        hipLaunchKernelGGL((grouped_gemm_kernel<BM, BNW, WAVES_M, WAVES_N, false, BK, NS, MINW, true, true>),
                           grid, block_pc, 0, s, p);
      else if (sw)
        hipLaunchKernelGGL((grouped_gemm_kernel<BM, BNW, WAVES_M, WAVES_N, true, BK, NS, MINW, false, true>),
                           grid, block_pc, 0, s, p);
      else
        hipLaunchKernelGGL((grouped_gemm_kernel<BM, BNW, WAVES_M, WAVES_N, false, BK, NS, MINW, false, true>),
                           grid, block_pc, 0, s, p);
      return hipGetLastError();
    }
  }
  if (wnt && sw)
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BNW, WAVES_M, WAVES_N, true, BK, NS, MINW, BM == 128>),
                       grid, block, 0, s, p);
  else if (wnt)
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BNW, WAVES_M, WAVES_N, false, BK, NS, MINW, BM == 128>),
                       grid, block, 0, s, p);
  else if (sw)
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BNW, WAVES_M, WAVES_N, true, BK, NS, MINW>), grid,
                       block, 0, s, p);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BNW, WAVES_M, WAVES_N, false, BK, NS, MINW>), grid,
                       block, 0, s, p);
  return hipGetLastError();
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
  int64_t nwg = (int64_t)(p.mblocks + p.nsb) * p.ntiles_n * (p.nseg > 0 ? p.nseg : 1);
  if (nwg == 0) return hipSuccess;
  // one workgroup per CU (the LDS of the 128- and 256-row tiles admits no second one),
  // each running tiles gridDim.x apart; the CU count is a multiple of 8, so a
  // workgroup stays on the XCD its tiles are numbered for.  Segmented launches
  // (the weight gradient, one segment per expert) too: their tiles' K differ
  // from segment to segment and the single-role loop takes each tile's own
  // (the weight gradient at the axolotl table's shapes: 2-10 % faster)
  bool persistent = false;
  if (BM >= 128 && !p.per_tile) {
    const int ncu = cu_count();
    if (ncu > 0 && ncu % 8 == 0 && nwg > ncu) {
      nwg = ncu;
      persistent = true;
    }
  }
  // The last-round slices (see grouped_gemm_kernel) pay with 256-row tiles
  // only: with 128-row tiles the main launch's last round is short and
  // overlaps the tile before it, and the split cost 2-3 %.  The grid is a
  // multiple of 32: the last round's at most nwg / 4 tiles, at most nwg / 32
  // per XCD, each in tail_s slices on its XCD's nwg / 8 workgroups.
  p.tail = persistent && BM == 256 && p.nseg == 0 && nwg % 32 == 0 ? 1 : 0;
  p.main_grid = (int)nwg;
  p.main_tile_n = tile_n;
  p.tail_s = tile_n / (sw ? 32 : 64);   // slices of 64 weight rows
  // Experts that hold on average at most one m-block (T * top_k <= E * BM)
  // use each weight tile in one tile only: with no dense second part (whose
  // weights every m-block reads), the 128-row tile then streams its weight
  // rows non-temporally, which keeps the token rows cached (relu2 at T = 2048,
  // 128 experts top-6: 620 -> 589 us per layer; where experts hold several
  // m-blocks the hint costs 6-10 %, so it is not used there)
  const bool wnt = BM == 128 && p.nseg == 0 && p.M2 == 0 && p.expert_ids &&
                   (int64_t)p.num_valid <= (int64_t)p.E * BM;
  const dim3 grid((unsigned)nwg), block(64 * WAVES_M * WAVES_N);
  return launch_main<BM, BNW, WAVES_M, WAVES_N, BK, NS, MINW>(p, grid, block, sw, wnt, s);
}

}  // namespace

// Tile configurations per BLOCK_M (compile-time knobs, defaults tuned on MI355X):
// BM, BNW, WAVES_M, WAVES_N, BK, NS, MINW.  (The 256-row tile's waves as 4 x 2,
// each 64 token rows x 128 weight rows: the dsv3 layer 1-3 % faster than 2 x 4;
// 8 x 1 needs all 256 VGPRs and spills, 4 % slower.)
#ifndef MOE_G256
#define MOE_G256 256, 256, 4, 2, 64, 2, 1
#endif
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
    case 256: return launch_bm<MOE_G256>(p, s);
    case 128: return launch_bm<MOE_G128>(p, s);
    case 64: return launch_bm<MOE_G64>(p, s);
    case 32: return launch_bm<MOE_G32>(p, s);
    case 16: return launch_bm<MOE_G16>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// out[t] = sum_j yslot[t*k + j] (+ yslot[T*k + t] for the shared expert), in j order.
// The per-slot rows are read once, with the non-temporal hint: kept out of the
// caches they leave the next kernels' weights and token rows there (zipf128,
// 738 MB of rows: 166 -> 128 us; the dsv3 layer 2 % faster in all).  A
// token's k <= 16 row loads are all issued before the sums (about 1 % more at
// dsv3 than one load per iteration).
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ yslot, int T, int k,
                                                      int H, int has_shared, float* __restrict__ out,
                                                      int* __restrict__ status) {
  if (status && blockIdx.x == 0 && threadIdx.x == 0) *status = 0;
  const int h4 = H / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * h4) return;
  const int t = (int)(idx / h4);
  const int c = (int)(idx % h4) * 4;
  auto row = [&](int64_t r) {
    return __builtin_nontemporal_load((const f32x4*)(yslot + r * H + c));
  };
  f32x4 y[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < k) y[j] = row((int64_t)t * k + j);
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < k) a += y[j];
  for (int j = 16; j < k; ++j) a += row((int64_t)t * k + j);   // (the ABI caps top_k at 16)
  if (has_shared) a += row((int64_t)T * k + t);
  *(f32x4*)(out + (int64_t)t * H + c) = a;
}

hipError_t launch_combine(const float* yslot, int T, int k, int H, int has_shared, float* out,
                          int* status, hipStream_t s) {
  int64_t n = (int64_t)T * (H / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, yslot, T, k,
                     H, has_shared, out, status);
  return hipGetLastError();
}

}  // namespace moe
