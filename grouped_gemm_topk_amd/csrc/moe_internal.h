// Internal declarations of libmoe: kernel parameter blocks and launchers.
// Host code (moe_api.cpp) validates arguments and carves the workspace; the
// .hip files own the kernels and expose one launcher per kernel family.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 256;

// The grouped GEMM's "no row" load offset: a masked load (pad row, ragged K
// tail, columns past N) reads zeros because this offset lies at or beyond the
// end of its buffer descriptor.  The host therefore accepts operand buffers
// (token rows, activation rows, one expert's weights) of fewer bytes than this.
constexpr int kNoRowOffset = 0x7fff0000;

// ---------------------------------------------------------------- gating
struct GateParams {
  const float* logits;  // [T, E]
  int T, E, k;
  int scoring;          // 0 softmax, 1 sigmoid
  int n_group, topk_group;
  int renorm;
  float scale;
  int* topk_ids;        // [T, k]
  float* topk_w;        // [T, k]
};

// ---------------------------------------------------------------- align
struct AlignParams {
  const int* topk_ids;  // [n]
  int n;                // T * k
  int E;
  int block_m;
  int* sorted_ids;      // [capacity]
  int* expert_ids;      // [capacity / block_m]
  int* ntpp;            // [1]
  int* block_counts;    // workspace [nblocks, E] (two-kernel path)
  int nblocks;          // chunks (workgroups) of the two-kernel path
  int chunk;            // slots per chunk
};

constexpr int kAlignMinChunk = 1024;    // slots per workgroup of the two-kernel path, at least
constexpr int kAlignMaxChunks = 64;     // workgroups of the two-kernel path, at most
constexpr int kSingleBlockSlots = 1024; // at most this many slots: one workgroup does it all
constexpr int kRouteFusedTokens = 64;   // gating fused into the one-workgroup align up to this T

// ---------------------------------------------------------------- grouped GEMM
struct GemmParams {
  const uint16_t* A;        // bf16 rows of K elements
  int a_row_div;            // >0: A row = sid / a_row_div; 0: A row = padded position
  const uint16_t* W;        // bf16 [E, N, K] (or one matrix when expert_ids is null)
  int E, N, K;
  int I;                    // SwiGLU: act columns (= N / 2); else N
  const int* sorted_ids;    // null: dense rows (row i is A row i, valid when i < M)
  const int* expert_ids;    // null: expert 0
  const int* ntpp;          // null: M rows in total
  int M;                    // dense mode: number of rows; routed: capacity
  int num_valid;            // pad threshold of sorted ids
  int epi;                  // 0 store, 1 swiglu, 2 relu2, 3 weighted scatter
  const float* topk_w;      // weighted scatter: routed weight per slot (null: 1)
  void* C;
  int c_fp32;
  int64_t c_row_offset;     // weighted scatter: added to the destination row
  int ldc;                  // output row stride in elements
  int a_rows;               // rows of A (bounds of its buffer descriptor)
  // optional dense second part with the same N, K and epilogue (the shared
  // expert): M2 token rows of A2 times W2 [N, K] into C2 (store epilogues: row
  // = token; weighted scatter: row c2_row_offset + token, weight 1).  Its
  // tiles follow the routed ones in the same launch.  M2 = 0: none.
  const uint16_t* A2;
  const uint16_t* W2;
  int M2;
  void* C2;
  int64_t c2_row_offset;
  int mblocks, nsb, ntiles_n;   // tile grid: routed and second-part m-blocks (set by the launcher)
  // row strides (elements) of A and W; the forward uses K for both
  int lda, ldw;
  // segmented reduction (nseg > 0): nseg independent dense products, segment s
  // reducing over columns [seg_beg[s], seg_end[s]) of A and W (K is ignored)
  // into C + s * seg_c_stride elements; no gather, no second part
  int nseg;
  const int* seg_beg;
  const int* seg_end;
  int64_t seg_c_stride;
  // one workgroup per tile instead of the persistent grid of the 128- and
  // 256-row tiles (same results; for comparisons)
  int per_tile;
  // set by the launcher: 1 in a persistent 256-row launch, which then runs a
  // last round filling at most a quarter of its grid with each of those tiles
  // cut into tail_s slices; main_grid = the persistent grid, main_tile_n =
  // the tile width in output columns
  int tail, tail_s, main_grid, main_tile_n;
};

// ---------------------------------------------------------------- decode GEMVs
constexpr int kGemvMaxTokens = 16;     // T at or below this takes the GEMV path

struct GemvParams {
  const uint16_t* x;        // [T, H]
  const float* logits;      // [T, E]
  const uint16_t* w13;      // [E, M1, H]
  const uint16_t* w2;       // [E, H, I]
  const uint16_t* sw13;     // shared expert [M1, H] or null
  const uint16_t* sw2;      // shared expert [H, I] or null
  // MXFP8 weights (mx = 1): the four matrices above hold FP8 E4M3 bytes and
  // these their E8M0 scales, one per 32 elements along each row
  int mx;
  const uint8_t* w13_s;     // [E, M1, H / 32]
  const uint8_t* w2_s;      // [E, H, I / 32]
  const uint8_t* sw13_s;    // [M1, H / 32] or null
  const uint8_t* sw2_s;     // [H, I / 32] or null
  // routing outputs: written by GEMV1's workgroup (0,0), read by GEMV2
  int* topk_ids;            // [T * k]
  float* topk_w;            // [T * k]
  int* sorted_ids;          // [capacity]
  int* expert_ids;          // [capacity / bm]
  int* ntpp;                // [1]
  int T, H, I, k, E, bm;
  int nblk;                 // routed blocks that can exist: min(E, T * k)
  int scoring, n_group, topk_group, renorm;
  float scale;
  int nt1, nt2;             // 16-row tiles per workgroup of GEMV1 / GEMV2 (set by the launcher)
  uint16_t* act;            // [capacity, I] rows in padded order
  uint16_t* act_sh;         // [T, I]
  float* out;               // [T, H], zeroed by GEMV1 or the route kernel, accumulated by the W2 GEMV
  int* ctl;                 // control block of the decode kernel (workspace, reset every call)
  int* status;              // the layer's status word: 0, or 1 when a bounded wait expired
};

hipError_t launch_gemv(const GemvParams& p, bool swiglu, hipStream_t s);

hipError_t launch_gate(const GateParams& p, hipStream_t s);
hipError_t launch_route_fused(const GateParams& g, const AlignParams& a, hipStream_t s);
// logits = x . router_w^T (written to `logits`, [T, E] fp32); with `gate`
// also the gating of every token (g.topk_ids / g.topk_w); g.logits is ignored
hipError_t launch_router(const GateParams& g, const uint16_t* x, const uint16_t* router_w, int H,
                         float* logits, bool gate, hipStream_t s);
hipError_t launch_align(const AlignParams& p, hipStream_t s);
hipError_t launch_grouped_gemm(const GemmParams& p, int block_m, hipStream_t s);
// bf16 [B, R, C] -> [B, C, R] (R and C multiples of 8)
hipError_t launch_transpose(const uint16_t* src, uint16_t* dst, int B, int R, int C, hipStream_t s);
// dst [C, ld] column j = row of src for padded position j < *ntpp: row
// sorted[j] / div (sorted[j] < num_valid) or zeros (a pad); C multiple of 8
hipError_t launch_gather_transpose(const uint16_t* src, int C, const int* sorted, const int* ntpp,
                                   int num_valid, int div, int cap, uint16_t* dst, int ld,
                                   hipStream_t s);
// seg_beg / seg_end of every expert's run of blocks in the aligned layout
// (padded positions; both 0 for an expert without blocks)
hipError_t launch_seg_table(const int* expert_ids, const int* ntpp, int block_m, int E,
                            int* seg_beg, int* seg_end, hipStream_t s);
// The no-allocation entry point's workspace: a static device array of this
// many bytes per GPU; *ptr = the current device's copy (its address is
// looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(void** ptr);

// also clears the layer's status word (`status`, may be null): the prefill
// path has no cross-workgroup waits
hipError_t launch_combine(const float* yslot, int T, int k, int H, int has_shared, float* out,
                          int* status, hipStream_t s);

}  // namespace moe
