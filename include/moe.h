/*
 * libmoe — fused Mixture-of-Experts forward for AMD Instinct MI355X (gfx950).
 *
 * The problem statement follows the fused-MoE recipe of the "Fused Moe Kernel"
 * skill card (zjli2013/fused-moe-kernel), sections *Token-Expert Routing*,
 * *Grouped GEMM Structure* and *Common Pitfalls*: top-k gating, sorting the
 * token slots by expert with every expert padded to a multiple of BLOCK_M,
 * then a tiled grouped GEMM that reaches its token rows through
 * `sorted_token_ids` and its weight matrix through `expert_ids`, skipping
 * blocks at or beyond `num_tokens_post_padded`.  The expert MLP is SwiGLU
 * (silu of the gate rows times the up rows, as in the axolotl DeepSeek-V3 MoE
 * forward) or squared ReLU
 * (fc1 -> relu^2 -> fc2, mlxcel PR #280).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers, row-major with the innermost
 *   dimension contiguous, 16-byte aligned.  bf16 tensors are raw uint16 bit
 *   patterns.  `stream` is a hipStream_t (NULL = the default stream).
 * - The caller owns every buffer, including the workspace.  The library never
 *   allocates device memory, never synchronises the stream and never copies to
 *   the host.  All work is enqueued asynchronously on `stream`.
 * - Workspace (moe_align, moe_grouped_gemm_backward and the moe_fused_forward
 *   family): `workspace_bytes` must not be NULL.  With `workspace == NULL` the call only writes the required byte
 *   count (possibly 0) to `*workspace_bytes` and launches nothing; call again
 *   with a non-NULL buffer of at least that many bytes and its size in
 *   `*workspace_bytes`.  moe_grouped_gemm needs no workspace and ignores both
 *   arguments.
 * - Arguments are validated on the host before anything is launched; a
 *   negative status is returned and nothing is written.  There is no fallback
 *   path: an unsupported case is an error.  HIP failures are returned as
 *   MOE_ERR_HIP_BASE - (int)hipError_t.
 * - Slot s = t * top_k + j indexes the routing of token t to its j-th expert;
 *   num_valid = T * top_k.  Pad entries of `sorted_token_ids` equal num_valid.
 * - Calls on one stream are ordered; calls on different streams that share
 *   output or workspace buffers race.
 */
#ifndef LIBMOE_MOE_H
#define LIBMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,         /* a required pointer is NULL                        */
  MOE_ERR_SHAPE = -2,        /* a size is out of range or inconsistent            */
  MOE_ERR_CAPACITY = -3,     /* an output or the workspace is too small           */
  MOE_ERR_UNSUPPORTED = -4,  /* valid request this build does not implement       */
  MOE_ERR_ALIGN = -5,        /* a pointer is not 16-byte aligned                  */
  MOE_ERR_DEVICE = -6,       /* the current device is not a gfx950 GPU            */
  MOE_ERR_HIP_BASE = -1000
} moe_status;

enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };
enum { MOE_ACT_SWIGLU = 0, MOE_ACT_RELU2 = 1 };
enum { MOE_EPI_STORE = 0, MOE_EPI_SWIGLU = 1, MOE_EPI_RELU2 = 2, MOE_EPI_WEIGHTED_SCATTER = 3 };

/* Tile schedules of moe_grouped_gemm (same results, bit for bit): at
 * BLOCK_M 128 and 256 one workgroup per compute unit runs a sequence of tiles
 * (PERSISTENT, the default), or one workgroup per tile (PER_TILE; the
 * axolotl page's benchmark times its persistent and its non-persistent
 * kernels side by side).  At BLOCK_M 256 the persistent launch runs a last
 * round of tiles that fills at most a quarter of the grid in narrower slices
 * (same results), one per workgroup as its full rounds end. */
enum { MOE_SCHED_PERSISTENT = 0, MOE_SCHED_PER_TILE = 1 };

/* Limits enforced by validation. */
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 16

/* Padded-length bound of moe_align: round_up(T*k + min(E, T*k) * (bm - 1), bm).
 * Every expert wastes at most bm - 1 pad slots and at most min(E, T*k) experts
 * are non-empty. */
#define MOE_ALIGN_CAPACITY(T, k, E, bm)                                              \
  ((((int64_t)(T) * (k) + ((int64_t)(E) < (int64_t)(T) * (k) ? (int64_t)(E)        \
                                                             : (int64_t)(T) * (k)) * \
         ((bm) - 1)) + (bm) - 1) / (bm) * (bm))

/* Same bound as a function (for bindings that cannot expand macros). */
int64_t moe_align_capacity(int32_t T, int32_t k, int32_t E, int32_t block_m);

/*
 * moe_align — sort token slots by expert and pad every expert to a multiple of
 * block_m (skill card, *Token-Expert Routing* steps 2-3; the sorted-id /
 * expert-id / padded-count triple of *Grouped GEMM Structure*).
 *
 *   topk_ids                int32 [T, k]   expert of each slot, 0 <= id < E
 *   block_m                 16, 32, 64, 128 or 256
 *   sorted_token_ids  (out) int32 [capacity]: for expert e with c_e slots, its
 *                           padded range [o_e, o_e + p_e) (p_e = ceil(c_e/bm)*bm,
 *                           0 when c_e = 0; o_e = sum of p over lower experts)
 *                           holds the expert's slots in ascending order, then
 *                           num_valid for the pads.
 *   expert_ids        (out) int32 [capacity / block_m]: expert of each block.
 *   num_tokens_post_padded (out) int32 [1]: sum of p_e.
 *   capacity                entries of sorted_token_ids; must be at least
 *                           MOE_ALIGN_CAPACITY(T, k, E, block_m).
 * Entries at or beyond num_tokens_post_padded (or its block count) are left
 * unspecified.  Ids outside [0, E) are an error of the caller (they are
 * dropped and the output is then unspecified).  T = 0 writes 0 to
 * num_tokens_post_padded.
 */
int moe_align(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t block_m,
              int32_t* sorted_token_ids, int32_t* expert_ids,
              int32_t* num_tokens_post_padded, int64_t capacity, void* workspace,
              size_t* workspace_bytes, void* stream);

/*
 * One grouped GEMM over the aligned layout (skill card, *Grouped GEMM
 * Structure*; expert weights stacked [E, N, K], *Common Pitfalls* 3):
 *
 *   for padded row i < num_tokens_post_padded, e = expert_ids[i / block_m],
 *   s = sorted_token_ids[i], a = A[s / a_row_div] (a_row_div > 0) or A[i]
 *   (a_row_div == 0), h = a . W[e]^T (fp32 accumulation) and
 *     STORE            C[i] = h                                   (N columns)
 *     SWIGLU           C[i] = silu(h[:N/2]) * h[N/2:]             (N/2 columns)
 *     RELU2            C[i] = max(h, 0)^2                         (N columns)
 *     WEIGHTED_SCATTER C[s] = topk_weights[s] * h, only if s < num_valid
 *                      (topk_weights NULL: weight 1, a plain scatter by slot)
 *   Row-ordered epilogues (STORE/SWIGLU/RELU2) write zero rows for pads.
 *
 * With top_k = 1 (moe_align over per-row expert indices) and WEIGHTED_SCATTER
 * without weights this is the contiguous grouped GEMM of the axolotl page
 * (`cg_grouped_gemm_forward`: output row i = input row i times the transposed
 * weight of its expert), for any grouping of the rows.
 */
typedef struct {
  const void* a;           /* bf16 A rows, row stride K                                  */
  int32_t a_row_div;       /* top_k to gather token rows of x; 0 = A in padded order     */
  const void* w;           /* bf16 [E, N, K]                                             */
  int32_t E, N, K;         /* K multiple of 8; N multiple of 8 (of 16 for SWIGLU)        */
  const int32_t* sorted_token_ids;        /* from moe_align                              */
  const int32_t* expert_ids;              /* from moe_align                              */
  const int32_t* num_tokens_post_padded;  /* device scalar from moe_align                */
  int32_t block_m;         /* the block_m moe_align used                                 */
  int32_t num_valid;       /* T * top_k                                                  */
  int32_t capacity;        /* entries of sorted_token_ids (multiple of block_m)          */
  int32_t epilogue;        /* MOE_EPI_*                                                  */
  const float* topk_weights; /* [num_valid] for WEIGHTED_SCATTER, or NULL (weight 1)     */
  void* c;                 /* output rows: capacity rows (row-ordered) or num_valid rows */
  int32_t c_is_fp32;       /* 1: fp32 output, 0: bf16 (round to nearest even)            */
  int32_t schedule;        /* MOE_SCHED_*; 0 (the default) = persistent                  */
} moe_gemm_args;

int moe_grouped_gemm(const moe_gemm_args* args, void* workspace, size_t* workspace_bytes,
                     void* stream);

/*
 * Gradients of the indexed grouped GEMM out[i] = x[i] . w[idx[i]]^T (the
 * axolotl page's cg_backward.py: cg_grouped_gemm_backward_inputs and
 * cg_grouped_gemm_backward_weights), for an output gradient dy:
 *
 *   dx[i] = dy[i] . w[idx[i]]                                   [M, K]
 *   dw[e] = sum over rows i with idx[i] == e of dy[i]^T x[i]     [E, N, K]
 *           (zero for an expert without rows)
 *
 * fp32 accumulation; output bf16 (round to nearest even) or fp32.  The rows'
 * grouping is the aligned layout moe_align produces for the per-row expert
 * indices with top_k = 1 (T = M); any grouping works (empty experts,
 * non-contiguous indices).
 *
 * Arguments (device pointers, row-major, 16-byte aligned; bf16 = raw uint16):
 *   x   [M, K], w [E, N, K], dy [M, N]; K and N multiples of 8
 *   sorted_token_ids, expert_ids, num_tokens_post_padded, block_m, capacity:
 *       moe_align's outputs for the indices (capacity = the sorted ids'
 *       length, at least MOE_ALIGN_CAPACITY(M, 1, E, block_m))
 *   dx  [M, K] or NULL (not computed); dw [E, N, K] or NULL (not computed)
 *   out_fp32: 1 fp32 outputs, 0 bf16
 * Workspace (CUB convention; NULL = size query): the transposed weights for
 * dx (E * N * K bf16), and for dw the gathered, transposed dy and x in the
 * aligned order (N * capacity and K * capacity bf16) plus a per-expert table.
 * Errors: as moe_grouped_gemm; a transposed operand above 2 GiB returns
 * MOE_ERR_UNSUPPORTED.  M = 0 writes dw = 0 (when requested) and nothing else;
 * x, dy, w and sorted_token_ids may then be NULL.
 */
typedef struct {
  const void* x;
  const void* w;
  const void* dy;
  int32_t M, E, N, K;
  const int32_t* sorted_token_ids;
  const int32_t* expert_ids;
  const int32_t* num_tokens_post_padded;
  int32_t block_m;
  int32_t capacity;
  void* dx;
  void* dw;
  int32_t out_fp32;
} moe_gemm_backward_args;

int moe_grouped_gemm_backward(const moe_gemm_backward_args* args, void* workspace,
                              size_t* workspace_bytes, void* stream);

/*
 * The whole routed MoE layer: gating -> align -> GEMM1 + activation ->
 * GEMM2 + routed weight -> combine (the axolotl DeepSeek-V3 MoE forward
 * `_moe_triton_forward`, fused; the skill card's recipe end to end).
 */
typedef struct {
  int32_t T, H, I, E, top_k;
  int32_t block_m;        /* 16, 32, 64, 128 or 256                                       */
  int32_t scoring;        /* MOE_SCORE_SOFTMAX or MOE_SCORE_SIGMOID                       */
  int32_t n_group;        /* expert groups (1 = no grouping); E % n_group == 0            */
  int32_t topk_group;     /* groups kept per token                                        */
  int32_t renormalize;    /* 1: weights sum to 1 over the selected experts                */
  float routed_scaling_factor; /* multiplies the routed weights (1.0 = none)              */
  int32_t activation;     /* MOE_ACT_SWIGLU or MOE_ACT_RELU2                              */
  int32_t n_shared;       /* 0 or 1 always-on shared expert, weight 1                     */
} moe_layer_params;

/*
 * Gating (per token; ties broken toward the lower expert index):
 *   softmax scoring: experts ranked by logit; weight_j = exp(l_j - m) / sum over
 *     the selected set (renormalize) or over all experts; times the scale.
 *   sigmoid scoring: with n_group > 1, groups of E/n_group contiguous experts
 *     are ranked by the sum of their two largest sigmoids (fp64) and only the
 *     best topk_group groups stay candidates; experts ranked by logit; weight_j =
 *     sigmoid_j / sum over the selected set (renormalize) or sigmoid_j; times
 *     the scale.
 *
 *   x             bf16 [T, H]
 *   router_logits fp32 [T, E] (finite)
 *   w13           bf16 [E, M1, H]; SwiGLU: M1 = 2I, rows [0,I) gate, [I,2I) up;
 *                 relu^2: M1 = I
 *   w2            bf16 [E, H, I]
 *   shared_w13    bf16 [M1, H] and shared_w2 bf16 [H, I] when n_shared = 1
 *   out     (out) fp32 [T, H]
 *   topk_ids, topk_weights (optional out) int32 / fp32 [T, top_k]
 *   sorted_token_ids, expert_ids, num_tokens_post_padded (optional out): as
 *     moe_align, sized for MOE_ALIGN_CAPACITY(T, top_k, E, block_m)
 * Limits: 1 <= E <= 256, 1 <= top_k <= min(E, 16), H and I multiples of 8,
 * topk_group * E / n_group >= top_k.  T = 0 returns MOE_OK with nothing launched.
 */
int moe_fused_forward(const moe_layer_params* p, const void* x, const float* router_logits,
                      const void* w13, const void* w2, const void* shared_w13,
                      const void* shared_w2, float* out, int32_t* topk_ids,
                      float* topk_weights, int32_t* sorted_token_ids, int32_t* expert_ids,
                      int32_t* num_tokens_post_padded, void* workspace,
                      size_t* workspace_bytes, void* stream);

/*
 * The same layer with the router's linear layer fused into gating: the router
 * logits x . router_w^T (the HF gate the axolotl benchmark calls on the hidden
 * states, before the top-k) are formed with bf16 MFMAs and fp32 accumulation,
 * 16 tokens per workgroup.  For T > 16 the gating launch forms them, keeps
 * them on chip for the top-k and writes them out; for T <= 16 one small launch
 * (16 experts per workgroup) writes them and the decode path gates them as
 * moe_fused_forward does.  They go to router_logits_out ([T, E] fp32) when it
 * is not NULL, else to the workspace.  The routing is decided on those fp32
 * logits exactly as moe_fused_forward decides it on given logits.
 *   router_w [E, H] bf16, 16-byte aligned; everything else as moe_fused_forward
 * (same workspace size).  Errors: router_w NULL (MOE_ERR_NULL) or misaligned
 * (MOE_ERR_ALIGN), then as moe_fused_forward.
 */
int moe_fused_forward_router(const moe_layer_params* p, const void* x, const void* router_w,
                             float* router_logits_out, const void* w13, const void* w2,
                             const void* shared_w13, const void* shared_w2, float* out,
                             int32_t* topk_ids, float* topk_weights, int32_t* sorted_token_ids,
                             int32_t* expert_ids, int32_t* num_tokens_post_padded,
                             void* workspace, size_t* workspace_bytes, void* stream);

/*
 * The same layer with MXFP8 expert weights, for decode shapes (T <= 16), where
 * the layer reads each touched expert's weights from HBM once and halving the
 * bytes per weight halves that stream.  MXFP8 is the OCP Microscaling format:
 * FP8 E4M3 elements (bias 7, no infinities, S.1111.111 = NaN) in blocks of 32
 * consecutive elements along a row's contiguous dimension, each block with one
 * E8M0 scale byte s meaning 2^(s - 127).  Element value = E4M3 value * 2^(s-127);
 * the library decodes it exactly to bf16 (three mantissa bits times a power of
 * two) and then computes exactly as moe_fused_forward does with those bf16
 * weights.  Quantised weights for decode are a ranked next step of the
 * axolotl page's grouped GEMM (its fp8 path is left unimplemented there) and
 * of the B70 grouped-Q8 decode experiment (8-bit blocks).
 *
 *   w13_q [E, M1, H] bytes + w13_scale [E, M1, H / 32]
 *   w2_q [E, H, I] bytes + w2_scale [E, H, I / 32]
 *   shared_w13_q / _scale, shared_w2_q / _scale likewise (n_shared = 1), or NULL
 * Everything else (routing, outputs, workspace and its size) as
 * moe_fused_forward.  Extra limits: T <= 16 (MOE_ERR_UNSUPPORTED above), H and
 * I multiples of 32 (MOE_ERR_SHAPE).  Scales must keep the decoded values
 * inside bf16's normal range (s in [10, 246] for every block that has nonzero
 * elements); E4M3 NaN codes give NaN.
 */
int moe_fused_forward_mxfp8(const moe_layer_params* p, const void* x, const float* router_logits,
                            const void* w13_q, const uint8_t* w13_scale, const void* w2_q,
                            const uint8_t* w2_scale, const void* shared_w13_q,
                            const uint8_t* shared_w13_scale, const void* shared_w2_q,
                            const uint8_t* shared_w2_scale, float* out, int32_t* topk_ids,
                            float* topk_weights, int32_t* sorted_token_ids, int32_t* expert_ids,
                            int32_t* num_tokens_post_padded, void* workspace,
                            size_t* workspace_bytes, void* stream);

/*
 * Byte offset, inside the workspace of moe_fused_forward (and its _router and
 * _mxfp8 forms) for these parameters, of the layer's int32 status word, or a
 * negative status for invalid parameters.  Every call with T > 0 rewrites the
 * word on its stream: 0 when every cross-workgroup wait of the call ended
 * normally, 1 when a bounded wait expired, in which case that call's output
 * is invalid.  Only the decode form with one launch for both expert GEMVs
 * (T <= 16 and T * top_k >= 48) waits across workgroups: its W2 workgroups
 * wait, bounded at about a second, for the W13 workgroups of their expert,
 * relying on workgroups being dispatched in index order.  Read the word after
 * the call has completed (the library itself never reads it back).
 */
int64_t moe_fused_forward_status_offset(const moe_layer_params* p);

/*
 * moe_fused_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The library's own device-resident
 * scratch array stands in for the workspace: MOE_NOALLOC_SCRATCH_BYTES (32 MiB)
 * per GPU, created with the library's code object and held until the process
 * ends.  The call itself allocates nothing.  Everything else (arguments,
 * routing, outputs, results) is exactly moe_fused_forward's.
 * Errors: as moe_fused_forward, plus MOE_ERR_CAPACITY when the layer's
 * workspace (the size moe_fused_forward reports for these parameters) exceeds
 * the scratch; nothing is launched then.  Every call on one GPU shares that
 * GPU's scratch and leaves its last contents there: calls that overlap on one
 * GPU (different streams or host threads) race and must not be issued.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int moe_fused_forward_noalloc(const moe_layer_params* p, const void* x,
                              const float* router_logits, const void* w13, const void* w2,
                              const void* shared_w13, const void* shared_w2, float* out,
                              int32_t* topk_ids, float* topk_weights, int32_t* sorted_token_ids,
                              int32_t* expert_ids, int32_t* num_tokens_post_padded,
                              void* stream);

/* Human-readable text of a status code (static storage). */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* LIBMOE_MOE_H */
