/*
 * moe.h -- C ABI of the fused Mixture-of-Experts layer forward for AMD MI355X
 * (gfx950).  Library: moe_layer_05_amd/libmoemi.so.
 *
 * The layer (pages on "Mixture-of-Experts kernel engineering on Amazon
 * SageMaker AI"): each token activates a few experts chosen by a router; the
 * tokens are grouped by expert for grouped matrix products; each expert is a
 * gated feed-forward network; the expert outputs are combined with the routing
 * weights (toolboxkart.tech page, "Why MoE inference needs specialized
 * kernels"; kongchang.com page, "Why MoE Inference Is So Sensitive to Kernel
 * Engineering" and "Swap-AB"; aib.vote page, second and third paragraphs).
 *
 * Notation: T tokens, H hidden size, I intermediate size per expert, E
 * experts, K experts per token.  A "pair" i = t*K + k is token t's k-th choice.
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a DEVICE pointer to row-major contiguous memory,
 *    owned by the caller.  The library allocates nothing, keeps no pointer
 *    after a call returns, and is re-entrant (its only global state is a table
 *    of device properties filled once per device).
 *  - Every call enqueues its kernels on `stream` and returns at once; nothing
 *    synchronises the host and nothing is read back to the host.
 *  - All argument checks run on the host before any HIP call and look at
 *    values only, never at tensor contents.  On any error nothing is enqueued.
 *  - T == 0 is valid: MOE_OK with nothing enqueued.
 *  - Non-finite logits or activations give undefined results.
 *  - No code is compiled at run time: every shape is a kernel argument, so a
 *    new token count never triggers a compilation (toolboxkart.tech page,
 *    section 3 on repeated compilation; aib.vote page, fourth paragraph).
 *  - A launch error is reported as MOE_ERR_HIP; device faults surface at the
 *    caller's next synchronisation as HIP errors.
 */
#ifndef MOE_LAYER_05_AMD_MOE_H
#define MOE_LAYER_05_AMD_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,         /* a required pointer is NULL                   */
  MOE_ERR_SHAPE = 2,        /* a size is negative or inconsistent (K > E)   */
  MOE_ERR_UNSUPPORTED = 3,  /* outside the supported range (see each call)  */
  MOE_ERR_WORKSPACE = 4,    /* workspace smaller than the size query        */
  MOE_ERR_HIP = 5           /* a HIP launch or runtime call failed          */
} moe_status;

typedef enum {
  MOE_BF16 = 0,             /* expert weights are bfloat16                  */
  MOE_FP8_E4M3 = 1,         /* expert weights are OCP E4M3 codes + scales   */
  MOE_FP8_E5M2 = 2          /* expert weights are OCP E5M2 codes + scales   */
} moe_wdtype;

typedef enum {
  MOE_SCALES_TENSOR = 0,    /* FP8: one scale per expert weight tensor, one for
                               x and one for the intermediate               */
  MOE_SCALES_ROW = 1        /* FP8: one scale per weight output row
                               (channel), per token row of x and per pair
                               row of the intermediate                      */
} moe_fp8_scales;

/* Human-readable name of a status code (static string). */
const char* moe_status_string(moe_status s);

/*
 * Router (a1).  For each token, the K largest of its E float32 logits, larger
 * first; equal logits go to the lower expert id (+0.0 and -0.0 are equal).
 * The choice is made on the logits themselves.  Weights:
 *   renormalize != 0: w_k = exp(l_k - l_max) / sum_{j<K} exp(l_j - l_max)
 *   renormalize == 0: w_k = softmax(l)_k over all E experts.
 * A few experts per token, routed dynamically: toolboxkart.tech page, "Why MoE
 * inference needs specialized kernels"; kongchang.com page, "Why MoE Inference
 * Is So Sensitive to Kernel Engineering".
 *
 *   logits        [T, E] float32
 *   topk_ids      [T, K] int32   (out)
 *   topk_weights  [T, K] float32 (out)
 * Supported: 1 <= K <= min(E, 64), E <= 1024.  16-byte alignment not needed.
 */
moe_status moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t K,
                          int32_t renormalize, int32_t* topk_ids,
                          float* topk_weights, hipStream_t stream);

/*
 * Align (a2).  Stable counting sort of the pairs i = t*K + k by expert:
 * experts in ascending id; inside an expert ascending i; each expert's run
 * padded with the sentinel T*K to a multiple of block_m; an expert with no
 * pair takes no block.  This groups the tokens of each expert for the grouped
 * products (kongchang.com page, "Swap-AB": grouped GEMMs; "Why MoE Inference Is
 * So Sensitive...": the number of tokens per expert varies).
 *
 *   topk_ids      [T, K] int32, values in [0, E)
 *   sorted_ids    [moe_align_capacity(...)] int32 (out); entries
 *                 [0, *num_post_pad) are defined
 *   block_expert  [moe_align_capacity(...) / block_m] int32 (out); entries
 *                 [0, *num_post_pad / block_m) are defined
 *   num_post_pad  [1] int32 (out): sum over experts of ceil(count/block_m)*block_m
 *   workspace     device scratch of moe_align_workspace_bytes(...) bytes
 * Supported: block_m in {16, 32, 64, 128, 256}; E <= 1024; T*K < 2^31.
 */
size_t moe_align_capacity(int64_t T, int32_t K, int32_t E, int32_t block_m);
size_t moe_align_workspace_bytes(int64_t T, int32_t K, int32_t E, int32_t block_m);
moe_status moe_align(const int32_t* topk_ids, int64_t T, int32_t K, int32_t E,
                     int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                     int32_t* num_post_pad, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * Activation quantisation (a0, FP8 path).  Per-tensor E4M3:
 *   scale = amax|x| / 448 (one float32 division; 1 when amax is 0)
 *   codes[j] = E4M3(x[j] / scale), x[j] / scale an IEEE float32 division,
 *   rounded to nearest even, saturated to +-448, sign kept.
 * FP8 E4M3 with a per-tensor scale: kongchang.com page, FP8 explainer under
 * "Triton Backend Routing"; aib.vote page, third paragraph.
 *
 *   x          [n] bfloat16 (raw 16-bit patterns), 16-byte aligned
 *   codes      [n] uint8 (out)
 *   scale      [1] float32 (out)
 *   workspace  >= moe_act_quant_workspace_bytes() bytes of device scratch
 * Supported: n % 8 == 0.
 */
size_t moe_act_quant_workspace_bytes(void);
moe_status moe_act_quant_fp8(const void* x, int64_t n, uint8_t* codes,
                             float* scale, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * Activation quantisation with one scale per row (a0 under MOE_SCALES_ROW).
 * Each row r of cols values is quantised on its own: scales[r] = amax|x_r| /
 * max (1 when the row is all zero) and codes = FP8(x / scales[r]) as in
 * moe_act_quant_fp8, where fmt selects the code format: MOE_FP8_E4M3 (max
 * 448) or MOE_FP8_E5M2 (OCP E5M2: bias 15, max 57344; round to nearest even,
 * saturating to +-57344; the kongchang.com page's FP8 explainer names E5M2 as
 * the wider-range, lower-precision variant).  rows = 1 gives one scale for
 * the whole tensor.  Finer granularity than one scale per tensor, read from the
 * kongchang.com page, "Triton Backend Routing: A Practical Path to FP8
 * Quantization" (numerical distributions differ, so a uniform scale loses
 * precision), taken down to rows.
 *
 *   x       [rows, cols] bfloat16 (raw 16-bit patterns), 16-byte aligned
 *   codes   [rows, cols] uint8 (out), 16-byte aligned
 *   scales  [rows] float32 (out)
 * Supported: cols % 8 == 0; fmt MOE_FP8_E4M3 or MOE_FP8_E5M2
 * (MOE_ERR_UNSUPPORTED otherwise).  No workspace.
 */
moe_status moe_act_quant_fp8_rows(const void* x, int64_t rows, int32_t cols,
                                  moe_wdtype fmt, uint8_t* codes, float* scales,
                                  hipStream_t stream);

/*
 * Fused layer forward (a0..a6).  out[t] = bfloat16_rne( sum_k w[t,k] *
 *   W2_e (silu(W1_e x^_t) * (W3_e x^_t)) ),  e = topk_ids[t,k],
 * with W1_e = w13[e, 0:I, :] (gate) and W3_e = w13[e, I:2I, :] (up).
 * The routing, the grouping of tokens by expert, the grouped products, the
 * scaling and the weighted aggregation all run on the device
 * (toolboxkart.tech page, "Why MoE inference needs specialized kernels": a
 * fused kernel combines routing, data movement and expert math; aib.vote
 * page, third paragraph: scaling, products and expert aggregation in one pass).
 * For thin token batches the expert weight rows take the row side of the
 * matrix instructions (the Swap-AB idea: toolboxkart.tech page, section 1;
 * kongchang.com page, "Swap-AB"; aib.vote page, second paragraph).
 *
 * MOE_BF16:     x^ = x; weights bfloat16.
 * MOE_FP8_E4M3, fp8_scales == MOE_SCALES_TENSOR:
 *               x^ = dequantised per-tensor E4M3 of x (as moe_act_quant_fp8);
 *               W = code * w13_scale[e] (or w2_scale[e]); the intermediate
 *               a = silu(g) * u is quantised per tensor over all pairs, from
 *               its float32 value, before the down projection.
 * MOE_FP8_E5M2: as MOE_FP8_E4M3 in either scale mode, with E5M2 codes for
 *               the weights, x and the intermediate and 57344 in place of
 *               448 in every activation scale (amax / 57344).
 * MOE_FP8_E4M3, fp8_scales == MOE_SCALES_ROW:
 *               x^ = per-token-row E4M3 of x (as moe_act_quant_fp8_rows);
 *               W[r, :] = code[r, :] * w13_scale[e, r] (w2_scale[e, r]); the
 *               intermediate is quantised per pair row.  No scale couples two
 *               tokens, so a token's output does not depend on the batch.
 *
 * Fields:
 *   x               [T, H] bfloat16
 *   router_logits   [T, E] float32
 *   w13             [E, 2I, H] bfloat16 or uint8 E4M3 / E5M2 codes
 *   w2              [E, H, I]  bfloat16 or uint8 E4M3 / E5M2 codes
 *   fp8_scales      moe_fp8_scales, FP8 only (ignored for bf16)
 *   w13_scale, w2_scale  FP8 only (ignored for bf16, may be NULL):
 *                   [E] float32 with MOE_SCALES_TENSOR; [E, 2I] and [E, H]
 *                   float32, 16-byte aligned, with MOE_SCALES_ROW
 *   out             [T, H] bfloat16 (out)
 *   topk_ids_out    [T, K] int32 (out, optional: NULL to skip)
 *   topk_weights_out[T, K] float32 (out, optional: NULL to skip)
 *   workspace       device scratch, >= moe_fused_workspace_bytes(args) bytes,
 *                   16-byte aligned; its contents on entry do not matter
 * Supported: H % 16 == 0, I % 16 == 0, 1 <= K <= min(E, 64), E <= 1024,
 * T*K < 2^31; x, w13, w2, out and workspace 16-byte aligned.
 */
typedef struct {
  moe_wdtype wdtype;
  moe_fp8_scales fp8_scales;
  int64_t T;
  int32_t H, I, E, K;
  int32_t renormalize;
  const void* x;
  const float* router_logits;
  const void* w13;
  const void* w2;
  const float* w13_scale;
  const float* w2_scale;
  void* out;
  int32_t* topk_ids_out;
  float* topk_weights_out;
  void* workspace;
  size_t workspace_bytes;
} moe_fused_args;

/* Workspace bytes moe_fused_forward needs for the shape in *args (pointers
 * are not read). 0 when the shape is invalid. */
size_t moe_fused_workspace_bytes(const moe_fused_args* args);

/*
 * Where moe_fused_forward keeps each intermediate result inside the caller's
 * workspace, for callers (tests, debuggers) that inspect the steps of a call
 * after it has completed on its stream and before the workspace is reused.
 * Each field is a byte offset from the workspace start, or MOE_NO_SECTION
 * when the call has no such result (for its weight type, scale mode or size).
 * Layout of the sections (P = T*K pairs, pair i = t*K + k):
 *   topk_ids, topk_weights  [T, K] int32 / float32 (used only when the caller
 *                           passes no topk_ids_out / topk_weights_out)
 *   sorted_ids, block_expert, num_post_pad  the align layout (as moe_align)
 *                           with block size block_m over `capacity` entries;
 *                           when `tiled` is 1 it holds only the experts with
 *                           fewer than tile_threshold pairs
 *   tile_sorted_ids, tile_block_expert, tile_num_post_pad  (tiled == 1) the
 *                           layout of the experts with >= tile_threshold pairs,
 *                           block size tile_block_m, tile_capacity entries
 *   x_amax                  uint32: the float bits of amax|x| (FP8, per tensor)
 *   x_codes                 [T, H] uint8 FP8 codes of x (FP8)
 *   x_scales                [T] float32 per-row scales of x (FP8, per row)
 *   a                       [P, I] the intermediate silu(g) * u in pair
 *                           order: float32 (FP8) or bfloat16 (bf16)
 *   a_amax                  uint32: the float bits of amax|a| over all pairs
 *                           (FP8, per tensor)
 *   a_codes                 [P, I] uint8 FP8 codes of a (FP8)
 *   a_scales                [P] float32 per-row scales of a (FP8, per row)
 * Pointers of *args are not read.  Errors: MOE_ERR_NULL, and the shape checks
 * of moe_fused_forward.
 */
#define MOE_NO_SECTION ((size_t)-1)
typedef struct {
  size_t total;                  /* == moe_fused_workspace_bytes(args) */
  int32_t block_m;
  int32_t tiled;
  int32_t tile_block_m;
  int32_t tile_threshold;
  int64_t capacity;
  int64_t tile_capacity;
  size_t topk_ids, topk_weights;
  size_t sorted_ids, block_expert, num_post_pad;
  size_t tile_sorted_ids, tile_block_expert, tile_num_post_pad;
  size_t x_amax, x_codes, x_scales;
  size_t a, a_amax, a_codes, a_scales;
} moe_fused_layout;
moe_status moe_fused_workspace_layout(const moe_fused_args* args, moe_fused_layout* layout);

/* Block size (tokens per expert block) moe_fused_forward uses for this shape;
 * moe_align with this block_m reproduces its layout. */
int32_t moe_fused_block_m(int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                          moe_wdtype wdtype);

/* Enqueues the whole layer on `stream` (see the block above moe_fused_args)
 * and returns.  The first call on a device also resolves every kernel of the
 * library in the runtime (a one-time host cost), so no later call, at any
 * token count, pays a kernel's first-launch lookup; nothing is compiled at
 * run time.  Errors: MOE_ERR_NULL for a missing pointer, MOE_ERR_SHAPE /
 * MOE_ERR_UNSUPPORTED for a shape or alignment outside the supported set,
 * MOE_ERR_WORKSPACE when workspace_bytes is too small (all checked on the
 * host before anything is enqueued), MOE_ERR_HIP when a launch fails. */
moe_status moe_fused_forward(const moe_fused_args* args, hipStream_t stream);

/*
 * Stage boundaries of the fused forward, for timing its kernels on the
 * stream they run on.  events[s] is recorded right before stage s is
 * enqueued and events[MOE_STAGE_COUNT] after the last one; a stage that has
 * no work for the weight type (the two quantisations with bfloat16 weights)
 * has its two events back to back.
 */
typedef enum {
  MOE_STAGE_ROUTE = 0,        /* a1 router                                   */
  MOE_STAGE_ACT_QUANT = 1,    /* a0 E4M3 quantisation of x (FP8 only)        */
  MOE_STAGE_ALIGN = 2,        /* a2 sort of the pairs by expert              */
  MOE_STAGE_GATE_UP = 3,      /* a3+a4 gate/up product, SiLU-and-mul         */
  MOE_STAGE_INTER_QUANT = 4,  /* E4M3 quantisation of the intermediate (FP8) */
  MOE_STAGE_DOWN = 5,         /* a5 down product and scales                  */
  MOE_STAGE_COMBINE = 6,      /* a6 routing-weighted sum, bfloat16 output    */
  MOE_STAGE_COUNT = 7
} moe_stage;

/*
 * moe_fused_forward with stage events: identical work and results, plus
 * hipEventRecord(events[s], stream) at each stage boundary.
 *   events  [MOE_STAGE_COUNT + 1] events created by the caller (owned by the
 *           caller; must be valid for the stream's device).  A NULL entry
 *           skips that boundary (each record costs a few microseconds of
 *           stream time, so a caller timing one kernel sets only its two).
 *           A NULL array gives MOE_ERR_NULL.  A failed record gives
 *           MOE_ERR_HIP.
 */
moe_status moe_fused_forward_timed(const moe_fused_args* args, hipStream_t stream,
                                   hipEvent_t* events);

/*
 * Inverse rotary position embedding of attention heads fused with one FP8
 * scale per (token, head): the attention-side kernel the pages name beside
 * the MoE layer, which must serve any number of tokens without compiling
 * anything for a new count (toolboxkart.tech page, section 3; aib.vote page,
 * fourth paragraph: a kernel recompiled per num_tokens until its
 * variable-length arguments were left unspecialised).  Here T, NH, D and R
 * are plain arguments of one precompiled kernel.
 *
 * For token t at position p = positions[t] and each head h, with the pairs
 * (i, i + R/2) (interleaved == 0) or (2i, 2i + 1) (interleaved != 0),
 * i < R/2, c = cos_sin[p][i] and s = cos_sin[p][R/2 + i]:
 *   y1 = x1 * c + x2 * s,   y2 = x2 * c - x1 * s      (rotation by -theta)
 * in float32, each product and sum rounded on its own; features R..D-1 pass
 * through.  Then scales[t][h] = amax|y| / max of fmt (448 for E4M3, 57344
 * for E5M2; 1 when the row is zero) and codes[t][h][:] = FP8(y / scale) with
 * an IEEE float32 division, nearest even, saturating (as moe_act_quant_fp8).
 *
 *   x          [T][NH][D] bfloat16; token t starts at element
 *              t * x_token_stride (heads contiguous inside a token), 16-byte
 *              aligned
 *   positions  [T] int64; a position outside [0, max_pos) is clamped into it
 *   cos_sin    [max_pos][R] float32: the R/2 cosines, then the R/2 sines, of
 *              each position's angles; 16-byte aligned
 *   codes      [T][NH][D] uint8 (out), 16-byte aligned
 *   scales     [T][NH] float32 (out)
 * Supported: D % 8 == 0 and D <= 512; R even, 0 < R <= D, R % 16 == 0
 * (R % 8 == 0 when interleaved); x_token_stride >= NH * D and a multiple of
 * 8; fmt MOE_FP8_E4M3 or MOE_FP8_E5M2.  Errors: MOE_ERR_SHAPE,
 * MOE_ERR_UNSUPPORTED, MOE_ERR_NULL (host checks, nothing enqueued),
 * MOE_ERR_HIP when the launch fails.  T == 0 enqueues nothing.
 */
moe_status moe_inv_rope_fp8_quant_per_head(const void* x, int64_t x_token_stride,
                                           const int64_t* positions, const float* cos_sin,
                                           int64_t max_pos, int64_t T, int32_t NH, int32_t D,
                                           int32_t R, int32_t interleaved, moe_wdtype fmt,
                                           uint8_t* codes, float* scales, hipStream_t stream);

/*
 * moe_fused_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same layer and the same kernels, with the workspace taken
 * from a scratch buffer the library holds in device memory instead of from
 * args->workspace (args->workspace and args->workspace_bytes are ignored).
 * Nothing is allocated: the buffer is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES, one copy per GPU the library runs on, held until
 * the process ends.  The first call on a device resolves the kernels and the
 * buffer's address there (no allocation).  Every call on a GPU uses that
 * GPU's one buffer and leaves the last call's contents in it (each call sets
 * up what it reads, so the contents on entry do not matter); calls whose
 * execution overlaps on one GPU (on different streams, or from different
 * threads without ordering) race on it and give undefined results.
 * Errors: as moe_fused_forward, and MOE_ERR_WORKSPACE, before anything is
 * enqueued, when moe_fused_workspace_bytes(args) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES (decode batches fit; a 4096-token call of a
 * 256-expert layer does not).
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_fused_forward_noalloc(const moe_fused_args* args, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LAYER_05_AMD_MOE_H */
