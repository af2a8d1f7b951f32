/*
 * moe_w4a16.h -- C ABI of the MI355X (gfx950) W4A16 routed-expert MoE layer.
 *
 * The layer (Kimi-K2.6 inference-research catalog entry, MoE and QUANT
 * paragraphs; lmdeploy pull request "support Kimi K2.6", Changes list, which
 * names the compressed-tensors W4A16 MoE kernels):
 *
 *   out[t] = bf16( S(x_t) + sum_{j<k, id_tj local} w_tj * F_{id_tj - base}(x_t) )
 *   F_e(v) = W2_e ( silu(W1_e v) * (W3_e v) ),   W1_e = W13_e[0:I], W3_e = W13_e[I:2I]
 *   W[n][c] = (u - 8) * s[n][c/32],  u = 4-bit field c%8 (bits 4(c%8)..) of word c/8
 *   S = the same MLP with the bf16 shared-expert weights, added with weight 1
 *
 * Routed experts are symmetric INT4 with one bf16 scale per 32 inputs along
 * the input dimension, eight codes per int32 word (QUANT and PARAMS
 * paragraphs); the shared expert is bf16 (QUANT paragraph: kept in higher
 * precision). Hidden 7168, 384 experts, top-8 and moe_intermediate 2048 are
 * the catalog's geometry; the library takes any shape meeting the limits
 * below.
 *
 * Conventions for every entry point
 *  - Tensors are dense, row-major, and live in device memory unless marked
 *    "host". Every device pointer must be 16-byte aligned.
 *  - The caller allocates and owns every buffer, including the workspace, and
 *    keeps it alive until the stream work completes. The library allocates
 *    no buffers, keeps no state or pointer after it returns, never
 *    synchronises the host and launches only on `stream` (a hipStream_t;
 *    NULL is the null stream) on the current device, so every entry point may
 *    be captured into a HIP graph at any time. Calls that share a workspace
 *    must not overlap. Every kernel is this library's own HIP code.
 *  - Every argument error is detected on the host before any launch (so a
 *    failing call writes nothing) and reported as a negative status. Routing
 *    data on the device is never an error: ids outside [expert_base,
 *    expert_base + num_experts), -1 included, contribute nothing. NaNs
 *    propagate.
 *  - Limits: 1 <= top_k <= 16; 1 <= num_experts <= 512; hidden and inter
 *    multiples of 128 (a 128-input chunk is four whole quantisation groups,
 *    and 16-byte loads then never straddle a row; every width of the model
 *    family is one: 7168, 2048, and 256 per GPU of an 8-way tensor-parallel
 *    split); group_size == 32; num_tokens * top_k < 2^31 - 1 (else
 *    MOE_ERR_SHAPE). The kernels address each array through 32-bit buffer
 *    descriptors, so a problem whose shared-expert matrix (2 * inter * hidden
 *    bf16), or, past the decode regime, whose x (num_tokens * hidden bf16) or
 *    bucketed intermediate rows (about (num_tokens * top_k + 95 *
 *    num_experts) * inter * 2 bytes) would reach 2 GiB is refused with
 *    MOE_ERR_UNSUPPORTED (at the Kimi-K2.6 shape: about 60,000 tokens per
 *    call).
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK 0
#define MOE_ERR_NULL (-1)        /* a required pointer is NULL */
#define MOE_ERR_SHAPE (-2)       /* a size is out of range */
#define MOE_ERR_ALIGNMENT (-3)   /* a device pointer is not 16-byte aligned */
#define MOE_ERR_WORKSPACE (-4)   /* workspace or output buffer too small */
#define MOE_ERR_UNSUPPORTED (-5) /* a valid but unsupported configuration */
#define MOE_ERR_HIP (-6)         /* a HIP call failed; see moe_w4a16_status_string */

#define MOE_MAX_TOP_K 16
#define MOE_MAX_EXPERTS 512
#define MOE_MAX_SCORED 1024 /* experts scored per token by the router step */

/* Problem sizes (host struct, read during the call only). */
typedef struct {
  int64_t num_tokens; /* T >= 0; T == 0 is a successful no-op */
  int32_t hidden;     /* H: input and output width, multiple of 128 */
  int32_t inter;      /* I: expert intermediate width, multiple of 128 */
  int32_t num_experts;/* E: experts present in packed_w13 / packed_w2 */
  int32_t expert_base;/* global id of local expert 0 (expert parallelism) */
  int32_t top_k;      /* k: routing slots per token */
  int32_t group_size; /* quantisation group along the input dim, must be 32 */
} moe_w4a16_problem;

/*
 * Bytes of device workspace moe_w4a16_forward needs for `p` (host-only, no
 * GPU call). Writes *bytes (host). Returns a status.
 */
int moe_w4a16_workspace_size(const moe_w4a16_problem *p, size_t *bytes);

/*
 * The bucket granularity (rows per GEMM block) moe_w4a16_forward uses for
 * `p`. Writes *block_m (host). Returns a status. With block_m 96 and fewer
 * than 8192 (token, slot) pairs, the experts that receive at most 4 pairs are
 * bucketed in 4 rows instead and computed as in a decode-sized call (see
 * moe_w4a16_forward); the others use 96-row buckets.
 */
int moe_w4a16_forward_block_m(const moe_w4a16_problem *p, int32_t *block_m);

/*
 * The split of the bucketing moe_w4a16_forward uses for `p`: writes to
 * *max_pairs (host) the largest pair count of an expert that is bucketed in
 * 4 rows beside the 96-row buckets (4 at present), or 0 when the call has no
 * such split (block_m 4, or 8192 pairs or more). Returns a status.
 */
int moe_w4a16_forward_split_max_pairs(const moe_w4a16_problem *p, int32_t *max_pairs);

/*
 * Capacities moe_w4a16_align needs: *sorted_capacity int32 entries for
 * sorted_ids and *block_capacity entries for block_expert (both host out).
 * sorted_capacity = T*k + min(E, T*k) * (block_m - 1), the largest possible
 * padded count; block_capacity = sorted_capacity / block_m.
 */
int moe_w4a16_align_capacity(const moe_w4a16_problem *p, int32_t block_m,
                             int64_t *sorted_capacity, int64_t *block_capacity);

/*
 * Token/expert bucketing used by the grouped GEMMs (exported so it can be
 * checked bit for bit). The pages name the grouped W4A16 MoE kernels without
 * their internals; the ordering defined here is the one this library uses.
 *
 *   topk_ids     int32 [T, k] (device)
 *   sorted_ids   int32 [sorted_capacity] (device, out): the valid pairs
 *                p = t*k + j of local expert 0 in ascending p, padded with the
 *                sentinel T*k to a multiple of block_m, then expert 1, ...;
 *                experts without pairs take no space. Entries at and past
 *                n_padded are left unspecified.
 *   block_expert int32 [block_capacity] (device, out): local expert of each
 *                block of block_m entries of sorted_ids.
 *   n_padded     int32 [1] (device, out): number of meaningful sorted_ids.
 *
 *   scratch      device, scratch_bytes long, or NULL. NULL: the bucketing runs
 *                in one work-group (one launch; suits small T*k). Otherwise at
 *                least moe_w4a16_align_scratch_size bytes: it runs in many
 *                work-groups (three launches, per-chunk counts in scratch).
 *                Both give identical output.
 *
 * 1 <= block_m <= 1024. Returns MOE_ERR_WORKSPACE if a capacity is below the
 * value moe_w4a16_align_capacity reports, or if scratch is given and shorter
 * than moe_w4a16_align_scratch_size.
 */
int moe_w4a16_align(const int32_t *topk_ids, const moe_w4a16_problem *p, int32_t block_m,
                    int32_t *sorted_ids, int64_t sorted_capacity, int32_t *block_expert,
                    int64_t block_capacity, int32_t *n_padded, void *scratch,
                    size_t scratch_bytes, void *stream);

/*
 * Scratch bytes (host out) of the many-work-group bucketing for this problem:
 * one int32 per (chunk of 256 pairs, local expert), plus one per local
 * expert (the bucket offsets).
 */
int moe_w4a16_align_scratch_size(const moe_w4a16_problem *p, size_t *bytes);

/*
 * The layer.
 *
 *   x            bf16  [T, H]
 *   topk_ids     int32 [T, k]   global expert ids; local expert = id - expert_base
 *   topk_weights fp32  [T, k]   applied as given (no renormalisation)
 *   packed_w13   int32 [E, 2I, H/8]  rows 0..I-1 gate, rows I..2I-1 up
 *   scales_w13   bf16  [E, 2I, H/32]
 *   packed_w2    int32 [E, H, I/8]
 *   scales_w2    bf16  [E, H, I/32]
 *   shared_w     bf16  [2I*H + H*I] (gate/up [2I, H], then down [H, I]) or NULL
 *   out          bf16  [T, H], fully overwritten; must not alias an input
 *   workspace    device scratch of at least moe_w4a16_workspace_size bytes
 *
 * Numerics: the dequantised int4 weights (u - 8) * s are never rounded, and
 * products accumulate in fp32. Decode-sized calls (moe_w4a16_forward_block_m
 * 4) put the codes into bf16 MFMAs and multiply each group's fp32 scale
 * after them, with h rounded to bf16. Larger calls (block_m 96) run the
 * routed products in fp16 (except experts with at most 4 pairs in a call of
 * fewer than 8192 pairs, which take the decode-sized path), where (u - 8) * s
 * is exact for bf16 group scales with 2^-17 <= |s| <= 2720 (smaller ones
 * round to fp16's subnormal grid, larger ones overflow the fp16 offset -24 s
 * of the dequantisation): x is converted once to fp16 with one power-of-two
 * scale per token (exact down to 2^-32 of the token's largest |x|), and h is
 * rounded once to fp16 with one power-of-two scale per row and 256 columns.
 * The bf16 shared expert uses bf16 products with its h rounded to bf16.
 * The routed and shared results are combined in fp32 and rounded once to
 * bf16 (round to nearest even).
 */
int moe_w4a16_forward(const void *x, const int32_t *topk_ids, const float *topk_weights,
                      const int32_t *packed_w13, const void *scales_w13,
                      const int32_t *packed_w2, const void *scales_w2, const void *shared_w,
                      void *out, const moe_w4a16_problem *p, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * moe_w4a16_forward with stage timing: identical work and results, and in
 * addition records the caller's HIP events (hipEvent_t, created by the caller;
 * stage_events holds 7 entries, NULL entries are skipped) on `stream`:
 * [0] before the bucketing, [1] before the gate_up GEMM, [2] before the down
 * GEMM, [3] before the combine, [4] after it, [5] after the gate_up launch and
 * [6] after the down launch (each launch carries the routed and the shared
 * experts; with block_m 96 the conversion of x to fp16 runs between [0] and
 * [1], and experts in 4-row buckets take a launch of their own just before
 * each GEMM launch, inside the same interval). Used to time each kernel on
 * its own stream.
 */
int moe_w4a16_forward_timed(const void *x, const int32_t *topk_ids, const float *topk_weights,
                            const int32_t *packed_w13, const void *scales_w13,
                            const int32_t *packed_w2, const void *scales_w2,
                            const void *shared_w, void *out, const moe_w4a16_problem *p,
                            void *workspace, size_t workspace_bytes, void *stream,
                            void *const *stage_events);

/*
 * The router step in front of the layer. The lmdeploy pull request "support
 * Kimi K2.6" (Runtime Validation) lists MoE routing among the validated paths
 * without a formula; the plainest rule is implemented:
 *
 *   topk_ids[t]     = the top_k experts with the largest scores[t, :], in
 *                     descending score order; equal scores in ascending
 *                     expert id (-0.0 equals +0.0)
 *   topk_weights[t] = softmax over the selected scores (fp32, largest score
 *                     subtracted first) -- the softmax over all experts
 *                     renormalised over the selected ones
 *
 *   scores       fp32  [T, num_scored]  one score per expert of the model
 *                      (global ids 0 .. num_scored-1); must not hold NaN
 *   topk_ids     int32 [T, k]   written (global ids)
 *   topk_weights fp32  [T, k]   written
 *
 * T and k come from `p` (the whole problem is validated); 1 <= k <=
 * num_scored <= MOE_MAX_SCORED and expert_base + num_experts <= num_scored,
 * else MOE_ERR_SHAPE. T == 0 is a no-op.
 */
int moe_w4a16_route(const float *scores, int32_t num_scored, const moe_w4a16_problem *p,
                    int32_t *topk_ids, float *topk_weights, void *stream);

/*
 * The router step followed by the layer, on `stream`: moe_w4a16_route into
 * the caller's topk_ids / topk_weights (outputs here), then moe_w4a16_forward
 * on them, with the same workspace and the same results as the two calls.
 */
int moe_w4a16_forward_scores(const void *x, const float *scores, int32_t num_scored,
                             const int32_t *packed_w13, const void *scales_w13,
                             const int32_t *packed_w2, const void *scales_w2,
                             const void *shared_w, void *out, int32_t *topk_ids,
                             float *topk_weights, const moe_w4a16_problem *p, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * Prepacked weights: the weight-loading step that the lmdeploy "support Kimi
 * K2.6" pull request (Changes list) names for the compressed-tensors W4A16
 * experts, done once ahead of the layer calls. The same int4 codes and bf16
 * scales, reordered in tiles of the order the GEMM kernels take them, so that
 * their register loads take whole cache lines (decode about 5% faster; the
 * large-batch kernel stages checkpoint-layout weights through LDS in whole
 * lines and runs at the same speed on either layout; the order is internal to
 * the library and may change between versions;
 * only moe_w4a16_prepack writes it and only the *_prepacked calls read it).
 * Results are bit for bit those of moe_w4a16_forward on the original weights.
 *
 * Supported widths: hidden % 512 == 0 and inter % 256 == 0 (e.g. the full
 * Kimi-K2.6 layer, 7168 / 2048, and one GPU's share of an 8-way tensor-
 * parallel split, 7168 / 256); others give MOE_ERR_UNSUPPORTED (use
 * moe_w4a16_forward). The buffer depends on hidden, inter and num_experts
 * only.
 *
 * moe_w4a16_prepack_size: bytes of the prepacked buffer (host only; about the
 * size of packed_w13 + scales_w13 + packed_w2 + scales_w2).
 */
int moe_w4a16_prepack_size(const moe_w4a16_problem *p, size_t *bytes);

/*
 * Writes the prepacked form of the four weight tensors (layouts as in
 * moe_w4a16_forward) into `prepacked` (device, prepacked_bytes long, at least
 * moe_w4a16_prepack_size), on `stream`. The inputs are only read and may be
 * freed once the stream work has completed. MOE_ERR_WORKSPACE if the buffer
 * is too small; the other errors as for moe_w4a16_forward.
 */
int moe_w4a16_prepack(const int32_t *packed_w13, const void *scales_w13,
                      const int32_t *packed_w2, const void *scales_w2,
                      const moe_w4a16_problem *p, void *prepacked, size_t prepacked_bytes,
                      void *stream);

/*
 * moe_w4a16_forward with the weights in prepacked form (written by
 * moe_w4a16_prepack for the same hidden, inter and num_experts); every other
 * argument, the workspace size and the results as for moe_w4a16_forward.
 * MOE_ERR_WORKSPACE if prepacked_bytes is below moe_w4a16_prepack_size.
 */
int moe_w4a16_forward_prepacked(const void *x, const int32_t *topk_ids,
                                const float *topk_weights, const void *prepacked,
                                size_t prepacked_bytes, const void *shared_w, void *out,
                                const moe_w4a16_problem *p, void *workspace,
                                size_t workspace_bytes, void *stream);

/* moe_w4a16_forward_prepacked with the stage events of moe_w4a16_forward_timed. */
int moe_w4a16_forward_prepacked_timed(const void *x, const int32_t *topk_ids,
                                      const float *topk_weights, const void *prepacked,
                                      size_t prepacked_bytes, const void *shared_w, void *out,
                                      const moe_w4a16_problem *p, void *workspace,
                                      size_t workspace_bytes, void *stream,
                                      void *const *stage_events);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_w4a16_forward with the workspace taken from a device array inside the
 * library instead of the caller. The array is MOE_NOALLOC_SCRATCH_BYTES
 * (64 MiB), one per GPU the library runs on, reserved with the library's code
 * and held until the process ends; its address is looked up on the first call
 * on each device (not a stream operation). Problems whose workspace
 * (moe_w4a16_workspace_size) exceeds it get MOE_ERR_WORKSPACE before any
 * launch: at the Kimi-K2.6 shape every decode batch up to 192 tokens fits.
 * Every other argument and result as for moe_w4a16_forward (bit for bit).
 * All calls on one GPU share that GPU's array: calls that overlap on one GPU
 * (on different streams, or from several threads without ordering) race, and
 * the array keeps whatever the last call left there.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_w4a16_forward_noalloc(const void *x, const int32_t *topk_ids, const float *topk_weights,
                              const int32_t *packed_w13, const void *scales_w13,
                              const int32_t *packed_w2, const void *scales_w2,
                              const void *shared_w, void *out, const moe_w4a16_problem *p,
                              void *stream);

/* The size of moe_w4a16_forward_noalloc's device array (host out). */
int moe_w4a16_noalloc_workspace_limit(size_t *bytes);

/*
 * A static description of `status`; for MOE_ERR_HIP it names the HIP error
 * of the failing call on this thread. Never NULL.
 */
const char *moe_w4a16_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H */
