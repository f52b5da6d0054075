/*
 * moe_mxfp4.h - C ABI of the routed MXFP4 Mixture-of-Experts block on
 * AMD Instinct MI355X (gfx950).
 *
 * The block (pages: turbospark-runtime `src/families/gptoss/mod.rs`, module
 * doc "One decoder layer"; goosedump `src/engine/model/gpt_oss.rs`,
 * `mixture_of_experts` and `mixture_of_experts_batch`):
 *
 *   xn   = norm_w ? rms_norm(hidden, norm_w, rms_eps) : hidden
 *   l    = xn . router_w^T + router_b                    (logits, fp64)
 *   idx  = top-k of l, ties to the lower expert index
 *   w    = route_scale * softmax(l[idx])                 (over the k selected)
 *   y_j  = down_j(swiglu(gate_j(xn) + bg_j, up_j(xn) + bu_j)) + bd_j
 *   out  = hidden + sum_j w_j * y_j  (+ shared experts, weight 1)
 *
 *   swiglu(g, u) = min(g, L) * sigmoid(alpha * min(g, L)) * (clamp(u, -L, L) + o)
 *
 * Conventions for every call below:
 * - Device pointers are caller-owned device allocations; the library never
 *   allocates, frees or keeps device memory between calls. Host pointers are
 *   marked "host".
 * - Compute calls enqueue work on `stream` and return without synchronising.
 *   Arguments are validated on the host before anything is enqueued; on an
 *   invalid argument nothing is enqueued, a negative moe_status is returned
 *   and moe_last_error() describes the problem.
 * - Row-major layouts; [A,B] means A rows of B contiguous elements.
 * - Numerics: weights are used exactly as stored. Activations meet them on
 *   the gfx950 block-scaled matrix cores as a sum of FP8 (E4M3) terms per
 *   value with one E8M0 scale per 32 values and term; n terms carry a value
 *   to within about 2^-4n of its block's largest magnitude. Decode uses four
 *   terms everywhere; prefill uses three for the SwiGLU output and, for the
 *   expert input, four on 16-row tiles and three on larger tiles. A bfloat16
 *   expert input without RMSNorm is not split in prefill: the weights are
 *   decoded to bfloat16 in registers (exact for scale bytes 1..252) and meet
 *   the input on the bfloat16 matrix cores (moe_prefill_plan tells which
 *   path a shape takes). Products accumulate in float32. Router logits are
 *   accumulated in float64.
 * - Shape limits: 1 <= E <= 512, 1 <= k <= min(E, 8), H and F multiples of
 *   32 and at most 16384, 0 <= T, n_shared in {0, 1}. Decode additionally
 *   needs T <= 64 and H, F <= 8192. With T = 0 a call only validates the
 *   shape and returns MOE_OK.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* null pointer, bad shape or constant */
    MOE_ERR_UNSUPPORTED = -2, /* valid request outside the supported limits */
    MOE_ERR_WORKSPACE = -3,   /* workspace missing, too small or misaligned */
    MOE_ERR_HIP = -4          /* a HIP launch or runtime call failed */
} moe_status;

typedef enum moe_dtype {
    MOE_F32 = 0,  /* float32 hidden/residual */
    MOE_BF16 = 1  /* bfloat16 hidden/residual (bits), widened exactly */
} moe_dtype;

/* Shape and constants of one MoE block.
 * alpha / limit / up_offset: gpt-oss uses 1.702 / 7.0 / 1.0 (goosedump
 * constants SWIGLU_ALPHA, SWIGLU_LIMIT); the DeepSeek-V4-Flash shape uses
 * 1.0 / 10.0 / 0.0 (antirez ds4.c DS4_DEFAULT_SWIGLU_CLAMP_EXP).
 * route_scale: 1.0 for gpt-oss, 1.5 for DeepSeek-V4-Flash (ds4.c
 * DS4_SHAPE_FLASH expert_weight_scale). rms_eps is used only when a norm
 * weight is passed (1e-5 for gpt-oss).
 * act_quant = 1 selects the quantised expert-input mode of
 * moe_forward_prefill: the experts' input (the normalised hidden state, as
 * float32) is rounded once to MX-FP4 - blocks of 32 values sharing the
 * power-of-two scale 2^e, e the smallest integer with amax <= 6 * 2^e (amax
 * held at no less than 6 * 2^-126), each value divided by it, clamped to
 * +-6 and replaced by the nearest E2M1 value, ties to the even code (page:
 * antirez ds4.c `dsv4_fp4_act_quantize_row_inplace_cpu`,
 * `dsv4_e2m1fn_dequant_cpu`) - and reused by every expert row that takes
 * the token (goosedump `mixture_of_experts`, `Q8Activation`). The gate/up
 * products then run FP4 x FP4 on the matrix cores, one instruction each.
 * Routing, the SwiGLU output and the residual are unaffected.
 * act_quant = 2 also rounds each routed row's SwiGLU output (float32, blocks
 * of 32 along F) through the same round trip before the down projection,
 * whose products then run FP4 x FP4 too. The decode entry points reject both
 * modes (MOE_ERR_UNSUPPORTED). */
typedef struct moe_shape {
    int32_t T;          /* tokens */
    int32_t H;          /* hidden size */
    int32_t F;          /* expert hidden size */
    int32_t E;          /* routed experts */
    int32_t k;          /* experts per token */
    int32_t act_dtype;  /* moe_dtype of hidden */
    int32_t n_shared;   /* always-on shared experts (0 or 1) */
    float swiglu_alpha;
    float swiglu_limit;
    float swiglu_up_offset;
    float route_scale;
    float rms_eps;
    int32_t act_quant;  /* 0: exact; 1: MX-FP4 expert input; 2: and MX-FP4 SwiGLU output */
} moe_shape;

/* Byte layout of one packed expert blob. Offsets are from the blob start;
 * every plane is 256-byte aligned. Expert e of a packed set starts at
 * base + e * stride.
 *   gate_q, up_q (F x H weights), down_q (H x F)   E2M1 codes, 16 bytes per
 *       32-value MX block, element 2i in the low nibble of byte i
 *   gate_s, up_s, down_s                            one E8M0 scale byte per
 *       block, value 2^(b-127)
 *   gate_b [F], up_b [F], down_b [H]                float32 biases
 * A code plane of R x K weights (R rows, K columns, both multiples of 32;
 * nb = K / 32 blocks per row) is tiled for the matrix cores: block c of row
 * r sits at byte
 *     (r / 16) * 256 * nb + (c / 4) * 1024 + ((c % 4) * 16 + r % 16) * 16
 * i.e. rows in tiles of 16, each tile in steps of four blocks (128 columns),
 * a step storing its blocks one after the other, 16 rows each. Its scale
 * byte sits at
 *     (r / 16) * 16 * nb + (c / 4) * 64 + (c % 4) * 16 + r % 16.
 * The weight of gate row f, column h is E2M1(code) * 2^(scale - 127) of block
 * h / 32 of row f (MXFP4: blocks of 32 sharing one power-of-two scale;
 * pages: ds4.c `dsv4_e2m1fn_value_cpu`, `dsv4_fp4_act_quantize_row_inplace_cpu`;
 * goosedump `validate_tensors`, Mxfp4 expert tensors with F32 biases).
 * Supported scale bytes: 2..252 (outside that range results are
 * unspecified). moe_pack_experts writes this layout from row-major planes. */
typedef struct moe_blob_layout {
    uint64_t gate_q, up_q, down_q;
    uint64_t gate_s, up_s, down_s;
    uint64_t gate_b, up_b, down_b;
    uint64_t bytes;   /* end of the last plane: bytes the block reads per expert */
    uint64_t stride;  /* bytes rounded up to 4096 */
} moe_blob_layout;

/* Host-side row-major MXFP4 weights of n experts, as produced by a
 * quantiser: gate_q/up_q [n, F, H/2], down_q [n, H, F/2] (element 2i of a
 * row in the low nibble of byte i); gate_s/up_s [n, F, H/32], down_s
 * [n, H, F/32]; gate_b/up_b [n, F], down_b [n, H]. All host. */
typedef struct moe_expert_planes {
    const uint8_t *gate_q, *up_q, *down_q;
    const uint8_t *gate_s, *up_s, *down_s;
    const float *gate_b, *up_b, *down_b;
} moe_expert_planes;

/* Routing results (all device, caller-owned; any field may be NULL to skip it).
 *   topk_idx [T, k] int32  expert of slot j of token t, by descending logit,
 *                          equal logits ordered by ascending expert index
 *   topk_w   [T, k] float  route weight (route_scale * softmax of the selected)
 *   counts   [E]    int32  routes per expert
 *   offsets  [E+1]  int32  exclusive prefix sum of counts
 *   perm     [T*k]  int32  route id t*k+j at each position, grouped by expert,
 *                          ascending token inside a group
 *   inv      [T*k]  int32  position of route t*k+j, perm[inv[r]] == r
 *   route_counts [E] uint64  accumulated, not overwritten: each call adds its
 *                          routes per expert (the T*k selections; the shared
 *                          expert is not a selection). Zero it once, then pass
 *                          the same table (or row `layer` of a [layers][E]
 *                          table) on every call to profile expert use. Calls
 *                          that add into one table must be ordered (one stream).
 *                          A counter wraps after 2^64 selections (the page's
 *                          counter saturates; neither is reachable in practice).
 * Pages: goosedump `top_experts` (strict-greater insertion: descending value,
 * lower index first on ties), `mixture_of_experts_batch` (routes pushed per
 * expert in token order), `route_output_index` (route id token*k + slot),
 * `ExpertRouteProfile::record` (one count per selected expert per layer,
 * called from `mixture_of_experts` and `mixture_of_experts_batch`). */
typedef struct moe_route_out {
    int32_t *topk_idx;
    float *topk_w;
    int32_t *counts;
    int32_t *offsets;
    int32_t *perm;
    int32_t *inv;
    uint64_t *route_counts;
} moe_route_out;

/* Summary of a route profile table. Host only.
 *   counts       [layers][E] uint64, host: route_counts tables read back
 *   selections   out: sum of all counters, saturating at UINT64_MAX
 *   unique_layer_experts  out: number of (layer, expert) counters that are nonzero
 *   layer_unique [layers] int32 out (or NULL): nonzero counters of each layer
 * Returns MOE_OK, or MOE_ERR_INVALID_ARG (NULL counts or outputs, layers < 0,
 * E < 1). Page: goosedump `ExpertRouteProfile` (`selections`,
 * `unique_layer_experts`, `layer_unique_counts`). */
int moe_route_profile_summary(const uint64_t *counts, int32_t layers, int32_t E,
                              uint64_t *selections, uint64_t *unique_layer_experts,
                              int32_t *layer_unique);

/* Outputs of moe_route_locality, host arrays owned by the caller; every one is
 * overwritten.
 *   hist              [layers][E]     selections of each expert
 *   weight_hist       [layers][E]     sum of their route weights (float64)
 *   cache_hits        [n_caps][layers] hits of the simulated cache of size caps[c]
 *   cache_weight_hits [n_caps][layers] route weight of those hits
 *   adjacent_pairs    [layers]        tokens compared with the one before them
 *   overlap_sum       [layers]        sum over those pairs of |shared| / k
 *   jaccard_sum       [layers]        sum of |shared| / (2k - |shared|)
 * The cache arrays may be NULL when n_caps is 0. */
typedef struct moe_locality_out {
    uint64_t *hist;
    double *weight_hist;
    uint64_t *cache_hits;
    double *cache_weight_hits;
    uint64_t *adjacent_pairs;
    double *overlap_sum;
    double *jaccard_sum;
} moe_locality_out;

/* Routed-expert locality of a decode trace. Host only.
 *   idx      [positions][layers][k] int32, host: the selected experts of
 *            consecutive decode positions (topk_idx of one T=1 call per layer
 *            and position, read back)
 *   weights  [positions][layers][k] float32, host: their route weights (topk_w)
 *   caps     [n_caps] int32, host: cache sizes, each in [1, E] (ds4.c's
 *            candidates are 1, 2, 4, ..., 256, 384, those not above E)
 * Per layer, in position order and slot order 0..k-1, each selection of an
 * expert in [0, E) counts in hist / weight_hist and is offered to one cache per
 * size: a list of at most caps[c] experts, most recent first, where a present
 * expert is a hit (added to cache_hits / cache_weight_hits) and moves to the
 * front, and an absent one is put at the front, the last entry dropping out
 * past caps[c]. From the second position on, each token is compared with the
 * previous one: |shared| counts the previous token's slots whose expert the
 * current token also selected (indices outside [0, E) included). Every
 * call starts from empty caches and zeroed outputs.
 * Returns MOE_OK, or MOE_ERR_INVALID_ARG (a NULL input or output, positions < 0,
 * layers < 1, k < 1, E < 1, n_caps outside [0, 16], a size outside [1, E]).
 * Page: antirez ds4.c, the Metal routed-expert locality profiler (its record
 * and cache-use steps). */
int moe_route_locality(const int32_t *idx, const float *weights, int64_t positions,
                       int32_t layers, int32_t k, int32_t E, const int32_t *caps,
                       int32_t n_caps, const moe_locality_out *out);

/* Hotlist order of a locality histogram. Host only.
 *   hist, weight_hist  [layers][E], as moe_route_locality writes them
 *   order              [layers * E] int32 out: every layer * E + expert, ranked by
 *                      count (descending), route weight (descending), layer, then
 *                      expert (ascending). A layer's own ranking is this order
 *                      restricted to that layer.
 * Returns MOE_OK or MOE_ERR_INVALID_ARG (NULL pointer, layers < 1, E < 1,
 * layers * E above 2^31 - 1, or a weight sum that is not finite).
 * Page: antirez ds4.c, the profiler's layer and hotlist writers (their sort
 * orders). */
int moe_route_hotlist(const uint64_t *hist, const double *weight_hist, int32_t layers,
                      int32_t E, int32_t *order);

/* Fill *layout for experts of this shape (uses H and F only). Host only.
 * Returns MOE_OK or MOE_ERR_INVALID_ARG. */
int moe_blob_layout_get(const moe_shape *shape, moe_blob_layout *layout);

/* Pack n experts from row-major planes into dst in the tiled blob layout
 * (host, n * layout.stride bytes, padding zeroed). Host only; MOE_OK or
 * MOE_ERR_INVALID_ARG. */
int moe_pack_experts(const moe_shape *shape, int32_t n, const moe_expert_planes *planes,
                     uint8_t *dst);

/* Device workspace bytes that moe_route / moe_forward_decode /
 * moe_forward_prefill need for this shape (the largest of the three).
 * Returns 0 for an invalid shape. Host only. The caller allocates the
 * workspace once per shape and passes it to every call, so no call allocates
 * (page: antirez ds4.c keeps every decode temporary in one preallocated
 * scratch, `ds4_cpu_decode_scratch`, and its allocation guard,
 * `ds4_alloc_guard_begin` / `_check`, rejects allocations during a guarded
 * phase). */
size_t moe_workspace_bytes(const moe_shape *shape);

/* DeepSeek-V4 routing variants (page: antirez ds4.c `ds4_layer_weights`
 * holds `ffn_exp_probs_b` and `ffn_gate_tid2eid`; `weights_validate_layout`
 * declares exp_probs_b F32 [n_expert], optional, and tid2eid I32
 * [n_expert_used, n_vocab] for the layers below `n_hash_layer`, 3 in
 * `DS4_SHAPE_FLASH`; the routing arithmetic itself is cut off the page).
 * Pass NULL, or a struct with both pointers NULL, for plain top-k routing.
 *   sel_bias   [E] float32, device, or NULL: selection-only bias. The k
 *              experts are the top-k of logit + sel_bias (fp64; equal values
 *              to the lower index); the route weights stay route_scale *
 *              softmax over the selected experts' own logits.
 *   tid2eid    [vocab, k] int32, device, or NULL: hash routing. Token t
 *              takes the k experts of row token_ids[t], in row order, with
 *              weights route_scale * softmax over their logits (the router
 *              still runs); sel_bias is not read.
 *   token_ids  [T] int32, device; required with tid2eid
 *   vocab      rows of tid2eid, >= 1 with tid2eid
 * Token ids outside [0, vocab) and table entries outside [0, E) are clamped
 * into those ranges (results are then unspecified; every access stays in
 * bounds). Rows should hold k distinct experts. MOE_ERR_INVALID_ARG for a
 * table without ids or vocab < 1, or a pointer not 4-byte aligned. */
typedef struct moe_routing {
    const float *sel_bias;
    const int32_t *tid2eid;
    const int32_t *token_ids;
    int32_t vocab;
} moe_routing;

/* Routing only: optional RMSNorm, router logits in fp64, top-k, route weights,
 * per-expert histogram, exclusive scan and stable permutation.
 *   x        [T, H] float32 or bfloat16 (shape->act_dtype), device
 *   norm_w   [H] float32 RMSNorm weight or NULL (no norm), device
 *   router_w [E, H] float32, router_b [E] float32, device
 *   routing  NULL (plain top-k) or a routing variant (moe_routing)
 *   x, norm_w and router_w 16-byte aligned (MOE_ERR_INVALID_ARG otherwise)
 *   out      non-NULL; NULL fields are not written (see moe_route_out)
 *   ws       >= moe_workspace_bytes(shape) bytes, 256-byte aligned, device
 * Pages: goosedump `mixture_of_experts_batch` (router matmul, add_bias_batch,
 * top_experts, softmax, routes_by_expert). */
int moe_route(const moe_shape *shape, const void *x, const float *norm_w,
              const float *router_w, const float *router_b, const moe_routing *routing,
              const moe_route_out *out, void *ws, size_t ws_bytes, hipStream_t stream);

/* The whole block for a few tokens (T <= 64): streams only the k selected
 * experts' bytes per token with GEMV kernels on the matrix cores.
 *   hidden   [T, H] float32 or bfloat16, device; it is also the residual
 *   experts  E packed blobs, layout.stride bytes apart, device
 *   shared   n_shared packed blobs (same layout) or NULL when n_shared == 0
 *   out      [T, H] float32, device; may alias a float32 hidden
 *   route_out NULL, or routing results to export (fields may be NULL)
 *   norm_w, router_w, router_b, routing, ws as for moe_route
 *   hidden, out, norm_w and router_w 16-byte aligned, expert blobs 256-byte
 * Pages: goosedump `mixture_of_experts` (router matvec, add_bias,
 * top_experts, softmax, per expert: matrix_vector_pair, biases, swiglu,
 * matrix_vector, bias, times the route weight, summed over slots). */
int moe_forward_decode(const moe_shape *shape, const void *hidden, const float *norm_w,
                       const float *router_w, const float *router_b, const moe_routing *routing,
                       const uint8_t *experts, const uint8_t *shared, float *out,
                       const moe_route_out *route_out, void *ws, size_t ws_bytes,
                       hipStream_t stream);

/* The whole block for a token batch: routing, permutation, grouped GEMMs on
 * the matrix cores (gate/up with bias and clamped SwiGLU fused; down with
 * bias and route weight fused), then a combine that adds each token's routes
 * to its residual in a fixed order (deterministic). Same arguments as
 * moe_forward_decode; any T up to the workspace and 2^32-byte FP8-term limits
 * (MOE_ERR_UNSUPPORTED past them). out may alias a float32 hidden.
 * Pages: goosedump `mixture_of_experts_batch`, `expert_batch_output`,
 * `mix_expert_outputs`. */
int moe_forward_prefill(const moe_shape *shape, const void *hidden, const float *norm_w,
                        const float *router_w, const float *router_b, const moe_routing *routing,
                        const uint8_t *experts, const uint8_t *shared, float *out,
                        const moe_route_out *route_out, void *ws, size_t ws_bytes,
                        hipStream_t stream);

/* Size of the fixed device scratch of moe_forward_decode_noalloc: 32 MiB per
 * GPU, enough for every decode shape up to T = 64 at gpt-oss-20b and
 * DeepSeek-V4-Flash sizes. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)

/* moe_forward_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc): the workspace is a fixed device array of
 * MOE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held from module
 * load until the process ends. The call allocates nothing, on the host or the
 * device; the caller still owns every input and output.
 *   arguments, layouts, results and errors as for moe_forward_decode
 *   MOE_ERR_UNSUPPORTED when moe_workspace_bytes(shape) exceeds
 *       MOE_NOALLOC_SCRATCH_BYTES (checked first, before any device call)
 * Every call on one GPU shares that GPU's array (nothing in it needs to start
 * zeroed; each call writes what it reads). Calls that overlap on one GPU -
 * on different streams, or from different host threads without ordering -
 * race on it and give undefined results; order them on one stream. The device
 * is the calling thread's current HIP device, which must own `stream`. */
int moe_forward_decode_noalloc(const moe_shape *shape, const void *hidden, const float *norm_w,
                               const float *router_w, const float *router_b, const moe_routing *routing,
                               const uint8_t *experts, const uint8_t *shared, float *out,
                               const moe_route_out *route_out, hipStream_t stream);

/* How moe_forward_prefill tiles its grouped GEMMs for a shape (host only; for
 * profilers and benchmarks that count the matrix-core work a call issues).
 *   with_norm   nonzero when the call passes an RMSNorm weight
 * Fills *plan; MOE_OK or MOE_ERR_INVALID_ARG (bad shape, NULL plan).
 * Page: goosedump `mixture_of_experts_batch` groups a batch's routed rows by
 * expert (`routes_by_expert`) and runs each expert over its rows; the plan is
 * this library's tiling of those per-expert row groups. */
typedef struct moe_prefill_plan_t {
    int32_t tile_rows;         /* routed rows of one expert per tile: 16, 32 or 64 */
    int32_t x_terms;           /* FP8 terms of the expert input in the gate/up products (3 or 4);
                                  1: a bfloat16 input with no RMSNorm, taken as it is by the
                                  bfloat16 matrix cores against weights decoded to bfloat16;
                                  0: the MX-FP4 expert input (act_quant >= 1), one FP4 operand */
    int32_t act_terms;         /* FP8 terms of the SwiGLU output in the down products;
                                  0: its MX-FP4 codes (act_quant = 2) */
    int32_t gate_up_features;  /* features (gate and up rows each) per gate/up work item */
    int32_t down_rows;         /* hidden rows per down work item */
} moe_prefill_plan_t;
int moe_prefill_plan(const moe_shape *shape, int32_t with_norm, moe_prefill_plan_t *plan);

/* Export the MX-FP4 expert input of the quantised mode (act_quant = 1) as
 * the prefill kernels compute with it, for bit-exact checks against the
 * round trip's definition (page: antirez ds4.c
 * `dsv4_fp4_act_quantize_row_inplace_cpu`, `dsv4_e2m1fn_dequant_cpu`).
 *   x, norm_w    as for moe_route (norm_w NULL: no norm)
 *   codes  [T, H / 2] bytes, device: E2M1 codes (bit 3 the sign, bits 0-2
 *          the magnitude index), element 2i in the low nibble of byte i
 *   scales [T, H / 32] bytes, device: E8M0 scale byte e + 127 per block
 *   ws     >= moe_workspace_bytes(shape) bytes, 256-byte aligned, device
 * shape->act_quant is not read. MOE_ERR_INVALID_ARG on NULL pointers or a
 * bad shape. */
int moe_act_quant_debug(const moe_shape *shape, const void *x, const float *norm_w,
                        uint8_t *codes, uint8_t *scales, void *ws, size_t ws_bytes,
                        hipStream_t stream);

/* Export the weights the kernels compute with, for bit-exact checks against
 * the MXFP4 definition (page: antirez ds4.c `dsv4_e2m1fn_value_cpu`, the
 * eight E2M1 magnitudes and the sign bit, times the block's power-of-two
 * scale).
 *   blob   one packed expert, device
 *   which  0 gate [F, H], 1 up [F, H], 2 down [H, F]
 *   path   0: decoded with the gfx950 scaled FP4-to-float32 converts;
 *          1: decoded with the scaled FP4-to-bfloat16 converts, widened;
 *          2: decoded by the block-scaled matrix core, as every forward
 *             kernel uses the weights (B operand one-hot 1.0)
 *   out    float32 [rows, cols] row-major, device */
int moe_dequant_debug(const moe_shape *shape, const uint8_t *blob, int32_t which, int32_t path,
                      float *out, hipStream_t stream);

/* Kernels of the block, as named by moe_profile_next_launch. */
typedef enum moe_kernel_id {
    MOE_KERNEL_RMSNORM = 0,
    MOE_KERNEL_ROUTER = 1,          /* router logits, either form */
    MOE_KERNEL_TOPK = 2,
    MOE_KERNEL_PERMUTE = 3,
    MOE_KERNEL_DECODE_GATE_UP = 4,
    MOE_KERNEL_DECODE_DOWN = 5,
    MOE_KERNEL_GATE_UP_GEMM = 6,
    MOE_KERNEL_DOWN_GEMM = 7,
    MOE_KERNEL_QUANTIZE = 8,        /* reserved: the FP8 terms of the expert input
                                       are made inside the router launch */
    MOE_KERNEL_COMBINE = 9          /* prefill: residual + sum of the routes' outputs */
} moe_kernel_id;

/* Measurement hook (for benchmarks and profilers, not needed to compute):
 * on the calling thread, the next launch of `kernel` made by any call of
 * this library carries `start` and `stop`, which the runtime stamps with
 * that kernel dispatch's own start and end (hipExtLaunchKernel events), so
 * hipEventElapsedTime(start, stop) is the kernel's duration. The events are
 * caller-owned and must allow timing; not for use under stream capture.
 * One-shot: the hook disarms after that launch; kernel < 0 disarms it.
 * Host only; MOE_OK or MOE_ERR_INVALID_ARG. */
int moe_profile_next_launch(int32_t kernel, hipEvent_t start, hipEvent_t stop);

/* Message of the last failing call on this thread ("" if none). Every call
 * returns a moe_status and leaves its reason here (page: turbospark-runtime
 * `produce_real_gpt_oss` rejects requests it does not support with a typed
 * error carrying a message, `RealForwardError::Unsupported`; a C caller gets
 * MOE_ERR_UNSUPPORTED and this text). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
