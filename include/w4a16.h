/*
 * w4a16.h - C ABI of the MI355X (gfx950) W4A16 group-32 library.
 *
 * The operation (web page "The Weight of Precision: Building Native INT4
 * Quantization for a Custom Speculative Decoding Engine", section "The Kernel:
 * w4a16_gemm"): y = x * W where W is stored as symmetric INT4 codes
 * (value = nibble - 8, range [-8, 7]) packed eight per int32 along the input
 * dimension K, with one float32 scale per group of 32 input rows per output
 * column.  Activations are float32 or bf16; accumulation and outputs are
 * float32 (page "The Final Wire: How a Single Edit Integrated INT4
 * Quantization into a Native DDTree Inference Engine", section "The
 * Multi-Step Integration Chain").  The same path serves the dense SwiGLU MLP
 * and the routed MoE experts (page "The Final Wire", section "What the Edit
 * Actually Changes").
 *
 * Conventions for every entry point:
 *  - Pointers to tensors are DEVICE pointers owned by the caller and must be
 *    16-byte aligned.  Descriptors (w4a16_weight_t) and out-descriptors are
 *    HOST pointers.  The library never allocates or frees device memory and
 *    never synchronises the stream.
 *  - Work is enqueued asynchronously on `stream`.  The returned status covers
 *    host-side argument checks and launch errors only; a fault inside a kernel
 *    surfaces at the caller's next synchronisation.
 *  - There is no fallback path of any kind: an unsupported argument returns
 *    an error and enqueues nothing.
 *  - Row-major throughout: x is [M][K], y is [M][N].  y must not alias x.
 *  - M == 0 (or a zero-sized weight) returns W4A16_OK and enqueues nothing.
 *  - Workspaces come from the caller, sized by the matching *_workspace_bytes
 *    query, and must be zero-filled once (w4a16_workspace_init) before their
 *    first use; every call leaves its workspace ready for the next call.  Two
 *    calls that may run at the same time must not share a workspace.
 *  - The library keeps no mutable global state; calls on different streams
 *    with different workspaces are independent.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#if defined(__GNUC__) || defined(__clang__)
#define W4A16_API __attribute__((visibility("default")))
#else
#define W4A16_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4A16_OK = 0,
  W4A16_ERR_INVALID_ARG = 1, /* null/misaligned pointer, negative size, bad id range */
  W4A16_ERR_UNSUPPORTED = 2, /* group size not 32/64/128, K % group != 0, N % 64 != 0, wrong layout */
  W4A16_ERR_WORKSPACE = 3,   /* workspace smaller than the *_workspace_bytes query */
  W4A16_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} w4a16_status_t;

typedef enum { W4A16_F32 = 0, W4A16_BF16 = 1 } w4a16_dtype_t;

/*
 * Weight layouts (both hold exactly K*N/8 int32 words per expert).
 *  CANONICAL: qw[E][K/8][N]; nibble j (bits 4j..4j+3) of word (i, n) holds row
 *             k = 8i + j.  This is the interchange format written by a
 *             quantizer (w4a16_quantize).
 *  GROUPED:   qw[E][K/32][N/64][64][4]; for 32-row block g and 64-column
 *             block j, the 16-byte slot 16b + l (b = 0..3, l = 0..15) holds
 *             canonical word 4g + b (rows 32g + 8b .. 32g + 8b + 7) of the
 *             columns 64j + 4l .. 64j + 4l + 3, in column order.  One matrix
 *             core lane reads one slot per block: its four columns' codes for
 *             one 8-row block.  The code layout does not depend on the group
 *             size.  Compute entry points read this layout only;
 *             w4a16_prepack converts.
 * Scales are sc[E][K/group_size][N] float32 in both layouts: row k of
 * column n uses sc[e][k / group_size][n].  Group sizes 32, 64 and 128 are
 * supported (the pages target 32; page "The First Line of Code", section
 * "What the Edit Actually Does", calls the group size configurable).
 */
typedef enum { W4A16_LAYOUT_CANONICAL = 0, W4A16_LAYOUT_GROUPED = 1 } w4a16_layout_t;

typedef struct {
  const int32_t* qw;       /* device: packed codes, layout per `layout` */
  const float* scales;     /* device: sc[E][K/group_size][N] */
  int32_t K;               /* input dim, multiple of group_size */
  int32_t N;               /* output dim, multiple of 64 */
  int32_t group_size;      /* rows per scale: 32, 64 or 128 */
  int32_t num_experts;     /* 1 for a dense weight; E for an expert stack */
  w4a16_layout_t layout;
} w4a16_weight_t;

/* Human-readable name of a status code (static storage, never NULL). */
W4A16_API const char* w4a16_status_string(w4a16_status_t status);

/*
 * Zero-fill a workspace of `bytes` bytes (a fill kernel, no memset node, so it
 * may be captured in a graph).  Call once after allocating a workspace.
 */
W4A16_API w4a16_status_t w4a16_workspace_init(void* ws, size_t bytes, hipStream_t stream);

/*
 * Quantize float32 weights w[E][K][N] into CANONICAL codes qw[E][K/8][N] and
 * scales sc[E][K/32][N] (page "The Weight of Precision", section "The Reference
 * and Bundle Pipeline": the quantizer's outputs are packed int32 codes and
 * float32 per-group scales).  The pages leave the rule open; this library
 * uses scale = max|w| / 7 per 32-row group and column (one IEEE float32
 * division) and code = clamp(round-half-even(w / scale), -8, 7) with the
 * quotient formed in float64; an all-zero group gets scale 0 and code 0.
 * Weights must be finite (not checked on the device).  qw_bytes and
 * scales_bytes are the sizes of the caller's output buffers: at least
 * E * K/8 * N * 4 and E * K/32 * N * 4 bytes.
 * Errors: INVALID_ARG for null/misaligned pointers, K, N, E < 0 or an output
 * buffer smaller than its size above (nothing is enqueued then);
 * UNSUPPORTED for K % 32 != 0.
 */
W4A16_API w4a16_status_t w4a16_quantize(const float* w, int32_t K, int32_t N, int32_t num_experts,
                              int32_t* qw, size_t qw_bytes, float* scales, size_t scales_bytes,
                              hipStream_t stream);

/*
 * w4a16_quantize with group_size rows per scale (32, 64 or 128): scales are
 * sc[E][K/group_size][N] (scales_bytes >= E * K/group_size * N * 4),
 * scale = max|w| / 7 over each group, codes as above.  Errors as
 * w4a16_quantize, plus UNSUPPORTED for another group size or
 * K % group_size != 0.
 */
W4A16_API w4a16_status_t w4a16_quantize_group(const float* w, int32_t K, int32_t N, int32_t num_experts,
                                    int32_t group_size, int32_t* qw, size_t qw_bytes, float* scales,
                                    size_t scales_bytes, hipStream_t stream);

/*
 * Bytes of GROUPED codes that w4a16_prepack writes for the weight `w`
 * (E * K/8 * N * 4: the GROUPED layout is a permutation of the canonical
 * words, so the size does not change; gate and up stay separate weights).
 * 0 for a descriptor that fails the checks of w4a16_prepack.
 */
W4A16_API size_t w4a16_prepacked_bytes(const w4a16_weight_t* w);

/*
 * Permute CANONICAL codes into the GROUPED layout the compute kernels stream
 * (one-time load step; the weight and scale maps of page "The Final Wire",
 * section "The Multi-Step Integration Chain").  Scales are not moved: `out`
 * receives a GROUPED descriptor that points at `dst_qw` and at src->scales.
 * dst_qw (dst_bytes bytes) must hold w4a16_prepacked_bytes(src) bytes and
 * must not overlap src->qw.  Errors: INVALID_ARG (null/misaligned, out ==
 * NULL, overlap, dst_bytes too small; nothing is enqueued then), UNSUPPORTED
 * (src not CANONICAL, group size, K % group size, N % 64).
 */
W4A16_API w4a16_status_t w4a16_prepack(const w4a16_weight_t* src, int32_t* dst_qw, size_t dst_bytes,
                             w4a16_weight_t* out, hipStream_t stream);

/*
 * Test hook, not on the hot path: materialise out[E][K][N] = float32(q * s),
 * the exact product rounded once (page "The First Line of Code: Implementing
 * W4A16 Quantization in a Native Speculative Decoding Engine", section "What
 * the Edit Actually Does": dequantization must be identical to the
 * reference's).  Accepts both layouts.  out_bytes is the size of `out`, at
 * least E * K * N * 4.  Errors: INVALID_ARG (null/misaligned, out_bytes too
 * small; nothing is enqueued then), UNSUPPORTED (group size, K % group size,
 * N % 64, layout).
 */
W4A16_API w4a16_status_t w4a16_dequantize(const w4a16_weight_t* w, float* out, size_t out_bytes,
                                hipStream_t stream);

/* Bytes of workspace w4a16_gemm needs for this M, weight and activation type. */
W4A16_API size_t w4a16_gemm_workspace_bytes(int32_t M, const w4a16_weight_t* w, w4a16_dtype_t xt);

/*
 * y[M][N] = x[M][K] * dequant(W), float32 accumulation and output (page "The
 * Weight of Precision", section "The Kernel: w4a16_gemm").  W must be a dense
 * (num_experts == 1) GROUPED weight.  Up to 8 rows (float32 activations) or
 * 16 rows (bf16) run a split-K GEMV on the matrix cores (all rows in one MFMA
 * tile); larger M runs 64-row MFMA tiles, and bf16 from 256 rows 256 x 128
 * tiles.
 * Deterministic: the same inputs give bitwise the same y.
 * Errors: INVALID_ARG (null/misaligned, M < 0, bad dtype, y aliasing x),
 * UNSUPPORTED (layout, group size, K % group size, N % 64, num_experts != 1),
 * WORKSPACE (ws_bytes too small), HIP (launch failure).
 */
W4A16_API w4a16_status_t w4a16_gemm(const void* x, w4a16_dtype_t xt, int32_t M, const w4a16_weight_t* w,
                          float* y, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Measurement variant of w4a16_gemm: identical work and results, and in
 * addition brackets each kernel it launches with two of the caller's events
 * (events[2i] at the start and events[2i+1] at the end of kernel i, taken by
 * the runtime from the kernel's own dispatch), at most `capacity` events;
 * *recorded (if not NULL) receives how many were used.  Up to 8 rows
 * (float32) or 16 (bf16) it launches one GEMV kernel; above, the activation
 * pieces and then the MFMA tiles.  Errors as w4a16_gemm, plus INVALID_ARG for
 * capacity < 0 or events == NULL with capacity > 0.
 */
W4A16_API w4a16_status_t w4a16_gemm_timed(const void* x, w4a16_dtype_t xt, int32_t M, const w4a16_weight_t* w,
                                          float* y, void* ws, size_t ws_bytes, hipStream_t stream,
                                          hipEvent_t* events, int32_t capacity, int32_t* recorded);

/* Bytes of workspace w4a16_swiglu_mlp needs. */
W4A16_API size_t w4a16_swiglu_mlp_workspace_bytes(int32_t M, w4a16_dtype_t xt, const w4a16_weight_t* gate,
                                        const w4a16_weight_t* up, const w4a16_weight_t* down);

/*
 * Dense SwiGLU MLP: y = (silu(x Wg) * (x Wu)) Wd with silu(z) = z / (1 + e^-z)
 * (page "The Final Wire", section "What the Edit Actually Changes": the dense
 * MLP's gate, up and down projections run through the W4A16 path; page "The
 * Weight of Precision", section "The Context That Produced This Message" names
 * SwiGLU).  gate and up are [H -> I], down is [I -> H], all dense GROUPED.
 * x is [M][H], y is [M][H] float32.  The gate and up projections run in one
 * pass with the SiLU-times-up product formed in the epilogue.  The down
 * projection reads the intermediate h[M][I] as f16 pieces (two for float32 x,
 * one for bf16 x), scaled by a power of two per row: on the GEMV path and
 * when a tile launch runs unsplit, h is first stored in the workspace in
 * float32; when both tile launches split K, the gate/up split sums become
 * pieces directly, scaled per row and down K split, and h is not stored.
 * Errors as w4a16_gemm, plus UNSUPPORTED if the three shapes do not chain.
 */
W4A16_API w4a16_status_t w4a16_swiglu_mlp(const void* x, w4a16_dtype_t xt, int32_t M,
                                const w4a16_weight_t* gate, const w4a16_weight_t* up,
                                const w4a16_weight_t* down, float* y, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/*
 * Measurement variant of w4a16_swiglu_mlp: identical work and results, and in
 * addition brackets each kernel it launches with two of the caller's events:
 * events[2i] at the start and events[2i+1] at the end of kernel i, taken by
 * the runtime from the kernel's own dispatch (hipExtLaunchKernel), so their
 * interval is the kernel's execution time without the launch gap.  At most
 * `capacity` events (kernels beyond capacity / 2 run unbracketed); *recorded
 * (if not NULL) receives how many were used.  Up to 8 rows (float32) or 16
 * (bf16) the dense MLP launches two kernels (fused gate/up
 * GEMV with the SwiGLU epilogue, down GEMV); for larger M four or five
 * (activation pieces, fused gate/up MFMA tiles, pieces of the intermediate,
 * down MFMA tiles, and the sum of the down projection's K splits when it is
 * split).  Events are created and owned by the caller.  Errors as w4a16_swiglu_mlp, plus INVALID_ARG for
 * capacity < 0 or events == NULL with capacity > 0, and HIP if recording fails.
 */
W4A16_API w4a16_status_t w4a16_swiglu_mlp_timed(const void* x, w4a16_dtype_t xt, int32_t M,
                                                const w4a16_weight_t* gate, const w4a16_weight_t* up,
                                                const w4a16_weight_t* down, float* y, void* ws,
                                                size_t ws_bytes, hipStream_t stream,
                                                hipEvent_t* events, int32_t capacity,
                                                int32_t* recorded);

/* Size of the static scratch array behind w4a16_swiglu_mlp_static (64 MiB per GPU). */
#define W4A16_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * w4a16_swiglu_mlp without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The same kernels and results as
 * w4a16_swiglu_mlp (bitwise), with the workspace taken from a static device
 * array of W4A16_STATIC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends.  The call allocates nothing and frees
 * nothing; its first call on a device looks up the array's address there and
 * zeroes its first 64 KiB with a fill kernel on `stream`.  Every call on one
 * GPU shares that GPU's array, so calls that may overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller.  The
 * caller still passes x and y.  Errors as w4a16_swiglu_mlp, plus WORKSPACE
 * (nothing enqueued) when the call needs more scratch than the array holds
 * (w4a16_swiglu_mlp_workspace_bytes above W4A16_STATIC_SCRATCH_BYTES; the
 * hidden 7168 / intermediate 18432 MLP fits up to M = 64 with float32 x and
 * up to M = 192 with bf16 x) and HIP if the array's address cannot be looked
 * up.
 */
W4A16_API w4a16_status_t w4a16_swiglu_mlp_static(const void* x, w4a16_dtype_t xt, int32_t M,
                                                 const w4a16_weight_t* gate, const w4a16_weight_t* up,
                                                 const w4a16_weight_t* down, float* y, hipStream_t stream);

/*
 * Router: the top_k experts of every token and their gate weights (page "The
 * Final Wire", section "What the Edit Actually Changes": for each token the
 * router selects top-k experts).  The pages give no gating rule; this library
 * takes, per token row of logits[M][E] (float32, finite), the top_k largest
 * logits in descending order, equal logits in ascending expert index, and
 * writes their expert ids to topk_ids[M][top_k] (int32, distinct per token)
 * and softmax weights over those top_k logits, exp(l - l_max) / sum, to
 * topk_w[M][top_k] (float32).  The outputs feed w4a16_moe_route and
 * w4a16_moe_grouped directly.  Deterministic.
 * Errors: INVALID_ARG (null/misaligned, M < 0, E < 1, top_k < 1, top_k > E),
 * UNSUPPORTED (E > 1024 or top_k > 32).  M == 0 enqueues nothing.
 */
W4A16_API w4a16_status_t w4a16_moe_topk(const float* logits, int32_t M, int32_t E, int32_t top_k,
                              int32_t* topk_ids, float* topk_w, hipStream_t stream);

/*
 * Group (token, slot) pairs by expert (page "The Final Wire", section "What
 * the Edit Actually Changes": the router picks top-k experts per token and
 * each expert runs its own projections).  Pair p = t * top_k + slot.  Outputs,
 * all device int32: counts[E]; offsets[E+1] (exclusive prefix sum of counts);
 * sorted_pairs[M*top_k], pair ids grouped by expert with ascending token
 * inside an expert (unique, since a token's top_k ids are distinct); inv[M*top_k],
 * the position of each pair in sorted_pairs.  topk_ids are int32 in [0, E),
 * distinct per token; ids outside [0, E) are skipped on the device (they
 * appear in no list and their inv entry is -1) rather than read out of bounds.
 * Errors: INVALID_ARG (null/misaligned, M < 0, top_k < 1, top_k > E, E < 1),
 * UNSUPPORTED (E > 6144).
 */
W4A16_API w4a16_status_t w4a16_moe_route(const int32_t* topk_ids, int32_t M, int32_t top_k, int32_t E,
                               int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                               int32_t* inv, hipStream_t stream);

/* Bytes of workspace w4a16_moe_grouped needs. */
W4A16_API size_t w4a16_moe_workspace_bytes(int32_t M, int32_t top_k, w4a16_dtype_t xt,
                                 const w4a16_weight_t* gate, const w4a16_weight_t* up,
                                 const w4a16_weight_t* down);

/*
 * Routed-expert SwiGLU MoE layer (page "The Final Wire", section "What the
 * Edit Actually Changes"):
 *   y[t] = sum over slot of topk_w[t][slot] * MLP_e(x[t]),  e = topk_ids[t][slot],
 * summed in slot order, MLP_e as in w4a16_swiglu_mlp with expert e's weights.
 * gate/up are GROUPED stacks [E][H -> Ie], down [E][Ie -> H].  x [M][H], topk_ids
 * and topk_w [M][top_k] (int32 / float32), y [M][H] float32.  The routing lists
 * (as w4a16_moe_route), the per-pair intermediate and the per-pair outputs
 * live in the workspace; per-expert row counts never leave the device.  The
 * per-pair intermediate and outputs are stored in float32 with float32 x and
 * in bf16 (round to nearest even) with bf16 x; the combine sums the outputs
 * in float32.
 * Experts with at most 8 rows (float32 activations) or 16 rows (bf16) run on
 * the GEMV kernels, heavier experts on MFMA tiles of 64 rows.
 * Errors as w4a16_swiglu_mlp plus INVALID_ARG for top_k < 1 or top_k > E and
 * UNSUPPORTED for more than 6144 experts.
 */
W4A16_API w4a16_status_t w4a16_moe_grouped(const void* x, w4a16_dtype_t xt, int32_t M,
                                 const int32_t* topk_ids, const float* topk_w, int32_t top_k,
                                 const w4a16_weight_t* gate, const w4a16_weight_t* up,
                                 const w4a16_weight_t* down, float* y, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/* Bytes of workspace w4a16_moe_grouped_shared needs (0 for invalid arguments). */
W4A16_API size_t w4a16_moe_shared_workspace_bytes(int32_t M, int32_t top_k, w4a16_dtype_t xt,
                                        const w4a16_weight_t* gate, const w4a16_weight_t* up,
                                        const w4a16_weight_t* down, const w4a16_weight_t* shared_gate,
                                        const w4a16_weight_t* shared_up,
                                        const w4a16_weight_t* shared_down);

/*
 * MoE layer with a shared expert (page "The Weight of Precision", section "The
 * Engine Dispatch: Model::linear": the shared expert runs on the INT4 path
 * beside the routed experts; the pages do not say how it joins the layer):
 *   y[t] = w4a16_moe_grouped's routed sum + MLP_shared(x[t]),
 * the shared term added last with weight 1.  shared_gate/up/down are one
 * GROUPED SwiGLU MLP (num_experts == 1) of the routed experts' shapes.  The
 * shared expert runs as one more expert inside the same grouped launches
 * (GEMV items of up to 8 rows while M <= 64, MFMA tiles beyond), so it
 * overlaps the routed experts instead of following them.  Arguments,
 * workspace and errors as
 * w4a16_moe_grouped, plus INVALID_ARG for a null shared descriptor and
 * UNSUPPORTED for a shared expert of another shape or with num_experts != 1.
 */
W4A16_API w4a16_status_t w4a16_moe_grouped_shared(const void* x, w4a16_dtype_t xt, int32_t M,
                                        const int32_t* topk_ids, const float* topk_w, int32_t top_k,
                                        const w4a16_weight_t* gate, const w4a16_weight_t* up,
                                        const w4a16_weight_t* down, const w4a16_weight_t* shared_gate,
                                        const w4a16_weight_t* shared_up,
                                        const w4a16_weight_t* shared_down, float* y, void* ws,
                                        size_t ws_bytes, hipStream_t stream);

/*
 * Measurement variant of w4a16_moe_grouped: identical work and results, and in
 * addition brackets each kernel it launches with two of the caller's events,
 * as w4a16_swiglu_mlp_timed does: events[2i] at the start and events[2i+1] at
 * the end of kernel i, taken by the runtime from the kernel's own dispatch, at
 * most `capacity` events; *recorded (if not NULL) receives how many were
 * used.  Kernels in launch order: expert grouping; gate/up GEMV for the light
 * experts (at most 8 rows with float32 activations, 16 with bf16); when some
 * expert can be heavier, activation pieces (one row per token) and gate/up
 * MFMA tiles; down GEMV; then pieces of the intermediate and down MFMA tiles;
 * weighted combine.
 * Errors as w4a16_moe_grouped, plus INVALID_ARG for capacity < 0 or
 * events == NULL with capacity > 0, and HIP if recording fails.
 */
W4A16_API w4a16_status_t w4a16_moe_grouped_timed(
    const void* x, w4a16_dtype_t xt, int32_t M, const int32_t* topk_ids, const float* topk_w,
    int32_t top_k, const w4a16_weight_t* gate, const w4a16_weight_t* up,
    const w4a16_weight_t* down, float* y, void* ws, size_t ws_bytes, hipStream_t stream,
    hipEvent_t* events, int32_t capacity, int32_t* recorded);

#ifdef __cplusplus
}
#endif
#endif /* W4A16_H */
