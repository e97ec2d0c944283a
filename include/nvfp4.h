/*
 * nvfp4.h - C ABI of the MI355X (gfx950) W4A16 NVFP4 routed-expert MLP.
 *
 * The library runs the expert weights of a ModelOpt NVFP4 checkpoint as
 * stored, with bf16 activations (W4A16). It follows the TensorFold issue #308,
 * "GLM-5.3-Flash on CUDA: read nvidia/GLM-5.3-Flash-NVFP4 (ModelOpt NVFP4) as
 * stored, W4A16":
 *   - section "The checkpoint": weights are e2m1 codes with one e4m3 scale per
 *     16 inputs and one fp32 weight_scale_2 per tensor;
 *   - section "What the branch does": the routed experts run in one grouped
 *     NVFP4 kernel, each expert's weight_scale_2 applied to its product; the
 *     dense MLP runs on Fp4Linear with separate gate and up projections, each
 *     keeping its own tensor scale; activations stay bf16, the only type the
 *     grouped kernel accepts; at load the MTP layer's BF16 experts are
 *     quantized to NVFP4, one projection after another.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every tensor argument is a DEVICE pointer to contiguous row-major
 *           memory owned by the caller. The library never allocates, frees,
 *           copies to the host or synchronizes; all work is enqueued on
 *           `stream` (a hipStream_t; NULL is the default stream). It does not
 *           change the current device. Between calls it keeps only per-device
 *           caches of device properties (compute-unit count, resident
 *           workgroups per kernel), filled on first use and safe to fill from
 *           several threads; nvfp4_moe_grouped_noalloc alone also uses one
 *           fixed scratch array per GPU, held until the process ends.
 * bf16.     bf16 tensors are passed as uint16_t bit patterns.
 * Weights.  A weight [n, k] (out x in) is described by nvfp4_weight_t:
 *             codes   [groups, n, k/2]  uint8: element 2j of a row in the LOW
 *                                       nibble of byte j, 2j+1 in the high;
 *             scales  [groups, n, k/16] uint8: e4m3fn bits, one per 16
 *                                       consecutive inputs of a row;
 *             scale_2 [groups]          fp32 in device memory.
 *           A weight is W[n,k] = e2m1(code) * e4m3(scale[n, k/16]) * scale_2.
 *           `layout` says how codes and scales sit in memory:
 *             NVFP4_LAYOUT_ROWS    as above, the checkpoint's row-major order;
 *             NVFP4_LAYOUT_TILED32 the same bytes regrouped by blocks of 32
 *               rows (n % 32 == 0 and k % 256 == 0 required): for row block
 *               R = n/32, row r = n%32,
 *                 code byte of (n, k)  at ((g*n_blocks + R)*(k/32) + k/32)*512
 *                                          + r*16 + (k%32)/2,
 *                 scale of (n, k/16)   at ((g*n_blocks + R)*(k/256) + k/256)*512
 *                                          + r*16 + (k%256)/16,
 *               (n_blocks = n/32 of the tensor; k here is the input index) so
 *               that the 32 rows of a block read one 16-byte piece each from a
 *               contiguous 512-byte run: full-width loads and no partially used
 *               cache lines. nvfp4_pack writes either layout; nvfp4_relayout
 *               converts a stored (row-major) checkpoint. Row-major weights of
 *               any valid shape work everywhere; tiled ones run on the fast
 *               GEMM paths only (see each entry point).
 * Shapes.   k must be a positive multiple of 32 (whole 16-input groups, in
 *           32-wide tiles); n >= 1; row counts >= 0 (0 is a no-op).
 * Alignment. codes, scales, activations and outputs must be 16-byte aligned.
 * Errors.   Argument errors are detected on the host before anything is
 *           enqueued; on error nothing is written. A failed launch returns
 *           NVFP4_ERR_HIP. No C++ exception crosses this interface.
 * Numerics. Products run on matrix cores with fp32 accumulation over exactly
 *           dequantized weights; scale_2 multiplies the fp32 accumulator. The
 *           dense entry points feed bf16 operands. The routed kernels feed fp16
 *           operands: a dequantized weight (at most 6 significant bits, within
 *           [2^-10, 2688]) is exact in fp16, and each activation row is first
 *           scaled by a power of two that puts its largest |value| in
 *           [2^14, 2^15), so every bf16 value down to 2^-28 of the row maximum
 *           converts exactly (smaller ones round, far below the output's bf16
 *           rounding); the scaling is undone exactly in fp32 afterwards.
 *           The summation order of an output element is fixed by the shapes and
 *           by the kernel class of the call (see nvfp4_moe_grouped_class). Some
 *           classes split K over the waves of a workgroup and add the partial
 *           sums in a fixed wave order; none uses atomics on outputs. So the
 *           order never depends on the values, on the other rows or on the tile a
 *           row lands in: within one class results are bitwise reproducible,
 *           permuting the tokens permutes the outputs bit for bit, and a batch
 *           split into chunks gives the same bits as the whole batch.
 */
#ifndef NVFP4_MOE_EXPERT_AMD_NVFP4_H
#define NVFP4_MOE_EXPERT_AMD_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 8

#define NVFP4_LAYOUT_ROWS 0
#define NVFP4_LAYOUT_TILED32 1

typedef enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,        /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,       /* inconsistent or unsupported sizes (k % 32 != 0, n < 1, ...) */
  NVFP4_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
  NVFP4_ERR_WORKSPACE = 4,   /* workspace missing or smaller than the *_workspace_size() figure */
  NVFP4_ERR_UNSUPPORTED = 5, /* a request the kernels do not cover (e.g. W4A4 on fallback shapes) */
  NVFP4_ERR_HIP = 6,         /* the HIP runtime reported an error when enqueueing */
  NVFP4_ERR_SCRATCH = 7      /* more scratch than nvfp4_moe_grouped_noalloc's fixed buffer holds */
} nvfp4_status;

typedef struct nvfp4_weight_t {
  const uint8_t* codes;   /* [groups, n, k/2] bytes */
  const uint8_t* scales;  /* [groups, n, k/16] bytes */
  const float* scale_2;   /* [groups] */
  int64_t n;              /* output features (rows) */
  int64_t k;              /* input features, multiple of 32 */
  int32_t groups;         /* number of tensors (experts); 1 for a dense weight */
  int32_t layout;         /* NVFP4_LAYOUT_ROWS or NVFP4_LAYOUT_TILED32 */
} nvfp4_weight_t;

/* Version of this interface (NVFP4_ABI_VERSION). */
int nvfp4_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* nvfp4_status_string(int status);

/*
 * nvfp4_pack - load-time BF16 -> NVFP4 pack of `batch` independent tensors.
 * Passage: issue #308 "What the branch does" (at load the MTP layer's BF16
 * experts are quantized to NVFP4 with ModelOpt's recipe, one projection after
 * another).
 * Recipe, per tensor, in fp32 with correctly rounded division:
 *   scale_2 = amax / 2688  (6 * 448);
 *   per 16-block along k: byte = e4m3(block_amax / 6 / scale_2), nearest-even,
 *   saturating at 448;  s_eff = e4m3(byte) * scale_2;
 *   per element: code = e2m1(w / s_eff), nearest-even, clamped at 6, sign bit
 *   of the quotient (so -0.0 encodes as 0x8).
 *   An all-zero tensor packs to scale_2 = 0, bytes 0, codes 0; a block whose
 *   s_eff is 0 packs to codes 0. Non-finite inputs are outside the contract.
 * w       [batch, n, k] bf16 (device).
 * codes   [batch, n, k/2] out;  scales [batch, n, k/16] out;  scale_2 [batch] out.
 * ws      device workspace of at least nvfp4_pack_workspace_size(batch, n, k)
 *         bytes (per-tensor partial maxima); contents need not be initialised.
 * layout  NVFP4_LAYOUT_ROWS or NVFP4_LAYOUT_TILED32 (then n % 32 == 0 and
 *         k % 256 == 0, else NVFP4_ERR_SHAPE): where codes and scales go.
 */
size_t nvfp4_pack_workspace_size(int32_t batch, int64_t n, int64_t k);
nvfp4_status nvfp4_pack(const uint16_t* w, int32_t batch, int64_t n, int64_t k,
                        uint8_t* codes, uint8_t* scales, float* scale_2,
                        void* ws, size_t ws_bytes, int32_t layout, void* stream);

/*
 * nvfp4_relayout - copy the codes and scales of `src` into dst->codes and
 * dst->scales in dst->layout (a pure permutation of bytes; scale_2 is not
 * touched, so dst->scale_2 may point at src's). Shapes and groups must match;
 * the buffers must not overlap. For a checkpoint loaded as stored: relayout it
 * once to NVFP4_LAYOUT_TILED32 for the fast GEMM paths.
 * Passage: issue #308 "The checkpoint" (the stored format being regrouped).
 */
nvfp4_status nvfp4_relayout(const nvfp4_weight_t* src, const nvfp4_weight_t* dst, void* stream);

/*
 * nvfp4_dequant - debug export of the dequantized weights (bit-exact checks).
 * Passage: issue #308 "The checkpoint" (code, block scale and tensor scale).
 * wq_unscaled [groups, n, k] bf16 out: e2m1(code) * e4m3(scale), exact in bf16.
 * wq_scaled   [groups, n, k] fp32 out: fp32(unscaled * scale_2), one rounding.
 * Either output may be NULL (not written); not both.
 */
nvfp4_status nvfp4_dequant(const nvfp4_weight_t* w, uint16_t* wq_unscaled, float* wq_scaled,
                           void* stream);

/*
 * nvfp4_selftest_fp4_convert - debug export behind the pack's e2m1 encoding.
 * Passage: issue #308 "The checkpoint" (e2m1 codes). The pack, the activation
 * quantization of W4A4 and their exports encode e2m1 codes with the device's
 * packed fp4 convert (unit scale) instead of comparisons against the rounding
 * midpoints. This runs both on every non-NaN fp32 bit pattern and its negation
 * (2^32 inputs, one launch) and counts the ones where the convert's code differs
 * from the reading of the pages (nearest, ties to the even code, saturation at
 * 6, sign bit of the input kept).
 * mismatches: device uint64, overwritten with the count (0 expected).
 */
nvfp4_status nvfp4_selftest_fp4_convert(unsigned long long* mismatches, void* stream);

/*
 * nvfp4_linear - dense Fp4Linear: y[m, n] = bf16(scale_2 * sum_k x[m,k] * W[n,k]).
 * Passage: issue #308 "What the branch does" (the dense MLP runs on Fp4Linear).
 * x [m, k] bf16; w: groups == 1, w->k == k of x; y [m, n] bf16 out (round to
 * nearest even). m may be 0. A tiled weight needs m*k*2 and n*k/2 below 2^31
 * bytes (32-bit buffer offsets of the fast paths), else NVFP4_ERR_SHAPE.
 */
nvfp4_status nvfp4_linear(const uint16_t* x, int64_t m, const nvfp4_weight_t* w, uint16_t* y,
                          void* stream);

/*
 * nvfp4_linear_gated - the dense MLP's gate and up projections, kept apart
 * because their tensor scales differ (issue #308, "What the branch does"), and
 * combined as h[m, n] = bf16(SiLU(g) * u) with g, u the fp32 outputs of
 * nvfp4_linear on w_gate and w_up, SiLU(z) = z / (1 + exp(-z)).
 * w_gate and w_up: same n and k, groups == 1, each its own scale_2.
 * h [m, n] bf16 out.
 */
nvfp4_status nvfp4_linear_gated(const uint16_t* x, int64_t m, const nvfp4_weight_t* w_gate,
                                const nvfp4_weight_t* w_up, uint16_t* h, void* stream);

/*
 * nvfp4_moe_route - debug export of the token permutation by expert (bit-exact checks).
 * Slot s = t*k + j holds topk_ids[t, j]; it is local iff
 * expert_begin <= id < expert_begin + n_experts. Outputs:
 *   offsets [n_experts + 1] int32: exclusive prefix sums of the per-expert counts;
 *   perm    [T*k] int32: the local slots ordered by (expert, slot) - stable;
 *           entries past offsets[n_experts] are left unspecified;
 *   inv     [T*k] int32: the position of each slot in perm, -1 if skipped.
 * The counts are a histogram; the offsets come from a wavefront prefix scan.
 * ws: optional 16-byte aligned device scratch. With at least
 * nvfp4_moe_route_workspace_size(T, k, n_experts) bytes (0 for at most 4096
 * slots, else 4 bytes per expert for each of at most 64 windows of slots), a
 * larger batch is counted and scattered by one workgroup per window; with less,
 * or ws = NULL, one workgroup routes it. The result is the same either way.
 * Limits: 1 <= n_experts <= 4096, 1 <= k <= 64.
 */
size_t nvfp4_moe_route_workspace_size(int64_t T, int32_t k, int32_t n_experts);
nvfp4_status nvfp4_moe_route(const int32_t* topk_ids, int64_t T, int32_t k, int32_t n_experts,
                             int32_t expert_begin, int32_t* offsets, int32_t* perm, int32_t* inv,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * nvfp4_moe_grouped - the routed expert MLP of one MoE layer.
 * Passage: issue #308 "What the branch does" (routed experts in the grouped
 * NVFP4 kernel on bf16 activations, each expert's weight_scale_2 applied to its
 * product).
 * For every local slot (t, j) with expert e = topk_ids[t, j] - expert_begin:
 *   g = s2g[e] * x_t . Wg_e^T,  u = s2u[e] * x_t . Wu_e^T   (fp32 accumulators)
 *   h = bf16(SiLU(g) * u)                                     [I]
 *   d = s2d[e] * h . Wd_e^T                                   (fp32)
 *   y_t = bf16( sum over j = 0..k-1, in that order, of topk_w[t, j] * d )
 * Slots whose id is not local contribute 0 (the expert-parallel hook:
 * expert_begin = 0 on one GPU). Duplicate ids in a token count separately.
 * y is overwritten. The sum over j is a fixed-order gather, not atomics.
 * x        [T, H] bf16;  topk_ids [T, k] int32;  topk_w [T, k] fp32.
 * gate, up: groups = E, n = I, k = H.   down: groups = E, n = H, k = I.
 * ws       at least nvfp4_moe_workspace_size(T, k, E, H, I) bytes.
 * y        [T, H] bf16 out.
 * Limits: 1 <= E <= 4096, 1 <= k <= 64, H and I multiples of 32. gate and up
 * share one layout; tiled weights need T*H*2, T*k*I*2, I*H/2 below 2^31 bytes.
 */
size_t nvfp4_moe_workspace_size(int64_t T, int32_t k, int32_t n_experts, int64_t H, int64_t I);
nvfp4_status nvfp4_moe_grouped(const uint16_t* x, int64_t T, int64_t H, const int32_t* topk_ids,
                               const float* topk_w, int32_t k, int32_t expert_begin,
                               const nvfp4_weight_t* gate, const nvfp4_weight_t* up,
                               const nvfp4_weight_t* down, void* ws, size_t ws_bytes,
                               uint16_t* y, void* stream);

/*
 * Kernel classes of the routed GEMMs. A class fixes the tile shape of both
 * projections and with it the summation order of every output element, which
 * then depends on the shapes alone (never on the batch size, the routing, the
 * other rows or the tile a row lands in):
 *   NVFP4_CLASS_DECODE  - tiles of at most 16 rows, weights streamed through
 *                         registers (decode-shaped calls);
 *   NVFP4_CLASS_PREFILL - tiles of at most 128 rows on the 32x32 matrix-core
 *                         kernel (prompt-shaped calls);
 *   NVFP4_CLASS_AUTO    - what nvfp4_moe_grouped runs: at most 32 slots take
 *                         4-row tiles whose gate/up splits K over four waves
 *                         (partials added in wave order); with at most 4 tokens
 *                         and 24 slots (W4A16, H and I multiples of 512,
 *                         H <= 4096, I <= 2048) these run as two launches with no route
 *                         kernel, the combine inside the down launch (same
 *                         sums: each slot's products in k order, the slots of a
 *                         token in j order); otherwise DECODE when
 *                         the average local expert gets at most 16 rows
 *                         (T*k <= 16 * min(T*k, n_experts)), else PREFILL. The
 *                         class, and so the bits, can change with the batch size.
 * Shapes that a class's kernel does not cover fall back the same way for every
 * batch (tiled weights to the prefill kernel, row-major ones to the tiled
 * fallback GEMM), so a pinned class stays bitwise chunk-invariant.
 */
#define NVFP4_CLASS_AUTO 0
#define NVFP4_CLASS_DECODE 1
#define NVFP4_CLASS_PREFILL 2

/*
 * nvfp4_moe_grouped_class - nvfp4_moe_grouped with the kernel class pinned.
 * Passage: TensorFold issue #308, "Questions", item 4 (a prompt-shaped expert
 * kernel whose sums do not change with the chunking). A prompt processed in
 * chunks with NVFP4_CLASS_PREFILL (or any pinned class) gives every token the
 * bits it gets when the whole prompt goes in one call. Same arguments, workspace
 * (nvfp4_moe_workspace_size covers every class), ownership and errors as
 * nvfp4_moe_grouped; an unknown class is NVFP4_ERR_UNSUPPORTED.
 */
nvfp4_status nvfp4_moe_grouped_class(const uint16_t* x, int64_t T, int64_t H, const int32_t* topk_ids,
                                     const float* topk_w, int32_t k, int32_t expert_begin,
                                     const nvfp4_weight_t* gate, const nvfp4_weight_t* up,
                                     const nvfp4_weight_t* down, int32_t kernel_class, void* ws, size_t ws_bytes,
                                     uint16_t* y, void* stream);

/* Kernels named by nvfp4_moe_plan. */
#define NVFP4_KERNEL_NONE 0
#define NVFP4_KERNEL_DECODE_KSPLIT 1   /* gate/up on 4-row tiles, K split over 4 waves */
#define NVFP4_KERNEL_DECODE 2          /* decode tiles, weights streamed, activations staged per stage */
#define NVFP4_KERNEL_DECODE_RESIDENT 3 /* down on decode tiles: whole H tile in LDS, 1/2/4 weight blocks per wave */
#define NVFP4_KERNEL_PREFILL 4         /* prefill tiles, 32x32 matrix-core kernel */
#define NVFP4_KERNEL_FALLBACK 5        /* tiled fallback GEMM (row-major weights of other shapes) */
#define NVFP4_KERNEL_TINY 6            /* at most 4 tokens, 24 slots: gate/up routing itself, down with the combine */

/*
 * nvfp4_moe_plan - which kernels a routed call of these shapes runs (host only:
 * nothing is enqueued; it reads the device's compute-unit count). Passage: as
 * nvfp4_moe_grouped_class. For T tokens (T = 0 is planned as one token), top-k,
 * n_experts local experts, hidden H, intermediate I, the gate/up and down
 * layouts and a kernel class, plan[5] receives:
 *   plan[0] rows per tile (4, 16 or 128);
 *   plan[1] the gate/up kernel (NVFP4_KERNEL_*);
 *   plan[2] the down kernel;
 *   plan[3] the down kernel's width: 64-row weight blocks per wave stream for
 *           NVFP4_KERNEL_DECODE_RESIDENT, 32-row weight blocks per wave for
 *           NVFP4_KERNEL_PREFILL, else 0;
 *   plan[4] 1 if the routed GEMMs run on fp16 operands (see Numerics), else 0.
 * The W4A16 and W4A4 entry points run the same kernels (W4A4 refuses plans
 * with the fallback GEMM), except that W4A4 runs NVFP4_KERNEL_DECODE_KSPLIT
 * gate/up and its decode down kernel where the plan names NVFP4_KERNEL_TINY. Errors: NVFP4_ERR_NULL, NVFP4_ERR_SHAPE, and those
 * of nvfp4_moe_grouped_class for the shapes and class.
 */
nvfp4_status nvfp4_moe_plan(int64_t T, int32_t k, int32_t n_experts, int64_t H, int64_t I, int32_t gate_layout,
                            int32_t down_layout, int32_t kernel_class, int32_t* plan);

/*
 * nvfp4_moe_grouped_timed - nvfp4_moe_grouped with a hipEvent_t recorded on
 * `stream` before the first kernel and after each of its stages (route,
 * gate/up, down, combine): events[0..4]. Same results; for per-stage timing.
 */
nvfp4_status nvfp4_moe_grouped_timed(const uint16_t* x, int64_t T, int64_t H,
                                     const int32_t* topk_ids, const float* topk_w, int32_t k,
                                     int32_t expert_begin, const nvfp4_weight_t* gate,
                                     const nvfp4_weight_t* up, const nvfp4_weight_t* down,
                                     void* ws, size_t ws_bytes, uint16_t* y, void* stream,
                                     void* const* events);

/*
 * nvfp4_moe_grouped_noalloc - nvfp4_moe_grouped for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. It takes no workspace: the call's scratch
 * (the permutation, tile list, H, the fp32 partials and the scaled activations)
 * lives in a fixed device array of NVFP4_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends. The first call on a
 * device looks up that device's copy (with the device current); no call
 * allocates or frees anything.
 * Same arguments (minus the workspace), results (bit for bit: the same
 * kernels), ownership and errors as nvfp4_moe_grouped, plus NVFP4_ERR_SCRATCH
 * when nvfp4_moe_workspace_size(T, k, E, H, I) exceeds the fixed size (about
 * 19.5 KB per routed slot at H = 4096, I = 1536: up to about 390 tokens of a
 * top-8 layer). NVFP4_ERR_HIP if the array's address cannot be looked up.
 * Every call on one GPU uses the same array: calls that can overlap on one GPU
 * (other streams, other host threads) race and must be serialized by the
 * caller; calls on one stream are ordered and safe. The array keeps the last
 * call's contents; nothing in it needs clearing between calls.
 */
#define NVFP4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
nvfp4_status nvfp4_moe_grouped_noalloc(const uint16_t* x, int64_t T, int64_t H, const int32_t* topk_ids,
                                       const float* topk_w, int32_t k, int32_t expert_begin,
                                       const nvfp4_weight_t* gate, const nvfp4_weight_t* up,
                                       const nvfp4_weight_t* down, uint16_t* y, void* stream);

/*
 * nvfp4_quantize_act - static NVFP4 quantization of bf16 activations, the W4A4
 * form (model card "GLM-5.3-Flash-NVFP4-W4A4-Experts", section "Quantization
 * boundary": NVFP4 weights with calibrated activations; TensorFold issue #308,
 * section "The checkpoint": an input_scale is stored beside each weight).
 *
 * Each 16-block of a row is quantized by the pack's block steps with the
 * calibrated input_scale in place of scale_2: byte = e4m3_rne(block_amax / 6 /
 * input_scale) (saturating at 448: larger activations clamp), code =
 * e2m1_rne(x / (e4m3(byte) * input_scale)). Nothing depends on the row's own amax.
 *
 *   x            [rows, k] bf16, device, 16-byte aligned.
 *   input_scale  one fp32 in device memory (4-byte aligned); 0 gives all-zero output.
 *   codes        [rows, k/2] out, device, 16-byte aligned (even k in the low nibble).
 *   scales       [rows, k/16] out (e4m3 bytes), device, 16-byte aligned.
 * Errors: ERR_SHAPE unless k % 32 == 0, k >= 32 and 0 <= rows <= 2^30; ERR_NULL,
 * ERR_ALIGN as stated; rows == 0 is a no-op.
 */
nvfp4_status nvfp4_quantize_act(const uint16_t* x, int64_t rows, int64_t k, const float* input_scale,
                                uint8_t* codes, uint8_t* scales, void* stream);

/*
 * nvfp4_moe_grouped_w4a4 - the routed expert MLP with W4A4 activations (the
 * checkpoint's own FP4 x FP4 math that TensorFold issue #308 defers, "What the
 * branch does" and "Questions", item 1).
 *
 * As nvfp4_moe_grouped (same arguments, workspace size, ownership and errors),
 * plus two calibrated activation scales, each one fp32 in device memory, shared
 * by all experts of the layer (the model card's activation-scale policy takes a
 * percentile across experts per projection):
 *   input_scale_gate_up - x is quantized (nvfp4_quantize_act) before gate/up;
 *   input_scale_down    - H, rounded to bf16 as stored, is quantized before down.
 * The quantized values e2m1 * e4m3 are exact in fp16, so the GEMMs run on them
 * exactly and the input scales multiply the fp32 results. ERR_NULL if either
 * scale pointer is null; ERR_UNSUPPORTED for shapes that only the fallback GEMM
 * covers (H and I multiples of 256 with N multiples of 32/64 are covered).
 */
nvfp4_status nvfp4_moe_grouped_w4a4(const uint16_t* x, int64_t T, int64_t H, const int32_t* topk_ids,
                                    const float* topk_w, int32_t k, int32_t expert_begin,
                                    const nvfp4_weight_t* gate, const nvfp4_weight_t* up,
                                    const nvfp4_weight_t* down, const float* input_scale_gate_up,
                                    const float* input_scale_down, void* ws, size_t ws_bytes, uint16_t* y,
                                    void* stream);

/* ------------------------------------------------------------------------
 * The BF16 steps either side of the routed experts (TensorFold issue #308,
 * "What the branch does": the shared expert runs as a BF16 MLP; model card
 * "GLM-5.3-Flash-NVFP4-W4A4-Experts", "Quantization boundary": routers and
 * shared experts stay BF16). bf16 weights are plain row-major [out, in] device
 * arrays, 16-byte aligned; products accumulate in fp32 (MFMA); small batches
 * split the inputs over workgroups and sum the splits in a fixed order, so
 * results are reproducible.
 * ------------------------------------------------------------------------ */

/*
 * nvfp4_router_topk - router logits and top-k selection.
 *   logits[t, e] = sum_h x[t, h] * w_router[e, h] (fp32); the k largest (ties to
 *   the lower expert index) go to topk_ids[t, 0..k) in decreasing order, and
 *   topk_w[t, j] is the softmax over the k selected logits.
 *   x [T, H] bf16; w_router [n_experts, H] bf16; ws of
 *   nvfp4_router_workspace_size(T, H, n_experts) bytes (16-byte aligned);
 *   topk_ids [T, k] int32 and topk_w [T, k] fp32 out (4-byte aligned).
 * Errors: ERR_SHAPE unless H % 64 == 0, n_experts % 4 == 0, 1 <= k <=
 * min(64, n_experts), n_experts <= 4096; ERR_NULL, ERR_ALIGN, ERR_WORKSPACE.
 */
size_t nvfp4_router_workspace_size(int64_t T, int64_t H, int32_t n_experts);
nvfp4_status nvfp4_router_topk(const uint16_t* x, int64_t T, int64_t H, const uint16_t* w_router,
                               int32_t n_experts, int32_t k, void* ws, size_t ws_bytes, int32_t* topk_ids,
                               float* topk_w, void* stream);

/*
 * nvfp4_bf16_mlp - the shared-expert BF16 MLP:
 *   y[m, :] = (SiLU(x . w_gate^T) * (x . w_up^T)) . w_down^T, fp32 out [M, H];
 *   the intermediate [M, Is] is rounded to bf16 (the down product's operand).
 *   x [M, H] bf16; w_gate, w_up [Is, H] bf16; w_down [H, Is] bf16; ws of
 *   nvfp4_bf16_mlp_workspace_size(M, H, Is) bytes.
 * Errors: ERR_SHAPE unless H and Is are multiples of 64; ERR_NULL, ERR_ALIGN,
 * ERR_WORKSPACE.
 */
size_t nvfp4_bf16_mlp_workspace_size(int64_t M, int64_t H, int64_t Is);
nvfp4_status nvfp4_bf16_mlp(const uint16_t* x, int64_t M, int64_t H, const uint16_t* w_gate, const uint16_t* w_up,
                            const uint16_t* w_down, int64_t Is, void* ws, size_t ws_bytes, float* y, void* stream);

/*
 * nvfp4_moe_block - one MoE block: router (nvfp4_router_topk over the
 * gate->groups experts), routed NVFP4 experts (nvfp4_moe_grouped with
 * expert_begin 0) and the shared expert (nvfp4_bf16_mlp, Is = shared
 * intermediate size), summed: y[t] = bf16(sum_j w[t,j] * expert_j(x_t) +
 * shared(x_t)), the shared term added after the k routed slots.
 *   ws of nvfp4_moe_block_workspace_size(T, k, E, H, I, Is) bytes.
 * Errors: those of the three parts.
 */
size_t nvfp4_moe_block_workspace_size(int64_t T, int32_t k, int32_t n_experts, int64_t H, int64_t I, int64_t Is);
nvfp4_status nvfp4_moe_block(const uint16_t* x, int64_t T, int64_t H, const uint16_t* w_router, int32_t k,
                             const nvfp4_weight_t* gate, const nvfp4_weight_t* up, const nvfp4_weight_t* down,
                             const uint16_t* shared_gate, const uint16_t* shared_up, const uint16_t* shared_down,
                             int64_t Is, void* ws, size_t ws_bytes, uint16_t* y, void* stream);

/*
 * nvfp4_moe_grouped_bf16 - the routed expert MLP on BF16 expert weights: the MTP
 * layer's draft experts kept in BF16, the alternative to packing them to NVFP4
 * at load that TensorFold issue #308 asks about ("What the branch does").
 *
 * Same routing, arguments and ownership as nvfp4_moe_grouped, with plain bf16
 * weights w_gate, w_up [n_experts, I, H] and w_down [n_experts, H, I] (device,
 * row-major, 16-byte aligned; no tensor scale) and a workspace of
 * nvfp4_moe_grouped_bf16_workspace_size(T, k, n_experts, H, I) bytes. fp32
 * accumulation (MFMA), H rounded to bf16 as the down product's operand, the
 * weighted sum over j in order. Errors: ERR_SHAPE unless H and I are multiples
 * of 64; ERR_NULL, ERR_ALIGN, ERR_WORKSPACE.
 */
size_t nvfp4_moe_grouped_bf16_workspace_size(int64_t T, int32_t k, int32_t n_experts, int64_t H, int64_t I);
nvfp4_status nvfp4_moe_grouped_bf16(const uint16_t* x, int64_t T, int64_t H, const int32_t* topk_ids,
                                    const float* topk_w, int32_t k, int32_t expert_begin, const uint16_t* w_gate,
                                    const uint16_t* w_up, const uint16_t* w_down, int32_t n_experts, int64_t I,
                                    void* ws, size_t ws_bytes, uint16_t* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_MOE_EXPERT_AMD_NVFP4_H */
