// Internal launcher interface between the C ABI (abi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Grouped GEMM epilogues.
enum GemmMode : int {
  kGateUp = 0,  // MoE: H[p] = bf16(SiLU(s2g*g) * s2u*u), rows gathered through perm
  kDown = 1,    // MoE: Ypart[perm[p]] = s2d * acc (fp32), scattered to slot order
  kLinear = 2,  // dense: Y[m] = bf16(s2 * acc)
  kGated = 3,   // dense: H[m] = bf16(SiLU(s2g*g) * s2u*u)
};

struct WeightDev {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* scale_2;
  int tiled;               // NVFP4_LAYOUT_TILED32 (blocks of 32 rows), else row-major
};

struct GemmArgs {
  const uint16_t* x;       // activation rows (bf16 bits), row stride K
  const int32_t* perm;     // MoE only: perm order -> slot
  int32_t topk;            // MoE gate/up: token = slot / topk
  const int32_t* tiles;    // MoE only: [max_tiles][4] = (expert, row_begin, rows, 0)
  const int32_t* n_tiles;  // MoE only: device count of valid tiles
  int64_t M;               // dense only: number of rows
  int64_t x_rows;          // rows of x (tokens for MoE gate/up, slots for down, M for dense)
  WeightDev w0, w1;        // w1 only for the two-weight modes
  int64_t N, K;            // weight rows / inputs
  void* out;               // H / Ypart / Y
  const float* act_scale;  // W4A4: the activations' input_scale (device), applied in the epilogue; else null
};

// Compute units of the current device (cached per device; 256 if the query fails).
int cu_count();

// Tile-shape variants of the grouped GEMM.
//   decode : 16-row tiles, activations staged through LDS per stage;
//   prefill: 128-row tiles, activations staged through LDS and shared by 8 waves;
//   small  : 4-row tiles of tiny batches, K split over the 4 waves of a workgroup.
enum GemmVariant : int { kDecode = 0, kPrefill = 1, kDecodeSmall = 2 };
int variant_tile_rows(GemmVariant v);

hipError_t launch_gemm(GemmMode mode, GemmVariant v, const GemmArgs& a, int64_t grid_tiles,
                       hipStream_t s);

// Inputs of the fp16 form of the routed GEMMs (decode and prefill tiles): the
// activations are fp16, each row scaled by a power of two so that its bf16
// values convert exactly.
struct F16Args {
  const uint16_t* x16;   // [T][H] fp16: x * 2^xexp[t]
  const int32_t* xexp;   // [T]
  uint32_t* hmax;        // [S] bits of max |H| per permuted row (zeroed by the prep)
};
// Decode-tile (<= 16 rows) weight-streaming GEMM. The fp16 form (routed gate/up and
// down only) reads x16 and converts H rows on the fly with hmax.
bool decode_supported(GemmMode mode, int64_t K, int64_t N);

// Tiny-batch tiles (<= 4 rows, routed modes, fp16 form): K % 512 == 0, K <= 4096, N % 16 == 0.
bool decode_small_supported(int64_t K, int64_t N);
hipError_t launch_decode_small(GemmMode mode, const GemmArgs& a, const F16Args& d, int64_t grid_tiles,
                               hipStream_t s);

// Routed experts of at most 4 tokens in two launches (gate/up; down with the
// combine), no route kernel: each gate/up workgroup derives its tile from the ids.
// H is written in slot order ([T*k][I] bf16) with the largest |H| of each block of
// 16 values in hpart ([T*k][I/16], fp32 bits). fp16 form, W4A16 only.
struct TinyArgs {
  const uint16_t* x;       // [T][H] bf16
  const int32_t* ids;      // [T][k]
  const float* tw;         // [T][k]
  int64_t T;
  int k, E, eb;            // top-k, local experts, first local expert id
  int64_t H, I;
  WeightDev gate, up, down;
  uint16_t* h;             // workspace: [T*k][I] bf16
  uint32_t* hpart;         // workspace: [T*k][I/16]
  const float* extra;      // null, or [extra_splits][T][H] fp32 added after the routed sum
  int extra_splits;
  uint16_t* y;             // [T][H] bf16
};
// T <= 4, T*k <= 32, H % 512 == 0 and H <= 4096, I % 512 == 0 and I <= 2048.
bool tiny_supported(int64_t T, int64_t k, int64_t H, int64_t I);
// down = false launches gate/up, true the down projection with the combine.
hipError_t launch_tiny(const TinyArgs& a, bool down, hipStream_t s);

// Prefill-tile (<= 128 rows) matrix-core GEMM; the tiled kernel covers other shapes.
bool prefill_supported(GemmMode mode, int64_t x_rows, int64_t K, int64_t N);
// The fp16 form (routed gate/up only; down takes bf16 H) reads the prep kernel's
// x16 (as GemmArgs::x) and xexp.
hipError_t launch_prefill(GemmMode mode, bool f16, const GemmArgs& a, const F16Args& d, int64_t grid_tiles,
                          hipStream_t s);
hipError_t launch_decode(GemmMode mode, bool f16, const GemmArgs& a, const F16Args& d, int64_t grid_tiles,
                         hipStream_t s);
// Routed down projection on decode tiles: 64-row weight blocks per wave stream of
// the resident-activation kernel (1, 2 or 4), or 0 when the streaming kernel runs.
int decode_down_streams(bool f16, int64_t x_rows, int64_t K, int64_t N, int64_t grid_tiles);
// Prefill tiles: 32-row weight blocks per wave (1: 256 weight rows per workgroup, 2: 512).
int prefill_weight_blocks(GemmMode mode, int64_t N, int64_t grid_tiles);

hipError_t launch_pack(const uint16_t* w, int batch, int64_t n, int64_t k, uint8_t* codes,
                       uint8_t* scales, float* scale_2, uint32_t* partial, bool tiled, hipStream_t s);
// codes and scales of `groups` [n, k] tensors from one layout into the other
hipError_t launch_relayout(const uint8_t* codes, const uint8_t* scales, bool from_tiled, int64_t groups,
                           int64_t n, int64_t k, uint8_t* codes_out, uint8_t* scales_out, hipStream_t s);
int pack_nblk(int64_t per_tensor);

// Static NVFP4 activation quantization (W4A4) of [rows, k] bf16 rows with the
// input_scale at `input_scale` (device): codes and scale bytes, row-major.
hipError_t launch_act_quant(const uint16_t* x, int64_t rows, int64_t k, const float* input_scale, uint8_t* codes,
                            uint8_t* scales, hipStream_t s);
// The same quantization of H rows in place (values become e2m1 * e4m3, exact in
// bf16) and hmax[row] = bits of the largest |value| of the row.
hipError_t launch_act_fakequant_rows(uint16_t* h, uint32_t* hmax, int64_t rows, int64_t k, const float* input_scale,
                                     hipStream_t s);

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* scale_2,
                          int groups, int64_t n, int64_t k, bool tiled, uint16_t* unscaled, float* scaled,
                          hipStream_t s);

// Permutation by expert; also writes the tile list (tile_rows rows per tile) when tiles != null.
// With prep.x16 != null, extra workgroups also write the pre-scaled fp16 activations
// (x16, xexp) and zero hmax[S].
struct RoutePrep {
  const uint16_t* x;     // [T][H] bf16
  int64_t T, H;
  int k;
  uint16_t* x16;
  int32_t* xexp;
  uint32_t* hmax;
  const float* act_scale;   // W4A4: x16 holds the NVFP4-quantized rows (unscaled values), xexp 0
  int rpb;                  // rows per prep workgroup (set by launch_route)
};
// Counts the fp32 inputs whose packed fp4 convert differs from e2m1_rne (into *bad).
hipError_t launch_fp4_convert_check(unsigned long long* bad, hipStream_t s);

hipError_t launch_route(const int32_t* ids, int64_t S, int E, int expert_begin, int tile_rows,
                        int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* tiles,
                        int32_t* n_tiles, const RoutePrep& prep, hipStream_t s,
                        int32_t* scratch = nullptr, size_t scratch_bytes = 0);
// Device scratch that lets launch_route spread a large batch over several
// workgroups (0 when one workgroup routes it); with less, one workgroup does.
size_t route_scratch_bytes(int64_t S, int E);

// y[t] = bf16(sum_j w[t,j] * Ypart[t*k+j] (j in order) + extra[t]); extra may be null,
// or hold `extra_splits` partials [extra_splits][T][H] summed in split order.
hipError_t launch_combine(const int32_t* ids, const float* w, const float* ypart, int64_t T, int k,
                          int64_t H, int E, int expert_begin, const float* extra, int extra_splits, uint16_t* y,
                          hipStream_t s);

// bf16 GEMM C[m, n] = sum_k x[m, k] * w[n, k] (K % 64 == 0, N % 4 == 0): fp32 C, or
// (gated) bf16 SiLU(x.w0^T) * (x.w1^T). `partial` holds bf16_gemm_partial_bytes
// of scratch for the K-split of small batches (unused when that is 0).
size_t bf16_gemm_partial_bytes(int64_t M, int64_t N, int64_t K, bool gated);
// With splits_left != null, an fp32 result split over K is left as its partials
// ([*splits_left][M][N] in `partial`, summed in split order by the consumer);
// otherwise (and when there is no split) the result is in `out`.
hipError_t launch_bf16_gemm(bool gated, const uint16_t* x, const uint16_t* w0, const uint16_t* w1, int64_t M,
                            int64_t N, int64_t K, void* out, float* partial, hipStream_t s,
                            int* splits_left = nullptr);
// Grouped bf16 GEMM over the route's tile list (tiles of <= tile_rows rows, 64 or
// 128): gated (gate/up, x rows gathered through perm / topk, H written in permuted
// order) or fp32 (down, topk 0: H rows in permuted order, written to Ypart at slot
// perm[p]). bf16_grouped_tile_rows picks the tile rows for S slots over E experts.
int bf16_grouped_tile_rows(int64_t S, int64_t E);
hipError_t launch_bf16_grouped(bool gated, const uint16_t* x, const uint16_t* w0, const uint16_t* w1,
                               const int32_t* tiles, const int32_t* n_tiles, int64_t max_tiles, const int32_t* perm,
                               int topk, int64_t N, int64_t K, void* out, hipStream_t s, int tile_rows);
// Per row of fp32 logits ([splits][T][E], summed in split order): the k largest
// (ties to the lower index) and their softmax.
hipError_t launch_topk_softmax(const float* logits, int splits, int64_t T, int E, int k, int32_t* ids, float* w,
                               hipStream_t s);

}  // namespace nvfp4
