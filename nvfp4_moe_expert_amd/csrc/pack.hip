// Load-time BF16 -> NVFP4 pack, and the dequant debug export.
//
// Pack recipe (ModelOpt's, which TensorFold issue #308 applies at load to the
// MTP layer's BF16 experts, "What the branch does"): per tensor
//   scale_2 = amax / 2688;  per 16-block: byte = e4m3_rne(block_amax / 6 / scale_2);
//   s_eff = e4m3(byte) * scale_2;  code = e2m1_rne(w / s_eff), sign of the quotient.
// Every step is fp32 with correctly rounded division and no contraction (the
// library is compiled with -ffp-contract=off), so the bytes are reproducible.
//
// Two kernels per call: (1) per-tensor partial maxima of |w| (no atomics, so no
// workspace clearing is needed), (2) the quantization, whose workgroups each
// finish the max reduction of their tensor from the partials.
#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int kPackThreads = 256;

__global__ __launch_bounds__(kPackThreads) void pack_amax_kernel(const uint16_t* __restrict__ w,
                                                                 int64_t per_tensor, int nblk,
                                                                 uint32_t* __restrict__ partial) {
  const int g = blockIdx.y;
  const uint16_t* base = w + (int64_t)g * per_tensor;
  uint32_t m = 0;
  const int64_t stride = (int64_t)nblk * kPackThreads * 8;
  for (int64_t i = ((int64_t)blockIdx.x * kPackThreads + threadIdx.x) * 8; i < per_tensor; i += stride)
    m = max(m, absmax8(ld16_nt(base + i)));   // streamed once (non-temporal loads read faster)
  // wave reduction then across the 4 waves
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t red[kPackThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
    for (int i = 1; i < kPackThreads / 64; ++i) r = max(r, red[i]);
    partial[(int64_t)g * nblk + blockIdx.x] = r;
  }
}

// One thread packs 32 consecutive elements of a row (two 16-blocks).
__global__ __launch_bounds__(kPackThreads) void pack_quant_kernel(
    const uint16_t* __restrict__ w, int64_t n, int64_t k, int nblk, const uint32_t* __restrict__ partial,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ scale_2, int tiled) {
  const int g = blockIdx.y;
  __shared__ float s_scale2;
  if (threadIdx.x < 64) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nblk; i += 64) m = max(m, partial[(int64_t)g * nblk + i]);
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if (threadIdx.x == 0) {
      float amax = __builtin_bit_cast(float, m << 16);
      float s2 = amax / 2688.0f;
      s_scale2 = s2;
      if (blockIdx.x == 0) scale_2[g] = s2;
    }
  }
  __syncthreads();
  const float s2 = s_scale2;
  const int64_t units_per_row = k / 32;
  const int64_t u = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
  if (u >= n * units_per_row) return;
  const int64_t row = u / units_per_row, c32 = u % units_per_row;
  const uint16_t* src = w + (int64_t)g * n * k + row * k + c32 * 32;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = ld16(src + 8 * i);
  uint32_t sbytes = 0;
  u32x4 out = {0, 0, 0, 0};
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const u32x4 a = v[2 * blk], b = v[2 * blk + 1];
    float s_eff;
    const uint32_t byte = block_byte(max(absmax8(a), absmax8(b)), s2, s_eff);
    out[2 * blk] = quant8(a, s_eff);
    out[2 * blk + 1] = quant8(b, s_eff);
    sbytes |= byte << (8 * blk);
  }
  st16(codes + (int64_t)g * n * (k / 2) + code_piece_off(tiled, row, c32, k), out);
  *reinterpret_cast<uint16_t*>(scales + (int64_t)g * n * (k / 16) + scale_off(tiled, row, 2 * c32, k)) =
      (uint16_t)sbytes;
}

// Tiled output layout: one wave per 32 rows x 256 inputs, lane (r, h) = row r of
// the block, inputs 128h .. 128h + 127 of the chunk (8 16-blocks). Each store
// instruction then writes whole 512-byte runs: code piece j of the 64 lanes is
// the 16-byte piece (row r, inputs 128h + 32j ..) of two runs, and the 8 scale
// bytes of the lanes fill the chunk's 512-byte scale run. (With one thread per
// 32 inputs of a row in row order, every 16-byte code store and 2-byte scale
// store landed in a different run: 1.28 ms per 288-tensor batch against 0.88 for
// the row-major layout.) Same arithmetic per block as pack_quant_kernel.
__global__ __launch_bounds__(kPackThreads) void pack_quant_tiled_kernel(
    const uint16_t* __restrict__ w, int64_t n, int64_t k, int nblk, const uint32_t* __restrict__ partial,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ scale_2) {
  const int g = blockIdx.y;
  __shared__ float s_scale2;
  if (threadIdx.x < 64) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nblk; i += 64) m = max(m, partial[(int64_t)g * nblk + i]);
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if (threadIdx.x == 0) {
      float amax = __builtin_bit_cast(float, m << 16);
      float s2 = amax / 2688.0f;
      s_scale2 = s2;
      if (blockIdx.x == 0) scale_2[g] = s2;
    }
  }
  __syncthreads();
  const float s2 = s_scale2;
  const int64_t chunks = k / 256;
  const int64_t item = (int64_t)blockIdx.x * (kPackThreads / 64) + (threadIdx.x >> 6);
  if (item >= (n / 32) * chunks) return;
  const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
  const int64_t R = item / chunks, c = item % chunks;
  const int64_t row = 32 * R + r;
  const uint16_t* src = w + (int64_t)g * n * k + row * k + 256 * c + 128 * h;
  u32x4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = ld16(src + 8 * i);
  uint8_t* cg = codes + (int64_t)g * n * (k / 2);
  uint32_t sb[2] = {0, 0};
#pragma unroll
  for (int j = 0; j < 4; ++j) {   // code piece j: 16-blocks 2j, 2j + 1 of the lane's 8
    u32x4 out;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const u32x4 a = v[4 * j + 2 * b], bb = v[4 * j + 2 * b + 1];
      float s_eff;
      const uint32_t byte = block_byte(max(absmax8(a), absmax8(bb)), s2, s_eff);
      out[2 * b] = quant8(a, s_eff);
      out[2 * b + 1] = quant8(bb, s_eff);
      const int blk = 2 * j + b;
      sb[blk / 4] |= byte << (8 * (blk % 4));
    }
    st16(cg + code_piece_off(true, row, 8 * c + 4 * h + j, k), out);
  }
  *reinterpret_cast<u32x2*>(scales + (int64_t)g * n * (k / 16) + scale_off(true, row, 16 * c + 8 * h, k)) =
      u32x2{sb[0], sb[1]};
}

// Static activation quantization (the W4A4 form): the block steps of the pack
// with a calibrated input_scale (one fp32 in device memory) in place of scale_2.
// One thread: 32 consecutive elements of a row -> 16 code bytes, 2 scale bytes
// (row-major, the layout of a stored weight).
__global__ __launch_bounds__(kPackThreads) void act_quant_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                 int64_t k, const float* __restrict__ gs_ptr,
                                                                 uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales) {
  const int64_t per_row = k / 32;
  const int64_t u = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
  if (u >= rows * per_row) return;
  const int64_t row = u / per_row, c32 = u % per_row;
  const float gs = *gs_ptr;
  const uint16_t* src = x + row * k + c32 * 32;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = ld16(src + 8 * i);
  u32x4 out;
  uint32_t sbytes = 0;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    float s_eff;
    sbytes |= block_byte(max(absmax8(v[2 * blk]), absmax8(v[2 * blk + 1])), gs, s_eff) << (8 * blk);
    out[2 * blk] = quant8(v[2 * blk], s_eff);
    out[2 * blk + 1] = quant8(v[2 * blk + 1], s_eff);
  }
  st16(codes + row * (k / 2) + c32 * 16, out);
  *reinterpret_cast<uint16_t*>(scales + row * (k / 16) + c32 * 2) = (uint16_t)sbytes;
}

// The same quantization of the routed intermediate H, in place: each bf16 value
// becomes e2m1(code) * e4m3(byte), the quantized value without input_scale (exact
// in bf16), and hmax[row] the fp32 bits of the row's largest magnitude, which
// the fp16 form of the down projection scales the row by. One wave per row, one
// 16-block per lane.
__global__ __launch_bounds__(256) void act_fakequant_rows_kernel(uint16_t* __restrict__ h,
                                                                 uint32_t* __restrict__ hmax, int64_t rows,
                                                                 int64_t k, const float* __restrict__ gs_ptr) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float gs = *gs_ptr;
  uint16_t* r = h + row * k;
  uint32_t m = 0;
  for (int64_t c = lane; c < k / 16; c += 64) {
    const u32x4 a = ld16(r + 16 * c), b = ld16(r + 16 * c + 8);
    float s_eff;
    const uint32_t byte = block_byte(max(absmax8(a), absmax8(b)), gs, s_eff);
    const float sv = e4m3_to_f32(byte);
    const u32x4 da = __builtin_bit_cast(u32x4, dequant8(quant8(a, s_eff), sv));
    const u32x4 db = __builtin_bit_cast(u32x4, dequant8(quant8(b, s_eff), sv));
    st16(r + 16 * c, da);
    st16(r + 16 * c + 8, db);
    m = max(m, max(absmax8(da), absmax8(db)));
  }
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if (lane == 0) hmax[row] = m << 16;
}

// One thread dequantizes 8 elements (one dword of codes).
__global__ __launch_bounds__(kPackThreads) void dequant_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ scale_2, int64_t n, int64_t k, int64_t total8,
    uint16_t* __restrict__ unscaled, float* __restrict__ scaled, int tiled) {
  const int64_t u = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
  if (u >= total8) return;
  const int64_t per_group8 = n * k / 8;
  const int64_t g = u / per_group8, r = u % per_group8;
  const int64_t row = r / (k / 8), c8 = r % (k / 8);
  const uint32_t w =
      *reinterpret_cast<const uint32_t*>(codes + g * n * (k / 2) + code_piece_off(tiled, row, c8 / 4, k) + (c8 % 4) * 4);
  const float s = e4m3_to_f32(scales[g * n * (k / 16) + scale_off(tiled, row, c8 / 2, k)]);
  const bf16x8 d = dequant8(w, s);
  const int64_t o = g * n * k + row * k + c8 * 8;
  if (unscaled) st16(unscaled + o, __builtin_bit_cast(u32x4, d));
  if (scaled) {
    const float s2 = scale_2[g];
    const u32x4 dw = __builtin_bit_cast(u32x4, d);
    f32x4 lo, hi;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lo[2 * i] = bf16_lo(dw[i]) * s2;
      lo[2 * i + 1] = bf16_hi(dw[i]) * s2;
      hi[2 * i] = bf16_lo(dw[i + 2]) * s2;
      hi[2 * i + 1] = bf16_hi(dw[i + 2]) * s2;
    }
    *reinterpret_cast<f32x4*>(scaled + o) = lo;
    *reinterpret_cast<f32x4*>(scaled + o + 4) = hi;
  }
}

__global__ void fill_u64_kernel(unsigned long long* p) {
  if (threadIdx.x == 0) *p = 0ull;
}

// Every non-NaN fp32 bit pattern b (and -b): the packed fp4 convert's code
// against e2m1_rne. Thread t of the grid takes patterns t, t + stride, ... in
// 32 bits; the count is added only on a mismatch.
__global__ __launch_bounds__(kPackThreads) void fp4_convert_check_kernel(unsigned long long* __restrict__ bad) {
  const uint32_t stride = gridDim.x * kPackThreads;
  uint32_t local = 0;
  for (uint64_t b = (uint64_t)blockIdx.x * kPackThreads + threadIdx.x; b < ((uint64_t)1 << 32); b += stride) {
    const float q = __builtin_bit_cast(float, (uint32_t)b);
    if (q != q) continue;
    const uint32_t hw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q, -q, 1.0f, 0);
    local += hw != (e2m1_rne(q) | (e2m1_rne(-q) << 4));
  }
  if (local) atomicAdd(bad, (unsigned long long)local);
}

hipError_t launch_fp4_convert_check(unsigned long long* bad, hipStream_t s) {
  hipLaunchKernelGGL(fill_u64_kernel, dim3(1), dim3(64), 0, s, bad);
  hipLaunchKernelGGL(fp4_convert_check_kernel, dim3(65536), dim3(kPackThreads), 0, s, bad);
  return hipGetLastError();
}

// ------------------------------------------------------------------ launchers
int pack_nblk(int64_t per_tensor) {
  int64_t per_block = (int64_t)kPackThreads * 8 * 16;   // 16 loads per thread per block
  int64_t nb = (per_tensor + per_block - 1) / per_block;
  if (nb < 1) nb = 1;
  if (nb > 512) nb = 512;
  return (int)nb;
}

hipError_t launch_pack(const uint16_t* w, int batch, int64_t n, int64_t k, uint8_t* codes,
                       uint8_t* scales, float* scale_2, uint32_t* partial, bool tiled, hipStream_t s) {
  const int64_t per_tensor = n * k;
  const int nblk = pack_nblk(per_tensor);
  hipLaunchKernelGGL(pack_amax_kernel, dim3(nblk, batch), dim3(kPackThreads), 0, s, w, per_tensor,
                     nblk, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (tiled && n % 32 == 0 && k % 256 == 0) {
    const int64_t items = (n / 32) * (k / 256);
    const int64_t gx = (items + kPackThreads / 64 - 1) / (kPackThreads / 64);
    hipLaunchKernelGGL(pack_quant_tiled_kernel, dim3((unsigned)gx, batch), dim3(kPackThreads), 0, s, w, n, k,
                       nblk, partial, codes, scales, scale_2);
    return hipGetLastError();
  }
  const int64_t units = n * (k / 32);
  const int64_t gx = (units + kPackThreads - 1) / kPackThreads;
  hipLaunchKernelGGL(pack_quant_kernel, dim3((unsigned)gx, batch), dim3(kPackThreads), 0, s, w, n, k,
                     nblk, partial, codes, scales, scale_2, (int)tiled);
  return hipGetLastError();
}

// One thread moves one 16-byte code piece (row n, inputs 32j ..) and, for the
// first K/256 pieces of a row, one 16-byte scale piece (row n, inputs 256c ..).
__global__ __launch_bounds__(kPackThreads) void relayout_kernel(const uint8_t* __restrict__ codes,
                                                                const uint8_t* __restrict__ scales,
                                                                int from_tiled, int64_t total, int64_t n,
                                                                int64_t k, uint8_t* __restrict__ codes_out,
                                                                uint8_t* __restrict__ scales_out) {
  const int64_t u = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
  if (u >= total) return;
  const int64_t per_group = n * (k / 32);
  const int64_t g = u / per_group, r = u % per_group;
  const int64_t row = r / (k / 32), j = r % (k / 32);
  const bool ft = from_tiled != 0;
  const int64_t cbase = g * n * (k / 2);
  st16(codes_out + cbase + code_piece_off(!ft, row, j, k), ld16(codes + cbase + code_piece_off(ft, row, j, k)));
  if (j < k / 256) {
    const int64_t sbase = g * n * (k / 16);
    st16(scales_out + sbase + scale_off(!ft, row, 16 * j, k), ld16(scales + sbase + scale_off(ft, row, 16 * j, k)));
  }
}

hipError_t launch_relayout(const uint8_t* codes, const uint8_t* scales, bool from_tiled, int64_t groups,
                           int64_t n, int64_t k, uint8_t* codes_out, uint8_t* scales_out, hipStream_t s) {
  const int64_t total = groups * n * (k / 32);
  if (total == 0) return hipSuccess;
  const int64_t gx = (total + kPackThreads - 1) / kPackThreads;
  hipLaunchKernelGGL(relayout_kernel, dim3((unsigned)gx), dim3(kPackThreads), 0, s, codes, scales,
                     (int)from_tiled, total, n, k, codes_out, scales_out);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* scale_2,
                          int groups, int64_t n, int64_t k, bool tiled, uint16_t* unscaled, float* scaled,
                          hipStream_t s) {
  const int64_t total8 = (int64_t)groups * n * k / 8;
  const int64_t gx = (total8 + kPackThreads - 1) / kPackThreads;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)gx), dim3(kPackThreads), 0, s, codes, scales,
                     scale_2, n, k, total8, unscaled, scaled, (int)tiled);
  return hipGetLastError();
}

}  // namespace nvfp4

namespace nvfp4 {

hipError_t launch_act_quant(const uint16_t* x, int64_t rows, int64_t k, const float* input_scale, uint8_t* codes,
                            uint8_t* scales, hipStream_t s) {
  const int64_t units = rows * (k / 32);
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL(act_quant_kernel, dim3((unsigned)((units + kPackThreads - 1) / kPackThreads)),
                     dim3(kPackThreads), 0, s, x, rows, k, input_scale, codes, scales);
  return hipGetLastError();
}

hipError_t launch_act_fakequant_rows(uint16_t* h, uint32_t* hmax, int64_t rows, int64_t k, const float* input_scale,
                                     hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(act_fakequant_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, h, hmax, rows, k,
                     input_scale);
  return hipGetLastError();
}

}  // namespace nvfp4
