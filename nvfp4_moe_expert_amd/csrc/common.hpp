// Device-side helpers shared by the gfx950 kernels of the NVFP4 expert library.
//
// Formats (TensorFold issue #308, section "The checkpoint"): e2m1 codes, two
// per byte with the even element in the low nibble; one e4m3fn scale byte per
// 16 consecutive inputs; one fp32 scale_2 per tensor.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- conversions
// e4m3fn byte (in the low 8 bits) -> fp32. gfx950's fp8 convert uses the OCP
// E4M3 encoding; it is exact for all 254 finite bytes (checked exhaustively on
// the device against the closed form).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8(byte, 0);
}

// Two e2m1 codes of byte `sel` of `w` -> two fp32 values (low nibble first).
// The scale operand of the gfx950 scaled convert contributes only its exponent,
// so 1.0f gives the plain e2m1 values.
template <int SEL>
__device__ __forceinline__ f32x2 e2m1x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Round two fp32 to bf16 (nearest even) and pack: lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Eight e2m1 codes (one dword, k..k+7, even k in the low nibble of each byte)
// times one block scale -> eight bf16 values in k order. Each product is exact
// in bf16 (<= 6 significant bits, magnitude 2^-10 .. 2688), so the fp32
// multiply and the bf16 packing introduce no rounding.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float scale) {
  f32x2 p0 = e2m1x2_to_f32<0>(w);
  f32x2 p1 = e2m1x2_to_f32<1>(w);
  f32x2 p2 = e2m1x2_to_f32<2>(w);
  f32x2 p3 = e2m1x2_to_f32<3>(w);
  u32x4 r;
  r[0] = pack_bf16x2(p0[0] * scale, p0[1] * scale);
  r[1] = pack_bf16x2(p1[0] * scale, p1[1] * scale);
  r[2] = pack_bf16x2(p2[0] * scale, p2[1] * scale);
  r[3] = pack_bf16x2(p3[0] * scale, p3[1] * scale);
  return __builtin_bit_cast(bf16x8, r);
}

// fp16 form of the same products: the e2m1 value (<= 6, one significant bit past
// the leading one) times the e4m3 scale (<= 448, three) has at most six
// significant bits and lies in [2^-10, 2688], so it is exact in fp16 too.
template <int SEL>
__device__ __forceinline__ f16x2 e2m1x2_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// 8 codes (one dword) times a block scale held in both halves of s -> 8 fp16.
__device__ __forceinline__ f16x8 dequant8_f16(uint32_t w, f16x2 s) {
  const f16x2 p0 = e2m1x2_f16<0>(w) * s, p1 = e2m1x2_f16<1>(w) * s;
  const f16x2 p2 = e2m1x2_f16<2>(w) * s, p3 = e2m1x2_f16<3>(w) * s;
  return __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                 __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}

// ------------------------------------------------------------------ encoders
// NVFP4 quantization of a 16-block (the pack recipe's steps per block, every
// step in fp32, correctly rounded division, no contraction): against a global
// scale gs (a weight's scale_2, or an activation's calibrated input_scale),
// byte = e4m3_rne(block_amax / 6 / gs), s_eff = e4m3(byte) * gs, and each code =
// e2m1_rne(value / s_eff) with the sign bit of the quotient.

// |bf16| ordered as an unsigned integer: for non-NaN values the magnitude bits
// (sign cleared) compare exactly like the magnitudes.
__device__ __forceinline__ uint32_t absmax8(u32x4 v) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t a = v[i] & 0x7FFFu, b = (v[i] >> 16) & 0x7FFFu;
    m = max(m, max(a, b));
  }
  return m;
}

// e4m3fn byte of a v >= 0 (not NaN), round to nearest even, saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  if (v >= 448.0f) return 0x7Eu;
  if (v < 0.015625f) {                       // below 2^-6: subnormal grid of 2^-9
    float m = __builtin_rintf(v * 512.0f);  // exact scaling, ties to even; 8 -> 0x08 (min normal)
    return (uint32_t)m;
  }
  uint32_t b = __builtin_bit_cast(uint32_t, v);
  int e = (int)(b >> 23) - 127;              // v = 2^e * 1.f, -6 <= e <= 8
  uint32_t m3 = (b >> 20) & 7u, rem = b & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
  if (m3 == 8u) { m3 = 0; ++e; }
  uint32_t code = ((uint32_t)(e + 7) << 3) | m3;
  return code > 0x7Eu ? 0x7Eu : code;
}

// e2m1 code of q: nearest even, clamped at 6, sign bit of q. Midpoints
// 0.25 .. 5.0 are passed when above them, or when on them and the upper code is even.
__device__ __forceinline__ uint32_t e2m1_rne(float q) {
  float a = fabsf(q);
  uint32_t idx = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                 (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                 (uint32_t)(a > 5.0f);
  return idx | ((__builtin_bit_cast(uint32_t, q) >> 31) << 3);
}

// Scale byte of a block whose amax has the bf16 magnitude bits `amax16`; s_eff
// receives e4m3(byte) * gs (0 when gs is 0, whose blocks get byte 0 and codes 0).
__device__ __forceinline__ uint32_t block_byte(uint32_t amax16, float gs, float& s_eff) {
  s_eff = 0.0f;
  if (gs == 0.0f) return 0u;
  const float bamax = __builtin_bit_cast(float, amax16 << 16);
  const uint32_t byte = e4m3_rne((bamax / 6.0f) / gs);
  s_eff = e4m3_to_f32(byte) * gs;
  return byte;
}

// Codes of 8 bf16 values (one u32x4) -> one dword, element 2j in the low nibble of byte j.
// code = e2m1_rne(q) with q the correctly rounded w / s_eff. The e2m1 code comes
// from the packed fp4 convert with a unit scale, which equals e2m1_rne bit for bit
// on every non-NaN fp32 input (checked exhaustively on the device, both signs:
// nearest even, saturation at 6, sign bit kept).
// Fast path without a division per element: with r = 1/s_eff rounded, and
// r_lo = r(1 - 2^-20), r_hi = r(1 + 2^-20) rounded, every |w * r_lo| <= |q| <=
// |w * r_hi| (the roundings move each product by at most 3 * 2^-24 relative, q by
// 2^-24), all with the sign of w. The convert is monotone in |q|, so where the
// codes of w * r_lo and w * r_hi agree they are the code of q; only a word with
// a value that close to a rounding boundary (a tie, for instance) takes the
// exact division.
__device__ __forceinline__ uint32_t quant8_exact(u32x4 v, float s_eff) {
  uint32_t word = 0;
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, bf16_lo(v[0]) / s_eff, bf16_hi(v[0]) / s_eff, 1.0f, 0);
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, bf16_lo(v[1]) / s_eff, bf16_hi(v[1]) / s_eff, 1.0f, 1);
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, bf16_lo(v[2]) / s_eff, bf16_hi(v[2]) / s_eff, 1.0f, 2);
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, bf16_lo(v[3]) / s_eff, bf16_hi(v[3]) / s_eff, 1.0f, 3);
  return word;
}

__device__ __forceinline__ uint32_t quant8_scaled(u32x4 v, float r) {
  uint32_t word = 0;
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, bf16_lo(v[0]) * r, bf16_hi(v[0]) * r, 1.0f, 0);
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, bf16_lo(v[1]) * r, bf16_hi(v[1]) * r, 1.0f, 1);
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, bf16_lo(v[2]) * r, bf16_hi(v[2]) * r, 1.0f, 2);
  word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, bf16_lo(v[3]) * r, bf16_hi(v[3]) * r, 1.0f, 3);
  return word;
}

__device__ __forceinline__ uint32_t quant8(u32x4 v, float s_eff) {
  if (s_eff == 0.0f) return 0u;
  const float r = 1.0f / s_eff;
  const float r_lo = r * (1.0f - 0x1p-20f), r_hi = r * (1.0f + 0x1p-20f);
  if (r_hi <= 3.0e38f) {   // finite (an s_eff near the bottom of the fp32 range takes the exact path)
    const uint32_t lo = quant8_scaled(v, r_lo), hi = quant8_scaled(v, r_hi);
    if (lo == hi) return lo;
  }
  return quant8_exact(v, s_eff);
}

// Power-of-two exponent p that puts a row maximum m (> 0, given by its fp32 bits)
// in [2^14, 2^15): the row times 2^p then fits fp16 with bf16 values down to
// 2^-28 of m converting exactly. 0 for an all-zero row.
__device__ __forceinline__ int row_exponent(uint32_t max_bits) {
  if (max_bits == 0) return 0;
  const int e = (int)((max_bits >> 23) & 0xFF) - 127;
  const int p = 14 - e;
  return p > 126 ? 126 : (p < -126 ? -126 : p);
}

// ------------------------------------------------------------ weight layouts
// Byte offsets inside one [N, K] tensor. Row-major: the checkpoint's order.
// Tiled (blocks of 32 rows; N % 32 == 0, K % 256 == 0): the 16-byte code piece
// (row n, inputs 32j .. 32j+31) sits at ((n/32)*(K/32) + j)*512 + (n%32)*16, and
// the 16 scale bytes (row n, inputs 256c .. 256c+255) at ((n/32)*(K/256) + c)*512
// + (n%32)*16, so 32 rows of a block read 512 contiguous bytes.
__device__ __forceinline__ int64_t code_piece_off(bool tiled, int64_t n, int64_t j, int64_t K) {
  return tiled ? ((n / 32) * (K / 32) + j) * 512 + (n % 32) * 16 : n * (K / 2) + j * 16;
}
__device__ __forceinline__ int64_t scale_off(bool tiled, int64_t n, int64_t b, int64_t K) {
  return tiled ? ((n / 32) * (K / 256) + b / 16) * 512 + (n % 32) * 16 + (b % 16) : n * (K / 16) + b;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ------------------------------------------------------------------- loads
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// Non-temporal 16-byte load, for bytes that one call reads exactly once (a weight
// stream): measured on MI355X, a plain read stream of a 4 GiB buffer reaches
// 6.2-6.4 TB/s with ordinary loads and 7.0-7.1 TB/s with these.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Buffer descriptor over `bytes` bytes from `base` for raw (untyped) buffer
// access on gfx9-family parts (word 3 below); loads at offsets past the end
// return zeros without touching memory.
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

}  // namespace nvfp4
