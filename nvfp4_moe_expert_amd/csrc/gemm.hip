// Grouped NVFP4 x bf16 GEMM on gfx950 matrix cores, with the expert-MLP epilogues.
//
// Passage: TensorFold issue #308, "What the branch does" - routed experts run in
// a grouped NVFP4 kernel on bf16 activations, each expert's weight_scale_2
// applied to its product; the dense MLP runs on Fp4Linear with separate gate
// and up projections (each keeps its own tensor scale).
//
// Work decomposition. A workgroup (4 waves) owns one tile of rows (up to
// 16*NCB activation rows of one expert) and 64 consecutive weight rows n
// (16 per wave). In the two-weight modes each wave owns the same 16 n of both
// the gate and the up weight, so SiLU(gate)*up is formed in registers.
//
// Operands of v_mfma_f32_16x16x32_bf16 (D = A*B, 16x16 fp32 per 32 k):
//   A = weights: lane l holds row n0 + l%16 and 8 consecutive k;
//   B = activations: lane l holds token l%16 (of a 16-row block) and the same 8 k.
// The MFMA sums over k, so any assignment of real k to (lane/16, element) works
// as long as A and B agree. Here lane l with q = l/16 reads 16 bytes of codes =
// 32 consecutive k [kb + 32q, kb + 32q + 32) of its row (two whole 16-input
// groups, two scale bytes) and feeds them to 4 MFMAs, 8 k each. So every code
// byte is read once from HBM with 128-bit loads and dequantized in registers:
// e2m1 -> fp32 by the gfx950 packed convert, times the e4m3 block scale (exact),
// packed to bf16 (exact). scale_2 multiplies the fp32 accumulator at the end.
//
// Activations for the tile are staged through LDS in stages of 128*U k,
// double-buffered, one barrier per stage; the weight registers of stage i+1 are
// loaded while stage i is multiplied.
//
// Summation order of an output element: stages in increasing k, within a stage
// u = 0..U-1 and s = 0..3, each MFMA over its 32 k. It depends on nothing but k,
// so results do not depend on the batch or on which tile a row lands in.
#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int kGemmThreads = 256;
constexpr int kWaveRows = 16;                       // weight rows per wave
constexpr int kBlockN = kWaveRows * (kGemmThreads / 64);

template <int SEL>
__device__ __forceinline__ float e4m3_byte_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(w, SEL);
}

template <int U>
struct WStage {
  u32x4 c[U];
  uint32_t s[U];
};

template <int U>
__device__ __forceinline__ void load_w(WStage<U>& st, const uint8_t* codes_row, const uint8_t* scales_row,
                                       bool row_ok, int64_t kb, int q, int64_t K) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t kk = kb + 128 * u + 32 * q;
    if (row_ok && kk < K) {
      st.c[u] = ld16(codes_row + kk / 2);
      st.s[u] = *reinterpret_cast<const uint16_t*>(scales_row + kk / 16);
    } else {
      st.c[u] = u32x4{0, 0, 0, 0};
      st.s[u] = 0;
    }
  }
}

template <int MODE, int NCB, int U>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmArgs a) {
  constexpr bool kTwo = (MODE == kGateUp || MODE == kGated);
  constexpr bool kMoe = (MODE == kGateUp || MODE == kDown);
  constexpr int MT = 16 * NCB;       // rows per tile
  constexpr int KC = 128 * U;        // k per stage
  constexpr int LW = KC + 8;         // LDS row pitch in elements (16-byte pad: conflict-free b128 reads)
  constexpr int XCH = NCB * U;       // 16-byte activation chunks per thread per stage
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][MT][LW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 15, q = lane >> 4;
  const int64_t N = a.N, K = a.K;

  // ---- tile of rows
  int e = 0, row_begin, rows;
  if (kMoe) {
    if ((int)blockIdx.x >= *a.n_tiles) return;
    const int32_t* t = a.tiles + 4 * (int64_t)blockIdx.x;
    e = t[0];
    row_begin = t[1];
    rows = t[2];
  } else {
    row_begin = (int)blockIdx.x * MT;
    rows = (int)min((int64_t)MT, a.M - row_begin);
  }

  // ---- this lane's weight row
  const int64_t nbase = (int64_t)blockIdx.y * kBlockN + wave * kWaveRows;
  const int64_t nrow = nbase + lr;
  const bool row_ok = nrow < N;
  const int64_t wrow = (int64_t)e * N + (row_ok ? nrow : 0);
  const uint8_t* c0 = a.w0.codes + wrow * (K / 2);
  const uint8_t* s0 = a.w0.scales + wrow * (K / 16);
  const uint8_t* c1 = kTwo ? a.w1.codes + wrow * (K / 2) : nullptr;
  const uint8_t* s1 = kTwo ? a.w1.scales + wrow * (K / 16) : nullptr;

  // ---- this thread's activation chunks: chunk i covers row r_i, 8 k at 8*cc_i
  const uint16_t* xsrc[XCH];
  int xr[XCH], xc[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int idx = i * kGemmThreads + tid;
    xr[i] = idx / (16 * U);
    xc[i] = idx % (16 * U);
    xsrc[i] = nullptr;
    if (xr[i] < rows) {
      int64_t src;
      if (MODE == kGateUp) src = a.perm[row_begin + xr[i]] / a.topk;
      else src = row_begin + xr[i];
      xsrc[i] = a.x + src * K;
    }
  }
  // rows past the tile stay zero in both buffers for the whole kernel
  for (int i = tid; i < 2 * MT * (LW / 8); i += kGemmThreads) {
    const int b = i / (MT * (LW / 8)), rem = i % (MT * (LW / 8));
    const int r = rem / (LW / 8), c = rem % (LW / 8);
    if (r >= rows) st16(&xs[b][r][c * 8], u32x4{0, 0, 0, 0});
  }

  auto load_x = [&](u32x4 (&reg)[XCH], int64_t kb) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int64_t k0 = kb + 8 * xc[i];
      reg[i] = (xsrc[i] != nullptr && k0 < K) ? ld16(xsrc[i] + k0) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_x = [&](const u32x4 (&reg)[XCH], int b) {
#pragma unroll
    for (int i = 0; i < XCH; ++i)
      if (xr[i] < rows) st16(&xs[b][xr[i]][8 * xc[i]], reg[i]);
  };

  f32x4 acc0[NCB], acc1[kTwo ? NCB : 1];
#pragma unroll
  for (int i = 0; i < NCB; ++i) acc0[i] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < (kTwo ? NCB : 1); ++i) acc1[i] = f32x4{0, 0, 0, 0};

  const int nst = (int)((K + KC - 1) / KC);
  WStage<U> wc0, wn0;
  WStage<kTwo ? U : 1> wc1, wn1;
  {
    u32x4 xreg[XCH];
    load_x(xreg, 0);
    load_w<U>(wc0, c0, s0, row_ok, 0, q, K);
    if constexpr (kTwo) load_w<U>(wc1, c1, s1, row_ok, 0, q, K);
    store_x(xreg, 0);
  }
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const int b = st & 1;
    const bool more = st + 1 < nst;
    u32x4 xreg[XCH];
    if (more) {
      const int64_t kb = (int64_t)(st + 1) * KC;
      load_w<U>(wn0, c0, s0, row_ok, kb, q, K);
      if constexpr (kTwo) load_w<U>(wn1, c1, s1, row_ok, kb, q, K);
      load_x(xreg, kb);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float sc0 = (s < 2) ? e4m3_byte_to_f32<0>(wc0.s[u]) : e4m3_byte_to_f32<1>(wc0.s[u]);
        const bf16x8 A0 = dequant8(wc0.c[u][s], sc0);
        bf16x8 A1;
        if constexpr (kTwo) {
          const float sc1 = (s < 2) ? e4m3_byte_to_f32<0>(wc1.s[u]) : e4m3_byte_to_f32<1>(wc1.s[u]);
          A1 = dequant8(wc1.c[u][s], sc1);
        }
        // Every 16-row block is multiplied, also past `rows`: those LDS rows are zero
        // and their outputs are not stored. (Skipping them with a branch splits the
        // accumulators' live ranges and makes the compiler spill.)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const bf16x8 B = *reinterpret_cast<const bf16x8*>(&xs[b][16 * cb + lr][128 * u + 32 * q + 8 * s]);
          acc0[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B, acc0[cb], 0, 0, 0);
          if constexpr (kTwo) acc1[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B, acc1[cb], 0, 0, 0);
        }
      }
    }
    if (more) {
      store_x(xreg, b ^ 1);
      wc0 = wn0;
      if constexpr (kTwo) wc1 = wn1;
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds D[n = nbase + 4q + r][token = 16cb + lr], r = 0..3
  const float s2a = a.w0.scale_2[e];
  const float s2b = kTwo ? a.w1.scale_2[e] : 0.0f;
  const int64_t n0 = nbase + 4 * q;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int tok = 16 * cb + lr;
    if (tok >= rows) continue;
    const int64_t p = row_begin + tok;
    if constexpr (MODE == kDown) {
      const int64_t slot = a.perm[p];
      float* dst = reinterpret_cast<float*>(a.out) + slot * N + n0;
      if ((N & 3) == 0 && n0 + 3 < N) {
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = s2a * acc0[cb][r];
        *reinterpret_cast<f32x4*>(dst) = v;
      } else {
        for (int r = 0; r < 4; ++r)
          if (n0 + r < N) dst[r] = s2a * acc0[cb][r];
      }
    } else {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (kTwo) v[r] = silu(s2a * acc0[cb][r]) * (s2b * acc1[cb][r]);
        else v[r] = s2a * acc0[cb][r];
      }
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + p * N + n0;
      if ((N & 3) == 0 && n0 + 3 < N) {
        u32x2 o;
        o[0] = pack_bf16x2(v[0], v[1]);
        o[1] = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<u32x2*>(dst) = o;
      } else {
        for (int r = 0; r < 4; ++r)
          if (n0 + r < N) dst[r] = (uint16_t)(pack_bf16x2(v[r], 0.0f) & 0xFFFFu);
      }
    }
  }
}

int variant_tile_rows(GemmVariant v) { return v == kDecodeSmall ? 4 : v == kDecode ? 16 : 128; }

template <int MODE>
static hipError_t launch_mode(GemmVariant v, const GemmArgs& a, int64_t grid_tiles, hipStream_t s) {
  const dim3 grid((unsigned)grid_tiles, (unsigned)((a.N + kBlockN - 1) / kBlockN));
  if (v == kDecode)
    hipLaunchKernelGGL((gemm_kernel<MODE, 1, 4>), grid, dim3(kGemmThreads), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel<MODE, 8, 1>), grid, dim3(kGemmThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm(GemmMode mode, GemmVariant v, const GemmArgs& a, int64_t grid_tiles, hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  switch (mode) {
    case kGateUp: return launch_mode<kGateUp>(v, a, grid_tiles, s);
    case kDown: return launch_mode<kDown>(v, a, grid_tiles, s);
    case kLinear: return launch_mode<kLinear>(v, a, grid_tiles, s);
    case kGated: return launch_mode<kGated>(v, a, grid_tiles, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
