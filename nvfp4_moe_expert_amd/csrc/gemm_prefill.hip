// Prefill-shaped grouped NVFP4 GEMM (tiles of up to 128 rows): matrix-core bound.
//
// Passage: TensorFold issue #308, "What the branch does" (routed experts in a
// grouped NVFP4 kernel on bf16 rows; the dense MLP on Fp4Linear with gate and
// up apart) and "Questions" item 4 (a prompt-shaped expert kernel whose sums
// do not depend on the chunking).
//
// Work decomposition. A workgroup (4 waves) takes one tile of <= 128 rows of
// one expert and 256 weight rows: each wave owns 64 weight rows (for gate/up:
// the same 32 output columns of both weights, so SiLU(gate)*up is formed in
// registers) against all rows of the tile. v_mfma_f32_32x32x16_bf16 with
//   A = weights, dequantized straight from HBM into registers: lane (r, h) of a
//       32-row block owns row r and the contiguous k range [kb + 64h, kb + 64h + 64)
//       of every 128-k stage: two 128-bit code loads and one 4-byte scale load;
//   B = activations, a [128 x 128k] bf16 tile in LDS shared by the 4 waves,
//       streamed in with gfx950's direct-to-LDS loads (no registers held while
//       in flight), double-buffered, one barrier per stage.
// MFMA step s of a stage pairs k = kb + 8s (h = 0) with kb + 64 + 8s (h = 1).
// The number of 32-row blocks multiplied follows the tile's real row count
// (1..4, a template parameter picked per tile), so small experts do not pay
// for padding rows. Per stage a wave issues 64 MFMAs (2048 matrix cycles)
// against 256 VALU dequant ops and 32 LDS reads.
//
// Summation order of an output element: stages in increasing k, within a
// stage MFMA steps s = 0..8*KS-1, each over its 16 k. It depends only on K.
#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace prefill_detail {

constexpr int kThreads = 256;
constexpr int KS = 2;               // 128-k halves per stage
constexpr int KC = 128 * KS;        // k per stage
constexpr int MT = 128;             // max rows per tile
constexpr int RCH = KC / 8;         // 16-byte activation chunks per tile row per stage
constexpr int XI = MT * KC * 2 / 1024;   // 1 KB direct-to-LDS instructions per stage

template <int SEL>
__device__ __forceinline__ float sc(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(w, SEL);
}

struct WRegs {
  u32x4 c[2][2 * KS];     // [row block][16-byte chunk]: 64*KS k of one row per row block
  uint32_t s[2][KS];      // [row block]: 4*KS scale bytes
};

}  // namespace prefill_detail

using namespace prefill_detail;

template <int MODE, int NB>
__device__ __forceinline__ void prefill_body(const GemmArgs& a, uint16_t (&xs)[2][MT][KC], int e, int rb, int rows) {
  constexpr bool kTwo = (MODE == kGateUp || MODE == kGated);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r32 = lane & 31, h = lane >> 5;
  const int64_t N = a.N, K = a.K;

  // ---- weight rows of this lane: two 32-row blocks
  // two-weight modes: block 0 = gate rows n0 + r32, block 1 = up rows n0 + r32 (n0 = 128*by + 32*wave)
  // one-weight modes: block b = rows n0 + 32b + r32 (n0 = 256*by + 64*wave)
  const int64_t nbase = kTwo ? (int64_t)blockIdx.y * 128 + 32 * wave : (int64_t)blockIdx.y * 256 + 64 * wave;
  const uint8_t* cp[2];
  const uint8_t* sp[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    int64_t n = kTwo ? nbase + r32 : nbase + 32 * b + r32;
    if (n > N - 1) n = N - 1;                 // rows past N: computed, never stored
    const WeightDev& w = (kTwo && b == 1) ? a.w1 : a.w0;
    const int64_t row = (int64_t)e * N + n;
    cp[b] = w.codes + row * (K / 2) + 32 * KS * h;     // lane's 64*KS k = 32*KS bytes
    sp[b] = w.scales + row * (K / 16) + 4 * KS * h;
  }
  auto load_w = [&](WRegs& wr, int64_t kb) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int c = 0; c < 2 * KS; ++c) wr.c[b][c] = ld16(cp[b] + kb / 2 + 16 * c);
      if constexpr (KS == 2) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(sp[b] + kb / 16);
        wr.s[b][0] = v[0];
        wr.s[b][1] = v[1];
      } else {
        wr.s[b][0] = *reinterpret_cast<const uint32_t*>(sp[b] + kb / 16);
      }
    }
  };

  // ---- activation tile: 128 rows x KC k bf16 per stage, loaded straight into LDS.
  // Row r of the tile holds its 16-byte chunk c at position c ^ (r & 15), so the
  // MFMA reads below hit 16 distinct bank groups. Wave w issues instructions
  // J = w + 4i; lane l of J fills row (64J + l) / RCH, position (64J + l) % RCH.
  // Rows past the tile load the tile's last row: their results are never stored.
  constexpr int XPW = XI / 4;                    // instructions per wave per stage
  const uint16_t* xsrc[XPW];
#pragma unroll
  for (int i = 0; i < XPW; ++i) {
    const int J = wave + 4 * i;
    int r = (64 * J + lane) / RCH;
    const int c = ((64 * J + lane) % RCH) ^ (r & 15);
    if (r > rows - 1) r = rows - 1;
    int64_t src;
    if (MODE == kGateUp) src = a.perm[rb + r] / a.topk;
    else src = rb + r;
    xsrc[i] = a.x + src * K + 8 * c;
  }
  auto issue_x = [&](int64_t kb, int buf) {
#pragma unroll
    for (int i = 0; i < XPW; ++i) {
      const int J = wave + 4 * i;
      __builtin_amdgcn_global_load_lds(xsrc[i] + kb, &xs[buf][0][0] + 512 * J, 16, 0, 0);
    }
  };

  f32x16 acc[2][NB];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int t = 0; t < NB; ++t) acc[b][t] = f32x16{};

  auto compute = [&](const WRegs& wr, int buf) {
#pragma unroll
    for (int s = 0; s < 8 * KS; ++s) {
      // A: 8 codes (k = kb + 64*KS*h + 8s ..) of each row block
      bf16x8 A[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const uint32_t word = wr.c[b][s / 4][s % 4];
        const uint32_t sw = wr.s[b][s / 8];
        const int g = (s / 2) % 4;
        const float scale = (g == 0) ? sc<0>(sw) : (g == 1) ? sc<1>(sw) : (g == 2) ? sc<2>(sw) : sc<3>(sw);
        A[b] = dequant8(word, scale);
      }
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        const int row = 32 * t + r32;
        const bf16x8 B = *reinterpret_cast<const bf16x8*>(&xs[buf][row][8 * ((8 * KS * h + s) ^ (row & 15))]);
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[b][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[b], B, acc[b][t], 0, 0, 0);
      }
    }
  };

  const int nst = (int)(K / KC);
  WRegs wa, wb;
  load_w(wa, 0);
  issue_x(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int st = 0;
  for (; st + 2 <= nst; st += 2) {
    // stage st from (wa, buffer 0) while stage st+1 streams into (wb, buffer 1)
    load_w(wb, (int64_t)(st + 1) * KC);
    issue_x((int64_t)(st + 1) * KC, 1);
    compute(wa, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const bool more = st + 2 < nst;
    if (more) {
      load_w(wa, (int64_t)(st + 2) * KC);
      issue_x((int64_t)(st + 2) * KC, 0);
    }
    compute(wb, 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (st < nst) compute(wa, 0);

  // ---- epilogue. 32x32 result layout: lane l holds column (row of the tile) l % 32
  // and weight rows 8*(j/4) + 4*(l/32) + j%4, j = 0..15.
  const float s2a = a.w0.scale_2[e];
  const float s2b = kTwo ? a.w1.scale_2[e] : 0.0f;
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const int tok = 32 * t + r32;
    if (tok >= rows) continue;
    const int64_t p = rb + tok;
#pragma unroll
    for (int g = 0; g < 4; ++g) {               // 4 groups of 4 consecutive weight rows
      float v0[4], v1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v0[j] = acc[0][t][4 * g + j];
        v1[j] = acc[1][t][4 * g + j];
      }
      const int off = 8 * g + 4 * h;            // weight row within the 32-row block
      if constexpr (kTwo) {
        const int64_t n = nbase + off;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = silu(s2a * v0[j]) * (s2b * v1[j]);
        if (n < N) {
          uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + p * N + n;
          u32x2 o;
          o[0] = pack_bf16x2(v[0], v[1]);
          o[1] = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<u32x2*>(dst) = o;
        }
      } else {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int64_t n = nbase + 32 * b + off;
          if (n >= N) continue;
          const float* vv = b == 0 ? v0 : v1;
          if constexpr (MODE == kDown) {
            float* dst = reinterpret_cast<float*>(a.out) + (int64_t)a.perm[p] * N + n;
            *reinterpret_cast<f32x4*>(dst) = f32x4{s2a * vv[0], s2a * vv[1], s2a * vv[2], s2a * vv[3]};
          } else {
            uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + p * N + n;
            u32x2 o;
            o[0] = pack_bf16x2(s2a * vv[0], s2a * vv[1]);
            o[1] = pack_bf16x2(s2a * vv[2], s2a * vv[3]);
            *reinterpret_cast<u32x2*>(dst) = o;
          }
        }
      }
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_prefill_kernel(GemmArgs a) {
  constexpr bool kMoe = (MODE == kGateUp || MODE == kDown);
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][MT][KC];
  int e = 0, rb, rows;
  if (kMoe) {
    if ((int)blockIdx.x >= *a.n_tiles) return;
    const int32_t* t = a.tiles + 4 * (int64_t)blockIdx.x;
    e = t[0];
    rb = t[1];
    rows = t[2];
  } else {
    rb = (int)blockIdx.x * MT;
    rows = (int)min((int64_t)MT, a.M - rb);
  }
  const int nb = (rows + 31) / 32;
  switch (nb) {
    case 1: prefill_body<MODE, 1>(a, xs, e, rb, rows); break;
    case 2: prefill_body<MODE, 2>(a, xs, e, rb, rows); break;
    case 3: prefill_body<MODE, 3>(a, xs, e, rb, rows); break;
    default: prefill_body<MODE, 4>(a, xs, e, rb, rows); break;
  }
}

bool prefill_supported(GemmMode mode, int64_t K, int64_t N) {
  (void)mode;
  return K % KC == 0 && K >= KC && N % 32 == 0;
}

hipError_t launch_prefill(GemmMode mode, const GemmArgs& a, int64_t grid_tiles, hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  const bool two = (mode == kGateUp || mode == kGated);
  const int64_t nw = two ? 128 : 256;
  const dim3 grid((unsigned)grid_tiles, (unsigned)((a.N + nw - 1) / nw));
  switch (mode) {
    case kGateUp: hipLaunchKernelGGL(gemm_prefill_kernel<kGateUp>, grid, dim3(kThreads), 0, s, a); break;
    case kDown: hipLaunchKernelGGL(gemm_prefill_kernel<kDown>, grid, dim3(kThreads), 0, s, a); break;
    case kLinear: hipLaunchKernelGGL(gemm_prefill_kernel<kLinear>, grid, dim3(kThreads), 0, s, a); break;
    case kGated: hipLaunchKernelGGL(gemm_prefill_kernel<kGated>, grid, dim3(kThreads), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace nvfp4
