// Prefill-shaped grouped NVFP4 GEMM (tiles of up to 128 rows): matrix-core bound.
//
// Passage: TensorFold issue #308, "What the branch does" (routed experts in a
// grouped NVFP4 kernel on bf16 rows; the dense MLP on Fp4Linear with gate and
// up apart) and "Questions" item 4 (a prompt-shaped expert kernel whose sums
// do not depend on the chunking).
//
// Work decomposition. A workgroup (4 waves, one per SIMD) takes one tile of
// <= 128 rows of one expert and 256 weight rows: each wave owns 64 weight rows
// (for gate/up: the same 32 output columns of both weights, so SiLU(gate)*up is
// formed in registers) against all rows of the tile. v_mfma_f32_32x32x16_bf16 with
//   A = weights, dequantized straight from HBM into registers: lane (r, h) of a
//       32-row block owns row r and, of every 256-k stage, the four 32-k pieces
//       [kb + 64c + 32h, +32), c = 0..3: four 128-bit code loads in which the two
//       lanes of a row read 32 adjacent bytes, and one 16-byte scale load;
//   B = activations, a [128 x 256k] bf16 tile in LDS shared by the 4 waves,
//       streamed in with direct-to-LDS buffer loads (no registers held while in
//       flight), double-buffered, one barrier per stage.
// MFMA step s = 4c + d (0..15) of a stage pairs k = kb + 64c + 8d (h = 0) with
// kb + 64c + 32 + 8d (h = 1). The number of 32-row blocks multiplied follows the tile's real row
// count (1..4, picked per tile), so small experts do not pay for padding rows.
//
// Schedule. With one wave per SIMD nothing else hides latency, so the kernel is
// software-pipelined by hand: step s issues its MFMAs interleaved one by one with
// the dequant VALU work and LDS reads of step s + 1, and the loads of stage
// st + 1 are issued two per step over the first steps of stage st.
//
// Summation order of an output element: stages in increasing k, within a stage
// MFMA steps s = 0..15, each over its 16 k. It depends only on K.
#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace prefill_detail {

constexpr int kThreads = 256;
constexpr int KC = 256;             // k per stage
constexpr int SPS = KC / 16;        // MFMA steps per stage
constexpr int MT = 128;             // max rows per tile
// Activation tile in LDS: rows of KC bf16 plus one 16-byte pad, so row r starts
// 33*r 16-byte units into the buffer and 16 consecutive rows hit 16 distinct
// bank groups at any common k; every read address is a per-lane base plus a
// compile-time offset.
constexpr int RSU = KC / 8 + 1;     // 16-byte units per tile row (data + pad)
constexpr int RSB = 16 * RSU;       // tile row stride in bytes
constexpr int XI = ((MT * RSU + 63) / 64 + 3) / 4 * 4;  // 1 KB direct-to-LDS loads per stage
constexpr int XPW = XI / 4;         // of them per wave
constexpr int XBUF = XI * 1024;     // bytes per buffer
// Buffer descriptor word 3 for raw (untyped) buffer access on gfx9-family parts.
constexpr int kRsrcWord3 = 0x00020000;

template <int SEL>
__device__ __forceinline__ float sc(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(w, SEL);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// MFMA operand type of the bf16 and fp16 forms
template <bool F16> struct Op { typedef bf16x8 T; };
template <> struct Op<true> { typedef f16x8 T; };

struct WRegs {
  u32x4 c[2][4];          // [row block][piece c]: k = kb + 64c + 32h .. +32 of one row
  u32x4 s[2];             // [row block]: the row's 16 scale bytes of the stage
};

}  // namespace prefill_detail

using namespace prefill_detail;

template <int MODE, int NB, bool F16>
__device__ __forceinline__ void prefill_body(const GemmArgs& a, const F16Args& d, char* xs, int e, int rb,
                                             int rows) {
  typedef typename Op<F16>::T AT;
  constexpr bool kTwo = (MODE == kGateUp || MODE == kGated);
  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t N = a.N, K = a.K;

  // ---- weight rows of this lane: two 32-row blocks
  // two-weight modes: block 0 = gate rows n0 + r32, block 1 = up rows n0 + r32 (n0 = 128*by + 32*wave)
  // one-weight modes: block b = rows n0 + 32b + r32 (n0 = 256*by + 64*wave)
  // Every load is a buffer load: a descriptor over one expert's codes / scales
  // (or over x) plus a 32-bit per-lane offset and a uniform stage offset.
  const int64_t nbase = kTwo ? (int64_t)blockIdx.y * 128 + 32 * wave : (int64_t)blockIdx.y * 256 + 64 * wave;
  __amdgpu_buffer_rsrc_t crs[2], srs[2];
  uint32_t co[2], so[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    int64_t n = kTwo ? nbase + r32 : nbase + 32 * b + r32;
    if (n > N - 1) n = N - 1;                 // rows past N: computed, never stored
    const WeightDev& w = (kTwo && b == 1) ? a.w1 : a.w0;
    crs[b] = rsrc(w.codes + (int64_t)e * N * (K / 2), N * (K / 2));
    srs[b] = rsrc(w.scales + (int64_t)e * N * (K / 16), N * (K / 16));
    co[b] = (uint32_t)(n * (K / 2) + 16 * h);
    so[b] = (uint32_t)(n * (K / 16));
  }
  // loads j in [j0, j1) of the 10 per stage: j = 5b + c, c < 4 codes, c = 4 scales
  auto load_w = [&](WRegs& wr, int kb, int j0, int j1) {
#pragma unroll
    for (int j = 0; j < 10; ++j) {
      if (j < j0 || j >= j1) continue;
      const int b = j / 5, c = j % 5;
      if (c < 4) wr.c[b][c] = __builtin_amdgcn_raw_buffer_load_b128(crs[b], co[b] + 32 * c, kb / 2, 0);
      else wr.s[b] = __builtin_amdgcn_raw_buffer_load_b128(srs[b], so[b], kb / 16, 0);
    }
  };

  // ---- activation tile: 128 rows x KC k per stage, loaded straight into LDS.
  // Load J (of XI) lane l fills 16-byte unit u = 64J + l of the buffer: tile row
  // u / RSU, k chunk u % RSU. The pad unit of each row and the units past the
  // last row load the row's first chunk (never read). Rows past the tile in the
  // last load J that holds tile rows load the tile's last row: their results are
  // never stored. Wave w issues loads J = w + 4i.
  const __amdgpu_buffer_rsrc_t xrs = rsrc(a.x, a.x_rows * K * 2);
  uint32_t xo[XPW];
#pragma unroll
  for (int i = 0; i < XPW; ++i) {
    const int u = 64 * (wave + 4 * i) + lane;
    int r = u / RSU;
    int c = u % RSU;
    if (c == RSU - 1) c = 0;
    if (r > rows - 1) r = rows - 1;
    int64_t src;
    if (MODE == kGateUp) src = a.perm[rb + r] / a.topk;
    else src = rb + r;
    xo[i] = (uint32_t)(2 * (src * K + 8 * c));
  }
  // loads i in [i0, i1) of this wave's XPW; only those that hold rows of the tile
  // (B columns past the tile then read stale LDS: they only reach results that are
  // never stored)
  const int xunits = rows * RSU;
  auto issue_x = [&](int kb, int buf, int i0, int i1) {
#pragma unroll
    for (int i = 0; i < XPW; ++i) {
      if (i < i0 || i >= i1) continue;
      if (64 * (wave + 4 * i) >= xunits) continue;
      auto* dst = (__attribute__((address_space(3))) void*)(xs + buf * XBUF + 1024 * (wave + 4 * i));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, dst, 16, xo[i], 2 * kb, 0, 0);
    }
  };

  f32x16 acc[2][NB];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int t = 0; t < NB; ++t) acc[b][t] = f32x16{};

  // A operands of MFMA step s = 4c + d: 8 codes (k = kb + 64c + 32h + 8d ..) of each
  // row block; their scale is byte 4c + 2h + d/2 of the stage's 16
  const uint32_t hs = 16 * h;
  auto prep_a = [&](const WRegs& wr, int s, AT (&A)[2]) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const uint32_t word = wr.c[b][s / 4][s % 4];
      const uint32_t sw = wr.s[b][s / 4] >> hs;
      if constexpr (F16) {
        const f16x2 s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
        A[b] = dequant8_f16(word, ((s % 4) < 2) ? f16x2{s2[0], s2[0]} : f16x2{s2[1], s2[1]});
      } else {
        A[b] = dequant8(word, ((s % 4) < 2) ? sc<0>(sw) : sc<1>(sw));
      }
    }
  };
  // B operands of MFMA step s = 4c + d: tile row 32t + r32, 16-byte unit 8c + 4h + d
  const char* const xrd = xs + r32 * RSB + 64 * h;
  auto prep_b = [&](int buf, int s, AT (&B)[NB]) {
#pragma unroll
    for (int t = 0; t < NB; ++t)
      B[t] = *reinterpret_cast<const AT*>(xrd + buf * XBUF + t * 32 * RSB + 16 * (8 * (s / 4) + s % 4));
  };
  // MFMAs i in [i0, i1) of one step, i = 2t + b
  auto mma = [&](const AT (&A)[2], const AT (&B)[NB], int i0, int i1) {
#pragma unroll
    for (int i = 0; i < 2 * NB; ++i) {
      if (i < i0 || i >= i1) continue;
      const int t = i / 2, b = i % 2;
      if constexpr (F16) acc[b][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[b], B[t], acc[b][t], 0, 0, 0);
      else acc[b][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[b], B[t], acc[b][t], 0, 0, 0);
    }
  };

  // ---- pipeline. Stage st computes from register set st % 2 and LDS buffer st % 2
  // while the loads of stage st + 1 go into the other set and buffer (both free
  // since the previous hand-over), spread over the first steps of the stage: a
  // burst of loads at one point stalls the LDS reads and MFMAs behind it. The last
  // stage reloads itself there instead (never read), which keeps the steps free of
  // branches. The last step of a stage hands over: wait for this wave's loads,
  // barrier (tile st + 1 complete everywhere, buffer st % 2 free), and prepare
  // step 0 of stage st + 1.
  const int nst = (int)(K / KC);
  WRegs wa, wb;
  issue_x(0, 0, 0, XPW);
  load_w(wa, 0, 0, 10);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  AT A[2], B[NB];
  prep_a(wa, 0, A);
  prep_b(0, 0, B);

  auto stage = [&](const WRegs& cur, WRegs& nxt, int buf, int st) {
    const int kn = (st + 1 < nst ? st + 1 : st) * KC;
#pragma unroll
    for (int s = 0; s < SPS; ++s) {
      AT An[2], Bn[NB];
      issue_x(kn, buf ^ 1, 2 * s, 2 * s + 2);
      load_w(nxt, kn, 2 * s, 2 * s + 2);
      if (s + 1 < SPS) {
        prep_a(cur, s + 1, An);
        prep_b(buf, s + 1, Bn);
        mma(A, B, 0, 2 * NB);
        // one MFMA, then (early) one LDS read, then a share of the dequant VALU
#pragma unroll
        for (int i = 0; i < 2 * NB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < NB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, (36 + 2 * NB - 1) / (2 * NB), 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        mma(A, B, 0, NB);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        prep_a(nxt, 0, An);
        prep_b(buf ^ 1, 0, Bn);
        mma(A, B, NB, 2 * NB);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) A[b] = An[b];
#pragma unroll
      for (int t = 0; t < NB; ++t) B[t] = Bn[t];
    }
  };
  // Pairs of stages, then an odd last one.
  int st = 0;
  for (; st + 1 < nst; st += 2) {
    stage(wa, wb, 0, st);
    stage(wb, wa, 1, st + 1);
  }
  if (st < nst) stage(wa, wb, 0, st);

  // ---- epilogue. 32x32 result layout: lane l holds column (row of the tile) l % 32
  // and weight rows 8*(j/4) + 4*(l/32) + j%4, j = 0..15.
  // fp16 form: the activation row was scaled by 2^p; the results are scaled back
  // here (exactly: a power of two). Routed gate/up also records max |H| of each
  // row as stored (order-free max, so deterministic) for the fp16 form of down.
  const float s2a0 = a.w0.scale_2[e];
  const float s2b0 = kTwo ? a.w1.scale_2[e] : 0.0f;
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const int tok = 32 * t + r32;
    if (tok >= rows) continue;
    const int64_t p = rb + tok;
    float unscale = 1.0f;
    if constexpr (F16 && MODE == kGateUp) unscale = ldexpf(1.0f, -d.xexp[a.perm[p] / a.topk]);
    if constexpr (F16 && MODE == kDown) unscale = ldexpf(1.0f, -row_exponent(d.hmax[p]));
    const float s2a = s2a0 * unscale, s2b = s2b0 * unscale;
    float hm = 0.0f;
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
          if constexpr (F16 && MODE == kGateUp) {
#pragma unroll
            for (int j = 0; j < 4; ++j) hm = fmaxf(hm, fabsf(bf16_lo(j & 1 ? o[j / 2] >> 16 : o[j / 2])));
          }
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
    if constexpr (F16 && MODE == kGateUp) {
      hm = fmaxf(hm, __shfl_xor(hm, 32));
      if (h == 0) atomicMax(reinterpret_cast<unsigned int*>(d.hmax + p), __builtin_bit_cast(unsigned int, hm));
    }
  }
}

template <int MODE, bool F16>
__global__ __launch_bounds__(kThreads, 1) void gemm_prefill_kernel(GemmArgs a, F16Args d) {
  constexpr bool kMoe = (MODE == kGateUp || MODE == kDown);
  __shared__ __attribute__((aligned(16))) char xs[2 * XBUF];
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
    case 1: prefill_body<MODE, 1, F16>(a, d, xs, e, rb, rows); break;
    case 2: prefill_body<MODE, 2, F16>(a, d, xs, e, rb, rows); break;
    case 3: prefill_body<MODE, 3, F16>(a, d, xs, e, rb, rows); break;
    default: prefill_body<MODE, 4, F16>(a, d, xs, e, rb, rows); break;
  }
}

bool prefill_supported(GemmMode mode, int64_t x_rows, int64_t K, int64_t N) {
  (void)mode;
  // 32-bit buffer ranges: x, and one expert's codes (its scales are smaller)
  const int64_t lim = (int64_t)1 << 31;
  return K % KC == 0 && K >= KC && N % 32 == 0 && x_rows * K * 2 < lim && N * (K / 2) < lim;
}

hipError_t launch_prefill(GemmMode mode, bool f16, const GemmArgs& a, const F16Args& d, int64_t grid_tiles,
                          hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  const bool two = (mode == kGateUp || mode == kGated);
  const int64_t nw = two ? 128 : 256;
  const dim3 grid((unsigned)grid_tiles, (unsigned)((a.N + nw - 1) / nw));
  switch (mode) {
    case kGateUp:
      if (f16) hipLaunchKernelGGL((gemm_prefill_kernel<kGateUp, true>), grid, dim3(kThreads), 0, s, a, d);
      else hipLaunchKernelGGL((gemm_prefill_kernel<kGateUp, false>), grid, dim3(kThreads), 0, s, a, d);
      break;
    case kDown:
      if (f16) hipLaunchKernelGGL((gemm_prefill_kernel<kDown, true>), grid, dim3(kThreads), 0, s, a, d);
      else hipLaunchKernelGGL((gemm_prefill_kernel<kDown, false>), grid, dim3(kThreads), 0, s, a, d);
      break;
    case kLinear: hipLaunchKernelGGL((gemm_prefill_kernel<kLinear, false>), grid, dim3(kThreads), 0, s, a, d); break;
    case kGated: hipLaunchKernelGGL((gemm_prefill_kernel<kGated, false>), grid, dim3(kThreads), 0, s, a, d); break;
  }
  return hipGetLastError();
}

// H rows (bf16, in place) -> fp16 times 2^p, p from the row's recorded max |H|:
// the input of the fp16 form of the routed down projection. 8 elements per thread.
__global__ __launch_bounds__(256) void h_to_f16_kernel(uint16_t* h, const uint32_t* hmax, int64_t S, int64_t I) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= S * I) return;
  const int64_t p = i / I;
  const float sc = ldexpf(1.0f, row_exponent(hmax[p]));
  const u32x4 v = ld16(h + i);
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x2 q = {(_Float16)(bf16_lo(v[j]) * sc), (_Float16)(bf16_hi(v[j]) * sc)};
    o[j] = __builtin_bit_cast(uint32_t, q);
  }
  st16(h + i, o);
}

hipError_t launch_h_to_f16(uint16_t* h, const uint32_t* hmax, int64_t S, int64_t I, hipStream_t s) {
  if (S * I == 0) return hipSuccess;
  const int64_t blocks = (S * I / 8 + 255) / 256;
  hipLaunchKernelGGL(h_to_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, h, hmax, S, I);
  return hipGetLastError();
}

}  // namespace nvfp4
