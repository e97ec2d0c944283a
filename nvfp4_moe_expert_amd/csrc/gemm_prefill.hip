// Prefill-shaped grouped NVFP4 GEMM (tiles of up to 128 rows): matrix-core bound.
//
// Passage: TensorFold issue #308, "What the branch does" (routed experts in a
// grouped NVFP4 kernel on bf16 rows; the dense MLP on Fp4Linear with gate and
// up apart) and "Questions" item 4 (a prompt-shaped expert kernel whose sums
// do not depend on the chunking).
//
// Work decomposition. A workgroup (8 waves, two per SIMD) takes one tile of
// <= 128 rows of one expert and 512 weight rows: each wave owns 64 weight rows
// (for gate/up: the same 32 output columns of both weights, so SiLU(gate)*up is
// formed in registers) against all rows of the tile. v_mfma_f32_32x32x16 with
//   A = weights, dequantized straight from HBM into registers: lane (r, h) of a
//       32-row block owns row r and the contiguous k range [kb + 128h, +128) of
//       every 256-k stage: four 128-bit code loads (pieces c of 32 k) and one
//       8-byte scale load;
//   B = activations, a [128 x 256k] tile in LDS shared by the 8 waves, streamed
//       in with direct-to-LDS buffer loads (no registers held while in flight),
//       double-buffered, one barrier per stage.
// MFMA step s (0..15) of a stage pairs k = kb + 8s (h = 0) with kb + 128 + 8s
// (h = 1). The number of 32-row blocks multiplied follows the
// tile's real row count (1..4, picked per tile), so small experts do not pay for
// padding rows. Eight waves share each activation tile, so a stage moves 64 KB of
// activations per 512 weight rows; the two waves of a SIMD hide each other's
// latencies.
//
// Schedule per wave: step s issues its LDS reads and MFMAs interleaved with the
// dequant of step s + 1 (sched_group_barrier). The loads of stage st + 1 go out
// during stage st: one activation load per step, the scales at step 0 (their
// registers are double-buffered), and code piece c at step 4c + 3, right after
// its last use (the code registers are single-buffered).
//
// Summation order of an output element: stages in increasing k, within a stage
// MFMA steps s = 0..15, each over its 16 k. It depends only on K.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace prefill_detail {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int KC = 256;             // k per stage
constexpr int SPS = KC / 16;        // MFMA steps per stage
constexpr int MT = 128;             // max rows per tile
// Activation tile in LDS: rows of KC bf16 plus one 16-byte pad, so row r starts
// 33*r 16-byte units into the buffer and 16 consecutive rows hit 16 distinct
// bank groups at any common k; every read address is a per-lane base plus a
// compile-time offset.
constexpr int RSU = KC / 8 + 1;     // 16-byte units per tile row (data + pad)
constexpr int RSB = 16 * RSU;       // tile row stride in bytes
constexpr int XI = ((MT * RSU + 63) / 64 + kWaves - 1) / kWaves * kWaves;  // 1 KB direct-to-LDS loads per stage
constexpr int XPW = XI / kWaves;    // of them per wave
constexpr int XBUF = XI * 1024;     // bytes per buffer
template <int SEL>
__device__ __forceinline__ float sc(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(w, SEL);
}


// MFMA operand type of the bf16 and fp16 forms
template <bool F16> struct Op { typedef bf16x8 T; };
template <> struct Op<true> { typedef f16x8 T; };



}  // namespace prefill_detail

using namespace prefill_detail;

template <int MODE, int NB, bool F16, int WB, bool TL>
__device__ __forceinline__ void prefill_body(const GemmArgs& a, const F16Args& d, char* xs, int e, int rb,
                                             int rows, int nblk) {
  typedef typename Op<F16>::T AT;
  constexpr bool kTwo = (MODE == kGateUp || MODE == kGated);
  constexpr int W = kTwo ? 2 : WB;     // 32-row weight blocks per wave
  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t N = a.N, K = a.K;

  // ---- weight rows of this lane: W 32-row blocks
  // two-weight modes: block 0 = gate rows n0 + r32, block 1 = up rows n0 + r32 (n0 = 256*by + 32*wave)
  // one-weight modes: block b = rows n0 + 32b + r32 (n0 = 32*WB*(8*by + wave))
  // Every load is a buffer load: a descriptor over one expert's codes / scales
  // (or over x) plus a 32-bit per-lane offset and a uniform stage offset.
  const int64_t nbase = kTwo ? (int64_t)nblk * (32 * kWaves) + 32 * wave
                             : (int64_t)nblk * (32 * WB * kWaves) + 32 * WB * wave;
  __amdgpu_buffer_rsrc_t crs[W], srs[W];
  uint32_t co[W], so[W];
#pragma unroll
  for (int b = 0; b < W; ++b) {
    int64_t n = kTwo ? nbase + r32 : nbase + 32 * b + r32;
    if (n > N - 1) n = N - 1;                 // rows past N: computed, never stored
    const WeightDev& w = (kTwo && b == 1) ? a.w1 : a.w0;
    crs[b] = rsrc(w.codes + (int64_t)e * N * (K / 2), N * (K / 2));
    srs[b] = rsrc(w.scales + (int64_t)e * N * (K / 16), N * (K / 16));
    if constexpr (TL) {   // blocks of 32 rows: 512-byte runs per 32-input chunk / 256-input scale chunk
      co[b] = (uint32_t)(((n / 32) * (K / 32) + 4 * h) * 512 + (n % 32) * 16);
      so[b] = (uint32_t)((n / 32) * (K / 256) * 512 + (n % 32) * 16 + 8 * h);
    } else {
      co[b] = (uint32_t)(n * (K / 2) + 64 * h);
      so[b] = (uint32_t)(n * (K / 16) + 8 * h);
    }
  }
  // codes: [set][row block][piece c] (k = kb + 128h + 32c .. +32 of the row);
  // scales: [set][row block] (the 8 scale bytes of the lane's 128 k). Tiles of up
  // to 64 rows (DEEP) keep two code sets and load weights two stages ahead: their
  // stages are short, and one stage of lead does not cover the memory latency.
  constexpr bool DEEP = NB <= 2;
  constexpr int CS = DEEP ? 2 : 1;
  u32x4 wc[CS][W][4];
  u32x2 wsc[2][W];
  auto load_codes = [&](int cs, int c, int kb) {
#pragma unroll
    for (int b = 0; b < W; ++b)
      wc[cs][b][c] = __builtin_amdgcn_raw_buffer_load_b128(crs[b], co[b] + (TL ? 512 : 16) * c, TL ? 16 * kb : kb / 2, 0);
  };
  auto load_scales = [&](int set, int kb) {
#pragma unroll
    for (int b = 0; b < W; ++b) wsc[set][b] = __builtin_amdgcn_raw_buffer_load_b64(srs[b], so[b], TL ? 2 * kb : kb / 16, 0);
  };

  // ---- activation tile: 128 rows x KC k per stage, loaded straight into LDS.
  // Load J (of XI) lane l fills 16-byte unit u = 64J + l of the buffer: tile row
  // u / RSU, k chunk u % RSU. The pad unit of each row and the units past the
  // last row load the row's first chunk (never read). Rows past the tile load the
  // tile's last row: their results are never stored. Wave w issues loads J = w + 8i.
  const __amdgpu_buffer_rsrc_t xrs = rsrc(a.x, a.x_rows * K * 2);
  uint32_t xo[XPW];
#pragma unroll
  for (int i = 0; i < XPW; ++i) {
    const int u = 64 * (wave + kWaves * i) + lane;
    int r = u / RSU;
    int c = u % RSU;
    if (c == RSU - 1) c = 0;
    if (r > rows - 1) r = rows - 1;
    int64_t src;
    if (MODE == kGateUp) src = a.perm[rb + r] / a.topk;
    else src = rb + r;
    xo[i] = (uint32_t)(2 * (src * K + 8 * c));
  }
  // loads i in [i0, i1) of this wave's XPW; only the loads that fill the NB
  // 32-row blocks the MFMAs read are issued
  constexpr int XN = (32 * NB * RSU + 63) / 64;
  // Row-major weights may have K % 256 != 0 (any multiple of 64: the shards of a
  // tensor-parallel split); then the last stage runs past K. Its activation chunks
  // past K are read through an offset beyond the descriptor's range (zeros, no
  // memory access), so the weights read there (the next row's finite bytes, or
  // zeros past the tensor) multiply zeros. Chunk of load i: (64 (wave + 8i) + lane)
  // mod RSU, the pad chunk read as chunk 0.
  const int cbase = (64 * wave + lane) % RSU;
  auto issue_x = [&](int kb, int buf, int i0, int i1) {
    const bool rag = kb + KC > K;   // uniform
#pragma unroll
    for (int i = 0; i < XPW; ++i) {
      if (i < i0 || i >= i1 || wave + kWaves * i >= XN) continue;
      uint32_t off = xo[i];
      if (rag) {
        int c = cbase + (64 * kWaves * i) % RSU;
        if (c >= RSU) c -= RSU;
        if (c == RSU - 1) c = 0;
        if (kb + 8 * c >= K) off = 0x80000000u;
      }
      auto* dst = (__attribute__((address_space(3))) void*)(xs + buf * XBUF + 1024 * (wave + kWaves * i));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, dst, 16, off, 2 * kb, 0, 0);
    }
  };

  f32x16 acc[W][NB];
#pragma unroll
  for (int b = 0; b < W; ++b)
#pragma unroll
    for (int t = 0; t < NB; ++t) acc[b][t] = f32x16{};

  // A operands of MFMA step s: 8 codes (k = kb + 128h + 8s ..) of each row block;
  // their scale is byte s/2 of the lane's 8
  auto prep_a = [&](int set, int s, AT (&A)[W]) {
#pragma unroll
    for (int b = 0; b < W; ++b) {
      const uint32_t word = wc[DEEP ? set : 0][b][s / 4][s % 4];
      const uint32_t sw = wsc[set][b][s / 8];
      const int g = (s / 2) % 4;
      if constexpr (F16) {
        const f16x2 s2 = (g >= 2) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true)
                                  : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
        A[b] = dequant8_f16(word, (g % 2 == 0) ? f16x2{s2[0], s2[0]} : f16x2{s2[1], s2[1]});
      } else {
        A[b] = dequant8(word, (g == 0) ? sc<0>(sw) : (g == 1) ? sc<1>(sw) : (g == 2) ? sc<2>(sw) : sc<3>(sw));
      }
    }
  };
  // B operands of MFMA step s: tile row 32t + r32, 16-byte unit 16h + s
  const char* const xrd = xs + r32 * RSB + 256 * h;
  auto prep_b = [&](int buf, int s, AT (&B)[NB]) {
#pragma unroll
    for (int t = 0; t < NB; ++t)
      B[t] = *reinterpret_cast<const AT*>(xrd + buf * XBUF + t * 32 * RSB + 16 * s);
  };
  // MFMAs i in [i0, i1) of one step, i = W*t + b
  auto mma = [&](const AT (&A)[W], const AT (&B)[NB], int i0, int i1) {
#pragma unroll
    for (int i = 0; i < W * NB; ++i) {
      if (i < i0 || i >= i1) continue;
      const int t = i / W, b = i % W;
      if constexpr (F16) acc[b][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[b], B[t], acc[b][t], 0, 0, 0);
      else acc[b][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[b], B[t], acc[b][t], 0, 0, 0);
    }
  };

  // ---- pipeline. Stage st reads LDS buffer st % 2 and scale set st % 2; the loads
  // of stage st + 1 are spread over its steps (see the header). The last stage
  // reloads itself there instead (never read), which keeps the steps free of
  // branches. The last step hands over: wait for this wave's activation and scale
  // loads of stage st + 1 (only the code loads issued after the last activation
  // load may still be in flight: 2W of them, 5W with DEEP), barrier (tile st + 1
  // complete everywhere, buffer st % 2 free), and prepare step 0 of stage st + 1.
  const int nst = (int)((K + KC - 1) / KC);
  issue_x(0, 0, 0, XPW);
  load_scales(0, 0);
#pragma unroll
  for (int c = 0; c < 4; ++c) load_codes(0, c, 0);
  if constexpr (DEEP) {
    const int k1 = (nst > 1 ? 1 : 0) * KC;
    load_scales(1, k1);
#pragma unroll
    for (int c = 0; c < 4; ++c) load_codes(1, c, k1);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  AT A[W], B[NB];

  // Stage st uses LDS buffer st % 2, scale set st % 2 and (DEEP) code set st % 2.
  // Activation loads of stage st + 1 go out one per step in steps 0..8.
  //   normal: scales of st + 1 at step 0 into the other set, code piece c of st + 1
  //           at step 4c + 3 (its last use); at the hand-over the 2W code loads of
  //           steps 11 and 15 may still be in flight;
  //   DEEP:   code piece c of st + 2 at step 9 + c (c < 3) and 15, scales of st + 2
  //           at step 15, all into this stage's sets; the 5W loads after the last
  //           activation load may be in flight at the hand-over.
  // (A wave whose activation loads end before step 8 waits for more: still safe.)
  auto stage = [&](int set, int buf, int st) {
    const int kn = (st + 1 < nst ? st + 1 : st) * KC;
    const int kn2 = (st + 2 < nst ? st + 2 : nst - 1) * KC;
#pragma unroll
    for (int s = 0; s < SPS; ++s) {
      issue_x(kn, buf ^ 1, s, s + 1);
      if (!DEEP && s == 0) load_scales(set ^ 1, kn);
      prep_b(buf, s, B);
      prep_a(set, s, A);
      if constexpr (DEEP) {
        if (s >= 9 && s <= 11) load_codes(set, s - 9, kn2);
        if (s == 15) {
          load_codes(set, 3, kn2);
          load_scales(set, kn2);
        }
      } else {
        if (s % 4 == 3) load_codes(0, s / 4, kn);   // piece s/4 was last used just above
      }
      // the wave issuing its MFMAs takes the SIMD's issue priority while it does, so
      // the other wave's dequant and loads fill the gaps instead of delaying them
      // (dense MLP 958 -> 1036 TFLOP/s)
      __builtin_amdgcn_s_setprio(3);
      mma(A, B, 0, W * NB);
      __builtin_amdgcn_s_setprio(0);
      // LDS reads and dequant first, then the MFMAs (the other wave of the SIMD
      // fills the gaps)
#pragma unroll
      for (int i = 0; i < NB; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 == SPS) {
        // vmcnt(5W) or vmcnt(2W); gfx9 encoding: vmcnt[3:0] (<= 10 here),
        // expcnt[6:4] = 7 (no wait), lgkmcnt[11:8] = 0
        constexpr int kVm = DEEP ? 5 * W : 2 * W;
        static_assert(kVm <= 15, "vmcnt field");
        __builtin_amdgcn_s_waitcnt(0x0070 | kVm);
        __syncthreads();
      }
    }
  };
  // Pairs of stages, then an odd last one.
  int st = 0;
  for (; st + 1 < nst; st += 2) {
    stage(0, 0, st);
    stage(1, 1, st + 1);
  }
  if (st < nst) stage(0, 0, st);
  __builtin_amdgcn_s_waitcnt(0);   // the last stage's reloads

  // ---- epilogue. 32x32 result layout: lane l holds column (row of the tile) l % 32
  // and weight rows 8*(j/4) + 4*(l/32) + j%4, j = 0..15.
  // fp16 form: the activation row was scaled by 2^p; the results are scaled back
  // here (exactly: a power of two). No row maxima of H are recorded: the down
  // projection after a prefill-tile gate/up is a prefill-tile one too (both take
  // K and N multiples of 256 and 32), and it reads H in bf16.
  const float act = a.act_scale ? *a.act_scale : 1.0f;   // W4A4: the activations' input_scale
  const float s2a0 = a.w0.scale_2[e] * act;
  const float s2b0 = kTwo ? a.w1.scale_2[e] * act : 0.0f;
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const int tok = 32 * t + r32;
    if (tok >= rows) continue;
    const int64_t p = rb + tok;
    float unscale = 1.0f;
    if constexpr (F16 && MODE == kGateUp) unscale = ldexpf(1.0f, -d.xexp[a.perm[p] / a.topk]);
    const float s2a = s2a0 * unscale, s2b = s2b0 * unscale;
#pragma unroll
    for (int g = 0; g < 4; ++g) {               // 4 groups of 4 consecutive weight rows
      float v0[4], v1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v0[j] = acc[0][t][4 * g + j];
        v1[j] = acc[W - 1][t][4 * g + j];
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
        for (int b = 0; b < W; ++b) {
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

// WB (one-weight modes): 32-row weight blocks per wave, 2 (512 weight rows per
// workgroup) or 1 (256, for grids that would not fill the chip otherwise).
template <int MODE, bool F16, int WB, bool TL>
__global__ __launch_bounds__(kThreads, 1) void gemm_prefill_kernel(GemmArgs a, F16Args d) {
  constexpr bool kMoe = (MODE == kGateUp || MODE == kDown);
  __shared__ __attribute__((aligned(16))) char xs[2 * XBUF];
  int e = 0, rb, rows, nblk;
  if (kMoe) {
    // Workgroups are dealt to the 8 XCDs round-robin by linear id. Remap so that
    // each XCD runs whole tiles (tile = 8*j + xcd), all n-blocks of a tile one
    // after another: the tile's activation rows stay in that XCD's L2 across its
    // n-blocks instead of being fetched again for each one.
    const int nby = (int)gridDim.y;
    const int64_t lin = (int64_t)blockIdx.x + (int64_t)gridDim.x * blockIdx.y;
    const int xcd = (int)(lin % 8);
    const int64_t j = lin / 8;
    const int64_t tile = (j / nby) * 8 + xcd;
    nblk = (int)(j % nby);
    if (tile >= *a.n_tiles) return;
    const int32_t* t = a.tiles + 4 * tile;
    e = t[0];
    rb = t[1];
    rows = t[2];
  } else {
    nblk = (int)blockIdx.y;
    rb = (int)blockIdx.x * MT;
    rows = (int)min((int64_t)MT, a.M - rb);
  }
  const int nb = (rows + 31) / 32;
  switch (nb) {
    case 1: prefill_body<MODE, 1, F16, WB, TL>(a, d, xs, e, rb, rows, nblk); break;
    case 2: prefill_body<MODE, 2, F16, WB, TL>(a, d, xs, e, rb, rows, nblk); break;
    case 3: prefill_body<MODE, 3, F16, WB, TL>(a, d, xs, e, rb, rows, nblk); break;
    default: prefill_body<MODE, 4, F16, WB, TL>(a, d, xs, e, rb, rows, nblk); break;
  }
}

// K: a multiple of 64 (the tiled layout, which these kernels also read, has
// K % 256 == 0 by its definition; row-major weights may end on a partial stage).
// A lane's 8 scale bytes are one 8-byte load, which needs the row pitch of the
// row-major scales, K/16 bytes, to be a multiple of 4.
bool prefill_supported(GemmMode mode, int64_t x_rows, int64_t K, int64_t N) {
  (void)mode;
  // 32-bit buffer ranges: x, and one expert's codes (its scales are smaller)
  const int64_t lim = (int64_t)1 << 31;
  return K % 64 == 0 && K >= 64 && N % 32 == 0 && x_rows * K * 2 < lim && N * (K / 2) < lim;
}

int cu_count() {
  // one cached count per device; threads that race on a first query store the same value
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int MODE, bool F16, int WB>
static void launch_pf(const GemmArgs& a, const F16Args& d, int64_t grid_tiles, hipStream_t s) {
  static_assert(WB == 1 || WB == 2, "weight blocks per wave");
  const bool two = (MODE == kGateUp || MODE == kGated);
  const int64_t nw = two ? 32 * kWaves : 32 * WB * kWaves;     // output columns per workgroup
  // routed modes: the grid holds ceil(tiles/8)*8 tiles' worth of workgroups (the
  // kernel maps them XCD by XCD); x * y is all that matters there
  const int64_t gt = (MODE == kGateUp || MODE == kDown) ? (grid_tiles + 7) / 8 * 8 : grid_tiles;
  const dim3 grid((unsigned)gt, (unsigned)((a.N + nw - 1) / nw));
  if (a.w0.tiled) hipLaunchKernelGGL((gemm_prefill_kernel<MODE, F16, WB, true>), grid, dim3(kThreads), 0, s, a, d);
  else hipLaunchKernelGGL((gemm_prefill_kernel<MODE, F16, WB, false>), grid, dim3(kThreads), 0, s, a, d);
}

int prefill_weight_blocks(GemmMode mode, int64_t N, int64_t grid_tiles) {
  if (mode == kGateUp || mode == kGated) return 2;   // 32 rows of each of the two weights per wave
  // one-weight modes: half-width workgroups when full-width ones would leave CUs idle
  return grid_tiles * ((N + 32 * 2 * kWaves - 1) / (32 * 2 * kWaves)) < 2 * (int64_t)cu_count() ? 1 : 2;
}

hipError_t launch_prefill(GemmMode mode, bool f16, const GemmArgs& a, const F16Args& d, int64_t grid_tiles,
                          hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  const bool narrow = prefill_weight_blocks(mode, a.N, grid_tiles) == 1;
  switch (mode) {
    case kGateUp:
      if (f16) launch_pf<kGateUp, true, 2>(a, d, grid_tiles, s);
      else launch_pf<kGateUp, false, 2>(a, d, grid_tiles, s);
      break;
    case kDown:
      if (f16) return hipErrorInvalidValue;   // the fp16 form is gate/up's only
      narrow ? launch_pf<kDown, false, 1>(a, d, grid_tiles, s) : launch_pf<kDown, false, 2>(a, d, grid_tiles, s);
      break;
    case kLinear:
      narrow ? launch_pf<kLinear, false, 1>(a, d, grid_tiles, s) : launch_pf<kLinear, false, 2>(a, d, grid_tiles, s);
      break;
    case kGated: launch_pf<kGated, false, 2>(a, d, grid_tiles, s); break;
  }
  return hipGetLastError();
}

}  // namespace nvfp4
