// Prefill-shaped grouped NVFP4 GEMM (tiles of up to 128 rows): matrix-core bound.
//
// Passage: TensorFold issue #308, "What the branch does" (routed experts in a
// grouped NVFP4 kernel on bf16 rows; the dense MLP on Fp4Linear with gate and
// up apart) and "Questions" item 4 (a prompt-shaped expert kernel whose sums
// do not depend on the chunking).
//
// Work decomposition. A workgroup (8 waves, two per SIMD) takes one tile of
// <= 128 rows of one expert and 256 or 512 weight rows; each wave owns W 32-row
// weight blocks (gate/up: one block of gate and the same 32 columns of up, so
// SiLU(gate)*up is formed in registers) against all rows of the tile.
// v_mfma_f32_32x32x16 with
//   A = weights, dequantized straight from HBM into registers: lane (r, h) of a
//       32-row block owns row r and the contiguous k range [kb + 128h, +128) of
//       every 256-k stage: four 128-bit code loads (pieces c of 32 k) and one
//       8-byte scale load;
//   B = activations, a [128 x 256k] tile in LDS shared by the 8 waves, streamed
//       in with direct-to-LDS buffer loads (no registers held while in flight),
//       double-buffered, one barrier per stage.
// MFMA step s (0..15) of a stage pairs k = kb + 8s (h = 0) with kb + 128 + 8s
// (h = 1). The number of 32-row tile blocks multiplied follows the tile's real
// row count (1..4, picked per tile), so small experts do not pay for padding rows.
// The two waves of a SIMD cover each other's waits (one wave per SIMD with twice
// the weight rows and the accumulators in the accumulation registers reads half
// the LDS operands per MFMA but ran slower).
//
// Schedule per wave, software-pipelined one MFMA step ahead: while the MFMAs of
// step s issue, the wave dequantizes the A operands of step s + 1 and, as soon as
// the last MFMA reading a B register has issued, reads that register's operand of
// step s + 1 from LDS. The loads of stage st + 1 go out during stage st: the
// activation loads in steps 0..8, the scales at step 0 (double-buffered), code
// piece c at step 4c + 3, after the dequant of step 4c + 3 read it (the code
// registers are single-buffered). Tiles of <= 64 rows keep two code sets and load
// weights two stages ahead.
//
// Epilogue: the routed down projection's fp32 partials and the two-weight modes'
// H go through LDS, so that every global store writes whole 128-byte lines.
//
// Summation order of an output element: stages in increasing k, within a stage
// MFMA steps s = 0..15, each over its 16 k. It depends only on K.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace prefill_detail {

constexpr int KC = 256;             // k per stage
constexpr int SPS = KC / 16;        // MFMA steps per stage
constexpr int MT = 128;             // max rows per tile
// Activation tile in LDS: rows of KC bf16 plus one 16-byte pad, so row r starts
// 33*r 16-byte units into the buffer and 16 consecutive rows hit 16 distinct
// bank groups at any common k; every read address is a per-lane base plus a
// compile-time offset.
constexpr int RSU = KC / 8 + 1;     // 16-byte units per tile row (data + pad)
constexpr int RSB = 16 * RSU;       // tile row stride in bytes
constexpr int NW = 8;               // waves per workgroup
constexpr int kThreads = 64 * NW;
constexpr int XI = ((MT * RSU + 63) / 64 + NW - 1) / NW * NW;  // 1 KB direct-to-LDS loads per stage
constexpr int XPW = XI / NW;        // of them per wave, one per step in steps 0..8
constexpr int XBUF = XI * 1024;     // bytes per buffer
static_assert(XPW <= 9, "activation loads per wave");

template <int SEL>
__device__ __forceinline__ float sc(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(w, SEL);
}

// MFMA operand type of the bf16 and fp16 forms
template <bool F16> struct Op { typedef bf16x8 T; };
template <> struct Op<true> { typedef f16x8 T; };

// s_waitcnt with vmcnt <= VM, lgkmcnt(0), expcnt not waited for (gfx9 encoding:
// vmcnt[3:0] in bits 3:0 and vmcnt[5:4] in bits 15:14, expcnt bits 6:4, lgkmcnt 11:8)
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | 0x0070);
}

}  // namespace prefill_detail

using namespace prefill_detail;

template <int MODE, int NB, bool F16, int WB, bool TL, bool RAG>
__device__ __forceinline__ void prefill_body(const GemmArgs& a, const F16Args& d, char* xs, int e, int rb,
                                             int rows, int nblk) {
  typedef typename Op<F16>::T AT;
  constexpr bool kTwo = (MODE == kGateUp || MODE == kGated);
  constexpr int W = kTwo ? 2 : WB;                // 32-row weight blocks per wave
  constexpr int CW = 32 * (kTwo ? W / 2 : W);     // output columns per wave
  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t N = a.N, K = a.K;

  // ---- weight rows of this lane: W 32-row blocks. The wave's output columns are
  // nbase .. nbase + CW; two-weight modes: block b < W/2 = gate rows nbase + 32b + r32,
  // block W/2 + b = the same up rows; one-weight modes: block b = rows nbase + 32b + r32.
  // Every load is a buffer load: a descriptor over one expert's codes / scales
  // (or over x) plus a 32-bit per-lane offset and a uniform stage offset.
  const int64_t nbase = (int64_t)nblk * (CW * NW) + CW * wave;
  __amdgpu_buffer_rsrc_t crs[W], srs[W];
  uint32_t co[W], so[W];
#pragma unroll
  for (int b = 0; b < W; ++b) {
    const int bc = kTwo ? b % (W / 2) : b;
    int64_t n = nbase + 32 * bc + r32;
    if (n > N - 1) n = N - 1;                 // rows past N: computed, never stored
    const WeightDev& w = (kTwo && b >= W / 2) ? a.w1 : a.w0;
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
  // tile's last row: their results are never stored. Wave w issues loads J = w + NW*i.
  const __amdgpu_buffer_rsrc_t xrs = rsrc(a.x, a.x_rows * K * 2);
  uint32_t xo[XPW];
#pragma unroll
  for (int i = 0; i < XPW; ++i) {
    const int u = 64 * (wave + NW * i) + lane;
    int r = u / RSU;
    int c = u % RSU;
    if (c == RSU - 1) c = 0;
    if (r > rows - 1) r = rows - 1;
    int64_t src;
    if (MODE == kGateUp) src = a.perm[rb + r] / a.topk;
    else src = rb + r;
    xo[i] = (uint32_t)(2 * (src * K + 8 * c));
  }
  // Only the loads that fill the NB 32-row blocks the MFMAs read fetch anything;
  // the others are issued with an offset beyond the descriptor's range (no memory
  // access) into units of the buffer no MFMA reads, which keeps the steps free of
  // branches. Row-major weights may have K % 256 != 0 (any multiple of 64: the
  // shards of a tensor-parallel split); then the last stage runs past K (RAG), and
  // its activation chunks past K are read the same way as zeros, so the weights
  // read there (the next row's finite bytes, or zeros past the tensor) multiply
  // zeros. Chunk of load i: (64 (wave + NW i) + lane) mod RSU, the pad read as 0.
  constexpr int XN = (32 * NB * RSU + 63) / 64;
  const int cbase = (64 * wave + lane) % RSU;
  auto issue_x = [&](int kb, int buf, int i0, int i1) {
#pragma unroll
    for (int i = 0; i < XPW; ++i) {
      if (i < i0 || i >= i1) continue;
      uint32_t off = (wave + NW * i < XN) ? xo[i] : 0x80000000u;
      if constexpr (RAG) {
        int c = cbase + (64 * NW * i) % RSU;
        if (c >= RSU) c -= RSU;
        if (c == RSU - 1) c = 0;
        if (kb + 8 * c >= K) off = 0x80000000u;
      }
      auto* dst = (__attribute__((address_space(3))) void*)(xs + buf * XBUF + 1024 * (wave + NW * i));
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
  // B operand of MFMA step s for tile block t: tile row 32t + r32, 16-byte unit 16h + s
  const char* const xrd = xs + r32 * RSB + 256 * h;
  auto read_b = [&](int buf, int s, int t) {
    return *reinterpret_cast<const AT*>(xrd + buf * XBUF + t * 32 * RSB + 16 * s);
  };

  // ---- pipeline. Stage st reads LDS buffer st % 2 and scale set st % 2 (DEEP:
  // code set st % 2). At its last step the wave waits for its activation loads of
  // stage st + 1 (only the code and scale loads issued after the last activation
  // load may still be in flight: 2W of them, 5W with DEEP), then a barrier makes
  // tile st + 1 complete everywhere and frees buffer st % 2. The last stage
  // reloads itself (never read), which keeps the steps free of branches.
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
  prep_a(0, 0, A);

  // VALU instructions of the next step's dequant placed after each tile block's
  // MFMAs (about 9 per A operand in fp16, 19 in bf16; the bf16 groups are kept
  // a little smaller, which measured 2% faster on the dense gated GEMM)
  constexpr int PV = (W * (F16 ? 9 : 15) + NB - 1) / NB;
  auto stage = [&](int set, int buf, int st) {
    const int kn = (st + 1 < nst ? st + 1 : st) * KC;
    const int kn2 = (st + 2 < nst ? st + 2 : nst - 1) * KC;
#pragma unroll
    for (int t = 0; t < NB; ++t) B[t] = read_b(buf, 0, t);
#pragma unroll
    for (int s = 0; s < SPS; ++s) {
      if (s <= 8) issue_x(kn, buf ^ 1, s, s + 1);
      if (!DEEP && s == 0) load_scales(set ^ 1, kn);
      if constexpr (DEEP) {
        if (s >= 9 && s <= 11) load_codes(set, s - 9, kn2);
        if (s == 15) {
          load_codes(set, 3, kn2);
          load_scales(set, kn2);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // the wave issuing its MFMAs takes the SIMD's issue priority while it does
      __builtin_amdgcn_s_setprio(3);
      AT An[W];
      if (s + 1 < SPS) prep_a(set, s + 1, An);
      else prep_a(set ^ 1, 0, An);      // the next stage's first step: its scale set (DEEP: its code set)
#pragma unroll
      for (int t = 0; t < NB; ++t) {
#pragma unroll
        for (int b = 0; b < W; ++b) {
          if constexpr (F16) acc[b][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[b], B[t], acc[b][t], 0, 0, 0);
          else acc[b][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[b], B[t], acc[b][t], 0, 0, 0);
        }
        if (s + 1 < SPS) B[t] = read_b(buf, s + 1, t);
      }
      if constexpr (!DEEP) {
        if (s % 4 == 3) load_codes(0, s / 4, kn);   // piece s/4: its last reader was the dequant of step s
      }
      // per tile block: its W MFMAs, the LDS read of its next operand, a share of the dequant
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, W, 0);
        if (s + 1 < SPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, PV, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int b = 0; b < W; ++b) A[b] = An[b];
      if (s + 1 == SPS) {
        wait_vm_lgkm0<DEEP ? 5 * W : 2 * W>();
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
  // Routed down and the two-weight modes: the results go through LDS (the stage
  // buffers are free once every wave has passed the barrier below), so that each
  // global store instruction writes whole 128-byte lines instead of 16- or 32-byte
  // pieces of 32 rows. Same values, same bits.
  if constexpr (MODE == kDown) {
    __syncthreads();
    constexpr int CWv = 32 * W;                 // output columns of this wave
    constexpr int PITCH = CWv + 4;              // floats per LDS row
    static_assert(NW * 64 * PITCH * 4 <= 2 * XBUF, "partials tile");
    float* lds = reinterpret_cast<float*>(xs) + wave * (64 * PITCH);
    constexpr int LPR = CWv / 4, RPI = 64 / LPR;   // lanes per row, rows per store instruction
#pragma unroll
    for (int half = 0; half < (NB + 1) / 2; ++half) {   // 64 tile rows at a time
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int t = 2 * half + tt;
        if (t >= NB) break;
#pragma unroll
        for (int b = 0; b < W; ++b)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16& vv = acc[b][t];
            *reinterpret_cast<f32x4*>(lds + (32 * tt + r32) * PITCH + 32 * b + 8 * g + 4 * h) =
                f32x4{s2a0 * vv[4 * g], s2a0 * vv[4 * g + 1], s2a0 * vv[4 * g + 2], s2a0 * vv[4 * g + 3]};
          }
      }
      wait_vm_lgkm0<63>();   // this wave's LDS writes are done (its own area: no barrier)
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < 64 / RPI; ++i) {
        const int rl = i * RPI + lane / LPR, ch = lane % LPR;
        const int tok = 64 * half + rl;
        const f32x4 v = *reinterpret_cast<const f32x4*>(lds + rl * PITCH + 4 * ch);
        const int64_t n = nbase + 4 * ch;
        if (tok < rows && n < N)   // the partials are read once, by the combine: stream them past the caches
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) +
                                                                 (int64_t)a.perm[rb + tok] * N + n));
      }
      wait_vm_lgkm0<63>();
      __builtin_amdgcn_wave_barrier();
    }
    return;
  }
  if constexpr (kTwo) {
    constexpr int HP = CW * NW + 8;   // LDS row pitch (bf16) of the workgroup's [MT][CW * NW] H tile
    static_assert(MT * HP * 2 <= 2 * XBUF, "H tile");
    __syncthreads();
    uint16_t* ht = reinterpret_cast<uint16_t*>(xs);
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const int tok = 32 * t + r32;
      float unscale = 1.0f;
      if constexpr (F16 && MODE == kGateUp) unscale = ldexpf(1.0f, -d.xexp[a.perm[rb + min(tok, rows - 1)] / a.topk]);
      const float s2a = s2a0 * unscale, s2b = s2b0 * unscale;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int off = 8 * g + 4 * h;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = silu(s2a * acc[0][t][4 * g + q]) * (s2b * acc[1][t][4 * g + q]);
        u32x2 o;
        o[0] = pack_bf16x2(v[0], v[1]);
        o[1] = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<u32x2*>(ht + tok * HP + CW * wave + off) = o;
      }
    }
    __syncthreads();
    const int64_t ncol0 = (int64_t)nblk * (CW * NW);
    constexpr int RPW = MT / NW;   // tile rows stored by each wave, two per instruction
#pragma unroll
    for (int i = 0; i < RPW / 2; ++i) {
      const int row = RPW * wave + 2 * i + (lane >> 5), ch = lane & 31;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ht + row * HP + 8 * ch);
      if (row < rows && ncol0 + 8 * ch < N)
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + (rb + row) * N + ncol0 + 8 * ch) = v;
    }
    return;
  }
  // the dense one-weight product: bf16 rows straight from the accumulators
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const int tok = 32 * t + r32;
    if (tok >= rows) continue;
    const int64_t p = rb + tok;
#pragma unroll
    for (int g = 0; g < 4; ++g) {               // 4 groups of 4 consecutive weight rows
      const int off = 8 * g + 4 * h;            // weight row within the 32-row block
#pragma unroll
      for (int b = 0; b < W; ++b) {
        const int64_t n = nbase + 32 * b + off;
        if (n >= N) continue;
        const f32x16& vv = acc[b][t];
        u32x2 o;
        o[0] = pack_bf16x2(s2a0 * vv[4 * g], s2a0 * vv[4 * g + 1]);
        o[1] = pack_bf16x2(s2a0 * vv[4 * g + 2], s2a0 * vv[4 * g + 3]);
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + p * N + n) = o;
      }
    }
  }
}

// WB (one-weight modes): 32-row weight blocks per wave, 2 (512 weight rows per
// workgroup) or 1 (256, for grids that would not fill the chip otherwise).
// Two-weight modes: 256 columns of each weight per workgroup.
template <int MODE, bool F16, int WB, bool TL, bool RAG>
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
    case 1: prefill_body<MODE, 1, F16, WB, TL, RAG>(a, d, xs, e, rb, rows, nblk); break;
    case 2: prefill_body<MODE, 2, F16, WB, TL, RAG>(a, d, xs, e, rb, rows, nblk); break;
    case 3: prefill_body<MODE, 3, F16, WB, TL, RAG>(a, d, xs, e, rb, rows, nblk); break;
    default: prefill_body<MODE, 4, F16, WB, TL, RAG>(a, d, xs, e, rb, rows, nblk); break;
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
  const int64_t nw = two ? 256 : 256 * WB;     // output columns per workgroup
  // routed modes: the grid holds ceil(tiles/8)*8 tiles' worth of workgroups (the
  // kernel maps them XCD by XCD); x * y is all that matters there
  const int64_t gt = (MODE == kGateUp || MODE == kDown) ? (grid_tiles + 7) / 8 * 8 : grid_tiles;
  const dim3 grid((unsigned)gt, (unsigned)((a.N + nw - 1) / nw));
  const dim3 blk(kThreads);
  const bool rag = a.K % KC != 0;
  if (a.w0.tiled) hipLaunchKernelGGL((gemm_prefill_kernel<MODE, F16, WB, true, false>), grid, blk, 0, s, a, d);
  else if (!rag) hipLaunchKernelGGL((gemm_prefill_kernel<MODE, F16, WB, false, false>), grid, blk, 0, s, a, d);
  else hipLaunchKernelGGL((gemm_prefill_kernel<MODE, F16, WB, false, true>), grid, blk, 0, s, a, d);
}

int prefill_weight_blocks(GemmMode mode, int64_t N, int64_t grid_tiles) {
  if (mode == kGateUp || mode == kGated) return 2;   // 256 columns of each of the two weights per workgroup
  // one-weight modes: half-width workgroups when full-width ones would leave CUs idle
  return grid_tiles * ((N + 511) / 512) < 2 * (int64_t)cu_count() ? 1 : 2;
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
