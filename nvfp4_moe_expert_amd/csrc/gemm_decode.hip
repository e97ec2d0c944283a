// Decode-shaped grouped NVFP4 GEMM (tiles of at most 16 rows): a weight stream.
//
// Passage: TensorFold issue #308, "What the branch does" - the routed experts
// run in one grouped NVFP4 kernel that accepts bf16 activations and nothing
// else, with each expert's weight_scale_2 applied to its product. In decode an expert sees one or two rows, so every weight byte is
// used for one 16x16 MFMA tile and the kernel is bound by HBM bandwidth.
//
// Layout of the work (measured on MI355X):
// * A workgroup = 4 waves = 64 output columns of one tile (for gate/up, the same
//   16 columns of both weights per wave). Lane (r, q) of a wave owns weight row
//   n0 + r and, in every 128*U-k stage, the contiguous k range
//   [kb + 32Uq, kb + 32Uq + 32U): U 128-bit code loads of its own row and ONE
//   2U-byte load of its block scales. (Loading the scales two bytes at a time
//   makes half the memory instructions carry 1/64 of the bytes and caps the
//   stream near 4.8 TB/s; with wide loads it reaches ~5.6 TB/s.)
// * Stage i+1's weights load into registers while stage i is multiplied; the
//   register sets ping-pong (the stage loop is unrolled by two).
// * Codes are dequantized in registers. In the fp16 form one packed convert
//   turns two e2m1 codes into fp16 and one packed multiply applies the e4m3
//   scale: 1 VALU op per weight, exact (code*scale has <= 6 significant bits and
//   lies in [2^-10, 2688]). The activations are then fp16 too, pre-scaled per
//   row by a power of two 2^p so the row maximum sits in [2^14, 2^15): every
//   bf16 value down to 2^-28 of its row maximum is exact in fp16, every product
//   is exact in the fp32 accumulator, and 2^-p is applied in the epilogue. The
//   bf16 form (2 VALU ops per weight) is used where no pre-scaled rows exist.
// * Activations are staged through LDS (double-buffered, one barrier per stage).
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace decode_detail {

constexpr int kThreads = 256;

// threadIdx.x through an opaque move: in the persistent loop this keeps the
// compiler from hoisting every per-thread index out of the loop and holding it in
// registers across the whole item body (it costs one VALU op per item).
__device__ __forceinline__ int opaque_tid() {
  int t = (int)threadIdx.x;
  asm volatile("; opaque" : "+v"(t));
  __builtin_assume(t >= 0 && t < kThreads);
  return t;
}
constexpr int kBlockN = 64;

template <int SEL>
__device__ __forceinline__ float scale_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(w, SEL);
}

// weight registers of one stage for one weight: U code chunks, 2U scale bytes
template <int U>
struct Stage {
  u32x4 c[U];
  uint32_t s[(U + 1) / 2];
};

// Stage offsets of a lane's codes and scales: row-major rows advance kb/2 and
// kb/16 bytes per kb inputs with 16-byte code chunks side by side; in the tiled
// layout (blocks of 32 rows) a 32-input chunk is 512 bytes on, and 256 inputs of
// scales are 512 bytes on (2*kb bytes per kb inputs).
// Tiled codes are read with non-temporal loads (each 128-byte line is read once,
// whole, by one instruction); row-major codes with ordinary ones: there a line is
// split over several instructions, and without the cache's copy each of them
// fetches it again.
// ok == false (only with U == 1: the lane's 32 inputs lie past K in the last stage
// of a K that is an odd multiple of 64): no load is issued and the codes and scale
// bytes read as zero, so the lane's products are exact zeros.
template <int U, bool TL>
__device__ __forceinline__ void load_codes(Stage<U>& st, const uint8_t* codes, int64_t kb, bool ok = true) {
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const uint8_t* p = codes + (TL ? 16 * kb : kb / 2) + (TL ? 512 : 16) * i;
    st.c[i] = !ok ? u32x4{0, 0, 0, 0} : TL ? ld16_nt(p) : ld16(p);
  }
}

template <int U, bool TL>
__device__ __forceinline__ void load_stage(Stage<U>& st, const uint8_t* codes, const uint8_t* scales, int64_t kb,
                                           bool ok = true) {
  load_codes<U, TL>(st, codes, kb, ok);
  const uint8_t* sp = scales + (TL ? 2 * kb : kb / 16);
  if constexpr (U == 4) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(sp);
    st.s[0] = v[0];
    st.s[1] = v[1];
  } else if constexpr (U == 2) {
    st.s[0] = *reinterpret_cast<const uint32_t*>(sp);
  } else {
    st.s[0] = ok ? *reinterpret_cast<const uint16_t*>(sp) : 0u;
  }
}

}  // namespace decode_detail

using namespace decode_detail;

// NS > 0: K has at most NS stages, and every lane loads the scale bytes of all of
// them up front. A row's 128-byte line of scales then is requested once, by its 4
// lanes together; loaded a stage at a time, the same line is asked for over four
// stages and a part of those requests misses again (13% more bytes fetched).
// One work item: tile `tile` (16 rows) x 64-row block `by` of the weights.
template <int MODE, int U, bool F16, int NS, bool TL>
__device__ __forceinline__ void decode_item(const GemmArgs& a, const F16Args& d,
                                            uint16_t (&xs)[2][16][128 * U + 8], int tile, int by) {
  constexpr bool kTwo = (MODE == kGateUp || MODE == kGated);
  constexpr bool kMoe = (MODE == kGateUp || MODE == kDown);
  constexpr int KC = 128 * U;          // k per stage
  constexpr int LW = KC + 8;           // LDS row pitch (16-byte pad)

  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6, lr = lane & 15, q = lane >> 4;
  const int64_t N = a.N, K = a.K;

  int e = 0, rb, rows;
  if (kMoe) {
    const int32_t* t = a.tiles + 4 * (int64_t)tile;
    e = t[0];
    rb = t[1];
    rows = t[2];
  } else {
    rb = tile * 16;
    rows = (int)min((int64_t)16, a.M - rb);
  }

  const int64_t nrow = (int64_t)by * kBlockN + wave * 16 + lr;   // N % 64 == 0
  const int64_t wrow = (int64_t)e * N + nrow;
  // lane (lr, q): row nrow, inputs [kb + 32Uq, +32U) of each stage
  int64_t coff, soff;
  if constexpr (TL) {
    const int64_t R = nrow / 32, r = nrow % 32;
    coff = (int64_t)e * N * (K / 2) + (R * (K / 32) + U * q) * 512 + r * 16;
    soff = (int64_t)e * N * (K / 16) + (R * (K / 256) + (2 * U * q) / 16) * 512 + r * 16 + (2 * U * q) % 16;
  } else {
    coff = wrow * (K / 2) + 16 * U * q;
    soff = wrow * (K / 16) + 2 * U * q;
  }
  const uint8_t* c0 = a.w0.codes + coff;
  const uint8_t* s0 = a.w0.scales + soff;
  const uint8_t* c1 = kTwo ? a.w1.codes + coff : nullptr;
  const uint8_t* s1 = kTwo ? a.w1.scales + soff : nullptr;
  constexpr int64_t SSTEP = TL ? 2 * KC : KC / 16;   // scale bytes from one stage to the next
  // U == 1 takes K in multiples of 64: when K % 128 == 64 the lanes q = 2, 3 of the
  // last stage hold no inputs (their weights and activations are zeros)
  auto kok = [&](int64_t kb) { return U != 1 || kb + 32 * U * q < K; };

  // activation chunks of this thread: U per stage, chunk i = row xr[i], 8 k at 8*xc[i]
  const uint16_t* xsrc[U];
  int xr[U], xc[U];
  float xscale[U];                   // down, fp16 form: 2^p of the H row
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int idx = i * kThreads + tid;
    xr[i] = idx / (16 * U);
    xc[i] = idx % (16 * U);
    xsrc[i] = nullptr;
    xscale[i] = 1.0f;
    if (xr[i] < rows) {
      const int p = rb + xr[i];
      int64_t src;
      if (MODE == kGateUp) src = a.perm[p] / a.topk;
      else src = p;
      const uint16_t* base = (MODE == kGateUp && F16) ? d.x16 : a.x;
      xsrc[i] = base + src * K + 8 * xc[i];
      if (MODE == kDown && F16) xscale[i] = ldexpf(1.0f, row_exponent(d.hmax[p]));
    }
  }
  for (int i = tid; i < 2 * 16 * (LW / 8); i += kThreads) {
    const int b = i / (16 * (LW / 8)), rem = i % (16 * (LW / 8));
    const int r = rem / (LW / 8), c = rem % (LW / 8);
    if (r >= rows) st16(&xs[b][r][c * 8], u32x4{0, 0, 0, 0});
  }
  auto ldx = [&](u32x4 (&v)[U], int64_t kb) {
#pragma unroll
    for (int i = 0; i < U; ++i)
      v[i] = (xsrc[i] && (U != 1 || kb + 8 * xc[i] < K)) ? ld16(xsrc[i] + kb) : u32x4{0, 0, 0, 0};
  };
  auto stx = [&](u32x4 (&v)[U], int b) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      if (xr[i] >= rows) continue;
      u32x4 o = v[i];
      if constexpr (MODE == kDown && F16) {
        // bf16 H row -> fp16 scaled by 2^p (exact for every value >= 2^-28 of the row max)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f16x2 h2 = {(_Float16)(bf16_lo(v[i][j]) * xscale[i]), (_Float16)(bf16_hi(v[i][j]) * xscale[i])};
          o[j] = __builtin_bit_cast(uint32_t, h2);
        }
      }
      st16(&xs[b][xr[i]][8 * xc[i]], o);
    }
  };

  f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  // scale dwords of one stage for this lane: (U + 1) / 2
  constexpr int SW = (U + 1) / 2;
  auto compute_s = [&](const Stage<U>& g, const Stage<U>& u, const uint32_t (&gsw)[SW], const uint32_t (&usw)[SW],
                       int b) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const uint32_t gw = gsw[i / 2] >> (16 * (i & 1));
      const uint32_t uw = kTwo ? (usw[i / 2] >> (16 * (i & 1))) : 0u;
      if constexpr (F16) {
        const f16x2 sg = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(gw, 1.0f, false);
        f16x2 su = {};
        if constexpr (kTwo) su = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(uw, 1.0f, false);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const f16x8 B = *reinterpret_cast<const f16x8*>(&xs[b][lr][32 * U * q + 32 * i + 8 * s]);
          const f16x2 gs = (s < 2) ? f16x2{sg[0], sg[0]} : f16x2{sg[1], sg[1]};
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant8_f16(g.c[i][s], gs), B, acc0, 0, 0, 0);
          if constexpr (kTwo) {
            const f16x2 us = (s < 2) ? f16x2{su[0], su[0]} : f16x2{su[1], su[1]};
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant8_f16(u.c[i][s], us), B, acc1, 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 B = *reinterpret_cast<const bf16x8*>(&xs[b][lr][32 * U * q + 32 * i + 8 * s]);
          const float gs = (s < 2) ? scale_f32<0>(gw) : scale_f32<1>(gw);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(g.c[i][s], gs), B, acc0, 0, 0, 0);
          if constexpr (kTwo) {
            const float us = (s < 2) ? scale_f32<0>(uw) : scale_f32<1>(uw);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(u.c[i][s], us), B, acc1, 0, 0, 0);
          }
        }
      }
    }
  };

  auto compute = [&](const Stage<U>& g, const Stage<U>& u, int b) {
    uint32_t gsw[SW], usw[SW];
#pragma unroll
    for (int j = 0; j < SW; ++j) {
      gsw[j] = g.s[j];
      usw[j] = kTwo ? u.s[j] : 0u;
    }
    compute_s(g, u, gsw, usw, b);
  };

  const int nst = (int)((K + KC - 1) / KC);
  if constexpr (NS > 0) {
    // all stage scales up front (scale bytes of stage st at s + st*KC/16), then the
    // stages fully unrolled so every register index is static
    uint32_t gs_all[NS][SW], us_all[NS][SW];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      if (st < nst) {
        if constexpr (SW == 2) {
          const u32x2 v = *reinterpret_cast<const u32x2*>(s0 + st * SSTEP);
          gs_all[st][0] = v[0];
          gs_all[st][1] = v[1];
          if constexpr (kTwo) {
            const u32x2 w = *reinterpret_cast<const u32x2*>(s1 + st * SSTEP);
            us_all[st][0] = w[0];
            us_all[st][1] = w[1];
          }
        } else if constexpr (U == 2) {
          gs_all[st][0] = *reinterpret_cast<const uint32_t*>(s0 + st * SSTEP);
          if constexpr (kTwo) us_all[st][0] = *reinterpret_cast<const uint32_t*>(s1 + st * SSTEP);
        } else {   // U == 1: two scale bytes per lane and stage
          const bool ok = kok((int64_t)st * KC);
          gs_all[st][0] = ok ? *reinterpret_cast<const uint16_t*>(s0 + st * SSTEP) : 0u;
          if constexpr (kTwo) us_all[st][0] = ok ? *reinterpret_cast<const uint16_t*>(s1 + st * SSTEP) : 0u;
        }
      }
      if constexpr (!kTwo) {
#pragma unroll
        for (int j = 0; j < SW; ++j) us_all[st][j] = 0u;
      }
    }
    Stage<U> Cg[2], Cu[2];
    u32x4 xv[U];
    load_codes<U, TL>(Cg[0], c0, 0, kok(0));
    if constexpr (kTwo) load_codes<U, TL>(Cu[0], c1, 0, kok(0));
    ldx(xv, 0);
    stx(xv, 0);
    __syncthreads();
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      if (st >= nst) break;
      const int b = st & 1;
      const bool more = st + 1 < nst;
      if (more) {
        const bool ok = kok((int64_t)(st + 1) * KC);
        load_codes<U, TL>(Cg[b ^ 1], c0, (int64_t)(st + 1) * KC, ok);
        if constexpr (kTwo) load_codes<U, TL>(Cu[b ^ 1], c1, (int64_t)(st + 1) * KC, ok);
        ldx(xv, (int64_t)(st + 1) * KC);
      }
      compute_s(Cg[b], Cu[b], gs_all[st], us_all[st], b);
      if (more) stx(xv, b ^ 1);
      __syncthreads();
    }
  } else {
  Stage<U> Ag, Au, Bg, Bu;
  u32x4 xv[U];
  load_stage<U, TL>(Ag, c0, s0, 0, kok(0));
  if constexpr (kTwo) load_stage<U, TL>(Au, c1, s1, 0, kok(0));
  ldx(xv, 0);
  stx(xv, 0);
  __syncthreads();
  int st = 0;
  for (; st + 2 <= nst; st += 2) {
    const int64_t k1 = (int64_t)(st + 1) * KC, k2 = (int64_t)(st + 2) * KC;
    load_stage<U, TL>(Bg, c0, s0, k1, kok(k1));
    if constexpr (kTwo) load_stage<U, TL>(Bu, c1, s1, k1, kok(k1));
    ldx(xv, k1);
    compute(Ag, Au, 0);
    stx(xv, 1);
    __syncthreads();
    const bool more = st + 2 < nst;
    if (more) {
      load_stage<U, TL>(Ag, c0, s0, k2, kok(k2));
      if constexpr (kTwo) load_stage<U, TL>(Au, c1, s1, k2, kok(k2));
      ldx(xv, k2);
    }
    compute(Bg, Bu, 1);
    if (more) stx(xv, 0);
    __syncthreads();
  }
  if (st < nst) compute(Ag, Au, 0);
  }

  // ---- epilogue: lane holds D[n = nbase + 4q + r][token lr], r = 0..3
  if (lr >= rows) return;
  const int64_t p = rb + lr;
  const int64_t n0 = (int64_t)by * kBlockN + wave * 16 + 4 * q;
  float unscale = 1.0f;
  if constexpr (F16 && MODE == kGateUp) unscale = ldexpf(1.0f, -d.xexp[a.perm[p] / a.topk]);
  if constexpr (F16 && MODE == kDown) unscale = ldexpf(1.0f, -row_exponent(d.hmax[p]));
  if (a.act_scale) unscale *= *a.act_scale;   // W4A4: the activations' input_scale
  const float s2a = a.w0.scale_2[e] * unscale;
  const float s2b = kTwo ? a.w1.scale_2[e] * unscale : 0.0f;
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if constexpr (kTwo) v[r] = silu(s2a * acc0[r]) * (s2b * acc1[r]);
    else v[r] = s2a * acc0[r];
  }
  if constexpr (MODE == kDown) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + (int64_t)a.perm[p] * N + n0) =
        f32x4{v[0], v[1], v[2], v[3]};
  } else {
    u32x2 o;
    o[0] = pack_bf16x2(v[0], v[1]);
    o[1] = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + p * N + n0) = o;
    if constexpr (MODE == kGateUp && F16) {
      // row maximum of |H| as stored (bf16) for the down projection's scaling;
      // max is order-independent, so the atomics keep the result deterministic
      float m = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf((float)(__bf16)v[r]));
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      if (q == 0) atomicMax(reinterpret_cast<unsigned int*>(d.hmax + p), __builtin_bit_cast(unsigned int, m));
    }
  }
}

// PER: persistent routed form. The grid holds as many workgroups as fit on the
// device at once, and workgroup w takes items w, w + grid, ... of the n_tiles x
// N/64 items (all of the same size), so every workgroup streams the same number
// of bytes and they end together (one-shot workgroups of the short down
// projection leave a tail in which too few are live to keep HBM busy).
template <int MODE, int U, bool F16, int NS, bool TL, bool PER>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(PER ? 3 : 1))) void gemm_decode_kernel(
    GemmArgs a, F16Args d) {
  constexpr bool kMoe = (MODE == kGateUp || MODE == kDown);
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][16][128 * U + 8];
  if constexpr (PER) {
    static_assert(kMoe, "persistent form is for the routed modes");
    const int nby = (int)(a.N / kBlockN);
    const int total = *a.n_tiles * nby;   // <= grid_tiles * nby < 2^31 (host)
    for (int it = blockIdx.x; it < total; it += gridDim.x) {
      __syncthreads();   // the previous item's last LDS reads are done
      decode_item<MODE, U, F16, NS, TL>(a, d, xs, it / nby, it % nby);
    }
  } else {
    if (kMoe && (int)blockIdx.x >= *a.n_tiles) return;
    decode_item<MODE, U, F16, NS, TL>(a, d, xs, (int)blockIdx.x, (int)blockIdx.y);
  }
}

// Routed down projection (fp16 form) with K <= 2048 (K = I): the whole
// activation tile (<= 16 rows x K) is staged in LDS once, and each wave then
// streams NB consecutive 64-row blocks of weights (its 16 rows of each) with the
// code loads LA stages ahead. No barrier after the staging, one prologue for NB
// blocks: with the per-stage tile (K / 512 = 3 stages for K = 1536) the short
// workgroups spent a large part of their life filling the pipeline.
template <int MODE, bool F16, int NST, int NB, bool TL>
__device__ __forceinline__ void res_item(const GemmArgs& a, const F16Args& d, uint16_t (&xs)[16][NST * 512 + 8],
                                         int tile, int by) {
  static_assert(MODE == kDown || MODE == kLinear, "one-weight modes");
  constexpr bool kMoe = (MODE == kDown);
  constexpr int U = 4, KC = 128 * U, KT = NST * KC;
  constexpr int G = NB * NST;   // stages of a wave's stream
  constexpr int LA = 2;         // stages in flight ahead of the one multiplied
  constexpr int XU = 16 * (KT / 8) / kThreads;   // 16-byte activation units per thread

  const int tid = opaque_tid(), lane = tid & 63, wave = tid >> 6, lr = lane & 15, q = lane >> 4;
  const int64_t N = a.N;

  // The item's own loads are issued in the order they are needed and none sits
  // behind a branch, so no wait covers more than it must: the tile entry, then
  // the activation tile, each lane's row maximum and output row, then the
  // weights. (An item used to end its prologue on a chain of dependent loads: the
  // tile entry, then the weights, then one staging load after another, then the
  // epilogue's row maximum and output row.)
  int e = 0, rb, rows;
  if (kMoe) {
    const int32_t* t = a.tiles + 4 * (int64_t)__builtin_amdgcn_readfirstlane(tile);
    e = t[0];
    rb = t[1];
    rows = t[2];
  } else {
    rb = tile * 16;
    rows = (int)min((int64_t)16, a.M - rb);
  }
  // the activation tile first: it comes from the cache (the previous kernel wrote
  // it) and is converted and staged while the weights are still on their way
  const __amdgpu_buffer_rsrc_t xrs = rsrc(a.x, a.x_rows * KT * 2);
  u32x4 hv[XU];
#pragma unroll
  for (int i = 0; i < XU; ++i) {
    const int u = i * kThreads + tid, r = u / (KT / 8), c = u % (KT / 8);
    const uint32_t off = r < rows ? (uint32_t)((rb + r) * (KT * 2) + 16 * c) : 0x80000000u;
    hv[i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
  }
  const bool live = lr < rows;
  const int64_t p = rb + lr;
  const int64_t pc = rb + min(lr, rows - 1);   // a valid row for every lane
  uint32_t hm = 0;
  if constexpr (F16) hm = d.hmax[pc];
  const int32_t orow_v = kMoe ? a.perm[pc] : 0;
  const float s2e = a.w0.scale_2[e];
  const float act = a.act_scale ? *a.act_scale : 1.0f;   // W4A4: the activations' input_scale

  // block j of this wave: rows nrow + 64j; in both layouts 64 rows are 32*K code
  // bytes and 4*K scale bytes further on
  const int64_t nrow = (int64_t)by * (kBlockN * NB) + wave * 16 + lr;
  int64_t coff, soff;
  if constexpr (TL) {
    const int64_t R = nrow / 32, r = nrow % 32;
    coff = (int64_t)e * N * (KT / 2) + (R * (KT / 32) + U * q) * 512 + r * 16;
    soff = (int64_t)e * N * (KT / 16) + (R * (KT / 256) + (2 * U * q) / 16) * 512 + r * 16 + (2 * U * q) % 16;
  } else {
    const int64_t wrow = (int64_t)e * N + nrow;
    coff = wrow * (KT / 2) + 16 * U * q;
    soff = wrow * (KT / 16) + 2 * U * q;
  }
  const uint8_t* c0 = a.w0.codes + coff;
  const uint8_t* s0 = a.w0.scales + soff;
  constexpr int64_t SSTEP = TL ? 2 * KC : KC / 16;
  auto cptr = [&](int g) { return c0 + (int64_t)(g / NST) * 32 * KT; };
  auto kofs = [&](int g) { return (int64_t)(g % NST) * KC; };

  Stage<U> C[LA + 1];
#pragma unroll
  for (int g = 0; g < LA && g < G; ++g) load_codes<U, TL>(C[g], cptr(g), kofs(g));
  u32x2 sc[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    sc[g] = *reinterpret_cast<const u32x2*>(s0 + (int64_t)(g / NST) * 4 * KT + (g % NST) * SSTEP);
  // nothing below may be scheduled above the weight loads (the conversion's first
  // use of a row maximum would make them wait for it)
  __builtin_amdgcn_sched_barrier(0);

  // ---- the activation tile, converted to fp16 * 2^p per row in the fp16 form
  // (units of rows past the tile's read zeros without a memory access)
  {
#pragma unroll
    for (int i = 0; i < XU; ++i) {
      const int u = i * kThreads + tid, r = u / (KT / 8), c = u % (KT / 8);
      u32x4 o = hv[i];
      if constexpr (F16) {
        // row r's maximum sits in lane r (r is the same across the wave: KT / 8 is a multiple of 64)
        const float hs = ldexpf(1.0f, row_exponent(__builtin_amdgcn_readlane(hm, __builtin_amdgcn_readfirstlane(r & 15))));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f16x2 h2 = {(_Float16)(bf16_lo(hv[i][j]) * hs), (_Float16)(bf16_hi(hv[i][j]) * hs)};
          o[j] = __builtin_bit_cast(uint32_t, h2);
        }
      }
      st16(&xs[r][8 * c], o);
    }
  }
  __syncthreads();

  float s2 = s2e;
  if constexpr (F16) {
    if (live) s2 *= ldexpf(1.0f, -row_exponent(hm));
  }
  if (a.act_scale) s2 *= act;
  const int64_t orow = kMoe ? (live ? (int64_t)orow_v : 0) : p;

  f32x4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g + LA < G) load_codes<U, TL>(C[(g + LA) % (LA + 1)], cptr(g + LA), kofs(g + LA));
    const Stage<U>& cs = C[g % (LA + 1)];
    const int kb = (g % NST) * KC;
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const uint32_t sw = sc[g][i / 2] >> (16 * (i & 1));
      if constexpr (F16) {
        const f16x2 sf = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const f16x8 B = *reinterpret_cast<const f16x8*>(&xs[lr][kb + 32 * U * q + 32 * i + 8 * s]);
          const f16x2 gs = (s < 2) ? f16x2{sf[0], sf[0]} : f16x2{sf[1], sf[1]};
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant8_f16(cs.c[i][s], gs), B, acc, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 B = *reinterpret_cast<const bf16x8*>(&xs[lr][kb + 32 * U * q + 32 * i + 8 * s]);
          const float gs = (s < 2) ? scale_f32<0>(sw) : scale_f32<1>(sw);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(cs.c[i][s], gs), B, acc, 0, 0, 0);
        }
      }
    }
    if (g % NST == NST - 1) {
      // block g / NST done: lane holds D[n = n0 + 4q + r][token lr]
      if (live) {
        const int64_t n0 = (int64_t)by * (kBlockN * NB) + (g / NST) * kBlockN + wave * 16 + 4 * q;
        if constexpr (MODE == kDown) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + orow * N + n0) =
              f32x4{s2 * acc[0], s2 * acc[1], s2 * acc[2], s2 * acc[3]};
        } else {
          u32x2 o;
          o[0] = pack_bf16x2(s2 * acc[0], s2 * acc[1]);
          o[1] = pack_bf16x2(s2 * acc[2], s2 * acc[3]);
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + orow * N + n0) = o;
        }
      }
      acc = f32x4{0, 0, 0, 0};
    }
    // keep each stage's LDS reads inside the stage: hoisting later stages' B
    // operands ahead (nothing orders them after the staging barrier) costs more
    // registers than the workgroups per CU can spare
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int MODE, bool F16, int NST, int NB, bool TL, bool PER>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(PER ? 3 : 1))) void gemm_decode_res_kernel(
    GemmArgs a, F16Args d) {
  constexpr bool kMoe = (MODE == kDown);
  __shared__ __attribute__((aligned(16))) uint16_t xs[16][NST * 512 + 8];
  if constexpr (PER) {
    static_assert(kMoe, "persistent form is for the routed modes");
    const int nby = (int)(a.N / (kBlockN * NB));
    const int total = *a.n_tiles * nby;   // <= grid_tiles * nby < 2^31 (host)
    for (int it = blockIdx.x; it < total; it += gridDim.x) {
      __syncthreads();   // the previous item's last LDS reads are done
      res_item<MODE, F16, NST, NB, TL>(a, d, xs, it / nby, it % nby);
    }
  } else {
    if (kMoe && (int)blockIdx.x >= *a.n_tiles) return;
    res_item<MODE, F16, NST, NB, TL>(a, d, xs, (int)blockIdx.x, (int)blockIdx.y);
  }
}

// Tiny batches (tiles of at most 4 rows, routed modes, fp16 form): the grid of
// 64-row workgroups is too small to fill the chip (one token: 8 experts x 24
// blocks of gate/up), and each workgroup streams K in a row of dependent stages.
// Here the 4 waves of a workgroup take the same 16 weight rows and split the
// stages of K among themselves (wave w: stages w, w + 4, ...), so there are 4x
// the workgroups with a quarter of the stages each. The whole activation tile
// (<= 4 rows x K <= 4096, fp16) sits in LDS; the waves' partial sums are added
// through LDS in wave order, then wave 0 applies the epilogue.
constexpr int kSmallRows = 4;
constexpr int kSmallMaxK = 4096;

// FULL (K = 4096): every wave takes exactly two stages, so no load sits behind a
// branch and the waits before the first stage's MFMAs do not also wait for the
// second stage's loads (a load issued under a branch makes those waits drain).
template <int MODE, bool TL, bool FULL>
__global__ __launch_bounds__(kThreads) void gemm_decode_ks_kernel(GemmArgs a, F16Args d) {
  static_assert(MODE == kGateUp, "gate/up: down has few stages and keeps the decode kernels");
  constexpr int U = 4, KC = 128 * U;
  __shared__ __attribute__((aligned(16))) uint16_t xs[kSmallRows][kSmallMaxK + 8];
  __shared__ f32x4 red[3][2][64];

  if ((int)blockIdx.x >= *a.n_tiles) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 15, q = lane >> 4;
  const int64_t N = a.N, K = a.K;
  const int32_t* t = a.tiles + 4 * (int64_t)blockIdx.x;
  const int e = t[0], rb = t[1], rows = t[2];

  const int64_t nrow = (int64_t)blockIdx.y * 16 + lr;
  int64_t coff, soff;
  if constexpr (TL) {
    const int64_t R = nrow / 32, r = nrow % 32;
    coff = (int64_t)e * N * (K / 2) + (R * (K / 32) + U * q) * 512 + r * 16;
    soff = (int64_t)e * N * (K / 16) + (R * (K / 256) + (2 * U * q) / 16) * 512 + r * 16 + (2 * U * q) % 16;
  } else {
    const int64_t wrow = (int64_t)e * N + nrow;
    coff = wrow * (K / 2) + 16 * U * q;
    soff = wrow * (K / 16) + 2 * U * q;
  }
  const uint8_t* c0 = a.w0.codes + coff;
  const uint8_t* s0 = a.w0.scales + soff;
  const uint8_t* c1 = a.w1.codes + coff;
  const uint8_t* s1 = a.w1.scales + soff;
  const int64_t SSTEP = TL ? 2 * KC : KC / 16;
  const int nst = (int)(K / KC);

  // this wave's first stage goes out before the activation staging
  Stage<U> Cg[2], Cu[2];
  u32x2 sg[2], su[2];
  auto load = [&](int b, int st) {
    load_codes<U, TL>(Cg[b], c0, (int64_t)st * KC);
    sg[b] = *reinterpret_cast<const u32x2*>(s0 + st * SSTEP);
    load_codes<U, TL>(Cu[b], c1, (int64_t)st * KC);
    su[b] = *reinterpret_cast<const u32x2*>(s1 + st * SSTEP);
  };
  // The tile's token rows and their exponents (gate/up) through scalar loads: they
  // neither queue behind the weight loads nor wait for them, and the epilogue
  // finds its scales ready instead of ending on two dependent loads.
  // (rows past the tile's last repeat its last row: no branches between the loads)
  if (FULL || wave < nst) load(0, wave);
  int tok[kSmallRows], xe[kSmallRows];
#pragma unroll
  for (int r = 0; r < kSmallRows; ++r) tok[r] = __builtin_amdgcn_readfirstlane(a.perm[rb + min(r, rows - 1)]);
#pragma unroll
  for (int r = 0; r < kSmallRows; ++r) tok[r] /= a.topk;
#pragma unroll
  for (int r = 0; r < kSmallRows; ++r) xe[r] = __builtin_amdgcn_readfirstlane(d.xexp[tok[r]]);
  const float s2g = a.w0.scale_2[e];
  const float s2u = a.w1.scale_2[e];

  // activation rows: the prep's x16 row of each slot's token. Buffer loads, all
  // issued before any is waited for; a unit past the tile's rows reads out of
  // the descriptor's range and gets zeros without a memory access.
  {
    constexpr int NU = kSmallRows * (kSmallMaxK / 8) / kThreads;
    const __amdgpu_buffer_rsrc_t xrs = rsrc(d.x16, a.x_rows * K * 2);
    u32x4 xv[NU];
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = i * kThreads + tid;
      const int r = u / (int)(K / 8), c = u % (int)(K / 8);   // r is the same across a wave (K >= 512)
      const int tr = r == 0 ? tok[0] : r == 1 ? tok[1] : r == 2 ? tok[2] : tok[3];
      const uint32_t off = r < rows ? (uint32_t)(tr * (int)K * 2 + 16 * c) : 0x80000000u;
      xv[i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
    }
    // K = 4096: the second stage goes out now, behind the activations; waiting
    // for those then counts the second stage's loads as still in flight
    if (FULL) load(1, wave + 4);
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = i * kThreads + tid;
      if (FULL || u < kSmallRows * (int)(K / 8)) st16(&xs[u / (int)(K / 8)][8 * (u % (int)(K / 8))], xv[i]);
    }
  }
  __syncthreads();

  f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  const f16x8 zero8 = {};
  // stage st from register set b (a literal at each call, so the sets stay in registers)
  auto step = [&](const int b, int st) {
    if (!FULL && st + 4 < nst) load(b ^ 1, st + 4);
    const int64_t kb = (int64_t)st * KC;
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const f16x2 sgf = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sg[b][i / 2] >> (16 * (i & 1)), 1.0f, false);
      const f16x2 suf = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(su[b][i / 2] >> (16 * (i & 1)), 1.0f, false);
#pragma unroll
      for (int sst = 0; sst < 4; ++sst) {
        const f16x8 B = lr < kSmallRows
                            ? *reinterpret_cast<const f16x8*>(&xs[lr < kSmallRows ? lr : 0][kb + 32 * U * q + 32 * i + 8 * sst])
                            : zero8;
        const f16x2 gs = (sst < 2) ? f16x2{sgf[0], sgf[0]} : f16x2{sgf[1], sgf[1]};
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant8_f16(Cg[b].c[i][sst], gs), B, acc0, 0, 0, 0);
        const f16x2 us = (sst < 2) ? f16x2{suf[0], suf[0]} : f16x2{suf[1], suf[1]};
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant8_f16(Cu[b].c[i][sst], us), B, acc1, 0, 0, 0);
      }
    }
  };
  if (FULL) {
    step(0, wave);
    step(1, wave + 4);
  } else {
    for (int st = wave; st < nst; st += 8) {
      step(0, st);
      if (st + 4 < nst) step(1, st + 4);
    }
  }

  // partial sums of waves 1..3 to wave 0, added in wave order
  if (wave > 0) {
    red[wave - 1][0][lane] = acc0;
    red[wave - 1][1][lane] = acc1;
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    const f32x4 p0 = red[w][0][lane], p1 = red[w][1][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      acc0[r] += p0[r];
      acc1[r] += p1[r];
    }
  }

  // ---- epilogue: lane holds D[n = 16 by + 4q + r][token lr], r = 0..3
  if (lr >= rows) return;
  const int64_t p = rb + lr;
  const int64_t n0 = (int64_t)blockIdx.y * 16 + 4 * q;
  const int xl = lr == 0 ? xe[0] : lr == 1 ? xe[1] : lr == 2 ? xe[2] : xe[3];
  float unscale = ldexpf(1.0f, -xl);
  if (a.act_scale) unscale *= *a.act_scale;   // W4A4: the activations' input_scale
  const float s2a = s2g * unscale;
  const float s2b = s2u * unscale;
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = silu(s2a * acc0[r]) * (s2b * acc1[r]);
  u32x2 o;
  o[0] = pack_bf16x2(v[0], v[1]);
  o[1] = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + p * N + n0) = o;
  // row maximum of |H| as stored, for the down projection's fp16 scaling (order-free)
  float m = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf((float)(__bf16)v[r]));
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  if (q == 0) atomicMax(reinterpret_cast<unsigned int*>(d.hmax + p), __builtin_bit_cast(unsigned int, m));
}

bool decode_small_supported(int64_t K, int64_t N) {
  return K % 512 == 0 && K >= 512 && K <= kSmallMaxK && N % 16 == 0;
}

hipError_t launch_decode_small(GemmMode mode, const GemmArgs& a, const F16Args& d, int64_t grid_tiles,
                               hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  const dim3 grid((unsigned)grid_tiles, (unsigned)(a.N / 16));
  const bool tl = a.w0.tiled;
  // gate/up only: down has few stages (K = I) and keeps the decode kernels
  if (mode != kGateUp) return hipErrorInvalidValue;
  const bool full = a.K == kSmallMaxK;
  if (tl && full) hipLaunchKernelGGL((gemm_decode_ks_kernel<kGateUp, true, true>), grid, dim3(kThreads), 0, s, a, d);
  else if (tl) hipLaunchKernelGGL((gemm_decode_ks_kernel<kGateUp, true, false>), grid, dim3(kThreads), 0, s, a, d);
  else if (full) hipLaunchKernelGGL((gemm_decode_ks_kernel<kGateUp, false, true>), grid, dim3(kThreads), 0, s, a, d);
  else hipLaunchKernelGGL((gemm_decode_ks_kernel<kGateUp, false, false>), grid, dim3(kThreads), 0, s, a, d);
  return hipGetLastError();
}

// K in multiples of 512 (U = 4) or 256 (U = 2) in either layout; other multiples of 64
// (U = 1, 128-input stages, the last one half masked when K % 128 == 64) are
// row-major only: the tiled layout needs K % 256 == 0. Those are the
// tensor-parallel shards of the intermediate size (1536 / 4 = 384, 1536 / 8 = 192).
bool decode_supported(GemmMode mode, int64_t K, int64_t N) {
  (void)mode;
  return N % kBlockN == 0 && K % 64 == 0 && K >= 128;
}

// Workgroups of `kern` resident on the current device at once (cached).
static int64_t resident_wgs(const void* kern) {
  static std::mutex mu;
  static struct { const void* k; int dev; int64_t n; } cache[128];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (cache[i].k == kern && cache[i].dev == dev) return cache[i].n;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, 0) != hipSuccess || per_cu < 1) per_cu = 1;
  const int64_t n = (int64_t)per_cu * cu_count();
  if (used < 128) cache[used++] = {kern, dev, n};
  return n;
}

// One-shot grid (tiles, N / rows per workgroup), or (persistent != null) a
// persistent grid of at most the resident workgroup count.
static void launch_items(const void* one_shot, const void* persistent, int64_t grid_tiles, int64_t nby,
                         const GemmArgs& a, const F16Args& d, hipStream_t s) {
  GemmArgs aa = a;
  F16Args dd = d;
  void* args[] = {&aa, &dd};
  const int64_t items = grid_tiles * nby;
  if (persistent && items < ((int64_t)1 << 31)) {   // the kernel counts items in 32 bits
    const int64_t g = std::min(items, resident_wgs(persistent));
    (void)hipLaunchKernel(persistent, dim3((unsigned)g), dim3(kThreads), args, 0, s);
  } else {
    (void)hipLaunchKernel(one_shot, dim3((unsigned)grid_tiles, (unsigned)nby), dim3(kThreads), args, 0, s);
  }
}

int decode_down_streams(bool f16, int64_t x_rows, int64_t K, int64_t N, int64_t grid_tiles) {
  // the fp16 form only (the bf16 form needs too many registers here); the
  // activation tile is read through a buffer descriptor: 32-bit offsets
  if (!f16 || K % 512 != 0 || K > 2048 || N % (kBlockN * 4) != 0 || x_rows * K * 2 >= ((int64_t)1 << 31)) return 0;
  // 64-row blocks per wave stream: as many as keep >= 4 workgroups per CU
  const int64_t want = 4 * (int64_t)cu_count();
  return grid_tiles * (N / (kBlockN * 4)) >= want ? 4 : grid_tiles * (N / (kBlockN * 2)) >= want ? 2 : 1;
}

template <int MODE, bool F16, bool TL>
static hipError_t launch_dec(const GemmArgs& a, const F16Args& d, int64_t grid_tiles, hipStream_t s) {
  constexpr int NS = 8;   // up to 8 stages: scales up front
  if constexpr (MODE == kDown && F16) {
    if (const int nb = decode_down_streams(true, a.x_rows, a.K, a.N, grid_tiles)) {
      switch (nb * 8 + (int)(a.K / 512)) {
#define NVFP4_RES(NB_, NST_)                                                                          \
  case NB_ * 8 + NST_:                                                                                 \
    launch_items((const void*)gemm_decode_res_kernel<MODE, F16, NST_, NB_, TL, false>,                \
                 (const void*)gemm_decode_res_kernel<MODE, F16, NST_, NB_, TL, true>, grid_tiles,       \
                 a.N / (kBlockN * NB_), a, d, s);                                                      \
    break;
        NVFP4_RES(1, 1) NVFP4_RES(1, 2) NVFP4_RES(1, 3) NVFP4_RES(1, 4)
        NVFP4_RES(2, 1) NVFP4_RES(2, 2) NVFP4_RES(2, 3) NVFP4_RES(2, 4)
        NVFP4_RES(4, 1) NVFP4_RES(4, 2) NVFP4_RES(4, 3) NVFP4_RES(4, 4)
#undef NVFP4_RES
        default: return hipErrorInvalidValue;
      }
      return hipGetLastError();
    }
  }
  const int64_t nby = a.N / kBlockN;
  // persistent for the routed down projection (its workgroups are short); the
  // gate/up loop body would need more registers than three waves per SIMD allow
#define NVFP4_DEC(U_, NS_)                                                                                      \
  launch_items((const void*)gemm_decode_kernel<MODE, U_, F16, NS_, TL, false>,                                  \
               MODE == kDown ? (const void*)gemm_decode_kernel<MODE, U_, F16, NS_, TL, MODE == kDown> : nullptr, \
               grid_tiles, nby, a, d, s)
  if (a.K % 512 == 0) {
    if (a.K / 512 <= NS) NVFP4_DEC(4, NS);
    else NVFP4_DEC(4, 0);
  } else if (a.K % 256 == 0) {
    if (a.K / 256 <= NS) NVFP4_DEC(2, NS);
    else NVFP4_DEC(2, 0);
  } else {
    if constexpr (TL) {
      return hipErrorInvalidValue;   // the tiled layout has K % 256 == 0
    } else {
      if ((a.K + 127) / 128 <= NS) NVFP4_DEC(1, NS);
      else NVFP4_DEC(1, 0);
    }
  }
#undef NVFP4_DEC
  return hipGetLastError();
}

template <int MODE, bool F16>
static hipError_t launch_dec(const GemmArgs& a, const F16Args& d, int64_t grid_tiles, hipStream_t s) {
  return a.w0.tiled ? launch_dec<MODE, F16, true>(a, d, grid_tiles, s) : launch_dec<MODE, F16, false>(a, d, grid_tiles, s);
}

hipError_t launch_decode(GemmMode mode, bool f16, const GemmArgs& a, const F16Args& d, int64_t grid_tiles,
                         hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  switch (mode) {
    case kGateUp: return f16 ? launch_dec<kGateUp, true>(a, d, grid_tiles, s) : launch_dec<kGateUp, false>(a, d, grid_tiles, s);
    case kDown: return f16 ? launch_dec<kDown, true>(a, d, grid_tiles, s) : launch_dec<kDown, false>(a, d, grid_tiles, s);
    case kLinear: return launch_dec<kLinear, false>(a, d, grid_tiles, s);
    case kGated: return launch_dec<kGated, false>(a, d, grid_tiles, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
