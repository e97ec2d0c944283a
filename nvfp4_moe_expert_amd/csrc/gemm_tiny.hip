// Routed experts of batches of at most four tokens: two launches in place of the
// route, gate/up, down and combine kernels.
//
// Passage: TensorFold issue #308, "What the branch does" (the routed experts in a
// grouped NVFP4 kernel on bf16 rows, each expert's weight_scale_2 applied to its
// product); the combine follows the fixed-order sum of the routed output.
// With one to four tokens a call streams the weights of at most 32 experts (one
// token: 57 MB for gate/up, 28 MB for down) and is bound by fixed costs: each
// launch costs some microseconds, and a weight load whose address comes from a
// table that an earlier kernel wrote waits a memory round trip first.
//
// tiny_gateup: workgroup (tile i, 16 weight rows nb). Wave w owns stages w and
// w + 4 of 512 inputs. Every wave loads the (at most 32) top-k ids and its two
// stage slices of every token's row, then derives the tile list itself (tiles in
// order of each local expert's first slot, its slots in slot order, 16 per tile)
// and requests the first stage of its gate and up weights (the second stage of
// each goes out when its first has arrived); nothing waits for weights before the
// MFMAs. Row
// maxima: each wave's over its slices (DPP reductions), combined after one
// barrier; each row is scaled into fp16 by 2^p (p puts its max |x| in
// [2^14, 2^15), as in the other kernel classes) and each wave stages its own
// slices in LDS. The MFMAs are those of the K-split kernel: lane (r, q) owns
// weight row 16 nb + r and inputs [kb + 128 q, +128) of each stage; the 4 waves'
// partial sums are added in wave order. Epilogue: H[slot] = bf16(SiLU(s2g * g) *
// s2u * u) in slot order, and the largest |H| of each (slot, nb) block of 16
// values into hpart[slot][nb].
//
// tiny_down: workgroup (nb, t) = 16 output rows of token t. Wave w (of 8) takes
// the token's slots w, w + 8, ...: the H row and the weights of its next slot are in flight while it
// multiplies the current one (H loads before weight loads, so waiting for a row
// never waits for weights that are not needed yet). The H row is scaled to fp16
// by 2^p, p from the largest of the slot's hpart entries, and staged in the
// wave's own LDS buffer. d = s2d[e] * 2^-p * acc goes to LDS; then y[t][16 rows]
// = bf16(sum over j = 0..k-1 in order of w[t, j] * d[t*k + j] over local slots,
// plus the extra rows summed in split order), the combine kernel's sum.
//
// Summation order of an element: one MFMA chain per (slot, weight) over the
// stages in increasing k; for gate/up the waves' chains are added in wave order.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace tiny_detail {

constexpr int kThreads = 256;
constexpr int kDownWaves = 8;     // down: waves per workgroup (two per SIMD)
constexpr int kMaxT = 4;          // tokens
constexpr int kMaxSlots = 32;     // T * k: the ids of a call fit the lanes of one wave
constexpr int kRows = 16;         // slots per gate/up tile: the columns of one MFMA
constexpr int kMaxH = 4096;       // gate/up inputs: at most 8 stages, two per wave
constexpr int kMaxI = 2048;       // down inputs: at most 4 stages per slot
constexpr int U = 4;              // 16-byte code chunks per lane and stage
constexpr int KC = 128 * U;       // inputs per stage

// codes and scale bytes of one stage for one lane
constexpr int kChunkLoads = U + 1;   // vector loads per Stage (U code chunks, one scale load)
struct Stage {
  u32x4 c[U];
  u32x2 s;
};

// A lane's code and scale offsets for weight row `nrow` of expert e of an [N, K]
// tensor (K % 512 == 0): inputs [128 q, +128) of each stage.
template <bool TL>
__device__ __forceinline__ void lane_offsets(int64_t e, int64_t N, int64_t K, int64_t nrow, int q, int64_t& coff,
                                             int64_t& soff) {
  if constexpr (TL) {   // blocks of 32 rows: 512-byte runs per 32-input chunk / 256-input scale chunk
    const int64_t R = nrow / 32, r = nrow % 32;
    coff = e * N * (K / 2) + (R * (K / 32) + U * q) * 512 + r * 16;
    soff = e * N * (K / 16) + (R * (K / 256) + q / 2) * 512 + r * 16 + 8 * (q % 2);
  } else {
    const int64_t wrow = e * N + nrow;
    coff = wrow * (K / 2) + 64 * q;
    soff = wrow * (K / 16) + 8 * q;
  }
}

template <bool TL>
__device__ __forceinline__ void load_stage(Stage& st, const uint8_t* codes, const uint8_t* scales, int kb) {
#pragma unroll
  for (int i = 0; i < U; ++i) {   // non-temporal for tiled codes only (whole lines per instruction)
    const uint8_t* p = codes + (TL ? 16 * (int64_t)kb : kb / 2) + (TL ? 512 : 16) * i;
    st.c[i] = TL ? ld16_nt(p) : ld16(p);
  }
  st.s = *reinterpret_cast<const u32x2*>(scales + (TL ? 2 * (int64_t)kb : kb / 16));
}

// s_waitcnt: at most N vector memory operations of this wave still outstanding
// (gfx9 encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt and
// lgkmcnt at their maxima, so neither is waited for)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070 | 0x0F00);
}

// the two e4m3 scale bytes of code chunk i (blocks 2i and 2i + 1 of the lane's 8) as fp16
__device__ __forceinline__ f16x2 chunk_scales(const u32x2& s, int i) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s[i / 2] >> (16 * (i & 1)), 1.0f, false);
}

// 8 bf16 (one 16-byte unit) times 2^p -> 8 fp16 (exact for values down to 2^-28 of
// a row maximum in [2^14, 2^15) after scaling)
__device__ __forceinline__ u32x4 f16_scaled(const u32x4& v, float sc) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const _Float16 lo = (_Float16)(bf16_lo(v[j]) * sc), hi = (_Float16)(bf16_hi(v[j]) * sc);
    o[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  return o;
}

__device__ __forceinline__ uint32_t absmax_bf16x8(const u32x4& v) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) m = max(m, max(v[j] & 0x7FFFu, (v[j] >> 16) & 0x7FFFu));
  return m;
}

// Largest value over the 64 lanes (unsigned), in every lane: DPP shifts within
// rows of 16 (each lane ends with the maximum of itself and the lanes below it in
// its row), then row broadcasts carry row maxima upward; lane 63 ends with all.
// Lanes a shift reaches past the edge of a row keep their own value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x111, 0xF, 0xF, false));   // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x112, 0xF, 0xF, false));   // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x114, 0xF, 0xF, false));   // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x118, 0xF, 0xF, false));   // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));   // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));   // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

}  // namespace tiny_detail

using namespace tiny_detail;

// NST = H / 512 stages (1..8).
template <bool TL, int NST>
__global__ __launch_bounds__(kThreads) void tiny_gateup_kernel(TinyArgs a) {
  constexpr int K = NST * KC;
  __shared__ __attribute__((aligned(16))) uint16_t xw[4][kMaxT][2][KC + 8];   // each wave's stages, fp16
  __shared__ f32x4 red[3][2][64];
  __shared__ uint32_t wmax[4][kMaxT];
  __shared__ int tslot[4][kRows];   // slot of each tile row, per wave

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, q = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t N = a.I;
  const int T = (int)a.T, S = T * a.k;
  // this wave's stages (wave w: w and w + 4); a wave without one takes a stage of
  // another wave again (loads, no MFMAs), so no load sits behind a branch and every
  // wait counts exactly the loads before the one it needs
  const bool has0 = NST >= 4 || wave < NST, has1 = NST >= 8 || wave + 4 < NST;   // uniform
  const int st0 = min(wave, NST - 1), st1 = has1 ? wave + 4 : st0;

  // ---- loads that need no routing: the ids, then this wave's two stage slices of
  // the T activation rows (lane l: inputs 512 st + 8 l .. +8 of each)
  const int idv = lane < S ? a.ids[lane] : 0;
  const __amdgpu_buffer_rsrc_t xrs = rsrc(a.x, (int64_t)T * K * 2);
  u32x4 xv[kMaxT][2];
#pragma unroll
  for (int r = 0; r < kMaxT; ++r)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int st = h ? st1 : st0;
      const uint32_t off = r < T ? (uint32_t)((r * K + st * KC + 8 * lane) * 2) : 0x80000000u;
      xv[r][h] = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
    }

  // ---- the tile list, from the ids (the same in every wave): tiles in order of
  // each local expert's first slot, its slots in slot order, 16 per tile
  const int e = (lane < S && idv - a.eb >= 0 && idv - a.eb < a.E) ? idv - a.eb : -1;
  // slots of this lane's expert, those of them before this lane, the first of them
  int cnt = 0, before = 0, fl = 64;
  for (int j = 0; j < S; ++j) {
    const bool eq = __builtin_amdgcn_readlane(e, j) == e;
    cnt += eq;
    before += eq & (j < lane);
    fl = (eq && j < fl) ? j : fl;
  }
  const bool first = e >= 0 && before == 0;
  const int ntl = first ? (cnt + kRows - 1) / kRows : 0;   // tiles of this lane's expert, at its first slot
  // tiles of the experts whose first slot comes before this lane's expert's
  int tbase = 0;
  if (__builtin_amdgcn_ballot_w64(ntl > 1) == 0) {
    const uint64_t below = fl >= 64 ? ~0ull : ((1ull << fl) - 1);
    tbase = __builtin_popcountll(__builtin_amdgcn_ballot_w64(first) & below);   // one tile per expert
  } else {
    for (int j = 0; j < S; ++j) tbase += j < fl ? __builtin_amdgcn_readlane(ntl, j) : 0;
  }
  const int nby = (int)(N / 16), tile = (int)blockIdx.x / nby, nb = (int)blockIdx.x % nby;
  const uint64_t m = __builtin_amdgcn_ballot_w64(e >= 0 && tbase + before / kRows == tile);
  if (m == 0) return;        // past the last tile (the same in every wave: no barrier passed yet)
  const int ex = __builtin_amdgcn_readlane(e, (int)__builtin_ctzll(m));
  const int rows = __builtin_popcountll(m);
  // tile row of each of the tile's slots (in slot order), through LDS to the lanes
  // that own the rows; a wave's LDS operations take effect in program order
  if ((m >> lane) & 1) tslot[wave][__builtin_popcountll(m & ((1ull << lane) - 1))] = lane;

  // ---- the weights of this wave's stages
  const int64_t nrow = (int64_t)nb * 16 + lr;
  int64_t coff, soff;
  lane_offsets<TL>(ex, N, K, nrow, q, coff, soff);
  // (the first stage of each weight now, the second one as each first one arrives)
  Stage G[2], Up[2];
  load_stage<TL>(G[0], a.gate.codes + coff, a.gate.scales + soff, st0 * KC);
  load_stage<TL>(Up[0], a.up.codes + coff, a.up.scales + soff, st0 * KC);
  const float s2g = a.gate.scale_2[ex], s2u = a.up.scale_2[ex];

  // ---- row maxima: each wave's over its slices (the waves' stages cover the row),
  // combined after one barrier; then the wave's slices in fp16 * 2^p into its own
  // LDS area (read back by this wave only)
#pragma unroll
  for (int r = 0; r < kMaxT; ++r) {
    const uint32_t mx = wave_max_u32(max(absmax_bf16x8(xv[r][0]), absmax_bf16x8(xv[r][1])));
    if (lane == 0) wmax[wave][r] = mx;
  }
  __syncthreads();
  int pr[kMaxT];
#pragma unroll
  for (int r = 0; r < kMaxT; ++r) {
    pr[r] = row_exponent(max(max(wmax[0][r], wmax[1][r]), max(wmax[2][r], wmax[3][r])) << 16);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (r < T) st16(&xw[wave][r][h][8 * lane], f16_scaled(xv[r][h], ldexpf(1.0f, pr[r])));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---- MFMAs: B = the token row of tile row lr. Lanes past the tile's rows read
  // the first token's row: their output columns are never stored (each column of
  // an MFMA result depends on its own column of B alone).
  const int trow = lr < rows ? tslot[wave][lr] / a.k : 0;
  f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  // one weight's stage h into acc
  auto step = [&](const Stage& g, f32x4& acc, const int h) {
    const uint16_t* xrow = &xw[wave][trow][h][128 * q];
    f16x8 B[U][4];   // the stage's activations, read from LDS together
#pragma unroll
    for (int i = 0; i < U; ++i)
#pragma unroll
      for (int sst = 0; sst < 4; ++sst) B[i][sst] = *reinterpret_cast<const f16x8*>(xrow + 32 * i + 8 * sst);
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const f16x2 gsc = chunk_scales(g.s, i);
#pragma unroll
      for (int sst = 0; sst < 4; ++sst) {
        const f16x2 gs = sst < 2 ? f16x2{gsc[0], gsc[0]} : f16x2{gsc[1], gsc[1]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant8_f16(g.c[i][sst], gs), B[i][sst], acc, 0, 0, 0);
      }
    }
  };
  // Weight chunks (one weight, one stage: kChunkLoads loads) stream two at a time:
  // when a first-stage chunk has arrived, the same weight's second stage is
  // requested, then the arrived chunk is multiplied. With all four chunks requested
  // at once, every wave's chunks arrived only towards the end of the stream and all
  // of the dequantization (eight VALU instructions per MFMA) ran after it; this way
  // only the last chunk's does. The scheduling barriers keep the loads where they
  // are written; the waits are the compiler's own plus the two explicit ones.
  wait_vm<kChunkLoads>();   // G[0] in, Up[0] may still be in flight
  __builtin_amdgcn_sched_barrier(0);
  load_stage<TL>(G[1], a.gate.codes + coff, a.gate.scales + soff, st1 * KC);
  __builtin_amdgcn_sched_barrier(0);
  if (has0) step(G[0], acc0, 0);
  wait_vm<kChunkLoads>();   // Up[0] in, G[1] may still be in flight
  __builtin_amdgcn_sched_barrier(0);
  load_stage<TL>(Up[1], a.up.codes + coff, a.up.scales + soff, st1 * KC);
  __builtin_amdgcn_sched_barrier(0);
  if (has0) step(Up[0], acc1, 0);
  if (has1) step(G[1], acc0, 1);
  if (has1) step(Up[1], acc1, 1);

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

  // ---- epilogue: lane holds D[n = 16 nb + 4q + r][tile row lr], r = 0..3
  if (lr >= rows) return;    // lanes lr, lr + 16, lr + 32, lr + 48 leave together
  const int sl = tslot[0][lr];
  const int tk = sl / a.k;
  const float unscale = ldexpf(1.0f, -(tk == 0 ? pr[0] : tk == 1 ? pr[1] : tk == 2 ? pr[2] : pr[3]));
  const float s2a = s2g * unscale, s2b = s2u * unscale;
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = silu(s2a * acc0[r]) * (s2b * acc1[r]);
  u32x2 o;
  o[0] = pack_bf16x2(v[0], v[1]);
  o[1] = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<u32x2*>(a.h + (int64_t)sl * N + nb * 16 + 4 * q) = o;
  float mv = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) mv = fmaxf(mv, fabsf((float)(__bf16)v[r]));
  mv = fmaxf(mv, __shfl_xor(mv, 16));
  mv = fmaxf(mv, __shfl_xor(mv, 32));
  if (q == 0) a.hpart[(int64_t)sl * (N / 16) + nb] = __builtin_bit_cast(uint32_t, mv);
}

// NST = I / 512 stages per slot (1..4); JW = slots per wave at most (1, 2 or 4).
// Workgroup (nb, t): 16 output rows of token t, its k slots over 8 waves.
template <bool TL, int NST, int JW>
__global__ __launch_bounds__(64 * kDownWaves) void tiny_down_kernel(TinyArgs a) {
  constexpr int K = NST * KC;
  constexpr int NB = JW > 1 ? 2 : 1;   // slots in flight per wave
  __shared__ __attribute__((aligned(16))) uint16_t hs[kDownWaves][NB][kMaxI + 8];
  __shared__ float part[kMaxSlots][16];
  __shared__ float wslot[kMaxSlots];   // w[t, j] of the token's slots
  __shared__ int okslot[kMaxSlots];    // slot j's expert is one of this GPU's

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, q = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t N = a.H;
  const int T = (int)a.T, kk = a.k, t = (int)blockIdx.y, s0 = t * kk;
  // lane j < k: the local expert of slot s0 + j
  int e = -1;
  float twv = 0.0f;
  if (lane < kk) {
    const int v = a.ids[s0 + lane] - a.eb;
    e = (v >= 0 && v < a.E) ? v : -1;
    twv = a.tw[s0 + lane];
  }
  const int64_t nrow = (int64_t)blockIdx.x * 16 + lr;

  // one register set per slot in flight: H units, hpart entries, weights
  struct Job {
    u32x4 h[NST];
    uint32_t hp[2];
    Stage w[NST];
  };
  Job J[NB];
  // slot s0 + j's loads into set b: H row and its block maxima first, then the
  // weights. Never behind a branch: a slot past the token's last is loaded as the
  // last one again, and an id outside this GPU's experts loads expert 0's rows
  // (neither is used).
  auto issue = [&](Job& b, int j) {
    j = min(j, kk - 1);
    const uint16_t* hrow = a.h + (int64_t)(s0 + j) * K;
#pragma unroll
    for (int i = 0; i < NST; ++i) b.h[i] = ld16(hrow + 8 * (lane + 64 * i));
    const uint32_t* hp = a.hpart + (int64_t)(s0 + j) * (K / 16);
    b.hp[0] = hp[lane % (K / 16)];
    b.hp[1] = hp[(lane + 64) % (K / 16)];
    const int ej = max(__builtin_amdgcn_readlane(e, j), 0);
    int64_t coff, soff;
    lane_offsets<TL>(ej, N, K, nrow, q, coff, soff);
#pragma unroll
    for (int st = 0; st < NST; ++st) load_stage<TL>(b.w[st], a.down.codes + coff, a.down.scales + soff, st * KC);
  };
  // slot s0 + j from set b through LDS buffer bb (a literal at each call)
  auto run = [&](Job& b, const int bb, int j) {
    const int ej = __builtin_amdgcn_readlane(e, j);
    if (ej < 0) return;      // uniform: not this GPU's expert
    const int p = row_exponent(wave_max_u32(max(b.hp[0], b.hp[1])));
    const float sc = ldexpf(1.0f, p);
    uint16_t* buf = hs[wave][bb];
#pragma unroll
    for (int i = 0; i < NST; ++i) st16(buf + 8 * (lane + 64 * i), f16_scaled(b.h[i], sc));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // B: the slot's H row in every column (only column 0 of the result is used)
    f32x4 acc = {0, 0, 0, 0};
    const uint16_t* hrow = buf + 128 * q;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      f16x8 B[U][4];
#pragma unroll
      for (int i = 0; i < U; ++i)
#pragma unroll
        for (int sst = 0; sst < 4; ++sst) B[i][sst] = *reinterpret_cast<const f16x8*>(hrow + st * KC + 32 * i + 8 * sst);
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const f16x2 sc2 = chunk_scales(b.w[st].s, i);
#pragma unroll
        for (int sst = 0; sst < 4; ++sst) {
          const f16x2 s = sst < 2 ? f16x2{sc2[0], sc2[0]} : f16x2{sc2[1], sc2[1]};
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant8_f16(b.w[st].c[i][sst], s), B[i][sst], acc, 0, 0, 0);
        }
      }
    }
    // lane (0, q) holds D[n = 16 nb + 4q + r][0]
    if (lr == 0) {
      const float s2 = a.down.scale_2[ej] * ldexpf(1.0f, -p);
#pragma unroll
      for (int r = 0; r < 4; ++r) part[j][4 * q + r] = s2 * acc[r];
    }
  };
  // this wave's slots wave, wave + 8, ... of the token: up to two in flight
  constexpr int W = kDownWaves;
  issue(J[0], wave);
  if constexpr (NB > 1) issue(J[NB - 1], wave + W);
#pragma unroll
  for (int i = 0; i < JW; i += 2) {
    const int j0 = wave + W * i, j1 = j0 + W;
    if (j0 < kk) run(J[0], 0, j0);
    if (i + 2 < JW) issue(J[0], j0 + 2 * W);
    if constexpr (NB > 1) {
      if (j1 < kk) run(J[NB - 1], NB - 1, j1);
      if (i + 2 < JW) issue(J[NB - 1], j1 + 2 * W);
    }
  }
  // the slots' weights and flags for the sum below, from the registers loaded at
  // the start (read back from LDS, so the sum waits on no global load per slot)
  if (wave == 0 && lane < kk) {
    wslot[lane] = twv;
    okslot[lane] = e >= 0;
  }
  __syncthreads();

  // ---- y[t][16 nb + 8 h .. +8] for thread h: the combine's fixed-order sum
  if (tid >= 2) return;
  const int h8 = 8 * tid;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = 0; j < kk; ++j) {
    if (!okslot[j]) continue;
    const float wt = wslot[j];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += wt * part[j][h8 + i];
  }
  const int64_t col = (int64_t)blockIdx.x * 16 + h8;
  if (a.extra) {   // a contribution summed after the routed slots (the shared expert), split by split
    float x8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int z = 0; z < a.extra_splits; ++z) {
      const f32x4* ex = reinterpret_cast<const f32x4*>(a.extra + ((int64_t)z * T + t) * N + col);
      const f32x4 p0 = ex[0], p1 = ex[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x8[i] += p0[i];
        x8[4 + i] += p1[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += x8[i];
  }
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
  st16(a.y + (int64_t)t * N + col, o);
}

static hipError_t launch_tiny_down(const TinyArgs& a, hipStream_t s) {
  const dim3 gd((unsigned)(a.H / 16), (unsigned)a.T);
  // slots per wave: 1 (top-k <= 8), 2 (<= 16) or 4
  const int jw = a.k <= 8 ? 0 : a.k <= 16 ? 1 : 2;
  switch ((int)(a.I / KC) * 6 + (a.down.tiled ? 3 : 0) + jw) {
#define NVFP4_TD(NST_)                                                                                             \
  case NST_ * 6: hipLaunchKernelGGL((tiny_down_kernel<false, NST_, 1>), gd, dim3(64 * kDownWaves), 0, s, a); break;    \
  case NST_ * 6 + 1: hipLaunchKernelGGL((tiny_down_kernel<false, NST_, 2>), gd, dim3(64 * kDownWaves), 0, s, a); break; \
  case NST_ * 6 + 2: hipLaunchKernelGGL((tiny_down_kernel<false, NST_, 4>), gd, dim3(64 * kDownWaves), 0, s, a); break; \
  case NST_ * 6 + 3: hipLaunchKernelGGL((tiny_down_kernel<true, NST_, 1>), gd, dim3(64 * kDownWaves), 0, s, a); break;  \
  case NST_ * 6 + 4: hipLaunchKernelGGL((tiny_down_kernel<true, NST_, 2>), gd, dim3(64 * kDownWaves), 0, s, a); break;  \
  case NST_ * 6 + 5: hipLaunchKernelGGL((tiny_down_kernel<true, NST_, 4>), gd, dim3(64 * kDownWaves), 0, s, a); break;
    NVFP4_TD(1) NVFP4_TD(2) NVFP4_TD(3) NVFP4_TD(4)
#undef NVFP4_TD
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}


bool tiny_supported(int64_t T, int64_t k, int64_t H, int64_t I) {
  return T >= 1 && T <= kMaxT && T * k <= kMaxSlots && H % KC == 0 && H <= kMaxH && I % KC == 0 && I <= kMaxI;
}

hipError_t launch_tiny(const TinyArgs& a, bool down, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (!tiny_supported(a.T, a.k, a.H, a.I)) return hipErrorInvalidValue;
  if (down) return launch_tiny_down(a, s);
  // tiles of at most 16 slots: sum over experts of ceil(slots / 16) <= (number of
  // experts with a slot) + (slots / 16)
  const int64_t S = a.T * a.k;
  const int64_t grid_tiles = std::min<int64_t>(S, a.E) + S / kRows;
  // one dimension, tile-major: the workgroups of tiles past the last real one (the
  // tile count is known on the device only) come last in the dispatch order, so the
  // real ones spread evenly over the compute units
  const dim3 gu((unsigned)(grid_tiles * (a.I / 16)));
  switch ((int)(a.H / KC) * 2 + (a.gate.tiled ? 1 : 0)) {
#define NVFP4_TG(NST_)                                                                               \
  case NST_ * 2: hipLaunchKernelGGL((tiny_gateup_kernel<false, NST_>), gu, dim3(kThreads), 0, s, a); break; \
  case NST_ * 2 + 1: hipLaunchKernelGGL((tiny_gateup_kernel<true, NST_>), gu, dim3(kThreads), 0, s, a); break;
    NVFP4_TG(1) NVFP4_TG(2) NVFP4_TG(3) NVFP4_TG(4) NVFP4_TG(5) NVFP4_TG(6) NVFP4_TG(7) NVFP4_TG(8)
#undef NVFP4_TG
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nvfp4
