// The BF16 steps either side of the routed experts: router logits with top-k
// softmax selection, and the shared-expert BF16 MLP (TensorFold issue #308,
// "What the branch does": the shared expert runs as a BF16 MLP; the model card
// "GLM-5.3-Flash-NVFP4-W4A4-Experts", "Quantization boundary": routers and
// shared experts stay BF16).
//
// bf16 GEMM, C[m, n] = sum_k X[m, k] * W[n, k] (activations and weights both
// K-contiguous), on v_mfma_f32_32x32x16_bf16 with fp32 accumulation:
// * a workgroup of 4 waves takes 64 activation rows x 64 weight rows (of each of
//   NW weight matrices: 2 for the gated form, whose gate and up rows n are
//   multiplied by the same wave, so SiLU(gate) * up is formed in registers; the
//   one-weight products on 128-row tiles take two adjacent 64-row blocks of
//   their weight the same way);
// * wave (t, w) multiplies activation rows 32t.. against weight rows 32w.. with
//   A = weights and B = activations, both read from LDS; the K loop runs in
//   stages of 64 inputs, double-buffered in LDS, each stage loaded into
//   registers one stage ahead of its LDS write (two register sets) when the
//   loop is long, else while the stage before it is multiplied (the weight
//   stream is bound by how many bytes are in flight); the tiles move in 16-byte
//   units, eight threads to each 128-byte row segment of a stage, and a wave
//   skips the MFMAs of its 32-row blocks that lie past the tile's rows;
// * small batches split K over up to 16 workgroups per tile; every split writes
//   its fp32 partial tile and a second kernel sums the splits in split order,
//   so the result does not depend on scheduling.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace block_detail {

constexpr int kThreads = 256;
constexpr int BM = 64;        // activation rows per workgroup
constexpr int BN = 64;        // weight rows per workgroup (per weight matrix)
constexpr int BK = 64;        // inputs per stage
constexpr int LDW = BK + 8;   // LDS row pitch in bf16 (16-byte pad: conflict-free 16-byte reads)

}  // namespace block_detail

using namespace block_detail;

// NW weight matrices (1: plain, 2: gate and up). Output per MODE:
//   kBf16F32  - C fp32 [M, N] (splits == 1) or the split's partial;
//   kBf16Gated- H bf16 [M, N] = bf16(SiLU(C_gate) * C_up) (splits == 1), or the
//               split's partials of C_gate and C_up ([2][M][N]);
//   kBf16F32W - as kBf16F32 (no split) with two adjacent 64-row blocks of the
//               one weight per workgroup: each activation tile loaded serves 128
//               weight rows, so a down projection (one weight, N = 4096) reads its
//               activation tiles half as often.
enum Bf16Mode : int { kBf16F32 = 0, kBf16Gated = 1, kBf16F32W = 2 };

// Grouped form (routed experts with bf16 weights): workgroup x takes tile x of
// the route's tile list (expert e, rows rb .. rb+rows of the permuted order, at
// most 64); weights are expert e's [N, K]; activation row r is x[perm[rb+r] /
// topk] (topk > 0: gate/up on tokens) or x[rb+r] (topk == 0: down on H rows in
// permuted order); results go to row rb+r (gate/up: H) or to slot perm[rb+r]
// (down: Ypart). No K split.
struct Bf16Group {
  const int32_t* tiles;    // null: plain GEMM
  const int32_t* n_tiles;
  const int32_t* perm;
  int topk;
  int64_t w_stride;        // elements of one expert's weight
};

// TM: 32-row activation blocks per wave (1: 64-row workgroup tiles; 2: 128-row
// tiles, for grouped calls whose experts average at least 64 rows: every weight
// row loaded then serves twice the activation rows, and a tile of a large expert
// re-reads its weights half as often).
template <int MODE, bool GROUPED, int TM, int R>
__global__ __launch_bounds__(kThreads, 2) void bf16_gemm_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w0,
                                                             const uint16_t* __restrict__ w1, int64_t M, int64_t N,
                                                             int64_t K, int64_t k_per_split, void* __restrict__ out,
                                                             float* __restrict__ partial, Bf16Group grp) {
  constexpr int NW = MODE == kBf16F32 ? 1 : 2;
  constexpr bool kWide = MODE == kBf16F32W;   // the NW blocks are rows n0 and n0 + BN of w0
  // 64-row routed tiles (decode-shaped batches) read each weight byte once per call:
  // non-temporal loads stream them faster. Larger tiles re-read an expert's weights
  // from the caches, which such loads would lose.
  constexpr bool kStreamW = GROUPED && TM == 1;
  constexpr int NT = kThreads;
  constexpr int TBM = BM * TM;   // activation rows per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][TBM][LDW];
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][NW * BN][LDW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wt = wave >> 1, wn = wave & 1;
  int64_t m0 = (int64_t)blockIdx.x * TBM, rb = 0;
  int64_t nb = blockIdx.y;   // 64-row block of the weights
  if constexpr (GROUPED) {
    int tile = (int)blockIdx.x;
    if constexpr (TM == 2) {
      // 128-row tiles (prefill-shaped calls): workgroups are dealt to the 8 XCDs
      // round-robin by linear id; each XCD runs whole tiles (tile = 8*j + xcd), all
      // weight blocks of a tile one after another, so the tile's activation rows stay
      // in that XCD's L2 across its blocks (4096-token layer 4.27 -> 3.96 ms)
      const int nby = (int)gridDim.y;
      const int64_t lin = (int64_t)blockIdx.x + (int64_t)gridDim.x * blockIdx.y;
      const int xcd = (int)(lin % 8);
      const int64_t j = lin / 8;
      tile = (int)((j / nby) * 8 + xcd);
      nb = j % nby;
    }
    if (tile >= *grp.n_tiles) return;
    const int32_t* t = grp.tiles + 4 * (int64_t)tile;
    w0 += (int64_t)t[0] * grp.w_stride;
    if (MODE == kBf16Gated) w1 += (int64_t)t[0] * grp.w_stride;
    rb = t[1];
    M = t[2];   // rows of this tile
    m0 = 0;
  }
  const int64_t n0 = nb * BN * (kWide ? 2 : 1);
  const int64_t kb0 = (int64_t)blockIdx.z * k_per_split;
  const int64_t kb1 = std::min(K, kb0 + k_per_split);
  const int nst = (int)((kb1 - kb0) / BK);

  // global -> LDS in 16-byte units (8 inputs): unit u of a stage is row u / 8,
  // inputs 8 (u % 8) ..; thread tid moves units tid, tid + NT, ... of the
  // activation tile (TBM rows) and of the weight tile (NW x BN rows)
  constexpr int XU = TBM * (BK / 8) / NT, WU = NW * BN * (BK / 8) / NT;
  static_assert(XU * NT == TBM * (BK / 8) && WU * NT == NW * BN * (BK / 8), "loader units");
  const uint16_t* xp[XU];
  int xl[XU];   // LDS row * LDW + column of each unit
#pragma unroll
  for (int i = 0; i < XU; ++i) {
    const int u = tid + NT * i, r = u >> 3, c = (u & 7) * 8;
    const bool ok = m0 + r < M;
    int64_t xrow = m0 + r;
    if constexpr (GROUPED) {
      if (ok) xrow = grp.topk > 0 ? grp.perm[rb + r] / grp.topk : rb + r;
    }
    xp[i] = x + (ok ? xrow * K : 0) + c;
    xl[i] = r * LDW + c;
  }
  const uint16_t* wp[WU];
  int wl[WU];
#pragma unroll
  for (int i = 0; i < WU; ++i) {
    const int u = tid + NT * i, j = u / (BN * (BK / 8)), r = (u % (BN * (BK / 8))) >> 3, c = (u & 7) * 8;
    const int64_t row = n0 + (kWide ? j * BN : 0) + r;
    const bool ok = row < N;
    wp[i] = (kWide || j == 0 ? w0 : w1) + (ok ? row * K : 0) + c;
    wl[i] = (j * BN + r) * LDW + c;
  }
  // Register ring of R sets: stage s is loaded into set s % R, R - 1 stages
  // before its registers are written to LDS, so each stage's loads have R - 1
  // stages of MFMAs to land. Rows past M or N read row 0 of their operand (their
  // results are never stored), so no load sits behind a branch and every wait
  // counts exactly the loads it needs; loads for stages past the last re-read it.
  // R == 1 (short K loops, where R stages of such re-reads would cost more than the
  // lead gains): the next stage is loaded while the current one is multiplied.
  u32x4 rx[R][XU], rw[R][WU];
  auto load = [&](int set, int s) {
    const int64_t kb = kb0 + (int64_t)std::min(s, nst - 1) * BK;
#pragma unroll
    for (int i = 0; i < XU; ++i) rx[set][i] = ld16(xp[i] + kb);
#pragma unroll
    for (int i = 0; i < WU; ++i) rw[set][i] = kStreamW ? ld16_nt(wp[i] + kb) : ld16(wp[i] + kb);
  };
  auto store = [&](int set, int b) {
#pragma unroll
    for (int i = 0; i < XU; ++i) st16(&xs[b][0][0] + xl[i], rx[set][i]);
#pragma unroll
    for (int i = 0; i < WU; ++i) st16(&ws[b][0][0] + wl[i], rw[set][i]);
  };

  f32x16 acc[NW][TM];
#pragma unroll
  for (int j = 0; j < NW; ++j)
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[j][t] = f32x16{};
  // the MFMAs of one stage, from LDS buffer b, for the wave's first NA 32-row
  // blocks (those past the tile's rows are never stored, so they are skipped)
  auto multiply_n = [&](int b, auto na_c) {
    constexpr int NA = decltype(na_c)::value;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kk = 16 * ks + 8 * (lane >> 5);
      bf16x8 B[TM];
#pragma unroll
      for (int t = 0; t < NA; ++t)
        B[t] = *reinterpret_cast<const bf16x8*>(&xs[b][32 * (TM * wt + t) + (lane & 31)][kk]);
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        const bf16x8 A = *reinterpret_cast<const bf16x8*>(&ws[b][j * BN + 32 * wn + (lane & 31)][kk]);
#pragma unroll
        for (int t = 0; t < NA; ++t) acc[j][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B[t], acc[j][t], 0, 0, 0);
      }
    }
  };
  const int64_t wrow0 = m0 + 32 * TM * wt;   // first activation row of this wave
  const int na = wrow0 >= M ? 0 : (int)std::min<int64_t>(TM, (M - wrow0 + 31) / 32);
  auto multiply = [&](int b) {
    if (na == TM) multiply_n(b, std::integral_constant<int, TM>{});
    else if (TM > 1 && na == 1) multiply_n(b, std::integral_constant<int, 1>{});
  };

  if (nst > 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) load(r, r);
    store(0, 0);
    __syncthreads();
    if constexpr (R == 1) {
      for (int s = 0; s < nst; ++s) {
        if (s + 1 < nst) load(0, s + 1);
        multiply(s & 1);
        if (s + 1 < nst) store(0, (s & 1) ^ 1);
        __syncthreads();
      }
    } else {
      // step s: refill set s % R (stage s is in LDS) with stage s + R, multiply
      // stage s from LDS buffer s % 2, then write stage s + 1 into the other buffer
      // (read by every wave in step s - 1, before the barrier that ended it). Steps
      // past the last stage only load and meet the barrier: every step issues the
      // same loads, so the waits stay exact across the loop's back edge.
      for (int st = 0; st < nst; st += R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int s = st + r;
          load(r, s + R);
          if (s < nst) {
            multiply(s & 1);
            if (s + 1 < nst) store((r + 1) % R, (s & 1) ^ 1);
          }
          __syncthreads();
        }
      }
      __builtin_amdgcn_s_waitcnt(0);   // the loads past the last stage
    }
  } else {
    __syncthreads();
  }

  // lane holds C[token m0 + 32(TM wt + t) + lane%32][weight row n0 + 32wn + 8(r/4) + 4(lane/32) + r%4]
  const bool split = !GROUPED && !kWide && partial != nullptr;   // the wide form is never split
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    int64_t m = m0 + 32 * (TM * wt + t) + (lane & 31);
    if (m >= M) continue;
    if constexpr (GROUPED) m = (MODE != kBf16Gated) ? grp.perm[rb + m] : rb + m;   // output row
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t n = n0 + 32 * wn + 8 * g + 4 * (lane >> 5);
      if (n >= N) continue;   // N % 4 == 0: the 4 rows are all in or all out
      if (split) {
#pragma unroll
        for (int j = 0; j < NW; ++j) {
          float* dst = partial + ((int64_t)blockIdx.z * NW + j) * M * N + m * N + n;
          *reinterpret_cast<f32x4*>(dst) =
              f32x4{acc[j][t][4 * g], acc[j][t][4 * g + 1], acc[j][t][4 * g + 2], acc[j][t][4 * g + 3]};
        }
      } else if constexpr (MODE == kBf16F32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + m * N + n) =
            f32x4{acc[0][t][4 * g], acc[0][t][4 * g + 1], acc[0][t][4 * g + 2], acc[0][t][4 * g + 3]};
      } else if constexpr (kWide) {
#pragma unroll
        for (int j = 0; j < NW; ++j) {
          if (n + j * BN >= N) continue;
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + m * N + n + j * BN) =
              f32x4{acc[j][t][4 * g], acc[j][t][4 * g + 1], acc[j][t][4 * g + 2], acc[j][t][4 * g + 3]};
        }
      } else {
        float h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) h[r] = silu(acc[0][t][4 * g + r]) * acc[NW - 1][t][4 * g + r];
        u32x2 o;
        o[0] = pack_bf16x2(h[0], h[1]);
        o[1] = pack_bf16x2(h[2], h[3]);
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + m * N + n) = o;
      }
    }
  }
}

// Sum of the splits in split order, then the epilogue of MODE. One thread: 4 outputs.
template <int MODE>
__global__ __launch_bounds__(256) void bf16_reduce_kernel(const float* __restrict__ partial, int splits, int64_t M,
                                                          int64_t N, void* __restrict__ out) {
  constexpr int NW = MODE == kBf16Gated ? 2 : 1;
  const int64_t u = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (u >= M * N) return;
  f32x4 s[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) s[j] = f32x4{0, 0, 0, 0};
  for (int z = 0; z < splits; ++z)
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(partial + ((int64_t)z * NW + j) * M * N + u);
#pragma unroll
      for (int r = 0; r < 4; ++r) s[j][r] += v[r];
    }
  if constexpr (MODE == kBf16F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + u) = s[0];
  } else {
    u32x2 o;
    o[0] = pack_bf16x2(silu(s[0][0]) * s[1][0], silu(s[0][1]) * s[1][1]);
    o[1] = pack_bf16x2(silu(s[0][2]) * s[1][2], silu(s[0][3]) * s[1][3]);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + u) = o;
  }
}

// Largest 64-bit key (hi, lo) over the wave, returned from lane 63: DPP shifts
// within rows of 16 and row broadcasts (lanes a shift reaches past a row's edge
// keep their own key).
template <int CTRL, int ROWS>
__device__ __forceinline__ void dpp_max_step(uint32_t& hi, uint32_t& lo) {
  const uint32_t h = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, ROWS, 0xF, false);
  const uint32_t l = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, ROWS, 0xF, false);
  const bool gt = h > hi || (h == hi && l > lo);
  hi = gt ? h : hi;
  lo = gt ? l : lo;
}
__device__ __forceinline__ void wave_max_key(uint32_t& hi, uint32_t& lo) {
  dpp_max_step<0x111, 0xF>(hi, lo);   // row_shr:1
  dpp_max_step<0x112, 0xF>(hi, lo);   // row_shr:2
  dpp_max_step<0x114, 0xF>(hi, lo);   // row_shr:4
  dpp_max_step<0x118, 0xF>(hi, lo);   // row_shr:8
  dpp_max_step<0x142, 0xA>(hi, lo);   // row_bcast:15
  dpp_max_step<0x143, 0xC>(hi, lo);   // row_bcast:31
  hi = (uint32_t)__builtin_amdgcn_readlane((int)hi, 63);
  lo = (uint32_t)__builtin_amdgcn_readlane((int)lo, 63);
}

// fp32 bits -> unsigned key of the same order (negatives below positives)
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Top-k of each row of fp32 logits (the sum of `splits` partial rows
// [splits][T][E], in split order), ties to the lower index, and the softmax over
// the selected. One wave per row: the row is summed once into LDS, then k rounds
// of a wave-wide arg-max run on it.
constexpr int kTopkMaxE = 4096;
constexpr int kMaxSplits = 16;   // the most K splits splits_for() makes
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ logits, int splits, int64_t T,
                                                           int E, int k, int32_t* __restrict__ ids,
                                                           float* __restrict__ w) {
  __shared__ float rows[4][kTopkMaxE];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wv;
  if (t >= T) return;   // whole wave: no barrier below
  float* row = rows[wv];
  for (int e = lane; e < E; e += 64) {
    float p[kMaxSplits];   // all split loads in flight together, then summed in split order
#pragma unroll
    for (int z = 0; z < kMaxSplits; ++z) p[z] = z < splits ? logits[(int64_t)z * T * E + t * E + e] : 0.0f;
    float v = p[0];
#pragma unroll
    for (int z = 1; z < kMaxSplits; ++z)
      if (z < splits) v += p[z];
    row[e] = v;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint64_t taken = 0;   // bit i: expert lane + 64 i already selected (E <= 4096)
  float sel_v = 0.0f, top = 0.0f, sum = 0.0f;
  int sel_e = 0;
  for (int r = 0; r < k; ++r) {
    // this lane's best remaining expert as a key (value order, then the lower
    // index), 0 if it has none; the wave's largest key is the round's pick
    uint32_t khi = 0, klo = 0;
    for (int i = 0, e = lane; e < E; ++i, e += 64) {
      if ((taken >> i) & 1) continue;
      const uint32_t h = ordered_bits(row[e]), l = ~(uint32_t)e;
      if (h > khi || (h == khi && l > klo)) {
        khi = h;
        klo = l;
      }
    }
    wave_max_key(khi, klo);
    const int be = (int)~klo;
    const float bv = __builtin_bit_cast(float, (khi & 0x80000000u) ? (khi & 0x7FFFFFFFu) : ~khi);
    if ((be & 63) == lane) taken |= 1ull << (be >> 6);
    if (r == 0) top = bv;
    const float p = expf(bv - top);
    sum += p;
    if (lane == r) {
      sel_v = p;
      sel_e = be;
    }
  }
  if (lane < k) {
    ids[t * k + lane] = sel_e;
    w[t * k + lane] = sel_v / sum;
  }
}

// ------------------------------------------------------------------ launchers
// Register sets of the K loop (see bf16_gemm_kernel): two for long loops (routed
// BF16 experts at 4096 tokens 3.96 -> 3.61 ms; three or four sets measured 3.68 and
// 3.65), one where a workgroup's K loop is short (the split-K products of small
// batches), which the re-reads past the last stage would cost more than they gain.
constexpr int kRing = 2;
static bool deep_ring(int64_t k_per_workgroup) { return k_per_workgroup / BK >= 12; }

static int splits_for(int64_t tiles, int64_t K) {
  // about two workgroups per CU in all; each split keeps >= 256 inputs
  if (tiles < 1) return 1;
  const int64_t want = (2 * (int64_t)cu_count() + tiles - 1) / tiles;
  const int64_t most = std::max<int64_t>(1, K / 256);
  return (int)std::max<int64_t>(1, std::min<int64_t>({want, most, (int64_t)kMaxSplits}));
}

size_t bf16_gemm_partial_bytes(int64_t M, int64_t N, int64_t K, bool gated) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int s = splits_for(tiles, K);
  return s > 1 ? (size_t)s * (gated ? 2 : 1) * (size_t)M * (size_t)N * sizeof(float) : 0;
}

int bf16_grouped_tile_rows(int64_t S, int64_t E) {
  const int64_t busy = S < E ? S : E;
  return (busy > 0 && S >= BM * busy) ? 2 * BM : BM;
}

hipError_t launch_bf16_grouped(bool gated, const uint16_t* x, const uint16_t* w0, const uint16_t* w1,
                               const int32_t* tiles, const int32_t* n_tiles, int64_t max_tiles, const int32_t* perm,
                               int topk, int64_t N, int64_t K, void* out, hipStream_t s, int tile_rows) {
  if (max_tiles <= 0) return hipSuccess;
  if (tile_rows != BM && tile_rows != 2 * BM) return hipErrorInvalidValue;
  const Bf16Group grp{tiles, n_tiles, perm, topk, N * K};
  // 128-row tiles: ceil(tiles / 8) * 8 tiles' worth of workgroups (the kernel maps them XCD by XCD)
  const int64_t gt = tile_rows == 2 * BM ? (max_tiles + 7) / 8 * 8 : max_tiles;
  // one-weight calls on 128-row tiles take 128 weight rows per workgroup (the wide form)
  const bool wide = !gated && tile_rows == 2 * BM;
  const dim3 grid((unsigned)gt, (unsigned)((N + (wide ? 2 : 1) * BN - 1) / ((wide ? 2 : 1) * BN)), 1u);
#define NVFP4_BF16G(MODE_, TM_, R_)                                                                                \
  hipLaunchKernelGGL((bf16_gemm_kernel<MODE_, true, TM_, R_>), grid, dim3(kThreads), 0, s, x, w0, w1, (int64_t)0, N, \
                     K, K, out, nullptr, grp)
  const bool deep = deep_ring(K);
  if (tile_rows == 2 * BM) {
    if (gated) { if (deep) NVFP4_BF16G(kBf16Gated, 2, kRing); else NVFP4_BF16G(kBf16Gated, 2, 1); }
    else { if (deep) NVFP4_BF16G(kBf16F32W, 2, kRing); else NVFP4_BF16G(kBf16F32W, 2, 1); }
  } else {
    if (gated) { if (deep) NVFP4_BF16G(kBf16Gated, 1, kRing); else NVFP4_BF16G(kBf16Gated, 1, 1); }
    else { if (deep) NVFP4_BF16G(kBf16F32, 1, kRing); else NVFP4_BF16G(kBf16F32, 1, 1); }
  }
#undef NVFP4_BF16G
  return hipGetLastError();
}

hipError_t launch_bf16_gemm(bool gated, const uint16_t* x, const uint16_t* w0, const uint16_t* w1, int64_t M,
                            int64_t N, int64_t K, void* out, float* partial, hipStream_t s, int* splits_left) {
  if (splits_left) *splits_left = 1;
  if (M <= 0) return hipSuccess;
  const int64_t gn = (N + BN - 1) / BN;
  // 128-row tiles where they still give one K split (at least two workgroups per CU)
  const int64_t gm2 = (M + 2 * BM - 1) / (2 * BM);
  if (M >= 4 * BM && splits_for(gm2 * gn, K) == 1) {
    // one-weight products take 128 weight rows per workgroup (the wide form)
    const dim3 grid2((unsigned)gm2, (unsigned)(gated ? gn : (N + 2 * BN - 1) / (2 * BN)), 1u);
    const Bf16Group none{};
#define NVFP4_BF16P(MODE_, R_)                                                                                     \
  hipLaunchKernelGGL((bf16_gemm_kernel<MODE_, false, 2, R_>), grid2, dim3(kThreads), 0, s, x, w0, w1, M, N, K, K, out, \
                     nullptr, none)
    const bool deep = deep_ring(K);
    if (gated) { if (deep) NVFP4_BF16P(kBf16Gated, kRing); else NVFP4_BF16P(kBf16Gated, 1); }
    else { if (deep) NVFP4_BF16P(kBf16F32W, kRing); else NVFP4_BF16P(kBf16F32W, 1); }
#undef NVFP4_BF16P
    return hipGetLastError();
  }
  const int64_t gm = (M + BM - 1) / BM;
  const int splits = splits_for(gm * gn, K);
  int64_t kps = (K / splits + BK - 1) / BK * BK;
  const int gz = (int)((K + kps - 1) / kps);
  float* part = gz > 1 ? partial : nullptr;
  const dim3 grid((unsigned)gm, (unsigned)gn, (unsigned)gz);
  const Bf16Group none{};
#define NVFP4_BF16S(MODE_, R_)                                                                                       \
  hipLaunchKernelGGL((bf16_gemm_kernel<MODE_, false, 1, R_>), grid, dim3(kThreads), 0, s, x, w0, w1, M, N, K, kps, out, \
                     part, none)
  const bool deep = deep_ring(kps);
  if (gated) { if (deep) NVFP4_BF16S(kBf16Gated, kRing); else NVFP4_BF16S(kBf16Gated, 1); }
  else { if (deep) NVFP4_BF16S(kBf16F32, kRing); else NVFP4_BF16S(kBf16F32, 1); }
#undef NVFP4_BF16S
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || gz == 1) return e;
  if (splits_left && !gated) {   // the consumer sums the fp32 splits itself
    *splits_left = gz;
    return e;
  }
  const unsigned rg = (unsigned)((M * N / 4 + 255) / 256);
  if (gated)
    hipLaunchKernelGGL(bf16_reduce_kernel<kBf16Gated>, dim3(rg), dim3(256), 0, s, part, gz, M, N, out);
  else
    hipLaunchKernelGGL(bf16_reduce_kernel<kBf16F32>, dim3(rg), dim3(256), 0, s, part, gz, M, N, out);
  return hipGetLastError();
}

hipError_t launch_topk_softmax(const float* logits, int splits, int64_t T, int E, int k, int32_t* ids, float* w,
                               hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_softmax_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, logits, splits, T, E, k,
                     ids, w);
  return hipGetLastError();
}

}  // namespace nvfp4
