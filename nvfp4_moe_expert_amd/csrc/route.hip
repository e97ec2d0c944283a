// Token permutation by expert, and the routing-weighted combine.
//
// route: one workgroup of 16 waves.
//   1. histogram of local expert ids, split into P slot ranges (LDS atomics:
//      counting is order-free); the lanes of a wave that hold the same expert
//      add their count with one atomic;
//   2. every thread owns a run of experts: it totals them over the ranges, a
//      workgroup prefix scan turns the totals into exclusive offsets, and the
//      owner turns its counts into a cursor per (range, expert) and writes its
//      part of the tile list (expert, first row, rows);
//   3. each range's wave walks its slots in order, 64 at a time: a slot's
//      rank among earlier lanes with the same expert plus that expert's cursor
//      is its position, so the order within an expert is slot order (stable).
//   The lanes holding the same expert are found with one ballot per bit of the
//   expert id (at most 13), not a pass over the 64 lanes.
// combine: y[t] = bf16(sum_j w[t,j] * Ypart[t*k+j]) over local slots, j in
// order - a fixed-order gather instead of a scatter-add, so results are
// bitwise reproducible (deterministic batch execution, as on the model card
// "GLM-5.3-Flash-NVFP4-W4A4-Experts", opening section).
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteLdsInts = 16384;   // per-(range, expert) counters: 64 KB

// Lanes of this wave whose value equals this lane's (v in [-1, 2^bits - 1]).
__device__ __forceinline__ uint64_t match_lanes(int v, int bits) {
  uint64_t m = __builtin_amdgcn_read_exec();
  const uint64_t neg = __builtin_amdgcn_ballot_w64(v < 0);
  m &= (v < 0) ? neg : ~neg;
  for (int b = 0; b < bits; ++b) {
    const bool bit = (v >> b) & 1;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  return v;
}

// Workgroups 1.. of the route kernel: one wave per activation row t -> fp16
// scaled by 2^p, p putting the row's max |x| in [2^14, 2^15) (bf16 values then
// convert exactly); also clears the row maxima of the token's k H rows. A wave
// reduces its row with shuffles alone, no barrier; a row of up to 4096 inputs is
// read once and held in registers (8 loads in flight per lane). A workgroup
// takes `rpb` rows (1..16): few rows per workgroup for small batches, so the
// rows spread over many compute units, 16 for large ones.
constexpr int kPrepRegChunks = 8;   // 512-input chunks of a row held in registers

__device__ __forceinline__ uint32_t absmax_bf16x8(const u32x4& v) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) m = max(m, max(v[j] & 0x7FFFu, (v[j] >> 16) & 0x7FFFu));
  return m;
}

__device__ __forceinline__ u32x4 to_f16_scaled(const u32x4& v, float sc) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const _Float16 lo = (_Float16)(bf16_lo(v[j]) * sc), hi = (_Float16)(bf16_hi(v[j]) * sc);
    o[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  return o;
}

// W4A4: the row's static NVFP4 quantization (threads 2j, 2j+1 hold one 16-block),
// stored as its unscaled values e2m1 * e4m3 in fp16 (exact); input_scale is
// applied in the GEMM epilogue, so the row exponent is 0. Thread `first` of
// `stride` (a multiple of 64).
__device__ void w4a4_row(const RoutePrep& pr, int64_t t, int first, int stride) {
  const uint16_t* xr = pr.x + t * pr.H;
  const float gs = *pr.act_scale;
  for (int64_t i = (int64_t)first * 8; i < pr.H; i += (int64_t)stride * 8) {
    const u32x4 v = ld16(xr + i);
    uint32_t am = absmax8(v);
    am = max(am, (uint32_t)__shfl_xor((int)am, 1));
    float s_eff;
    const uint32_t byte = block_byte(am, gs, s_eff);
    const _Float16 sv = (_Float16)e4m3_to_f32(byte);
    st16(pr.x16 + t * pr.H + i, __builtin_bit_cast(u32x4, dequant8_f16(quant8(v, s_eff), f16x2{sv, sv})));
  }
  if (first == 0) pr.xexp[t] = 0;
  for (int j = first; j < pr.k; j += stride) pr.hmax[t * pr.k + j] = 0u;
}

__device__ void prep_row(const RoutePrep& pr, int64_t t) {
  const int lane = threadIdx.x & 63;
  const uint16_t* xr = pr.x + t * pr.H;
  uint16_t* orow = pr.x16 + t * pr.H;
  if (pr.act_scale) {
    w4a4_row(pr, t, lane, 64);
    return;
  }
  const bool in_regs = pr.H <= 512 * kPrepRegChunks;
  u32x4 v[kPrepRegChunks];
  uint32_t m = 0;
  if (in_regs) {
#pragma unroll
    for (int c = 0; c < kPrepRegChunks; ++c) {
      const int64_t i = (int64_t)c * 512 + lane * 8;
      v[c] = i < pr.H ? ld16(xr + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int c = 0; c < kPrepRegChunks; ++c) m = max(m, absmax_bf16x8(v[c]));
  } else {
    for (int64_t i = (int64_t)lane * 8; i < pr.H; i += 512) m = max(m, absmax_bf16x8(ld16(xr + i)));
  }
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  int p = 0;
  if (m != 0) {
    const int e = (int)((m >> 7) & 0xFF) - 127;   // bf16 exponent of the row max
    p = 14 - e;
    p = p > 126 ? 126 : (p < -126 ? -126 : p);
  }
  if (lane == 0) pr.xexp[t] = p;
  const float sc = ldexpf(1.0f, p);
  if (in_regs) {
#pragma unroll
    for (int c = 0; c < kPrepRegChunks; ++c) {
      const int64_t i = (int64_t)c * 512 + lane * 8;
      if (i < pr.H) st16(orow + i, to_f16_scaled(v[c], sc));
    }
  } else {
    for (int64_t i = (int64_t)lane * 8; i < pr.H; i += 512) st16(orow + i, to_f16_scaled(ld16(xr + i), sc));
  }
  for (int j = lane; j < pr.k; j += 64) pr.hmax[t * pr.k + j] = 0u;
}

// ---- the three steps, over the slot window [s0, s1) of one workgroup

// 1. histogram of the window's local expert ids into cnt[P][E]: range p holds
// slots [s0 + p*chunk, +chunk) (chunk a multiple of 64, so a wave's 64 slots lie
// in one range). Ends with a barrier.
__device__ void range_hist(const int32_t* __restrict__ ids, int s0, int s1, int E, int eb, int P, int chunk,
                           int bits, int32_t* cnt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i = tid; i < P * E; i += kRouteThreads) cnt[i] = 0;
  __syncthreads();
  for (int base = s0 + wave * 64; base < s1; base += kRouteThreads) {
    const int s = base + lane;
    int e = -1;
    if (s < s1) {
      e = ids[s] - eb;
      if (e < 0 || e >= E) e = -1;
    }
    const uint64_t m = match_lanes(e, bits);
    if (e >= 0 && (m & below) == 0) atomicAdd(&cnt[((base - s0) / chunk) * E + e], __builtin_popcountll(m));
  }
  __syncthreads();
}

// 2. Given per-expert totals (total(e)), a workgroup scan gives the exclusive
// offsets, the tile list (expert, first row, rows) and the tile count; then
// cursors(e, first) is called once per expert with its first position.
template <typename Total, typename Cursors>
__device__ void scan_experts(int E, int tile_rows, Total total, Cursors cursors, int32_t* __restrict__ offsets,
                             int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
  __shared__ int wrows[kRouteWaves], wtl[kRouteWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int run = (E + kRouteThreads - 1) / kRouteThreads;
  const int e0 = min(tid * run, E), e1 = min(e0 + run, E);
  int rows = 0, ntl = 0;
  for (int e = e0; e < e1; ++e) {
    const int tot = total(e);
    rows += tot;
    ntl += (tot + tile_rows - 1) / tile_rows;
  }
  const int rows_incl = wave_incl_scan(rows, lane);
  const int tl_incl = wave_incl_scan(ntl, lane);
  if (lane == 63) {
    wrows[wave] = rows_incl;
    wtl[wave] = tl_incl;
  }
  __syncthreads();
  int rbase = 0, tbase = 0;
  for (int w = 0; w < wave; ++w) {
    rbase += wrows[w];
    tbase += wtl[w];
  }
  int off = rbase + rows_incl - rows, toff = tbase + tl_incl - ntl;
  for (int e = e0; e < e1; ++e) {
    offsets[e] = off;
    const int tot = cursors(e, off);
    if (tiles) {
      for (int r = 0; r < tot; r += tile_rows, ++toff) {
        tiles[4 * toff + 0] = e;
        tiles[4 * toff + 1] = off + r;
        tiles[4 * toff + 2] = min(tile_rows, tot - r);
        tiles[4 * toff + 3] = 0;
      }
    }
    off += tot;
  }
  if (tid == kRouteThreads - 1) {
    offsets[E] = rbase + rows_incl;
    if (n_tiles) *n_tiles = tbase + tl_incl;
  }
}

// counts cnt[p][e] -> cursors, range by range from `first`; returns the total
__device__ __forceinline__ int counts_to_cursors(int32_t* cnt, int P, int E, int e, int first) {
  int cur = first;
  for (int p = 0; p < P; ++p) {
    const int c = cnt[p * E + e];
    cnt[p * E + e] = cur;
    cur += c;
  }
  return cur - first;
}

// 3. stable scatter of the window: wave p < P walks range p in slot order; a
// slot's position is its expert's cursor plus its rank among earlier lanes of
// the same expert.
__device__ void range_scatter(const int32_t* __restrict__ ids, int s0, int s1, int E, int eb, int P, int chunk,
                              int bits, int32_t* cnt, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (wave >= P) return;
  const int r_begin = s0 + wave * chunk, r_end = min(s1, r_begin + chunk);
  for (int base = r_begin; base < r_end; base += 64) {
    const int s = base + lane;
    int e = -1;
    if (s < r_end) {
      e = ids[s] - eb;
      if (e < 0 || e >= E) e = -1;
    }
    const uint64_t m = match_lanes(e, bits);
    const int rank = __builtin_popcountll(m & below), tot = __builtin_popcountll(m);
    if (e >= 0) {
      const int pos = cnt[wave * E + e] + rank;
      perm[pos] = s;
      if (inv) inv[s] = pos;
    } else if (s < r_end && inv) {
      inv[s] = -1;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (e >= 0 && rank == tot - 1) cnt[wave * E + e] += tot;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
}

__device__ __forceinline__ int id_bits(int E) {
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  return bits;
}

// Small batches (rpb == 1): the whole workgroup converts one row, two passes (max,
// then convert) with a workgroup reduction between them; its loads spread over 16
// waves rather than queueing in one (a one-wave row cost ~1 us more per route).
__device__ void prep_row_wg(const RoutePrep& pr, int64_t t) {
  __shared__ uint32_t red[kRouteWaves];
  __shared__ int pexp;
  const int tid = threadIdx.x;
  if (pr.act_scale) {
    w4a4_row(pr, t, tid, kRouteThreads);
    return;
  }
  const uint16_t* xr = pr.x + t * pr.H;
  uint32_t m = 0;
  for (int64_t i = (int64_t)tid * 8; i < pr.H; i += kRouteThreads * 8) m = max(m, absmax_bf16x8(ld16(xr + i)));
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    uint32_t r = 0;
    for (int i = 0; i < kRouteWaves; ++i) r = max(r, red[i]);
    int p = 0;
    if (r != 0) {
      const int e = (int)((r >> 7) & 0xFF) - 127;   // bf16 exponent of the row max
      p = 14 - e;
      p = p > 126 ? 126 : (p < -126 ? -126 : p);
    }
    pexp = p;
    pr.xexp[t] = p;
  }
  __syncthreads();
  const float sc = ldexpf(1.0f, pexp);
  for (int64_t i = (int64_t)tid * 8; i < pr.H; i += kRouteThreads * 8)
    st16(pr.x16 + t * pr.H + i, to_f16_scaled(ld16(xr + i), sc));
  for (int j = tid; j < pr.k; j += kRouteThreads) pr.hmax[t * pr.k + j] = 0u;
}

__device__ __forceinline__ bool prep_block(const RoutePrep& prep, int64_t pb) {
  if (pb < 0) return false;
  if (prep.rpb == 1) {
    prep_row_wg(prep, pb);
    return true;
  }
  const int w = threadIdx.x >> 6;
  const int64_t t = pb * prep.rpb + w;
  if (w < prep.rpb && t < prep.T) prep_row(prep, t);
  return true;
}

// One workgroup routes all S slots (workgroups 1.. run the activation prep).
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const int32_t* __restrict__ ids, int S, int E, int eb, int P, int chunk, int tile_rows,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles, RoutePrep prep) {
  if (prep_block(prep, (int64_t)blockIdx.x - 1)) return;
  extern __shared__ int32_t cnt[];      // [P][E]
  const int bits = id_bits(E);
  range_hist(ids, 0, S, E, eb, P, chunk, bits, cnt);
  scan_experts(
      E, tile_rows,
      [&](int e) {
        int tot = 0;
        for (int p = 0; p < P; ++p) tot += cnt[p * E + e];
        return tot;
      },
      [&](int e, int first) { return counts_to_cursors(cnt, P, E, e, first); }, offsets, tiles, n_tiles);
  __syncthreads();
  range_scatter(ids, 0, S, E, eb, P, chunk, bits, cnt, perm, inv);
}

// Large batches: the same three steps over NB workgroups of C slots each (the
// single workgroup's ballot work grows with S and ran ~50 us at 32768 slots).
// count: workgroup b's per-expert totals -> wsum[b][E] (workgroups NB.. run the
// activation prep); scan: one workgroup turns them into offsets, the tile list
// and each workgroup's first position per expert (in place: wsum[b][e] becomes
// offsets[e] + the rows of expert e in workgroups < b); scatter: workgroup b
// recounts its window per range and scatters from those bases. Workgroup order
// then range order then slot order: the permutation stays stable.
__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(
    const int32_t* __restrict__ ids, int S, int E, int eb, int P, int chunk, int C, int NB,
    int32_t* __restrict__ wsum, RoutePrep prep) {
  if (prep_block(prep, (int64_t)blockIdx.x - NB)) return;
  extern __shared__ int32_t cnt[];      // [P][E]
  const int s0 = (int)blockIdx.x * C, s1 = min(S, s0 + C);
  range_hist(ids, s0, s1, E, eb, P, chunk, id_bits(E), cnt);
  for (int e = threadIdx.x; e < E; e += kRouteThreads) {
    int tot = 0;
    for (int p = 0; p < P; ++p) tot += cnt[p * E + e];
    wsum[(int64_t)blockIdx.x * E + e] = tot;
  }
}

__global__ __launch_bounds__(kRouteThreads) void route_scan_kernel(int E, int NB, int tile_rows,
                                                                   int32_t* __restrict__ wsum,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ tiles,
                                                                   int32_t* __restrict__ n_tiles) {
  scan_experts(
      E, tile_rows,
      [&](int e) {
        int tot = 0;
#pragma unroll 8
        for (int b = 0; b < NB; ++b) tot += wsum[(int64_t)b * E + e];
        return tot;
      },
      [&](int e, int first) {
        int cur = first;
        for (int b = 0; b < NB; ++b) {
          const int c = wsum[(int64_t)b * E + e];
          wsum[(int64_t)b * E + e] = cur;
          cur += c;
        }
        return cur - first;
      },
      offsets, tiles, n_tiles);
}

__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(
    const int32_t* __restrict__ ids, int S, int E, int eb, int P, int chunk, int C,
    const int32_t* __restrict__ wsum, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  extern __shared__ int32_t cnt[];      // [P][E]
  const int s0 = (int)blockIdx.x * C, s1 = min(S, s0 + C);
  const int bits = id_bits(E);
  range_hist(ids, s0, s1, E, eb, P, chunk, bits, cnt);
  for (int e = threadIdx.x; e < E; e += kRouteThreads)
    counts_to_cursors(cnt, P, E, e, wsum[(int64_t)blockIdx.x * E + e]);
  __syncthreads();
  range_scatter(ids, s0, s1, E, eb, P, chunk, bits, cnt, perm, inv);
}

namespace {
// ranges per workgroup (one wave each) and their length for a window of n slots
void route_ranges(int64_t n, int E, int& P, int64_t& chunk) {
  P = kRouteLdsInts / E;
  if (P > kRouteWaves) P = kRouteWaves;
  // no more ranges than 64-slot steps: every range costs a row of counters to
  // clear and a term in each expert's cursor sum
  const int64_t steps = (n + 63) / 64;
  if (P > steps) P = (int)steps;
  if (P < 1) P = 1;
  chunk = (n + P - 1) / P;
  chunk = ((chunk + 63) / 64) * 64;
  if (chunk < 64) chunk = 64;
}

// window of the multi-workgroup form: >= kRouteWindow slots, at most kRouteMaxWgs workgroups
constexpr int64_t kRouteSingleMax = 4096;   // slots one workgroup routes
constexpr int64_t kRouteWindow = 2048;
constexpr int64_t kRouteMaxWgs = 64;
int64_t route_window(int64_t S) {
  int64_t C = (S + kRouteMaxWgs - 1) / kRouteMaxWgs;
  C = ((C + 63) / 64) * 64;
  return C < kRouteWindow ? kRouteWindow : C;
}
}  // namespace

size_t route_scratch_bytes(int64_t S, int E) {
  if (S <= kRouteSingleMax) return 0;
  const int64_t NB = (S + route_window(S) - 1) / route_window(S);
  return sizeof(int32_t) * (size_t)NB * (size_t)E;
}

hipError_t launch_route(const int32_t* ids, int64_t S, int E, int eb, int tile_rows, int32_t* offsets,
                        int32_t* perm, int32_t* inv, int32_t* tiles, int32_t* n_tiles,
                        const RoutePrep& prep, hipStream_t s, int32_t* scratch, size_t scratch_bytes) {
  // rows per prep workgroup: one while that still leaves <= 256 workgroups, up to 16
  RoutePrep pp = prep;
  pp.rpb = (int)std::min<int64_t>(kRouteWaves, std::max<int64_t>(1, prep.T / 256));
  const int64_t prep_wgs = prep.x16 ? (prep.T + pp.rpb - 1) / pp.rpb : 0;
  const size_t need = route_scratch_bytes(S, E);
  if (need > 0 && scratch && scratch_bytes >= need) {
    const int64_t C = route_window(S), NB = (S + C - 1) / C;
    int P;
    int64_t chunk;
    route_ranges(C, E, P, chunk);
    const size_t lds = (size_t)P * E * sizeof(int32_t);
    hipLaunchKernelGGL(route_count_kernel, dim3((unsigned)(NB + prep_wgs)), dim3(kRouteThreads), lds, s, ids,
                       (int)S, E, eb, P, (int)chunk, (int)C, (int)NB, scratch, pp);
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kRouteThreads), 0, s, E, (int)NB, tile_rows, scratch,
                       offsets, tiles, n_tiles);
    hipLaunchKernelGGL(route_scatter_kernel, dim3((unsigned)NB), dim3(kRouteThreads), lds, s, ids, (int)S, E,
                       eb, P, (int)chunk, (int)C, scratch, perm, inv);
    return hipGetLastError();
  }
  int P;
  int64_t chunk;
  route_ranges(S, E, P, chunk);
  const size_t lds = (size_t)P * E * sizeof(int32_t);
  hipLaunchKernelGGL(route_kernel, dim3((unsigned)(1 + prep_wgs)), dim3(kRouteThreads), lds, s, ids, (int)S, E,
                     eb, P, (int)chunk, tile_rows, offsets, perm, inv, tiles, n_tiles, pp);
  return hipGetLastError();
}

// One thread: 8 outputs of one token. KM > 0 (k <= KM): the ids,
// weights and partial rows of all k slots are loaded before the sum, so the
// loads overlap; the sum runs over j in order either way.
// NT: the partials are read with non-temporal loads (large batches, whose partials
// do not stay in the caches: 4096 tokens 114 -> 108 us; at 64 tokens, where down
// has just written them into the caches, plain loads are faster, 7.0 against 7.9 us).
// WL (H % 512 == 0): the 64 threads of a wave take 512 columns of one token, lane l
// the 4 columns at 4l and the 4 at 256 + 4l, so that every 16-byte load and 8-byte
// store instruction of the wave covers whole 128-byte lines (each line once);
// otherwise a thread takes 8 consecutive columns, and each line is split over two
// load instructions.
template <int KM, bool NT, bool WL>
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ ids,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ ypart, int64_t T, int k,
                                                      int64_t H, int E, int eb, const float* __restrict__ extra,
                                                      int extra_splits, uint16_t* __restrict__ y) {
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_tok = H / 8;
  if (u >= T * per_tok) return;
  const int64_t t = u / per_tok, c8 = u % per_tok;
  const int64_t ca = WL ? (c8 / 64) * 512 + 4 * (c8 % 64) : 8 * c8;   // first and second group of 4
  const int64_t cb = WL ? ca + 256 : ca + 4;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (KM > 0) {
    // the partial rows are loaded before the ids are known (a skipped slot's row is
    // workspace of no meaning: it is loaded, then left out of the sum by a select),
    // so the two loads overlap instead of the partials waiting for the ids
    int id[KM];
    float wt[KM];
    f32x4 a[KM], b[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      id[j] = (j < k) ? ids[t * k + j] : eb - 1;
      wt[j] = (j < k) ? w[t * k + j] : 0.0f;
      a[j] = b[j] = f32x4{0, 0, 0, 0};
      if (j < k) {
        const float* row = ypart + (t * k + j) * H;
        const f32x4* pa = reinterpret_cast<const f32x4*>(row + ca);
        const f32x4* pb = reinterpret_cast<const f32x4*>(row + cb);
        if constexpr (NT) {
          a[j] = __builtin_nontemporal_load(pa);
          b[j] = __builtin_nontemporal_load(pb);
        } else {
          a[j] = *pa;
          b[j] = *pb;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const int e = id[j] - eb;
      if (e < 0 || e >= E) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += wt[j] * a[j][i];
        acc[4 + i] += wt[j] * b[j][i];
      }
    }
  } else {
    for (int j = 0; j < k; ++j) {
      const int64_t slot = t * k + j;
      const int e = ids[slot] - eb;
      if (e < 0 || e >= E) continue;
      const float wt = w[slot];
      const f32x4 a = *reinterpret_cast<const f32x4*>(ypart + slot * H + ca);
      const f32x4 b = *reinterpret_cast<const f32x4*>(ypart + slot * H + cb);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += wt * a[i];
        acc[4 + i] += wt * b[i];
      }
    }
  }
  if (extra) {   // a contribution summed after the routed slots (the shared expert)
    f32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
#pragma unroll 4
    for (int z = 0; z < extra_splits; ++z) {   // its K splits, in split order
      const float* ex = extra + (int64_t)z * T * H + t * H;
      const f32x4 p = *reinterpret_cast<const f32x4*>(ex + ca), q = *reinterpret_cast<const f32x4*>(ex + cb);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] += p[i];
        b[i] += q[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] += a[i];
      acc[4 + i] += b[i];
    }
  }
  u32x2 oa, ob;
  oa[0] = pack_bf16x2(acc[0], acc[1]);
  oa[1] = pack_bf16x2(acc[2], acc[3]);
  ob[0] = pack_bf16x2(acc[4], acc[5]);
  ob[1] = pack_bf16x2(acc[6], acc[7]);
  if constexpr (WL) {
    *reinterpret_cast<u32x2*>(y + t * H + ca) = oa;
    *reinterpret_cast<u32x2*>(y + t * H + cb) = ob;
  } else {
    st16(y + t * H + ca, u32x4{oa[0], oa[1], ob[0], ob[1]});
  }
}

hipError_t launch_combine(const int32_t* ids, const float* w, const float* ypart, int64_t T, int k,
                          int64_t H, int E, int eb, const float* extra, int extra_splits, uint16_t* y,
                          hipStream_t s) {
  const int64_t n = T * (H / 8);
  // small batches: one-wave workgroups, so the partials stream through the load
  // pipes of as many CUs as possible (one token: 8 CUs instead of 2)
  const int bs = n < 256 * 256 ? 64 : 256;
  const int64_t gx = (n + bs - 1) / bs;
  const bool nt = T * k * H * (int64_t)sizeof(float) > ((int64_t)128 << 20);   // partials beyond 128 MB
  const bool wl = H % 512 == 0;
#define NVFP4_CB(KM_, NT_, WL_) \
  hipLaunchKernelGGL((combine_kernel<KM_, NT_, WL_>), dim3((unsigned)gx), dim3(bs), 0, s, ids, w, ypart, T, k, H, E, \
                     eb, extra, extra_splits, y)
  if (k <= 8 && nt) {
    if (wl) NVFP4_CB(8, true, true); else NVFP4_CB(8, true, false);
  } else if (k <= 8) {
    if (wl) NVFP4_CB(8, false, true); else NVFP4_CB(8, false, false);
  } else {
    if (wl) NVFP4_CB(0, false, true); else NVFP4_CB(0, false, false);
  }
#undef NVFP4_CB
  return hipGetLastError();
}

}  // namespace nvfp4
