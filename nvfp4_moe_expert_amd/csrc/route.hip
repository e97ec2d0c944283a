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

// Workgroup 1 + t (t < T) of the route kernel: activation row t -> fp16 scaled by 2^p,
// p putting the row's max |x| in [2^14, 2^15) (bf16 values then convert exactly);
// also clears the row maxima of the token's k H rows.
__device__ void prep_row(const RoutePrep& pr, int64_t t) {
  __shared__ uint32_t red[kRouteThreads / 64];
  __shared__ int pexp;
  const int tid = threadIdx.x;
  const uint16_t* xr = pr.x + t * pr.H;
  if (pr.act_scale) {
    // W4A4: the row's static NVFP4 quantization (lanes 2j, 2j+1 hold one 16-block),
    // stored as its unscaled values e2m1 * e4m3 in fp16 (exact); input_scale is
    // applied in the GEMM epilogue, so the row exponent is 0
    const float gs = *pr.act_scale;
    for (int64_t i = (int64_t)tid * 8; i < pr.H; i += kRouteThreads * 8) {
      const u32x4 v = ld16(xr + i);
      uint32_t am = absmax8(v);
      am = max(am, (uint32_t)__shfl_xor((int)am, 1));
      float s_eff;
      const uint32_t byte = block_byte(am, gs, s_eff);
      const _Float16 sv = (_Float16)e4m3_to_f32(byte);
      st16(pr.x16 + t * pr.H + i, __builtin_bit_cast(u32x4, dequant8_f16(quant8(v, s_eff), f16x2{sv, sv})));
    }
    if (tid == 0) pr.xexp[t] = 0;
    for (int j = tid; j < pr.k; j += kRouteThreads) pr.hmax[t * pr.k + j] = 0u;
    return;
  }
  uint32_t m = 0;
  for (int64_t i = (int64_t)tid * 8; i < pr.H; i += kRouteThreads * 8) {
    const u32x4 v = ld16(xr + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, max(v[j] & 0x7FFFu, (v[j] >> 16) & 0x7FFFu));
  }
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    uint32_t r = 0;
    for (int i = 0; i < kRouteThreads / 64; ++i) r = max(r, red[i]);
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
  for (int64_t i = (int64_t)tid * 8; i < pr.H; i += kRouteThreads * 8) {
    const u32x4 v = ld16(xr + i);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const _Float16 lo = (_Float16)(bf16_lo(v[j]) * sc), hi = (_Float16)(bf16_hi(v[j]) * sc);
      o[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    st16(pr.x16 + t * pr.H + i, o);
  }
  for (int j = tid; j < pr.k; j += kRouteThreads) pr.hmax[t * pr.k + j] = 0u;
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const int32_t* __restrict__ ids, int S, int E, int eb, int P, int chunk, int tile_rows,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles, RoutePrep prep) {
  if (blockIdx.x > 0) {
    prep_row(prep, (int64_t)blockIdx.x - 1);
    return;
  }
  extern __shared__ int32_t cnt[];      // [P][E]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < P * E; i += kRouteThreads) cnt[i] = 0;
  __syncthreads();
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // 1. histogram per slot range; chunk is a multiple of 64, so a wave's 64 slots
  // lie in one range
  for (int base = wave * 64; base < S; base += kRouteThreads) {
    const int s = base + lane;
    int e = -1;
    if (s < S) {
      e = ids[s] - eb;
      if (e < 0 || e >= E) e = -1;
    }
    const uint64_t m = match_lanes(e, bits);
    if (e >= 0 && (m & below) == 0) atomicAdd(&cnt[(base / chunk) * E + e], __builtin_popcountll(m));
  }
  __syncthreads();
  // 2. per-expert totals, workgroup scan, cursors and tile list
  {
    __shared__ int wrows[kRouteWaves], wtl[kRouteWaves];
    const int run = (E + kRouteThreads - 1) / kRouteThreads;
    const int e0 = min(tid * run, E), e1 = min(e0 + run, E);
    int rows = 0, ntl = 0;
    for (int e = e0; e < e1; ++e) {
      int tot = 0;
      for (int p = 0; p < P; ++p) tot += cnt[p * E + e];
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
      int cur = off;
      for (int p = 0; p < P; ++p) {   // counts -> cursors, range by range
        const int c = cnt[p * E + e];
        cnt[p * E + e] = cur;
        cur += c;
      }
      const int tot = cur - off;
      if (tiles) {
        for (int r = 0; r < tot; r += tile_rows, ++toff) {
          tiles[4 * toff + 0] = e;
          tiles[4 * toff + 1] = off + r;
          tiles[4 * toff + 2] = min(tile_rows, tot - r);
          tiles[4 * toff + 3] = 0;
        }
      }
      off = cur;
    }
    if (tid == kRouteThreads - 1) {
      offsets[E] = rbase + rows_incl;
      if (n_tiles) *n_tiles = tbase + tl_incl;
    }
  }
  __syncthreads();
  // 3. stable scatter, one wave per slot range
  if (wave < P) {
    const int s_begin = wave * chunk, s_end = min(S, s_begin + chunk);
    for (int base = s_begin; base < s_end; base += 64) {
      const int s = base + lane;
      int e = -1;
      if (s < s_end) {
        e = ids[s] - eb;
        if (e < 0 || e >= E) e = -1;
      }
      const uint64_t m = match_lanes(e, bits);
      const int rank = __builtin_popcountll(m & below), tot = __builtin_popcountll(m);
      if (e >= 0) {
        const int pos = cnt[wave * E + e] + rank;
        perm[pos] = s;
        if (inv) inv[s] = pos;
      } else if (s < s_end && inv) {
        inv[s] = -1;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (e >= 0 && rank == tot - 1) cnt[wave * E + e] += tot;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
  }
}

hipError_t launch_route(const int32_t* ids, int64_t S, int E, int eb, int tile_rows, int32_t* offsets,
                        int32_t* perm, int32_t* inv, int32_t* tiles, int32_t* n_tiles,
                        const RoutePrep& prep, hipStream_t s) {
  int P = kRouteLdsInts / E;
  if (P > kRouteWaves) P = kRouteWaves;
  if (P < 1) P = 1;
  int64_t chunk = (S + P - 1) / P;
  chunk = ((chunk + 63) / 64) * 64;
  if (chunk < 64) chunk = 64;
  const size_t lds = (size_t)P * E * sizeof(int32_t);
  const unsigned grid = 1 + (prep.x16 ? (unsigned)prep.T : 0u);
  hipLaunchKernelGGL(route_kernel, dim3(grid), dim3(kRouteThreads), lds, s, ids, (int)S, E, eb, P,
                     (int)chunk, tile_rows, offsets, perm, inv, tiles, n_tiles, prep);
  return hipGetLastError();
}

// One thread: 8 consecutive outputs of one token. KM > 0 (k <= KM): the ids,
// weights and partial rows of all k slots are loaded before the sum, so the
// loads overlap; the sum runs over j in order either way.
template <int KM>
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ ids,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ ypart, int64_t T, int k,
                                                      int64_t H, int E, int eb, const float* __restrict__ extra,
                                                      int extra_splits, uint16_t* __restrict__ y) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_tok = H / 8;
  if (u >= T * per_tok) return;
  const int64_t t = u / per_tok, c8 = u % per_tok;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (KM > 0) {
    bool ok[KM];
    float wt[KM];
    f32x4 a[KM], b[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const int e = (j < k) ? ids[t * k + j] - eb : -1;
      ok[j] = e >= 0 && e < E;
      wt[j] = ok[j] ? w[t * k + j] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      a[j] = b[j] = f32x4{0, 0, 0, 0};
      if (ok[j]) {
        const f32x4* src = reinterpret_cast<const f32x4*>(ypart + (t * k + j) * H + c8 * 8);
        a[j] = src[0];
        b[j] = src[1];
      }
    }
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (!ok[j]) continue;
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
      const f32x4* src = reinterpret_cast<const f32x4*>(ypart + slot * H + c8 * 8);
      const f32x4 a = src[0], b = src[1];
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
      const f32x4* ex = reinterpret_cast<const f32x4*>(extra + (int64_t)z * T * H + t * H + c8 * 8);
      const f32x4 p = ex[0], q = ex[1];
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
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
  st16(y + t * H + c8 * 8, o);
}

hipError_t launch_combine(const int32_t* ids, const float* w, const float* ypart, int64_t T, int k,
                          int64_t H, int E, int eb, const float* extra, int extra_splits, uint16_t* y,
                          hipStream_t s) {
  const int64_t n = T * (H / 8);
  const int64_t gx = (n + 255) / 256;
  if (k <= 8)
    hipLaunchKernelGGL(combine_kernel<8>, dim3((unsigned)gx), dim3(256), 0, s, ids, w, ypart, T, k, H, E, eb, extra, extra_splits, y);
  else
    hipLaunchKernelGGL(combine_kernel<0>, dim3((unsigned)gx), dim3(256), 0, s, ids, w, ypart, T, k, H, E, eb, extra, extra_splits, y);
  return hipGetLastError();
}

}  // namespace nvfp4
