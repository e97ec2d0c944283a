// C ABI of the NVFP4 expert library: host-side validation, workspace layout and
// launch orchestration. The declarations and the contract are in include/nvfp4.h.
//
// No entry point allocates, frees, synchronizes, copies to the host, or changes
// the current device; everything is enqueued on the caller's stream. Every
// argument check runs before the first launch, so an error writes nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "../../include/nvfp4.h"
#include "launch.hpp"

using namespace nvfp4;

// Scratch of nvfp4_moe_grouped_noalloc: one fixed array in device memory. Every
// GPU that runs this library holds its own copy, at its own address, until the
// process ends. On the host the name is only a stand-in: its device address is
// looked up once per device and kept (noalloc_scratch below), and only that
// address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device (with it current) and kept.
hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}


constexpr int64_t kMaxExperts = 4096;
constexpr int kMaxTopk = 64;
constexpr int64_t kMaxSlots = (int64_t)1 << 30;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t v) { return (v + 255) & ~(size_t)255; }

nvfp4_status check_weight(const nvfp4_weight_t* w) {
  if (!w || !w->codes || !w->scales || !w->scale_2) return NVFP4_ERR_NULL;
  if (w->n < 1 || w->k < 32 || (w->k % 32) != 0 || w->groups < 1) return NVFP4_ERR_SHAPE;
  // grid.y of the GEMM counts 64-row blocks of n (<= 65535); dequant grid < 2^31 blocks
  if (w->n > (int64_t)64 * 65535 || w->k > ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  if ((int64_t)w->groups * w->n * (w->k / 8) / 256 >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  if (w->layout != NVFP4_LAYOUT_ROWS && w->layout != NVFP4_LAYOUT_TILED32) return NVFP4_ERR_SHAPE;
  if (w->layout == NVFP4_LAYOUT_TILED32 && (w->n % 32 != 0 || w->k % 256 != 0)) return NVFP4_ERR_SHAPE;
  if (!aligned16(w->codes) || !aligned16(w->scales)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

WeightDev dev_weight(const nvfp4_weight_t* w) {
  return WeightDev{w->codes, w->scales, w->scale_2, w->layout == NVFP4_LAYOUT_TILED32 ? 1 : 0};
}

// Which GEMM kernel runs a projection: the decode-tile weight stream, the
// prefill-tile matrix-core kernel, or the tiled fallback (row-major weights
// only). Tiled weights take the prefill kernel wherever the decode kernel does
// not apply; kNone if no kernel covers the call.
enum Kern { kKDec, kKPre, kKV1, kKNone, kKDecS, kKTiny };
Kern pick(GemmMode mode, GemmVariant v, bool tiled, int64_t x_rows, int64_t K, int64_t N) {
  // tiny batches: gate/up splits K over the waves (its 8 stages of 512 inputs are the
  // long pole); down (few stages) keeps the decode kernels, on the same 4-row tiles
  if (v == kDecodeSmall) return mode == kGateUp ? kKDecS : (decode_supported(mode, K, N) ? kKDec : kKV1);
  if (v == kDecode && decode_supported(mode, K, N)) return kKDec;
  if ((v == kPrefill || tiled) && prefill_supported(mode, x_rows, K, N)) return kKPre;
  return tiled ? kKNone : kKV1;
}

nvfp4_status from_hip(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

// Workspace of nvfp4_moe_grouped, in order: offsets[E+1], perm[S], tiles[tile_cap][4],
// n_tiles, H[S][I] bf16, Ypart[S][H] fp32, x16[T][H] fp16, xexp[T], hmax[S].
// Each region starts on a 256-byte boundary.
struct MoeLayout {
  size_t offsets, perm, tiles, n_tiles, h, ypart, x16, xexp, hmax, total;
};

// Kernel class of the routed GEMMs, which fixes the tile shape and with it the
// summation order of every output. NVFP4_CLASS_AUTO: decode tiles (16 rows) when the
// average local expert gets at most 16 rows, else prefill tiles; for at most 32
// slots, 4-row tiles with gate/up's K split over the waves (when the shapes fit).
GemmVariant moe_variant(int64_t S, int64_t E, int64_t H, int64_t I, int cls) {
  if (cls == NVFP4_CLASS_DECODE) return kDecode;
  if (cls == NVFP4_CLASS_PREFILL) return kPrefill;
  const int64_t busy = S < E ? S : E;
  if (S <= 32 && decode_small_supported(H, I) && decode_supported(kDown, I, H)) return kDecodeSmall;
  return (busy > 0 && S <= 16 * busy) ? kDecode : kPrefill;
}

// Tiles of at most tr rows over S slots and E experts: sum over experts of
// ceil(rows/tr) <= floor(S/tr) + (number of non-empty experts).
int64_t tile_bound(int64_t S, int64_t E, int64_t tr) { return S / tr + (S < E ? S : E); }

MoeLayout moe_layout(int64_t T, int k, int64_t E, int64_t H, int64_t I) {
  MoeLayout L{};
  const int64_t S = T * k;
  // room for the smallest tiles (4 rows), so the same workspace serves every class
  const int64_t cap = tile_bound(S, E, variant_tile_rows(kDecodeSmall));
  size_t off = 0;
  L.offsets = off; off += round_up(sizeof(int32_t) * (size_t)(E + 1));
  L.perm = off;    off += round_up(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
  L.tiles = off;   off += round_up(sizeof(int32_t) * 4 * (size_t)(cap > 0 ? cap : 1));
  L.n_tiles = off; off += 256;
  L.h = off;       off += round_up(sizeof(uint16_t) * (size_t)S * (size_t)I);
  L.ypart = off;   off += round_up(sizeof(float) * (size_t)S * (size_t)H);
  L.x16 = off;     off += round_up(sizeof(uint16_t) * (size_t)T * (size_t)H);
  L.xexp = off;    off += round_up(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  L.hmax = off;    off += round_up(sizeof(uint32_t) * (size_t)(S > 0 ? S : 1));
  L.total = off;
  return L;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off);
}

// The kernels one routed call runs, decided on the host from the shapes alone.
struct MoePlan {
  GemmVariant v;
  Kern kg, kd;             // gate/up and down kernels
  bool f16;                // fp16 form of the routed GEMMs
  int64_t S, E, I;
  int64_t grid_tiles;      // tile-list bound of the class's tile rows
  MoeLayout L;
};

// Shapes and kernel choice of a routed call (no pointers looked at).
nvfp4_status moe_shape_plan(int64_t T, int64_t H, int32_t k, int64_t E, int64_t I, bool gate_tiled, bool down_tiled,
                            bool w4a4, int cls, MoePlan& P) {
  if (T < 0 || k < 1 || k > kMaxTopk || E < 1 || E > kMaxExperts) return NVFP4_ERR_SHAPE;
  if (cls != NVFP4_CLASS_AUTO && cls != NVFP4_CLASS_DECODE && cls != NVFP4_CLASS_PREFILL) return NVFP4_ERR_UNSUPPORTED;
  if (T * (int64_t)k > kMaxSlots) return NVFP4_ERR_SHAPE;
  P.S = T * k;
  P.E = E;
  P.I = I;
  P.v = moe_variant(P.S, E, H, I, cls);
  P.kg = pick(kGateUp, P.v, gate_tiled, T, H, I);
  P.kd = pick(kDown, P.v, down_tiled, P.S, I, H);
  // at most 24 slots (automatic class, W4A16): the two-launch path without a route
  // kernel. Its gate/up workgroups each derive the tile list and stage their
  // activation slices, a fixed cost per workgroup that outweighs the route kernel
  // it saves once the grid takes about three rounds of the device (32 slots of
  // 4096 x 1536 experts: 78 against 74 us a step).
  if (cls == NVFP4_CLASS_AUTO && !w4a4 && P.v == kDecodeSmall && P.S <= 24 && tiny_supported(T, k, H, I))
    P.kg = P.kd = kKTiny;
  if (T > 0 && (P.kg == kKNone || P.kd == kKNone)) return NVFP4_ERR_SHAPE;
  // a prefill-tile gate/up records no row maxima of H, which a decode-tile down
  // (fp16 form) needs; the class rules never pair the two (their shape conditions exclude it)
  if (T > 0 && P.kg == kKPre && (P.kd == kKDec || P.kd == kKDecS)) return NVFP4_ERR_UNSUPPORTED;
  // W4A4 runs on the fp16 form (quantized activations are exact in fp16), which
  // the decode and prefill kernels provide
  if (w4a4 && T > 0 && (P.kg == kKV1 || P.kd == kKV1)) return NVFP4_ERR_UNSUPPORTED;
  // fp16 form of the routed GEMMs (x16 and H rows scaled per row by a power of two)
  // when the decode or prefill kernels run both projections
  P.f16 = P.kg != kKV1 && P.kd != kKV1;
  P.grid_tiles = tile_bound(P.S, E, variant_tile_rows(P.v));
  P.L = moe_layout(T, k, E, H, I);
  return NVFP4_OK;
}

// Every argument check of a routed call, before anything is enqueued.
nvfp4_status moe_check(const uint16_t* x, int64_t T, int64_t H, const int32_t* ids, const float* tw, int32_t k,
                       const nvfp4_weight_t* gate, const nvfp4_weight_t* up, const nvfp4_weight_t* down,
                       const uint16_t* y, const void* ws, size_t ws_bytes, bool w4a4, int cls, MoePlan& P,
                       bool fixed_scratch = false) {
  nvfp4_status st;
  if ((st = check_weight(gate)) != NVFP4_OK) return st;
  if ((st = check_weight(up)) != NVFP4_OK) return st;
  if ((st = check_weight(down)) != NVFP4_OK) return st;
  const int64_t E = gate->groups, I = gate->n;
  if (gate->k != H || up->k != H || up->n != I || up->groups != E) return NVFP4_ERR_SHAPE;
  if (down->groups != E || down->n != H || down->k != I) return NVFP4_ERR_SHAPE;
  if (gate->layout != up->layout) return NVFP4_ERR_SHAPE;
  if (T < 0 || k < 1 || k > kMaxTopk || E > kMaxExperts || T * (int64_t)k > kMaxSlots) return NVFP4_ERR_SHAPE;
  if (T > 0 && (!x || !ids || !tw || !y)) return NVFP4_ERR_NULL;
  if (T > 0 && (!aligned16(x) || !aligned16(y))) return NVFP4_ERR_ALIGN;
  if (T > 0 && fixed_scratch) {
    // the no-allocation entry point: its fixed scratch must hold the workspace
    if (moe_layout(T, k, E, H, I).total > ws_bytes) return NVFP4_ERR_SCRATCH;
  } else if (T > 0) {
    if (!ws) return NVFP4_ERR_WORKSPACE;
    if (!aligned16(ws)) return NVFP4_ERR_ALIGN;
    if (ws_bytes < moe_layout(T, k, E, H, I).total) return NVFP4_ERR_WORKSPACE;
  }
  return moe_shape_plan(T, H, k, E, I, gate->layout == NVFP4_LAYOUT_TILED32, down->layout == NVFP4_LAYOUT_TILED32,
                        w4a4, cls, P);
}

// The launches of a checked routed call. in_gu / in_d: null for W4A16; for W4A4 the
// device pointers of the two calibrated activation input scales (gate/up input x,
// down input H). extra: fp32 terms added by the combine after the k slots.
nvfp4_status moe_run(const MoePlan& P, const uint16_t* x, int64_t T, int64_t H, const int32_t* ids, const float* tw,
                     int32_t k, int32_t eb, const nvfp4_weight_t* gate, const nvfp4_weight_t* up,
                     const nvfp4_weight_t* down, void* ws, uint16_t* y, hipStream_t s, void* const* events,
                     const float* in_gu = nullptr, const float* in_d = nullptr, const float* extra = nullptr,
                     int extra_splits = 1) {
  const bool w4a4 = in_gu || in_d;
  const MoeLayout& L = P.L;
  const int64_t S = P.S, E = P.E, I = P.I;
  const Kern kg = P.kg, kd = P.kd;
  const GemmVariant v = P.v;
  hipEvent_t ev[5] = {};
  if (events)
    for (int i = 0; i < 5; ++i) ev[i] = reinterpret_cast<hipEvent_t>(events[i]);
  auto mark = [&](int i) -> hipError_t { return events ? hipEventRecord(ev[i], s) : hipSuccess; };
  hipError_t e = mark(0);
  if (T == 0) {
    for (int i = 1; i < 5 && e == hipSuccess; ++i) e = mark(i);
    return from_hip(e);
  }
  if (kg == kKTiny) {
    // no route stage; the combine runs inside the down launch
    TinyArgs ta{x, ids, tw, T, k, (int)E, eb, H, I, dev_weight(gate), dev_weight(up), dev_weight(down),
                at<uint16_t>(ws, L.h), at<uint32_t>(ws, L.ypart), extra, extra_splits, y};
    if (e == hipSuccess) e = mark(1);
    if (e == hipSuccess) e = launch_tiny(ta, false, s);
    if (e == hipSuccess) e = mark(2);
    if (e == hipSuccess) e = launch_tiny(ta, true, s);
    if (e == hipSuccess) e = mark(3);
    if (e == hipSuccess) e = mark(4);
    return from_hip(e);
  }
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* perm = at<int32_t>(ws, L.perm);
  int32_t* tiles = at<int32_t>(ws, L.tiles);
  int32_t* n_tiles = at<int32_t>(ws, L.n_tiles);
  uint16_t* hbuf = at<uint16_t>(ws, L.h);
  float* ypart = at<float>(ws, L.ypart);
  const bool f16 = P.f16;
  F16Args dx{at<uint16_t>(ws, L.x16), at<int32_t>(ws, L.xexp), at<uint32_t>(ws, L.hmax)};
  RoutePrep prep{};
  if (f16)
    prep = RoutePrep{x, T, H, k, at<uint16_t>(ws, L.x16), at<int32_t>(ws, L.xexp), at<uint32_t>(ws, L.hmax), in_gu};

  if (e == hipSuccess)
    // Ypart is not written before down: it holds the route's scratch meanwhile
    e = launch_route(ids, S, (int)E, eb, variant_tile_rows(v), offsets, perm, nullptr, tiles, n_tiles, prep, s,
                     at<int32_t>(ws, L.ypart), L.x16 - L.ypart);
  if (e == hipSuccess) e = mark(1);

  GemmArgs g{};
  g.perm = perm;
  g.topk = k;
  g.tiles = tiles;
  g.n_tiles = n_tiles;
  if (e == hipSuccess) {
    g.x = (f16 && kg == kKPre) ? dx.x16 : x;
    g.x_rows = T;
    g.w0 = dev_weight(gate);
    g.w1 = dev_weight(up);
    g.N = I;
    g.K = H;
    g.out = hbuf;
    g.act_scale = in_gu;
    e = kg == kKDecS  ? launch_decode_small(kGateUp, g, dx, P.grid_tiles, s)
        : kg == kKDec ? launch_decode(kGateUp, f16, g, dx, P.grid_tiles, s)
        : kg == kKPre ? launch_prefill(kGateUp, f16, g, dx, P.grid_tiles, s)
                      : launch_gemm(kGateUp, v, g, P.grid_tiles, s);
  }
  // W4A4: H quantized in place (its row maxima replace the ones gate/up recorded)
  if (e == hipSuccess && w4a4) e = launch_act_fakequant_rows(hbuf, dx.hmax, S, I, in_d, s);
  if (e == hipSuccess) e = mark(2);
  if (e == hipSuccess) {
    g.x = hbuf;
    g.x_rows = S;
    g.w0 = dev_weight(down);
    g.w1 = WeightDev{nullptr, nullptr, nullptr, 0};
    g.N = H;
    g.K = I;
    g.out = ypart;
    g.act_scale = in_d;
    e = kd == kKDecS  ? launch_decode_small(kDown, g, dx, P.grid_tiles, s)
        : kd == kKDec ? launch_decode(kDown, f16, g, dx, P.grid_tiles, s)
        // prefill down takes H in bf16: its fp16 form would need H converted in place
        // first, a pass over H that costs more than the fp16 operands save (the
        // decode kernels convert while staging)
        : kd == kKPre ? launch_prefill(kDown, false, g, dx, P.grid_tiles, s)
                      : launch_gemm(kDown, v, g, P.grid_tiles, s);
  }
  if (e == hipSuccess) e = mark(3);
  if (e == hipSuccess) e = launch_combine(ids, tw, ypart, T, k, H, (int)E, eb, extra, extra_splits, y, s);
  if (e == hipSuccess) e = mark(4);
  return from_hip(e);
}

// A whole routed call: checks, then launches.
nvfp4_status moe_impl(const uint16_t* x, int64_t T, int64_t H, const int32_t* ids, const float* tw, int32_t k,
                      int32_t eb, const nvfp4_weight_t* gate, const nvfp4_weight_t* up, const nvfp4_weight_t* down,
                      void* ws, size_t ws_bytes, uint16_t* y, hipStream_t s, void* const* events,
                      const float* in_gu, const float* in_d, int cls) {
  const bool w4a4 = in_gu || in_d;
  if (w4a4 && !(in_gu && in_d)) return NVFP4_ERR_NULL;
  MoePlan P{};
  const nvfp4_status st = moe_check(x, T, H, ids, tw, k, gate, up, down, y, ws, ws_bytes, w4a4, cls, P);
  if (st != NVFP4_OK) return st;
  if (events)
    for (int i = 0; i < 5; ++i)
      if (!events[i]) return NVFP4_ERR_NULL;
  return moe_run(P, x, T, H, ids, tw, k, eb, gate, up, down, ws, y, s, events, in_gu, in_d);
}

// Plan entries (include/nvfp4.h, nvfp4_moe_plan) of a gate/up or down kernel.
int32_t kernel_id(Kern kn, bool down, const MoePlan& P, int64_t H, int32_t* detail) {
  *detail = 0;
  switch (kn) {
    case kKDecS: return NVFP4_KERNEL_DECODE_KSPLIT;
    case kKTiny: return NVFP4_KERNEL_TINY;
    case kKDec:
      if (down) {
        if (const int nb = decode_down_streams(P.f16, P.S, P.I, H, P.grid_tiles)) {
          *detail = nb;
          return NVFP4_KERNEL_DECODE_RESIDENT;
        }
      }
      return NVFP4_KERNEL_DECODE;
    case kKPre:
      *detail = prefill_weight_blocks(down ? kDown : kGateUp, down ? H : P.I, P.grid_tiles);
      return NVFP4_KERNEL_PREFILL;
    case kKV1: return NVFP4_KERNEL_FALLBACK;
    case kKNone: break;
  }
  return NVFP4_KERNEL_NONE;
}

// ---- BF16 steps either side of the routed experts
struct BlockLayout {
  size_t logits, ids, w, hs, ys, part, moe, total;
};

size_t part_bytes(int64_t T, int64_t E, int64_t H, int64_t Is) {
  return std::max({bf16_gemm_partial_bytes(T, E, H, false), bf16_gemm_partial_bytes(T, Is, H, true),
                   bf16_gemm_partial_bytes(T, H, Is, false), (size_t)256});
}

BlockLayout block_layout(int64_t T, int k, int64_t E, int64_t H, int64_t I, int64_t Is) {
  BlockLayout L{};
  size_t off = 0;
  L.logits = off; off += round_up(sizeof(float) * (size_t)(T * E > 0 ? T * E : 1));
  L.ids = off;    off += round_up(sizeof(int32_t) * (size_t)(T * k > 0 ? T * k : 1));
  L.w = off;      off += round_up(sizeof(float) * (size_t)(T * k > 0 ? T * k : 1));
  L.hs = off;     off += round_up(sizeof(uint16_t) * (size_t)(T * Is > 0 ? T * Is : 1));
  L.ys = off;     off += round_up(sizeof(float) * (size_t)(T * H > 0 ? T * H : 1));
  L.part = off;   off += round_up(part_bytes(T, E, H, Is));
  L.moe = off;    off += moe_layout(T, k, E, H, I).total;
  L.total = off;
  return L;
}

bool bf16_shape_ok(int64_t N, int64_t K) { return N >= 4 && N % 4 == 0 && K >= 64 && K % 64 == 0; }

nvfp4_status linear_impl(const uint16_t* x, int64_t m, const nvfp4_weight_t* w0,
                         const nvfp4_weight_t* w1, uint16_t* out, hipStream_t s) {
  nvfp4_status st;
  if ((st = check_weight(w0)) != NVFP4_OK) return st;
  if (w1) {
    if ((st = check_weight(w1)) != NVFP4_OK) return st;
    if (w1->n != w0->n || w1->k != w0->k || w1->groups != 1) return NVFP4_ERR_SHAPE;
  }
  if (w0->groups != 1 || m < 0 || m > kMaxSlots) return NVFP4_ERR_SHAPE;
  if (m == 0) return NVFP4_OK;
  if (!x || !out) return NVFP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(out)) return NVFP4_ERR_ALIGN;
  if (w1 && w1->layout != w0->layout) return NVFP4_ERR_SHAPE;
  const GemmVariant v = m <= 16 ? kDecode : kPrefill;
  const GemmMode mode = w1 ? kGated : kLinear;
  const Kern kn = pick(mode, v, w0->layout == NVFP4_LAYOUT_TILED32, m, w0->k, w0->n);
  if (kn == kKNone) return NVFP4_ERR_SHAPE;
  GemmArgs g{};
  g.x = x;
  g.M = m;
  g.x_rows = m;
  g.w0 = dev_weight(w0);
  if (w1) g.w1 = dev_weight(w1);
  g.N = w0->n;
  g.K = w0->k;
  g.out = out;
  if (kn == kKDec) return from_hip(launch_decode(mode, false, g, F16Args{}, 1, s));
  const int64_t tr = variant_tile_rows(kn == kKPre ? kPrefill : v);
  if (kn == kKPre) return from_hip(launch_prefill(mode, false, g, F16Args{}, (m + tr - 1) / tr, s));
  return from_hip(launch_gemm(mode, v, g, (m + tr - 1) / tr, s));
}

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "inconsistent or unsupported sizes";
    case NVFP4_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_UNSUPPORTED: return "unsupported request (a kernel class, or a W4A4 call on shapes only the fallback GEMM covers)";
    case NVFP4_ERR_HIP: return "HIP runtime error while enqueueing";
    case NVFP4_ERR_SCRATCH:
      return "the call needs more scratch than the no-allocation entry point's fixed buffer holds";
  }
  return "unknown status";
}

size_t nvfp4_pack_workspace_size(int32_t batch, int64_t n, int64_t k) {
  if (batch < 1 || n < 1 || k < 32) return 0;
  return sizeof(uint32_t) * (size_t)batch * (size_t)pack_nblk(n * k);
}

nvfp4_status nvfp4_pack(const uint16_t* w, int32_t batch, int64_t n, int64_t k, uint8_t* codes,
                        uint8_t* scales, float* scale_2, void* ws, size_t ws_bytes, int32_t layout,
                        void* stream) {
  if (batch < 1 || batch > 65535 || n < 1 || k < 32 || (k % 32) != 0) return NVFP4_ERR_SHAPE;
  if (layout != NVFP4_LAYOUT_ROWS && layout != NVFP4_LAYOUT_TILED32) return NVFP4_ERR_SHAPE;
  if (layout == NVFP4_LAYOUT_TILED32 && (n % 32 != 0 || k % 256 != 0)) return NVFP4_ERR_SHAPE;
  if (n * k / 32 > ((int64_t)1 << 38)) return NVFP4_ERR_SHAPE;
  if (!w || !codes || !scales || !scale_2) return NVFP4_ERR_NULL;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales)) return NVFP4_ERR_ALIGN;
  if (!ws || ws_bytes < nvfp4_pack_workspace_size(batch, n, k)) return NVFP4_ERR_WORKSPACE;
  if (!aligned16(ws)) return NVFP4_ERR_ALIGN;
  return from_hip(launch_pack(w, batch, n, k, codes, scales, scale_2, static_cast<uint32_t*>(ws),
                              layout == NVFP4_LAYOUT_TILED32, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_relayout(const nvfp4_weight_t* src, const nvfp4_weight_t* dst, void* stream) {
  nvfp4_status st;
  if ((st = check_weight(src)) != NVFP4_OK) return st;
  if ((st = check_weight(dst)) != NVFP4_OK) return st;
  if (src->n != dst->n || src->k != dst->k || src->groups != dst->groups) return NVFP4_ERR_SHAPE;
  // the tiled side's constraints hold for both once either is tiled
  if (src->layout == dst->layout) {
    if (src->codes == dst->codes && src->scales == dst->scales) return NVFP4_OK;
    const size_t cb = (size_t)src->groups * src->n * (src->k / 2), sb = cb / 8;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(const_cast<uint8_t*>(dst->codes), src->codes, cb, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(const_cast<uint8_t*>(dst->scales), src->scales, sb, hipMemcpyDeviceToDevice, s);
    return from_hip(e);
  }
  if ((int64_t)src->groups * src->n * (src->k / 32) / 256 >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  return from_hip(launch_relayout(src->codes, src->scales, src->layout == NVFP4_LAYOUT_TILED32, src->groups,
                                  src->n, src->k, const_cast<uint8_t*>(dst->codes),
                                  const_cast<uint8_t*>(dst->scales), static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_selftest_fp4_convert(unsigned long long* mismatches, void* stream) {
  if (!mismatches) return NVFP4_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(mismatches) % 8 != 0) return NVFP4_ERR_ALIGN;
  return from_hip(launch_fp4_convert_check(mismatches, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_dequant(const nvfp4_weight_t* w, uint16_t* wq_unscaled, float* wq_scaled,
                           void* stream) {
  nvfp4_status st = check_weight(w);
  if (st != NVFP4_OK) return st;
  if (!wq_unscaled && !wq_scaled) return NVFP4_ERR_NULL;
  if ((wq_unscaled && !aligned16(wq_unscaled)) || (wq_scaled && !aligned16(wq_scaled)))
    return NVFP4_ERR_ALIGN;
  return from_hip(launch_dequant(w->codes, w->scales, w->scale_2, w->groups, w->n, w->k,
                                 w->layout == NVFP4_LAYOUT_TILED32, wq_unscaled,
                                 wq_scaled, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_linear(const uint16_t* x, int64_t m, const nvfp4_weight_t* w, uint16_t* y,
                          void* stream) {
  return linear_impl(x, m, w, nullptr, y, static_cast<hipStream_t>(stream));
}

nvfp4_status nvfp4_linear_gated(const uint16_t* x, int64_t m, const nvfp4_weight_t* w_gate,
                                const nvfp4_weight_t* w_up, uint16_t* h, void* stream) {
  if (!w_up) return NVFP4_ERR_NULL;
  return linear_impl(x, m, w_gate, w_up, h, static_cast<hipStream_t>(stream));
}

size_t nvfp4_moe_route_workspace_size(int64_t T, int32_t k, int32_t n_experts) {
  if (T < 0 || k < 1 || n_experts < 1) return 0;
  return route_scratch_bytes(T * (int64_t)k, n_experts);
}

nvfp4_status nvfp4_moe_route(const int32_t* topk_ids, int64_t T, int32_t k, int32_t n_experts,
                             int32_t expert_begin, int32_t* offsets, int32_t* perm, int32_t* inv,
                             void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k < 1 || k > kMaxTopk || n_experts < 1 || n_experts > kMaxExperts) return NVFP4_ERR_SHAPE;
  if (T * (int64_t)k > kMaxSlots) return NVFP4_ERR_SHAPE;
  if (!offsets || !perm || !inv || (T > 0 && !topk_ids)) return NVFP4_ERR_NULL;
  if (ws && !aligned16(ws)) return NVFP4_ERR_ALIGN;
  return from_hip(launch_route(topk_ids, T * k, n_experts, expert_begin, 16, offsets, perm, inv, nullptr,
                               nullptr, RoutePrep{}, static_cast<hipStream_t>(stream),
                               static_cast<int32_t*>(ws), ws ? ws_bytes : 0));
}

size_t nvfp4_moe_workspace_size(int64_t T, int32_t k, int32_t n_experts, int64_t H, int64_t I) {
  if (T < 0 || k < 1 || n_experts < 1 || H < 1 || I < 1) return 0;
  return moe_layout(T, k, n_experts, H, I).total;
}

nvfp4_status nvfp4_moe_grouped(const uint16_t* x, int64_t T, int64_t H, const int32_t* topk_ids,
                               const float* topk_w, int32_t k, int32_t expert_begin,
                               const nvfp4_weight_t* gate, const nvfp4_weight_t* up,
                               const nvfp4_weight_t* down, void* ws, size_t ws_bytes, uint16_t* y,
                               void* stream) {
  return moe_impl(x, T, H, topk_ids, topk_w, k, expert_begin, gate, up, down, ws, ws_bytes, y,
                  static_cast<hipStream_t>(stream), nullptr, nullptr, nullptr, NVFP4_CLASS_AUTO);
}

nvfp4_status nvfp4_moe_grouped_class(const uint16_t* x, int64_t T, int64_t H, const int32_t* topk_ids,
                                     const float* topk_w, int32_t k, int32_t expert_begin,
                                     const nvfp4_weight_t* gate, const nvfp4_weight_t* up,
                                     const nvfp4_weight_t* down, int32_t kernel_class, void* ws, size_t ws_bytes,
                                     uint16_t* y, void* stream) {
  return moe_impl(x, T, H, topk_ids, topk_w, k, expert_begin, gate, up, down, ws, ws_bytes, y,
                  static_cast<hipStream_t>(stream), nullptr, nullptr, nullptr, kernel_class);
}

nvfp4_status nvfp4_moe_plan(int64_t T, int32_t k, int32_t n_experts, int64_t H, int64_t I, int32_t gate_layout,
                            int32_t down_layout, int32_t kernel_class, int32_t* plan) {
  if (!plan) return NVFP4_ERR_NULL;
  for (int i = 0; i < 5; ++i) plan[i] = 0;
  if (H < 32 || H % 32 != 0 || I < 32 || I % 32 != 0) return NVFP4_ERR_SHAPE;
  for (int32_t lay : {gate_layout, down_layout})
    if (lay != NVFP4_LAYOUT_ROWS && lay != NVFP4_LAYOUT_TILED32) return NVFP4_ERR_SHAPE;
  if (gate_layout == NVFP4_LAYOUT_TILED32 && (I % 32 != 0 || H % 256 != 0)) return NVFP4_ERR_SHAPE;
  if (down_layout == NVFP4_LAYOUT_TILED32 && (H % 32 != 0 || I % 256 != 0)) return NVFP4_ERR_SHAPE;
  MoePlan P{};
  // at least one row, so the plan names the kernels a non-empty call of this class runs
  const nvfp4_status st = moe_shape_plan(T > 0 ? T : 1, H, k, n_experts, I, gate_layout == NVFP4_LAYOUT_TILED32,
                                         down_layout == NVFP4_LAYOUT_TILED32, false, kernel_class, P);
  if (st != NVFP4_OK) return st;
  int32_t gate_detail = 0, down_detail = 0;
  plan[0] = variant_tile_rows(P.v);
  plan[1] = kernel_id(P.kg, false, P, H, &gate_detail);
  plan[2] = kernel_id(P.kd, true, P, H, &down_detail);
  plan[3] = down_detail;
  plan[4] = P.f16 ? 1 : 0;
  return NVFP4_OK;
}

nvfp4_status nvfp4_moe_grouped_timed(const uint16_t* x, int64_t T, int64_t H,
                                     const int32_t* topk_ids, const float* topk_w, int32_t k,
                                     int32_t expert_begin, const nvfp4_weight_t* gate,
                                     const nvfp4_weight_t* up, const nvfp4_weight_t* down,
                                     void* ws, size_t ws_bytes, uint16_t* y, void* stream,
                                     void* const* events) {
  if (!events) return NVFP4_ERR_NULL;
  return moe_impl(x, T, H, topk_ids, topk_w, k, expert_begin, gate, up, down, ws, ws_bytes, y,
                  static_cast<hipStream_t>(stream), events, nullptr, nullptr, NVFP4_CLASS_AUTO);
}

nvfp4_status nvfp4_moe_grouped_w4a4(const uint16_t* x, int64_t T, int64_t H, const int32_t* topk_ids,
                                    const float* topk_w, int32_t k, int32_t expert_begin,
                                    const nvfp4_weight_t* gate, const nvfp4_weight_t* up,
                                    const nvfp4_weight_t* down, const float* input_scale_gate_up,
                                    const float* input_scale_down, void* ws, size_t ws_bytes, uint16_t* y,
                                    void* stream) {
  if (!input_scale_gate_up || !input_scale_down) return NVFP4_ERR_NULL;
  return moe_impl(x, T, H, topk_ids, topk_w, k, expert_begin, gate, up, down, ws, ws_bytes, y,
                  static_cast<hipStream_t>(stream), nullptr, input_scale_gate_up, input_scale_down,
                  NVFP4_CLASS_AUTO);
}

nvfp4_status nvfp4_moe_grouped_noalloc(const uint16_t* x, int64_t T, int64_t H, const int32_t* topk_ids,
                                       const float* topk_w, int32_t k, int32_t expert_begin,
                                       const nvfp4_weight_t* gate, const nvfp4_weight_t* up,
                                       const nvfp4_weight_t* down, uint16_t* y, void* stream) {
  MoePlan P{};
  const nvfp4_status st = moe_check(x, T, H, topk_ids, topk_w, k, gate, up, down, y, nullptr,
                                    NVFP4_NOALLOC_SCRATCH_BYTES, false, NVFP4_CLASS_AUTO, P, true);
  if (st != NVFP4_OK) return st;
  if (T == 0) return NVFP4_OK;
  void* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess) return NVFP4_ERR_HIP;
  // every byte of the routed call's workspace is written before it is read within
  // the call, so the previous call's contents need no clearing
  return moe_run(P, x, T, H, topk_ids, topk_w, k, expert_begin, gate, up, down, ws, y,
                 static_cast<hipStream_t>(stream), nullptr);
}

nvfp4_status nvfp4_quantize_act(const uint16_t* x, int64_t rows, int64_t k, const float* input_scale,
                                uint8_t* codes, uint8_t* scales, void* stream) {
  if (rows < 0 || k < 32 || k % 32 != 0 || rows > kMaxSlots) return NVFP4_ERR_SHAPE;
  if (rows == 0) return NVFP4_OK;
  if (!x || !input_scale || !codes || !scales) return NVFP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || (reinterpret_cast<uintptr_t>(input_scale) & 3))
    return NVFP4_ERR_ALIGN;
  return from_hip(launch_act_quant(x, rows, k, input_scale, codes, scales, static_cast<hipStream_t>(stream)));
}

size_t nvfp4_router_workspace_size(int64_t T, int64_t H, int32_t n_experts) {
  if (T < 0 || H < 1 || n_experts < 1) return 0;
  return round_up(sizeof(float) * (size_t)(T * n_experts > 0 ? T * n_experts : 1)) +
         round_up(bf16_gemm_partial_bytes(T, n_experts, H, false) + 256);
}

nvfp4_status nvfp4_router_topk(const uint16_t* x, int64_t T, int64_t H, const uint16_t* w_router,
                               int32_t n_experts, int32_t k, void* ws, size_t ws_bytes, int32_t* topk_ids,
                               float* topk_w, void* stream) {
  if (T < 0 || T > kMaxSlots || n_experts < 1 || n_experts > kMaxExperts || k < 1 || k > kMaxTopk ||
      k > n_experts || !bf16_shape_ok(n_experts, H))
    return NVFP4_ERR_SHAPE;
  if (T == 0) return NVFP4_OK;
  if (!x || !w_router || !topk_ids || !topk_w || !ws) return NVFP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(ws) || (reinterpret_cast<uintptr_t>(topk_ids) & 3) ||
      (reinterpret_cast<uintptr_t>(topk_w) & 3))
    return NVFP4_ERR_ALIGN;
  if (ws_bytes < nvfp4_router_workspace_size(T, H, n_experts)) return NVFP4_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* logits = reinterpret_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                         round_up(sizeof(float) * (size_t)(T * n_experts)));
  int splits = 1;
  hipError_t e = launch_bf16_gemm(false, x, w_router, nullptr, T, n_experts, H, logits, part, s, &splits);
  if (e == hipSuccess)
    e = launch_topk_softmax(splits > 1 ? part : logits, splits, T, n_experts, k, topk_ids, topk_w, s);
  return from_hip(e);
}

size_t nvfp4_bf16_mlp_workspace_size(int64_t M, int64_t H, int64_t Is) {
  if (M < 0 || H < 1 || Is < 1) return 0;
  return round_up(sizeof(uint16_t) * (size_t)(M * Is > 0 ? M * Is : 1)) +
         round_up(std::max(bf16_gemm_partial_bytes(M, Is, H, true), bf16_gemm_partial_bytes(M, H, Is, false)) + 256);
}

nvfp4_status nvfp4_bf16_mlp(const uint16_t* x, int64_t M, int64_t H, const uint16_t* w_gate, const uint16_t* w_up,
                            const uint16_t* w_down, int64_t Is, void* ws, size_t ws_bytes, float* y, void* stream) {
  if (M < 0 || M > kMaxSlots || !bf16_shape_ok(Is, H) || !bf16_shape_ok(H, Is)) return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (!x || !w_gate || !w_up || !w_down || !ws || !y) return NVFP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(ws) ||
      !aligned16(y))
    return NVFP4_ERR_ALIGN;
  if (ws_bytes < nvfp4_bf16_mlp_workspace_size(M, H, Is)) return NVFP4_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + round_up(sizeof(uint16_t) * (size_t)(M * Is)));
  hipError_t e = launch_bf16_gemm(true, x, w_gate, w_up, M, Is, H, h, part, s);
  if (e == hipSuccess) e = launch_bf16_gemm(false, h, w_down, nullptr, M, H, Is, y, part, s);
  return from_hip(e);
}

size_t nvfp4_moe_block_workspace_size(int64_t T, int32_t k, int32_t n_experts, int64_t H, int64_t I, int64_t Is) {
  if (T < 0 || k < 1 || n_experts < 1 || H < 1 || I < 1 || Is < 1) return 0;
  return block_layout(T, k, n_experts, H, I, Is).total;
}

nvfp4_status nvfp4_moe_block(const uint16_t* x, int64_t T, int64_t H, const uint16_t* w_router, int32_t k,
                             const nvfp4_weight_t* gate, const nvfp4_weight_t* up, const nvfp4_weight_t* down,
                             const uint16_t* shared_gate, const uint16_t* shared_up, const uint16_t* shared_down,
                             int64_t Is, void* ws, size_t ws_bytes, uint16_t* y, void* stream) {
  nvfp4_status st;
  if ((st = check_weight(gate)) != NVFP4_OK) return st;
  const int64_t E = gate->groups, I = gate->n;
  if (T < 0 || k < 1 || k > kMaxTopk || k > E || E > kMaxExperts || !bf16_shape_ok(E, H) ||
      !bf16_shape_ok(Is, H) || !bf16_shape_ok(H, Is))
    return NVFP4_ERR_SHAPE;
  if (T > 0 && (!x || !w_router || !shared_gate || !shared_up || !shared_down || !ws || !y)) return NVFP4_ERR_NULL;
  if (T > 0 && (!aligned16(x) || !aligned16(w_router) || !aligned16(shared_gate) || !aligned16(shared_up) ||
                !aligned16(shared_down) || !aligned16(ws) || !aligned16(y)))
    return NVFP4_ERR_ALIGN;
  const BlockLayout L = block_layout(T, k, E, H, I, Is);
  if (T > 0 && ws_bytes < L.total) return NVFP4_ERR_WORKSPACE;
  // the routed part's checks (weights, layouts, kernel cover) before the first launch;
  // its ids, weights and workspace lie inside ws (valid pointers when T > 0)
  void* moe_ws = T > 0 ? at<void>(ws, L.moe) : nullptr;
  const int32_t* ids_c = T > 0 ? at<int32_t>(ws, L.ids) : nullptr;
  const float* tw_c = T > 0 ? at<float>(ws, L.w) : nullptr;
  MoePlan P{};
  if ((st = moe_check(x, T, H, ids_c, tw_c, k, gate, up, down, y, moe_ws, T > 0 ? ws_bytes - L.moe : 0, false,
                      NVFP4_CLASS_AUTO, P)) != NVFP4_OK)
    return st;
  if (T == 0) return NVFP4_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* logits = at<float>(ws, L.logits);
  int32_t* ids = at<int32_t>(ws, L.ids);
  float* tw = at<float>(ws, L.w);
  uint16_t* hs = at<uint16_t>(ws, L.hs);
  float* ys = at<float>(ws, L.ys);
  float* part = at<float>(ws, L.part);
  // router, then the shared expert (its fp32 result is added by the routed MLP's
  // combine, after the k routed slots), then the routed experts. The router's and
  // the shared down product's K splits are summed by their consumers (top-k,
  // combine); `part` is free again once each consumer ran, in stream order.
  int rs = 1, ds = 1;
  hipError_t e = launch_bf16_gemm(false, x, w_router, nullptr, T, E, H, logits, part, s, &rs);
  if (e == hipSuccess) e = launch_topk_softmax(rs > 1 ? part : logits, rs, T, (int)E, k, ids, tw, s);
  if (e == hipSuccess) e = launch_bf16_gemm(true, x, shared_gate, shared_up, T, Is, H, hs, part, s);
  if (e == hipSuccess) e = launch_bf16_gemm(false, hs, shared_down, nullptr, T, H, Is, ys, part, s, &ds);
  if (e != hipSuccess) return from_hip(e);
  return moe_run(P, x, T, H, ids, tw, k, 0, gate, up, down, moe_ws, y, s, nullptr, nullptr, nullptr,
                 ds > 1 ? part : ys, ds);
}

size_t nvfp4_moe_grouped_bf16_workspace_size(int64_t T, int32_t k, int32_t n_experts, int64_t H, int64_t I) {
  if (T < 0 || k < 1 || n_experts < 1 || H < 1 || I < 1) return 0;
  const int64_t S = T * k, max_tiles = S / 64 + (S < n_experts ? S : n_experts);
  return round_up(sizeof(int32_t) * (size_t)(n_experts + 1)) + round_up(sizeof(int32_t) * (size_t)(S > 0 ? S : 1)) +
         round_up(sizeof(int32_t) * 4 * (size_t)(max_tiles > 0 ? max_tiles : 1)) + 256 +
         round_up(sizeof(uint16_t) * (size_t)(S * I > 0 ? S * I : 1)) +
         round_up(sizeof(float) * (size_t)(S * H > 0 ? S * H : 1));
}

nvfp4_status nvfp4_moe_grouped_bf16(const uint16_t* x, int64_t T, int64_t H, const int32_t* topk_ids,
                                    const float* topk_w, int32_t k, int32_t expert_begin, const uint16_t* w_gate,
                                    const uint16_t* w_up, const uint16_t* w_down, int32_t n_experts, int64_t I,
                                    void* ws, size_t ws_bytes, uint16_t* y, void* stream) {
  if (T < 0 || k < 1 || k > kMaxTopk || n_experts < 1 || n_experts > kMaxExperts || T * (int64_t)k > kMaxSlots ||
      !bf16_shape_ok(I, H) || !bf16_shape_ok(H, I) || H % 8 != 0)
    return NVFP4_ERR_SHAPE;
  if (T == 0) return NVFP4_OK;
  if (!x || !topk_ids || !topk_w || !w_gate || !w_up || !w_down || !ws || !y) return NVFP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(ws) ||
      !aligned16(y))
    return NVFP4_ERR_ALIGN;
  if (ws_bytes < nvfp4_moe_grouped_bf16_workspace_size(T, k, n_experts, H, I)) return NVFP4_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t S = T * k, max_tiles = S / 64 + (S < n_experts ? S : n_experts);
  char* p = reinterpret_cast<char*>(ws);
  int32_t* offsets = reinterpret_cast<int32_t*>(p);
  p += round_up(sizeof(int32_t) * (size_t)(n_experts + 1));
  int32_t* perm = reinterpret_cast<int32_t*>(p);
  p += round_up(sizeof(int32_t) * (size_t)S);
  int32_t* tiles = reinterpret_cast<int32_t*>(p);
  p += round_up(sizeof(int32_t) * 4 * (size_t)max_tiles);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(p);
  p += 256;
  uint16_t* h = reinterpret_cast<uint16_t*>(p);
  p += round_up(sizeof(uint16_t) * (size_t)(S * I));
  float* ypart = reinterpret_cast<float*>(p);
  // tiles of 64 or 128 rows (the tile list above is sized for 64)
  const int tr = bf16_grouped_tile_rows(S, n_experts);
  const int64_t grid_tiles = S / tr + (S < n_experts ? S : n_experts);
  // Ypart is not written before down: it holds the route's scratch meanwhile
  hipError_t e = launch_route(topk_ids, S, n_experts, expert_begin, tr, offsets, perm, nullptr, tiles, n_tiles,
                              RoutePrep{}, s, reinterpret_cast<int32_t*>(ypart), sizeof(float) * (size_t)(S * H));
  if (e == hipSuccess)
    e = launch_bf16_grouped(true, x, w_gate, w_up, tiles, n_tiles, grid_tiles, perm, k, I, H, h, s, tr);
  if (e == hipSuccess)
    e = launch_bf16_grouped(false, h, w_down, nullptr, tiles, n_tiles, grid_tiles, perm, 0, H, I, ypart, s, tr);
  if (e == hipSuccess) e = launch_combine(topk_ids, topk_w, ypart, T, k, H, n_experts, expert_begin, nullptr, 1, y, s);
  return from_hip(e);
}

}  // extern "C"
