// C-ABI entry points: argument checks, launch configuration, kernel launch.
// Declared and documented in include/tkg.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <stdint.h>

#include "tkg.h"
#include "tkg_device.hpp"
#include "tkg_kernels.hpp"
#include "tkg_finish.hpp"
#include "tkg_layout.hpp"
#include "tkg_attn_layout.hpp"

namespace {

using tkg::kBM;
using tkg::kBN;

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not queried yet

// Compute units of the current device (cached per device).
int cu_count(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return TKG_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return TKG_OK;
    }
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess ||
      n <= 0)
    return TKG_ERR_DEVICE;
  if (dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return TKG_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Scratch of the allocation-free split-K entry point: the fp32 partial sums
// live in this file-scope device array, which each device that loads the
// library holds until the process ends. In host code `scratch` names a
// host-side stand-in, never the device memory: kernels and copies take the
// address hipGetSymbolAddress gives for the current device, resolved once
// per device and kept in g_scratch. Calls that overlap on one device share
// the array and race; nothing in it needs clearing (every work unit writes
// its whole slot before the reduction reads it).
__device__ __attribute__((aligned(256))) uint8_t scratch[TKG_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TKG_ERR_DEVICE;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr)
        return TKG_ERR_DEVICE;
      g_scratch[dev].store(q, std::memory_order_release);
      p = q;
    }
  }
  *out = p;
  return TKG_OK;
}

struct Plan {
  int32_t tiles_m, tiles_n, num_tiles, group_m, xcd_remap, grid;
  // two-launch dense products: the first launch runs units [0, full_units),
  // the tail launch (tail_units > 0) the rest as 128 x 128 quadrants
  int32_t full_units, tail_units, tail_grid;
};

// panel_bytes > 0 (bf16/fp8 products whose operands exceed the last-level
// cache): with group_m left automatic, the XCD-block order on bands of the
// most tile rows (8 .. 32, a power of two) whose A panels of panel_bytes
// each fit in half the cache, so a band's A panels stay cached while the
// band's rounds stream B. Otherwise bands of 8 rows in the grouped order.
// `cus`: the device's compute units (the default grid is cus x occ).
int make_plan(int64_t M, int64_t N, int64_t bt, int occ, const tkg_opts* o, int cus,
              Plan* pl, int64_t panel_bytes = 0) {
  pl->tiles_m = (int32_t)((M + bt - 1) / bt);
  pl->tiles_n = (int32_t)((N + bt - 1) / bt);
  const int64_t tiles = (int64_t)pl->tiles_m * pl->tiles_n;
  if (tiles > INT32_MAX / 2) return TKG_ERR_SHAPE;
  pl->num_tiles = (int32_t)tiles;
  int grid = (o && o->grid > 0) ? o->grid : cus * occ;
  if (grid > pl->num_tiles) grid = pl->num_tiles;
  pl->grid = grid;
  int gm = (o && o->group_m > 0) ? o->group_m : 8;
  pl->xcd_remap = o == nullptr ? 1 : (o->xcd_remap == 2 ? 2 : (o->xcd_remap != 0 ? 1 : 0));
  if (panel_bytes > 0 && !(o && o->group_m > 0)) {
    while (gm < 32 && 2 * gm * panel_bytes <= tkg::kLastLevelCacheBytes / 2) gm *= 2;
    if (pl->xcd_remap == 1) pl->xcd_remap = 2;
  }
  if (gm > pl->tiles_m) gm = pl->tiles_m;
  pl->group_m = gm;
  pl->full_units = pl->num_tiles;
  pl->tail_units = 0;
  pl->tail_grid = 0;
  return TKG_OK;
}

// Checks shared by every dtype. `kmult` is the required multiple of K and
// `kbytes_per_elem_x2` twice the bytes of one K-element of the staged rows.
int check_common(int64_t M, int64_t N, int64_t K, int64_t kmult,
                 int64_t kmax) {
  if (M < 0 || N < 0 || K < 0) return TKG_ERR_SHAPE;
  if (M > INT32_MAX || N > INT32_MAX || K > kmax) return TKG_ERR_SHAPE;
  if (K % kmult != 0) return TKG_ERR_SHAPE;
  return TKG_OK;
}

// The configuration and launch plan of a dense product on `cus` compute
// units. Variant 0 takes 128 x 128 tiles when 256 x 256 ones would leave
// compute units idle (fewer tiles than units), e.g. one GPU's N/8 shard of a
// product split over 8 GPUs, or K-heavy small products; for operands beyond
// the last-level cache, the bf16 5-slot ring. With group_m 0, such operands
// also take the cache-sized XCD-block order (make_plan).
int dense_plan(tkg::DenseType dt, int64_t M, int64_t N, int64_t K, const tkg_opts* opts,
               int cus, int* variant_out, Plan* pl) {
  const int64_t eb = 1 + (dt == tkg::kBf16);
  int variant = opts ? opts->variant : 0;
  if (variant < 0 || variant >= tkg::dense_num_variants(dt)) return TKG_ERR_SHAPE;
  const bool large = (M + N) * K * eb > tkg::kLastLevelCacheBytes;
  if (variant == 0) {
    const int64_t tiles256 = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    if (tiles256 < cus) variant = tkg::kDenseSmallTileVariant;
    else if (large && dt == tkg::kBf16) variant = tkg::kDenseLargeVariantBf16;
  }
  const int64_t bt = tkg::dense_tile(dt, variant);
  *variant_out = variant;
  const int st = make_plan(M, N, bt, tkg::dense_occupancy(dt, variant), opts, cus, pl,
                           large ? bt * K * eb : 0);
  if (st != TKG_OK) return st;
  // Wave quantization: when the 256 x 256 tiles leave a partial last round
  // whose tiles, split into 128 x 128 quadrants, fit one round of the
  // small-tile configuration's workgroup slots (2 per CU), the full rounds
  // run as usual and the leftover tiles' quadrants run in a second launch:
  // a partial round of big tiles takes as long as a full one, its quadrants
  // about 0.6 of it (measured: 6144^3). Whole tiles only; automatic variant
  // and grid only. Both configurations compute the same bits.
  const bool auto_variant = opts == nullptr || opts->variant == 0;
  const bool auto_grid = opts == nullptr || opts->grid <= 0;
  if (auto_variant && auto_grid && bt == kBM && K > 0 && M % kBM == 0 && N % kBN == 0) {
    const int g = pl->grid;
    const int full = (pl->num_tiles / g) * g, tail = pl->num_tiles - full;
    const int slots = cus * tkg::dense_occupancy(dt, tkg::kDenseSmallTileVariant);
    if (full > 0 && tail > 0 && 4 * tail <= slots) {
      pl->full_units = full;
      pl->tail_units = 4 * tail;
      pl->tail_grid = 4 * tail;
    }
  }
  return TKG_OK;
}

int run_dense(tkg::DenseType dt, int64_t M, int64_t N, int64_t K,
              const void* A, const void* B, void* C, float scale,
              void* stream, const tkg_opts* opts) {
  const int64_t eb = 1 + (dt == tkg::kBf16);
  const int64_t kmult = (dt == tkg::kBf16) ? 8 : 16;
  // 256 rows of K*eb bytes must stay below 2^31 (one buffer resource).
  const int64_t kmax = (dt == tkg::kBf16) ? 4194303 : 8388607;
  int st = check_common(M, N, K, kmult, kmax);
  if (st != TKG_OK) return st;
  if (M == 0 || N == 0) return TKG_OK;
  if (C == nullptr || (K > 0 && (A == nullptr || B == nullptr)))
    return TKG_ERR_NULL;
  if (!aligned16(C) || (K > 0 && (!aligned16(A) || !aligned16(B))))
    return TKG_ERR_ALIGN;
  int cus = 0;
  st = cu_count(&cus);
  if (st != TKG_OK) return st;
  int variant = 0;
  Plan pl;
  st = dense_plan(dt, M, N, K, opts, cus, &variant, &pl);
  if (st != TKG_OK) return st;
  tkg::DenseArgs a;
  a.A = static_cast<const uint8_t*>(A);
  a.B = static_cast<const uint8_t*>(B);
  a.C = static_cast<uint16_t*>(C);
  a.M = (int32_t)M;
  a.N = (int32_t)N;
  a.kbytes = (uint32_t)(K * eb);
  a.scale = scale;
  a.tiles_m = pl.tiles_m;
  a.tiles_n = pl.tiles_n;
  a.num_tiles = pl.num_tiles;
  a.group_m = pl.group_m;
  a.xcd_remap = pl.xcd_remap;
  a.splits = 1;
  a.num_units = pl.full_units;
  a.ksplit = a.kbytes;
  a.ws = nullptr;
  a.quad_base = -1;
  a.quad_tiles_m = a.quad_tiles_n = a.quad_group_m = a.quad_grid = a.quad_remap = 0;
  if (K == 0) {  // empty reduction: the kernel's zero accumulators are C
    a.A = a.B = static_cast<const uint8_t*>(C);
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = tkg::launch_dense(dt, a, pl.grid, variant, s);
  if (e != hipSuccess || pl.tail_units == 0) return e == hipSuccess ? TKG_OK : TKG_ERR_LAUNCH;
  // the leftover tiles as 128 x 128 quadrants, in the first launch's order
  tkg::DenseArgs q = a;
  q.tiles_m = 2 * pl.tiles_m;
  q.tiles_n = 2 * pl.tiles_n;
  q.num_tiles = 4 * pl.num_tiles;
  q.num_units = pl.tail_units;
  q.xcd_remap = 1;
  q.quad_base = pl.full_units;
  q.quad_tiles_m = pl.tiles_m;
  q.quad_tiles_n = pl.tiles_n;
  q.quad_group_m = pl.group_m;
  q.quad_grid = pl.grid;
  q.quad_remap = pl.xcd_remap;
  e = tkg::launch_dense(dt, q, pl.tail_grid, tkg::kDenseSmallTileVariant, s);
  return e == hipSuccess ? TKG_OK : TKG_ERR_LAUNCH;
}

// Split-K plan on the small-tile configuration: `req` splits (0 = enough
// work units for every workgroup slot of the device), each a multiple of
// two stages of K, at most 64; splits = 1 means the plain product.
struct SplitPlan {
  int splits;
  uint32_t ksplit;
  size_t ws_bytes;
  int tiles;
};

int splitk_plan(tkg::DenseType dt, int64_t M, int64_t N, int64_t K, int req, SplitPlan* sp) {
  if (req < 0) return TKG_ERR_SHAPE;
  const int v = tkg::kDenseSmallTileVariant;
  const int64_t bt = tkg::dense_tile(dt, v);
  const int64_t tiles = ((M + bt - 1) / bt) * ((N + bt - 1) / bt);
  const int64_t kbytes = K * (1 + (dt == tkg::kBf16));
  const int64_t unit = 2 * (int64_t)tkg::dense_variant_stage_kbytes(dt, v);  // K bytes
  const int64_t chunks = (kbytes + unit - 1) / unit;
  int64_t s = req;
  if (s == 0) {
    int cus = 0;
    const int st = cu_count(&cus);
    if (st != TKG_OK) return st;
    const int64_t slots = (int64_t)cus * tkg::dense_occupancy(dt, v);
    s = tiles > 0 ? (slots + tiles - 1) / tiles : 1;
    // at least 16 two-stage chunks per range: shorter ranges lose more to
    // the partial-sum traffic and the second kernel than the idle units
    // cost (measured: 1024 x 1024 x 4096 bf16, 8 ranges of 4 chunks, 216 ->
    // 165 TFLOP/s; 1024 x 1024 x 16384, 8 ranges of 16, 232 -> 414)
    const int64_t cap = chunks / 16;
    if (s > cap) s = cap;
  }
  sp->tiles = (int)tiles;
  if (chunks == 0) {   // empty reduction: the plain product writes zeros
    sp->splits = 1;
    sp->ksplit = 0;
    sp->ws_bytes = 0;
    return TKG_OK;
  }
  if (s > 64) s = 64;
  if (s > chunks) s = chunks;
  if (s < 1) s = 1;
  const int64_t per = (chunks + s - 1) / s;        // two-stage chunks per split
  if (per * unit > (int64_t)UINT32_MAX) return TKG_ERR_SHAPE;
  sp->ksplit = (uint32_t)(per * unit);
  sp->splits = (int)((kbytes + sp->ksplit - 1) / sp->ksplit);
  if (sp->splits < 1) sp->splits = 1;
  sp->tiles = (int)tiles;
  sp->ws_bytes = sp->splits > 1 ? (size_t)tiles * sp->splits * tkg::dense_unit_ws_bytes(dt, v) : 0;
  return TKG_OK;
}

int run_dense_splitk(tkg::DenseType dt, int64_t M, int64_t N, int64_t K, const void* A,
                     const void* B, void* C, float scale, void* ws, size_t ws_bytes,
                     int req, void* stream) {
  const int64_t eb = 1 + (dt == tkg::kBf16);
  const int64_t kmult = (dt == tkg::kBf16) ? 8 : 16;
  const int64_t kmax = (dt == tkg::kBf16) ? 4194303 : 8388607;
  int st = check_common(M, N, K, kmult, kmax);
  if (st != TKG_OK) return st;
  if (req < 0) return TKG_ERR_SHAPE;
  if (M == 0 || N == 0) return TKG_OK;
  SplitPlan sp;
  st = splitk_plan(dt, M, N, K, req, &sp);
  if (st != TKG_OK) return st;
  if (sp.splits == 1) {
    tkg_opts o{0, 0, 1, tkg::kDenseSmallTileVariant};
    return run_dense(dt, M, N, K, A, B, C, scale, stream, &o);
  }
  if (C == nullptr || A == nullptr || B == nullptr) return TKG_ERR_NULL;
  if (!aligned16(C) || !aligned16(A) || !aligned16(B)) return TKG_ERR_ALIGN;
  if (ws == nullptr || ws_bytes < sp.ws_bytes) return TKG_ERR_WORKSPACE;
  if (!aligned16(ws)) return TKG_ERR_ALIGN;
  const int v = tkg::kDenseSmallTileVariant;
  int cus = 0;
  st = cu_count(&cus);
  if (st != TKG_OK) return st;
  Plan pl;
  st = make_plan(M, N, tkg::dense_tile(dt, v), tkg::dense_occupancy(dt, v), nullptr, cus, &pl);
  if (st != TKG_OK) return st;
  const int64_t units = (int64_t)pl.num_tiles * sp.splits;
  if (units > INT32_MAX / 2) return TKG_ERR_SHAPE;
  int grid = cus * tkg::dense_occupancy(dt, v);
  if (grid > units) grid = (int)units;
  tkg::DenseArgs a;
  a.A = static_cast<const uint8_t*>(A);
  a.B = static_cast<const uint8_t*>(B);
  a.C = static_cast<uint16_t*>(C);
  a.M = (int32_t)M;
  a.N = (int32_t)N;
  a.kbytes = (uint32_t)(K * eb);
  a.scale = scale;
  a.tiles_m = pl.tiles_m;
  a.tiles_n = pl.tiles_n;
  a.num_tiles = pl.num_tiles;
  a.group_m = pl.group_m;
  a.xcd_remap = pl.xcd_remap;
  a.splits = sp.splits;
  a.num_units = (int32_t)units;
  a.ksplit = sp.ksplit;
  a.ws = static_cast<float*>(ws);
  a.quad_base = -1;
  a.quad_tiles_m = a.quad_tiles_n = a.quad_group_m = a.quad_grid = a.quad_remap = 0;
  hipError_t e = tkg::launch_dense(dt, a, grid, v, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return TKG_ERR_LAUNCH;
  e = tkg::launch_dense_reduce(dt, a, v, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TKG_OK : TKG_ERR_LAUNCH;
}

int run_fp4(int64_t M, int64_t N, int64_t K, const void* A, const void* As,
            float sa, const void* B, const void* Bs, float sb, void* C,
            void* stream, const tkg_opts* opts) {
  int st = check_common(M, N, K, 64, 16777215);
  if (st != TKG_OK) return st;
  const int variant = opts ? opts->variant : 0;
  if (variant < 0 || variant >= tkg::fp4_num_variants()) return TKG_ERR_SHAPE;
  if (M == 0 || N == 0) return TKG_OK;
  if (C == nullptr ||
      (K > 0 && (A == nullptr || B == nullptr || As == nullptr || Bs == nullptr)))
    return TKG_ERR_NULL;
  if (!aligned16(C) || (K > 0 && (!aligned16(A) || !aligned16(B) ||
                                  !aligned16(As) || !aligned16(Bs))))
    return TKG_ERR_ALIGN;
  int cus = 0;
  st = cu_count(&cus);
  if (st != TKG_OK) return st;
  Plan pl;
  st = make_plan(M, N, kBM, 1, opts, cus, &pl);
  if (st != TKG_OK) return st;
  tkg::Fp4Args a;
  a.A = static_cast<const uint8_t*>(A);
  a.As = static_cast<const uint8_t*>(As);
  a.B = static_cast<const uint8_t*>(B);
  a.Bs = static_cast<const uint8_t*>(Bs);
  a.C = static_cast<uint16_t*>(C);
  a.M = (int32_t)M;
  a.N = (int32_t)N;
  a.vbytes = (uint32_t)(K / 2);
  a.sbytes = (uint32_t)(K / 16);
  const uint32_t sk = tkg::fp4_stage_vbytes();
  a.nk = (a.vbytes + sk - 1) / sk;
  a.scale = sa * sb;
  a.tiles_m = pl.tiles_m;
  a.tiles_n = pl.tiles_n;
  a.num_tiles = pl.num_tiles;
  a.group_m = pl.group_m;
  a.xcd_remap = pl.xcd_remap;
  if (K == 0) {
    a.A = a.B = a.As = a.Bs = static_cast<const uint8_t*>(C);
  }
  const hipError_t e =
      tkg::launch_fp4(a, pl.grid, variant, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TKG_OK : TKG_ERR_LAUNCH;
}

int run_mx(tkg::MxType fmt, int64_t M, int64_t N, int64_t K, const void* A,
           const void* As, const void* B, const void* Bs, float scale, void* C,
           void* stream, const tkg_opts* opts) {
  // K % 128: value rows and scale rows (K/32 bytes) stay 16- and 4-byte
  // aligned; 256 rows of values below 2^31 bytes (one buffer resource)
  const int64_t kmax = (fmt == tkg::kMxfp4) ? 16777088 : 8388480;
  int st = check_common(M, N, K, 128, kmax);
  if (st != TKG_OK) return st;
  const int variant = opts ? opts->variant : 0;
  if (variant < 0 || variant >= tkg::mx_num_variants()) return TKG_ERR_SHAPE;
  if (M == 0 || N == 0) return TKG_OK;
  if (C == nullptr ||
      (K > 0 && (A == nullptr || B == nullptr || As == nullptr || Bs == nullptr)))
    return TKG_ERR_NULL;
  if (!aligned16(C) || (K > 0 && (!aligned16(A) || !aligned16(B) ||
                                  !aligned16(As) || !aligned16(Bs))))
    return TKG_ERR_ALIGN;
  int cus = 0;
  st = cu_count(&cus);
  if (st != TKG_OK) return st;
  Plan pl;
  st = make_plan(M, N, kBM, 1, opts, cus, &pl);
  if (st != TKG_OK) return st;
  tkg::MxArgs a;
  a.A = static_cast<const uint8_t*>(A);
  a.As = static_cast<const uint8_t*>(As);
  a.B = static_cast<const uint8_t*>(B);
  a.Bs = static_cast<const uint8_t*>(Bs);
  a.C = static_cast<uint16_t*>(C);
  a.M = (int32_t)M;
  a.N = (int32_t)N;
  a.vbytes = (uint32_t)(fmt == tkg::kMxfp4 ? K / 2 : K);
  a.sbytes = (uint32_t)(K / 32);
  a.scale = scale;
  a.tiles_m = pl.tiles_m;
  a.tiles_n = pl.tiles_n;
  a.num_tiles = pl.num_tiles;
  a.group_m = pl.group_m;
  a.xcd_remap = pl.xcd_remap;
  if (K == 0) {
    a.A = a.B = a.As = a.Bs = static_cast<const uint8_t*>(C);
  }
  const hipError_t e = tkg::launch_mx(fmt, a, pl.grid, variant, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TKG_OK : TKG_ERR_LAUNCH;
}

int run_attention(const void* Q, const void* K, const void* V, void* O, float* lse,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                  float scale, int causal, void* stream) {
  if (D != 64 && D != 128) return TKG_ERR_SHAPE;
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0) return TKG_ERR_SHAPE;
  if (Hq > 0 && (Hkv <= 0 || Hq % Hkv != 0)) return TKG_ERR_SHAPE;
  if (causal && Nq != Nk) return TKG_ERR_SHAPE;
  // one buffer resource per head's Q (and K, V) rows: below 2^31 bytes
  // (compared by division, so that no product of the sizes can overflow)
  if (Nq > INT32_MAX / (2 * D) || Nk > INT32_MAX / (2 * D)) return TKG_ERR_SHAPE;
  const int64_t bq = tkg::attn_block_q((int)D);
  const int64_t qblocks = (Nq + bq - 1) / bq;
  if (B > INT32_MAX || Hq > INT32_MAX || (B > 0 && Hq * qblocks > INT32_MAX / B))
    return TKG_ERR_SHAPE;
  if (B == 0 || Hq == 0 || Nq == 0) return TKG_OK;
  if (Nk == 0) return TKG_ERR_SHAPE;  // a softmax over no keys
  if (!(scale > 0.0f) || !(scale <= 3.402823466e38f)) return TKG_ERR_VALUE;
  if (Q == nullptr || K == nullptr || V == nullptr || O == nullptr) return TKG_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return TKG_ERR_ALIGN;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TKG_ERR_DEVICE;
  tkg::AttnArgs a;
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.O = static_cast<uint16_t*>(O);
  a.lse = lse;
  a.Hq = (int32_t)Hq;
  a.Hkv = (int32_t)Hkv;
  a.Nq = (int32_t)Nq;
  a.Nk = (int32_t)Nk;
  a.group = (int32_t)(Hq / Hkv);
  a.qblocks = (int32_t)qblocks;
  a.num_wg = (int32_t)(B * Hq * qblocks);
  a.c = (float)((double)scale * 1.4426950408889634);  // scale * log2(e)
  a.xcd_remap = 1;
  const hipError_t e = tkg::launch_attn(a, (int)D, causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TKG_OK : TKG_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int tkg_attention_fwd(const void* Q, const void* K, const void* V, void* O, float* lse,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                      float scale, int causal, void* stream) {
  return run_attention(Q, K, V, O, lse, B, Hq, Hkv, Nq, Nk, D, scale, causal, stream);
}

int tkg_attn_lds_offsets(int d, int kind, int i0, int i1, int i2, int i3, uint32_t* out64) {
  if (out64 == nullptr) return TKG_ERR_NULL;
  if ((d != 64 && d != 128) || i0 < 0 || i1 < 0 || i2 < 0 || i3 < 0) return TKG_ERR_SHAPE;
  const uint32_t D = (uint32_t)d;
  for (uint32_t lane = 0; lane < 64; ++lane) {
    switch (kind) {
      case 0:  // K fragment read (kb = i0 = 0: a slot holds 32 keys, ks = i1 < D/16)
        if (i0 >= 1 || i1 >= d / 16) return TKG_ERR_SHAPE;
        out64[lane] = tkg::attn_k_read(D, lane, (uint32_t)i0, (uint32_t)i1);
        break;
      case 1:  // V transposing read (kb = 0, s < 2, t < 2, db < D/32)
        if (i0 >= 1 || i1 >= 2 || i2 >= 2 || i3 >= d / 32) return TKG_ERR_SHAPE;
        out64[lane] = tkg::attn_v_read(D, lane, (uint32_t)i0, (uint32_t)i1, (uint32_t)i2,
                                       (uint32_t)i3);
        break;
      case 2:  // ring copy into the K tile: piece i0 < D/16 (1 KiB of 32 rows)
      case 3: {  // ... into the V tile
        if (i0 >= d / 16) return TKG_ERR_SHAPE;
        const uint32_t chunk = (uint32_t)i0 * 64 + lane;
        const uint32_t row = chunk / (D / 8), cs = chunk % (D / 8);
        // the global chunk this lane fetches, and where the layout puts it
        const uint32_t c = cs ^ (kind == 2 ? tkg::attn_k_swz(D, row) : tkg::attn_v_swz(D, row));
        const uint32_t at = kind == 2 ? tkg::attn_k_offset(D, row, c) : tkg::attn_v_offset(D, row, c);
        if (at != chunk * 16) return TKG_ERR_SHAPE;  // layout and copy disagree
        out64[lane] = row * 2 * D + 16 * c;         // global byte offset in the block
        break;
      }
      default:
        return TKG_ERR_SHAPE;
    }
  }
  return TKG_OK;
}

int gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A, const void* B,
              void* C, void* stream) {
  return run_dense(tkg::kBf16, M, N, K, A, B, C, 1.0f, stream, nullptr);
}

int gemm_fp8(int64_t M, int64_t N, int64_t K, const void* A, float scale_a,
             const void* B, float scale_b, void* C, void* stream) {
  return run_dense(tkg::kFp8, M, N, K, A, B, C, scale_a * scale_b, stream,
                   nullptr);
}

int gemm_fp4_blockscaled(int64_t M, int64_t N, int64_t K, const void* A,
                         const void* A_scales, float a_scale, const void* B,
                         const void* B_scales, float b_scale, void* C,
                         void* stream) {
  return run_fp4(M, N, K, A, A_scales, a_scale, B, B_scales, b_scale, C,
                 stream, nullptr);
}

int gemm_mxfp4(int64_t M, int64_t N, int64_t K, const void* A,
               const void* A_scales, const void* B, const void* B_scales,
               void* C, void* stream) {
  return run_mx(tkg::kMxfp4, M, N, K, A, A_scales, B, B_scales, 1.0f, C, stream,
                nullptr);
}

int gemm_mxfp8(int64_t M, int64_t N, int64_t K, const void* A,
               const void* A_scales, const void* B, const void* B_scales,
               void* C, void* stream) {
  return run_mx(tkg::kMxfp8, M, N, K, A, A_scales, B, B_scales, 1.0f, C, stream,
                nullptr);
}

int tkg_gemm_ex(int dtype, int64_t M, int64_t N, int64_t K, const void* A,
                const void* A_scales, float a_scale, const void* B,
                const void* B_scales, float b_scale, void* C, void* stream,
                const tkg_opts* opts) {
  switch (dtype) {
    case TKG_DTYPE_BF16:
      return run_dense(tkg::kBf16, M, N, K, A, B, C, 1.0f, stream, opts);
    case TKG_DTYPE_FP8:
      return run_dense(tkg::kFp8, M, N, K, A, B, C, a_scale * b_scale, stream,
                       opts);
    case TKG_DTYPE_FP4_BLOCKSCALED:
      return run_fp4(M, N, K, A, A_scales, a_scale, B, B_scales, b_scale, C,
                     stream, opts);
    case TKG_DTYPE_MXFP4:
      return run_mx(tkg::kMxfp4, M, N, K, A, A_scales, B, B_scales,
                    a_scale * b_scale, C, stream, opts);
    case TKG_DTYPE_MXFP8:
      return run_mx(tkg::kMxfp8, M, N, K, A, A_scales, B, B_scales,
                    a_scale * b_scale, C, stream, opts);
    default:
      return TKG_ERR_SHAPE;
  }
}

const char* tkg_status_string(int status) {
  switch (status) {
    case TKG_OK: return "TKG_OK: success";
    case TKG_ERR_NULL: return "TKG_ERR_NULL: a required pointer is NULL";
    case TKG_ERR_SHAPE: return "TKG_ERR_SHAPE: unsupported or invalid shape";
    case TKG_ERR_ALIGN: return "TKG_ERR_ALIGN: pointer not 16-byte aligned";
    case TKG_ERR_LAUNCH: return "TKG_ERR_LAUNCH: kernel launch failed";
    case TKG_ERR_DEVICE: return "TKG_ERR_DEVICE: no usable HIP device";
    case TKG_ERR_WORKSPACE:
      return "TKG_ERR_WORKSPACE: split-K workspace missing or too small (or, without "
             "allocation, more than TKG_NOALLOC_SCRATCH_BYTES)";
    case TKG_ERR_VALUE: return "TKG_ERR_VALUE: a scalar argument is out of range";
    default: return "unknown tkg status";
  }
}

int tkg_lds_row_bytes(int dtype) {
  switch (dtype) {
    case TKG_DTYPE_BF16:
    case TKG_DTYPE_FP8: return (int)tkg::dense_stage_kbytes();
    case TKG_DTYPE_FP4_BLOCKSCALED: return (int)tkg::fp4_stage_vbytes();
    default: return TKG_ERR_SHAPE;
  }
}

int tkg_lds_fragment_rows(int dtype) {
  switch (dtype) {
    case TKG_DTYPE_BF16: return tkg::dense_default_mi(tkg::kBf16);
    case TKG_DTYPE_FP8: return tkg::dense_default_mi(tkg::kFp8);
    case TKG_DTYPE_FP4_BLOCKSCALED: return 32;
    default: return TKG_ERR_SHAPE;
  }
}

int tkg_lds_fragment_offsets(int dtype, int step, int part, int frag,
                             uint32_t* out64) {
  if (out64 == nullptr) return TKG_ERR_NULL;
  const int rb = tkg_lds_row_bytes(dtype);
  if (rb < 0) return rb;
  const int mi = tkg_lds_fragment_rows(dtype);
  // K bytes per row of one MFMA k-step: 32 for the 32x32 blocks of bf16
  // (16 elements) and of the 4-bit path (a 16-byte chunk of packed values
  // per lane half), 64 for 32x32x64 fp8; the 16x16 blocks take twice that.
  int kstep_bytes;
  if (dtype == TKG_DTYPE_FP8) kstep_bytes = 64 * (32 / mi);
  else kstep_bytes = 32 * (32 / mi);
  const int steps = rb / kstep_bytes;
  const int cpk = kstep_bytes / 16;       // 16-byte chunks per k-step
  const int lanes_per_row = 64 / mi;      // lanes reading one row
  const int parts = cpk / lanes_per_row;  // 16-byte reads per lane
  if (step < 0 || step >= steps || part < 0 || part >= parts || frag < 0 ||
      frag >= kBM / mi)
    return TKG_ERR_SHAPE;
  for (uint32_t lane = 0; lane < 64; ++lane) {
    const uint32_t row = (uint32_t)(frag * mi) + lane % (uint32_t)mi;
    const uint32_t chunk = (uint32_t)(step * cpk) + (lane / (uint32_t)mi) * (uint32_t)parts + (uint32_t)part;
    out64[lane] = tkg::swz_offset((uint32_t)rb, row, chunk);
  }
  return steps;
}

int tkg_lds_finish_offsets(int mi, int rj, int kind, int index, uint32_t* out64) {
  if (out64 == nullptr) return TKG_ERR_NULL;
  const int rb = rj * mi * 2;
  if ((mi != 16 && mi != 32) || (rb != 64 && rb != 128 && rb != 256) ||
      (mi == 16 && rj % 2 != 0))
    return TKG_ERR_SHAPE;
  // writes: MI = 32, chunk constant 4*jj + 2*p (2 per block); MI = 16,
  // 2*jj for each pair of blocks; reads: one per 4 lines of 256 bytes
  const int writes = mi == 32 ? 2 * rj : rj / 2;
  const int reads = mi * rb / 1024;
  const int count = kind == 0 ? writes : reads;
  if ((kind != 0 && kind != 1) || index < 0 || index >= count) return TKG_ERR_SHAPE;
  for (uint32_t lane = 0; lane < 64; ++lane) {
    if (kind == 0) {
      const uint32_t cc = mi == 32 ? 4u * (uint32_t)(index / 2) + 2u * (uint32_t)(index % 2)
                                   : 4u * (uint32_t)index;
      out64[lane] = tkg::finish_write_offset((uint32_t)mi, (uint32_t)rb, lane, cc);
    } else {
      out64[lane] = tkg::finish_read_offset(lane, (uint32_t)index);
    }
  }
  return count;
}

int tkg_gemm_splitk(int dtype, int64_t M, int64_t N, int64_t K, const void* A,
                    float a_scale, const void* B, float b_scale, void* C, void* workspace,
                    size_t workspace_bytes, int splits, void* stream) {
  if (dtype == TKG_DTYPE_BF16)
    return run_dense_splitk(tkg::kBf16, M, N, K, A, B, C, 1.0f, workspace, workspace_bytes,
                            splits, stream);
  if (dtype == TKG_DTYPE_FP8)
    return run_dense_splitk(tkg::kFp8, M, N, K, A, B, C, a_scale * b_scale, workspace,
                            workspace_bytes, splits, stream);
  return TKG_ERR_SHAPE;
}

int tkg_gemm_splitk_noalloc(int dtype, int64_t M, int64_t N, int64_t K, const void* A,
                            float a_scale, const void* B, float b_scale, void* C, int splits,
                            void* stream) {
  if (dtype != TKG_DTYPE_BF16 && dtype != TKG_DTYPE_FP8) return TKG_ERR_SHAPE;
  const tkg::DenseType dt = dtype == TKG_DTYPE_BF16 ? tkg::kBf16 : tkg::kFp8;
  void* ws = nullptr;
  const int st = scratch_ptr(&ws);
  if (st != TKG_OK) return st;
  return run_dense_splitk(dt, M, N, K, A, B, C, dt == tkg::kBf16 ? 1.0f : a_scale * b_scale,
                          ws, (size_t)TKG_NOALLOC_SCRATCH_BYTES, splits, stream);
}

int64_t tkg_gemm_splitk_workspace_size(int dtype, int64_t M, int64_t N, int64_t K,
                                       int splits) {
  if (dtype != TKG_DTYPE_BF16 && dtype != TKG_DTYPE_FP8) return TKG_ERR_SHAPE;
  const tkg::DenseType dt = dtype == TKG_DTYPE_BF16 ? tkg::kBf16 : tkg::kFp8;
  const int64_t kmult = (dt == tkg::kBf16) ? 8 : 16;
  const int64_t kmax = (dt == tkg::kBf16) ? 4194303 : 8388607;
  int st = check_common(M, N, K, kmult, kmax);
  if (st != TKG_OK) return st;
  if (M == 0 || N == 0) return 0;
  SplitPlan sp;
  st = splitk_plan(dt, M, N, K, splits, &sp);
  if (st != TKG_OK) return st;
  return (int64_t)sp.ws_bytes;
}

int tkg_gemm_splitk_count(int dtype, int64_t M, int64_t N, int64_t K, int splits) {
  if (dtype != TKG_DTYPE_BF16 && dtype != TKG_DTYPE_FP8) return TKG_ERR_SHAPE;
  const tkg::DenseType dt = dtype == TKG_DTYPE_BF16 ? tkg::kBf16 : tkg::kFp8;
  const int64_t kmult = (dt == tkg::kBf16) ? 8 : 16;
  const int64_t kmax = (dt == tkg::kBf16) ? 4194303 : 8388607;
  int st = check_common(M, N, K, kmult, kmax);
  if (st != TKG_OK) return st;
  SplitPlan sp;
  st = splitk_plan(dt, M, N, K, splits, &sp);
  return st != TKG_OK ? st : sp.splits;
}

int tkg_tile_order(int32_t t, int32_t grid, int32_t xcd_remap, int32_t tiles_m,
                   int32_t tiles_n, int32_t group_m, int32_t quad_base, int32_t* pm,
                   int32_t* pn) {
  if (pm == nullptr || pn == nullptr) return TKG_ERR_NULL;
  if (grid <= 0 || tiles_m <= 0 || tiles_n <= 0 || group_m <= 0 || group_m > tiles_m ||
      xcd_remap < 0 || xcd_remap > 2)
    return TKG_ERR_SHAPE;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  if (tiles > INT32_MAX / 4) return TKG_ERR_SHAPE;
  int r = 0, c = 0;
  if (quad_base < 0) {
    if (t < 0 || t >= tiles) return TKG_ERR_SHAPE;
    tkg::order_tile(t, grid, xcd_remap, tiles_m, tiles_n, group_m, r, c);
  } else {
    if (quad_base > tiles || t < 0 || t >= 4 * (tiles - quad_base)) return TKG_ERR_SHAPE;
    tkg::quadrant_tile(t, quad_base, grid, xcd_remap, tiles_m, tiles_n, group_m, r, c);
  }
  *pm = r;
  *pn = c;
  return TKG_OK;
}

int tkg_plan_launch(int dtype, int64_t M, int64_t N, int64_t K, const tkg_opts* opts,
                    int cus, tkg_launch_plan* out) {
  if (cus <= 0) return TKG_ERR_SHAPE;
  int variant = opts ? opts->variant : 0;
  int64_t bt = kBM;
  Plan pl{};
  int st = TKG_OK;
  bool empty = false;
  switch (dtype) {
    case TKG_DTYPE_BF16:
    case TKG_DTYPE_FP8: {
      const tkg::DenseType dt = dtype == TKG_DTYPE_BF16 ? tkg::kBf16 : tkg::kFp8;
      st = check_common(M, N, K, dt == tkg::kBf16 ? 8 : 16,
                        dt == tkg::kBf16 ? 4194303 : 8388607);
      if (st != TKG_OK) return st;
      if (variant < 0 || variant >= tkg::dense_num_variants(dt)) return TKG_ERR_SHAPE;
      empty = M == 0 || N == 0;
      if (!empty) {
        st = dense_plan(dt, M, N, K, opts, cus, &variant, &pl);
        bt = tkg::dense_tile(dt, variant);
      }
      break;
    }
    case TKG_DTYPE_FP4_BLOCKSCALED:
      st = check_common(M, N, K, 64, 16777215);
      if (st != TKG_OK) return st;
      if (variant < 0 || variant >= tkg::fp4_num_variants()) return TKG_ERR_SHAPE;
      empty = M == 0 || N == 0;
      if (!empty) st = make_plan(M, N, kBM, 1, opts, cus, &pl);
      break;
    case TKG_DTYPE_MXFP4:
    case TKG_DTYPE_MXFP8:
      st = check_common(M, N, K, 128, dtype == TKG_DTYPE_MXFP4 ? 16777088 : 8388480);
      if (st != TKG_OK) return st;
      if (variant < 0 || variant >= tkg::mx_num_variants()) return TKG_ERR_SHAPE;
      empty = M == 0 || N == 0;
      if (!empty) st = make_plan(M, N, kBM, 1, opts, cus, &pl);
      break;
    default:
      return TKG_ERR_SHAPE;
  }
  if (st != TKG_OK) return st;
  if (out != nullptr) {
    const bool tail = !empty && pl.tail_units > 0;
    *out = tkg_launch_plan{variant, (int32_t)bt, empty ? 0 : pl.num_tiles, empty ? 0 : pl.grid,
                           empty ? 0 : pl.group_m, empty ? 0 : pl.xcd_remap,
                           empty ? 0 : pl.full_units,
                           tail ? tkg::kDenseSmallTileVariant : -1,
                           tail ? pl.tail_units : 0, tail ? pl.tail_grid : 0};
  }
  return TKG_OK;
}

int tkg_device_info(int32_t* cus, int32_t* peak_clock_khz) {
  if (cus == nullptr || peak_clock_khz == nullptr) return TKG_ERR_NULL;
  int n = 0;
  const int st = cu_count(&n);
  if (st != TKG_OK) return st;
  int dev = 0, clk = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&clk, hipDeviceAttributeClockRate, dev) != hipSuccess || clk <= 0)
    return TKG_ERR_DEVICE;
  *cus = n;
  *peak_clock_khz = clk;
  return TKG_OK;
}

int tkg_variant_info(int dtype, int variant, tkg_variant_desc* out) {
  tkg_variant_desc d{};
  int n = 0;
  if (dtype == TKG_DTYPE_BF16 || dtype == TKG_DTYPE_FP8) {
    const tkg::DenseType dt = dtype == TKG_DTYPE_BF16 ? tkg::kBf16 : tkg::kFp8;
    n = tkg::dense_num_variants(dt);
    if (variant < 0 || variant >= n) return TKG_ERR_SHAPE;
    tkg::dense_variant_desc(dt, variant, &d.stage_kbytes, &d.slots, &d.waves, &d.load_waves,
                            &d.mfma_block, &d.tile, &d.per_cu, &d.swizzle, &d.schedule);
  } else if (dtype == TKG_DTYPE_FP4_BLOCKSCALED) {
    n = tkg::fp4_num_variants();
    if (variant < 0 || variant >= n) return TKG_ERR_SHAPE;
    // a stage of 64 bytes of packed values per row (and 8 of scales); a
    // ring of 4 stages, i.e. 8 operand slabs
    d = tkg_variant_desc{(int32_t)tkg::fp4_stage_vbytes(), 8, variant == 1 ? 8 : 4,
                         variant == 1 ? 8 : 4, 32, kBM, 1, 1, 0};
  } else if (dtype == TKG_DTYPE_MXFP4 || dtype == TKG_DTYPE_MXFP8) {
    n = tkg::mx_num_variants();
    if (variant < 0 || variant >= n) return TKG_ERR_SHAPE;
    d = tkg_variant_desc{128, 4, 8, 4, 32, kBM, 1, 1, variant == 1 ? 3 : 0};
  } else {
    return TKG_ERR_SHAPE;
  }
  if (out != nullptr) *out = d;
  return n;
}

int tkg_launch_masked(int dtype, int64_t M, int64_t N, int64_t K, int variant) {
  if (M < 0 || N < 0 || K < 0) return TKG_ERR_SHAPE;
  const int n = tkg_variant_info(dtype, variant, nullptr);
  if (n < 0) return n;
  switch (dtype) {
    case TKG_DTYPE_BF16:
      return tkg::dense_masked(tkg::kBf16, variant, M, N, (uint32_t)(K * 2)) ? 1 : 0;
    case TKG_DTYPE_FP8:
      return tkg::dense_masked(tkg::kFp8, variant, M, N, (uint32_t)K) ? 1 : 0;
    case TKG_DTYPE_FP4_BLOCKSCALED:
      return 1;   // every load of the 4-bit kernel carries its whole offset per lane
    case TKG_DTYPE_MXFP4:
      return tkg::mx_masked(tkg::kMxfp4, M, N, (uint32_t)(K / 2), (uint32_t)(K / 32)) ? 1 : 0;
    default:
      return tkg::mx_masked(tkg::kMxfp8, M, N, (uint32_t)K, (uint32_t)(K / 32)) ? 1 : 0;
  }
}

}  // extern "C"
