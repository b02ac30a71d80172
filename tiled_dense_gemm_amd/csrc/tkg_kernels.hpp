// Launch interface between the C-ABI entry points and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tkg {

enum DenseType { kBf16 = 0, kFp8 = 1 };

// One dense problem: C (M x N, bf16, row-major) = scale * A (M x K) * B,
// with A row-major and B given as an N x K row-major array; both operands
// hold `kbytes` bytes per row.
struct DenseArgs {
  const uint8_t* A;
  const uint8_t* B;
  uint16_t* C;
  int32_t M, N;
  uint32_t kbytes;  // bytes of K per operand row
  float scale;
  int32_t tiles_m, tiles_n, num_tiles, group_m;
  int32_t xcd_remap;  // 1: give each XCD a contiguous range of tiles
  // split-K: work unit u is split u % splits of tile u / splits and covers
  // K bytes [split * ksplit, min((split + 1) * ksplit, kbytes)); with
  // splits > 1 the units write fp32 partial sums to ws (see
  // launch_dense_reduce) instead of C. splits = 1: ksplit >= kbytes.
  int32_t splits, num_units;
  uint32_t ksplit;
  float* ws;
  // Tail launch of a two-launch product (quad_base >= 0; 128 x 128 tile
  // configurations, whole tiles, one split): unit u is quadrant u % 4 (row
  // half (u % 4) / 2, column half u % 2) of tile quad_base + u / 4 of the
  // 256 x 256 launch that ran the full rounds, placed by that launch's tile
  // order (quad_tiles_m x quad_tiles_n tiles, bands of quad_group_m rows,
  // quad_grid workgroups, remap quad_remap). quad_base < 0: tiles_m,
  // tiles_n, group_m and this launch's grid place the tiles.
  int32_t quad_base, quad_tiles_m, quad_tiles_n, quad_group_m, quad_grid, quad_remap;
};

// Block-scaled 4-bit problem: values packed two per byte (K/2 bytes per row)
// and one e4m3 scale per 16 K-elements (K/16 bytes per row).
struct Fp4Args {
  const uint8_t* A;
  const uint8_t* As;
  const uint8_t* B;
  const uint8_t* Bs;
  uint16_t* C;
  int32_t M, N;
  uint32_t vbytes;  // K/2
  uint32_t sbytes;  // K/16
  uint32_t nk;
  float scale;
  int32_t tiles_m, tiles_n, num_tiles, group_m;
  int32_t xcd_remap;
};

// MX block-scaled problem: e2m1 values two per byte (K/2 bytes per row) or
// e4m3 values (K bytes per row), one E8M0 scale per 32 K-elements (K/32
// bytes per row).
enum MxType { kMxfp4 = 0, kMxfp8 = 1 };
struct MxArgs {
  const uint8_t* A;
  const uint8_t* As;
  const uint8_t* B;
  const uint8_t* Bs;
  uint16_t* C;
  int32_t M, N;
  uint32_t vbytes;  // value bytes per row
  uint32_t sbytes;  // K/32
  float scale;
  int32_t tiles_m, tiles_n, num_tiles, group_m;
  int32_t xcd_remap;
};

// Softmax attention forward: O = softmax(scale * Q K^T) V per (batch, query
// head), bf16 [B, H, N, D] tensors, D contiguous. Query head h reads
// key/value head h / group. lse (fp32 [B, Hq, Nq], natural log) may be null.
struct AttnArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  uint16_t* O;
  float* lse;
  int32_t Hq, Hkv, Nq, Nk;
  int32_t group;       // Hq / Hkv
  int32_t qblocks;     // query blocks per head
  int32_t num_wg;      // B * Hq * qblocks
  float c;             // scale * log2(e)
  int32_t xcd_remap;
  int32_t lpt_heads;   // causal order: heads per longest-first window (set by launch_attn)
};
// query rows per workgroup for head dimension D (0: unsupported D)
int attn_block_q(int D);
hipError_t launch_attn(const AttnArgs& a, int D, bool causal, hipStream_t stream);

// Tile shape shared by the kernels and the host-side argument checks.
constexpr int kBM = 256;
constexpr int kBN = 256;

// variant: index of a compiled ring shape (0 = default), below
// dense_num_variants(dt); hipErrorInvalidValue otherwise.
hipError_t launch_dense(DenseType dt, const DenseArgs& a, int grid, int variant,
                        hipStream_t stream);
int dense_num_variants(DenseType dt);
// the configuration of `variant` (see tkg_variant_desc in tkg.h)
void dense_variant_desc(DenseType dt, int variant, int32_t* stage_kbytes, int32_t* slots,
                        int32_t* waves, int32_t* load_waves, int32_t* mfma_block,
                        int32_t* tile, int32_t* per_cu, int32_t* swizzle, int32_t* schedule);
// whether the launch runs the masked instance (every load's whole offset
// per-lane and bounds-checked): ragged M or N tiles, or a K tail
bool dense_masked(DenseType dt, int variant, int64_t M, int64_t N, uint32_t kbytes);
// MFMA block (16 or 32) of the default configuration for dt
int dense_default_mi(DenseType dt);
// workgroup tile edge (256 or 128) of variant `variant`
int dense_tile(DenseType dt, int variant);
// workgroups per compute unit of variant `variant` (the default grid)
int dense_occupancy(DenseType dt, int variant);
// bytes of fp32 partial sums one split-K work unit of `variant` writes
uint32_t dense_unit_ws_bytes(DenseType dt, int variant);
// K bytes of one stage of `variant` (split boundaries are multiples of two)
uint32_t dense_variant_stage_kbytes(DenseType dt, int variant);
// C = scale * (sum over splits of the partial sums in a.ws), one workgroup
// per output tile, splits added in order 0, 1, ...
hipError_t launch_dense_reduce(DenseType dt, const DenseArgs& a, int variant,
                               hipStream_t stream);
// the variant that variant 0 resolves to when the product has fewer
// 256 x 256 output tiles than compute units
constexpr int kDenseSmallTileVariant = 4;
// the bf16 variant that variant 0 resolves to when the operands exceed the
// last-level cache (kLastLevelCacheBytes): the 5-slot ring
constexpr int kDenseLargeVariantBf16 = 18;
// MI355X's memory-side last-level cache (the MALL), shared by the XCDs
constexpr int64_t kLastLevelCacheBytes = 256ll << 20;
hipError_t launch_fp4(const Fp4Args& a, int grid, int variant,
                      hipStream_t stream);
int fp4_num_variants();
// variant 0: fragment reads after their last use; 1: early reads
hipError_t launch_mx(MxType fmt, const MxArgs& a, int grid, int variant, hipStream_t stream);
int mx_num_variants();
// whether the MX launch runs the masked instance (ragged M or N tiles, or a
// ragged last stage): every load's whole offset per lane, bounds-checked
bool mx_masked(MxType fmt, int64_t M, int64_t N, uint32_t vbytes, uint32_t sbytes);

// K bytes per stage row of each kernel family (for the host).
uint32_t dense_stage_kbytes();
uint32_t fp4_stage_vbytes();

}  // namespace tkg
