// Device-side building blocks for the gfx950 GEMM kernels: vector types,
// buffer resources for bounds-checked global->LDS staging, explicit wait
// counters, and the MFMA instructions the 16x16-based tile grid is built of.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tkg_layout.hpp"  // TKG_HD

#define TKG_LDS __attribute__((address_space(3)))

namespace tkg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Offset that lies outside every resource this library builds (their
// num_records never exceeds 2^31 - 1): a load there returns zeros.
constexpr uint32_t kOobOffset = 0x80000000u;

// Raw buffer resource over [base, base + nbytes): loads past nbytes return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                            uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)nbytes, 0x00020000);
}

// 16 bytes per lane straight from global memory into LDS: the wave writes
// 1 KiB at `lds` (wave-uniform), lane l at byte 16*l.
__device__ __forceinline__ void dma_b128(__amdgpu_buffer_rsrc_t r,
                                         TKG_LDS void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, 0, 0, 0);
}
// The same with a wave-uniform byte offset `soff` added to every lane's
// offset (kept in a scalar register instead of per-lane arithmetic).
__device__ __forceinline__ void dma_b128_soff(__amdgpu_buffer_rsrc_t r,
                                              TKG_LDS void* lds, uint32_t voff,
                                              uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, soff, 0, 0);
}
// 4 bytes per lane: the wave writes 256 bytes at `lds`, lane l at byte 4*l.
__device__ __forceinline__ void dma_b32(__amdgpu_buffer_rsrc_t r,
                                        TKG_LDS void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 4, voff, 0, 0, 0);
}

__device__ __forceinline__ void dma_b32_soff(__amdgpu_buffer_rsrc_t r,
                                             TKG_LDS void* lds, uint32_t voff,
                                             uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 4, voff, soff, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) |
                             (0xF << 8));
}

// Workgroup barrier for the LDS ring: waits for this wave's own LDS reads,
// then s_barrier. Unlike __syncthreads() it does not wait for outstanding
// global loads (that fence would drain the whole ring at every stage); the
// caller waits with wait_vmcnt for exactly the stage it needs. The asm
// clobber keeps memory operations from moving across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename T>
__device__ __forceinline__ T lds_read(const TKG_LDS uint8_t* base,
                                      uint32_t off) {
  return *reinterpret_cast<const TKG_LDS T*>(base + off);
}

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16). Lane l supplies row
// l%32 of A and column l%32 of B, 8 consecutive k each (k-half l/32); it
// receives column l%32 of D, rows 8*(r/4) + 4*(l/32) + r%4 in element r.
__device__ __forceinline__ f32x16_t mfma_bf16(bf16x8_t a, bf16x8_t b,
                                              f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(32x32, fp32) += A(32x64, OCP e4m3) * B(64x32, OCP e4m3); 32 k per lane.
__device__ __forceinline__ f32x16_t mfma_fp8(i32x8_t a, i32x8_t b,
                                             f32x16_t c) {
  // format 0 = fp8 e4m3 for both operands, no block scaling
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0,
                                                         0, 0);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16). Lane l supplies row
// l%16 of A and column l%16 of B, 8 consecutive k each (k-quarter l/16); it
// receives column l%16 of D, rows 4*(l/16) + r in element r.
__device__ __forceinline__ f32x4_t mfma16_bf16(bf16x8_t a, bf16x8_t b,
                                               f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x128, OCP e4m3) * B(128x16, OCP e4m3); 32 k per lane.
__device__ __forceinline__ f32x4_t mfma16_fp8(i32x8_t a, i32x8_t b,
                                              f32x4_t c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0,
                                                          0, 0);
}

// Four fp32 -> four bf16 (round to nearest even), packed in 8 bytes.
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c,
                                             float d) {
  bf16x2_t lo = {(__bf16)a, (__bf16)b};
  bf16x2_t hi = {(__bf16)c, (__bf16)d};
  uint2 r;
  r.x = __builtin_bit_cast(uint32_t, lo);
  r.y = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// Persistent-grid tile order. Workgroups are dispatched round-robin over the
// 8 XCDs (workgroup w runs on XCD w % 8), each XCD with its own L2. The
// virtual id gives every XCD a contiguous range of G/8 ids, so the tiles an
// XCD runs at the same time are neighbours in the grouped order below and
// share operand panels in that XCD's L2. (Host and device: the library
// reports the order the kernels run, tkg_tile_order.)
TKG_HD inline int xcd_virtual_id(int w, int G, int remap) {
  return (remap && G % 8 == 0) ? (w % 8) * (G / 8) + (w / 8) : w;
}

// Grouped order: tiles are walked in bands of `group_m` tile rows; inside a
// band, column by column. Consecutive tiles then reuse the same few A row
// panels and B column panels (the pages' {8, N, M/8} block order).
TKG_HD inline void grouped_tile(int t, int tiles_m, int tiles_n, int group_m, int& pm,
                                int& pn) {
  const int per_group = group_m * tiles_n;
  const int g = t / per_group;
  const int first = g * group_m;
  const int rows = tiles_m - first < group_m ? tiles_m - first : group_m;
  const int r = t - g * per_group;
  pm = first + r % rows;
  pn = r / rows;
}

// Tile t of the persistent order over a grid of G workgroups (workgroup w
// runs tiles xcd_virtual_id(w) + k*G). remap 0 and 1: the grouped order.
// remap 2 (XCD blocks): a round is the G consecutive tiles run at the same
// time; when a round fills a group_m x (G / group_m) rectangle of one full
// band, it is re-dealt so that the G/8 tiles of each XCD form an h x w block
// of it (h + w operand panels per K stage in that XCD's L2, instead of up to
// G/8 + 1 when group_m does not match the XCD's share). Any other round
// keeps the grouped order, so the map stays a bijection.
TKG_HD inline void order_tile(int t, int G, int remap, int tiles_m, int tiles_n,
                              int group_m, int& pm, int& pn) {
  const int per_group = group_m * tiles_n;
  const int g = t / per_group;
  const int first = g * group_m;
  if (remap == 2 && G % 8 == 0 && G % group_m == 0 && per_group % G == 0 &&
      tiles_m - first >= group_m) {
    const int cols = G / group_m;    // columns of the round's rectangle
    const int per = G / 8;           // tiles per XCD per round
    // split the rectangle into (8 / b) x b blocks, the most compact one
    int b = 8, best = 1 << 30;
#pragma unroll
    for (int c = 8; c >= 1; c >>= 1) {
      const int a = 8 / c;
      if (group_m % a == 0 && cols % c == 0 && group_m / a + cols / c < best) {
        best = group_m / a + cols / c;
        b = c;
      }
    }
    if (best < (1 << 30)) {
      const int h = group_m / (8 / b), w = cols / b;
      const int r = t - g * per_group;   // index in the band
      const int i = r % G;               // index in the round = virtual id
      const int x = i / per, s = i - (i / per) * per;
      pm = first + (x / b) * h + s % h;
      pn = (r - i) / group_m + (x % b) * w + s / h;
      return;
    }
  }
  grouped_tile(t, tiles_m, tiles_n, group_m, pm, pn);
}

// Tail launch of a two-launch product: unit u is quadrant u % 4 (row half
// (u % 4) / 2, column half u % 2) of tile base + u / 4 in the first launch's
// order (grid G, remap, tiles_m x tiles_n tiles, bands of group_m rows);
// (pm, pn) indexes the half-edge tiles.
TKG_HD inline void quadrant_tile(int u, int base, int G, int remap, int tiles_m, int tiles_n,
                                 int group_m, int& pm, int& pn) {
  int PM, PN;
  order_tile(base + u / 4, G, remap, tiles_m, tiles_n, group_m, PM, PN);
  pm = 2 * PM + (u & 3) / 2;
  pn = 2 * PN + (u & 1);
}

}  // namespace tkg
