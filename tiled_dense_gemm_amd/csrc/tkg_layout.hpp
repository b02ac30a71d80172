// LDS layout of the staged operand tiles: the XOR swizzle and the byte
// offsets every lane reads. Host- and device-side (constexpr), so the host
// library can report the exact addresses the kernels use.
//
// The pages' swizzle (page "ThunderKittens: Simple, Fast, and Adorable AI
// Kernels", section 3.4, "Shared Memory Tiles: Automated Swizzling to
// Eliminate Bank Conflicts"; page "ThunderKittens: 16x16 Tiles, ...",
// section "Warp level: tiles are the only data structure") XORs the 16-byte
// chunk index of an address with bits of its row so that the rows a tensor
// core load touches together land in different banks. The same idea is
// re-derived here for how a gfx950 wave reads LDS, by measurement (a probe
// kernel issuing each read pattern, with the SQ_LDS_BANK_CONFLICT counter):
//
// * LDS has 64 banks of 4 bytes. ds_read_b128 is served in phases of 16
//   consecutive lanes; the bank of an address is hashed from more address
//   bits than its word index, so layouts are checked by reading them on the
//   hardware rather than against a model.
// * An operand tile is stored row by row, one row per M (or N) index, with
//   ROW_BYTES bytes of K per row (both A and the column-major B are
//   K-contiguous). A row holds ROW_BYTES / 16 chunks of 16 bytes.
// * A fragment read is ds_read_b128: lane l reads 16 bytes of row
//   (l mod MI) of the fragment, lanes in groups of MI at different chunks
//   (MI = 16 or 32, the MFMA block). For 128-byte rows, among all 4096
//   linear row-to-mask maps on rows mod 16, the form below is one of the
//   1344 that read the 16x16 fragment pattern conflict-free, and it also
//   keeps the 32x32 patterns conflict-free; XOR-ing with (r & 7) ^ (r >> 3
//   & 1) instead, which a word-index bank map calls conflict-free, measures
//   2-way for the 16x16 pattern.
//
// For 128-byte rows (8 chunks): chunk' = chunk ^ (r & 7) ^ (7 * ((r >> 3) & 1))
// For  64-byte rows (4 chunks): chunk' = chunk ^ ((r >> 2) & 3)
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define TKG_HD __host__ __device__
#else
#define TKG_HD
#endif

namespace tkg {

// XOR mask applied to the chunk index of row `r` in a tile whose rows are
// `row_bytes` long (64 or 128). `on` = false gives the plain row-major
// layout (no swizzle), kept for the swizzle ablation.
TKG_HD constexpr uint32_t swz_mask(uint32_t row_bytes, uint32_t r, bool on = true) {
  return !on ? 0u
             : row_bytes == 128 ? ((r & 7u) ^ (((r >> 3) & 1u) * 7u)) : ((r >> 2) & 3u);
}

// Byte offset, inside a tile of `row_bytes`-long rows, of logical chunk
// `chunk` (16 bytes) of row `r`.
TKG_HD constexpr uint32_t swz_offset(uint32_t row_bytes, uint32_t r,
                                     uint32_t chunk, bool on = true) {
  return r * row_bytes + ((chunk ^ swz_mask(row_bytes, r, on)) << 4);
}

// Direct global->LDS staging: one wave instruction writes 1 KiB of LDS, lane
// l at byte 16*l. Writing in storage order means lane l fills physical chunk
// slot (l mod S) of row (l / S), S = row_bytes/16; it must therefore fetch
// the logical chunk that the swizzle stores there (XOR is an involution).
TKG_HD constexpr uint32_t dma_row(uint32_t row_bytes, uint32_t instr,
                                  uint32_t lane) {
  return instr * (1024u / row_bytes) + lane / (row_bytes / 16u);
}
TKG_HD constexpr uint32_t dma_chunk(uint32_t row_bytes, uint32_t instr,
                                    uint32_t lane, bool on = true) {
  return (lane % (row_bytes / 16u)) ^ swz_mask(row_bytes, dma_row(row_bytes, instr, lane), on);
}

// Rows of a slab that one staging instruction fills.
TKG_HD constexpr uint32_t dma_rows_per_instr(uint32_t row_bytes) {
  return 1024u / row_bytes;
}

// The per-lane part of a staging offset: instruction q's offset is
// q * dma_rows_per_instr * row_stride (the same for every lane) plus
// dma_lane_offset(row_bytes, q & 1, lane, row_stride). The swizzle of a row
// depends on q only through its parity (rows of one instruction share
// their upper bits), so two per-lane values cover every instruction.
TKG_HD constexpr uint32_t dma_lane_offset(uint32_t row_bytes, uint32_t parity,
                                          uint32_t lane, uint32_t row_stride,
                                          bool on = true) {
  return (dma_row(row_bytes, parity, lane) - parity * dma_rows_per_instr(row_bytes)) * row_stride +
         dma_chunk(row_bytes, parity, lane, on) * 16u;
}

// Checks that split for every instruction of a 256-row slab and every lane.
TKG_HD constexpr bool dma_offset_split_holds(uint32_t row_bytes, bool on) {
  const uint32_t stride = 1u << 20;  // any row stride larger than a row
  for (uint32_t q = 0; q < 256u / dma_rows_per_instr(row_bytes); ++q)
    for (uint32_t lane = 0; lane < 64; ++lane) {
      const uint32_t full =
          dma_row(row_bytes, q, lane) * stride + dma_chunk(row_bytes, q, lane, on) * 16u;
      const uint32_t split = q * dma_rows_per_instr(row_bytes) * stride +
                             dma_lane_offset(row_bytes, q & 1u, lane, stride, on);
      if (full != split) return false;
    }
  return true;
}
static_assert(dma_offset_split_holds(128, true) && dma_offset_split_holds(64, true) &&
                  dma_offset_split_holds(128, false) && dma_offset_split_holds(64, false),
              "staging offsets split into a uniform and a two-valued per-lane part");

}  // namespace tkg
