// LDS layout of the attention forward kernel's key/value ring (host and
// device: the library reports the addresses so the bank model can check
// them without a GPU).
//
// A ring slot holds one block of BK = 32 keys: the K tile, then the V tile,
// each BK rows of D bf16 (ROWB = 2D bytes), a row's 16-byte chunk c stored
// at chunk c XOR f(row):
// * K is read 16 bytes per lane (one MFMA A fragment: 8 consecutive d of
//   one key), a 16-lane phase covering 16 consecutive keys at one chunk;
//   f_K(row) = (row / RPL) mod CPR spreads them over the 16 chunk positions
//   of a 256-byte bank line (RPL = rows per line, CPR = chunks per row).
// * V is read with the transposing 8-byte read: a 32-lane phase covers 4
//   consecutive keys (aligned to 4) x 4 consecutive chunks of one 64-byte
//   d-group; f_V(row) = 4 * ((row / RPL) mod (CPR / 4)) moves the 4 keys
//   into different 64-byte groups of the line.
#pragma once
#include <stdint.h>

#include "tkg_layout.hpp"  // TKG_HD

namespace tkg {

// Kernel shape: W waves of 32 query rows each (BQ = 32 W rows per
// workgroup), SLOTS ring slots of BK = 32 keys.
template <int D, int W, int SL>
struct AttnShape {
  static_assert(D == 64 || D == 128, "head dimension 64 or 128");
  static constexpr int WAVES = W;        // waves per workgroup
  static constexpr int QW = 32;          // query rows per wave
  static constexpr int BQ = WAVES * QW;  // query rows per workgroup
  static constexpr int BK = 32;          // keys per ring slot
  static constexpr int ROWB = 2 * D;     // bytes per K/V row
  static constexpr int CPR = D / 8;      // 16-byte chunks per row
  static constexpr int RPL = 256 / ROWB; // rows per 256-byte line
  static constexpr int TILE = BK * ROWB; // bytes of K (or V) per slot
  static constexpr int STAGE = 2 * TILE; // bytes per slot
  static constexpr int SLOTS = SL;
  static constexpr int NI = STAGE / 1024;  // 1 KiB DMA pieces per slot
  static constexpr int NPW = NI / WAVES;   // pieces per wave
  static constexpr int KS = D / 16;        // k-steps of Q K^T (its MFMAs per block)
  static constexpr int DB = D / 32;        // 32-row blocks of O^T (2 DB MFMAs per block)
  static_assert(NPW * WAVES == NI && (NI / 2) % NPW == 0, "a wave loads K or V, not both");
  static_assert(SLOTS >= 3, "ring of three slots at least");
};

TKG_HD constexpr uint32_t attn_rpl(uint32_t d) { return 256 / (2 * d); }
TKG_HD constexpr uint32_t attn_k_swz(uint32_t d, uint32_t row) {
  return (row / attn_rpl(d)) % (d / 8);
}
TKG_HD constexpr uint32_t attn_v_swz(uint32_t d, uint32_t row) {
  return 4 * ((row / attn_rpl(d)) % (d / 32));
}
// Byte offset, within its tile, of chunk c (16 bytes) of row `row`.
TKG_HD constexpr uint32_t attn_k_offset(uint32_t d, uint32_t row, uint32_t c) {
  return row * 2 * d + 16 * (c ^ attn_k_swz(d, row));
}
TKG_HD constexpr uint32_t attn_v_offset(uint32_t d, uint32_t row, uint32_t c) {
  return row * 2 * d + 16 * (c ^ attn_v_swz(d, row));
}

// Lane `lane`'s read of K fragment (kb, ks): key row 32 kb + lane % 32,
// chunk 2 ks + lane / 32 (a 32-key slot uses kb = 0).
TKG_HD constexpr uint32_t attn_k_read(uint32_t d, uint32_t lane, uint32_t kb, uint32_t ks) {
  return attn_k_offset(d, 32 * kb + lane % 32, 2 * ks + lane / 32);
}
// Lane `lane`'s address for transposing read t of V fragment (kb, s, db):
// key row 32 kb + 16 s + 8 t + 4 (lane / 32) + (lane % 16) / 4 and the
// 8 bytes at d = 32 db + 16 ((lane / 16) % 2) + 4 (lane % 4). The read hands
// lane 16g + 4a + b the b-th element of the 8 bytes addressed by lanes
// 16g + a + 4j (j = 0..3), i.e. column d = 32 db + lane % 32 of four keys.
TKG_HD constexpr uint32_t attn_v_read(uint32_t d, uint32_t lane, uint32_t kb, uint32_t s,
                                      uint32_t t, uint32_t db) {
  return attn_v_offset(d, 32 * kb + 16 * s + 8 * t + 4 * (lane / 32) + (lane % 16) / 4,
                       4 * db + 2 * ((lane / 16) % 2) + (lane % 4) / 2) +
         8 * ((lane % 4) % 2);
}

}  // namespace tkg
