// The "finish" step of a tile (page "ThunderKittens: Simple, Fast, and
// Adorable AI Kernels", section 3.4, "The LCSF Template": load, compute,
// store, finish): C = bf16_RNE(scale * acc) written from the accumulators
// of one wave.
//
// The MFMAs run with B as their first operand, so accumulator block (i, j)
// holds the transposed MIxMI block: lane l owns C row l % MI and, in its
// elements 4g .. 4g+3, the four columns 4*P*g + 4*(l / MI) .. +3 (P = 64 /
// MI). Stored straight from registers, one store instruction then covers MI
// rows with 16 (MI = 32) or 32 (MI = 16) contiguous bytes each, and the
// address processing of those many short pieces, not memory bandwidth,
// bounds the finish (measured: the same stores into a 128 KiB region that
// stays in L2 take as long).
//
// Staged form: each wave owns an LDS area of MI rows x RJ*MI columns of bf16
// (RB = RJ*MI*2 bytes a row, 64 to 256). A round packs RJ accumulator blocks
// to bf16, pairs them up across lanes with one permlane swap per dword so
// that every lane holds 8 consecutive columns of its row (16 bytes), writes
// them, reads the strip back 16 bytes per lane in row order and stores it:
// one store instruction then writes 1 KiB as whole row pieces of RB bytes.
// LDS layout, chosen by measurement (SQ_LDS_BANK_CONFLICT on each write
// and read pattern): the area is NR = MI*RB/256 lines of 256 bytes; row r
// lives in line R = r mod NR at slot h = r / NR, and its 16-byte chunk c at
// line chunk (h*RB/16 + c) XOR (R mod 16). The rows one write phase (16
// lanes) touches then sit in different lines at different chunks, and a
// read phase covers one whole line; both are served without conflicts
// (packing 128-byte rows one per line-half instead, with any XOR of row
// bits, measures 2-way on the writes). A wave's LDS operations execute in
// order, so the next round may overwrite the area without a wait.
#pragma once
#include "tkg_device.hpp"
#include "tkg_layout.hpp"

namespace tkg {

// ---- staging addresses (host and device: the library reports them) --------
// Byte offset (in the wave's area) where lane `lane` writes its 16 bytes
// for the write whose chunk constant is `cchunk` (MI = 32: 4*jj + 2*p for
// element-group pair p of block jj; MI = 16: 2*jj for blocks jj, jj+1), in
// a strip of `rb`-byte rows. After the swap the lane holds chunk
// cchunk ^ lchunk of row lane % MI; lchunk shares no bits with cchunk nor
// with the slot h * (rb/16), so the whole address is one XOR away from a
// per-lane base.
TKG_HD constexpr uint32_t finish_write_base(uint32_t mi, uint32_t rb, uint32_t lane) {
  const uint32_t lrow = lane % mi, lgrp = lane / mi;
  const uint32_t lchunk = mi == 32 ? lgrp : 2 * (lgrp & 1) + (lgrp >> 1);
  const uint32_t nr = mi * rb / 256, line = lrow % nr, slot = lrow / nr;
  return line * 256 + (((slot * (rb / 16)) ^ lchunk ^ (line % 16)) << 4);
}
TKG_HD constexpr uint32_t finish_write_offset(uint32_t mi, uint32_t rb, uint32_t lane,
                                              uint32_t cchunk) {
  return finish_write_base(mi, rb, lane) ^ (cchunk << 4);
}
// Read q covers lines 4q .. 4q+3: lane l reads line 4q + l/16 at line chunk
// l % 16, whose XOR (4q + l/16) mod 16 = (4q mod 16) ^ (l/16).
TKG_HD constexpr uint32_t finish_read_base(uint32_t lane) {
  return (lane / 16) * 256 + (((lane % 16) ^ (lane / 16)) << 4);
}
TKG_HD constexpr uint32_t finish_read_offset(uint32_t lane, uint32_t q) {
  return q * 1024 + (finish_read_base(lane) ^ (((4 * q) % 16) << 4));
}
// Row and first column of the strip that read q gives lane `lane`.
TKG_HD constexpr uint32_t finish_read_row(uint32_t mi, uint32_t rb, uint32_t lane, uint32_t q) {
  return ((lane % 16) / (rb / 16)) * (mi * rb / 256) + lane / 16 + 4 * q;
}
TKG_HD constexpr uint32_t finish_read_col(uint32_t rb, uint32_t lane) {
  return 8 * ((lane % 16) % (rb / 16));
}

template <int MI, int RJ>
struct FinishShape {
  static constexpr int P = 64 / MI;
  static constexpr int NE = MI * MI / 64;      // accumulator elements per lane
  static constexpr int RB = RJ * MI * 2;       // staged row bytes
  static constexpr int CPR = RB / 16;          // 16-byte chunks per row
  static constexpr int NR = MI * RB / 256;     // 256-byte LDS lines
  static constexpr int BYTES = MI * RB;        // LDS bytes per wave
  static_assert(RB == 64 || RB == 128 || RB == 256, "staged row of 64, 128 or 256 bytes");
  static_assert(MI == 32 || RJ % 2 == 0, "16x16 blocks pair up across lane groups");
  static_assert(NR % 4 == 0, "whole 1 KiB reads");
};

// The widest strip (RJ blocks of the wave tile's FN, rows of 64 to 256
// bytes) that fits a per-wave LDS budget of BUDGET bytes; USE is false when
// none fits (the finish then stores from registers).
template <int MI, int FM, int FN, int BUDGET>
struct FinishPlan {
  static constexpr bool fits(int rj) {
    return FN % rj == 0 && (MI == 32 || rj % 2 == 0) && rj * MI * 2 >= 64 &&
           rj * MI * 2 <= 256 && MI * rj * MI * 2 <= BUDGET;
  }
  static constexpr int fit(int rj) { return rj < 1 ? 0 : (fits(rj) ? rj : fit(rj / 2)); }
  static constexpr int RJ = fit(FN);
  static constexpr bool USE = RJ > 0;
  static constexpr int BYTES = USE ? MI * RJ * MI * 2 : 0;
};

// Writes the wave tile whose top-left element is C[m0][n0] (ld = N) and
// zeroes the accumulators. SCALE multiplies by `scale` before rounding.
template <int MI, int FM, int FN, int RJ, bool SCALE, typename Acc>
__device__ __forceinline__ void finish_staged(Acc (&acc)[FM][FN], float scale,
                                              TKG_LDS uint8_t* stg, uint16_t* C,
                                              int M, int N, int m0, int n0,
                                              uint32_t lane) {
  using F = FinishShape<MI, RJ>;
  const bool vec8 = (N & 7) == 0;
  uint32_t wlane = finish_write_base(MI, F::RB, lane);
  uint32_t rlane = finish_read_base(lane);
  const uint32_t rrow = finish_read_row(MI, F::RB, lane, 0);  // + 4q
  const uint32_t rcol = finish_read_col(F::RB, lane);
  // opaque per tile: keeps the per-round XORs below from being hoisted
  // into registers held across the whole kernel
  asm volatile("" : "+v"(wlane), "+v"(rlane));
  auto pk = [&](const Acc& a, int g) -> u32x2_t {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = SCALE ? a[4 * g + u] * scale : a[4 * g + u];
    const uint2 r = pack_bf16x4(v[0], v[1], v[2], v[3]);
    return u32x2_t{r.x, r.y};
  };
  auto put = [&](uint32_t cchunk, u32x2_t x, u32x2_t y) {
    // X in the low lane group of each swap pair, Y in the high one; after
    // the swap [X, Y] are 8 consecutive columns
    const auto s0 = MI == 32 ? __builtin_amdgcn_permlane32_swap(x[0], y[0], false, false)
                             : __builtin_amdgcn_permlane16_swap(x[0], y[0], false, false);
    const auto s1 = MI == 32 ? __builtin_amdgcn_permlane32_swap(x[1], y[1], false, false)
                             : __builtin_amdgcn_permlane16_swap(x[1], y[1], false, false);
    *reinterpret_cast<TKG_LDS i32x4_t*>(stg + (wlane ^ (cchunk << 4))) =
        i32x4_t{(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
  };
#pragma unroll
  for (int bi = 0; bi < FM; ++bi) {
#pragma unroll
    for (int bj = 0; bj < FN; bj += RJ) {
      if constexpr (MI == 32) {
#pragma unroll
        for (int jj = 0; jj < RJ; ++jj) {
#pragma unroll
          for (int pp = 0; pp < 2; ++pp)
            put(4 * jj + 2 * pp, pk(acc[bi][bj + jj], 2 * pp), pk(acc[bi][bj + jj], 2 * pp + 1));
          acc[bi][bj + jj] = Acc{};
          // one block's values in flight at a time (register pressure)
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < RJ; jj += 2) {
          put(2 * jj, pk(acc[bi][bj + jj], 0), pk(acc[bi][bj + jj + 1], 0));
          acc[bi][bj + jj] = Acc{};
          acc[bi][bj + jj + 1] = Acc{};
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int q = 0; q < F::NR / 4; ++q) {
        const i32x4_t v = lds_read<i32x4_t>(stg, q * 1024 + (rlane ^ (((4u * q) % 16) << 4)));
        const int m = m0 + bi * MI + (int)rrow + 4 * q;
        const int n = n0 + bj * MI + (int)rcol;
        if (m < M) {
          uint16_t* cp = C + (size_t)m * (size_t)N + n;
          if (vec8 && n + 7 < N) {
            // Rows of whole 128-byte lines are stored non-temporally: the
            // kernel never reads C, so its lines need not displace operand
            // lines in L2 (0.3-2% at 8192^3 and 16384^3, bf16 and fp8, same
            // process). 64-byte rows keep the default policy, under which
            // L2 merges the two halves of a line into one write (streamed,
            // the halves went out separately: 20-25% more bytes written).
            if constexpr (F::RB >= 128)
              __builtin_nontemporal_store(v, reinterpret_cast<i32x4_t*>(cp));
            else
              *reinterpret_cast<i32x4_t*>(cp) = v;
          } else {
#pragma unroll
            for (int u = 0; u < 8; ++u)
              if (n + u < N) cp[u] = (uint16_t)((uint32_t)v[u / 2] >> (16 * (u & 1)));
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

}  // namespace tkg
