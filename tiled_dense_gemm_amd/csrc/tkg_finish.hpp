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
// Staged form: each wave owns an LDS area of RI*MI rows x RJ*MI columns of
// bf16. A round writes RI x RJ accumulator blocks there (8 bytes per lane,
// row-major; rows padded by 16 bytes so that the MI rows one write touches
// start in different banks, and every address is a per-lane base plus a
// constant), reads them back 16 bytes per lane in row order and stores them:
// one store instruction then writes 1 KiB as whole row pieces of RJ*MI*2
// bytes (64 to 256). A wave's LDS operations execute in order, so the next
// round may overwrite the area without a wait.
#pragma once
#include "tkg_device.hpp"

namespace tkg {

template <int MI, int FM, int FN, int RI, int RJ>
struct FinishShape {
  static constexpr int P = 64 / MI;
  static constexpr int NE = MI * MI / 64;      // accumulator elements per lane
  static constexpr int ROWS = RI * MI;
  static constexpr int RB = RJ * MI * 2;       // staged row bytes
  static constexpr int RS = RB + 16;           // LDS row stride (padded)
  static constexpr int CPR = RB / 16;          // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;         // rows per 1 KiB read
  static constexpr int BYTES = ROWS * RS;      // LDS bytes per wave
  static_assert(FM % RI == 0 && FN % RJ == 0, "rounds tile the wave tile");
  static_assert(CPR >= 4 && CPR <= 64 && (ROWS * RB) % 1024 == 0, "staged strip shape");
};

// The widest strip (RI = 1, RJ blocks of the wave tile's FN, at most 256
// bytes a row) that fits a per-wave LDS budget of BUDGET bytes, with rows of
// at least 64 bytes; USE is false when none fits (the finish then stores
// from registers).
template <int MI, int FM, int FN, int BUDGET>
struct FinishPlan {
  static constexpr bool fits(int rj) {
    return FN % rj == 0 && rj * MI * 2 >= 64 && rj * MI * 2 <= 256 &&
           MI * (rj * MI * 2 + 16) <= BUDGET && (MI * rj * MI * 2) % 1024 == 0;
  }
  static constexpr int fit(int rj) { return rj < 1 ? 0 : (fits(rj) ? rj : fit(rj / 2)); }
  static constexpr int RJ = fit(FN);
  static constexpr bool USE = RJ > 0;
  static constexpr int BYTES = USE ? MI * (RJ * MI * 2 + 16) : 0;
};

// Writes the wave tile whose top-left element is C[m0][n0] (ld = N) and
// zeroes the accumulators. SCALE multiplies by `scale` before rounding.
template <int MI, int FM, int FN, int RI, int RJ, bool SCALE, typename Acc>
__device__ __forceinline__ void finish_staged(Acc (&acc)[FM][FN], float scale,
                                              TKG_LDS uint8_t* stg, uint16_t* C,
                                              int M, int N, int m0, int n0,
                                              uint32_t lane) {
  using F = FinishShape<MI, FM, FN, RI, RJ>;
  const uint32_t lrow = lane % MI, lgrp = lane / MI;
  const bool vec8 = (N & 7) == 0;
  // per-lane bases: writes at row lrow, column 4*lgrp; reads at row
  // lane / CPR, chunk lane % CPR
  const uint32_t wbase = lrow * F::RS + 8 * lgrp;
  const uint32_t rrow = lane / F::CPR, rchunk = lane % F::CPR;
  const uint32_t rbase = rrow * F::RS + 16 * rchunk;
#pragma unroll
  for (int bi = 0; bi < FM; bi += RI) {
#pragma unroll
    for (int bj = 0; bj < FN; bj += RJ) {
#pragma unroll
      for (int ii = 0; ii < RI; ++ii)
#pragma unroll
        for (int jj = 0; jj < RJ; ++jj) {
#pragma unroll
          for (int g = 0; g < F::NE / 4; ++g) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
              v[u] = SCALE ? acc[bi + ii][bj + jj][4 * g + u] * scale
                           : acc[bi + ii][bj + jj][4 * g + u];
            // row ii*MI + lrow, column jj*MI + 4*P*g + 4*lgrp
            const uint2 pk = pack_bf16x4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<TKG_LDS u32x2_t*>(
                stg + wbase + ii * MI * F::RS + (jj * MI + 4 * F::P * g) * 2) = u32x2_t{pk.x, pk.y};
          }
          acc[bi + ii][bj + jj] = Acc{};
          // one block's values in flight at a time (register pressure)
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
      for (int q = 0; q < F::ROWS / F::RPI; ++q) {
        const i32x4_t v = lds_read<i32x4_t>(stg, rbase + q * F::RPI * F::RS);
        const int m = m0 + bi * MI + q * F::RPI + (int)rrow;
        const int n = n0 + bj * MI + 8 * (int)rchunk;
        if (m < M) {
          uint16_t* cp = C + (size_t)m * (size_t)N + n;
          if (vec8 && n + 7 < N) {
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
