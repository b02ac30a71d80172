// bf16 and fp8 tiled dense GEMM for gfx950 (MI355X).
//
// C = scale * A * B, fp32 accumulation, bf16 output. The structure follows
// the three levels of the pages' design, rebuilt for CDNA4:
//
// * Tiles (page "ThunderKittens: 16x16 Tiles, ...", section "Warp level:
//   tiles are the only data structure"; page "ThunderKittens: Simple, Fast,
//   and Adorable AI Kernels", section 3.4 "The Warp-Level Tile
//   Abstraction"): the 256x256 workgroup tile is a 2x2 grid of 128x128 wave
//   tiles, each a 4x4 grid of 32x32 MFMA accumulators (2x2 blocks of the
//   16x16 base tile). A is read row-major and B column-major, so both
//   operands are K-contiguous, the layout the matrix cores take.
// * Load-compute-store-finish (page 2, section 3.4 "The LCSF Template" and
//   "Multi-Stage Buffer: The Pipeline Depth Parameter", Table 1): every wave
//   streams its share of a K step straight from global memory into a ring of
//   STAGES LDS buffers, STAGES - 1 steps ahead of the MFMAs; s_waitcnt +
//   s_barrier play the part of arrive/expect. The loads of a step are issued
//   between the MFMAs of the current one. The finish step converts the fp32
//   accumulators (times the fp8 scale) to bf16 and stores them while the
//   next tile's first stages are already loading.
// * Swizzled LDS (page 2, section 3.4 "Shared Memory Tiles: Automated
//   Swizzling to Eliminate Bank Conflicts"): see tkg_layout.hpp.
// * Persistent grid and block order (page 2, section 3.4 "Persistent Grid
//   Launch", Table 2, and "Block Launch Order and L2 Cache Reuse", Table 3):
//   one workgroup per CU loops over output tiles in grouped order, with the
//   workgroup id remapped so each XCD works on neighbouring tiles.
//
// A stage holds 64 bytes of K per row: 32 bf16 (two 32x32x16 MFMA k-steps)
// or 64 fp8 (one 32x32x64 k-step).
#include "tkg_device.hpp"
#include "tkg_kernels.hpp"
#include "tkg_layout.hpp"

#include <type_traits>

namespace tkg {
namespace {

constexpr int BM = kBM, BN = kBN;
constexpr int BKB = 64;                  // K bytes per row per stage
constexpr int TILE = BM * BKB;           // 16 KiB per operand per stage
constexpr int STAGE_BYTES = 2 * TILE;    // A then B
constexpr int WAVES = kThreads / 64;     // 4, as 2 x 2
constexpr int WM = 128, WN = 128;        // wave tile
constexpr int FM = WM / 32, FN = WN / 32;  // 32x32 accumulators per wave
constexpr int DMA = TILE / 1024 / WAVES;   // b128 loads per wave per operand
constexpr int STAGES = 5;
static_assert(BM == BN, "A and B stage tiles share offsets");
static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS budget");

struct TileState {
  int m0, n0;
  __amdgpu_buffer_rsrc_t ra, rb;
};

__device__ __forceinline__ TileState tile_state(const DenseArgs& p, int t) {
  TileState s;
  if (t >= p.num_tiles) {  // past the last tile: empty resources read zeros
    s.m0 = s.n0 = 0;
    s.ra = make_rsrc(p.A, 0);
    s.rb = make_rsrc(p.B, 0);
    return s;
  }
  int pm, pn;
  grouped_tile(t, p.tiles_m, p.tiles_n, p.group_m, pm, pn);
  s.m0 = pm * BM;
  s.n0 = pn * BN;
  // Resources cover only the rows of this tile that exist, so rows past M
  // (or N) read as zeros. 256 * kbytes < 2^31 is checked on the host.
  const uint32_t rows_a = (uint32_t)min(p.M - s.m0, BM);
  const uint32_t rows_b = (uint32_t)min(p.N - s.n0, BN);
  s.ra = make_rsrc(p.A + (size_t)s.m0 * p.kbytes, rows_a * p.kbytes);
  s.rb = make_rsrc(p.B + (size_t)s.n0 * p.kbytes, rows_b * p.kbytes);
  return s;
}

template <int DT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_dense_kernel(DenseArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[STAGES * STAGE_BYTES];
  TKG_LDS uint8_t* smem = (TKG_LDS uint8_t*)smem_raw;

  // MFMA k-steps per stage and 16-byte reads per operand fragment
  constexpr int KSTEPS = (DT == kBf16) ? 2 : 1;
  constexpr int PARTS = (DT == kBf16) ? 1 : 2;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int G = gridDim.x;
  int t = xcd_virtual_id(blockIdx.x, G, p.xcd_remap);
  if (t >= p.num_tiles) return;

  // Number of K stages per tile. fp8 walks two stages per loop trip, so its
  // count is rounded up to even; the extra stage reads zeros.
  const uint32_t nk = (KSTEPS == 1) ? (p.nk + (p.nk & 1)) : p.nk;

  // ---- per-lane staging offsets (tile independent) -----------------------
  // DMA instruction i of this wave fills rows dma_row(q), q = wave*DMA + i;
  // with 64-byte rows the fetched chunk depends on the lane only.
  uint32_t dma_off[DMA];
#pragma unroll
  for (int i = 0; i < DMA; ++i) {
    const uint32_t q = wave * DMA + i;
    dma_off[i] = dma_row(BKB, q, lane) * p.kbytes + dma_chunk(BKB, q, lane) * 16u;
  }
  const uint32_t dma_kb = dma_chunk(BKB, wave * DMA, lane) * 16u;

  // ---- per-lane fragment read offsets ------------------------------------
  // Fragment rows are (multiple of 32) + lane%32, so the swizzle mask only
  // depends on the lane. k-step s of a stage reads chunk 2s + lane/32 (bf16)
  // or chunks 2*(lane/32) and 2*(lane/32) + 1 (fp8): the same K order for A
  // and B, so the MFMA reduces over matching elements.
  const uint32_t frow = lane & 31;
  const uint32_t khalf = lane >> 5;
  uint32_t roff[KSTEPS][PARTS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
    for (int q = 0; q < PARTS; ++q)
      roff[s][q] = swz_offset(BKB, frow, (DT == kBf16) ? 2 * s + khalf : 2 * khalf + q);
  const uint32_t a_base = wm * WM * BKB;
  const uint32_t b_base = TILE + wn * WN * BKB;

  // ---- load cursor: (tile lt, stage lkt), STAGES stages ahead -------------
  TileState cur = tile_state(p, t);
  TileState lts = cur;
  int lt = t;
  uint32_t lkt = 0;
  auto advance_load = [&]() {
    if (++lkt == nk) {
      lkt = 0;
      lt += G;
      lts = tile_state(p, lt);
    }
  };
  // Loads of stage (lts, lkt) into buffer `buf`; stages past K read zeros.
  auto issue = [&](int buf) {
    const uint32_t k0 = lkt * BKB;
    TKG_LDS uint8_t* st = smem + buf * STAGE_BYTES;
    const bool kok = k0 + dma_kb < p.kbytes;  // this lane's chunk exists
#pragma unroll
    for (int i = 0; i < DMA; ++i) {
      const uint32_t off = kok ? dma_off[i] + k0 : kOobOffset;
      const uint32_t q = wave * DMA + i;
      dma_b128(lts.ra, st + q * 1024, off);
      dma_b128(lts.rb, st + TILE + q * 1024, off);
    }
  };

  using Frag = typename std::conditional<DT == kBf16, bf16x8_t, i32x8_t>::type;
  Frag fa[2][FM], fb[2][FN];
  auto read_frags = [&](int buf, int s, Frag (&a)[FM], Frag (&b)[FN]) {
    const TKG_LDS uint8_t* st = smem + buf * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if constexpr (DT == kBf16) {
        a[i] = lds_read<bf16x8_t>(st, a_base + i * 32 * BKB + roff[s][0]);
      } else {
        const i32x4_t lo = lds_read<i32x4_t>(st, a_base + i * 32 * BKB + roff[s][0]);
        const i32x4_t hi = lds_read<i32x4_t>(st, a_base + i * 32 * BKB + roff[s][PARTS - 1]);
        a[i] = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if constexpr (DT == kBf16) {
        b[j] = lds_read<bf16x8_t>(st, b_base + j * 32 * BKB + roff[s][0]);
      } else {
        const i32x4_t lo = lds_read<i32x4_t>(st, b_base + j * 32 * BKB + roff[s][0]);
        const i32x4_t hi = lds_read<i32x4_t>(st, b_base + j * 32 * BKB + roff[s][PARTS - 1]);
        b[j] = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16_t{};
  auto mma_step = [&](const Frag (&a)[FM], const Frag (&b)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        // B first: the accumulator holds the transposed block (see finish)
        if constexpr (DT == kBf16)
          acc[i][j] = mfma_bf16(b[j], a[i], acc[i][j]);
        else
          acc[i][j] = mfma_fp8(b[j], a[i], acc[i][j]);
      }
  };

  // ---- prologue: the first STAGES stages in flight ------------------------
#pragma unroll
  for (int b = 0; b < STAGES; ++b) {
    issue(b);
    advance_load();
  }
  wait_vmcnt<(STAGES - 1) * 2 * DMA>();  // stage 0 has landed
  __syncthreads();
  read_frags(0, 0, fa[0], fb[0]);

  // One MFMA k-step. Register set c holds its fragments; the next k-step's
  // fragments go to set c ^ 1. At the last k-step of a stage the next stage
  // must have landed (wait + barrier); after the barrier every wave has read
  // the current stage, so its buffer is refilled STAGES stages ahead.
  int buf = 0;
  bool fresh_tile = false;  // finish stores are in flight
  auto kstep = [&](int c, int s, bool last) {
    if (!last) {
      read_frags(buf, s + 1, fa[c ^ 1], fb[c ^ 1]);
      mma_step(fa[c], fb[c]);
#pragma unroll
      for (int q = 0; q < FM + FN; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, PARTS, 0);      // ds_read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN), 0);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      if (fresh_tile) wait_vmcnt<0>();
      else wait_vmcnt<(STAGES - 2) * 2 * DMA>();
      fresh_tile = false;
      lds_barrier();
      issue(buf);
      const int nbuf = (buf + 1 == STAGES) ? 0 : buf + 1;
      read_frags(nbuf, 0, fa[c ^ 1], fb[c ^ 1]);
      mma_step(fa[c], fb[c]);
#pragma unroll
      for (int q = 0; q < FM + FN; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);          // DMA
        __builtin_amdgcn_sched_group_barrier(0x100, PARTS, 0);      // ds_read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN), 0);
      __builtin_amdgcn_sched_barrier(0);
      buf = nbuf;
      advance_load();
    }
  };

  for (;;) {
    // two k-steps per trip: one bf16 stage, or two fp8 stages
    for (uint32_t kt = 0; kt < nk; kt += 2 / KSTEPS) {
      if constexpr (KSTEPS == 2) {
        kstep(0, 0, false);
        kstep(1, 1, true);
      } else {
        kstep(0, 0, true);
        kstep(1, 0, true);
      }
    }

    // ---- finish: C[m][n .. n+3] from accumulator rows 4g .. 4g+3 ----------
    // The MFMA ran with B as its first operand, so accumulator (i, j) holds
    // the transposed 32x32 block: lane l owns C row m = l%32 and, in element
    // r, column 8*(r/4) + 4*(l/32) + r%4.
    const bool vec_ok = (p.N & 3) == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = cur.m0 + wm * WM + i * 32 + (int)frow;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = cur.n0 + wn * WN + j * 32 + 8 * g + 4 * (int)khalf;
          float v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            v[u] = (DT == kBf16) ? acc[i][j][4 * g + u] : acc[i][j][4 * g + u] * p.scale;
          const uint2 pk = pack_bf16x4(v[0], v[1], v[2], v[3]);
          if (m < p.M) {
            uint16_t* cp = p.C + (size_t)m * (size_t)p.N + n;
            if (vec_ok && n + 3 < p.N) {
              *reinterpret_cast<uint2*>(cp) = pk;
            } else {
              const uint16_t e[4] = {(uint16_t)(pk.x & 0xFFFF), (uint16_t)(pk.x >> 16),
                                     (uint16_t)(pk.y & 0xFFFF), (uint16_t)(pk.y >> 16)};
#pragma unroll
              for (int u = 0; u < 4; ++u)
                if (n + u < p.N) cp[u] = e[u];
            }
          }
        }
        acc[i][j] = f32x16_t{};
        // keep the scheduler from hoisting every accumulator read at once
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    fresh_tile = true;

    t += G;
    if (t >= p.num_tiles) break;
    cur = tile_state(p, t);
  }
  // The load cursor ran ahead into empty resources; let those LDS writes
  // land before the workgroup's LDS is released.
  wait_vmcnt<0>();
}

}  // namespace

uint32_t dense_stage_kbytes() { return BKB; }

hipError_t launch_dense(DenseType dt, const DenseArgs& a, int grid,
                        hipStream_t stream) {
  if (dt == kBf16)
    hipLaunchKernelGGL(gemm_dense_kernel<kBf16>, dim3(grid), dim3(kThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(gemm_dense_kernel<kFp8>, dim3(grid), dim3(kThreads), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace tkg
