// bf16 and fp8 tiled dense GEMM for gfx950 (MI355X).
//
// C = scale * A * B, fp32 accumulation, bf16 output. The structure follows
// the three levels of the pages' design, rebuilt for CDNA4:
//
// * Tiles (page "ThunderKittens: 16x16 Tiles, ...", section "Warp level:
//   tiles are the only data structure"; page "ThunderKittens: Simple, Fast,
//   and Adorable AI Kernels", section 3.4 "The Warp-Level Tile
//   Abstraction"): the 256x256 workgroup tile is a 2x4 grid of 128x64 wave
//   tiles (two waves per SIMD; a 2x2 grid of 128x128 tiles is the one-wave
//   configuration), each a grid of 16x16 (bf16) or 32x32 (fp8) MFMA
//   accumulators built on the 16x16 base tile. A is read row-major and B
//   column-major, so both operands are K-contiguous, the layout the matrix
//   cores take.
// * Load-compute-store-finish (page 2, section 3.4 "The LCSF Template" and
//   "Multi-Stage Buffer: The Pipeline Depth Parameter", Table 1): the waves
//   stream each K step straight from global memory into a ring of LDS slots
//   (one operand slab each, see Ring), several K steps ahead of the MFMAs;
//   s_waitcnt + s_barrier play the part of arrive/expect. The loads are
//   issued between the MFMAs of the current K step. The finish step converts
//   the fp32 accumulators (times the fp8 scale) to bf16 and stores them
//   while the next tile's first stages are already loading.
// * Swizzled LDS (page 2, section 3.4 "Shared Memory Tiles: Automated
//   Swizzling to Eliminate Bank Conflicts"): see tkg_layout.hpp.
// * Persistent grid and block order (page 2, section 3.4 "Persistent Grid
//   Launch", Table 2, and "Block Launch Order and L2 Cache Reuse", Table 3):
//   one workgroup per CU loops over output tiles in grouped order, with the
//   workgroup id remapped so each XCD works on neighbouring tiles.
//
// A K stage holds BKB bytes of K per row: BKB/2 bf16 or BKB fp8 elements,
// i.e. BKB / KSTEP_BYTES MFMA k-steps.
#include "tkg_device.hpp"
#include "tkg_finish.hpp"
#include "tkg_kernels.hpp"
#include "tkg_layout.hpp"

#include <type_traits>

namespace tkg {
namespace {

static_assert(kBM == kBN, "A and B slabs share offsets");

// How a stage's loads, reads and MFMAs are ordered.
// * kInterleaved: every wave spreads its LDS reads (and, if it loads, its
//   slab loads) over its own MFMAs in program order; one barrier per stage
//   frees both slots of the stage just read.
// * kEarlyB: as kInterleaved, plus a second barrier per stage right after
//   the last read of the stage's B slab (those reads come first in the
//   stage's second-to-last k-step), so the B slab is refilled half a stage
//   before the A slab: each operand slot is released after its own last
//   read (page "ThunderKittens reaches 22.4 PFLOPS on NVIDIA Rubin",
//   "Feeding the faster tensor cores": releasing an operand's buffer
//   early). The loads of a stage then go out over two k-steps.
// * kPingPong: the two waves of a SIMD alternate between a memory phase
//   (the k-step's LDS reads and its share of the slab loads) and an MFMA
//   phase, one barrier between phases; the second wave row starts one phase
//   late, so on every SIMD one wave reads while the other multiplies.
// * kEarlyReads: as kInterleaved, but the A fragments are double-buffered
//   like the B fragments, and every fragment read of the next k-step goes
//   out in the first half of the current k-step, in the order the next
//   k-step first uses them. The reads then finish long before the stage-end
//   barrier waits for them (with a single A set, the last A read is issued
//   just before a k-step's last MFMA and its latency shows at the barrier
//   and at the next k-step's first row). For one wave per SIMD, where no
//   partner wave covers such a wait.
enum Sched { kInterleaved = 0, kEarlyB = 1, kPingPong = 2, kEarlyReads = 3 };

// Ring shapes. The LDS ring holds SLOTS operand slabs; a slab is one
// operand's BT rows x BKB bytes of K, and a K stage is an A slab and a B
// slab. Slab j (stage j/2, operand j%2) lives in slot j % SLOTS, so an odd
// slot count lets the loads of a stage's A slab start a stage earlier than
// its B slab. SLOTS = 2 is the one-stage ring: the next stage is loaded
// only after every wave has finished the current one (no overlap).
// WAVES_N: the 2 x WAVES_N wave grid of the workgroup tile; 4 gives 8 waves
// (two per SIMD) of 128 x 64 each, 2 gives 4 waves of 128 x 128.
// LOADERS: 1 = only the waves of the first wave row (one per SIMD) issue
// the slab loads, so their partner wave on each SIMD keeps issuing MFMAs
// while the loaders wait for the memory pipeline to accept loads.
// MI: the MFMA block, 32 (32x32x16 bf16 / 32x32x64 fp8) or 16 (16x16x32 /
// 16x16x128). BT: the workgroup tile, BT x BT (256, or 128 for products
// with fewer 256 x 256 tiles than compute units). OCC: workgroups per
// compute unit (2 lets one workgroup's MFMAs cover the other's barriers and
// loads, for the short stages of 128 x 128 tiles). SWZ: 1 = the swizzled
// LDS layout, 0 = plain rows (the swizzle ablation). SCHED: see Sched.
struct Ring {
  int bkb, slots, waves_n, loaders, mi, bt, occ, swz, sched;
};
// One table per operand type (variant v selects entry v). Entry 0 is the
// default, the fastest measured at 8192^3 on random operands: for bf16 two
// waves per SIMD with 16x16x32 MFMAs (the 16x16 shape runs at a higher
// clock on the power-limited chip) and early fragment reads; for fp8 two
// waves per SIMD with 32x32x64 MFMAs (16x16x128 at two waves per SIMD
// spills; early reads measure the same). Entry kDenseSmallTileVariant (4)
// is what variant 0 resolves to for products with fewer 256 x 256 tiles
// than compute units, and kDenseLargeVariantBf16 (18) what it resolves to
// for bf16 products whose operands exceed the 256 MB last-level cache:
// their loads then come from HBM, and the 5-slot ring keeps half a stage
// more in flight. The others are the measured alternatives: ring depth (2
// and 5 slots; the 64-byte-stage entries sweep 1 to 5 stages), MFMA shape,
// waves per SIMD, swizzle off, the schedules. The ring-depth sweep runs on
// 32x32x16 blocks (on 16x16 blocks its deeper rings spill registers).
constexpr Ring kRingsBf16[] = {
    {128, 4, 4, 1, 16, 256, 1, 1, kEarlyReads},    // 0 default
    {128, 5, 4, 1, 16, 256, 1, 1, kInterleaved},   // 1 5-slot ring (2.5 stages)
    {128, 4, 4, 1, 32, 256, 1, 1, kInterleaved},   // 2 32x32x16 blocks
    {128, 4, 2, 0, 16, 256, 1, 1, kInterleaved},   // 3 one wave per SIMD, 128x128
    {128, 4, 2, 0, 16, 128, 2, 1, kEarlyReads},    // 4 128x128 tiles, 2 per CU
    {128, 4, 2, 0, 16, 128, 1, 1, kInterleaved},   // 5 128x128 tiles, 1 per CU
    {128, 4, 4, 1, 16, 256, 1, 0, kEarlyReads},    // 6 swizzle off
    {128, 4, 4, 1, 16, 256, 1, 1, kEarlyB},        // 7 early B release
    {128, 4, 4, 0, 16, 256, 1, 1, kPingPong},      // 8 ping-pong
    {128, 2, 4, 1, 16, 256, 1, 1, kInterleaved},   // 9 one-stage ring
    {64, 2, 4, 1, 32, 256, 1, 1, kInterleaved},    // 10 64-byte stages: 1 stage
    {64, 4, 4, 1, 32, 256, 1, 1, kInterleaved},    // 11 ... 2 stages
    {64, 6, 4, 1, 32, 256, 1, 1, kInterleaved},    // 12 ... 3 stages
    {64, 8, 4, 1, 32, 256, 1, 1, kInterleaved},    // 13 ... 4 stages
    {64, 10, 4, 1, 32, 256, 1, 1, kInterleaved},   // 14 ... 5 stages
    {64, 8, 4, 0, 16, 256, 1, 1, kPingPong},       // 15 ping-pong, 4 stages of 64 bytes
    {128, 4, 2, 0, 16, 256, 1, 1, kEarlyReads},    // 16 one wave per SIMD, early reads
    {128, 4, 4, 1, 16, 256, 1, 1, kInterleaved},   // 17 interleaved schedule
    {128, 5, 4, 1, 16, 256, 1, 1, kEarlyReads},    // 18 5-slot ring, early reads
    {128, 4, 2, 0, 16, 128, 2, 1, kInterleaved},   // 19 128x128 tiles, 2 per CU, interleaved
};
constexpr Ring kRingsFp8[] = {
    {128, 4, 4, 1, 32, 256, 1, 1, kInterleaved},   // 0 default
    {128, 5, 4, 1, 32, 256, 1, 1, kInterleaved},   // 1 5-slot ring
    {128, 4, 2, 0, 16, 256, 1, 1, kInterleaved},   // 2 one wave per SIMD, 16x16x128
    {128, 4, 2, 0, 32, 256, 1, 1, kInterleaved},   // 3 one wave per SIMD, 32x32x64
    {128, 4, 2, 0, 16, 128, 2, 1, kEarlyReads},    // 4 128x128 tiles, 2 per CU
    {128, 4, 2, 0, 16, 128, 1, 1, kInterleaved},   // 5 128x128 tiles, 1 per CU
    {128, 4, 4, 1, 32, 256, 1, 0, kInterleaved},   // 6 swizzle off
    {128, 4, 4, 1, 32, 256, 1, 1, kEarlyB},        // 7 early B release
    {128, 4, 4, 0, 32, 256, 1, 1, kPingPong},      // 8 ping-pong
    {128, 4, 2, 0, 32, 256, 1, 1, kEarlyReads},    // 9 one wave per SIMD, 32x32x64, early reads
    {128, 4, 2, 0, 16, 256, 1, 1, kEarlyReads},    // 10 one wave per SIMD, 16x16x128, early reads
    {128, 4, 4, 1, 32, 256, 1, 1, kEarlyReads},    // 11 two waves per SIMD, early reads
    {128, 5, 4, 1, 32, 256, 1, 1, kEarlyReads},    // 12 5-slot ring, early reads
    {128, 4, 2, 0, 16, 128, 2, 1, kInterleaved},   // 13 128x128 tiles, 2 per CU, interleaved
};
constexpr int kNumBf16 = sizeof(kRingsBf16) / sizeof(kRingsBf16[0]);
constexpr int kNumFp8 = sizeof(kRingsFp8) / sizeof(kRingsFp8[0]);
static_assert(kRingsBf16[kDenseLargeVariantBf16].slots == 5 &&
                  kRingsBf16[kDenseLargeVariantBf16].bt == 256,
              "the large-product entry is the 5-slot ring");
static_assert(kRingsBf16[kDenseSmallTileVariant].bt == 128 &&
                  kRingsFp8[kDenseSmallTileVariant].bt == 128,
              "the small-tile entry has 128 x 128 tiles");
template <int DT>
constexpr Ring ring_of(int v) {
  return DT == kBf16 ? kRingsBf16[v] : kRingsFp8[v];
}
inline Ring ring_at(DenseType dt, int v) { return dt == kBf16 ? kRingsBf16[v] : kRingsFp8[v]; }

struct TileState {
  int m0, n0;
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t k0, nk;   // the unit's first K byte and its stage count
};

// Work unit u: split u % splits of tile u / splits (one split: the tile).
// The unit's stage count is rounded up to whole loop trips (TRIP stages);
// the extra stage reads zeros.
template <int BT, int BKB, int TRIP, bool SPLITK>
__device__ __forceinline__ TileState tile_state(const DenseArgs& p, int u) {
  TileState s;
  if (u >= p.num_units) {  // past the last unit: empty resources read zeros
    s.m0 = s.n0 = 0;
    s.ra = make_rsrc(p.A, 0);
    s.rb = make_rsrc(p.B, 0);
    s.k0 = 0;
    s.nk = TRIP;
    return s;
  }
  int t = u;
  uint32_t klen = p.kbytes;
  s.k0 = 0;
  if constexpr (SPLITK) {
    t = u / p.splits;
    s.k0 = (uint32_t)(u - t * p.splits) * p.ksplit;
    klen = min(p.ksplit, p.kbytes - s.k0);
  }
  const uint32_t nk_raw = (klen + BKB - 1) / BKB;
  s.nk = (TRIP == 2) ? (nk_raw + (nk_raw & 1)) : nk_raw;
  int pm, pn;
  if (!SPLITK && BT == 128 && p.quad_base >= 0) {
    // a quadrant of a 256 x 256 tile the full-round launch left over
    quadrant_tile(t, p.quad_base, p.quad_grid, p.quad_remap, p.quad_tiles_m, p.quad_tiles_n,
                  p.quad_group_m, pm, pn);
  } else {
    // split-K launches use the grouped order (the reduction walks tiles in it)
    order_tile(t, gridDim.x, SPLITK ? 0 : p.xcd_remap, p.tiles_m, p.tiles_n, p.group_m, pm, pn);
  }
  s.m0 = pm * BT;
  s.n0 = pn * BT;
  // Resources cover only the rows of this tile that exist. A load reads
  // zeros past them only where its whole offset is per-lane (the masked
  // instance, chosen on the host for ragged tiles): the scalar offset is
  // excluded from the buffer bounds check. 256 * kbytes < 2^31 is checked
  // on the host.
  const uint32_t rows_a = (uint32_t)min(p.M - s.m0, BT);
  const uint32_t rows_b = (uint32_t)min(p.N - s.n0, BT);
  s.ra = make_rsrc(p.A + (size_t)s.m0 * p.kbytes, rows_a * p.kbytes);
  s.rb = make_rsrc(p.B + (size_t)s.n0 * p.kbytes, rows_b * p.kbytes);
  return s;
}

template <int DT, int BKB, int SLOTS, int WAVES_N, int LOADERS, int MI, int BT, int OCC,
          int SWZ, int SCHED, bool SPLITK, bool MASKED>
__global__ __launch_bounds__(128 * WAVES_N)
__attribute__((amdgpu_waves_per_eu(OCC * WAVES_N / 2, OCC * WAVES_N / 2)))
void gemm_dense_kernel(DenseArgs p) {
  constexpr int WAVES = 2 * WAVES_N;
  constexpr int WM = BT / 2, WN = BT / WAVES_N;   // wave tile
  constexpr int FM = WM / MI, FN = WN / MI;       // MIxMI accumulators
  constexpr int NMMA = FM * FN;                   // MFMAs per k-step
  constexpr int SLAB = BT * BKB;           // bytes of one operand slab
  // waves that issue slab loads, and b128 loads per such wave per slab
  constexpr int LOAD_WAVES = LOADERS ? WAVES_N : WAVES;
  constexpr int DMA = SLAB / 1024 / LOAD_WAVES;
  static_assert(SLOTS == 2 || SLOTS >= 4, "one stage, or two stages at least");
  static_assert(FM >= 1 && FN >= 1 && DMA >= 1, "wave tile and loads fit the workgroup tile");
  constexpr int LDS_BUDGET = 160 * 1024 / OCC;   // per workgroup
  static_assert(SLOTS * SLAB <= LDS_BUDGET, "LDS budget");
  // the finish stages through the LDS the ring leaves free (tkg_finish.hpp)
  using FP = FinishPlan<MI, FM, FN, (LDS_BUDGET - SLOTS * SLAB) / WAVES>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[SLOTS * SLAB + WAVES * FP::BYTES];
  TKG_LDS uint8_t* smem = (TKG_LDS uint8_t*)smem_raw;
  constexpr bool SW = SWZ != 0;

  // K bytes per row of one MFMA k-step, 16-byte chunks per k-step (CPK),
  // lane groups sharing a row (P: lanes l, l+MI, ... read the same row at
  // different chunks) and 16-byte reads per lane per fragment (PARTS). The
  // interleaved loop body runs an even number of k-steps (the fragment
  // registers alternate between two sets): one stage, or two when a stage
  // is a single k-step.
  constexpr int KSTEP_BYTES = (DT == kBf16 ? 32 : 64) * (32 / MI);
  constexpr int KSTEPS = BKB / KSTEP_BYTES;
  constexpr int CPK = KSTEP_BYTES / 16;
  constexpr int P = 64 / MI;
  constexpr int PARTS = CPK / P;
  constexpr bool PP = SCHED == kPingPong;
  constexpr int TRIP_STAGES = (KSTEPS >= 2 || PP) ? 1 : 2;
  using Acc = typename std::conditional<MI == 32, f32x16_t, f32x4_t>::type;
  constexpr int NE = MI * MI / 64;                // accumulator elements per lane
  static_assert(KSTEPS % 2 == 0 || KSTEPS == 1, "k-steps per trip must be even");
  static_assert(SCHED != kEarlyB || (KSTEPS >= 2 && SLOTS == 4),
                "early B release needs two k-steps per stage and a two-stage ring");
  static_assert(!PP || (WAVES_N == 4 && !LOADERS && SLOTS % 2 == 0 && SLOTS >= 4),
                "ping-pong pairs the two wave rows, and every wave loads");
  static_assert(SCHED != kEarlyReads || SLOTS >= 4, "early reads need a two-stage ring");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int G = gridDim.x;
  int t = xcd_virtual_id(blockIdx.x, G, p.xcd_remap);   // work unit
  if (t >= p.num_units) return;

  // ---- per-lane staging offsets (tile independent) -----------------------
  // DMA instruction i of this wave fills rows dma_row(q), q = lw*DMA + i.
  // loader index of this wave (waves with wm > 0 load nothing if LOADERS)
  const int lw = LOADERS ? wn : wave;
  const bool loader = !LOADERS || wm == 0;
  // Unmasked, the offset of load q is a uniform part (scalar) plus one of
  // two per-lane values (dma_lane_offset). The hardware leaves the scalar
  // part out of the buffer bounds check, so that form only runs when every
  // row and K chunk a load reaches exists. Masked (a ragged M or N tile, or
  // a K tail), each load keeps its full per-lane offset, bounds-checked, and
  // its K chunk for the K test.
  constexpr int NOFF = MASKED ? DMA : 2;
  uint32_t dma_off[NOFF], dma_kb[MASKED ? DMA : 1];
  if constexpr (MASKED) {
#pragma unroll
    for (int i = 0; i < DMA; ++i) {
      const uint32_t q = lw * DMA + i;
      dma_kb[i] = dma_chunk(BKB, q, lane, SW) * 16u;
      dma_off[i] = dma_row(BKB, q, lane) * p.kbytes + dma_kb[i];
    }
  } else {
    dma_kb[0] = 0;
#pragma unroll
    for (int par = 0; par < 2; ++par)
      dma_off[par] = dma_lane_offset(BKB, par, lane, p.kbytes, SW);
  }
  const uint32_t rows_step = dma_rows_per_instr(BKB) * p.kbytes;  // bytes per load q

  // ---- per-lane fragment read offsets ------------------------------------
  // Fragment rows are (multiple of MI) + lane%MI, so the swizzle mask only
  // depends on the lane. Lane l reads, at k-step s, the PARTS chunks from
  // s*CPK + (l/MI)*PARTS on: the same K order for A and B, so the MFMA
  // reduces over matching elements.
  const uint32_t frow = lane % MI;
  const uint32_t kpart = lane / MI;
  uint32_t roff[KSTEPS][PARTS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
    for (int q = 0; q < PARTS; ++q)
      roff[s][q] = swz_offset(BKB, frow, s * CPK + kpart * PARTS + q, SW);
  const uint32_t a_base = wm * WM * BKB;   // within an A slab
  const uint32_t b_base = wn * WN * BKB;   // within a B slab

  // ---- load cursor: slab (tile lt, stage lkt, operand lop) ----------------
  TileState cur = tile_state<BT, BKB, TRIP_STAGES, SPLITK>(p, t);
  TileState lts = cur;
  int lt = t;
  uint32_t lkt = 0, lop = 0, lslot = 0;
  auto advance_load = [&]() {
    lslot = (lslot + 1 == SLOTS) ? 0 : lslot + 1;
    if (lop == 0) {
      lop = 1;
    } else {
      lop = 0;
      if (++lkt == lts.nk) {
        lkt = 0;
        lt += G;
        lts = tile_state<BT, BKB, TRIP_STAGES, SPLITK>(p, lt);
      }
    }
  };
  // The cursor's next slab: its resource, slot and K offset (then advance).
  struct SlabLoad {
    __amdgpu_buffer_rsrc_t r;
    uint32_t slot, k0;
  };
  auto next_slab = [&]() {
    SlabLoad s;
    s.r = lop ? lts.rb : lts.ra;
    s.slot = lslot;
    s.k0 = lts.k0 + lkt * BKB;
    advance_load();
    return s;
  };
  // Load i of one slab. Unmasked, every row and chunk exists: the per-lane
  // offset is loop invariant and the row block and stage K offset are the
  // scalar offset. Masked, rows past M or N and chunks past K read zeros.
  auto issue_one = [&](const SlabLoad& s, int i) {
    TKG_LDS uint8_t* dst = smem + s.slot * SLAB + (lw * DMA + i) * 1024;
    if constexpr (MASKED) {
      const uint32_t off = (s.k0 + dma_kb[i] < p.kbytes) ? dma_off[i] + s.k0 : kOobOffset;
      dma_b128(s.r, dst, off);
    } else {
      const uint32_t q = lw * DMA + i;
      dma_b128_soff(s.r, dst, dma_off[q & 1], s.k0 + q * rows_step);
    }
  };
  auto issue = [&](const SlabLoad& s) {
#pragma unroll
    for (int i = 0; i < DMA; ++i) issue_one(s, i);
  };

  using Frag = typename std::conditional<DT == kBf16, bf16x8_t, i32x8_t>::type;
  auto read_one = [&](const TKG_LDS uint8_t* base, uint32_t row0, int s, Frag& v) {
    if constexpr (DT == kBf16) {
      v = lds_read<bf16x8_t>(base, row0 + roff[s][0]);
    } else {
      const i32x4_t lo = lds_read<i32x4_t>(base, row0 + roff[s][0]);
      const i32x4_t hi = lds_read<i32x4_t>(base, row0 + roff[s][PARTS - 1]);
      v = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  auto mma = [&](const Frag& b, const Frag& a, Acc& c) {
    // B first: the accumulator holds the transposed block (see finish)
    if constexpr (MI == 32) {
      if constexpr (DT == kBf16) c = mfma_bf16(b, a, c);
      else c = mfma_fp8(b, a, c);
    } else {
      if constexpr (DT == kBf16) c = mfma16_bf16(b, a, c);
      else c = mfma16_fp8(b, a, c);
    }
  };

  // ---- finish: C[m][n .. n+3] from accumulator elements 4g .. 4g+3 -------
  // The MFMA ran with B as its first operand, so accumulator (i, j) holds
  // the transposed MIxMI block: lane l owns C row m = l%MI and, in element
  // r, column 4*P*(r/4) + 4*(l/MI) + r%4. Zeroes the accumulators.
  auto finish = [&](Acc (&acc)[FM][FN]) {
    if constexpr (SPLITK) {
      // split-K: this unit's fp32 partial sums, in accumulator order
      // (wave, block, element group, lane), 16 bytes per lane per store
      float* w = p.ws + ((size_t)t * WAVES + wave) * (FM * FN * NE * 64);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
          for (int g = 0; g < NE / 4; ++g)
            *reinterpret_cast<f32x4_t*>(w + (((i * FN + j) * (NE / 4) + g) * 64 + lane) * 4) =
                f32x4_t{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                        acc[i][j][4 * g + 3]};
          acc[i][j] = Acc{};
          __builtin_amdgcn_sched_barrier(0);
        }
    } else if constexpr (FP::USE) {
      finish_staged<MI, FM, FN, FP::RJ, DT != kBf16>(
          acc, p.scale, smem + SLOTS * SLAB + wave * FP::BYTES, p.C, p.M, p.N,
          cur.m0 + wm * WM, cur.n0 + wn * WN, (uint32_t)lane);
    } else {
      const bool vec_ok = (p.N & 3) == 0;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = cur.m0 + wm * WM + i * MI + (int)frow;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
          for (int g = 0; g < NE / 4; ++g) {
            const int n = cur.n0 + wn * WN + j * MI + 4 * P * g + 4 * (int)kpart;
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
          acc[i][j] = Acc{};
          // keep the scheduler from hoisting every accumulator read at once
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  // The interleaved and early-release loops, in two copies: waves that
  // issue slab loads and (with LOADERS) waves that only compute. Both run
  // the same barriers.
  auto main_loop = [&](auto loader_tag) {
  constexpr bool IS_LOADER = decltype(loader_tag)::value;
  // Fragment registers. A fragment i is last used by MFMA (i, FN-1) of a
  // k-step, so the next k-step's A fragment i is read into the same
  // registers right after it. B fragments are used until the k-step's last
  // row of MFMAs: two sets, the next one read at the k-step's start, unless
  // registers are short (fp8 16x16 at two waves per SIMD: one set, each B
  // fragment re-read right after its last use, a few MFMAs before its next
  // one).
  constexpr bool EARLY = SCHED == kEarlyReads;
  constexpr bool B_SINGLE = (DT == kFp8 && MI == 16 && WAVES_N == 4) && !EARLY;
  constexpr int BSETS = B_SINGLE ? 1 : 2;
  constexpr int ASETS = EARLY ? 2 : 1;
  Frag fa[ASETS][FM], fb[BSETS][FN];
  auto read_a = [&](int aslot, int s, int i, Frag& v) {
    read_one(smem + aslot * SLAB, a_base + i * MI * BKB, s, v);
  };
  auto read_b = [&](int bslot, int s, int j, Frag& v) {
    read_one(smem + bslot * SLAB, b_base + j * MI * BKB, s, v);
  };

  Acc acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = Acc{};
  // One k-step in program order: after MFMA (i, j) come the instructions of
  // its slot, and a scheduling fence keeps that order, so loads and reads
  // are spread over the MFMAs exactly as written. Fragment reads of the
  // next k-step come from slots (ns_a, ns_b) at k-step ns (none if !READS).
  auto kstep_body = [&](int c, int ns, int ns_a, int ns_b, auto&& extra, auto reads_tag) {
    constexpr bool READS = decltype(reads_tag)::value;
    Frag (&b)[FN] = fb[B_SINGLE ? 0 : c];
    Frag (&bn)[FN] = fb[B_SINGLE ? 0 : c ^ 1];
    Frag (&a)[FM] = fa[EARLY ? c : 0];
    Frag (&an)[FM] = fa[EARLY ? c ^ 1 : 0];
    // early reads: read r (first-use order b0, a0, b1 .. b[FN-1], a1 ..
    // a[FM-1]) follows MFMA slot r * RSTRIDE, within the k-step's first half
    constexpr int NREAD = FM + FN;
    constexpr int RSTRIDE = NMMA >= 2 * NREAD ? NMMA / (2 * NREAD) : 1;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        mma(b[j], a[i], acc[i][j]);
        const int q = i * FN + j;
        if constexpr (READS) {
          if constexpr (EARLY) {
            if (q % RSTRIDE == 0 && q / RSTRIDE < NREAD) {
              const int r = q / RSTRIDE;
              if (r == 0) read_b(ns_b, ns, 0, bn[0]);
              else if (r == 1) read_a(ns_a, ns, 0, an[0]);
              else if (r <= FN) read_b(ns_b, ns, r - 1, bn[r - 1]);
              else read_a(ns_a, ns, r - FN, an[r - FN]);
            }
          } else {
            if constexpr (B_SINGLE) {
              if (i == FM - 1) read_b(ns_b, ns, j, bn[j]);
            } else {
              if (q < FN) read_b(ns_b, ns, q, bn[q]);
            }
            if (j == FN - 1) read_a(ns_a, ns, i, fa[0][i]);
          }
        }
        extra(q);
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  using WithReads = std::true_type;

  // ---- prologue: the first SLOTS slabs in flight -------------------------
#pragma unroll
  for (int b = 0; b < SLOTS; ++b) {
    const SlabLoad l = next_slab();
    if constexpr (IS_LOADER) issue(l);
  }
  wait_vmcnt<(SLOTS - 2) * DMA>();  // slabs 0 and 1 (stage 0) have landed
  __syncthreads();
  int aslot = 0, bslot = 1;         // slots of the stage being computed
#pragma unroll
  for (int i = 0; i < FM; ++i) read_a(aslot, 0, i, fa[0][i]);
#pragma unroll
  for (int j = 0; j < FN; ++j) read_b(bslot, 0, j, fb[0][j]);

  // One MFMA k-step; c selects the B register set. At the last k-step of a
  // stage the next stage must have landed (wait + barrier): SLOTS slabs were
  // issued before stage k's end, so at most SLOTS - 4 slabs may still be
  // loading. After the barrier every wave has read the current stage, so
  // its two slots are refilled with the next two slabs of the cursor, the
  // loads spread over the MFMAs.
  bool fresh_tile = false;  // finish stores are in flight
  constexpr int NDMA = 2 * DMA;             // slab loads per stage boundary
  // MFMA slots the loads are spread over: the whole boundary k-step, or its
  // first three quarters when a stage is a single k-step (the loads are
  // waited for at the next boundary, one k-step later, and need time to
  // land; measured: all of it 2640, half 2980, three quarters 3010 TFLOP/s
  // for fp8 16x16 at 8192^3)
  constexpr int NSPAN = KSTEPS == 1 ? (3 * NMMA + 3) / 4 : NMMA;
  // early B release: the B slab's loads go out over the MFMAs after the
  // second-to-last k-step's B reads (and the barrier behind them), the A
  // slab's over the last k-step
  constexpr int QREL = FN - 1;              // MFMA slot of the last B read
  constexpr int NSPAN_B = NMMA > FN ? NMMA - FN : 1;
  auto kstep = [&](int c, int s, const SlabLoad& l0, const SlabLoad& l1) {
    const bool last = s == KSTEPS - 1;
    if (!last) {
      bool done = false;
      if constexpr (SCHED == kEarlyB) {
        if (s == KSTEPS - 2) {
          // finish stores in flight (a tile's first stage): drain them and
          // the ring before the k-step, not inside its MFMA chain
          if (fresh_tile) wait_vmcnt<0>();
          fresh_tile = false;
          kstep_body(c, s + 1, aslot, bslot, [&](int q) {
            // every wave has read this stage's B slab: release it
            if (q == QREL) lds_barrier();
            if constexpr (IS_LOADER) {
              if (q > QREL) {
                const int r = q - FN;
#pragma unroll
                for (int d = r * DMA / NSPAN_B; d < (r + 1) * DMA / NSPAN_B; ++d)
                  issue_one(l1, d);
              }
            }
          }, WithReads{});
          done = true;
        }
      }
      if (!done) kstep_body(c, s + 1, aslot, bslot, [&](int) {}, WithReads{});
    } else if constexpr (SLOTS == 2) {
      // one-stage ring: finish the stage's MFMAs, then every wave is done
      // with both slots; load the next stage into them, wait, read
      kstep_body(c, 0, aslot, bslot, [&](int) {}, std::false_type{});
      lds_barrier();
      if constexpr (IS_LOADER) {
        issue(l0);
        issue(l1);
      }
      wait_vmcnt<0>();
      fresh_tile = false;
      lds_barrier();
      Frag (&bn)[FN] = fb[B_SINGLE ? 0 : c ^ 1];
#pragma unroll
      for (int i = 0; i < FM; ++i) read_a(aslot, 0, i, fa[0][i]);
#pragma unroll
      for (int j = 0; j < FN; ++j) read_b(bslot, 0, j, bn[j]);
    } else {
      if constexpr (SCHED == kEarlyB) {
        wait_vmcnt<DMA>();   // stage k+1 landed; stage k+2's B may be in flight
      } else {
        if (fresh_tile) wait_vmcnt<0>();
        else wait_vmcnt<(SLOTS - 4) * DMA>();
        fresh_tile = false;
      }
      lds_barrier();
      const int na = (aslot + 2) % SLOTS, nb = (bslot + 2) % SLOTS;
      kstep_body(c, 0, na, nb, [&](int q) {
        if constexpr (IS_LOADER) {
          if constexpr (SCHED == kEarlyB) {
#pragma unroll
            for (int d = q * DMA / NMMA; d < (q + 1) * DMA / NMMA; ++d) issue_one(l0, d);
          } else {
#pragma unroll
            for (int d = q * NDMA / NSPAN; d < (q + 1) * NDMA / NSPAN && d < NDMA; ++d) {
              if (d < DMA) issue_one(l0, d);
              else issue_one(l1, d - DMA);
            }
          }
        }
      }, WithReads{});
      aslot = na;
      bslot = nb;
    }
  };

  for (;;) {
    for (uint32_t kt = 0; kt < cur.nk; kt += TRIP_STAGES) {
#pragma unroll
      for (int st = 0; st < TRIP_STAGES; ++st) {
        // the cursor moves (and may branch to a new tile) at the top of the
        // stage, so that no MFMA of the stage is moved past that branch and
        // behind the stage-end wait
        const SlabLoad l0 = next_slab();
        const SlabLoad l1 = next_slab();
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) kstep((st * KSTEPS + s) & 1, s, l0, l1);
      }
    }
    finish(acc);
    fresh_tile = true;

    t += G;
    if (t >= p.num_units) break;
    cur = tile_state<BT, BKB, TRIP_STAGES, SPLITK>(p, t);
  }
  };

  // ---- ping-pong ---------------------------------------------------------
  // Wave row g = wm. Per k-step each wave runs a memory phase M (its
  // fragment reads of the k-step and, at a stage's first k-step, its share
  // of the slab loads; then the reads' wait) and an MFMA phase C, with a
  // workgroup barrier after each. Row 1 passes one extra barrier first, so
  // between two barriers one row is in M and the other in C: on every SIMD
  // one wave multiplies while its partner reads. A ring of D = SLOTS/2
  // stages: the slots of stage i-1 are free once row 1 has read it (before
  // the M phases of stage i), so stage i-1+D goes out during stage i's
  // first M phase; it must have landed before row 0 reads it, so each wave
  // waits for its loads of stage i+1 at the end of its last phase before
  // that read (row 0: C of stage i's last k-step; row 1: its M).
  auto pingpong_loop = [&](auto) {   // generic: instantiated only when called
    constexpr int D = SLOTS / 2;
    Frag fa[FM], fb[FN];
    Acc acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = Acc{};
#pragma unroll
    for (int b = 0; b < SLOTS; ++b) issue(next_slab());
    wait_vmcnt<(SLOTS - 2) * DMA>();   // this wave's loads of stage 0
    __syncthreads();
    if (wm == 1) __builtin_amdgcn_s_barrier();
    bool fresh_tile = false, first_stage = true;
    int aslot = 0, bslot = 1;
    auto stage_wait = [&]() {
      if (fresh_tile) wait_vmcnt<0>();
      else wait_vmcnt<(D - 2) * 2 * DMA>();
      fresh_tile = false;
    };
    for (;;) {
      for (uint32_t kt = 0; kt < cur.nk; ++kt) {
        SlabLoad l0, l1;
        const bool refill = !first_stage;
        if (refill) {
          l0 = next_slab();
          l1 = next_slab();
        }
        first_stage = false;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          // M: reads of k-step s, loads spread between them
#pragma unroll
          for (int f = 0; f < FM + FN; ++f) {
            if (f < FM) read_one(smem + aslot * SLAB, a_base + f * MI * BKB, s, fa[f]);
            else read_one(smem + bslot * SLAB, b_base + (f - FM) * MI * BKB, s, fb[f - FM]);
            if (s == 0 && refill) {
#pragma unroll
              for (int d = f * 2 * DMA / (FM + FN); d < (f + 1) * 2 * DMA / (FM + FN); ++d) {
                if (d < DMA) issue_one(l0, d);
                else issue_one(l1, d - DMA);
              }
            }
          }
          if (s == KSTEPS - 1 && wm == 1) stage_wait();
          lds_barrier();
          // C: the k-step's MFMAs
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) mma(fb[j], fa[i], acc[i][j]);
          if (s == KSTEPS - 1 && wm == 0) stage_wait();
          if (s == KSTEPS - 1 && kt + 1 == cur.nk) {
            finish(acc);
            fresh_tile = true;
          }
          __builtin_amdgcn_s_barrier();
        }
        aslot = (aslot + 2) % SLOTS;
        bslot = (bslot + 2) % SLOTS;
      }
      if (cur.nk == 0) {   // K = 0: no k-step wrote the (zero) tile
        finish(acc);
        fresh_tile = true;
      }
      t += G;
      if (t >= p.num_units) break;
      cur = tile_state<BT, BKB, TRIP_STAGES, SPLITK>(p, t);
    }
    if (wm == 0) __builtin_amdgcn_s_barrier();
  };

  if constexpr (PP) {
    pingpong_loop(0);
  } else {
    if (loader)
      main_loop(std::true_type{});
    else
      main_loop(std::false_type{});
  }
  // The load cursor ran ahead into empty resources; let those LDS writes
  // land before the workgroup's LDS is released.
  wait_vmcnt<0>();
}

// Split-K reduction: one workgroup per output tile; thread q of the tile's
// BT*BT/4 element groups adds the splits' partials in order, scales, rounds
// to bf16 and stores the four columns it covers (the layout of the main
// kernel's accumulators: wave, block (i, j), element group g, lane).
template <int DT, int WAVES_N, int MI, int BT>
__global__ __launch_bounds__(256) void gemm_dense_reduce(DenseArgs p) {
  constexpr int WAVES = 2 * WAVES_N;
  constexpr int WM = BT / 2, WN = BT / WAVES_N;
  constexpr int FM = WM / MI, FN = WN / MI;
  constexpr int NE = MI * MI / 64, P = 64 / MI;
  constexpr int UNIT = FM * FN * NE * 64 * WAVES;   // floats per unit
  const int tile = blockIdx.x;
  int pm, pn;
  grouped_tile(tile, p.tiles_m, p.tiles_n, p.group_m, pm, pn);
  const float* base = p.ws + (size_t)tile * p.splits * UNIT;
  for (int q = threadIdx.x; q < UNIT / 4; q += 256) {
    const int lane = q % 64;
    const int g = (q / 64) % (NE / 4);
    const int blk = (q / 64 / (NE / 4)) % (FM * FN);
    const int wave = q / 64 / (NE / 4) / (FM * FN);
    const int i = blk / FN, j = blk % FN;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    f32x4_t sum = *reinterpret_cast<const f32x4_t*>(base + (size_t)q * 4);
    for (int sp = 1; sp < p.splits; ++sp) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(base + (size_t)sp * UNIT + (size_t)q * 4);
      sum[0] += v[0];
      sum[1] += v[1];
      sum[2] += v[2];
      sum[3] += v[3];
    }
    const int m = pm * BT + wm * WM + i * MI + lane % MI;
    const int n = pn * BT + wn * WN + j * MI + 4 * P * g + 4 * (lane / MI);
    if (m >= p.M) continue;
    const float sc = DT == kBf16 ? 1.0f : p.scale;
    const uint2 pk = pack_bf16x4(sum[0] * sc, sum[1] * sc, sum[2] * sc, sum[3] * sc);
    uint16_t* cp = p.C + (size_t)m * (size_t)p.N + n;
    if ((p.N & 3) == 0 && n + 3 < p.N) {
      *reinterpret_cast<uint2*>(cp) = pk;
    } else {
      const uint16_t e[4] = {(uint16_t)(pk.x & 0xFFFF), (uint16_t)(pk.x >> 16),
                             (uint16_t)(pk.y & 0xFFFF), (uint16_t)(pk.y >> 16)};
      for (int u = 0; u < 4; ++u)
        if (n + u < p.N) cp[u] = e[u];
    }
  }
}

template <int DT, int R, bool MASKED, bool SPLITK = false>
void launch_ring(const DenseArgs& a, int grid, hipStream_t stream) {
  constexpr Ring r = ring_of<DT>(R);
  hipLaunchKernelGGL((gemm_dense_kernel<DT, r.bkb, r.slots, r.waves_n, r.loaders, r.mi, r.bt,
                                        r.occ, r.swz, r.sched, SPLITK, MASKED>),
                     dim3(grid), dim3(128 * r.waves_n), 0, stream, a);
}

// Launch table: entry v launches ring v of the operand type, in its masked
// or unmasked instance.
template <int DT, bool MASKED, int... V>
void launch_variant_seq(int v, const DenseArgs& a, int grid, hipStream_t stream,
                        std::integer_sequence<int, V...>) {
  using Fn = void (*)(const DenseArgs&, int, hipStream_t);
  static constexpr Fn table[] = {&launch_ring<DT, V, MASKED>...};
  table[v](a, grid, stream);
}

template <int DT, bool MASKED>
void launch_variant(int v, const DenseArgs& a, int grid, hipStream_t stream) {
  constexpr int n = DT == kBf16 ? kNumBf16 : kNumFp8;
  launch_variant_seq<DT, MASKED>(v, a, grid, stream, std::make_integer_sequence<int, n>{});
}

template <int DT, int R>
void launch_reduce_ring(const DenseArgs& a, hipStream_t stream) {
  constexpr Ring r = ring_of<DT>(R);
  hipLaunchKernelGGL((gemm_dense_reduce<DT, r.waves_n, r.mi, r.bt>), dim3(a.num_tiles), dim3(256), 0,
                     stream, a);
}

}  // namespace

uint32_t dense_stage_kbytes() { return kRingsBf16[0].bkb; }
static_assert(kRingsBf16[0].bkb == kRingsFp8[0].bkb, "one default stage width");
int dense_num_variants(DenseType dt) { return dt == kBf16 ? kNumBf16 : kNumFp8; }
int dense_default_mi(DenseType dt) { return ring_at(dt, 0).mi; }
int dense_tile(DenseType dt, int variant) { return ring_at(dt, variant).bt; }
int dense_occupancy(DenseType dt, int variant) { return ring_at(dt, variant).occ; }
void dense_variant_desc(DenseType dt, int variant, int32_t* stage_kbytes, int32_t* slots,
                        int32_t* waves, int32_t* load_waves, int32_t* mfma_block,
                        int32_t* tile, int32_t* per_cu, int32_t* swizzle, int32_t* schedule) {
  const Ring r = ring_at(dt, variant);
  *stage_kbytes = r.bkb;
  *slots = r.slots;
  *waves = 2 * r.waves_n;
  *load_waves = r.loaders ? r.waves_n : 2 * r.waves_n;
  *mfma_block = r.mi;
  *tile = r.bt;
  *per_cu = r.occ;
  *swizzle = r.swz;
  *schedule = r.sched;
}
uint32_t dense_unit_ws_bytes(DenseType dt, int variant) {
  const int bt = dense_tile(dt, variant);
  return (uint32_t)(bt * bt * 4);
}
uint32_t dense_variant_stage_kbytes(DenseType dt, int variant) {
  return ring_at(dt, variant).bkb;
}

// Whether a launch needs the masked instance: a ragged M or N tile (rows
// past the operand, which only a bounds-checked per-lane offset turns into
// zeros), or a stage that can reach past K (a ragged last stage, or the
// zero stage that pads an odd stage count when a loop trip runs two
// stages).
bool dense_masked(DenseType dt, int variant, int64_t M, int64_t N, uint32_t kbytes) {
  const Ring r = ring_at(dt, variant);
  return M % r.bt != 0 || N % r.bt != 0 || kbytes % (2 * r.bkb) != 0;
}

hipError_t launch_dense_reduce(DenseType dt, const DenseArgs& a, int variant, hipStream_t stream) {
  // split-K runs on the small-tile configuration only
  if (variant != kDenseSmallTileVariant) return hipErrorInvalidValue;
  if (dt == kBf16) launch_reduce_ring<kBf16, kDenseSmallTileVariant>(a, stream);
  else launch_reduce_ring<kFp8, kDenseSmallTileVariant>(a, stream);
  return hipGetLastError();
}

hipError_t launch_dense(DenseType dt, const DenseArgs& a, int grid, int variant,
                        hipStream_t stream) {
  if (variant < 0 || variant >= dense_num_variants(dt)) return hipErrorInvalidValue;
  const bool masked = dense_masked(dt, variant, a.M, a.N, a.kbytes);
  if (a.splits > 1) {
    // split-K work units: a separate instance of the small-tile kernel
    // (the per-unit K range and the partial-sum store stay out of the
    // plain kernels' registers)
    if (variant != kDenseSmallTileVariant) return hipErrorInvalidValue;
    constexpr int V = kDenseSmallTileVariant;
    if (dt == kBf16) {
      if (masked) launch_ring<kBf16, V, true, true>(a, grid, stream);
      else launch_ring<kBf16, V, false, true>(a, grid, stream);
    } else {
      if (masked) launch_ring<kFp8, V, true, true>(a, grid, stream);
      else launch_ring<kFp8, V, false, true>(a, grid, stream);
    }
    return hipGetLastError();
  }
  if (dt == kBf16) {
    if (masked) launch_variant<kBf16, true>(variant, a, grid, stream);
    else launch_variant<kBf16, false>(variant, a, grid, stream);
  } else {
    if (masked) launch_variant<kFp8, true>(variant, a, grid, stream);
    else launch_variant<kFp8, false>(variant, a, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace tkg
