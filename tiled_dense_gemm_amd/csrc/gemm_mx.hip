// MX block-scaled tiled GEMM for gfx950 (MI355X): MXFP4 and MXFP8.
//
// The pages' block-scaled low-precision path (page "ThunderKittens reaches
// 22.4 PFLOPS on NVIDIA Rubin", "Feeding the faster tensor cores": scale
// factors travel with the 4-bit values) in the form CDNA4's matrix cores
// execute natively: v_mfma_scale_f32_32x32x64_f8f6f4 multiplies e2m1 (fp4)
// or e4m3 (fp8) elements and applies one E8M0 scale (2^(e-127)) per 32
// K-elements of each row and column inside the instruction (OCP Microscaling
// formats). The product runs at the fp4 / fp8 MFMA rate with no conversion
// work; C = scale * A * B with fp32 accumulation, bf16 output.
//
// Structure as the dense kernels (gemm_dense.hip): 256x256 workgroup tile of
// 2x4 waves with 128x64 wave tiles (two waves per SIMD, 4x2 accumulators of
// 32x32) when the scales are staged wide, else 2x2 waves with 128x128 wave
// tiles (one wave per SIMD, 4x4 accumulators in AGPRs); a 4-slot LDS ring
// of operand slabs fed straight from global memory, k-steps emitted in
// program order with the loads and reads placed after the MFMAs,
// persistent grouped grid with XCD remap. Next to
// each value slab (256 rows x 128 bytes) the ring holds its scale slab (256
// rows x the stage's scale bytes).
//
// Lane data of one 32x32x64 MFMA (measured on MI355X): lane l supplies row
// (or column) l % 32. For fp4 its 32 elements are K-elements 32*(l/32) ..
// +31 of the k-step (16 bytes, two per byte, low nibble first), and its
// scale is the one of that 32-element block. For fp8 its 32 bytes are
// K-elements 16*(l/32) .. +15 and 32 + 16*(l/32) .. +15, and its scale is
// the one of block (l/32) of the k-step, which the two lane halves share.
#include "tkg_device.hpp"
#include "tkg_finish.hpp"
#include "tkg_kernels.hpp"
#include "tkg_layout.hpp"

#include <type_traits>

namespace tkg {
namespace {

constexpr int BM = kBM, BN = kBN;
constexpr int BKB = 128;                  // value bytes per row per stage
constexpr int SLOTS = 4;
constexpr int SLAB = BM * BKB;            // 32 KiB
constexpr int WM = BM / 2;               // wave tile rows (2 x WAVES_N waves)
// The wide-scale kernel runs 4 waves per workgroup row (8 waves, 128 x 64
// wave tiles, two per SIMD; against 2, i.e. 4 waves of 128 x 128 at one per
// SIMD, at 8192^3, same process, bit-identical: MXFP4 4364 against 4029
// TFLOP/s, MXFP8 2622 against 2564), of which only the first wave row (one
// wave per SIMD) issues the global->LDS loads, as in the dense kernels
// (against all waves loading: MXFP4 4415 against 4319 TFLOP/s, MXFP8 2665
// against 2630). The other kernels run 2 waves per row, all loading.
constexpr int kWideWavesN = 4;

template <int FMT, int WAVES>
struct Mx {
  static constexpr bool FP4 = FMT == kMxfp4;
  static constexpr int SB = FP4 ? 8 : 4;          // 32-element blocks per row per stage
  static constexpr int KSTEPS = FP4 ? 4 : 2;      // 64-element k-steps per stage
  static constexpr int PARTS = FP4 ? 1 : 2;       // 16-byte reads per lane per fragment
  static constexpr int SSLAB = BM * SB;           // scale bytes per slab
  static constexpr int SDMA = SSLAB / 256 / WAVES;  // 4-byte scale loads per wave per slab
  static constexpr int ROWS_PER_SDMA = 256 / SB;  // rows one scale load covers
  static constexpr int CB = FP4 ? 4 : 0;          // MFMA operand format: 4 = fp4, 0 = fp8
  static_assert(SDMA >= 1 || WAVES != 4, "scale slab needs a load per wave");
};

struct TileState {
  int m0, n0;
  __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
};

__device__ __forceinline__ TileState tile_state(const MxArgs& p, int t) {
  TileState s;
  if (t >= p.num_tiles) {  // past the last tile: empty resources read zeros
    s.m0 = s.n0 = 0;
    s.ra = make_rsrc(p.A, 0);
    s.rb = make_rsrc(p.B, 0);
    s.rsa = make_rsrc(p.As, 0);
    s.rsb = make_rsrc(p.Bs, 0);
    return s;
  }
  int pm, pn;
  order_tile(t, gridDim.x, p.xcd_remap, p.tiles_m, p.tiles_n, p.group_m, pm, pn);
  s.m0 = pm * BM;
  s.n0 = pn * BN;
  const uint32_t rows_a = (uint32_t)min(p.M - s.m0, BM);
  const uint32_t rows_b = (uint32_t)min(p.N - s.n0, BN);
  s.ra = make_rsrc(p.A + (size_t)s.m0 * p.vbytes, rows_a * p.vbytes);
  s.rb = make_rsrc(p.B + (size_t)s.n0 * p.vbytes, rows_b * p.vbytes);
  s.rsa = make_rsrc(p.As + (size_t)s.m0 * p.sbytes, rows_a * p.sbytes);
  s.rsb = make_rsrc(p.Bs + (size_t)s.n0 * p.sbytes, rows_b * p.sbytes);
  return s;
}

// One scaled MFMA: D += (Bfrag, B scale) x (Afrag, A scale); OPSEL picks the
// byte of each scale word that holds this k-step's E8M0 scale.
template <int CB, int OPSEL>
__device__ __forceinline__ f32x16_t mfma_mx(i32x8_t b, int sb, i32x8_t a, int sa,
                                            f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, CB, CB, OPSEL, sb,
                                                         OPSEL, sa);
}

// Scale staging. Narrow (WIDE = false): every slab load also fetches the
// stage's SB scale bytes of its 256 rows, 4 bytes per lane. Each lane then
// touches its own cache line, so these loads cost as many cache lookups as
// the value loads. Wide (K a multiple of 512, so rows of scales are a whole
// number of 16-byte pieces): one 16-byte load per row covers U = 16 / SB
// stages (a superstage); superstages alternate between two LDS slots of
// 256 rows x 16 bytes per operand, and a stage's scale word sits at byte
// SB * (stage mod U) of its row.
// EARLY: the A fragments are double-buffered like the B fragments and every
// fragment read of the next k-step goes out over the current k-step's first
// MFMAs, in the order the next k-step first uses them (the early-reads
// schedule of gemm_dense.hip); otherwise each A fragment is re-read right
// after its last MFMA of the k-step.
template <int FMT, bool KTAIL, bool WIDE, int WAVES_N, bool EARLY>
__global__ __launch_bounds__(128 * WAVES_N)
__attribute__((amdgpu_waves_per_eu(WAVES_N / 2, WAVES_N / 2)))
void gemm_mx_kernel(MxArgs p) {
  constexpr int WAVES = 2 * WAVES_N;
  constexpr int WN = BN / WAVES_N;                // wave tile columns
  constexpr int FM = WM / 32, FN = WN / 32;       // 32x32 accumulators
  constexpr bool LOADERS = WAVES == 8;
  constexpr int LOAD_WAVES = LOADERS ? 4 : WAVES;   // waves that issue loads
  constexpr int DMA = SLAB / 1024 / LOAD_WAVES;   // value loads per loading wave per slab
  static_assert(WIDE || WAVES == 4, "eight waves stage their scales wide");
  using S = Mx<FMT, LOAD_WAVES>;
  constexpr int KSTEPS = S::KSTEPS, PARTS = S::PARTS, SB = S::SB;
  constexpr int SSLAB = S::SSLAB, SDMA = S::SDMA;
  static_assert(!(WIDE && KTAIL), "wide scale staging needs whole stages");
  static_assert(SLOTS == 4, "the stage-end wait drains every load, superstages included");
  constexpr uint32_t U = 16 / SB;                 // stages per superstage
  constexpr uint32_t WSLOT = 2 * BM * 16;         // one superstage, A then B
  constexpr int SCALE_LDS = WIDE ? 2 * WSLOT : SLOTS * SSLAB;
  // the finish stages through the LDS the ring leaves free (tkg_finish.hpp)
  using FP = FinishPlan<32, FM, FN, (160 * 1024 - SLOTS * SLAB - SCALE_LDS) / WAVES>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[SLOTS * SLAB + SCALE_LDS + WAVES * FP::BYTES];
  TKG_LDS uint8_t* smem = (TKG_LDS uint8_t*)smem_raw;
  TKG_LDS uint8_t* ssm = smem + SLOTS * SLAB;   // scale slabs

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lw = LOADERS ? wn : wave;             // index among the loading waves
  const bool loader = !LOADERS || wm == 0;
  const int G = gridDim.x;
  int t = xcd_virtual_id(blockIdx.x, G, p.xcd_remap);
  if (t >= p.num_tiles) return;
  const uint32_t nk = (p.vbytes + BKB - 1) / BKB;

  // ---- staging offsets -----------------------------------------------------
  // values: load q = wave*DMA + i of a slab fills rows dma_row(q); without a
  // K tail its offset is a scalar part plus one of two per-lane values
  constexpr int NOFF = KTAIL ? DMA : 2;
  uint32_t dma_off[NOFF], dma_kb[KTAIL ? DMA : 1];
  if constexpr (KTAIL) {
#pragma unroll
    for (int i = 0; i < DMA; ++i) {
      const uint32_t q = lw * DMA + i;
      dma_kb[i] = dma_chunk(BKB, q, lane) * 16u;
      dma_off[i] = dma_row(BKB, q, lane) * p.vbytes + dma_kb[i];
    }
  } else {
    dma_kb[0] = 0;
#pragma unroll
    for (int par = 0; par < 2; ++par) dma_off[par] = dma_lane_offset(BKB, par, lane, p.vbytes);
  }
  const uint32_t rows_step = dma_rows_per_instr(BKB) * p.vbytes;
  // scales: load i of this wave covers rows (wave*SDMA + i) * ROWS_PER_SDMA
  // onward, lane l row l / (SB/4), bytes 4 * (l % (SB/4)) of the stage
  constexpr uint32_t LPR = SB / 4;   // lanes per row
  const uint32_t s_row = lane / LPR, s_part = (lane % LPR) * 4u;
  const uint32_t s_lane_off = s_row * p.sbytes + s_part;
  const uint32_t s_rows_step = S::ROWS_PER_SDMA * p.sbytes;
  // wide: with 4 waves, wave w fetches rows 64w .. 64w+63 of both
  // operands; with 8, rows 64 (w % 4) .. +63 of A (w < 4) or B; lane l
  // the row's 16 bytes from the superstage's first scale byte
  const uint32_t w_lane_off = lane * p.sbytes;

  // ---- fragment reads --------------------------------------------------------
  // lane l reads row l % 32 of a fragment; k-step s, part q at chunk
  // fp4: 2s + l/32; fp8: 4s + 2q + l/32 (see the header)
  const uint32_t frow = lane & 31;
  const uint32_t khalf = lane >> 5;
  uint32_t roff[KSTEPS][PARTS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
    for (int q = 0; q < PARTS; ++q)
      roff[s][q] = swz_offset(BKB, frow, S::FP4 ? 2 * s + khalf : 4 * s + 2 * q + khalf);
  const uint32_t a_base = wm * WM * BKB, b_base = wn * WN * BKB;
  // scale word of fragment i: narrow at slot * SSLAB + as_base + i * SFRAG,
  // wide at (superstage slot, stage) + as_base + i * SFRAG
  constexpr uint32_t SROW = WIDE ? 16 : SB;   // LDS bytes per row of scales
  constexpr uint32_t SFRAG = 32 * SROW;
  const uint32_t as_base = (wm * WM + frow) * SROW;
  const uint32_t bs_base = (WIDE ? BM * 16 : 0) + (wn * WN + frow) * SROW;

  // ---- load cursor: slab (tile lt, stage lkt, operand lop) -------------------
  TileState cur = tile_state(p, t);
  TileState lts = cur;
  int lt = t;
  uint32_t lkt = 0, lop = 0, lslot = 0;
  auto advance_load = [&]() {
    lslot = (lslot + 1 == SLOTS) ? 0 : lslot + 1;
    if (lop == 0) {
      lop = 1;
    } else {
      lop = 0;
      if (++lkt == nk) {
        lkt = 0;
        lt += G;
        lts = tile_state(p, lt);
      }
    }
  };
  struct SlabLoad {
    __amdgpu_buffer_rsrc_t r, rs;
    uint32_t slot, k0, s0;
  };
  auto next_slab = [&]() {
    SlabLoad s;
    s.r = lop ? lts.rb : lts.ra;
    s.rs = lop ? lts.rsb : lts.rsa;
    s.slot = lslot;
    s.k0 = lkt * BKB;
    s.s0 = lkt * SB;
    advance_load();
    return s;
  };
  // load i of a slab: i < DMA values, then (narrow) SDMA scale loads
  constexpr int NLOAD = DMA + (WIDE ? 0 : SDMA);
  auto issue_one = [&](const SlabLoad& s, int i) {
    if (i < DMA) {
      TKG_LDS uint8_t* dst = smem + s.slot * SLAB + (lw * DMA + i) * 1024;
      const uint32_t q = lw * DMA + i;
      if constexpr (KTAIL) {
        const uint32_t off = (s.k0 + dma_kb[i] < p.vbytes) ? dma_off[i] + s.k0 : kOobOffset;
        dma_b128(s.r, dst, off);
      } else {
        dma_b128_soff(s.r, dst, dma_off[q & 1], s.k0 + q * rows_step);
      }
    } else {
      const int j = i - DMA;
      TKG_LDS uint8_t* dst = ssm + s.slot * SSLAB + (lw * SDMA + j) * 256;
      const uint32_t base = (uint32_t)(lw * SDMA + j) * s_rows_step + s.s0;
      if constexpr (KTAIL) {
        const uint32_t off = (s.s0 + s_part < p.sbytes) ? s_lane_off + base : kOobOffset;
        dma_b32(s.rs, dst, off);
      } else {
        dma_b32_soff(s.rs, dst, s_lane_off, base);
      }
    }
  };
  auto issue = [&](const SlabLoad& s) {
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) issue_one(s, i);
  };
  // wide: the superstage of tile ts that starts at `stage`, into `slot`
  auto load_superstage = [&](const TileState& ts, uint32_t stage, uint32_t slot) {
    if constexpr (LOAD_WAVES == 4) {
      TKG_LDS uint8_t* dst = ssm + slot * WSLOT + lw * 1024;
      const uint32_t soff = (uint32_t)lw * 64u * p.sbytes + stage * SB;
      dma_b128_soff(ts.rsa, dst, w_lane_off, soff);
      dma_b128_soff(ts.rsb, dst + BM * 16, w_lane_off, soff);
    } else {
      const int w4 = wave % 4;
      TKG_LDS uint8_t* dst = ssm + slot * WSLOT + (wave / 4) * (BM * 16) + w4 * 1024;
      const uint32_t soff = (uint32_t)w4 * 64u * p.sbytes + stage * SB;
      dma_b128_soff(wave < 4 ? ts.rsa : ts.rsb, dst, w_lane_off, soff);
    }
  };

  // The rest in two copies: waves that issue loads and (with LOADERS) waves
  // that only compute. Both run the same barriers.
  auto main_loop = [&](auto loader_tag) {
  constexpr bool IS_LOADER = decltype(loader_tag)::value;
  // ---- registers ---------------------------------------------------------------
  // A fragments single-buffered (re-read after their last MFMA) unless
  // EARLY, B double; scale words of the stage per fragment, read during the
  // previous stage's last k-step and shifted so that this lane's block sits
  // in bytes 0 and 2
  i32x8_t fa[EARLY ? 2 : 1][FM], fb[2][FN];
  using SW = typename std::conditional<S::FP4, u32x2_t, uint32_t>::type;
  SW sa[FM], sbs[FN];
  auto read_frag = [&](int slot, uint32_t row0, int s, i32x8_t& v) {
    const TKG_LDS uint8_t* base = smem + slot * SLAB;
    const i32x4_t lo = lds_read<i32x4_t>(base, row0 + roff[s][0]);
    if constexpr (PARTS == 2) {
      const i32x4_t hi = lds_read<i32x4_t>(base, row0 + roff[s][PARTS - 1]);
      v = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      v = i32x8_t{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
    }
  };
  // The raw scale bytes a lane reads: narrow, the stage's word(s); wide,
  // the row's whole 16-byte superstage (reading 32 rows of 16 bytes whole
  // is conflict-free on the LDS, reading one word of each is not), from
  // which pick() takes the stage's. lane_block() then moves this lane's
  // block into place, after the k-step's MFMAs, so that the wait for the
  // read falls there.
  using RW = typename std::conditional<WIDE, i32x4_t, SW>::type;
  auto read_scale = [&](uint32_t off, RW& w) { w = lds_read<RW>(ssm, off); };
  auto pick = [&](const RW& r, uint32_t j) -> SW {
    if constexpr (!WIDE) {
      (void)j;
      return r;
    } else if constexpr (S::FP4) {
      return j ? u32x2_t{(uint32_t)r[2], (uint32_t)r[3]} : u32x2_t{(uint32_t)r[0], (uint32_t)r[1]};
    } else {
      return (uint32_t)(j == 0 ? r[0] : j == 1 ? r[1] : j == 2 ? r[2] : r[3]);
    }
  };
  // where the scale bytes of the stage after global stage g (this
  // workgroup's running stage count) are read, given the slot of its
  // values; wide, the stage inside the superstage is (g + 1) mod U
  auto scale_base = [&](uint32_t g, int vslot) -> uint32_t {
    if constexpr (WIDE) return (((g + 1) / U) & 1u) * WSLOT;
    else return (uint32_t)vslot * SSLAB;
  };
  auto lane_block = [&](const SW& w) -> SW {
    if constexpr (S::FP4) return u32x2_t{w[0] >> (8 * khalf), w[1] >> (8 * khalf)};
    else return w >> (8 * khalf);
  };
  // the word and byte (OPSEL) of k-step s
  auto sword = [&](const SW& w, int s) -> int {
    if constexpr (S::FP4) return (int)w[s / 2];
    else return (int)w;
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16_t{};

  // ---- prologue --------------------------------------------------------------
  if constexpr (WIDE && IS_LOADER) load_superstage(cur, 0, 0);
#pragma unroll
  for (int b = 0; b < SLOTS; ++b) {
    const SlabLoad l = next_slab();
    if constexpr (IS_LOADER) issue(l);
  }
  wait_vmcnt<(SLOTS - 2) * NLOAD>();   // slabs 0 and 1 (stage 0) have landed
  __syncthreads();
  int aslot = 0, bslot = 1;
  {
    const uint32_t sa0 = WIDE ? 0u : (uint32_t)aslot * SSLAB;
    const uint32_t sb0 = WIDE ? 0u : (uint32_t)bslot * SSLAB;
    RW ra[FM], rb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      read_frag(aslot, a_base + i * 32 * BKB, 0, fa[0][i]);
      read_scale(sa0 + as_base + i * SFRAG, ra[i]);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      read_frag(bslot, b_base + j * 32 * BKB, 0, fb[0][j]);
      read_scale(sb0 + bs_base + j * SFRAG, rb[j]);
    }
    if constexpr (WIDE) {
      // whole rows, as at the stage boundary (a single-word read conflicts)
#pragma unroll
      for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(ra[i]));
#pragma unroll
      for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(rb[j]));
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) sa[i] = lane_block(pick(ra[i], 0));
#pragma unroll
    for (int j = 0; j < FN; ++j) sbs[j] = lane_block(pick(rb[j], 0));
  }

  // One k-step in program order (see gemm_dense.hip): after MFMA (i, j) the
  // instructions of its slot. The next k-step's fragments come from slots
  // (na, nb) at k-step ns; at a stage boundary the next stage's scale words
  // are read after the k-step's last MFMA that uses the current ones.
  bool fresh_tile = false;
  uint32_t g = 0;   // stages this workgroup has computed (all tiles)
  constexpr int NDMA = 2 * NLOAD;
  RW sa_n[FM], sb_n[FN];
  auto kstep_body = [&](int c, int s, auto sc, int ns, int na, int nb, bool boundary,
                        const SlabLoad* l0, const SlabLoad* l1) {
    const uint32_t nsa = boundary ? scale_base(g, na) : 0u;
    const uint32_t nsb = boundary ? scale_base(g, nb) : 0u;
    constexpr int SC = decltype(sc)::value;   // k-step index inside the stage
    constexpr int OPSEL = S::FP4 ? 2 * (SC % 2) : 2 * SC;
    i32x8_t (&a)[FM] = fa[EARLY ? c : 0];
    i32x8_t (&an)[FM] = fa[EARLY ? c ^ 1 : 0];
    constexpr int NREAD = FM + FN, NMMA = FM * FN;
    constexpr int RSTRIDE = NMMA >= 2 * NREAD ? NMMA / (2 * NREAD) : 1;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        acc[i][j] = mfma_mx<S::CB, OPSEL>(fb[c][j], sword(sbs[j], SC), a[i],
                                         sword(sa[i], SC), acc[i][j]);
        const int q = i * FN + j;
        if constexpr (EARLY) {
          // read r (b0, a0, b1 .. b[FN-1], a1 .. a[FM-1]) after slot r * RSTRIDE
          if (q % RSTRIDE == 0 && q / RSTRIDE < NREAD) {
            const int r = q / RSTRIDE;
            if (r == 0) read_frag(nb, b_base, ns, fb[c ^ 1][0]);
            else if (r == 1) read_frag(na, a_base, ns, an[0]);
            else if (r <= FN) read_frag(nb, b_base + (r - 1) * 32 * BKB, ns, fb[c ^ 1][r - 1]);
            else read_frag(na, a_base + (r - FN) * 32 * BKB, ns, an[r - FN]);
          }
        } else {
          if (q < FN) read_frag(nb, b_base + q * 32 * BKB, ns, fb[c ^ 1][q]);
          if (j == FN - 1) read_frag(na, a_base + i * 32 * BKB, ns, an[i]);
        }
        if (boundary) {
          if (q < FM) read_scale(nsa + as_base + q * SFRAG, sa_n[q]);
          else if (q < FM + FN) read_scale(nsb + bs_base + (q - FM) * SFRAG, sb_n[q - FM]);
          if constexpr (IS_LOADER) {
#pragma unroll
            for (int d = q * NDMA / (FM * FN); d < (q + 1) * NDMA / (FM * FN); ++d) {
              if (d < NLOAD) issue_one(*l0, d);
              else issue_one(*l1, d - NLOAD);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    (void)s;
  };
  auto kstep = [&](int c, auto sc, const SlabLoad& l0, const SlabLoad& l1) {
    constexpr int SC = decltype(sc)::value;
    if constexpr (SC != KSTEPS - 1) {
      kstep_body(c, SC, sc, SC + 1, aslot, bslot, false, nullptr, nullptr);
    } else {
      if (fresh_tile) wait_vmcnt<0>();
      else wait_vmcnt<(SLOTS - 4) * NLOAD>();
      fresh_tile = false;
      lds_barrier();
      const int na = (aslot + 2) % SLOTS, nb = (bslot + 2) % SLOTS;
      kstep_body(c, SC, sc, 0, na, nb, true, &l0, &l1);
      const uint32_t jn = (g + 1) % U;
      if constexpr (WIDE) {
        // whole rows were read: keep the compiler from narrowing each read
        // to the one word pick() takes (that single-word form conflicts)
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(sa_n[i]));
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(sb_n[j]));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) sa[i] = lane_block(pick(sa_n[i], jn));
#pragma unroll
      for (int j = 0; j < FN; ++j) sbs[j] = lane_block(pick(sb_n[j], jn));
      aslot = na;
      bslot = nb;
    }
  };

  for (;;) {
    for (uint32_t kt = 0; kt < nk; ++kt) {
      // the cursor moves (and may branch to a new tile) at the top of the
      // stage, so that no MFMA of the stage is moved past that branch and
      // behind the stage-end wait
      const SlabLoad l0 = next_slab();
      const SlabLoad l1 = next_slab();
      if constexpr (WIDE && IS_LOADER) {
        // the next stage opens a superstage: fetch it now, into the slot no
        // wave reads any more (the other one holds this stage's scales)
        if ((g + 1) % U == 0) {
          const uint32_t slot = ((g + 1) / U) & 1u;
          if (kt + 1 < nk) load_superstage(cur, kt + 1, slot);
          else if (t + G < p.num_tiles) load_superstage(tile_state(p, t + G), 0, slot);
        }
      }
      kstep(0, std::integral_constant<int, 0>{}, l0, l1);
      kstep(1, std::integral_constant<int, 1>{}, l0, l1);
      if constexpr (KSTEPS == 4) {
        kstep(0, std::integral_constant<int, 2>{}, l0, l1);
        kstep(1, std::integral_constant<int, 3>{}, l0, l1);
      }
      ++g;
    }

    // ---- finish (as in gemm_dense.hip, 32x32 blocks) ---------------------------
    if constexpr (FP::USE) {
      finish_staged<32, FM, FN, FP::RJ, true>(
          acc, p.scale, smem + SLOTS * SLAB + SCALE_LDS + wave * FP::BYTES, p.C, p.M, p.N,
          cur.m0 + wm * WM, cur.n0 + wn * WN, (uint32_t)lane);
    } else {
    const bool vec_ok = (p.N & 3) == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = cur.m0 + wm * WM + i * 32 + (int)frow;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = cur.n0 + wn * WN + j * 32 + 8 * g + 4 * (int)khalf;
          const uint2 pk = pack_bf16x4(acc[i][j][4 * g + 0] * p.scale, acc[i][j][4 * g + 1] * p.scale,
                                       acc[i][j][4 * g + 2] * p.scale, acc[i][j][4 * g + 3] * p.scale);
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
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    }
    fresh_tile = true;

    t += G;
    if (t >= p.num_tiles) break;
    cur = tile_state(p, t);
  }
  };
  if (loader)
    main_loop(std::true_type{});
  else
    main_loop(std::false_type{});
  // the load cursor ran ahead into empty resources; let those LDS writes land
  wait_vmcnt<0>();
}

template <int FMT, bool EARLY>
void launch_fmt(const MxArgs& a, int grid, hipStream_t stream) {
  // A ragged last stage, or a ragged M or N tile (rows past the operand,
  // which the scalar part of an unmasked load's offset would reach outside
  // the bounds check), runs the masked instance. Scale rows that are whole
  // 16-byte pieces (K % 512 == 0) are staged wide.
  constexpr int WW = kWideWavesN;
  if (mx_masked((MxType)FMT, a.M, a.N, a.vbytes, a.sbytes))
    hipLaunchKernelGGL((gemm_mx_kernel<FMT, true, false, 2, EARLY>), dim3(grid), dim3(256), 0,
                       stream, a);
  else if (a.sbytes % 16 == 0)
    hipLaunchKernelGGL((gemm_mx_kernel<FMT, false, true, WW, EARLY>), dim3(grid), dim3(128 * WW),
                       0, stream, a);
  else
    hipLaunchKernelGGL((gemm_mx_kernel<FMT, false, false, 2, EARLY>), dim3(grid), dim3(256), 0,
                       stream, a);
}

}  // namespace

bool mx_masked(MxType fmt, int64_t M, int64_t N, uint32_t vbytes, uint32_t sbytes) {
  (void)fmt;
  (void)sbytes;
  return vbytes % BKB != 0 || M % BM != 0 || N % BN != 0;
}

int mx_num_variants() { return 2; }

hipError_t launch_mx(MxType fmt, const MxArgs& a, int grid, int variant, hipStream_t stream) {
  const bool early = variant == 1;
  if (fmt == kMxfp4) {
    if (early) launch_fmt<kMxfp4, true>(a, grid, stream);
    else launch_fmt<kMxfp4, false>(a, grid, stream);
  } else {
    if (early) launch_fmt<kMxfp8, true>(a, grid, stream);
    else launch_fmt<kMxfp8, false>(a, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace tkg
