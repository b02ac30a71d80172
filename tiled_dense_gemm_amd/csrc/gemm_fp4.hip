// Block-scaled 4-bit tiled GEMM for gfx950 (MI355X).
//
// Format (page "ThunderKittens reaches 22.4 PFLOPS on NVIDIA Rubin": NVFP4,
// a block-scaled 4-bit float whose block-scaling factors travel with the
// values, "Feeding the faster tensor cores"): e2m1 values, one e4m3 scale
// per 16 consecutive K-elements of a row, one fp32 scale per tensor.
//
// gfx950's block-scaled MFMA takes power-of-two (E8M0) scales per 32
// elements, which cannot express an e4m3 scale per 16. Each e2m1 value
// times its e4m3 block scale has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in fp16: the kernel dequantizes in
// registers, right after the LDS read, and multiplies on the fp16 matrix
// cores with fp32 accumulation. The product is therefore exact up to fp32
// summation, at the 16-bit MFMA rate.
//
// Structure as in gemm_dense.hip (256x256 workgroup tile of 2x2 wave tiles
// of 32x32 accumulators, one wave per SIMD, or 2x4 with two per SIMD;
// persistent grouped grid with XCD remap; LDS ring fed by direct global->LDS
// loads), with a 4-deep ring:
// one stage holds 128 K-elements per row, i.e. 64 bytes of packed values
// (swizzled as in tkg_layout.hpp) and 8 bytes of block scales.
#include "tkg_device.hpp"
#include "tkg_finish.hpp"
#include "tkg_kernels.hpp"
#include "tkg_layout.hpp"

#include <type_traits>

namespace tkg {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int BM = kBM, BN = kBN;
constexpr int VB = 64;                    // value bytes per row per stage
constexpr int SB = 8;                     // scale bytes per row per stage
constexpr int STAGES = 4;
constexpr int TILE_V = BM * VB;           // 16 KiB
constexpr int TILE_S = BM * SB;           // 2 KiB
constexpr int OFF_BV = TILE_V;
constexpr int OFF_AS = 2 * TILE_V;
constexpr int OFF_BS = 2 * TILE_V + TILE_S;
constexpr int STAGE_BYTES = 2 * TILE_V + 2 * TILE_S;  // 36 KiB

static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS budget");

struct TileState {
  int m0, n0;
  __amdgpu_buffer_rsrc_t rav, rbv, ras, rbs;
};

__device__ __forceinline__ TileState tile_state(const Fp4Args& p, int t) {
  TileState s;
  if (t >= p.num_tiles) {
    s.m0 = s.n0 = 0;
    s.rav = make_rsrc(p.A, 0);
    s.rbv = make_rsrc(p.B, 0);
    s.ras = make_rsrc(p.As, 0);
    s.rbs = make_rsrc(p.Bs, 0);
    return s;
  }
  int pm, pn;
  grouped_tile(t, p.tiles_m, p.tiles_n, p.group_m, pm, pn);
  s.m0 = pm * BM;
  s.n0 = pn * BN;
  const uint32_t ra = (uint32_t)min(p.M - s.m0, BM);
  const uint32_t rb = (uint32_t)min(p.N - s.n0, BN);
  s.rav = make_rsrc(p.A + (size_t)s.m0 * p.vbytes, ra * p.vbytes);
  s.rbv = make_rsrc(p.B + (size_t)s.n0 * p.vbytes, rb * p.vbytes);
  s.ras = make_rsrc(p.As + (size_t)s.m0 * p.sbytes, ra * p.sbytes);
  s.rbs = make_rsrc(p.Bs + (size_t)s.n0 * p.sbytes, rb * p.sbytes);
  return s;
}

// Eight e2m1 values (one dword, element 2t in the low nibble of byte t)
// times a block scale -> eight exact fp16 values.
__device__ __forceinline__ f16x8_t dequant8(uint32_t packed, float scale,
                                            f16x2_t mant) {
  f16x2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, scale, 0);
  f16x2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, scale, 1);
  f16x2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, scale, 2);
  f16x2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, scale, 3);
  h0 = h0 * mant;
  h1 = h1 * mant;
  h2 = h2 * mant;
  h3 = h3 * mant;
  return f16x8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// Block scale (byte BYTE of `word`, OCP e4m3) -> the scale operand of the
// convert and the fp16 factor still to apply. The convert uses only the
// magnitude of its scale's power of two (measured on gfx950: mantissa and
// sign are ignored), so the scale is passed as decoded and the factor
// carries the sign and the mantissa: +-(1 + m/8) for m in 0..7, exact in
// fp16. Subnormal e4m3 scales decode to normal fp32 values, so they split
// the same way; a zero scale gives a zero power of two (fp16 underflow).
template <int BYTE>
__device__ __forceinline__ void split_scale(uint32_t word, float& s,
                                            f16x2_t& mant) {
  s = __builtin_amdgcn_cvt_f32_fp8((int)word, BYTE);
  const uint32_t u = __builtin_bit_cast(uint32_t, s);
  const _Float16 m =
      (_Float16)__builtin_bit_cast(float, (u & 0x807FFFFFu) | 0x3F800000u);
  mant = f16x2_t{m, m};
}

// VALU instructions placed after each MFMA (6 measured fastest among
// 3, 4, 6, 8 and 12 at 8192^3).
constexpr int kValuPerMfma = 6;

// Scheduling recipe for one k-step of NMMA MFMAs: the LDS reads (NREAD,
// three after each of the first MFMAs) and slab loads (NDMA, one after each
// MFMA) are front-loaded; the dequantization VALU work of the next k-step is
// spread over all MFMAs, so the matrix core is fed while the VALU converts.
template <int NMMA, int NREAD, int NDMA, int Q = 0>
__device__ __forceinline__ void interleave_fp4() {
  if constexpr (Q < NMMA) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    constexpr int r = NREAD - 3 * Q >= 3 ? 3 : (NREAD - 3 * Q > 0 ? NREAD - 3 * Q : 0);
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
    if constexpr (Q < NDMA) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);  // VALU
    interleave_fp4<NMMA, NREAD, NDMA, Q + 1>();
  }
}

template <int WAVES_N>
__global__ __launch_bounds__(128 * WAVES_N)
__attribute__((amdgpu_waves_per_eu(WAVES_N / 2, WAVES_N / 2)))
void gemm_fp4_kernel(Fp4Args p) {
  constexpr int WAVES = 2 * WAVES_N;
  constexpr int WM = BM / 2, WN = BN / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int VDMA = TILE_V / 1024 / WAVES;  // b128 loads per wave per operand
  constexpr int SDMA = TILE_S / 256 / WAVES;   // b32 loads per wave per operand
  constexpr int DMA_PER_STAGE = 2 * VDMA + 2 * SDMA;  // per lane
  static_assert(SDMA >= 1, "scale staging needs a load per wave");

  // the finish stages through the LDS the ring leaves free (tkg_finish.hpp)
  using FP = FinishPlan<32, FM, FN, (160 * 1024 - STAGES * STAGE_BYTES) / WAVES>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[STAGES * STAGE_BYTES + WAVES * FP::BYTES];
  TKG_LDS uint8_t* smem = (TKG_LDS uint8_t*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int G = gridDim.x;
  int t = xcd_virtual_id(blockIdx.x, G, p.xcd_remap);
  if (t >= p.num_tiles) return;

  // ---- staging offsets ---------------------------------------------------
  uint32_t voff[VDMA], vkb[VDMA];
#pragma unroll
  for (int i = 0; i < VDMA; ++i) {
    const uint32_t q = wave * VDMA + i;
    vkb[i] = dma_chunk(VB, q, lane) * 16u;
    voff[i] = dma_row(VB, q, lane) * p.vbytes + vkb[i];
  }
  // scales: one wave b32 load covers 32 rows x 8 bytes
  uint32_t soff[SDMA];
  const uint32_t skb = (lane & 1) * 4u;
#pragma unroll
  for (int i = 0; i < SDMA; ++i) {
    const uint32_t q = wave * SDMA + i;
    soff[i] = (q * 32u + (lane >> 1)) * p.sbytes + skb;
  }

  // ---- load cursor (tile lt, stage lkt) ------------------------------------
  TileState cur = tile_state(p, t);
  TileState lts = cur;
  int lt = t;
  uint32_t lkt = 0;
  struct StageLoad {
    __amdgpu_buffer_rsrc_t rav, rbv, ras, rbs;
    uint32_t k0, s0;
  };
  auto next_stage = [&]() {
    StageLoad s{lts.rav, lts.rbv, lts.ras, lts.rbs, lkt * VB, lkt * SB};
    if (++lkt == p.nk) {
      lkt = 0;
      lt += G;
      lts = tile_state(p, lt);
    }
    return s;
  };
  // Branch-free loads of one stage into buffer `buf`; past K reads zeros.
  auto issue = [&](const StageLoad& s, int buf) {
    TKG_LDS uint8_t* st = smem + buf * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < VDMA; ++i) {
      const uint32_t off = (s.k0 + vkb[i] < p.vbytes) ? voff[i] + s.k0 : kOobOffset;
      const uint32_t q = wave * VDMA + i;
      dma_b128(s.rav, st + q * 1024, off);
      dma_b128(s.rbv, st + OFF_BV + q * 1024, off);
    }
#pragma unroll
    for (int i = 0; i < SDMA; ++i) {
      const uint32_t off = (s.s0 + skb < p.sbytes) ? soff[i] + s.s0 : kOobOffset;
      const uint32_t q = wave * SDMA + i;
      dma_b32(s.ras, st + OFF_AS + q * 256, off);
      dma_b32(s.rbs, st + OFF_BS + q * 256, off);
    }
  };

  // ---- fragment reads ------------------------------------------------------
  // Lane l works on row l%32 of each 32-row fragment. Per stage it reads two
  // 16-byte chunks of packed values, chunk 2s + l/32 for s = 0, 1 (32
  // K-elements each, 4 MFMA k-steps of 8), and, once per stage, the row's 8
  // scale bytes (one 8-byte read: 32 consecutive rows fill the banks without
  // conflict). The same K order is used for A and B, so the MFMA's reduction
  // is over the same K-elements on both sides.
  const uint32_t frow = lane & 31;
  const uint32_t khalf = lane >> 5;
  uint32_t roff[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) roff[s] = swz_offset(VB, frow, 2 * s + khalf);
  const uint32_t av_base = wm * WM * VB, bv_base = OFF_BV + wn * WN * VB;
  const uint32_t as_base = OFF_AS + (wm * WM + frow) * SB;
  const uint32_t bs_base = OFF_BS + (wn * WN + frow) * SB;

  struct Raw {
    i32x4_t a[FM], b[FN];     // packed values of one chunk
    u32x2_t sa[FM], sb[FN];   // the row's 8 block scales of the stage
  };
  // chunk s of buffer `buf`; the scales are read with chunk 0 and carried
  auto read_raw = [&](int buf, int s, Raw& r, const Raw& prev) {
    const TKG_LDS uint8_t* st = smem + buf * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      r.a[i] = lds_read<i32x4_t>(st, av_base + i * 32 * VB + roff[s]);
      r.sa[i] = (s == 0) ? lds_read<u32x2_t>(st, as_base + i * 32 * SB) : prev.sa[i];
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      r.b[j] = lds_read<i32x4_t>(st, bv_base + j * 32 * VB + roff[s]);
      r.sb[j] = (s == 0) ? lds_read<u32x2_t>(st, bs_base + j * 32 * SB) : prev.sb[j];
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16_t{};

  // Dequantized fragments of one MFMA k-step (8 K-elements per lane). Two
  // sets alternate: while the MFMAs consume one, the VALU fills the other
  // with the next k-step, so conversion and matrix work overlap.
  struct Deq {
    f16x8_t a[FM], b[FN];
  };
  // k-step q (0..3) of chunk s: dword q of the chunk, whose block (16
  // elements) is 2*(2s + khalf) + q/2 of the stage, i.e. byte
  // 2*khalf + q/2 of scale word s.
  auto dequant = [&](const Raw& r, int s, auto qc, Deq& d) {
    constexpr int q = decltype(qc)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float sc; f16x2_t m;
      split_scale<q / 2>(r.sa[i][s] >> (16 * khalf), sc, m);
      d.a[i] = dequant8((uint32_t)r.a[i][q], sc, m);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      float sc; f16x2_t m;
      split_scale<q / 2>(r.sb[j][s] >> (16 * khalf), sc, m);
      d.b[j] = dequant8((uint32_t)r.b[j][q], sc, m);
    }
  };
  // Keeps the conversion of a k-step ahead of a block boundary: without it
  // the compiler sinks the VALU work past the loop's branch, where it can no
  // longer overlap the MFMAs.
  auto pin = [&](Deq& d) {
#pragma unroll
    for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(d.a[i]));
#pragma unroll
    for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(d.b[j]));
  };
  auto mma = [&](const Deq& d) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(d.b[j], d.a[i], acc[i][j], 0, 0, 0);
  };
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using Q3 = std::integral_constant<int, 3>;
  constexpr int NMMA = FM * FN;
  constexpr int NREAD0 = 2 * (FM + FN);   // chunk 0: values + scales
  constexpr int NREAD1 = FM + FN;         // chunk 1: values
  constexpr int NDMA = 2 * VDMA + 2 * SDMA;

  // ---- prologue ------------------------------------------------------------
#pragma unroll
  for (int b = 0; b < STAGES; ++b) issue(next_stage(), b);
  wait_vmcnt<(STAGES - 1) * DMA_PER_STAGE>();
  __syncthreads();

  Raw raw[2];
  Deq deq[2];
  read_raw(0, 0, raw[0], raw[0]);
  dequant(raw[0], 0, Q0{}, deq[0]);

  // Eight k-steps per stage (chunk s = u/4, k-step q = u%4). k-step u
  // multiplies deq[u&1] while deq[(u+1)&1] is filled with k-step u+1; the
  // last k-step converts chunk 0 of the next stage. Chunk 1 is read from LDS
  // at u = 0; at u = 4 (all waves have read the stage) the next stage must
  // have landed, the barrier frees this buffer for the cursor's next stage,
  // and chunk 0 of the next stage is read.
  int buf = 0;
  bool fresh_tile = false;  // finish stores are in flight
  for (;;) {
    for (uint32_t kt = 0; kt < p.nk; ++kt) {
      // the cursor moves here so that no branch splits the stage's k-steps
      const StageLoad nl = next_stage();
      read_raw(buf, 1, raw[1], raw[0]);
      dequant(raw[0], 0, Q1{}, deq[1]);
      mma(deq[0]);
      interleave_fp4<NMMA, NREAD1, 0>();
      __builtin_amdgcn_sched_barrier(0);
      dequant(raw[0], 0, Q2{}, deq[0]);
      mma(deq[1]);
      interleave_fp4<NMMA, 0, 0>();
      __builtin_amdgcn_sched_barrier(0);
      dequant(raw[0], 0, Q3{}, deq[1]);
      mma(deq[0]);
      interleave_fp4<NMMA, 0, 0>();
      __builtin_amdgcn_sched_barrier(0);
      dequant(raw[1], 1, Q0{}, deq[0]);
      mma(deq[1]);
      interleave_fp4<NMMA, 0, 0>();
      pin(deq[0]);
      __builtin_amdgcn_sched_barrier(0);

      if (fresh_tile) wait_vmcnt<0>();
      else wait_vmcnt<(STAGES - 2) * DMA_PER_STAGE>();
      fresh_tile = false;
      lds_barrier();
      issue(nl, buf);
      const int nbuf = (buf + 1 == STAGES) ? 0 : buf + 1;
      read_raw(nbuf, 0, raw[0], raw[0]);
      dequant(raw[1], 1, Q1{}, deq[1]);
      mma(deq[0]);
      interleave_fp4<NMMA, NREAD0, NDMA>();
      __builtin_amdgcn_sched_barrier(0);
      dequant(raw[1], 1, Q2{}, deq[0]);
      mma(deq[1]);
      interleave_fp4<NMMA, 0, 0>();
      __builtin_amdgcn_sched_barrier(0);
      dequant(raw[1], 1, Q3{}, deq[1]);
      mma(deq[0]);
      interleave_fp4<NMMA, 0, 0>();
      __builtin_amdgcn_sched_barrier(0);
      dequant(raw[0], 0, Q0{}, deq[0]);
      mma(deq[1]);
      interleave_fp4<NMMA, 0, 0>();
      pin(deq[0]);
      __builtin_amdgcn_sched_barrier(0);
      buf = nbuf;
    }

    // ---- finish (as in gemm_dense.hip) -----------------------------------
    if constexpr (FP::USE) {
      finish_staged<32, FM, FN, FP::RJ, true>(
          acc, p.scale, smem + STAGES * STAGE_BYTES + wave * FP::BYTES, p.C, p.M, p.N,
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
          const uint2 pk = pack_bf16x4(acc[i][j][4 * g + 0] * p.scale,
                                       acc[i][j][4 * g + 1] * p.scale,
                                       acc[i][j][4 * g + 2] * p.scale,
                                       acc[i][j][4 * g + 3] * p.scale);
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
  // The load cursor ran ahead into empty resources; let those LDS writes
  // land before the workgroup's LDS is released.
  wait_vmcnt<0>();
}

}  // namespace

uint32_t fp4_stage_vbytes() { return VB; }

int fp4_num_variants() { return 2; }

// variant 0: 4 waves (one per SIMD, 128x128 wave tiles: each fragment is
// dequantized by fewer waves); 1: 8 waves (two per SIMD, 128x64)
hipError_t launch_fp4(const Fp4Args& a, int grid, int variant,
                      hipStream_t stream) {
  if (variant == 1)
    hipLaunchKernelGGL(gemm_fp4_kernel<4>, dim3(grid), dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL(gemm_fp4_kernel<2>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tkg
