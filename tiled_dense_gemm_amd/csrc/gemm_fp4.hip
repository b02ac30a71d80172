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
  order_tile(t, gridDim.x, p.xcd_remap, p.tiles_m, p.tiles_n, p.group_m, pm, pn);
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

// Dequantization in fp16, exactly: every OCP e4m3 value (subnormals and
// 448 included) is an fp16 value, every e2m1 value is, and their product has
// at most 6 significant bits and a magnitude in [2^-10, 2688] when nonzero
// (0.5 x 2^-9 up to 6 x 448), inside fp16's normal range. So a value pair
// is converted with unit scale and multiplied by its block scale in fp16
// with no rounding; the two block scales a lane needs per 16-byte chunk
// come from one fp8 -> fp16 convert of their two bytes.

// Compile-time loop: f(integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
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
  constexpr int NMMA = FM * FN;
  constexpr int NF = FM + FN;               // fragments converted per k-step
  constexpr int NDMA = 2 * VDMA + 2 * SDMA;
  static_assert(NDMA <= NMMA && NF <= NMMA, "one load and two reads per MFMA at most");
  // LDS reads of one fragment: its 16 bytes of packed values of chunk s,
  // and (with chunk 0) the row's 8 scale bytes of the stage
  auto read_val = [&](int b, int s, int f, Raw& r) {
    const TKG_LDS uint8_t* st = smem + b * STAGE_BYTES;
    if (f < FM) r.a[f] = lds_read<i32x4_t>(st, av_base + f * 32 * VB + roff[s]);
    else r.b[f - FM] = lds_read<i32x4_t>(st, bv_base + (f - FM) * 32 * VB + roff[s]);
  };
  auto read_scale = [&](int b, int f, Raw& r) {
    const TKG_LDS uint8_t* st = smem + b * STAGE_BYTES;
    if (f < FM) r.sa[f] = lds_read<u32x2_t>(st, as_base + f * 32 * SB);
    else r.sb[f - FM] = lds_read<u32x2_t>(st, bs_base + (f - FM) * 32 * SB);
  };
  auto issue_one = [&](const StageLoad& s, int buf_, int d) {
    TKG_LDS uint8_t* st = smem + buf_ * STAGE_BYTES;
    if (d < 2 * VDMA) {
      const int i = d / 2;
      const uint32_t off = (s.k0 + vkb[i] < p.vbytes) ? voff[i] + s.k0 : kOobOffset;
      const uint32_t q = wave * VDMA + i;
      if (d % 2 == 0) dma_b128(s.rav, st + q * 1024, off);
      else dma_b128(s.rbv, st + OFF_BV + q * 1024, off);
    } else {
      const int i = (d - 2 * VDMA) / 2;
      const uint32_t off = (s.s0 + skb < p.sbytes) ? soff[i] + s.s0 : kOobOffset;
      const uint32_t q = wave * SDMA + i;
      if (d % 2 == 0) dma_b32(s.ras, st + OFF_AS + q * 256, off);
      else dma_b32(s.rbs, st + OFF_BS + q * 256, off);
    }
  };
  // Half h of fragment f's conversion for k-step q of chunk s (f < FM: A
  // fragment f, else B fragment f - FM): half 0 converts values 0-3, half 1
  // values 4-7. Dword q of the chunk lies in block 2 (2s + khalf) + q/2 of
  // the stage, i.e. byte 2 khalf + q/2 of scale word s: at q = 0 (the
  // chunk's first k-step) both of the chunk's block scales go to fp16 into
  // bscale[f], whose half q/2 later k-steps of the chunk use.
  f16x2_t bscale[NF];
  auto conv_half = [&](const Raw& r, int s, auto qc, auto fc, auto hc, Deq& d) {
    constexpr int q = decltype(qc)::value, f = decltype(fc)::value, h = decltype(hc)::value;
    constexpr bool IS_A = f < FM;
    constexpr int fi = IS_A ? f : f - FM;
    const i32x4_t& rv = [&]() -> const i32x4_t& {
      if constexpr (IS_A) return r.a[fi];
      else return r.b[fi];
    }();
    const u32x2_t& rs = [&]() -> const u32x2_t& {
      if constexpr (IS_A) return r.sa[fi];
      else return r.sb[fi];
    }();
    f16x8_t& v = [&]() -> f16x8_t& {
      if constexpr (IS_A) return d.a[fi];
      else return d.b[fi];
    }();
    const uint32_t packed = (uint32_t)rv[q];
    if constexpr (q == 0 && h == 0)
      bscale[f] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(rs[s] >> (16 * khalf), 1.0f, false);
    const _Float16 sc = bscale[f][q / 2];
    const f16x2_t m = {sc, sc};
    const f16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 2 * h) * m;
    const f16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 2 * h + 1) * m;
    v[4 * h + 0] = lo[0];
    v[4 * h + 1] = lo[1];
    v[4 * h + 2] = hi[0];
    v[4 * h + 3] = hi[1];
  };
  // One k-step in program order: MFMA (i, j), then the conversion halves
  // and the loads or reads of its slot, then a scheduling fence, so the
  // conversion of the next k-step (from raw r, chunk s, dword q) is spread
  // evenly over this k-step's MFMAs.
  auto kstep = [&](const Deq& cur, Deq& nxt, const Raw& r, int s, auto qc, auto&& extra) {
    static_for<0, NMMA>([&](auto slot_c) {
      constexpr int slot = decltype(slot_c)::value;
      constexpr int i = slot / FN, j = slot % FN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.b[j], cur.a[i], acc[i][j], 0, 0, 0);
      static_for<slot * 2 * NF / NMMA, (slot + 1) * 2 * NF / NMMA>([&](auto hx_c) {
        constexpr int hx = decltype(hx_c)::value;
        conv_half(r, s, qc, std::integral_constant<int, hx / 2>{},
                  std::integral_constant<int, hx % 2>{}, nxt);
      });
      extra(slot);
      __builtin_amdgcn_sched_barrier(0);
    });
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
  auto none = [&](int) {};
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using Q3 = std::integral_constant<int, 3>;

  // ---- prologue ------------------------------------------------------------
#pragma unroll
  for (int b = 0; b < STAGES; ++b) issue(next_stage(), b);
  wait_vmcnt<(STAGES - 1) * DMA_PER_STAGE>();
  __syncthreads();

  Raw raw[2];
  Deq deq[2];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    read_val(0, 0, f, raw[0]);
    read_scale(0, f, raw[0]);
  }
  static_for<0, NF>([&](auto fc) {
    conv_half(raw[0], 0, Q0{}, fc, std::integral_constant<int, 0>{}, deq[0]);
    conv_half(raw[0], 0, Q0{}, fc, std::integral_constant<int, 1>{}, deq[0]);
  });

  // Eight k-steps per stage (chunk s = u/4, k-step q = u%4). k-step u
  // multiplies deq[u&1] while deq[(u+1)&1] is filled with k-step u+1; the
  // last k-step converts chunk 0 of the next stage. Chunk 1 is read from LDS
  // during k-step 0; before k-step 4 (all waves have read the stage) the
  // next stage must have landed, the barrier frees this buffer for the
  // cursor's next stage, whose loads go out during k-step 4 together with
  // the reads of the next stage's chunk 0.
  int buf = 0;
  bool fresh_tile = false;  // finish stores are in flight
  for (;;) {
    for (uint32_t kt = 0; kt < p.nk; ++kt) {
      // the cursor moves here so that no branch splits the stage's k-steps
      const StageLoad nl = next_stage();
#pragma unroll
      for (int f = 0; f < FM; ++f) raw[1].sa[f] = raw[0].sa[f];
#pragma unroll
      for (int f = 0; f < FN; ++f) raw[1].sb[f] = raw[0].sb[f];
      kstep(deq[0], deq[1], raw[0], 0, Q1{}, [&](int slot) {
        if (slot < NF) read_val(buf, 1, slot, raw[1]);
      });
      kstep(deq[1], deq[0], raw[0], 0, Q2{}, none);
      kstep(deq[0], deq[1], raw[0], 0, Q3{}, none);
      kstep(deq[1], deq[0], raw[1], 1, Q0{}, none);
      pin(deq[0]);

      if (fresh_tile) wait_vmcnt<0>();
      else wait_vmcnt<(STAGES - 2) * DMA_PER_STAGE>();
      fresh_tile = false;
      lds_barrier();
      const int nbuf = (buf + 1 == STAGES) ? 0 : buf + 1;
      // The freed buffer's loads go out over k-steps 4-6, one every few
      // MFMAs, and the next stage's chunk-0 and scale reads over k-steps 5
      // and 6 (k-step 7 converts them; raw[0] is free since k-step 3).
      // Bunched into k-step 4 they made it the stage's slowest (measured
      // with s_memtime: 2550 cycles for k-steps 4-7 against 2280 for 0-3).
      auto late = [&](int j) {
        return [&, j](int slot) {
          const int pos = j * NMMA + slot;
#pragma unroll
          for (int d = pos * NDMA / (3 * NMMA); d < (pos + 1) * NDMA / (3 * NMMA); ++d)
            issue_one(nl, buf, d);
          if (j >= 1) {
            const int r = (j - 1) * NMMA + slot;
#pragma unroll
            for (int e = r * NF / NMMA; e < (r + 1) * NF / NMMA; ++e) {
              if (e % 2 == 0) read_val(nbuf, 0, e / 2, raw[0]);
              else read_scale(nbuf, e / 2, raw[0]);
            }
          }
        };
      };
      kstep(deq[0], deq[1], raw[1], 1, Q1{}, late(0));
      kstep(deq[1], deq[0], raw[1], 1, Q2{}, late(1));
      kstep(deq[0], deq[1], raw[1], 1, Q3{}, late(2));
      kstep(deq[1], deq[0], raw[0], 0, Q0{}, none);
      pin(deq[0]);
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
