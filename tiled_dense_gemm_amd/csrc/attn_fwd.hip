// Softmax attention forward on gfx950: O = softmax(scale * Q K^T) V, bf16
// inputs and output, fp32 accumulation (page "ThunderKittens: Simple, Fast,
// and Adorable AI Kernels", section 3, "PyTorch-Like Operations on Tiles":
// Q K^T, row max, exp, row sum, P V, and the online rescaling of the output
// when the row max grows; "The LCSF Template": key/value tiles stream
// through a multi-stage shared-memory buffer while the queries stay put, the
// finish step divides by the normalisation constant).
//
// Workgroup: 8 waves, 256 query rows of one (batch, head), 32 rows per wave
// held in registers for the whole kernel. Keys and values stream through a
// 4-slot LDS ring, 64 keys per slot, loaded by direct global->LDS copies.
//
// Per wave and key block the MFMAs run with the keys as the A operand, so
// the score accumulator holds S^T: lane l owns query l % 32 and 16 of the
// 32 keys of each 32-key block (the other 16 sit in lane l ^ 32). The row
// max and row sum are then lane-local plus one exchange with the partner
// lane, and O is accumulated as O^T = V^T P^T: lane l owns query l % 32 of
// every output block, so rescaling by the new max and the final division
// are lane-local too. P^T needs no data movement: the accumulator elements
// 8s .. 8s+7 of a 32-key block are exactly the lane's B operand of k-step s
// once V^T's A operand lists the keys in the same order, which the
// transposing LDS read (ds_read_b64_tr_b16) delivers straight from the
// row-major V tile.
//
// The exponentials are taken in base 2 with the scale folded in
// (c = scale * log2 e). The reference max m used in exp2(c s - m) is only
// raised when a block's row max exceeds it by more than 8 (in log2 units):
// the probabilities then stay below 2^8, and most blocks skip the rescale
// of O. The row sum adds the bf16-rounded probabilities that enter the P V
// product, so numerator and denominator use the same weights.
#include <math.h>

#include "tkg_attn_layout.hpp"
#include "tkg_device.hpp"
#include "tkg_kernels.hpp"

namespace tkg {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

constexpr float kRescaleSlack = 8.0f;  // log2 units
constexpr float kLn2 = 0.69314718055994530942f;

// 8-byte transposing LDS read (see attn_v_read in tkg_attn_layout.hpp).
__device__ __forceinline__ s16x4_t lds_read_tr16(const TKG_LDS uint8_t* base, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((TKG_LDS s16x4_t*)(base + off));
}

// 16 bytes per lane from global memory into LDS (the wave writes 1 KiB at
// LDS byte address `lds`, lane l at 16 l), bounds-checked by the resource
// words `r` (loads at or past r[2] bytes return zeros). Issued from asm so
// that the compiler does not treat it as an LDS write it must order reads
// after: it would otherwise wait for every copy in flight (the whole ring)
// before each transposing read, which it cannot tell apart from the slot
// being filled. The ring's own waits (vmcnt, then a barrier) order the
// slots.
// m0 is reserved for the compiler, which only loads it right before its own
// uses of it (none in this kernel); the clobber documents the write.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_b128_ring(i32x4_t r, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop
// Resource words of a raw buffer over [base, base + nbytes) (stride 0).
__device__ __forceinline__ i32x4_t rsrc_words(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4_t{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), (int)nbytes,
                 0x00020000};
}

__device__ __forceinline__ float max_with_partner(float x) {
  // lanes l and l ^ 32 exchange values: {x of lane l % 32, x of lane l % 32 + 32}
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(AttnArgs p) {
  using S = AttnShape<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[S::SLOTS * S::STAGE];
  TKG_LDS uint8_t* smem = (TKG_LDS uint8_t*)smem_raw;
  const uint32_t lane = threadIdx.x % 64;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);  // uniform
  const uint32_t lr = lane % 32, hh = lane / 32;

  // ---- work item: query block qb of head (b, h); causal blocks heaviest first
  const int v = xcd_virtual_id(blockIdx.x, p.num_wg, p.xcd_remap);
  const int bh = v / p.qblocks;
  int qb = v - bh * p.qblocks;
  if (CAUSAL) qb = p.qblocks - 1 - qb;
  const int b = bh / p.Hq, h = bh - b * p.Hq;
  const size_t qoff = (size_t)bh * (size_t)p.Nq * D;
  const size_t kvoff = ((size_t)b * p.Hkv + h / p.group) * (size_t)p.Nk * D;
  const int q0 = qb * S::BQ;
  const int q0w = q0 + (int)wave * S::QW;
  const int kend = CAUSAL ? min(p.Nk, q0 + S::BQ) : p.Nk;
  const int nblk = (kend + S::BK - 1) / S::BK;          // key blocks of the workgroup
  const int wend = CAUSAL ? min(p.Nk, q0w + S::QW) : p.Nk;
  const int wblk = q0w < p.Nq ? (wend + S::BK - 1) / S::BK : 0;  // of this wave

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.Q + qoff, (uint32_t)p.Nq * S::ROWB);
  const bool loads_v = (int)wave * S::NPW >= S::NI / 2;  // waves 0..3 load K, 4..7 V
  const i32x4_t rkv = rsrc_words((loads_v ? p.V : p.K) + kvoff, (uint32_t)p.Nk * S::ROWB);

  // ---- ring loads: piece i (1 KiB) of a slot is K (i < NI/2) or V. Lane
  // offsets are relative to the block's first key; keys past Nk read zeros.
  uint32_t dma_off[S::NPW];
#pragma unroll
  for (int j = 0; j < S::NPW; ++j) {
    const uint32_t i = wave * S::NPW + j;
    const uint32_t chunk = (i % (S::NI / 2)) * 64 + lane;
    const uint32_t row = chunk / S::CPR, cs = chunk % S::CPR;
    const uint32_t c = cs ^ (loads_v ? attn_v_swz(D, row) : attn_k_swz(D, row));
    dma_off[j] = row * S::ROWB + 16 * c;
  }
  auto issue = [&](int blk, int slot) {
    const uint32_t k0b = (uint32_t)blk * (S::BK * S::ROWB);
    const uint32_t dst = (uint32_t)(uintptr_t)smem + slot * S::STAGE + wave * S::NPW * 1024;
#pragma unroll
    for (int j = 0; j < S::NPW; ++j) dma_b128_ring(rkv, dst + j * 1024, dma_off[j] + k0b);
  };

  // ---- LDS read addresses: K fragment (kb, ks) at 32 kb ROWB + (lane_k ^
  // 32 ks); V read (kb, s, t, db) at TILE + (32 kb + 16 s + 8 t) ROWB +
  // (lane_v ^ 64 db) (attn_k_read / attn_v_read)
  const uint32_t lane_k = attn_k_read(D, lane, 0, 0);
  const uint32_t lane_v = attn_v_read(D, lane, 0, 0, 0, 0);

  bf16x8_t qf[S::KS];  // filled below, once the ring's first block is issued
  f32x16_t o[S::DB];
#pragma unroll
  for (int db = 0; db < S::DB; ++db) o[db] = f32x16_t{};
  float m = -INFINITY;  // reference max, log2 units (same in lanes l, l ^ 32)
  float l = 0.0f;       // this lane's part of the row sum
  const float c = p.c;

  auto compute = [&](int blk, uint32_t sbase) {
    // S^T = K Q^T for two 32-key blocks
    f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t kf =
            lds_read<bf16x8_t>(smem, sbase + 32 * kb * S::ROWB + (lane_k ^ (32u * ks)));
        sacc[kb] = mfma_bf16(kf, qf[ks], sacc[kb]);
      }
    }
    // keys past Nk, and (causal) keys after the query, get -inf
    const int key0 = blk * S::BK;
    if (key0 + S::BK > p.Nk || (CAUSAL && key0 + S::BK - 1 > q0w)) {
      const int q = q0w + (int)lr;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = key0 + 32 * kb + 8 * (e / 4) + 4 * (int)hh + e % 4;
          if (key >= p.Nk || (CAUSAL && key > q)) sacc[kb][e] = -INFINITY;
        }
    }
    // row max of the block (scores are scaled after: c > 0)
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
    const float mloc = max_with_partner(mx) * c;
    if (__builtin_amdgcn_ballot_w64(mloc > m + kRescaleSlack)) {
      const float mn = fmaxf(m, mloc);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);  // 0 on the first block
      l *= alpha;
#pragma unroll
      for (int db = 0; db < S::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      m = mn;
    }
    // probabilities in bf16; P^T operand of k-step s = elements 8s .. 8s+7
    bf16x8_t pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8_t x;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          x[j] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * s + j], c, -m));
        pf[kb][s] = x;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const bf16x2_t pair = {x[j], x[j + 1]};
          const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
          l = __builtin_amdgcn_fdot2_f32_bf16(pair, one, l, false);
        }
      }
    // O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int db = 0; db < S::DB; ++db) {
          const uint32_t a = sbase + S::TILE + (32 * kb + 16 * s) * S::ROWB + (lane_v ^ (64u * db));
          const s16x4_t v0 = lds_read_tr16(smem, a);
          const s16x4_t v1 = lds_read_tr16(smem, a + 8 * S::ROWB);
          const s16x8_t vv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          o[db] = mfma_bf16(__builtin_bit_cast(bf16x8_t, vv), pf[kb][s], o[db]);
        }
  };

  // ---- the ring: wait for this wave's copies of block blk, barrier (all
  // copies landed, everyone done with the slot about to be refilled), issue
  // block blk + SLOTS - 1, compute blk. Blocks past the last one read
  // zeros, or keys the workgroup does not use, into slots that are never
  // read: the prologue issues them unconditionally so the counts are exact.
  issue(0, 0);
  // Q^T fragments (B operand): lane l holds query q0w + l % 32, d =
  // 16 ks + 8 (l / 32) .. +7; rows past Nq read zeros. They arrive with
  // block 0 (copies complete in order); the other prologue blocks are
  // issued after, so the wait for Q does not wait for them.
  {
    const uint32_t off = (uint32_t)(q0w + (int)lr) * S::ROWB + 16 * hh;
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                rq, (int)(off + 32 * ks), 0, 0));
  }
  wait_vmcnt<0>();
#pragma unroll
  for (int ks = 0; ks < S::KS; ++ks) asm volatile("" : "+v"(qf[ks]));
#pragma unroll
  for (int st = 1; st < S::SLOTS - 1; ++st) issue(st, st);
  for (int blk = 0; blk < nblk; ++blk) {
    if (blk + S::SLOTS - 2 < nblk)
      wait_vmcnt<(S::SLOTS - 2) * S::NPW>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    const int nx = blk + S::SLOTS - 1;
    if (nx < nblk) issue(nx, nx % S::SLOTS);
    if (blk < wblk) compute(blk, (uint32_t)(blk % S::SLOTS) * S::STAGE);
  }

  // ---- finish: divide by the row sum, store bf16 rows and the log-sum-exp
  const float lt = sum_with_partner(l);
  const int q = q0w + (int)lr;
  if (wblk > 0 && q < p.Nq) {
    const float inv = 1.0f / lt;
    uint16_t* orow = p.O + qoff + (size_t)q * D;
#pragma unroll
    for (int db = 0; db < S::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint2 w = pack_bf16x4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv,
                                    o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * db + 8 * g + 4 * hh) = w;
      }
    if (p.lse != nullptr && hh == 0)
      p.lse[(size_t)bh * p.Nq + q] = (m + __builtin_log2f(lt)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const AttnArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL>), dim3(a.num_wg), dim3(64 * AttnShape<D>::WAVES),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, int D, bool causal, hipStream_t stream) {
  if (D == 64) return causal ? launch_one<64, true>(a, stream) : launch_one<64, false>(a, stream);
  if (D == 128) return causal ? launch_one<128, true>(a, stream) : launch_one<128, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace tkg
