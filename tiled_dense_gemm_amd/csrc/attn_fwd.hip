// Softmax attention forward on gfx950: O = softmax(scale * Q K^T) V, bf16
// inputs and output, fp32 accumulation (page "ThunderKittens: Simple, Fast,
// and Adorable AI Kernels", section 3, "PyTorch-Like Operations on Tiles":
// Q K^T, row max, exp, row sum, P V, and the online rescaling of the output
// when the row max grows; "The LCSF Template": key/value tiles stream
// through a multi-stage shared-memory buffer while the queries stay put, the
// finish step divides by the normalisation constant).
//
// Workgroup: W waves (4 by default), 32 query rows of one (batch, head) per
// wave, held in registers for the whole kernel. Keys and values stream
// through an LDS ring of 32-key slots, loaded by direct global->LDS copies.
// Two loop forms: one block per iteration (the resident waves hide each
// other's waits), or a software pipeline that computes the next block's
// scores on the MFMAs while the VALUs turn the current block's scores into
// probabilities (launch configurations at the end of the file).
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
// product, so numerator and denominator use the same weights; it is kept
// in fp32 per window of key blocks and totalled in fp64.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "tkg_attn_layout.hpp"
#include "tkg_device.hpp"
#include "tkg_kernels.hpp"

namespace tkg {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // 4 bf16 pairs

constexpr float kRescaleSlack = 8.0f;  // log2 units
// The row sum is kept in fp32 over windows of this many key blocks and
// folded into an fp64 total after each: one fp32 sum over a million keys
// and more drifts by a part in a few hundred (a term of 1/8 beside a total
// near 2^21, where the fp32 spacing is 1/4), the windowed one by < 1e-3.
constexpr int kRowSumWindow = 64;
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

// Compile-time loop: f(integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
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

// OCC: waves per SIMD, i.e. OCC * 4 / W workgroups per compute unit.
template <int D, bool CAUSAL, int W, int SL, int OCC, bool PIPE>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void attn_fwd_kernel(AttnArgs p) {
  using S = AttnShape<D, W, SL>;
  static_assert(W % 4 == 0 && (OCC * 4) % W == 0, "whole workgroups per compute unit");
  static_assert(S::SLOTS * S::STAGE * (OCC * 4 / W) <= 160 * 1024, "LDS of the resident workgroups");
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[S::SLOTS * S::STAGE];
  TKG_LDS uint8_t* smem = (TKG_LDS uint8_t*)smem_raw;
  const uint32_t lane = threadIdx.x % 64;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);  // uniform
  const uint32_t lr = lane % 32, hh = lane / 32;

  // ---- work item: query block qb of head bh = (b, h). Non-causal: the
  // query blocks of a head are consecutive, and the XCD remap gives every
  // XCD whole heads (their K and V stay in its L2). Causal (work grows with
  // qb): every XCD still owns whole heads and walks them in windows of
  // lpt_heads heads, whose K and V stay cached; inside a window it runs the
  // items heaviest first across the window's heads (longest-processing-
  // time order, so light blocks fill the gaps at the end). Without whole
  // heads per XCD, the order is heaviest first over the grid.
  int bh, qb;
  {
    const int nbh = p.num_wg / p.qblocks;
    if (!CAUSAL) {
      const int v = xcd_virtual_id(blockIdx.x, p.num_wg, p.xcd_remap);
      bh = v / p.qblocks;
      qb = v - bh * p.qblocks;
    } else if (p.xcd_remap && nbh % 8 == 0) {
      const int v = xcd_virtual_id(blockIdx.x, p.num_wg, 1);
      const int per = p.num_wg / 8, hpx = nbh / 8;  // items and heads per XCD
      const int x = v / per, r = v - x * per;
      const int wi = p.lpt_heads * p.qblocks;       // items per window
      const int w = r / wi, rr = r - w * wi;
      qb = p.qblocks - 1 - rr / p.lpt_heads;
      bh = x * hpx + w * p.lpt_heads + rr % p.lpt_heads;
    } else {
      const int v = blockIdx.x;
      qb = p.qblocks - 1 - v / nbh;
      bh = v % nbh;
    }
  }
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
  // the first half of the waves copies K tiles, the second half V tiles
  const bool loads_v = (int)wave * S::NPW >= S::NI / 2;
  const uint16_t* kv = (loads_v ? p.V : p.K) + kvoff;
  const uint32_t kv_bytes = (uint32_t)p.Nk * S::ROWB;

  // ---- ring loads: piece i (1 KiB) of a slot is K (i < NI/2) or V. Lane
  // offsets are relative to the block's first key, where each block's
  // buffer starts (base and size in scalar registers, so the per-lane
  // offsets stay fixed); keys past Nk read zeros.
  uint32_t dma_off[S::NPW];
#pragma unroll
  for (int j = 0; j < S::NPW; ++j) {
    const uint32_t i = wave * S::NPW + j;
    const uint32_t chunk = (i % (S::NI / 2)) * 64 + lane;
    const uint32_t row = chunk / S::CPR, cs = chunk % S::CPR;
    const uint32_t c = cs ^ (loads_v ? attn_v_swz(D, row) : attn_k_swz(D, row));
    dma_off[j] = row * S::ROWB + 16 * c;
  }
  auto issue = [&](int blk, uint32_t slot_off) {
    const uint32_t k0b = (uint32_t)blk * (S::BK * S::ROWB);
    // bytes left from the block's first key: 0 for the prologue's blocks
    // past the last key (k0b can then pass 2^31 while kv_bytes < 2^31, so
    // the difference is taken in 64 bits); uniform, and kept in a scalar
    // register for the asm's resource operand
    const int64_t rest = (int64_t)kv_bytes - (int64_t)k0b;
    const uint32_t left = rest > 0 ? (uint32_t)rest : 0u;
    const i32x4_t r = rsrc_words(reinterpret_cast<const uint8_t*>(kv) + k0b,
                                 (uint32_t)__builtin_amdgcn_readfirstlane((int)left));
    const uint32_t dst = (uint32_t)(uintptr_t)smem + slot_off + wave * S::NPW * 1024;
#pragma unroll
    for (int j = 0; j < S::NPW; ++j) dma_b128_ring(r, dst + j * 1024, dma_off[j]);
  };

  // ---- LDS read addresses: K fragment ks at (lane_k ^ 32 ks); V read (s, t,
  // db) at TILE + (16 s + 8 t) ROWB + (lane_v ^ 64 db) (attn_k_read and
  // attn_v_read with kb = 0)
  const uint32_t lane_k = attn_k_read(D, lane, 0, 0);
  const uint32_t lane_v = attn_v_read(D, lane, 0, 0, 0, 0);

  bf16x8_t qf[S::KS];  // filled below, once the ring's first block is issued
  f32x16_t o[S::DB];
#pragma unroll
  for (int db = 0; db < S::DB; ++db) o[db] = f32x16_t{};
  float m = -INFINITY;  // reference max, log2 units (same in lanes l, l ^ 32)
  float thr = -INFINITY;  // m + kRescaleSlack
  float l = 0.0f;       // this lane's part of the row sum, current window
  double lw = 0.0;      // ... over the finished windows
  const float c = p.c;
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};

  // ---- the steps of one 32-key block. A slot's K tile is at its base, its
  // V tile TILE bytes after.
  // S^T = K Q^T
  auto s_mma = [&](uint32_t sbase, f32x16_t& sa) {
    sa = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
      const bf16x8_t kf = lds_read<bf16x8_t>(smem, sbase + (lane_k ^ (32u * ks)));
      sa = mfma_bf16(kf, qf[ks], sa);
    }
  };
  // keys past Nk, and (causal) keys after the query, get -inf; only the
  // wave's last block can hold such keys
  auto needs_mask = [&](int blk) {
    const int key0 = blk * S::BK;
    return key0 + S::BK > p.Nk || (CAUSAL && key0 + S::BK - 1 > q0w);
  };
  auto mask = [&](f32x16_t& sa, int blk) {
    const int key0 = blk * S::BK, q = q0w + (int)lr;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = key0 + 8 * (e / 4) + 4 * (int)hh + e % 4;
      if (key >= p.Nk || (CAUSAL && key > q)) sa[e] = -INFINITY;
    }
  };
  // the block's row max in log2 units (scores scale after: c > 0), both
  // halves of the row (lanes l, l ^ 32); raises the reference max m when
  // it grows by more than the slack, rescaling O and the row sum. Whether
  // any row grows that much is decided on each lane's half of its row
  // (max(a, b) c = max(a c, b c) for c > 0, so the wave's decision is the
  // same); the halves are combined only when some row does.
  auto update_max = [&](const f32x16_t& sa) {
    float mx = sa[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = __builtin_elementwise_maximum(mx, sa[e]);
    if (__builtin_amdgcn_ballot_w64(mx * c > thr)) {
      const float mloc = max_with_partner(mx) * c;
      const float mn = fmaxf(m, mloc);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);  // 0 on the first block
      l *= alpha;
      lw *= (double)alpha;
#pragma unroll
      for (int db = 0; db < S::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      m = mn;
      thr = m + kRescaleSlack;
    }
  };
  // probability pair t (scores 2t, 2t+1) in bf16, into the P^T operand of
  // k-step t / 4 (accumulator elements 8s .. 8s+7), added to the row sum
  // (a pair is kept as one 32-bit word, so it is converted once)
  auto prob_pair = [&](const f32x16_t& sa, int t, u32x4_t (&pk)[2]) {
    const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[2 * t], c, -m));
    const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[2 * t + 1], c, -m));
    const bf16x2_t pr = {(__bf16)e0, (__bf16)e1};
    pk[t / 4][t % 4] = __builtin_bit_cast(uint32_t, pr);
    l = __builtin_amdgcn_fdot2_f32_bf16(pr, one, l, false);
    return pr;
  };
  // V^T fragments of the block (A operands of its P V MFMAs)
  auto v_frags = [&](uint32_t sbase, bf16x8_t (&vf)[2][S::DB]) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int db = 0; db < S::DB; ++db) {
        const uint32_t a = sbase + S::TILE + 16 * s * S::ROWB + (lane_v ^ (64u * db));
        const s16x4_t v0 = lds_read_tr16(smem, a);
        const s16x4_t v1 = lds_read_tr16(smem, a + 8 * S::ROWB);
        vf[s][db] = __builtin_bit_cast(bf16x8_t,
                                       __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
  };
  // O^T += V^T P^T
  auto pv_mma = [&](const u32x4_t (&pk)[2], const bf16x8_t (&vf)[2][S::DB]) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int db = 0; db < S::DB; ++db)
        o[db] = mfma_bf16(vf[s][db], __builtin_bit_cast(bf16x8_t, pk[s]), o[db]);
  };
  // Pipelined phase 1, in issue order: the K fragment reads of the next
  // block (four in flight) and the V^T fragment reads of the current one,
  // then per MFMA of the next block's S^T one or two pairs of the current
  // block's probabilities ahead of it; the fences keep this order.
  auto phase1 = [&](uint32_t cur, uint32_t nxt, f32x16_t& sn, const f32x16_t& sc,
                    u32x4_t (&pk)[2], bf16x8_t (&vf)[2][S::DB]) {
    constexpr int PPM = 8 / S::KS;              // probability pairs per MFMA
    constexpr int KA = S::KS < 4 ? S::KS : 4;   // K reads in flight
    bf16x8_t kf[S::KS];
#pragma unroll
    for (int i = 0; i < KA; ++i) kf[i] = lds_read<bf16x8_t>(smem, nxt + (lane_k ^ (32u * i)));
    v_frags(cur, vf);
    __builtin_amdgcn_sched_barrier(0);
    sn = f32x16_t{};
#pragma unroll
    for (int i = 0; i < S::KS; ++i) {
#pragma unroll
      for (int t = PPM * i; t < PPM * (i + 1); ++t) {
        const bf16x2_t pr = prob_pair(sc, t, pk);
        // (anchors the pair here: it is only read after the mask branch,
        // and the compiler would otherwise sink it there)
        asm volatile("" : "+v"(l) : "v"(pr));
      }
      __builtin_amdgcn_sched_barrier(0);
      if (i + KA < S::KS)
        kf[i + KA] = lds_read<bf16x8_t>(smem, nxt + (lane_k ^ (32u * (i + KA))));
      sn = mfma_bf16(kf[i], qf[i], sn);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- the ring. At the top of an iteration: wait for this wave's copies
  // of the blocks the iteration reads, barrier (every copy landed; every
  // wave is done with the slot about to be refilled, block blk - 1's),
  // issue block blk + SLOTS - 1. Blocks past the last one read zeros, or
  // keys the workgroup does not use, into slots that are never read: the
  // prologue issues them unconditionally so the counts are exact.
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
  for (int st = 1; st < S::SLOTS - 1; ++st) issue(st, st * S::STAGE);
  // The loops below run SLOTS blocks per iteration, so the slot of every
  // block (blk mod SLOTS) is a compile-time constant J and its LDS offsets
  // fold into the LDS instructions. Blocks blk + AHEAD + 1 .. blk + SLOTS -
  // 2 may still be in flight when block blk starts (the pipelined loop also
  // reads block blk + 1).
  constexpr int AHEAD = PIPE ? 1 : 0;
  auto top = [&](auto J, int blk) {
    constexpr int j = decltype(J)::value;
    if (blk + S::SLOTS - 2 < nblk)
      wait_vmcnt<(S::SLOTS - 2 - AHEAD) * S::NPW>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    const int nx = blk + S::SLOTS - 1;
    if (nx < nblk) issue(nx, (uint32_t)((j + S::SLOTS - 1) % S::SLOTS) * S::STAGE);
  };

  // after the pass starting at block b0: at a window's end, the window's
  // row sum goes into the fp64 total (the branch is uniform)
  static_assert(kRowSumWindow % S::SLOTS == 0, "whole passes per row-sum window");
  auto fold_row_sum = [&](int b0) {
    if ((b0 + S::SLOTS) % kRowSumWindow == 0) {
      lw += (double)l;
      l = 0.0f;
    }
  };

  if constexpr (!PIPE) {
    // one block per step: scores, max, probabilities, P V; the other waves
    // on the SIMD fill each wave's dependency waits
    for (int b0 = 0; b0 < nblk; b0 += S::SLOTS) {
      static_for<0, S::SLOTS>([&](auto J) {
        constexpr int j = decltype(J)::value;
        const int blk = b0 + j;
        if (blk >= nblk) return;
        top(J, blk);
        if (blk < wblk) {
          constexpr uint32_t cur = (uint32_t)j * S::STAGE;
          f32x16_t sc;
          u32x4_t pk[2];
          bf16x8_t vf[2][S::DB];
          s_mma(cur, sc);
          if (needs_mask(blk)) mask(sc, blk);
          update_max(sc);
#pragma unroll
          for (int t = 0; t < 8; ++t) prob_pair(sc, t, pk);
          v_frags(cur, vf);
          pv_mma(pk, vf);
        }
      });
      fold_row_sum(b0);
    }
  } else {
    // Software pipeline: step blk computes block blk + 1's scores on the
    // MFMAs while the VALUs turn block blk's scores into probabilities
    // (phase1), then accumulates block blk's P V while the VALUs take block
    // blk + 1's max. On a wave's last block, block blk + 1 lies wholly past
    // its keys (past Nk, or after every query of the wave): its scores are
    // masked to -inf, which leaves the max alone, so the last step needs no
    // other path. Scores alternate between two accumulators (even and odd
    // blocks), so SLOTS is even.
    static_assert(!PIPE || S::SLOTS % 2 == 0, "even and odd blocks alternate within a pass");
    auto step = [&](auto J, int blk, f32x16_t& sc, f32x16_t& sn) {
      constexpr int j = decltype(J)::value;
      top(J, blk);
      if (blk < wblk) {
        constexpr uint32_t cur = (uint32_t)j * S::STAGE;
        constexpr uint32_t nxt = (uint32_t)((j + 1) % S::SLOTS) * S::STAGE;
        u32x4_t pk[2];
        bf16x8_t vf[2][S::DB];
        phase1(cur, nxt, sn, sc, pk, vf);
        if (needs_mask(blk + 1)) mask(sn, blk + 1);
        pv_mma(pk, vf);
        update_max(sn);
      }
    };
    lds_barrier();  // block 0 landed in every wave
    f32x16_t sa, sb;  // scores of even / odd blocks
    if (wblk > 0) {
      s_mma(0, sa);
      if (needs_mask(0)) mask(sa, 0);
      update_max(sa);
    }
    for (int b0 = 0; b0 < nblk; b0 += S::SLOTS) {
      static_for<0, S::SLOTS>([&](auto J) {
        constexpr int j = decltype(J)::value;
        if (b0 + j >= nblk) return;
        if constexpr (j % 2 == 0)
          step(J, b0 + j, sa, sb);
        else
          step(J, b0 + j, sb, sa);
      });
      fold_row_sum(b0);
    }
  }

  // ---- finish: divide by the row sum, store bf16 rows and the log-sum-exp
  const float lt = sum_with_partner((float)(lw + (double)l));
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

// Launch configurations: (waves, ring slots, waves per SIMD, pipelined).
// Measured on the B=16 N=4096 workloads (TFLOP/s, non-causal / causal):
// D = 128: (4, 4, 2, pipelined) 1080 / 933, (4, 3, 3, plain) 1020 / 930,
// (8, 8, 2, pipelined) 993 / 853; D = 64: (4, 4, 4, plain) 950,
// (8, 8, 2, pipelined) 810, (4, 4, 2, pipelined) 839; against (4, 4, 4,
// plain) at 905-918 in another run, (4, 4, 5, plain) 910-916 and (4, 5, 4,
// plain) 860. Four waves per
// workgroup (128 query rows) balance causal work better than eight; at
// D = 64 the softmax outweighs the MFMAs and more resident waves win.
template <int D, int W, int SL, int OCC, bool PIPE>
struct AttnCfg {
  static constexpr int BQ = AttnShape<D, W, SL>::BQ;
  template <bool CAUSAL>
  static hipError_t launch(const AttnArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, W, SL, OCC, PIPE>), dim3(a.num_wg),
                       dim3(64 * W), 0, stream, a);
    return hipGetLastError();
  }
};
using Cfg128 = AttnCfg<128, 4, 4, 2, true>;
using Cfg64 = AttnCfg<64, 4, 4, 4, false>;

}  // namespace

int attn_block_q(int D) { return D == 64 ? Cfg64::BQ : D == 128 ? Cfg128::BQ : 0; }

// Causal longest-first windows: as many of an XCD's heads as keep their
// keys and values within this many bytes. Measured (causal, TFLOP/s):
// ordering across all of an XCD's heads pushed the working set out to HBM
// at B=16 Hq=16 N=4096 D=128 (6.8x the compulsory bytes, 808); windows of
// 1, 2, 4, 8 and 16 MiB gave 933, 937, 961, 968 and 948 there, and over
// ten causal workloads (N 1024-16384, D 64 and 128) 8 MiB was best or
// within 2% except D=128 N=1024 (4 MiB 750, 8 MiB 709).
constexpr int64_t kAttnLptBytes = 8 << 20;
static int lpt_window(const AttnArgs& a, int D) {
  const int nbh = a.num_wg / a.qblocks;
  if (nbh % 8 != 0) return 1;
  const int hpx = nbh / 8;
  // K and V bytes per query head (a key/value head serves `group` of them)
  const int64_t share = std::max<int64_t>(1, (int64_t)a.Nk * D * 4 / a.group);
  int w = (int)std::min<int64_t>(hpx, std::max<int64_t>(1, kAttnLptBytes / share));
  while (hpx % w != 0) --w;
  return w;
}

hipError_t launch_attn(const AttnArgs& args, int D, bool causal, hipStream_t stream) {
  AttnArgs a = args;
  a.lpt_heads = causal ? lpt_window(a, D) : 1;
  if (D == 64) return causal ? Cfg64::launch<true>(a, stream) : Cfg64::launch<false>(a, stream);
  if (D == 128) return causal ? Cfg128::launch<true>(a, stream) : Cfg128::launch<false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace tkg
