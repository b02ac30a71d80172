// LDS bank-conflict probe for gfx950 (MI355X). One dispatch per address
// pattern: every lane of 256 workgroups x 4 waves reads its own LDS address
// (16, 8 or 4 bytes) 2048 times, alternately at +0 and +32 KiB, so the
// SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE counters of the dispatch give the
// pattern's conflict degree. Patterns:
//   * geometry: contiguous reads and lane pairs sharing a bank group, for
//     ds_read_b128 / b64 / b32;
//   * every fragment read of the default GEMM kernels (16x16 bf16 blocks,
//     32x32 fp8 blocks and the 4-bit kernel's 64-byte rows), with the
//     swizzle of tkg_layout.hpp and without it;
//   * the 4-bit kernel's 8-byte block-scale reads, and the MX kernels'
//     16-byte superstage scale rows (whole-row reads, and the single-word
//     reads they replace);
//   * the finish's staging strip (tkg_finish.hpp): the writes and reads of
//     every strip shape, restated here, and two layouts it rejects (rows
//     padded by 16 bytes with 8-byte writes; 128-byte rows with the chunk
//     XOR-ed by row bits);
//   * a search over all 4096 linear row swizzles of 128-byte rows,
//     chunk ^ A*bits(row mod 16), read with the 16x16 fragment pattern.
// Writes (ds_write) run in a kernel of their own. It prints one line per
// dispatch, in order: "pattern <id> <bytes> <op> <name> : <64 addresses>"
// (op r or w), which lds_probe_summary.py joins with the counters.
//
// Build: hipcc --offload-arch=gfx950 -O2 -std=c++17 lds_bank_probe.hip -o lds_bank_probe
#include <hip/hip_runtime.h>

#include <cstdio>
#include <string>
#include <vector>

#define LDS_AS __attribute__((address_space(3)))
typedef int i4 __attribute__((ext_vector_type(4)));
typedef int i2 __attribute__((ext_vector_type(2)));

constexpr unsigned kSpan = 32768;  // addresses are < kSpan; reads alternate +kSpan

template <int BYTES, bool WRITE>
__global__ __launch_bounds__(256) void lds_probe(const unsigned* addrs, int* out, int iters) {
  __shared__ __attribute__((aligned(16))) int smem[2 * kSpan / 4];
  for (unsigned i = threadIdx.x; i < 2 * kSpan / 4; i += 256) smem[i] = (int)(i * 7 + 1);
  __syncthreads();
  const unsigned lane = threadIdx.x & 63;
  const unsigned a = addrs[lane];
  LDS_AS char* base = (LDS_AS char*)smem;
  int acc = 0;
  for (int it = 0; it < iters; ++it) {
    const unsigned off = a + ((it & 1) ? kSpan : 0);
    if constexpr (WRITE && BYTES == 16) {
      *(LDS_AS i4*)(base + off) = i4{it, (int)lane, acc, 1};
    } else if constexpr (WRITE) {
      *(LDS_AS i2*)(base + off) = i2{it, (int)lane};
    } else if constexpr (BYTES == 16) {
      const i4 v = *(const LDS_AS i4*)(base + off);
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    } else if constexpr (BYTES == 8) {
      const i2 v = *(const LDS_AS i2*)(base + off);
      acc ^= v[0] ^ v[1];
    } else {
      acc ^= *(const LDS_AS int*)(base + off);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (WRITE) {
    __syncthreads();
    acc = smem[threadIdx.x];
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

struct Pattern {
  std::string name;
  unsigned bytes;
  std::vector<unsigned> addr;
  bool write = false;
};

// The swizzle of tkg_layout.hpp, restated: XOR mask of the 16-byte chunk
// index of row r for 128- and 64-byte rows.
static unsigned swz_mask(unsigned row_bytes, unsigned r) {
  return row_bytes == 128 ? ((r & 7u) ^ (((r >> 3) & 1u) * 7u)) : ((r >> 2) & 3u);
}
static unsigned swz(unsigned row_bytes, unsigned r, unsigned c, bool on) {
  return r * row_bytes + ((c ^ (on ? swz_mask(row_bytes, r) : 0u)) << 4);
}

// Fragment read of a kernel: MFMA block `mi` rows per fragment, lanes l and
// l + mi read the same row; k-step `step` covers `cpk` 16-byte chunks, lane
// group l / mi reads `parts` consecutive ones (part `part`).
static Pattern fragment(const char* kind, unsigned row_bytes, unsigned mi, unsigned cpk,
                        unsigned step, unsigned part, unsigned frag, bool swizzled) {
  const unsigned parts = cpk / (64 / mi);
  Pattern p{std::string(kind) + (swizzled ? " swizzled" : " unswizzled") + " step " +
                std::to_string(step) + " part " + std::to_string(part) + " frag " +
                std::to_string(frag),
            16, std::vector<unsigned>(64)};
  for (unsigned l = 0; l < 64; ++l) {
    const unsigned row = frag * mi + l % mi;
    const unsigned chunk = step * cpk + (l / mi) * parts + part;
    p.addr[l] = swz(row_bytes, row, chunk, swizzled);
  }
  return p;
}

// The finish strip of tkg_finish.hpp, restated: MI-row strip of rb-byte
// rows kept in 256-byte lines (row r in line r mod NR at slot r / NR, the
// 16-byte chunk XOR-ed with line mod 16); lane l writes 16 bytes of row
// l % MI at chunk cchunk ^ lchunk, and read q gives lane l line 4q + l/16
// at line chunk l % 16.
static unsigned fin_write(unsigned mi, unsigned rb, unsigned l, unsigned cc) {
  const unsigned lrow = l % mi, lgrp = l / mi;
  const unsigned lch = mi == 32 ? lgrp : 2 * (lgrp & 1) + (lgrp >> 1);
  const unsigned nr = mi * rb / 256, line = lrow % nr, slot = lrow / nr;
  return line * 256 + ((((slot * (rb / 16)) ^ lch ^ (line % 16)) ^ cc) << 4);
}
static unsigned fin_read(unsigned l, unsigned q) {
  return q * 1024 + ((((l / 16) * 256) + (((l % 16) ^ (l / 16)) << 4)) ^ (((4 * q) % 16) << 4));
}

int main() {
  std::vector<Pattern> pats;
  auto add = [&](std::string name, unsigned bytes, auto f) {
    Pattern p{name, bytes, std::vector<unsigned>(64)};
    for (unsigned l = 0; l < 64; ++l) p.addr[l] = f(l);
    pats.push_back(p);
  };
  // geometry
  for (unsigned bytes : {16u, 8u, 4u}) {
    const std::string w = "b" + std::to_string(bytes * 8);
    add(w + " contiguous", bytes, [&](unsigned l) { return bytes * l; });
    for (unsigned d = 1; d <= 32; d <<= 1)
      add(w + " lanes l and l^" + std::to_string(d) + " share a bank group", bytes,
          [&](unsigned l) { return bytes * (l & ~d) + ((l & d) ? 4096u : 0u); });
  }
  add("b64 4-bit block scales (row l%32, 8-byte rows)", 8, [](unsigned l) { return 8 * (l % 32); });
  add("b32 4-bit block scale word (row l%16, word l/32 of 8-byte rows)", 4,
      [](unsigned l) { return 8 * (l % 16) + 4 * (l / 32); });
  add("b128 MX superstage scale rows (row l%32, 16-byte rows)", 16, [](unsigned l) { return 16 * (l % 32); });
  add("b32 MX scale word of 16-byte rows (row l%32)", 4, [](unsigned l) { return 16 * (l % 32); });
  add("b64 MX scale pair of 16-byte rows (row l%32)", 8, [](unsigned l) { return 16 * (l % 32); });
  // the finish strip: every shape the kernels use (mi, rj)
  const unsigned fshapes[][2] = {{32, 4}, {32, 2}, {32, 1}, {16, 8}, {16, 4}, {16, 2}};
  for (const auto& fs : fshapes) {
    const unsigned mi = fs[0], rj = fs[1], rb = rj * mi * 2;
    const unsigned nw = mi == 32 ? 2 * rj : rj / 2, nrd = mi * rb / 1024;
    for (unsigned w = 0; w < nw; ++w) {
      const unsigned cc = mi == 32 ? 4 * (w / 2) + 2 * (w % 2) : 4 * w;
      Pattern p{"finish mi" + std::to_string(mi) + " rj" + std::to_string(rj) + " write " +
                    std::to_string(w),
                16, std::vector<unsigned>(64), true};
      for (unsigned l = 0; l < 64; ++l) p.addr[l] = fin_write(mi, rb, l, cc);
      pats.push_back(p);
    }
    for (unsigned q = 0; q < nrd; ++q) {
      Pattern p{"finish mi" + std::to_string(mi) + " rj" + std::to_string(rj) + " read " +
                    std::to_string(q),
                16, std::vector<unsigned>(64)};
      for (unsigned l = 0; l < 64; ++l) p.addr[l] = fin_read(l, q);
      pats.push_back(p);
    }
  }
  // rejected finish layouts: 144-byte rows written 8 bytes per lane (the
  // accumulator layout without the swap), and 128-byte rows whose chunk is
  // XOR-ed by (row / 2) mod 8, written 16 bytes per lane
  {
    Pattern p{"finish rejected padded rows b64 write", 8, std::vector<unsigned>(64), true};
    for (unsigned l = 0; l < 64; ++l) p.addr[l] = (l % 32) * 144 + 8 * (l / 32);
    pats.push_back(p);
    Pattern q{"finish rejected 128-byte rows xor write", 16, std::vector<unsigned>(64), true};
    for (unsigned l = 0; l < 64; ++l) q.addr[l] = (l % 32) * 128 + (((l / 32) ^ ((l % 32) / 2 % 8)) << 4);
    pats.push_back(q);
  }
  // the kernels' fragment reads, swizzled and not
  for (bool on : {true, false}) {
    for (unsigned s = 0; s < 2; ++s)
      for (unsigned f = 0; f < 16; ++f) pats.push_back(fragment("bf16 16x16x32", 128, 16, 4, s, 0, f, on));
    for (unsigned s = 0; s < 2; ++s)
      for (unsigned q = 0; q < 2; ++q)
        for (unsigned f = 0; f < 8; ++f) pats.push_back(fragment("fp8 32x32x64", 128, 32, 4, s, q, f, on));
    for (unsigned q = 0; q < 2; ++q)
      for (unsigned f = 0; f < 16; ++f) pats.push_back(fragment("fp8 16x16x128", 128, 16, 8, 0, q, f, on));
    for (unsigned s = 0; s < 2; ++s)
      for (unsigned f = 0; f < 8; ++f) pats.push_back(fragment("4-bit values", 64, 32, 2, s, 0, f, on));
    for (unsigned f = 0; f < 16; ++f) pats.push_back(fragment("4-bit values 16x16x32", 64, 16, 4, 0, 0, f, on));
  }
  // linear swizzle search on the 16x16 pattern (rows 0..15, chunks 0..3)
  for (unsigned A = 0; A < 4096; ++A)
    add("search A=" + std::to_string(A), 16, [&](unsigned l) {
      const unsigned r = l % 16, c = l / 16;
      unsigned m = 0;
      for (unsigned b = 0; b < 3; ++b) m |= (unsigned)(__builtin_popcount(((A >> (4 * b)) & 15u) & r) & 1) << b;
      return r * 128 + ((c ^ m) << 4);
    });

  for (const Pattern& p : pats)
    for (unsigned a : p.addr)
      if (a + p.bytes > kSpan || a % p.bytes) {
        fprintf(stderr, "address %u out of range in %s\n", a, p.name.c_str());
        return 3;
      }
  unsigned* d_addr;
  int* out;
  if (hipMalloc(&d_addr, 64 * sizeof(unsigned)) || hipMalloc(&out, 256 * 256 * sizeof(int))) return 1;
  for (size_t i = 0; i < pats.size(); ++i) {
    const Pattern& p = pats[i];
    if (hipMemcpy(d_addr, p.addr.data(), 64 * sizeof(unsigned), hipMemcpyHostToDevice)) return 1;
    if (p.write && p.bytes == 16) hipLaunchKernelGGL((lds_probe<16, true>), dim3(256), dim3(256), 0, 0, d_addr, out, 2048);
    else if (p.write) hipLaunchKernelGGL((lds_probe<8, true>), dim3(256), dim3(256), 0, 0, d_addr, out, 2048);
    else if (p.bytes == 16) hipLaunchKernelGGL((lds_probe<16, false>), dim3(256), dim3(256), 0, 0, d_addr, out, 2048);
    else if (p.bytes == 8) hipLaunchKernelGGL((lds_probe<8, false>), dim3(256), dim3(256), 0, 0, d_addr, out, 2048);
    else hipLaunchKernelGGL((lds_probe<4, false>), dim3(256), dim3(256), 0, 0, d_addr, out, 2048);
    if (hipDeviceSynchronize() != hipSuccess) return 2;
    printf("pattern %zu %u %c %s :", i, p.bytes, p.write ? 'w' : 'r', p.name.c_str());
    for (unsigned a : p.addr) printf(" %u", a);
    printf("\n");
  }
  return 0;
}
