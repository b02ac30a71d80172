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
//   * the 4-bit kernel's 8-byte block-scale reads;
//   * a search over all 4096 linear row swizzles of 128-byte rows,
//     chunk ^ A*bits(row mod 16), read with the 16x16 fragment pattern.
// It prints one line per dispatch, in order: "pattern <id> <bytes> <name>
// : <64 addresses>", which lds_probe_summary.py joins with the counters.
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

template <int BYTES>
__global__ __launch_bounds__(256) void lds_probe(const unsigned* addrs, int* out, int iters) {
  __shared__ __attribute__((aligned(16))) int smem[2 * kSpan / 4];
  for (unsigned i = threadIdx.x; i < 2 * kSpan / 4; i += 256) smem[i] = (int)(i * 7 + 1);
  __syncthreads();
  const unsigned lane = threadIdx.x & 63;
  const unsigned a = addrs[lane];
  const LDS_AS char* base = (const LDS_AS char*)smem;
  int acc = 0;
  for (int it = 0; it < iters; ++it) {
    const unsigned off = a + ((it & 1) ? kSpan : 0);
    if constexpr (BYTES == 16) {
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
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

struct Pattern {
  std::string name;
  unsigned bytes;
  std::vector<unsigned> addr;
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
  // the kernels' fragment reads, swizzled and not
  for (bool on : {true, false}) {
    for (unsigned s = 0; s < 2; ++s)
      for (unsigned f = 0; f < 16; ++f) pats.push_back(fragment("bf16 16x16x32", 128, 16, 4, s, 0, f, on));
    for (unsigned s = 0; s < 2; ++s)
      for (unsigned q = 0; q < 2; ++q)
        for (unsigned f = 0; f < 8; ++f) pats.push_back(fragment("fp8 32x32x64", 128, 32, 4, s, q, f, on));
    for (unsigned s = 0; s < 2; ++s)
      for (unsigned f = 0; f < 8; ++f) pats.push_back(fragment("4-bit values", 64, 32, 2, s, 0, f, on));
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
    if (p.bytes == 16) hipLaunchKernelGGL(lds_probe<16>, dim3(256), dim3(256), 0, 0, d_addr, out, 2048);
    else if (p.bytes == 8) hipLaunchKernelGGL(lds_probe<8>, dim3(256), dim3(256), 0, 0, d_addr, out, 2048);
    else hipLaunchKernelGGL(lds_probe<4>, dim3(256), dim3(256), 0, 0, d_addr, out, 2048);
    if (hipDeviceSynchronize() != hipSuccess) return 2;
    printf("pattern %zu %u %s :", i, p.bytes, p.name.c_str());
    for (unsigned a : p.addr) printf(" %u", a);
    printf("\n");
  }
  return 0;
}
