// LDS bank-geometry probe for gfx950: one kernel per address pattern, each
// lane reading in-bounds LDS addresses (< 16 KiB) repeatedly. Counted per
// dispatch with rocprofv3 (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE), the
// patterns show which lane bits share a phase for b128 / b64 / b32 reads and
// how addresses map to banks; the results calibrate lds_bank_model.py.
//
// Build: hipcc --offload-arch=gfx950 -O2 -std=c++17 lds_bank_probe.hip -o lds_bank_probe
#include <hip/hip_runtime.h>
#include <cstdio>
#define LDS_AS __attribute__((address_space(3)))
typedef int i4 __attribute__((ext_vector_type(4)));
typedef int i2 __attribute__((ext_vector_type(2)));

__host__ __device__ constexpr unsigned swz128(unsigned r, unsigned c) { return r * 128 + ((c ^ ((r & 7) ^ ((r >> 3) & 1))) << 4); }
__host__ __device__ constexpr unsigned swz64(unsigned r, unsigned c) { return r * 64 + ((c ^ (((r >> 1) ^ (r >> 3)) & 3)) << 4); }

template <int P> __device__ unsigned addr(unsigned l) {
  // P: 0 contig b128; 1..6 T_d b128 (d=1<<(P-1)); 7 dense swz; 8 dense unswz; 9 fp4v swz; 10 fp4v unswz
  //    20 contig b64; 21..26 T_d b64; 27 fp4 scale (8*(l%32))
  //    40 contig b32; 41..46 T_d b32
  if (P == 0) return 16 * l;
  if (P >= 1 && P <= 6) { unsigned d = 1u << (P - 1); return 16 * (l & ~d) + ((l & d) ? 4096 : 0); }
  if (P == 7) return swz128(l % 32, l / 32);
  if (P == 8) return (l % 32) * 128 + 16 * (l / 32);
  if (P == 9) return swz64(l % 32, l / 32);
  if (P == 10) return (l % 32) * 64 + 16 * (l / 32);
  if (P == 11) return swz64(l % 32, 2 + l / 32);
  if (P == 20) return 8 * l;
  if (P >= 21 && P <= 26) { unsigned d = 1u << (P - 21); return 8 * (l & ~d) + ((l & d) ? 4096 : 0); }
  if (P == 27) return 8 * (l % 32);
  if (P == 40) return 4 * l;
  if (P >= 41 && P <= 46) { unsigned d = 1u << (P - 41); return 4 * (l & ~d) + ((l & d) ? 4096 : 0); }
  return 0;
}
template <int P> constexpr int width() { return P < 20 ? 16 : (P < 40 ? 8 : 4); }

template <int P>
__global__ __launch_bounds__(256) void lds_probe(int* out, int iters) {
  __shared__ __attribute__((aligned(16))) int smem[4096];  // 16 KiB
  for (int i = threadIdx.x; i < 4096; i += 256) smem[i] = i * 7 + 1;
  __syncthreads();
  const unsigned lane = threadIdx.x & 63;
  const unsigned a = addr<P>(lane);          // < 4096 + 1024 bytes
  const LDS_AS char* base = (const LDS_AS char*)smem;
  int acc = 0;
  for (int it = 0; it < iters; ++it) {
    const unsigned off = a + ((it & 1) ? 8192 : 0);   // stay < 16 KiB
    if constexpr (width<P>() == 16) { i4 v = *(const LDS_AS i4*)(base + off); acc ^= v[0] ^ v[1] ^ v[2] ^ v[3]; }
    else if constexpr (width<P>() == 8) { i2 v = *(const LDS_AS i2*)(base + off); acc ^= v[0] ^ v[1]; }
    else { acc ^= *(const LDS_AS int*)(base + off); }
    __builtin_amdgcn_sched_barrier(0);
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

template <int P> void run(int* out) {
  hipLaunchKernelGGL(lds_probe<P>, dim3(256), dim3(256), 0, 0, out, 4096);
}
int main() {
  int* out; if (hipMalloc(&out, 256 * 256 * 4) != hipSuccess) return 1;
  // max address: 4096 + 1024 + 8192 < 16384 for every pattern
  run<0>(out); run<1>(out); run<2>(out); run<3>(out); run<4>(out); run<5>(out); run<6>(out);
  run<7>(out); run<8>(out); run<9>(out); run<10>(out); run<11>(out);
  run<20>(out); run<21>(out); run<22>(out); run<23>(out); run<24>(out); run<25>(out); run<26>(out); run<27>(out);
  run<40>(out); run<41>(out); run<42>(out); run<43>(out); run<44>(out); run<45>(out); run<46>(out);
  if (hipDeviceSynchronize() != hipSuccess) return 2;
  printf("lds probe done\n");
  return 0;
}
