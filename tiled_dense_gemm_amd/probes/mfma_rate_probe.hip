// MFMA throughput probe for gfx950: register operands only, no memory in
// the loop, one workgroup per CU (an LDS reservation keeps it so). Each wave
// works like a GEMM main loop on a 128x64 (8 waves, two per SIMD) or
// 128x128 (4 waves, one per SIMD) tile of accumulators, with operand
// fragments that change from one MFMA to the next (two sets, alternated),
// as GEMM data does (one random set, walked forward then backward so that
// consecutive MFMAs take different operands); "constant" rows feed the same
// fragment to every MFMA.
// Reports TFLOP/s and the shader clock during the loop (s_memtime against
// the 100 MHz s_memrealtime): the ceiling a GEMM main loop can reach, and
// how much the data toggling of an instruction shape costs in clock.
//
// Build: hipcc --offload-arch=gfx950 -O3 -std=c++17 -Xclang -target-feature
//        -Xclang -packed-fp32-ops mfma_rate_probe.hip -o mfma_rate_probe
#include <hip/hip_runtime.h>
#include <cstdio>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ unsigned hsh(unsigned x) { x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16; return x; }
__device__ __bf16 rbf(unsigned h) {  // random bf16, magnitude about [2^-7, 2)
  const unsigned short b = (unsigned short)(((h & 1) << 15) | ((120 + (h >> 1) % 8) << 7) | ((h >> 4) & 0x7F));
  return __builtin_bit_cast(__bf16, b);
}
__device__ int rf8(unsigned h) {  // four random OCP e4m3 codes, no NaN
  int r = 0;
  for (int i = 0; i < 4; ++i) { unsigned c = (h >> (8 * i)) & 0xFF; if ((c & 0x7F) == 0x7F) c ^= 1; r |= (int)(c << (8 * i)); }
  return r;
}

// KIND: 0 bf16 32x32x16, 1 bf16 16x16x32, 2 fp8 32x32x64, 3 fp8 16x16x128,
// 4 fp8 32x32x64 with E8M0 block scales, 5 fp4 32x32x64 with scales,
// 6 fp4 16x16x128 with scales.
// TOGGLE: 1 = two fragment sets alternated; 0 = one set.
template <int KIND, int WAVES, int TOGGLE>
__global__ __launch_bounds__(64 * WAVES) void mfma_loop(float* out, long long* clk, int iters) {
  constexpr bool MI32 = (KIND == 0 || KIND == 2 || KIND == 4 || KIND == 5);
  constexpr bool FP8 = (KIND >= 2);
  constexpr int FM = MI32 ? 4 : 8;
  constexpr int FN = (MI32 ? 2 : 4) * (WAVES == 8 ? 1 : 2);
  using Acc = typename std::conditional<MI32, f32x16, f32x4>::type;
  using Frag = typename std::conditional<FP8, i32x8, bf16x8>::type;
  const unsigned l = threadIdx.x;
  const unsigned seed = blockIdx.x * 4096u + l * 64u;
  Frag a[FM], b[FN];
  for (int i = 0; i < FM; ++i)
    for (int e = 0; e < 8; ++e) {
      const unsigned h = hsh(seed + (TOGGLE ? i : 0) * 31u + e);
      if constexpr (FP8) a[i][e] = rf8(h); else a[i][e] = rbf(h);
    }
  for (int j = 0; j < FN; ++j)
    for (int e = 0; e < 8; ++e) {
      const unsigned h = hsh(seed + 50000u + (TOGGLE ? j : 0) * 31u + e);
      if constexpr (FP8) b[j][e] = rf8(h); else b[j][e] = rbf(h);
    }
  Acc acc[FM][FN];
  for (int i = 0; i < FM; ++i) for (int j = 0; j < FN; ++j) acc[i][j] = Acc{};
  const int scl = 120 + (int)(hsh(seed) % 8);   // E8M0 scale words of the scaled kinds
  const long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const Frag& x = b[c ? FN - 1 - j : j];
          const Frag& y = a[c ? FM - 1 - i : i];
          if constexpr (KIND == 0) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc[i][j], 0, 0, 0);
          else if constexpr (KIND == 1) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc[i][j], 0, 0, 0);
          else if constexpr (KIND == 2) acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, acc[i][j], 0, 0, 0, 0, 0, 0);
          else if constexpr (KIND == 3) acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, acc[i][j], 0, 0, 0, 0, 0, 0);
          else if constexpr (KIND == 4) acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, acc[i][j], 0, 0, 0, scl + i, 0, scl + j);
          else if constexpr (KIND == 5) acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, acc[i][j], 4, 4, 0, scl + i, 0, scl + j);
          else acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, acc[i][j], 4, 4, 0, scl + i, 0, scl + j);
        }
  const long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0;
  for (int i = 0; i < FM; ++i) for (int j = 0; j < FN; ++j) for (int e = 0; e < (MI32 ? 16 : 4); ++e) s += acc[i][j][e];
  out[blockIdx.x * 512 + l] = s;
  if (l == 0) { clk[blockIdx.x * 2] = t1 - t0; clk[blockIdx.x * 2 + 1] = r1 - r0; }
}

template <int KIND, int WAVES, int TOGGLE>
void run(const char* name, float* out, long long* clk, bool print) {
  const int iters = 4000, grid = 256;
  const size_t lds = 96 * 1024;  // one workgroup per CU
  constexpr bool MI32 = (KIND == 0 || KIND == 2 || KIND == 4 || KIND == 5);
  const double kdepth = (KIND == 0) ? 16 : (KIND == 1) ? 32 : (KIND == 2 || KIND == 4 || KIND == 5) ? 64 : 128;
  const double fm = MI32 ? 4 : 8, fn = (MI32 ? 2 : 4) * (WAVES == 8 ? 1 : 2), blk = MI32 ? 32 : 16;
  const double flop_per_iter_wave = 2.0 * 2 * fm * fn * blk * blk * kdepth;
  if (hipFuncSetAttribute((const void*)mfma_loop<KIND, WAVES, TOGGLE>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) return;
  hipEvent_t e0, e1; hipEventCreate(&e0); hipEventCreate(&e1);
  hipLaunchKernelGGL((mfma_loop<KIND, WAVES, TOGGLE>), dim3(grid), dim3(64 * WAVES), lds, 0, out, clk, iters);
  hipEventRecord(e0);
  hipLaunchKernelGGL((mfma_loop<KIND, WAVES, TOGGLE>), dim3(grid), dim3(64 * WAVES), lds, 0, out, clk, iters);
  hipEventRecord(e1); hipEventSynchronize(e1);
  float ms; hipEventElapsedTime(&ms, e0, e1);
  long long h[2]; hipMemcpy(h, clk, 16, hipMemcpyDeviceToHost);
  const double flops = (double)grid * WAVES * iters * flop_per_iter_wave;
  const double ghz = (double)h[0] / ((double)h[1] / 100e6) / 1e9;
  if (print)
    printf("| %s | %d | %s | %.1f | %.2f |\n", name, WAVES / 4, TOGGLE ? "toggling" : "constant", flops / ms / 1e9, ghz);
}

int main() {
  float* out; long long* clk;
  if (hipMalloc(&out, 256 * 512 * 4) || hipMalloc(&clk, 256 * 16)) return 1;
  // the whole list twice; the first pass warms the chip up and is not printed
  for (int pass = 0; pass < 2; ++pass) {
    const bool p = pass == 1;
    if (p) printf("| instruction | waves/SIMD | operands | TFLOP/s | shader clock (GHz) |\n|---|---|---|---|---|\n");
    run<0, 8, 1>("bf16 32x32x16", out, clk, p);
    run<1, 8, 1>("bf16 16x16x32", out, clk, p);
    run<0, 8, 0>("bf16 32x32x16", out, clk, p);
    run<1, 8, 0>("bf16 16x16x32", out, clk, p);
    run<0, 4, 1>("bf16 32x32x16", out, clk, p);
    run<2, 8, 1>("fp8 32x32x64", out, clk, p);
    run<3, 8, 1>("fp8 16x16x128", out, clk, p);
    run<2, 4, 1>("fp8 32x32x64", out, clk, p);
    run<3, 4, 1>("fp8 16x16x128", out, clk, p);
    run<2, 8, 0>("fp8 32x32x64", out, clk, p);
    run<3, 8, 0>("fp8 16x16x128", out, clk, p);
    run<4, 4, 1>("fp8 32x32x64, E8M0 scales", out, clk, p);
    run<5, 4, 1>("fp4 32x32x64, E8M0 scales", out, clk, p);
    run<6, 4, 1>("fp4 16x16x128, E8M0 scales", out, clk, p);
    run<5, 8, 1>("fp4 32x32x64, E8M0 scales", out, clk, p);
    run<6, 8, 1>("fp4 16x16x128, E8M0 scales", out, clk, p);
  }
  if (hipDeviceSynchronize() != hipSuccess) return 2;
  return 0;
}
