// MFMA issue-rate probe for gfx950: register operands only, no memory in
// the loop. Reports TFLOP/s, the shader clock during the loop (s_memtime
// against the 100 MHz s_memrealtime) and cycles per MFMA per wave, for one
// and two waves per SIMD: the ceiling a GEMM main loop can reach.
//
// Build: hipcc --offload-arch=gfx950 -O3 -std=c++17 -Xclang -target-feature
//        -Xclang -packed-fp32-ops mfma_rate_probe.hip -o mfma_rate_probe
#include <hip/hip_runtime.h>
#include <cstdio>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int KIND, int NACC, int THREADS>
__global__ __launch_bounds__(THREADS) void mfma_loop(float* out, long long* clk, int iters) {
  const int l = threadIdx.x;
  bf16x8 a, b; i32x8 fa, fb;
  for (int i = 0; i < 8; ++i) { a[i] = (__bf16)(0.001f * (l + i)); b[i] = (__bf16)(0.002f * (l - i)); fa[i] = l * 3 + i; fb[i] = l * 5 - i; }
  long long t0 = __builtin_amdgcn_s_memtime();
  long long r0 = __builtin_amdgcn_s_memrealtime();
  if constexpr (KIND == 0 || KIND == 2) {
    f32x16 acc[NACC];
    for (int j = 0; j < NACC; ++j) acc[j] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < NACC; ++j) {
        if constexpr (KIND == 0) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
        else acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc[j], 0, 0, 0, 0, 0, 0);
      }
    }
    float s = 0; for (int j = 0; j < NACC; ++j) for (int e = 0; e < 16; ++e) s += acc[j][e];
    out[blockIdx.x * 512 + l] = s;
  } else {
    f32x4 acc[NACC];
    for (int j = 0; j < NACC; ++j) acc[j] = f32x4{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < NACC; ++j) {
        if constexpr (KIND == 1) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
        else acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb, acc[j], 0, 0, 0, 0, 0, 0);
      }
    }
    float s = 0; for (int j = 0; j < NACC; ++j) for (int e = 0; e < 4; ++e) s += acc[j][e];
    out[blockIdx.x * 512 + l] = s;
  }
  long long t1 = __builtin_amdgcn_s_memtime();
  long long r1 = __builtin_amdgcn_s_memrealtime();
  if (l == 0) { clk[blockIdx.x * 2] = t1 - t0; clk[blockIdx.x * 2 + 1] = r1 - r0; }
}

template <int KIND, int NACC, int THREADS>
void run(const char* name, int threads, float* out, long long* clk, double flop_per_mfma) {
  const int iters = 2000, grid = 256;
  hipEvent_t e0, e1; hipEventCreate(&e0); hipEventCreate(&e1);
  hipLaunchKernelGGL((mfma_loop<KIND, NACC, THREADS>), dim3(grid), dim3(THREADS), 0, 0, out, clk, iters);
  hipEventRecord(e0);
  hipLaunchKernelGGL((mfma_loop<KIND, NACC, THREADS>), dim3(grid), dim3(THREADS), 0, 0, out, clk, iters);
  hipEventRecord(e1); hipEventSynchronize(e1);
  float ms; hipEventElapsedTime(&ms, e0, e1);
  long long h[2]; hipMemcpy(h, clk, 16, hipMemcpyDeviceToHost);
  double flops = (double)grid * (threads / 64) * iters * NACC * flop_per_mfma;
  double ghz = (double)h[0] / ((double)h[1] / 100e6) / 1e9;   // memrealtime = 100 MHz
  printf("%-34s waves/WG=%d  %.3f ms  %8.1f TF  shader-clock %.2f GHz  cycles/mfma/wave=%.1f\n", name, threads / 64, ms,
         flops / ms / 1e9, ghz, (double)h[0] / (iters * NACC));
}
int main() {
  float* out; long long* clk;
  if (hipMalloc(&out, 256 * 512 * 4) || hipMalloc(&clk, 256 * 16)) return 1;
  run<0, 16, 256>("bf16 32x32x16, 16 acc", 256, out, clk, 32768);
  run<0, 8, 512>("bf16 32x32x16, 8 acc", 512, out, clk, 32768);
  run<0, 4, 256>("bf16 32x32x16, 4 acc", 256, out, clk, 32768);
  run<1, 16, 256>("bf16 16x16x32, 16 acc", 256, out, clk, 16384);
  run<1, 16, 512>("bf16 16x16x32, 16 acc (2 waves/SIMD)", 512, out, clk, 16384);
  run<2, 16, 256>("fp8 32x32x64, 16 acc", 256, out, clk, 131072);
  run<2, 8, 512>("fp8 32x32x64, 8 acc (2 waves/SIMD)", 512, out, clk, 131072);
  run<3, 16, 256>("fp8 16x16x128, 16 acc", 256, out, clk, 65536);
  if (hipDeviceSynchronize() != hipSuccess) return 2;
  return 0;
}
