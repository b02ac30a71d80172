/*
 * Reference GEMM for the oracle -- TEST INFRASTRUCTURE, not the product.
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark load this library. The GPU path shares no code with it.
 *
 * Computes the plain definition of the tiled dense product
 *     C[i][j] = scale * sum_{k=0}^{K-1} A[i][k] * B[k][j]
 * in IEEE double precision, with A an M x K row-major array and B given in
 * column-major order, i.e. as an N x K array Bt with Bt[j][k] = B[k][j].
 * (Page "ThunderKittens: Simple, Fast, and Adorable AI Kernels", section 3.4
 * "Integration: How the Three Levels Compose into a Complete Kernel" defines
 * C = A x B with A of size M x K and B of size K x N; page "ThunderKittens:
 * 16x16 Tiles, the Load-Compute-Store-Finish Template ...", section "Warp
 * level: tiles are the only data structure", fixes A row-major and B
 * column-major for mma_AB.)
 *
 * The sum over k runs in order k = 0, 1, ..., K-1 for every output element;
 * the scale is applied once, after the sum. There is no blocking and no
 * reordering: rows of C are only distributed over OpenMP threads, which does
 * not change any element's arithmetic.
 */
#include <stdint.h>

void ref_gemm_f64(int64_t M, int64_t N, int64_t K, const double *A,
                  const double *Bt, double scale, double *C) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < M; ++i) {
    const double *a = A + i * K;
    for (int64_t j = 0; j < N; ++j) {
      const double *b = Bt + j * K;
      double s = 0.0;
      for (int64_t k = 0; k < K; ++k)
        s += a[k] * b[k];
      C[i * N + j] = scale * s;
    }
  }
}

/* Number of threads the parallel loop above uses (for reporting). */
int ref_gemm_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp master
    {
#ifdef _OPENMP
      extern int omp_get_num_threads(void);
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}
