/*
 * tkg -- tiled dense GEMM for AMD MI355X (gfx950): the C ABI.
 *
 * Every entry point computes one matrix product
 *
 *     C = s * A * B          (A: M x K, B: K x N, C: M x N)
 *
 * with fp32 accumulation on the matrix cores and a bf16 result, as defined
 * on page "ThunderKittens: Simple, Fast, and Adorable AI Kernels", section
 * 3.4, "Integration: How the Three Levels Compose into a Complete Kernel"
 * (C = A x B, A is M x K, B is K x N), with A row-major and B column-major
 * as the tensor-core layout rule of page "ThunderKittens: 16x16 Tiles, the
 * Load-Compute-Store-Finish Template, and Why 40 Lines Can Match cuBLAS",
 * section "Warp level: tiles are the only data structure", requires.
 *
 * Common conventions
 * ------------------
 * - All matrix pointers are DEVICE pointers owned by the caller; the
 *   library never allocates, frees or keeps them.
 * - A is row-major M x K (leading dimension K). B is column-major K x N,
 *   i.e. stored as an N x K row-major array (leading dimension K): both
 *   operands are contiguous along K. C is row-major M x N bf16 (leading
 *   dimension N) and is overwritten.
 * - Every matrix pointer must be 16-byte aligned.
 * - `stream` is a hipStream_t (NULL = the default stream). The call only
 *   enqueues work and returns; the product is complete when the stream
 *   reaches that point. Calls on one stream run in order; separate calls may
 *   run concurrently on different streams as long as their C do not overlap.
 * - The bf16 result is round-to-nearest-even of the fp32 accumulator times
 *   the scale. The summation order over K is unspecified.
 * - M == 0 or N == 0 is an empty product: nothing is launched, TKG_OK is
 *   returned and no pointer is read. K == 0 writes zeros to C.
 * - Return value: TKG_OK (0) once the kernel is enqueued, or a negative
 *   tkg_status. On any error nothing is enqueued and C is untouched.
 *   tkg_status_string() names every status.
 * - The library holds no mutable state besides per-device caches of the
 *   compute-unit count and of the address of the allocation-free entry
 *   point's scratch array (tkg_gemm_splitk_noalloc, whose calls on one GPU
 *   share that array); all entry points are thread-safe.
 */
#ifndef TKG_H
#define TKG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tkg_status {
  TKG_OK = 0,
  TKG_ERR_NULL = -1,   /* a required pointer is NULL                        */
  TKG_ERR_SHAPE = -2,  /* negative size, unsupported multiple or too large  */
  TKG_ERR_ALIGN = -3,  /* a matrix pointer is not 16-byte aligned           */
  TKG_ERR_LAUNCH = -4, /* the HIP runtime rejected the launch               */
  TKG_ERR_DEVICE = -5, /* no usable HIP device / device query failed        */
  TKG_ERR_WORKSPACE = -6, /* split-K workspace NULL or smaller than required */
  TKG_ERR_VALUE = -7   /* a scalar argument is out of range                 */
} tkg_status;

/*
 * bf16 x bf16 -> bf16, s = 1.
 *   A: M x K bf16, B: N x K bf16 (B column-major), C: M x N bf16.
 *   Requires K % 8 == 0 (16-byte rows) and K <= 4194303.
 * The operand type and fp32 accumulation: page "ThunderKittens: Simple,
 * Fast, and Adorable AI Kernels", section 3.4, "Warp-Level: Tile
 * Operations".
 */
int gemm_bf16(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
              void *C, void *stream);

/*
 * fp8 x fp8 -> bf16 with per-tensor scales, s = scale_a * scale_b.
 *   A: M x K bytes, B: N x K bytes, both OCP FP8 e4m3 (largest finite 448;
 *   0x7F/0xFF are NaN). scale_a, scale_b: fp32 dequantization scales, so
 *   A_real = scale_a * A and B_real = scale_b * B. Their product is formed
 *   in fp32 and multiplies the fp32 accumulator before rounding to bf16.
 *   Requires K % 16 == 0 and K <= 8388607.
 * FP8 operands: page "ThunderKittens reaches 22.4 PFLOPS on NVIDIA Rubin"
 * (FP8 GEMM); the 16 x 32 fp8 base tile: page "ThunderKittens DSL for GPU
 * kernels" (tile abstractions).
 */
int gemm_fp8(int64_t M, int64_t N, int64_t K, const void *A, float scale_a,
             const void *B, float scale_b, void *C, void *stream);

/*
 * Block-scaled 4-bit x block-scaled 4-bit -> bf16, s = a_scale * b_scale.
 *   A: M x K/2 bytes of packed e2m1 values, element 2t of a row in the LOW
 *      nibble of byte t (sign bit 3, 2 exponent bits with bias 1, 1 mantissa
 *      bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).
 *   A_scales: M x K/16 bytes, OCP e4m3 scale of each block of 16 consecutive
 *      K-elements of a row.
 *   a_scale: fp32 per-tensor scale. A_real[i][k] =
 *      a_scale * e4m3(A_scales[i][k/16]) * e2m1(A[i][k]).
 *   B, B_scales, b_scale: the same for B in column-major order (N x K/2
 *      values, N x K/16 scales).
 *   Each e2m1 value times its block scale is exact in fp16 (at most 6
 *   significant bits, magnitude within [2^-10, 2688]), so the product runs
 *   on the fp16 matrix cores with fp32 accumulation and no rounding of the
 *   operands; a_scale * b_scale (fp32) multiplies the accumulator before
 *   rounding to bf16.
 *   Requires K % 64 == 0 and K <= 16777215. All five pointers 16-byte
 *   aligned.
 * The block-scaled 4-bit format with scale factors kept next to the
 * values: page "ThunderKittens reaches 22.4 PFLOPS on NVIDIA Rubin",
 * sections "Rubin widens the data path" and "Feeding the faster tensor
 * cores".
 */
int gemm_fp4_blockscaled(int64_t M, int64_t N, int64_t K, const void *A,
                         const void *A_scales, float a_scale, const void *B,
                         const void *B_scales, float b_scale, void *C,
                         void *stream);

/*
 * MX block-scaled operands -> bf16 (OCP Microscaling formats, the form of
 * block scaling gfx950's matrix cores execute natively; an external
 * specification, not the pages').
 *   gemm_mxfp4: A is M x K/2 bytes of packed e2m1 values (element 2t of a
 *      row in the LOW nibble of byte t, as gemm_fp4_blockscaled).
 *   gemm_mxfp8: A is M x K bytes of OCP e4m3 values.
 *   A_scales: M x K/32 bytes, the E8M0 scale of each block of 32 consecutive
 *      K-elements of a row: A_real[i][k] = 2^(A_scales[i][k/32] - 127) *
 *      elem(A[i][k]) (0xFF encodes NaN).
 *   B, B_scales: the same for B in column-major order (N x K/2 or N x K
 *      values, N x K/32 scales).
 *   The matrix cores apply the scales inside the MFMA; fp32 accumulation,
 *   bf16 result. Requires K % 128 == 0 (K <= 16777088 for MXFP4, 8388480
 *   for MXFP8). All five pointers 16-byte aligned.
 * Block scaling factors that travel with low-precision values: page
 * "ThunderKittens reaches 22.4 PFLOPS on NVIDIA Rubin", section "Feeding
 * the faster tensor cores".
 */
int gemm_mxfp4(int64_t M, int64_t N, int64_t K, const void *A,
               const void *A_scales, const void *B, const void *B_scales,
               void *C, void *stream);
int gemm_mxfp8(int64_t M, int64_t N, int64_t K, const void *A,
               const void *A_scales, const void *B, const void *B_scales,
               void *C, void *stream);

/*
 * Split-K bf16 / fp8 product for shapes with few output tiles and long K
 * (small M x N), as C = s * A * B above (dtype TKG_DTYPE_BF16, s = 1, the
 * scales ignored; or TKG_DTYPE_FP8, s = a_scale * b_scale; same operand
 * layouts, alignment and K rules as gemm_bf16 / gemm_fp8). K is cut into
 * `splits` ranges of whole stages (0 = automatic: enough (tile, range)
 * work units for every workgroup slot of the device, each range at least
 * 32 stages long; at most 64); each
 * work unit computes its tile's partial sum over its range in fp32 into
 * `workspace`, and a second kernel adds the partials of each output
 * element in range order, multiplies by s and rounds to bf16. The result
 * equals the plain product up to fp32 summation order. When the plan has
 * one range the plain product runs and the workspace is not used.
 *   workspace -- device memory owned by the caller, 16-byte aligned, at
 *               least tkg_gemm_splitk_workspace_size(...) bytes, not
 *               shared with a concurrent call; its contents are scratch.
 * Returns TKG_ERR_WORKSPACE if the workspace is NULL or too small (when
 * one is needed), else the errors of gemm_bf16 / gemm_fp8. Splitting the
 * reduction over K is the stream-K / split-K reading of page
 * "ThunderKittens: Simple, Fast, and Adorable AI Kernels", section 3.4,
 * "Persistent Grid Launch" (Table 2: setup-bound products with short work
 * per tile).
 */
int tkg_gemm_splitk(int dtype, int64_t M, int64_t N, int64_t K, const void *A,
                    float a_scale, const void *B, float b_scale, void *C,
                    void *workspace, size_t workspace_bytes, int splits,
                    void *stream);
/*
 * The split-K product of tkg_gemm_splitk without a caller workspace and
 * without any allocation: for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). The fp32 partial sums go to a scratch array of
 * TKG_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds in device
 * memory on each device it runs on, for the life of the process; the call
 * itself allocates and frees nothing. Same arguments, results and errors
 * as tkg_gemm_splitk, except: TKG_ERR_WORKSPACE when the plan needs more
 * than TKG_NOALLOC_SCRATCH_BYTES (tkg_gemm_splitk_workspace_size() gives
 * the need; fewer splits need less), nothing launched; TKG_ERR_DEVICE if
 * the scratch address cannot be resolved. Calls on one device share the
 * scratch: calls that overlap in time on one device (different streams
 * without ordering between them) race and give wrong results; calls on one
 * stream are ordered and safe. The caller passes A, B and C.
 */
#define TKG_NOALLOC_SCRATCH_BYTES (32u << 20)
int tkg_gemm_splitk_noalloc(int dtype, int64_t M, int64_t N, int64_t K,
                            const void *A, float a_scale, const void *B,
                            float b_scale, void *C, int splits, void *stream);

/* Bytes of workspace tkg_gemm_splitk needs for these arguments (0 when it
 * runs the plain product), or a negative tkg_status. */
int64_t tkg_gemm_splitk_workspace_size(int dtype, int64_t M, int64_t N,
                                       int64_t K, int splits);
/* The number of K ranges tkg_gemm_splitk uses for these arguments, or a
 * negative tkg_status. */
int tkg_gemm_splitk_count(int dtype, int64_t M, int64_t N, int64_t K,
                          int splits);

/*
 * Softmax attention forward, bf16 in and out, fp32 accumulation:
 *   O[b, h, i, :] = sum_j softmax_j(scale * Q[b, h, i, :] . K[b, g, j, :]) V[b, g, j, :]
 *   lse[b, h, i]  = log sum_j exp(scale * Q[b, h, i, :] . K[b, g, j, :])
 * with g = h / (Hq / Hkv) (grouped-query attention; Hkv = Hq is plain
 * multi-head attention) and, if `causal`, j <= i only. The operation and
 * its steps are those of page "ThunderKittens: Simple, Fast, and Adorable
 * AI Kernels", section 3, "PyTorch-Like Operations on Tiles" (Q K^T, row
 * max, exp, row sum, P V, online rescaling) and "The LCSF Template" (the
 * finish divides by the normalisation constant); its variants (causal,
 * non-causal, grouped-query, head dimension 64 or 128) are those of the
 * same page's section 5, "Attention: Matching FA3 on Forward,
 * Outperforming on Backward".
 *   Q:   [B, Hq, Nq, D] bf16, row-major (D contiguous), device memory.
 *   K,V: [B, Hkv, Nk, D] bf16, row-major, device memory.
 *   O:   [B, Hq, Nq, D] bf16, written; must not overlap the inputs.
 *   lse: [B, Hq, Nq] fp32 (natural log), written; may be NULL (not stored).
 *   D is 64 or 128; Hq % Hkv == 0; causal requires Nq == Nk; Nq * 2D and
 *   Nk * 2D below 2^31 bytes (one head's rows); scale finite and > 0
 *   (1/sqrt(D) is the usual choice). The caller owns every buffer; the
 *   call allocates nothing and is asynchronous on `stream` (a hipStream_t,
 *   NULL = default stream).
 * Accuracy: scores are fp32 sums of exact bf16 products; each probability
 * is rounded to bf16 before the P V product, and the row sum adds those
 * same rounded values (in fp32 over windows of 2048 keys, totalled in
 * fp64), so numerator and denominator use the same weights; O is rounded
 * once to bf16.
 * Returns TKG_OK (nothing launched when B, Hq or Nq is 0), TKG_ERR_SHAPE
 * (unsupported D, negative or inconsistent sizes, Nk = 0 with queries, or
 * too large), TKG_ERR_VALUE (scale), TKG_ERR_NULL (Q, K, V or O NULL),
 * TKG_ERR_ALIGN (Q, K, V, O not 16-byte aligned or lse not 4-byte aligned),
 * TKG_ERR_LAUNCH.
 */
int tkg_attention_fwd(const void *Q, const void *K, const void *V, void *O,
                      float *lse, int64_t B, int64_t Hq, int64_t Hkv,
                      int64_t Nq, int64_t Nk, int64_t D, float scale,
                      int causal, void *stream);

/*
 * LDS addresses of the attention kernel's key/value ring, for host-side
 * checks of its bank-conflict freedom (no GPU work). Writes 64 values to
 * out64, one per lane of a wave, for head dimension d (64 or 128):
 *   kind 0: byte offset in the K tile (32 keys) of K fragment read
 *           (kb = i0 = 0, ks = i1 < d/16), 16 bytes per lane;
 *   kind 1: byte offset in the V tile of transposing read (kb = i0 = 0,
 *           s = i1 < 2, t = i2 < 2, db = i3 < d/32), 8 bytes per lane;
 *   kind 2, 3: for ring copy piece i0 < d/16 of the K (2) or V (3) tile,
 *           the byte offset, within the key block, of the global 16 bytes
 *           each lane copies (lane l lands at LDS byte 1024 i0 + 16 l).
 * Returns TKG_OK, TKG_ERR_SHAPE or TKG_ERR_NULL.
 */
int tkg_attn_lds_offsets(int d, int kind, int i0, int i1, int i2, int i3,
                         uint32_t *out64);

/* Static, human-readable name of a tkg_status value (never NULL). */
const char *tkg_status_string(int status);

/*
 * Launch options for measurement and ablation. tkg_gemm_ex() runs the same
 * kernels as the three entry points above with these knobs exposed:
 *   grid     -- workgroups to launch; 0 = one per compute unit (persistent),
 *               a value >= the number of output tiles gives one workgroup
 *               per tile (non-persistent).
 *   group_m  -- tile rows per band of the grouped tile order; 1 = plain
 *               row-major tile order; 0 = automatic: 8, except for bf16 and
 *               fp8 products whose A and B together exceed the 256 MB
 *               last-level cache, which take the most rows (up to 32, a
 *               power of two) whose A panels fit in half of it, with the
 *               XCD-block order (xcd_remap 1 becomes 2).
 *   xcd_remap -- 1 (default when grid is a multiple of 8) gives each XCD a
 *               contiguous range of tiles; 0 leaves the hardware's
 *               round-robin order; 2 (XCD blocks) also re-deals each round
 *               of grid tiles that fills a group_m x (grid / group_m)
 *               rectangle so each XCD's tiles form a compact block of it
 *               (split-K launches use 1 instead). Every setting computes
 *               the same bits.
 *   variant  -- bf16/fp8: index of a kernel configuration, 0 .. n-1
 *               with n = tkg_variant_info(dtype, 0, NULL);
 *               tkg_variant_info() describes each (LDS ring shape, waves,
 *               MFMA block, tile, swizzle, schedule). 0 = automatic: the
 *               default configuration, or the 128 x 128 tile
 *               configuration 4 when the product has fewer 256 x 256
 *               output tiles than the device has compute units, or for
 *               bf16 products whose A and B exceed the 256 MB last-level
 *               cache configuration 18 (5-slot ring). The others
 *               are the measured alternatives: bf16 1 = 5-slot ring,
 *               2 = 32x32x16 blocks, 3 = one wave per SIMD, 4 / 5 = 128 x
 *               128 tiles at two / one workgroups per compute unit, 6 =
 *               swizzle off (plain LDS rows), 7 = early release of the B
 *               slab, 8 = ping-pong, 9 = one-stage ring, 10 .. 14 = 64-byte
 *               stages (32x32x16 blocks) in a ring of 1 .. 5 stages,
 *               15 = ping-pong on four 64-byte stages, 16 = one wave per
 *               SIMD with early reads, 17 = the interleaved schedule,
 *               18 = 5-slot ring with early reads, 19 = configuration 4
 *               on the interleaved schedule; fp8 1 = 5-slot
 *               ring, 2 = one wave per SIMD
 *               on 16x16x128 blocks, 3 = one wave per SIMD on 32x32x64,
 *               4 / 5 as bf16, 6 = swizzle off, 7 = early B release,
 *               8 = ping-pong, 9 / 10 = one wave per SIMD on 32x32x64 /
 *               16x16x128 with early reads, 11 = early reads, 12 = 5-slot
 *               ring with early reads, 13 = configuration 4 on the
 *               interleaved schedule. TKG_ERR_SHAPE outside 0 .. n-1.
 *               4-bit product: 0 = 4 waves (default), 1 = 8 waves;
 *               TKG_ERR_SHAPE outside 0..1. Variants that issue the same
 *               MFMA instruction compute the same bits. bf16's 16x16x32
 *               and 32x32x16 blocks also agree bit for bit (16384^3
 *               included). fp8's 16x16x128 configurations (2, 4, 5, 10,
 *               13) round the fp32 accumulation at other points than the
 *               32x32x64 ones once partial sums are inexact: an element
 *               whose sum lies next to a bf16 rounding midpoint can round
 *               to the neighbouring value (at 16384^3, 11 of 2^28 elements
 *               on normal operands scaled by amax/448, each within the
 *               fp8 error bound either way; none up to K = 8192 in the
 *               tests and measurements).
 * Page "ThunderKittens: Simple, Fast, and Adorable AI Kernels", section
 * 3.4, "Persistent Grid Launch" (Table 2) and "Block Launch Order and L2
 * Cache Reuse" (Table 3), measure these choices.
 */
typedef struct tkg_opts {
  int32_t grid;
  int32_t group_m;
  int32_t xcd_remap;
  int32_t variant;
} tkg_opts;

enum {
  TKG_DTYPE_BF16 = 0,
  TKG_DTYPE_FP8 = 1,
  TKG_DTYPE_FP4_BLOCKSCALED = 2,
  TKG_DTYPE_MXFP4 = 3,
  TKG_DTYPE_MXFP8 = 4
};

/*
 * dtype: TKG_DTYPE_*. Arguments that a dtype does not use (A_scales,
 * B_scales for bf16/fp8; the scales for bf16) are ignored. For the MX
 * types a_scale * b_scale multiplies the result (the typed entry points
 * pass 1). opts may be NULL (defaults). The MX types have two kernel
 * configurations: 0 (each fragment re-read after its last MFMA of the
 * k-step) and 1 (early reads), bit-identical. Same contract and errors as
 * the typed entry points.
 */
int tkg_gemm_ex(int dtype, int64_t M, int64_t N, int64_t K, const void *A,
                const void *A_scales, float a_scale, const void *B,
                const void *B_scales, float b_scale, void *C, void *stream,
                const tkg_opts *opts);

/*
 * Description of kernel configuration `variant` of dtype (TKG_DTYPE_BF16,
 * _FP8, _FP4_BLOCKSCALED, or the MX types' two: 0 and 1 = early reads),
 * written to *out when out is not NULL. Returns the number of
 * configurations of the dtype, or a negative tkg_status (TKG_ERR_SHAPE for
 * an unknown dtype or variant). No GPU work.
 */
typedef struct tkg_variant_desc {
  int32_t stage_kbytes; /* K bytes per row of one LDS operand slab            */
  int32_t slots;        /* operand slabs in the LDS ring (2 = one stage)      */
  int32_t waves;        /* waves per workgroup                                */
  int32_t load_waves;   /* waves that issue the global->LDS loads             */
  int32_t mfma_block;   /* 16 (16x16 MFMA blocks) or 32 (32x32)               */
  int32_t tile;         /* workgroup tile edge (tile x tile outputs)          */
  int32_t per_cu;       /* workgroups per compute unit of the default grid    */
  int32_t swizzle;      /* 1 = swizzled LDS rows, 0 = plain rows              */
  int32_t schedule;     /* 0 interleaved, 1 early B release, 2 ping-pong,
                           3 early reads                                      */
} tkg_variant_desc;
int tkg_variant_info(int dtype, int variant, tkg_variant_desc *out);

/*
 * Whether tkg_gemm_ex(dtype, M, N, K, ..., variant) runs the masked kernel
 * instance, whose every global->LDS load carries its whole offset per lane
 * so that the buffer bounds check turns rows past M or N and chunks past K
 * into zeros (1), or the unmasked one, which passes part of each offset as
 * the scalar offset that the bounds check does not cover (0). The unmasked
 * instance runs only when every tile is whole (M and N multiples of the
 * tile edge) and every stage lies inside K. `variant` is the configuration
 * itself (0 = the default one, not resolved by tile count). Returns 1, 0 or
 * a negative tkg_status. No GPU work.
 */
int tkg_launch_masked(int dtype, int64_t M, int64_t N, int64_t K, int variant);

/*
 * The launch tkg_gemm_ex(dtype, M, N, K, ..., opts) makes on a device with
 * `cus` compute units (MI355X: 256), written to *out when out is not NULL:
 * the configuration it runs (variant 0 resolved: 128 x 128 tiles for
 * products with fewer 256 x 256 tiles than compute units, the bf16 5-slot
 * ring for operands beyond the 256 MB last-level cache), its tile edge, the
 * tile count, the grid, and the tile order applied (group_m, xcd_remap; see
 * tkg_opts); and, for whole-tile bf16/fp8 products with automatic variant
 * and grid whose last round of 256 x 256 tiles is partial and small enough
 * that its tiles' 128 x 128 quadrants fit one round of the small-tile
 * configuration (two workgroups per compute unit), the second launch that
 * runs those quadrants (the first launch then runs the full rounds' units
 * only). opts may be NULL (the defaults). An empty product (M or N = 0)
 * reports tiles = grid = units = 0. Returns TKG_OK, or the negative tkg_status that
 * tkg_gemm_ex's shape checks return (TKG_ERR_SHAPE also for cus <= 0).
 * Host logic only, no GPU work; the caller owns *out.
 */
typedef struct tkg_launch_plan {
  int32_t variant;   /* configuration run (tkg_variant_info)               */
  int32_t tile;      /* workgroup tile edge                                */
  int32_t tiles;     /* output tiles                                       */
  int32_t grid;      /* workgroups launched                                */
  int32_t group_m;   /* tile rows per band of the tile order               */
  int32_t xcd_remap; /* 0, 1 or 2 (XCD blocks) as applied                  */
  int32_t units;     /* tiles the first launch runs                        */
  int32_t tail_variant; /* configuration of the second launch, -1: none    */
  int32_t tail_units;   /* 128 x 128 quadrants it runs (0: no second launch) */
  int32_t tail_grid;    /* its workgroups                                  */
} tkg_launch_plan;
int tkg_plan_launch(int dtype, int64_t M, int64_t N, int64_t K, const tkg_opts *opts,
                    int cus, tkg_launch_plan *out);

/*
 * The current HIP device as the launches see it: *cus its compute units
 * (the default persistent grid is built on them; tkg_plan_launch's `cus`)
 * and *peak_clock_khz the peak shader clock the runtime reports, the clock
 * the published dense MFMA peaks assume (under the chip's power limit the
 * kernels run below it). Returns TKG_OK, TKG_ERR_NULL for a null pointer,
 * or TKG_ERR_DEVICE when no usable HIP device is current. Queries the
 * runtime only, launches nothing; the caller owns both outputs.
 */
int tkg_device_info(int32_t *cus, int32_t *peak_clock_khz);

/*
 * The persistent-grid tile order the kernels run (page "ThunderKittens:
 * Simple, Fast, and Adorable AI Kernels", section 3.4, "Block Launch Order
 * and L2 Cache Reuse"), computed by the same code: writes the tile row *pm
 * and column *pn of work item `t` of a launch with `grid` workgroups over
 * tiles_m x tiles_n tiles in bands of group_m tile rows, with xcd_remap
 * 0, 1 or 2 as applied (tkg_launch_plan reports grid, group_m and
 * xcd_remap). Workgroup w runs items v(w), v(w) + grid, ... where v(w) is
 * its XCD-contiguous id. quad_base >= 0 describes the second launch of a
 * two-launch product instead: item t is quadrant t % 4 of item
 * quad_base + t / 4 of the first launch (whose grid, tile counts, group_m
 * and remap the other arguments then are), and *pm, *pn index the
 * half-edge tiles. Returns TKG_OK, TKG_ERR_NULL for a null pm or pn, or
 * TKG_ERR_SHAPE for a non-positive grid, tile count or group_m, a group_m
 * above tiles_m, an xcd_remap outside 0..2, or t outside the items of the
 * launch described. Host logic only, no GPU work.
 */
int tkg_tile_order(int32_t t, int32_t grid, int32_t xcd_remap, int32_t tiles_m,
                   int32_t tiles_n, int32_t group_m, int32_t quad_base, int32_t *pm,
                   int32_t *pn);

/*
 * LDS layout introspection for the CPU bank-conflict model (no GPU work).
 * Writes the 64 per-lane LDS byte offsets (relative to the operand tile)
 * of one ds_read_b128 fragment read of the staged operand tiles:
 *   dtype  -- TKG_DTYPE_*;
 *   step   -- MFMA k-step inside a stage (0 .. steps-1);
 *   part   -- 0 or 1, which 16-byte half of a 32-byte fp8 operand
 *             (0 for bf16 and for the 4-bit values);
 *   frag   -- fragment index inside the 256-row workgroup tile
 *             (0 .. 256/R - 1, R = tkg_lds_fragment_rows(dtype)).
 * These are the reads of the default kernel configuration (variant 0).
 * Returns the number of k-steps per stage for the dtype, or a negative
 * tkg_status for an invalid argument.
 */
int tkg_lds_fragment_offsets(int dtype, int step, int part, int frag,
                             uint32_t *out64);

/*
 * Rows R of one operand fragment of the default kernel for dtype (the MFMA
 * block: 16 for the 16x16 blocks, 32 for 32x32), or a negative tkg_status.
 */
int tkg_lds_fragment_rows(int dtype);

/*
 * LDS layout introspection of the finish (C = bf16(scale * acc) through a
 * per-wave LDS strip; page "ThunderKittens: Simple, Fast, and Adorable AI
 * Kernels", section 3.4, "The LCSF Template"). Writes the 64 per-lane byte
 * offsets, relative to the wave's strip, of one 16-byte LDS access:
 *   mi     -- MFMA block rows, 16 or 32;
 *   rj     -- accumulator blocks per strip row (strip rows of rj*mi*2 =
 *             64, 128 or 256 bytes; even for mi = 16);
 *   kind   -- 0 = the writes of one round (after the lane-pair swap each
 *             lane writes 8 consecutive columns of its row), 1 = the reads;
 *   index  -- which write or read of the round.
 * Returns the number of accesses of that kind per round, or a negative
 * tkg_status (TKG_ERR_SHAPE for an unsupported shape or index,
 * TKG_ERR_NULL for a null out64). No GPU work.
 */
int tkg_lds_finish_offsets(int mi, int rj, int kind, int index,
                           uint32_t *out64);

/*
 * Row length in bytes of the staged operand tiles for dtype (the unit the
 * swizzle works on), or a negative tkg_status.
 */
int tkg_lds_row_bytes(int dtype);

#ifdef __cplusplus
}
#endif

#endif /* TKG_H */
