/*
 * glu_gemv_tuning.h -- launch-shape overrides of glu_dual_gemv, for
 * benchmark sweeps and tests that pin a particular kernel.
 *
 * Same operation, arguments, ownership, execution and error contract as
 * glu_dual_gemv (include/glu_gemv.h); `tuning` only changes how the work is
 * laid out on the GPU, never the result contract.  A zero field keeps the
 * default.  A combination the library was not built with, or a kernel that
 * cannot serve the shape (GLU_KERNEL_VALU above M = 8, any fast kernel on
 * unaligned input or K % 8 != 0), returns GLU_ERR_UNSUPPORTED and launches
 * nothing.  tuning == NULL is glu_dual_gemv.
 */
#ifndef GLU_GEMV_TUNING_H
#define GLU_GEMV_TUNING_H

#include "glu_gemv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct glu_tuning {
    int kernel;           /* 0 = automatic, else GLU_KERNEL_VALU / _MFMA / _GENERIC / _GEMM */
    int rows_per_wave;    /* VALU: output rows per wave per group (1; 2 at M = 1).
                             MFMA: weight rows per wave, 4, or 8 with mfma_hidden = 3 */
    int waves_per_block;  /* VALU, MFMA: waves per workgroup (1..8) */
    int grid;             /* VALU, MFMA: workgroups of the persistent grid */
    int mfma_segments;    /* MFMA: K segments per pipeline stage; a segment is 128
                             elements at 4 rows per wave (2, 4, 5, 8), 64 at 8 (4, 8) */
    int mfma_hidden;      /* MFMA: where hidden lives: 1 = all in LDS (M*K*2 <= 64 KiB),
                             2 = read from L2 per stage, 3 = per-stage K-slices in LDS
                             with the workgroup's 4 waves in lockstep (segments 2 or 4
                             at 4 rows per wave) */
    int mfma_depth;       /* MFMA with mfma_hidden = 3: pipeline stages of weights kept
                             in flight (4 rows: 4 at 2 segments, 2 at 4; 8 rows: 2 or 4
                             at 4 segments, 1 or 2 at 8).  GEMM: stages of loads in
                             flight while a stage computes (1 to 4) */
    int gemm_tile_n;      /* GEMM: weight rows per output tile (64 or 128) */
    int gemm_tile_m;      /* GEMM: hidden rows per output tile (64 or 128) */
    int xcd_bands;        /* glu_read_ceiling: 1 = the workgroups one XCD runs take one
                             contiguous band of rows (grid a multiple of 8) */
    int gemv_dot;         /* VALU at M = 1: 1 = dot products as fp32 FMAs on the vector ALU,
                             2 = on the matrix cores (the diagonal of one MFMA per 512-element
                             piece of a row; at most 4 waves per workgroup) */
    int mfma_order;       /* MFMA, 8 rows per wave: 1 = each block of 32 weight rows walks K
                             in turn; 2 = a workgroup walks K once for all its blocks (at
                             most 3), loading each K-slice of hidden once (depth 1, more
                             than 8 rows of hidden; 8 segments for launches of up to 32
                             rows, 4 segments for launches of 64 rows: the default
                             above 32 rows) */
} glu_tuning;

glu_status glu_dual_gemv_tuned(const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w,
                               uint16_t* out, int64_t M, int64_t N, int64_t K, void* stream,
                               const glu_tuning* tuning);

/* glu_dual_gemv_strided (glu_gemv.h) with the same overrides. */
glu_status glu_dual_gemv_strided_tuned(const uint16_t* hidden, int64_t ldh, const uint16_t* gate_w, int64_t ldg,
                                       const uint16_t* up_w, int64_t ldu, uint16_t* out, int64_t ldo,
                                       int64_t M, int64_t N, int64_t K, void* stream, const glu_tuning* tuning);

/* glu_grouped_gemv (glu_gemv.h) with overrides: kernel GLU_KERNEL_VALU,
 * GLU_KERNEL_MFMA or GLU_KERNEL_GENERIC; for VALU rows_per_wave 1 or 2 (2
 * only up to M = 4); for MFMA mfma_segments (2, 4, 5; 2 with hidden read
 * from L2) and mfma_hidden 1 or 2; waves_per_block and grid for both.
 * With every N a multiple of 8, mfma_hidden 3 (the default above 8 rows of
 * hidden) streams K-slices of hidden under the weights in 8-row groups,
 * launches of up to 64 rows, stages of 8 segments (4 on request, above 32
 * rows only). */
glu_status glu_grouped_gemv_tuned(const uint16_t* hidden, int64_t ldh, const glu_projection* proj, int n,
                                  int64_t M, int64_t K, void* stream, const glu_tuning* tuning);

/* glu_grouped_gemv_plan with overrides (host only, no HIP call). */
glu_status glu_grouped_gemv_plan_tuned(int64_t M, int64_t K, int64_t rows, int fast, const glu_tuning* tuning,
                                       glu_plan* plan);

/* glu_dual_gemv_plan with overrides (host only, no HIP call). */
glu_status glu_dual_gemv_plan_tuned(int64_t M, int64_t N, int64_t K, int aligned16,
                                    const glu_tuning* tuning, glu_plan* plan);

/*
 * Name of the kernel instance the first launch of a call would run, as a
 * profiler prints it (e.g. "glu::valu_kernel<1, 1, 5, 1, false, false>"),
 * NUL-terminated into buf[len].  Host only, no HIP call.  Returns the plan's
 * status; GLU_ERR_NULL_POINTER if buf is NULL or len < 1 (truncates silently
 * when len is short).
 */
glu_status glu_dual_gemv_describe(int64_t M, int64_t N, int64_t K, int aligned16,
                                  const glu_tuning* tuning, char* buf, int len);

/* The same for glu_grouped_gemv: arguments as glu_grouped_gemv_plan_tuned
 * (glu_gemv.h), e.g. "glu::grouped_mfma_kernel<1, 5, true, false>". */
glu_status glu_grouped_gemv_describe(int64_t M, int64_t K, int64_t rows, int fast, const glu_tuning* tuning,
                                     char* buf, int len);

/*
 * Streaming-read ceiling, a measuring stick for the M = 1 GEMV rather than a
 * part of the projection.  The pages put the GEMV's distance from peak
 * bandwidth down to launch overhead and the memory access pattern (DeepSpeed
 * PR #8602, comment "Plan B: Dual-Weight GEMV", section on why library-level
 * performance is reachable at batch 1); this call isolates those two.  It
 * reads two matrices a and b of `rows` rows of row_bytes bytes each (dense,
 * device memory, 16-byte aligned) with the GEMV's own access pattern and
 * launch shape (glu_dual_gemv_plan at M = 1 and K = row_bytes / 2: the same
 * grid, waves and rows per wave; `tuning` may override rows_per_wave (1, 2 or
 * 4), waves_per_block, grid and xcd_bands, nothing else) and does no arithmetic beyond
 * an XOR of the words read.  sink: 64 uint32 of device memory, written only if
 * that XOR equals one fixed 32-bit value (it exists so that the loads cannot
 * be removed); it may not overlap a or b.
 *
 * row_bytes must be a multiple of 1024 up to 8192 (K = 512 ... 4096 bf16),
 * else GLU_ERR_UNSUPPORTED.  rows == 0: GLU_OK, nothing launched.  Errors as
 * glu_dual_gemv (NULL -> GLU_ERR_NULL_POINTER, alignment ->
 * GLU_ERR_MISALIGNED, sink overlapping -> GLU_ERR_ALIASING, shape ->
 * GLU_ERR_BAD_SHAPE), decided before any HIP call.  Asynchronous on stream,
 * graph-capturable, allocates nothing.
 */
glu_status glu_read_ceiling(const void* a, const void* b, int64_t rows, int64_t row_bytes, uint32_t* sink,
                            const glu_tuning* tuning, void* stream);

/* The launch glu_read_ceiling would make (host only, no HIP call):
 * kernel GLU_KERNEL_CEILING, grid and block. */
glu_status glu_read_ceiling_plan(int64_t rows, int64_t row_bytes, const glu_tuning* tuning, glu_plan* plan);

/*
 * Read/write ceiling: copies a to ca and b to cb (each `rows` rows of
 * row_bytes bytes, dense device memory, 16-byte aligned) in the launch shape
 * of glu_read_ceiling, with nontemporal 16-byte loads and stores.  It is the
 * measuring stick for the backward's one-pass kernels, which read both weight
 * matrices once and write both weight gradients once (the same bytes each
 * way at M = 1).  tuning: as glu_read_ceiling, with rows_per_wave 1 or 2 and
 * no xcd_bands.  The four arrays may not overlap (GLU_ERR_ALIASING); other
 * errors as glu_read_ceiling, all decided before any HIP call.  rows == 0:
 * GLU_OK, nothing launched.  Asynchronous on stream, graph-capturable,
 * allocates nothing.
 */
glu_status glu_copy_ceiling(const void* a, const void* b, void* ca, void* cb, int64_t rows, int64_t row_bytes,
                            const glu_tuning* tuning, void* stream);

/*
 * Unit ceilings: the issue rate of one unit of a compute unit, a measuring stick
 * for the matrix-core kernels (the tiled GEMM, the backward's contractions)
 * rather than a part of the projection.  `workgroups` workgroups of
 * waves_per_cu waves run (pass the device's compute-unit count for one
 * workgroup per CU); every wave repeats one body `iterations` times:
 *   GLU_UNIT_MFMA_16X16X32_BF16: 8 independent v_mfma_f32_16x16x32_bf16 on
 *     register operands, 8 * 16384 flops;
 *   GLU_UNIT_MFMA_32X32X16_BF16: 4 independent v_mfma_f32_32x32x16_bf16,
 *     4 * 32768 flops;
 *   GLU_UNIT_LDS_READ_B128: 16 conflict-free ds_read_b128 of a 64 KiB LDS
 *     array folded by XOR, 16 KiB read.
 * glu_unit_ceiling_work gives the flops (MFMA) or LDS bytes (LDS) of one
 * launch.  sink: 64 uint32 of device memory, written only if a folded result
 * equals one fixed 32-bit value (it keeps the work from being removed).
 * unit outside the three, waves_per_cu outside 1..16, workgroups outside
 * 1..65536 or iterations outside 1..2^20 -> GLU_ERR_UNSUPPORTED; sink NULL ->
 * GLU_ERR_NULL_POINTER, not 4-byte aligned -> GLU_ERR_MISALIGNED; all decided
 * before any HIP call.  Asynchronous on stream, graph-capturable, allocates
 * nothing.
 */
#define GLU_UNIT_MFMA_16X16X32_BF16 1
#define GLU_UNIT_MFMA_32X32X16_BF16 2
#define GLU_UNIT_LDS_READ_B128 3

glu_status glu_unit_ceiling(int unit, int waves_per_cu, int64_t workgroups, int64_t iterations, uint32_t* sink,
                            void* stream);

/* The work of that launch (host only): flops for the MFMA units, bytes read for
 * the LDS unit, in *work; same argument checks. */
glu_status glu_unit_ceiling_work(int unit, int waves_per_cu, int64_t workgroups, int64_t iterations, double* work);

#ifdef __cplusplus
}
#endif

#endif /* GLU_GEMV_TUNING_H */
