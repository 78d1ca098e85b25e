/*
 * glu_gemv.h -- C ABI of the dual-weight GLU projection for MI355X (gfx950).
 *
 * The operation (DeepSpeed PR #8602, "HybridEngineRollout graph capture +
 * segment-KI for Qwen3.5 hybrid", comment "Plan B: Dual-Weight GEMV": the
 * DualWeightGluGEMV forward and its kernel, which read gate.weight and
 * up.weight directly instead of a concatenated copy; rounding per DeepSpeed
 * PR #9057, "preserve HF precision boundaries in segKI kernels", section
 * "Changes"):
 *
 *   G[m,j]   = sum_k hidden[m,k] * gate_w[j,k]        (fp32 accumulation)
 *   U[m,j]   = sum_k hidden[m,k] * up_w[j,k]          (fp32 accumulation)
 *   g = bf16(G), u = bf16(U)                          (round to nearest even)
 *   s = bf16( g / (1 + exp(-g)) )                     (fp32 silu, IEEE steps)
 *   out[m,j] = bf16( s * u )                          (fp32 product)
 *
 * Every array is dense and row-major; bf16 values travel as their raw 16-bit
 * patterns (uint16_t), so this header needs no HIP or bf16 type:
 *   hidden [M, K]   activations, one row per token
 *   gate_w [N, K]   gate projection weight, nn.Linear layout [out, in]
 *   up_w   [N, K]   up projection weight, same layout
 *   out    [M, N]   result
 *
 * Ownership: the caller allocates all four buffers in device memory of the
 * current HIP device and keeps them alive until the work on `stream` is
 * done.  The library allocates nothing, copies nothing, concatenates
 * nothing and caches nothing keyed on pointers: every call reads the weights
 * as they are at execution time, so in-place weight updates are seen by the
 * next call.
 *
 * Execution: asynchronous on `stream` (a hipStream_t; NULL is the null
 * stream).  No host synchronisation, no allocation, a launch configuration
 * fixed by (M, N, K) and the pointers' alignment: the call may be captured
 * into a HIP graph.  Deterministic: identical inputs give bitwise-identical
 * output on every call (no atomics, fixed reduction order).  Stateless and
 * reentrant; concurrent calls on different streams are independent.
 *
 * Errors are returned, never thrown; arguments are validated before any HIP
 * call, so an invalid call launches nothing.
 */
#ifndef GLU_GEMV_H
#define GLU_GEMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum glu_status {
    GLU_OK = 0,
    GLU_ERR_NULL_POINTER = 1, /* a non-empty array was given as NULL */
    GLU_ERR_BAD_SHAPE = 2,    /* M, N or K negative, or an element/byte count overflows int64 */
    GLU_ERR_MISALIGNED = 3,   /* a pointer is not 2-byte aligned */
    GLU_ERR_ALIASING = 4,     /* out overlaps hidden, gate_w or up_w */
    GLU_ERR_LAUNCH = 5,       /* the HIP launch failed; see glu_last_hip_error() */
    GLU_ERR_UNSUPPORTED = 6,  /* a tuning override the library cannot serve (glu_gemv_tuning.h) */
    GLU_ERR_BAD_STRIDE = 7,   /* glu_dual_gemv_strided: a row stride below its row length, or
                                 rows whose extent overflows int64 */
    GLU_ERR_WORKSPACE = 8,    /* glu_dual_gemv_backward: workspace NULL, not 256-byte aligned
                                 or smaller than glu_dual_gemv_backward_workspace asks */
    GLU_ERR_SCRATCH_LIMIT = 9 /* glu_dual_gemv_backward_noalloc: the call needs more scratch than
                                 the library's fixed device array holds */
} glu_status;

/*
 * out = bf16(bf16(silu(bf16(hidden @ gate_w^T))) * bf16(hidden @ up_w^T)).
 *
 * M >= 0, N >= 0, K >= 0.  M == 0 or N == 0: nothing to do, GLU_OK, pointers
 * unchecked.  K == 0: every output is +0 (the empty sums give silu(0) * 0).
 * Fast path: hidden, gate_w and up_w 16-byte aligned, K a multiple of 8 and
 * K <= 2^25; any other 2-byte-aligned input takes a slower path with the same
 * result contract.  M == 1 with K <= 4096 runs a VALU GEMV; other shapes up
 * to M = 64 run a block-diagonal MFMA kernel (one launch, reading the
 * weights once); M > 64 runs a tiled MFMA GEMM (GLU_KERNEL_GEMM), one launch
 * per 65536 rows of hidden, each reading the weights once.
 */
glu_status glu_dual_gemv(const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w,
                         uint16_t* out, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * glu_dual_gemv on row-strided operands: row m of hidden starts at
 * hidden + m*ldh, row j of gate_w at gate_w + j*ldg, row j of up_w at
 * up_w + j*ldu, row m of out at out + m*ldo (strides in elements; the K, resp.
 * N, elements of a row are contiguous).  This is what a view sliced out of a
 * wider row block looks like, e.g. the gate and up halves of a fused
 * projection's output or a column slice of a larger matrix.  The fix for
 * exactly such a view, read as if it were packed, is in DeepSpeed PR #9057
 * "fix(module-inject): preserve HF precision boundaries in segKI kernels"
 * (commit notes: q sliced from the fused q|k|v block keeps the fused row
 * stride; pass the real stride and fail closed on one that disagrees); see
 * also PR #8602's commit notes on the strided gdn_gates input.
 *
 * Strides must be at least the row length: ldh, ldg, ldu >= K (when K > 0)
 * and ldo >= N, else GLU_ERR_BAD_STRIDE and nothing is launched; nothing
 * ever reads or writes between rows.  Rows may not overlap (a stride below
 * the row length is refused, never read as broadcast).  The fast kernels
 * run when the pointers are 16-byte aligned, K and ldh, ldg, ldu are
 * multiples of 8 and the strides are at most 2^25; any other layout takes
 * the 2-byte generic kernel with the same result.  The result is bitwise
 * the result of glu_dual_gemv on the same rows stored packed.  Ownership,
 * execution and the other errors are those of glu_dual_gemv (aliasing is
 * checked on the strided extents).  glu_dual_gemv(h, g, u, o, M, N, K, s) is
 * glu_dual_gemv_strided(h, K, g, K, u, K, o, N, M, N, K, s).
 */
glu_status glu_dual_gemv_strided(const uint16_t* hidden, int64_t ldh, const uint16_t* gate_w, int64_t ldg,
                                 const uint16_t* up_w, int64_t ldu, uint16_t* out, int64_t ldo,
                                 int64_t M, int64_t N, int64_t K, void* stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* glu_status_string(int status);

/* hipError_t of the most recent GLU_ERR_LAUNCH on the calling thread (0 if none). */
int glu_last_hip_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int glu_version(void);

/*
 * Which kernel glu_dual_gemv would launch for a shape, decided on the host
 * alone (no HIP call; usable without a GPU).  `aligned16` states whether
 * hidden, gate_w and up_w are all 16-byte aligned.
 */
typedef struct glu_plan {
    int kernel;        /* GLU_KERNEL_* */
    int m_per_launch;  /* rows of hidden one launch covers */
    int launches;      /* launches one call makes */
    int grid;          /* workgroups per launch */
    int block;         /* threads per workgroup */
    int accum_depth;   /* longest chain of fp32 additions behind one output */
} glu_plan;

enum {
    GLU_KERNEL_NONE = 0,    /* M == 0 or N == 0 */
    GLU_KERNEL_ZERO = 1,    /* K == 0: fill out with +0 */
    GLU_KERNEL_VALU = 2,    /* M == 1, K <= 4096, fast path (any M <= 8 on request) */
    GLU_KERNEL_MFMA = 3,    /* other fast-path shapes up to M = 64 */
    GLU_KERNEL_GENERIC = 4, /* unaligned, K % 8 != 0 or K > 2^25 */
    GLU_KERNEL_GEMM = 5,    /* M > 64, fast path: tiled MFMA GEMM, slices of 65536 rows of hidden */
    GLU_KERNEL_BACKWARD = 6, /* glu_dual_gemv_backward_plan: the backward's launches (2 to 6) */
    GLU_KERNEL_CEILING = 7   /* glu_read_ceiling_plan (glu_gemv_tuning.h): the streaming-read yardstick */
};

glu_status glu_dual_gemv_plan(int64_t M, int64_t N, int64_t K, int aligned16, glu_plan* plan);

/*
 * Grouped GEMV: n projections of one hidden, out_i = bf16(hidden @ W_i^T)
 * for i < n, each W_i read in place.  This is the pages' single/triple/quad
 * GEMV (the QKV and GatedDeltaNet input projections), which DeepSpeed PR
 * #9057 "fix(module-inject): preserve HF precision boundaries in segKI
 * kernels" (commit notes) folds into one grouped_linear dispatcher, without
 * the GLU epilogue: every output is the fp32 dot product rounded once to
 * bf16 (round to nearest, ties to even), as a bf16 nn.Linear output.
 */
#define GLU_GROUP_MAX 8

typedef struct glu_projection {
    const uint16_t* weight;  /* [N, K] bf16 bits, row j at weight + j*ldw */
    uint16_t* out;           /* [M, N] bf16 bits, row m at out + m*ldo */
    int64_t N;               /* output features (>= 0; 0 skips the projection) */
    int64_t ldw;             /* weight row stride in elements, >= K */
    int64_t ldo;             /* output row stride in elements, >= N */
} glu_projection;

/*
 * hidden [M, K] at row stride ldh (>= K), 1 <= n <= GLU_GROUP_MAX entries in
 * proj (host memory, read during the call only; the arrays they point to are
 * device memory owned by the caller).  Validation before any HIP call, in
 * this order: n or a size out of range -> GLU_ERR_BAD_SHAPE; a stride below
 * its row length or an overflowing extent -> GLU_ERR_BAD_STRIDE; M == 0 or
 * every N == 0 -> GLU_OK, nothing launched; a NULL array that would be read
 * or written -> GLU_ERR_NULL_POINTER; a pointer not 2-byte aligned ->
 * GLU_ERR_MISALIGNED; an output overlapping hidden, a weight or another
 * output -> GLU_ERR_ALIASING.  K == 0 writes +0 everywhere.
 *
 * Kernels ("fast layout": hidden and every weight 16-byte aligned, K, ldh and
 * every ldw multiples of 8, strides at most 2^25): for M >= 2 with a fast
 * layout and every N a multiple of 4, a block-diagonal MFMA GEMV, M <= 32
 * rows of hidden per launch (M <= 64 above 8 rows when every N is a multiple
 * of 8: K-slices of hidden streamed under the weights); else, with a fast
 * layout and K <= 8192, a VALU
 * GEMV, M <= 8 rows per launch (both stream the n weights as one row space;
 * larger M runs in slices, each streaming the weights again); any other
 * layout takes a generic kernel with 2-byte loads and the same result
 * contract.  Asynchronous on stream, deterministic, allocates nothing.
 */
glu_status glu_grouped_gemv(const uint16_t* hidden, int64_t ldh, const glu_projection* proj, int n,
                            int64_t M, int64_t K, void* stream);

/*
 * The launch glu_grouped_gemv would make for M rows of hidden, K, and `rows`
 * = sum of N over the projections (host only, no HIP call).  `fast` is a
 * bit set: 1 = the layout is a fast layout (above), 2 = every N is a
 * multiple of 4, 4 = every N is a multiple of 8 (above 8 rows of hidden
 * held in LDS the MFMA kernel then takes groups of 8 weight rows).
 */
glu_status glu_grouped_gemv_plan(int64_t M, int64_t K, int64_t rows, int fast, glu_plan* plan);

/*
 * Backward of glu_dual_gemv: the gradients of hidden, gate_w and up_w for an
 * upstream gradient dout of out.  The segKI "Plan B" autograd Function keeps
 * hidden, gate_w and up_w and returns gradients equal to those of the
 * composite silu(h Wg^T) * (h Wu^T) (DeepSpeed PR #8602, comment "Plan B:
 * Dual-Weight GEMV", sections "Plan B Design" and "Verification Results");
 * over bf16 tensors each
 * gradient tensor is rounded once to bf16, round to nearest even, as
 * autograd of the bf16 composite rounds it.  With g, u, s the forward's bf16
 * gate, up and silu(g) (glu_dual_gemv):
 *   ds = bf16(dout * u)          du = bf16(dout * s)
 *   dg = bf16(ds * sig * (1 + g * (1 - sig))), sig = 1 / (1 + exp(-g)),
 *        evaluated in fp32 as (ds * sig) * (1 + g * (1 - sig))
 *   dhidden = bf16(fp32(bf16(dg @ gate_w) + bf16(du @ up_w)))      [M,K]
 *   dgate_w = bf16(dg^T @ hidden),  dup_w = bf16(du^T @ hidden)     [N,K]
 * The contractions accumulate in fp32; dgate_w and dup_w sum the M rows of
 * hidden in order, dhidden sums over the N weight rows in a fixed order.
 *
 * Arrays: bf16 bit patterns, dense row-major, on the current HIP device,
 * caller-owned: hidden [M,K], gate_w and up_w [N,K], dout [M,N]; outputs
 * dhidden [M,K], dgate_w and dup_w [N,K] (overwritten, not accumulated into).
 * workspace: device memory of at least glu_dual_gemv_backward_workspace()
 * bytes, 256-byte aligned, not overlapping any argument.  On return it
 * begins with dg and du, the bf16 gradients of the gate and up
 * pre-activations ([2][M][N], dense); the rest is scratch.  Limits:
 * M <= 65536 (else GLU_ERR_UNSUPPORTED); hidden, gate_w, up_w, dgate_w, dup_w
 * 16-byte aligned and K % 8 == 0 (else GLU_ERR_UNSUPPORTED).
 * Empty sums give +0: N == 0 zero-fills dhidden, M == 0 zero-fills both
 * weight gradients; K == 0 has nothing to write.  Validation (NULL arrays,
 * shapes, 2-byte alignment, overlap of an output or the workspace with an
 * input or another output, workspace) happens before any HIP call.  On
 * stream, asynchronous, deterministic, allocating nothing: for M <= 2 with
 * K <= 2560, for M <= 2 with 2560 < K <= 8192, and for M = 3 or 4 with
 * 3584 < K <= 4096, two launches, a pass that reads each
 * weight row once and the reduction of dhidden's partial sums; otherwise
 * dg and du from one launch of the forward's MFMA kernel for (M, N, K) with
 * the elementwise step as its epilogue (the 4-row kernel with hidden in LDS
 * up to M = 16, the slice-major 8-row kernel up to M = 64, where the
 * forward runs that kernel in one launch), or above M = 64, or above 32 when
 * only N % 4 == 0, of a tiled GEMM with that step in its epilogue, else from
 * the grouped GEMV for g and u and the elementwise step; then the gradient
 * kernels (above M = 8 on the matrix cores; above M = 64 dhidden
 * over slices of 128 rows of hidden, above M = 128 of 256, and the weight
 * gradients as one tiled GEMM contracting over the rows of hidden).
 */
glu_status glu_dual_gemv_backward(const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w,
                                  const uint16_t* dout, uint16_t* dhidden, uint16_t* dgate_w, uint16_t* dup_w,
                                  int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                                  void* stream);

/*
 * glu_dual_gemv_backward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument, no allocation.  The scratch the backward
 * needs lives in one 48 MiB device array of the library (50,331,648 bytes;
 * each GPU the library runs on holds its own copy until the process ends).
 * Same arguments, results and validation as glu_dual_gemv_backward without the
 * workspace; a shape whose glu_dual_gemv_backward_workspace exceeds 48 MiB
 * returns GLU_ERR_SCRATCH_LIMIT before any HIP call (e.g. K=2560 N=9216 is
 * served up to M = 197, K=4096 N=12288 up to M = 158).  The first
 * call on a device looks the array up (hipGetSymbolAddress).  All calls on one
 * GPU share its array and leave the last call's contents there (on return it
 * begins with dg and du, as the workspace does): calls that overlap on one GPU
 * (two streams, or a graph replay and another call in flight) race and must
 * be ordered by the caller.
 */
glu_status glu_dual_gemv_backward_noalloc(const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w,
                                          const uint16_t* dout, uint16_t* dhidden, uint16_t* dgate_w,
                                          uint16_t* dup_w, int64_t M, int64_t N, int64_t K, void* stream);

/* Workspace bytes glu_dual_gemv_backward needs for (M, N, K), into *bytes
 * (0 when an extent is zero).  Host only.  GLU_ERR_BAD_SHAPE or
 * GLU_ERR_UNSUPPORTED (M > 65536) as the call would return. */
glu_status glu_dual_gemv_backward_workspace(int64_t M, int64_t N, int64_t K, int64_t* bytes);

/* The backward's launches for (M, N, K), host only: kernel
 * GLU_KERNEL_BACKWARD, launches per call, grid and block of the kernel that
 * reads the weights for the gradients, accum_depth = longest fp32 addition
 * chain behind one of dhidden's two contributions or, where that kernel
 * also forms them, behind the gate and up pre-activations. */
glu_status glu_dual_gemv_backward_plan(int64_t M, int64_t N, int64_t K, glu_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* GLU_GEMV_H */
