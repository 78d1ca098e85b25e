// Internal interface of the backward kernels (glu_backward.hip).
#pragma once

#include "../../include/glu_gemv.h"
#include "glu_device.h"
#include "glu_launch.h"

namespace glu {

// The backward's elementwise step.  From g and u (the bf16 gate and up values of the forward) and go
// (the bf16 upstream gradient of the output): du = bf16(go s) with s = bf16(silu(g)), and
// dg = bf16(bf16(go u) sigma(g) (1 + g (1 - sigma(g)))), each fp32 step computed in fp64 and rounded
// once to fp32 (for +, -, *, / of fp32 operands this equals the IEEE fp32 result: 53 >= 2 * 24 + 2
// bits), exp as in the forward's epilogue.
__device__ __forceinline__ void glu_act_grad(float g, float u, float go, uint16_t* dg_out, uint16_t* du_out)
{
    const float e = (float)exp(-(double)g);
    const float d = (float)(1.0 + (double)e);
    const float s = bf16_to_f32(f32_to_bf16_rne((float)((double)g / (double)d)));  // silu(g) as a bf16 tensor
    const float ds = bf16_to_f32(f32_to_bf16_rne((float)((double)go * (double)u)));
    *du_out = f32_to_bf16_rne((float)((double)go * (double)s));
    const float sig = (float)(1.0 / (double)d);
    const float t1 = (float)((double)ds * (double)sig);
    const float t2 = (float)(1.0 - (double)sig);
    const float t3 = (float)((double)g * (double)t2);
    const float t4 = (float)(1.0 + (double)t3);
    *dg_out = f32_to_bf16_rne((float)((double)t1 * (double)t4));
}

// Two fp32 values to a packed pair of bf16 (lo in bits 0-15), round to nearest with ties to even:
// gfx950's v_cvt_pk_bf16_f32, one instruction for the pair (f32_to_bf16_rne takes about five per
// value).  Used where a result is written once and never fed to further arithmetic (a NaN comes
// out as some quiet NaN).
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, v);
}


constexpr int kBwdMaxM = 1 << 16;  // rows of hidden per call
constexpr int kBwdMfmaMaxM = 64;   // the matrix-core contractions of kPathMfma serve up to here
constexpr int kBwdChunkM = 8;   // rows of hidden of the VALU contraction kernel at most
constexpr int kBwdTargetBlocks = 512;  // contraction workgroups aimed for (2 per CU)

constexpr int kFusedMaxU = 5;        // one-pass kernel: up to 5 16-byte chunks per lane (K <= 2560)
constexpr int kFusedWaves = 4;       // waves per workgroup of the one-pass kernel
// persistent waves per CU it aims for: 8, or 4 at 5 chunks per lane (over 256 registers a wave)
constexpr int kFusedMaxM = 2;        // one-pass kernel: up to 2 rows of hidden (with 3 the four-launch
                                      // path measured faster: 57.7 against 68.0 us at K=2048 N=8192)
constexpr int fused_max_u(int M) { return M <= 2 ? kFusedMaxU : 0; }
// M = 1 at U = 5 (K = 2560) keeps hidden in LDS, within 256 registers
constexpr bool fused1_hidden_in_lds(int M, int U) { return M == 1 && U == 5; }
constexpr int fused_waves_per_cu(int M, int U) { return M == 1 && U < 5 ? 8 : 4; }
constexpr int kCUsForPlan = 256;     // MI355X compute units

constexpr int kSplitMaxWaves = 8;     // K-split kernel: waves per workgroup at most (256 VGPRs a lane)
constexpr int kSplitMaxM = 4;         // rows of hidden at most (beyond, the dot products' butterflies
                                      // and the dh accumulators make the four-launch path faster)
constexpr int kSplitMaxM2 = 3;        // rows of hidden at most with two chunks per lane
constexpr int kSplitMinK = 2568;      // at K <= 2560 a workgroup of at most 5 waves per CU hides too
                                      // little latency: M = 1 takes fused1_kernel, M >= 2 the four launches
constexpr int kSplitMaxThreads = kSplitMaxWaves * 64;
// weight rows per batch of the K-split kernel (their loads are issued one batch ahead): as many as
// the registers beside M rows of dh accumulators allow
constexpr int split_rows(int M, int U) { return U == 1 ? (M <= 2 ? 4 : 2) : (M <= 2 ? 2 : 1); }

// which kernels a backward call runs
constexpr int kPathChunks = 0;   // 2 <= M <= 8: dg and du (the forward's 4-row kernel with the gradient
                                 // step as its epilogue, or the grouped GEMV and the gradient step),
                                 // contraction, reduction
constexpr int kPathFused1 = 1;   // M == 1, K <= 2560: fused1_kernel, reduction
constexpr int kPathSplitK = 2;   // M <= 2 with 2560 < K <= 8192, M = 3, 4 with 3584 < K <= 4096:
                                 // splitk_kernel, reduction
constexpr int kPathMfma = 3;     // 8 < M <= 64: dg and du (the forward's slice-major or 4-row kernel with
                                 // the gradient step as its epilogue, or the grouped GEMV and the
                                 // gradient step), repacking, dh_mfma_kernel, reduction, dw_mfma_kernel
constexpr int kPathGemm = 4;     // M > 64: tiled GEMM for g and u with the gradient step in its
                                 // epilogue, repacking, dh_mfma_kernel over slices of 128 or 256 rows of
                                 // hidden, reduction, and the weight gradients as one transposed tiled
                                 // GEMM (gemm_dw_launch)
constexpr int kBwdMfmaMinM = 9;  // rows of hidden from which the contractions run on MFMA
// where dg and du come from when the tiled GEMM does not form them (BwdPlan::gu_fused)
constexpr int kGuGrouped = 0;
constexpr int kGuFusedPass = 1;
constexpr int kGuFusedMfma4 = 2;
// columns of dh per dh_mfma_kernel workgroup for mt 16-row tiles of hidden per slice
constexpr int dh_cols(int mt) { return mt <= 4 ? 128 : 64; }

struct BwdPlan {
    int path;                // kPathChunks, kPathFused1, kPathSplitK, kPathMfma or kPathGemm
    bool fused;              // M == 1, K <= 2560: the one-pass kernel
    int fused_grid;          // its workgroups (each leaves one partial of dh)
    int split_u;             // K-split kernel: chunks per lane (1 or 2)
    int split_waves;         // waves per workgroup
    int split_rpb;           // weight rows per workgroup
    int split_grid;          // workgroups (each leaves one partial of dh)
    int mp16, mp32;          // MFMA path: M rounded up to 16, 32 or 64, above 64 rows 128 and above 128 rows
                             // 256 per slice (dh's B operand), and M rounded up to 32 (dW's)
    int np32;                // N rounded up to 32 (the columns of dg2, du2)
    int dh_splits, dh_jr;    // ranges of weight rows (jr rows each, a multiple of 32) = dh's partials
    int dh_mslices;          // slices of mp16 rows of hidden dh's grid covers (1 up to 128 rows)
    int dh_steps;            // 32-row steps of the longest range
    bool gu_gemm;            // g and u from the tiled GEMM (N % 4 == 0 and M > 64, or M > 32 with N % 8 != 0)
                             // instead of the grouped GEMV
    int gu_fused;            // without gu_gemm, set by the API's planner: kGuFusedPass (8 < M <= 64) or
                             // kGuFusedMfma4 (2 <= M <= 16) where the forward's plan for (M, N, K) is
                             // that kernel in one launch: dg and du from it, with the
                             // elementwise step as its epilogue; else kGuGrouped (the grouped GEMV, then
                             // act_grad_kernel)
    MfmaConfig gu_cfg;       // the forward's launch it repeats
    int64_t off_g2, off_gT, off_hT, off_partial;  // workspace offsets of dg2/du2, dgT/duT, hT, the partials
    int nslabs;              // 512-column slabs of K
    int nranges;             // row ranges of N (the one-pass kernel: its workgroups)
    int rows_per_range;
    int64_t gu_bytes;        // workspace head: [2][M][N] bf16 (g, u, then dg, du), 256-byte padded
    int64_t partial_bytes;   // then [nranges][2][M][K] fp32 partial sums of dh
    int64_t workspace_bytes;
    int accum_depth;         // longest fp32 addition chain behind one dh contribution
};

BwdPlan bwd_plan(int64_t M, int64_t N, int64_t K);
// glu_dual_gemv_backward's validation and launches (glu_api.hip); validate_only: return after the
// checks that need no workspace, before any HIP call
glu_status backward_entry(const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w, const uint16_t* dout,
                          uint16_t* dh, uint16_t* dwg, uint16_t* dwu, int64_t M, int64_t N, int64_t K, void* ws,
                          int64_t ws_bytes, void* stream, bool validate_only);
// GLU_ERR_LAUNCH, recording e as the calling thread's last HIP error
glu_status launch_failed(hipError_t e);
// workspace bytes of a backward call (0 when an extent is zero), with plan_backward's status
glu_status backward_workspace(int64_t M, int64_t N, int64_t K, int64_t* bytes);
hipError_t act_grad_launch(uint16_t* gu, const uint16_t* dout, int64_t ldd, int M, int N, hipStream_t stream);
// g and u with the elementwise step as the epilogue, on the forward's slice-major 8-row kernel
// (glu_mfma8_act.hip): dg, du into gu ([2][M][N]).  U, nsg, ragged and grid as the forward's plan for
// (M, N, K) has them (one launch, M <= 64); dense operands, K % 8 == 0.
// the same on the forward's 4-row kernel with hidden in LDS, up to kMfmaActMaxM rows (glu_mfma_act.hip)
constexpr int kMfmaActMaxM = 16;
bool mfma_act_supported(const MfmaConfig& c, int M);
hipError_t mfma_act_launch(const MfmaConfig& c, int M, const uint16_t* hidden, const uint16_t* gate_w,
                           const uint16_t* up_w, const uint16_t* dout, uint16_t* gu, int64_t N, int64_t K,
                           hipStream_t stream);
hipError_t mfma8_act_launch(int M, int U, int nsg, bool ragged, int grid, const uint16_t* hidden,
                            const uint16_t* gate_w, const uint16_t* up_w, const uint16_t* dout, uint16_t* gu,
                            int64_t N, int64_t K, hipStream_t stream);
// K % 8 == 0, hidden / gate_w / up_w / dwg / dwu 16-byte aligned, packed rows.  M <= 8; dw: also
// the weight gradients (then these M rows are all rows of hidden).  dgm, dum: [M][N].
hipError_t contract_launch(const BwdPlan& p, int M, const uint16_t* hidden, const uint16_t* gate_w,
                           const uint16_t* up_w, const uint16_t* dgm, const uint16_t* dum, uint16_t* dwg,
                           uint16_t* dwu, float* partial, int N, int K, hipStream_t stream);
// weight gradients over all M <= kBwdMaxM rows of hidden
hipError_t fused1_launch(const BwdPlan& p, int M, const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w,
                        const uint16_t* dout, uint16_t* dgu, uint16_t* dwg, uint16_t* dwu, float* partial, int N, int K,
                        hipStream_t stream);
hipError_t splitk_launch(const BwdPlan& p, int M, const uint16_t* hidden, const uint16_t* gate_w,
                         const uint16_t* up_w, const uint16_t* dout, uint16_t* dgu, uint16_t* dwg, uint16_t* dwu,
                         float* partial, int N, int K, hipStream_t stream);
// zero-padded copies of R x C bf16 matrices (rows ld elements apart) for the MFMA backward
struct RepackJob {
    const uint16_t* src;
    int64_t ld;
    uint16_t* dst;
    int R, C, Rp, Cp;   // Rp >= R rows (transposed: the row length), Cp >= C columns (not transposed)
    int transpose;
    int64_t first_block, nblocks;  // set by repack_launch: the job's workgroups of the launch
    int vec;                       // set by repack_launch: 16-byte accesses (see repack_kernel)
};
constexpr int kMaxRepackJobs = 5;
struct RepackJobs {
    RepackJob job[kMaxRepackJobs];
    int n;
};
hipError_t repack_launch(RepackJobs jobs, hipStream_t stream);
hipError_t dw_mfma_launch(const BwdPlan& p, const uint16_t* hT, const uint16_t* dgT, const uint16_t* duT,
                          uint16_t* dwg, uint16_t* dwu, int N, int K, hipStream_t stream);
hipError_t dh_mfma_launch(const BwdPlan& p, int M, const uint16_t* gate_w, const uint16_t* up_w, const uint16_t* g2,
                          const uint16_t* u2, float* partial, int N, int K, hipStream_t stream);
hipError_t dh_reduce_launch(const BwdPlan& p, const float* partial, uint16_t* dh, int64_t ldh_out, int M, int K,
                            hipStream_t stream);

}  // namespace glu
