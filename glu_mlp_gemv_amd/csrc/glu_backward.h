// Internal interface of the backward kernels (glu_backward.hip).
#pragma once

#include "glu_launch.h"

namespace glu {

constexpr int kBwdMaxM = 64;    // rows of hidden per call
constexpr int kBwdChunkM = 8;   // rows of hidden per contraction launch (dh); dw_kernel takes all
constexpr int kBwdTargetBlocks = 512;  // contraction workgroups aimed for (2 per CU)

constexpr int kFusedMaxU = 5;        // one-pass kernel: up to 5 16-byte chunks per lane (K <= 2560)
constexpr int kFusedWaves = 4;       // waves per workgroup of the one-pass kernel
// persistent waves per CU it aims for: 8, or 4 at 5 chunks per lane (over 256 registers a wave)
constexpr int fused_waves_per_cu(int U) { return U >= 5 ? 4 : 8; }
constexpr int kCUsForPlan = 256;     // MI355X compute units

struct BwdPlan {
    bool fused;              // M == 1, K <= 2560: the one-pass kernel
    int fused_grid;          // its workgroups (each leaves one partial of dh)
    int nslabs;              // 512-column slabs of K
    int nranges;             // row ranges of N (the one-pass kernel: its workgroups)
    int rows_per_range;
    int64_t gu_bytes;        // workspace head: [2][M][N] bf16 (g, u, then dg, du), 256-byte padded
    int64_t partial_bytes;   // then [nranges][2][M][K] fp32 partial sums of dh
    int64_t workspace_bytes;
    int accum_depth;         // longest fp32 addition chain behind one dh contribution
};

BwdPlan bwd_plan(int64_t M, int64_t N, int64_t K);
hipError_t act_grad_launch(uint16_t* gu, const uint16_t* dout, int64_t ldd, int M, int N, hipStream_t stream);
// K % 8 == 0, hidden / gate_w / up_w / dwg / dwu 16-byte aligned, packed rows.  M <= 8; dw: also
// the weight gradients (then these M rows are all rows of hidden).  dgm, dum: [M][N].
hipError_t contract_launch(const BwdPlan& p, int M, bool dw, const uint16_t* hidden, const uint16_t* gate_w,
                           const uint16_t* up_w, const uint16_t* dgm, const uint16_t* dum, uint16_t* dwg,
                           uint16_t* dwu, float* partial, int N, int K, hipStream_t stream);
// weight gradients over all M <= kBwdMaxM rows of hidden
hipError_t dw_launch(const BwdPlan& p, int M, const uint16_t* hidden, const uint16_t* dgm, const uint16_t* dum,
                     uint16_t* dwg, uint16_t* dwu, int N, int K, hipStream_t stream);
hipError_t fused1_launch(const BwdPlan& p, const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w,
                        const uint16_t* dout, uint16_t* dgu, uint16_t* dwg, uint16_t* dwu, float* partial, int N, int K,
                        hipStream_t stream);
hipError_t dh_reduce_launch(const BwdPlan& p, const float* partial, uint16_t* dh, int64_t ldh_out, int M, int K,
                            hipStream_t stream);

}  // namespace glu
