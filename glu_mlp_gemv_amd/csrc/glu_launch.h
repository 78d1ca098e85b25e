// Internal launch interface between the C ABI (glu_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace glu {

constexpr int kWave = 64;
constexpr int kWaveSumDepth = 6;  // fp32 addition levels of the wave64 butterfly
constexpr int kValuMaxM = 8;
constexpr int kValuMaxThreads = 512;
constexpr int kLdsBudget = 64 * 1024;  // dynamic LDS per workgroup, bytes
constexpr int kLdsMax = 160 * 1024;    // LDS of one workgroup on gfx950, bytes
constexpr int kMfmaMaxThreads = 256;  // 4 waves: the compiler may use AGPRs for the accumulators
constexpr int kXcds = 8;               // accelerator complex dies of an MI355X; workgroups are dealt to them in turn

struct ValuConfig {
    int M;        // rows of hidden in this launch (1..8)
    int R;        // output rows per wave per group
    int U;        // 16-byte chunks per lane per stage
    int NB;       // stages per row group (1 or 2): NB * U * 64 >= K / 8
    bool ragged;  // NB * U * 64 > K / 8: clamp and zero the excess chunks
    int grid;     // workgroups (persistent)
    int block;    // threads per workgroup (multiple of 64)
    bool diag;    // M == 1: dot products on the matrix cores (the diagonal of one MFMA per chunk-set)
};

// Where the MFMA kernel keeps hidden [M,K]:
constexpr int kHiddenLds = 0;     // all of it in LDS (mfma_hidden_lds_bytes <= 64 KiB)
constexpr int kHiddenL2 = 1;      // read from L2 with each stage's weights
constexpr int kHiddenSlices = 2;  // per-stage K-slices in an LDS ring, waves in lockstep

// Order of the 8-row K-slice kernel's work (MfmaConfig::order)
constexpr int kOrderBlocks = 0;  // each block of 4 groups walks K in turn
constexpr int kOrderSlices = 1;  // K walked once for all of a workgroup's blocks (at most kPassBlocks)
constexpr int kPassBlocks = 3;

struct MfmaConfig {
    int rows;         // weight rows per wave: 4, or 8 (kHiddenSlices only)
    int MT4;          // hidden-row tiles of 4 (M <= 4 * MT4 <= 32; 64 for the slice-major 8-row kernel)
    int U;            // K segments per pipeline stage: 128 elements at 4 rows, 64 at 8
    int nsg;          // stages per row group: nsg * U * seg >= K, seg = 128 or 64
    bool ragged;      // the stages run past K: clamp and zero the excess chunks
    int hidden;       // kHiddenLds, kHiddenL2 or kHiddenSlices
    int depth;        // kHiddenSlices: pipeline stages of weights in flight
    int order;        // 8 rows per wave: kOrderBlocks or kOrderSlices
    int grid;         // workgroups (persistent)
    int block;        // threads per workgroup (multiple of 64)
};

// Row strides in elements: row m of hidden at hidden + m*h, row j of gate_w
// at gate_w + j*g, of up_w at up_w + j*u, row m of out at out + m*o.  The
// fast kernels take h, g and u as multiples of 8 no larger than 2^25 (their
// lane offsets are 32-bit: byte counts over up to 32 rows, or counts of
// 16-byte chunks over the 64 rows of the slice-major 8-row kernel).
struct RowStrides {
    int64_t h, g, u, o;
};

// per-M instantiation tables (glu_valu_m<M>.hip)
using ValuFn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, int, int, RowStrides);
ValuFn valu_pick_1(int R, int U, int NB, bool ragged, bool diag);
ValuFn valu_pick_2(int R, int U, int NB, bool ragged);
ValuFn valu_pick_3(int R, int U, int NB, bool ragged);
ValuFn valu_pick_4(int R, int U, int NB, bool ragged);
ValuFn valu_pick_5(int R, int U, int NB, bool ragged);
ValuFn valu_pick_6(int R, int U, int NB, bool ragged);
ValuFn valu_pick_7(int R, int U, int NB, bool ragged);
ValuFn valu_pick_8(int R, int U, int NB, bool ragged);

// whether hidden is staged in LDS (else held in registers) for a VALU configuration
constexpr bool valu_hidden_in_lds(int M, int U, int NB) { return M * U * NB > 16; }

bool valu_supported(const ValuConfig& c);
hipError_t valu_launch(const ValuConfig& c, const uint16_t* hidden, const uint16_t* gate_w,
                       const uint16_t* up_w, uint16_t* out, int64_t N, int64_t K, RowStrides ld,
                       hipStream_t stream);

bool mfma_supported(const MfmaConfig& c);
size_t mfma_slice_lds_bytes(int mt4, int u);
// default weight stages the lockstep kernel keeps in flight for U segments per stage
int mfma_slice_depth(int u);
size_t mfma_hidden_lds_bytes(int m, int64_t k);
// the 8-row lockstep kernel (glu_mfma8.hip): mt8 hidden tiles of 8 rows
size_t mfma8_slice_lds_bytes(int mt8, int u);
int mfma8_slice_depth(int u);
// order: kOrderBlocks walks K per block of 4 groups in turn (mfma8_slice_kernel); kOrderSlices walks K
// once for all of a workgroup's blocks (mfma8_pass_kernel: depth 1, grid * kPassBlocks >= blocks; U == 8
// for mt8 2..4, U == 4 for mt8 5..8)
bool mfma8_supported(int mt8, int U, int depth, bool ragged, int block, int order);
int64_t mfma8_blocks(int64_t N);  // blocks of 4 groups of 8 weight rows
hipError_t mfma8_launch(int M, int U, int depth, int order, int nsg, bool ragged, int grid, const uint16_t* hidden,
                        const uint16_t* gate_w, const uint16_t* up_w, uint16_t* out, int64_t N, int64_t K,
                        RowStrides ld, hipStream_t stream);
hipError_t mfma_launch(const MfmaConfig& c, int M, const uint16_t* hidden, const uint16_t* gate_w,
                       const uint16_t* up_w, uint16_t* out, int64_t N, int64_t K, RowStrides ld,
                       hipStream_t stream);

// Streaming-read ceiling (glu_ceiling.hip): two [rows, U * 1024 bytes] matrices read
// as the VALU GEMV reads gate_w and up_w, R rows per group, U in 1..8, R in {1, 2, 4}.
bool read_ceiling_supported(int U, int R);
hipError_t read_ceiling_launch(const void* a, const void* b, int rows, int U, int R, int grid, int block,
                               bool xcd_bands, uint32_t* sink, hipStream_t stream);

// Any alignment (2-byte), any K >= 1, any strides; M <= 8 per launch.
hipError_t generic_launch(int M, const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w,
                          uint16_t* out, int64_t N, int64_t K, RowStrides ld, hipStream_t stream);

// out[m*ldo + j] = +0 for m < M, j < N (K == 0).
hipError_t zero_launch(uint16_t* out, int64_t M, int64_t N, int64_t ldo, hipStream_t stream);

// Tiled dual GEMM for large M (glu_gemm.hip): bn x bm output tiles (bn weight
// rows, bm hidden rows; each 64 or 128), K in stages of 64 elements.
struct GemmConfig {
    int bn;
    int bm;
    bool ktail;  // K % 64 != 0
    int depth;   // stages of global loads in flight (1 or 2)
};
size_t gemm_lds_bytes(int bn, int bm);
bool gemm_supported(const GemmConfig& c);
int64_t gemm_grid(const GemmConfig& c, int64_t M, int64_t N);
// K % 8 == 0, 16-byte aligned rows (fast layout); out rows may have any stride
hipError_t gemm_launch(const GemmConfig& c, int M, const uint16_t* hidden, const uint16_t* gate_w,
                       const uint16_t* up_w, uint16_t* out, int N, int K, const RowStrides& ld, hipStream_t stream);
// g = bf16(h Wg^T) into gu [M][N] and u = bf16(h Wu^T) into gu + M N: the same tiles (64 x 64) without
// the GLU epilogue, for the backward at M > 32.  Dense operands; N % 4 == 0, K % 8 == 0.  With dout
// ([M][N]) the backward's elementwise step runs in the epilogue: dg and du are stored instead.
hipError_t gemm_linear_launch(int M, const uint16_t* hidden, const uint16_t* gate_w, const uint16_t* up_w,
                              uint16_t* gu, int N, int K, const uint16_t* dout, hipStream_t stream);
// dWg = bf16(dgT hT^T) [N][K] and dWu likewise, contraction over mp (a multiple of 32) padded rows of
// hidden: hT [K][mp], dgT, duT [N][mp], all dense and 16-byte aligned, K % 8 == 0.
hipError_t gemm_dw_launch(int mp, const uint16_t* hT, const uint16_t* dgT, const uint16_t* duT, uint16_t* dwg,
                          uint16_t* dwu, int N, int K, hipStream_t stream);

}  // namespace glu
