// Operand types and helpers shared by the MFMA kernels.
#pragma once

#include <type_traits>

#include "glu_launch.h"

namespace glu {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// D = A * B + C for one 16x16x32 bf16 tile: lane l supplies A[l%16][8(l/16)..+7]
// and B[8(l/16)..+7][l%16] as 8 bf16 each, and holds D[4(l/16)+e][l%16], e < 4
__device__ __forceinline__ f32x4_t mfma16(const u32x4_t& a, const u32x4_t& b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// LDS reads of the hidden operand.  A ds_read_b128 is served in groups of 16
// lanes from 64 four-byte banks (256 bytes): within each half-wave, the 4-lane quads
// whose index l/4 has even bit parity form one group and the odd ones the
// other ({0-3, 12-15, 20-23, 24-27} and {4-7, 8-11, 16-19, 28-31}), and a
// group reads without conflict when its 16 lanes touch 16 different 16-byte
// slots of 256 bytes (measured on gfx950 with SQ_LDS_BANK_CONFLICT).  Rows of
// hidden in LDS start on a 256-byte boundary and chunk c of row r is stored at
// c ^ swz(r); these XOR masks make the operand reads of the block-diagonal
// layouts conflict-free (4 weight rows x 4 blocks, 8 rows x 2 blocks).  The
// row's chunk count must be a multiple of 4, resp. 16.
__device__ __forceinline__ int lds_swz4(int r) { return r & 2; }
__device__ __forceinline__ int lds_swz8(int r) { return (r & 3) | ((r & 4) << 1); }

// calls f(integral_constant<Q>, s0 + Q) for Q = Q0 .. L-1 while s0 + Q < n
template <int Q, int L, class F>
__device__ __forceinline__ void run_stages(F& f, int s0, int n)
{
    if constexpr (Q < L) {
        if (s0 + Q < n) {
            f(std::integral_constant<int, Q>{}, s0 + Q);
            run_stages<Q + 1, L>(f, s0, n);
        }
    }
}

// calls f(integral_constant<Q>) for Q = Q0 .. L-1
template <int Q, int L, class F>
__device__ __forceinline__ void for_positions(F& f)
{
    if constexpr (Q < L) {
        f(std::integral_constant<int, Q>{});
        for_positions<Q + 1, L>(f);
    }
}

}  // namespace glu
