// mfma_tile.h -- a (b, h) state tile held in registers in the operand layout of the fp32 matrix
// instruction v_mfma_f32_16x16x4_f32, and helpers for chains of that instruction (gfx950). Used by
// the Gated DeltaNet fold and the prefills.
//
// Operand layouts of the instruction, lane l: A[l % 16][l / 16]; B[l / 16][l % 16]; accumulator
// register r holds D[4 (l / 16) + r][l % 16]. Lane (g, c) = (l / 16, l % 16) of wave w keeps, for
// each of its i-blocks ib (16 rows of the ROWS x COLS tile, ib' = w IBW + ib) and each k-block kb
// (16 columns), the float4
//     S[16 ib' + c][16 kb + 4 g + r],  r = 0..3.
// Taking the inner index of step r of k-block kb to be 16 kb + 4 g + r, that float4 is the B
// operand of X S^T for any 16 x COLS operand X (rows of X on the A side), and the accumulator of
// Y^T Z for Y 16 x COLS and Z 16 x ROWS (the transpose of the rank-16 update S += Z^T Y), so the
// tile never leaves the registers.
#pragma once

#include "dev_common.h"

namespace rssm {

template <int ROWS, int COLS, int NWAVES = TileShape<ROWS, COLS>::TPB / 64>
struct MfmaTile {
    static constexpr int TPB = 64 * NWAVES, NW = NWAVES;
    static constexpr int IB = ROWS / 16, KB = COLS / 16, IBW = IB / NW;   // i-blocks per wave
    static constexpr int RS = ROWS + 4, CS = COLS + 4;   // padded LDS strides of ROWS / COLS rows
    static_assert(IBW >= 1 && IBW * NW == IB, "tile map");
};

// Element offset, inside a tile, of the float4 S[16 ib' + c][4 g] of thread t's i-block ib (add
// 16 kb for k-block kb).
template <int ROWS, int COLS, int NWAVES = TileShape<ROWS, COLS>::TPB / 64>
__device__ __forceinline__ int mfma_tile_offset(int t, int ib)
{
    using F = MfmaTile<ROWS, COLS, NWAVES>;
    const int w = t >> 6, l = t & 63;
    return (16 * (w * F::IBW + ib) + (l & 15)) * COLS + 4 * (l >> 4);
}

__device__ __forceinline__ v4f mfma4(float a, float b, v4f c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// The fp32 MFMA adds its four products to the accumulator in sequence, so a chain over a long
// inner dimension is a sequential sum. Long products keep NA independent chains over interleaved
// k-blocks and add them as a tree: shorter sequential sums, and independent work for the cores.
template <int NA>
__device__ __forceinline__ v4f tree_sum(const v4f (&p)[NA])
{
    if constexpr (NA == 1) return p[0];
    else if constexpr (NA == 2) return p[0] + p[1];
    else return (p[0] + p[1]) + (p[2] + p[3]);
}

// Wait states after an MFMA chain whose accumulators are next read on the far side of a branch
// (a loop back-edge or exit): 16, more than an 8-pass 16x16x4 f32 result needs, with scheduling
// barriers that keep the chain ahead of them.
__device__ __forceinline__ void mfma_settle()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Completes the loads of a register tile before a loop that keeps it: an empty statement that
// reads every element, so the wait for those loads sits here. Left in flight at the loop entry,
// they would make each iteration wait for every memory operation issued before its first use of
// the tile, the prefetch of the next iteration's inputs among them.
template <int IBW, int KB>
__device__ __forceinline__ void tile_loaded(const float4 (&s)[IBW][KB])
{
#pragma unroll
    for (int ib = 0; ib < IBW; ++ib)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            asm volatile("" ::"v"(s[ib][kb].x), "v"(s[ib][kb].y), "v"(s[ib][kb].z), "v"(s[ib][kb].w));
}

}  // namespace rssm
