// gdn_layout.h -- the layout of a Gated DeltaNet checkpoint tile in device memory (gfx950).
//
// A d_v x d_k tile S is stored in the operand layout of mfma_tile.h, k-block by k-block: with
// IB = d_v / 16 row blocks, float4 number (kb IB + ib) 64 + 16 g + c holds
// S[16 ib + c][16 kb + 4 g .. 4 g + 3]. The wave that keeps row block ib in registers (lane
// (g, c) = 16 g + c) reads or writes each of its k-blocks as 1 KB contiguous, and at each k-block
// the waves of a workgroup touch neighbouring kilobytes (8 KB contiguous for a 128-row tile in 8
// waves). Row-major tiles give 16 rows x 64 bytes per instruction instead; ordering the blocks
// row block by row block (each wave's 8 KB contiguous, waves 8 KB apart at each step) made the
// replay launch 11 % slower than k-block order in a same-box comparison. The layout is internal:
// the state goes in and out row-major through rssm_init_checkpoint and rssm_materialize, and
// per-sequence copies move the tile as bytes.
#pragma once

#include <stddef.h>

#include "dev_common.h"

namespace rssm {

// Float offset, inside a tile with dv rows, of element (i, k).
__host__ __device__ __forceinline__ size_t ckpt_offset(int i, int k, int dv)
{
    const int ibs = dv >> 4;
    return ((size_t)((k >> 4) * ibs + (i >> 4)) * 64 + ((k & 15) >> 2) * 16 + (i & 15)) * 4 + (k & 3);
}

// Thread t's float4s of a tile held in the operand layout by waves of IBW 16-row blocks each (wave
// w holds row blocks w IBW .. w IBW + IBW - 1): a 32-bit offset per thread, then one base per
// k-block (the k-blocks lie IB KB apart, beyond the instruction's immediate offset). Each base is
// formed where it is used; bases computed early and held across the kernel would cost registers.
template <int IBW>
__device__ __forceinline__ int ckpt_thread_offset(int t)
{
    return (t >> 6) * (IBW * 256) + (t & 63) * 4;
}

template <int DV, int IBW, int KB>
__device__ __forceinline__ void ckpt_load(float4 (&s)[IBW][KB], const float *tile, int t)
{
    constexpr int IB = DV / 16;
    const int o = ckpt_thread_offset<IBW>(t);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        int ob = o + kb * IB * 256;
        if (kb > 0) asm volatile("" : "+v"(ob));
#pragma unroll
        for (int ib = 0; ib < IBW; ++ib) s[ib][kb] = ld4_nt(tile + ob + ib * 256);
    }
}

template <int DV, int IBW, int KB>
__device__ __forceinline__ void ckpt_store(const float4 (&s)[IBW][KB], float *tile, int t)
{
    constexpr int IB = DV / 16;
    asm volatile("" : "+v"(t));         // the offset is recomputed here, not kept from the load
    const int o = ckpt_thread_offset<IBW>(t);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        int ob = o + kb * IB * 256;
        asm volatile("" : "+v"(ob));
#pragma unroll
        for (int ib = 0; ib < IBW; ++ib) st4_nt(tile + ob + ib * 256, s[ib][kb]);
    }
}

}  // namespace rssm
