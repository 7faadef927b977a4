// dev_common.h -- device helpers shared by the librssm kernels (gfx950, wave64).
//
// A state tile is one (sequence, head) matrix [P x N] fp32, row-major. A workgroup owns one tile.
// Lanes own EPL consecutive columns of R consecutive rows, so every global load is 16 bytes
// (8 bytes for the bf16 copy of the smallest tiles) and the LPR lanes of one row read a
// contiguous run of the row: loads are fully coalesced along the fastest dimension.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rssm {

// Threads per workgroup for a P x N tile: about 8 float4 per thread, 64..512 threads.
template <int P, int N>
struct TileShape {
    static constexpr int NF4 = P * N / 4;
    static constexpr int TPB = NF4 / 8 < 64 ? 64 : (NF4 / 8 > 512 ? 512 : NF4 / 8);
};

// Lane <-> element map of a P x N tile read EPL columns per lane.
template <int P, int N, int TPB, int EPL>
struct RowMap {
    static constexpr int LPR = N / EPL;     // lanes per row (a power of two, <= 64)
    static constexpr int RG = TPB / LPR;    // row groups
    static constexpr int R = P / RG;        // consecutive rows per lane
    static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "lanes per row");
    static_assert(RG * LPR == TPB && R * RG == P && R >= 1 && R <= LPR, "tile map");
};

// The fp32 map (16-byte loads of 4 columns) of a tile's workgroup.
template <int P, int N>
using Map4 = RowMap<P, N, TileShape<P, N>::TPB, 4>;

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// Value of the butterfly partner at distance X (a power of two <= 16) within aligned groups of 2X
// lanes. Distances 1 and 2 are xor partners (DPP quad permutes); 4 and 8 use the DPP mirrors
// inside 8- and 16-lane rows (lane i <-> 7 - i, 15 - i), whose partner differs from i in bit
// log2(X) and in the bits below it; 16 is an xor swizzle within 32-lane groups. For the sums
// and reduce-scatters below this is as good as a plain xor: each step merges two disjoint lane
// sets that agree on every bit above X, and the steps together reach all lanes of the group.
// Every lane of the group must be active. DPP = false uses plain shuffles through the LDS
// crossbar instead, which is faster where the VALU is the busier unit (the read-modify-write
// comparators, measured).
template <int X, bool DPP = true>
__device__ __forceinline__ float bfly(float v)
{
    const int i = __float_as_int(v);
    int r;
    if constexpr (!DPP) r = __shfl_xor(i, X);
    else if constexpr (X == 1) r = __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true);       // [1,0,3,2]
    else if constexpr (X == 2) r = __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true);  // [2,3,0,1]
    else if constexpr (X == 4) r = __builtin_amdgcn_mov_dpp(i, 0x141, 0xF, 0xF, true); // half-row mirror
    else if constexpr (X == 8) r = __builtin_amdgcn_mov_dpp(i, 0x140, 0xF, 0xF, true); // row mirror
    else if constexpr (X == 16) r = __builtin_amdgcn_ds_swizzle(i, 0x401F);            // xor 16
    else r = __shfl_xor(i, X);
    return __int_as_float(r);
}

// Sum over the LANES consecutive lanes of an aligned lane group (butterfly).
template <int LANES, bool DPP = true>
__device__ __forceinline__ float group_sum(float s)
{
    if constexpr (LANES >= 32) s += bfly<16, DPP>(s);
    if constexpr (LANES >= 16) s += bfly<8, DPP>(s);
    if constexpr (LANES >= 8) s += bfly<4, DPP>(s);
    if constexpr (LANES >= 4) s += bfly<2, DPP>(s);
    if constexpr (LANES >= 2) s += bfly<1, DPP>(s);
    static_assert(LANES <= 32, "lane groups up to 32");
    return s;
}

// One halving step of the reduce-scatter below: a lane holding C row partials keeps half of them
// (the upper half when bit X of its column index is set) and adds the partner's values for that
// half. Recurses down to one row per lane.
template <int C, int X, int R, bool DPP>
__device__ __forceinline__ void rs_halve(float (&v)[R], int cg, int &base)
{
    if constexpr (C > 1) {
        const bool up = (cg & X) != 0;
#pragma unroll
        for (int i = 0; i < C / 2; ++i) {
            // The empty asm makes lo / hi opaque register values, so the lane-dependent choice
            // below stays a select instead of becoming a dynamic index into v (which would push
            // the array to scratch memory).
            float lo = v[i], hi = v[i + C / 2];
            asm volatile("" : "+v"(lo), "+v"(hi));
            const float send = up ? lo : hi;
            const float keep = up ? hi : lo;
            v[i] = keep + bfly<X, DPP>(send);
        }
        base += up ? C / 2 : 0;
        rs_halve<C / 2, X / 2, R, DPP>(v, cg, base);
    }
}

template <int X, bool DPP>
__device__ __forceinline__ float sum_down(float s)
{
    if constexpr (X >= 1) return sum_down<X / 2, DPP>(s + bfly<X, DPP>(s));
    else return s;
}

// Row sums of an R-row partial-dot block spread over LPR lanes: a reduce-scatter butterfly.
// Each of the first log2(R) exchange steps halves the number of rows a lane keeps; the rest are
// plain sums. On return every lane holds the full sum of row `rsel` (an index in 0..R-1), and
// the LPR/R lanes with equal (cg & ~(LPR/R - 1)) hold the same row.
template <int R, int LPR, bool DPP = true>
__device__ __forceinline__ float row_reduce_scatter(float (&v)[R], int cg, int &rsel)
{
    static_assert(LPR <= 32 && R <= LPR, "row map");
    int base = 0;
    rs_halve<R, LPR / 2, R, DPP>(v, cg, base);
    rsel = base;
    return sum_down<LPR / (2 * R), DPP>(v[0]);
}

// The one lane of each duplicate set that writes the row result.
template <int R, int LPR>
__device__ __forceinline__ bool row_writer(int cg) { return (cg & (LPR / R - 1)) == 0; }

// fp32 -> bf16, round to nearest even (finite values).
__device__ __forceinline__ uint32_t bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return bf16_bits(lo) | (bf16_bits(hi) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ void st4(float *p, float4 v) { *reinterpret_cast<float4 *>(p) = v; }

// Streaming (non-temporal) loads/stores for data touched once per launch. The builtins take
// clang vector types.
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float4 ld4_nt(const float *p)
{
    const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st4_nt(float *p, float4 v)
{
    const v4f w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<v4f *>(p));
}
__device__ __forceinline__ uint4 ldu4_nt(const void *p)
{
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ldu2_nt(const void *p)
{
    const v2u v = __builtin_nontemporal_load(reinterpret_cast<const v2u *>(p));
    return make_uint2(v.x, v.y);
}

}  // namespace rssm
