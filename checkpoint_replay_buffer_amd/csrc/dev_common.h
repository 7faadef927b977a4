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

// Sum over the LANES consecutive lanes of an aligned lane group (xor butterfly).
template <int LANES>
__device__ __forceinline__ float group_sum(float s)
{
#pragma unroll
    for (int st = 0; st < ilog2(LANES); ++st) s += __shfl_xor(s, LANES >> (st + 1));
    return s;
}

// Row sums of an R-row partial-dot block spread over LPR lanes: a reduce-scatter butterfly.
// Each of the first log2(R) exchange steps halves the number of rows a lane keeps; the rest are
// plain sums. On return every lane holds the full sum of row `rsel` (an index in 0..R-1), and
// the LPR/R lanes with equal (cg & ~(LPR/R - 1)) hold the same row.
template <int R, int LPR>
__device__ __forceinline__ float row_reduce_scatter(float (&v)[R], int cg, int &rsel)
{
    int base = 0;
#pragma unroll
    for (int st = 0; st < ilog2(R); ++st) {
        const int c = R >> st;            // rows still held
        const int X = LPR >> (st + 1);    // partner distance
        const bool up = (cg & X) != 0;
#pragma unroll
        for (int i = 0; i < c / 2; ++i) {
            // The empty asm makes lo / hi opaque register values, so the lane-dependent choice
            // below stays a select instead of becoming a dynamic index into v (which would push
            // the array to scratch memory).
            float lo = v[i], hi = v[i + c / 2];
            asm volatile("" : "+v"(lo), "+v"(hi));
            const float send = up ? lo : hi;
            const float keep = up ? hi : lo;
            v[i] = keep + __shfl_xor(send, X);
        }
        base += up ? c / 2 : 0;
    }
    float s = v[0];
#pragma unroll
    for (int st = ilog2(R); st < ilog2(LPR); ++st) s += __shfl_xor(s, LPR >> (st + 1));
    rsel = base;
    return s;
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

__device__ __forceinline__ float f4get(const float4 &v, int e)
{
    return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}

}  // namespace rssm
