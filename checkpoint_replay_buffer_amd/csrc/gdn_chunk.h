// gdn_chunk.h -- blocks of a run of up to 32 Gated DeltaNet entries taken at once, shared by the
// chunked prefill and the speculative verify (gfx950).
//
// For entries t = 0..n-1 (key k_t, value v_t, beta_t, alpha_t) with Gram entries G_it = k_i . k_t,
// the lower-triangular T of the WY form of the delta rule solves y = T K for
// y_t = beta_t (k_t - sum_{i<t} G_it y_i):
//     T[t][t] = beta_t,   T[t][q] = -beta_t sum_{q<=i<t} G_it T[i][q],
// and the decay ratios are R[t][q] = prod_{q<i<=t} alpha_i, Gam_t = prod_{i<=t} alpha_i (the gated
// delta rule of the Gated DeltaNet layer, one of the layer types ReplaySSM targets, news.hamidun.com
// item "NVIDIA présente ReplaySSM...", section "Pourquoi les hybrides sont devenus la norme").
// T of the first m entries is the leading m x m block of T, which is what lets one T serve every
// prefix of the run.
#pragma once

#include "dev_common.h"
#include "mfma_tile.h"

namespace rssm {

constexpr int kChunk = 16;
constexpr int kTS = kChunk + 4;   // row stride of the 16 x 16 blocks in LDS

// 16 x 16 dot products of the rows of two 16-row LDS blocks x and y (16 KB columns, row stride RS)
// on the matrix cores: lane (g, c) ends with x_{4 g + r} . y_c in register r. With SELF, x = y and
// each float4 serves as both operands. NA independent chains over interleaved k-blocks, summed as
// a tree.
template <int KB, int RS, int NA, bool SELF>
__device__ __forceinline__ v4f row_dots16(const float *x, const float *y)
{
    const int lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
    v4f p[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) p[a] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const float4 xv = ld4(x + cl * RS + 16 * kb + 4 * g);                 // A: x_c[k]
        const float4 yv = SELF ? xv : ld4(y + cl * RS + 16 * kb + 4 * g);     // B: y_c[k]
        v4f &d = p[kb % NA];
        d = mfma4(xv.x, yv.x, d);
        d = mfma4(xv.y, yv.y, d);
        d = mfma4(xv.z, yv.z, d);
        d = mfma4(xv.w, yv.w, d);
    }
    return tree_sum<NA>(p);
}

// T by forward substitution over NP entries (a power of two, at most 64), one column per lane
// (q = lane % NP) held in registers; the Gram rows (G[t][i] at sh_G[t GS + i], i < t) and the betas
// are read at addresses common to the wave. Rows with beta = 0 (padding) come out zero. The
// substitution and the store are separate steps, so that a caller can place other work between
// them in the same straight-line code. A caller inside a loop may pass the lane's column q through
// an empty asm statement, so that the identity's selectors are formed here and not kept in
// registers across the loop.
template <int NP, int GS>
__device__ __forceinline__ void t_solve_cols(const float *sh_G, const float *sh_be, float (&tq)[NP],
                                             int q = threadIdx.x & (NP - 1))
{
#pragma unroll
    for (int t = 0; t < NP; ++t) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < t; ++i) acc = fmaf(sh_G[t * GS + i], tq[i], acc);
        tq[t] = sh_be[t] * ((t == q ? 1.f : 0.f) - acc);
    }
}

template <int NP, int TS>
__device__ __forceinline__ void t_store_cols(const float (&tq)[NP], float *sh_T)
{
    const int lane = threadIdx.x & 63, q = lane & (NP - 1);
    if (lane < NP) {
#pragma unroll
        for (int t = 0; t < NP; ++t) sh_T[t * TS + q] = tq[t];
    }
}

template <int NP, int GS, int TS>
__device__ __forceinline__ void t_solve_regs(const float *sh_G, const float *sh_be, float *sh_T)
{
    float tq[NP];
    t_solve_cols<NP, GS>(sh_G, sh_be, tq);
    t_store_cols<NP, TS>(tq, sh_T);
}

// Decay row of lane l < 16 for entries 0..p applied (p < NP): R[l][q] = prod_{q<i<=p} alpha_i for
// q < NP (1 for q >= p), a running product from q = NP - 1 down, and Gam[l] = prod_{i<=p} alpha_i.
template <int NP, int RS>
__device__ __forceinline__ void decay_row(const float *sh_al, int p, float *sh_R, float *sh_gam)
{
    const int l = threadIdx.x & 63;
    float al[NP];
#pragma unroll
    for (int i = 0; i < NP; i += 4) {
        const float4 x = ld4(sh_al + i);
        al[i] = x.x; al[i + 1] = x.y; al[i + 2] = x.z; al[i + 3] = x.w;
    }
    float pr = 1.f, row[NP];
#pragma unroll
    for (int q = NP - 1; q >= 0; --q) {
        if (q < NP - 1 && q + 1 <= p) pr *= al[q + 1];
        row[q] = pr;
    }
    if (l < kChunk) {
#pragma unroll
        for (int q = 0; q < NP; q += 4) st4(sh_R + l * RS + q, make_float4(row[q], row[q + 1], row[q + 2], row[q + 3]));
        sh_gam[l] = pr * al[0];
    }
}

}  // namespace rssm
