// gdn_prefill.hip -- Gated DeltaNet prefill into the checkpoint, on the matrix cores (gfx950).
//
// A prompt of T tokens runs through S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
// o_t = S_t q_t, and its final state becomes the checkpoint with an empty ring (the persistent
// state the decode path starts from; Gated DeltaNet is one of the layer types ReplaySSM targets,
// news.hamidun.com item "NVIDIA présente ReplaySSM...", section "Pourquoi les hybrides sont
// devenus la norme"). Every prompt token's output is written.
//
// Chunks of 16 tokens. With S the state at the chunk start, G_it = k_i . k_t, the lower-triangular
// T of the WY fold (T[t][t] = beta_t, T[t][q] = -beta_t sum_{q<=i<t} G_it T[i][q]), the decay
// ratios R[t][q] = prod_{q<i<=t} alpha_i and Gam_t = prod_{i<=t} alpha_i, the fold formula applied
// to every prefix of the chunk gives, for A[t][t'] = q_t . k_t' (t' <= t, else 0) and U = A T,
//     O = Gam o (Q S^T - U F) + (U o R) V,        F = K S^T   (F[q] = S k_q),
// and at the end of the chunk (the fold of all 16 entries)
//     S <- gam S + C^T K,   C = T Z,   Z_q = R[15][q] v_q - gam F_q,   gam = Gam_15;
// every decay factor is at most 1. K S^T, Q S^T, K K^T, Q K^T, U, U F, (U o R) V, T Z and the
// rank-16 update are v_mfma_f32_16x16x4_f32 chains on the register-resident tile of mfma_tile.h.
#include "dev_common.h"
#include "internal.h"
#include "gdn_chunk.h"
#include "gdn_layout.h"
#include "mfma_tile.h"

namespace rssm {
namespace {

// LDS floats: two staging buffers (q and k [16][d_k+4], v [16][d_v+4], beta and alpha [16]),
// then the Gram, T, A and R blocks [16][20] and Gam [16] of the current chunk
template <int DV, int DK>
__host__ __device__ constexpr int gp_buf_floats()
{
    return kChunk * (2 * (DK + 4) + (DV + 4)) + 2 * kChunk;
}
template <int DV, int DK>
__host__ __device__ constexpr int gp_lds_floats()
{
    return 2 * gp_buf_floats<DV, DK>() + 4 * kChunk * kTS + kChunk;
}

// Waves per (b, h) workgroup: 4 for 128 x 128 (two i-blocks per wave, so that two workgroups share
// a compute unit and fill each other's barriers), else the tile's usual count.
template <int DV, int DK>
struct GpShape {
    static constexpr int NW = DV * DK >= 128 * 128 ? 4 : TileShape<DV, DK>::TPB / 64;
    static constexpr int TPB = 64 * NW;
};

// The chunk's q, k, v rows and beta, alpha held in registers between their load and their LDS
// store; the lane-dependent part of each address is computed once per prompt.
template <int DV, int DK>
struct GdnRows {
    static constexpr int TPB = GpShape<DV, DK>::TPB, KF = DK / 4, VF = DV / 4;
    static constexpr int KQ = (kChunk * KF + TPB - 1) / TPB, VQ = (kChunk * VF + TPB - 1) / TPB;
    float4 q[KQ], k[KQ], v[VQ];
    float be, al;
    size_t ko[KQ], vo[VQ];
    int kj[KQ], vj[VQ];

    __device__ __forceinline__ void init(size_t BH, int t)
    {
#pragma unroll
        for (int i = 0; i < KQ; ++i) {
            const int u = t + i * TPB, j = u / KF, o = (u - j * KF) * 4;
            kj[i] = u < kChunk * KF ? j : kChunk;
            ko[i] = (size_t)j * BH * DK + o;
        }
#pragma unroll
        for (int i = 0; i < VQ; ++i) {
            const int u = t + i * TPB, j = u / VF, o = (u - j * VF) * 4;
            vj[i] = u < kChunk * VF ? j : kChunk;
            vo[i] = (size_t)j * BH * DV + o;
        }
    }

    // tokens t0 .. t0 + ct - 1; the pointers are at token t0's row of this tile
    __device__ __forceinline__ void load(const float *qb, const float *kb, const float *vb,
                                         const float *bb, const float *ab, size_t BH, int ct, int t)
    {
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < KQ; ++i) {
            q[i] = kj[i] < ct ? ld4(qb + ko[i]) : z;
            k[i] = kj[i] < ct ? ld4(kb + ko[i]) : z;
        }
#pragma unroll
        for (int i = 0; i < VQ; ++i) v[i] = vj[i] < ct ? ld4(vb + vo[i]) : z;
        be = t < ct ? bb[(size_t)t * BH] : 0.f;        // padding rows: beta 0, alpha 1
        al = t < ct ? ab[(size_t)t * BH] : 1.f;
    }

    __device__ __forceinline__ void store(float *sh_q, float *sh_k, float *sh_v, float *sh_be,
                                          float *sh_al, int t) const
    {
        constexpr int KS = DK + 4, VS = DV + 4;
#pragma unroll
        for (int i = 0; i < KQ; ++i) {
            const int u = t + i * TPB, j = u / KF, o = (u - j * KF) * 4;
            if (KQ * TPB == kChunk * KF || u < kChunk * KF) {
                st4(sh_q + j * KS + o, q[i]);
                st4(sh_k + j * KS + o, k[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < VQ; ++i) {
            const int u = t + i * TPB, j = u / VF, o = (u - j * VF) * 4;
            if (VQ * TPB == kChunk * VF || u < kChunk * VF) st4(sh_v + j * VS + o, v[i]);
        }
        if (t < kChunk) {
            sh_be[t] = be;
            sh_al[t] = al;
        }
    }
};

// NARROW: 16 token rows of the outputs span less than 4 GiB, so a chunk's output stores go
// through a buffer resource whose record range ends after the chunk's last real row: the stores of
// padding rows fall outside it and are dropped, and every store issues unpredicated (a predicated
// store leaves the compiler without a count of the stores in flight, and its wait for the next
// chunk's rows then covers those stores too).
template <int DV, int DK, bool NARROW>
__global__ void __launch_bounds__((GpShape<DV, DK>::TPB), 2) k_gdn_prefill(GdnPrefillArgs a)
{
    using F = MfmaTile<DV, DK, GpShape<DV, DK>::NW>;
    constexpr int NW = F::NW, IBW = F::IBW, KB = F::KB, KS = F::CS, VS = F::RS;
    constexpr int NA = KB >= 2 ? 2 : KB;   // independent accumulators of the d_k products
                                           // (two: wave 0 keeps its T column registers beside them)
    constexpr int BUF = gp_buf_floats<DV, DK>();
    extern __shared__ float smem[];
    float *sh_G = smem + 2 * BUF;          // [16][kTS]  k_i . k_t
    float *sh_T = sh_G + kChunk * kTS;     // [16][kTS]  T
    float *sh_A = sh_T + kChunk * kTS;     // [16][kTS]  q_t . k_t' for t' <= t, else 0
    float *sh_R = sh_A + kChunk * kTS;     // [16][kTS]  R[t][q]
    float *sh_gam = sh_R + kChunk * kTS;   // [16]       Gam_t

    const int B = a.d.B, H = a.d.H, T = a.T;
    const int tile = blockIdx.x, b = tile / H, h = tile - b * H;
    const size_t bh = (size_t)tile, BH = (size_t)B * H;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6, g = lane >> 4, cl = lane & 15;

    const float *q0 = a.q + bh * DK, *k0 = a.k + bh * DK, *v0 = a.v + bh * DV;
    const float *b0 = a.beta + bh, *a0 = a.alpha + bh;
    float *o0 = a.o + bh * DV;
    GdnRows<DV, DK> rows;
    rows.init(BH, t);
    rows.load(q0, k0, v0, b0, a0, BH, T < kChunk ? T : kChunk, t);
    float4 s[IBW][KB];
    float *S0 = a.S0 + bh * (size_t)(DV * DK);
    ckpt_load<DV>(s, S0, t);
    tile_loaded(s);

    int buf = 0;
    for (int t0 = 0; t0 < T; t0 += kChunk, buf ^= 1) {
        const int ct = T - t0 < kChunk ? T - t0 : kChunk;
        float *sh_q = smem + buf * BUF;
        float *sh_k = sh_q + kChunk * KS;
        float *sh_v = sh_k + kChunk * KS;
        float *sh_be = sh_v + kChunk * VS;
        float *sh_al = sh_be + kChunk;
        rows.store(sh_q, sh_k, sh_v, sh_be, sh_al, t);
        __syncthreads();
        if (t0 + kChunk < T) {             // the next chunk's rows, in flight during this chunk
            const size_t t1 = t0 + kChunk;
            rows.load(q0 + t1 * BH * DK, k0 + t1 * BH * DK, v0 + t1 * BH * DV, b0 + t1 * BH,
                      a0 + t1 * BH, BH, T - (int)t1 < kChunk ? T - (int)t1 : kChunk, t);
        }

        // 1. the chunk's S-independent blocks first, so that their latency overlaps the other
        //    waves' matrix work: wave 0 the Gram block and T, wave 1 the masked Q K^T, the last
        //    wave the decays (one wave does all three when it is alone); then every wave
        //    F = K S^T and Qs = Q S^T for its i-blocks (S at the chunk start). Wave 0's forward
        //    substitution sits in the same straight-line code as its products, so that its LDS
        //    waits interleave with the matrix-core chains; its store of T comes after them.
        v4f fz[IBW], qs[IBW];
        auto products = [&]() {
#pragma unroll
            for (int ib = 0; ib < IBW; ++ib) {
                v4f fp[NA], qp[NA];
#pragma unroll
                for (int p = 0; p < NA; ++p) fp[p] = qp[p] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const float4 kv = ld4(sh_k + cl * KS + 16 * kb + 4 * g);
                    const float4 qv = ld4(sh_q + cl * KS + 16 * kb + 4 * g);
                    v4f &f = fp[kb % NA], &x = qp[kb % NA];
                    f = mfma4(kv.x, s[ib][kb].x, f);
                    f = mfma4(kv.y, s[ib][kb].y, f);
                    f = mfma4(kv.z, s[ib][kb].z, f);
                    f = mfma4(kv.w, s[ib][kb].w, f);
                    x = mfma4(qv.x, s[ib][kb].x, x);
                    x = mfma4(qv.y, s[ib][kb].y, x);
                    x = mfma4(qv.z, s[ib][kb].z, x);
                    x = mfma4(qv.w, s[ib][kb].w, x);
                }
                fz[ib] = tree_sum<NA>(fp);     // (S k_q)[i] for q = 4 g + r, i = 16 ib' + c
                qs[ib] = tree_sum<NA>(qp);     // (S q_t)[i] for t = 4 g + r
            }
        };
        auto q_kt = [&]() {
            const v4f qk = row_dots16<KB, KS, NA, false>(sh_q, sh_k);     // q_{4g+r} . k_c
#pragma unroll
            for (int r = 0; r < 4; ++r) sh_A[(4 * g + r) * kTS + cl] = cl <= 4 * g + r ? qk[r] : 0.f;
        };
        if (wv == 0) {
            if constexpr (NW == 1) {
                q_kt();
                decay_row<kChunk, kTS>(sh_al, lane, sh_R, sh_gam);
            }
            const v4f gk = row_dots16<KB, KS, NA, true>(sh_k, sh_k);      // k_{4g+r} . k_c
#pragma unroll
            for (int r = 0; r < 4; ++r) sh_G[(4 * g + r) * kTS + cl] = gk[r];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            float tq[kChunk];
            t_solve_cols<kChunk, kTS>(sh_G, sh_be, tq);
            products();
            t_store_cols<kChunk, kTS>(tq, sh_T);
        } else {
            if (wv == 1) q_kt();
            if (wv == NW - 1) decay_row<kChunk, kTS>(sh_al, lane, sh_R, sh_gam);
            products();
        }
        mfma_settle();
        __syncthreads();

        // 2. decays per lane: R[t = c][q = 4 g + r], Gam of the output rows t = 4 g + r, the fold's
        //    R[15][q = 4 g + r] and gam
        const float4 rr = ld4(sh_R + cl * kTS + 4 * g), gm = ld4(sh_gam + 4 * g);
        const float4 rf = ld4(sh_R + (kChunk - 1) * kTS + 4 * g);
        const float gam = sh_gam[kChunk - 1];

        // 3. U = A T, as U^T = T^T A^T so that lane (g, c) ends with U[t = c][q = 4 g + r], the A
        //    operand of U F
        v4f ut = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r)
            ut = mfma4(sh_T[(4 * g + r) * kTS + cl], sh_A[cl * kTS + 4 * g + r], ut);
        const float ua[4] = {ut[0], ut[1], ut[2], ut[3]};
        // the chunk's output rows; records end after row ct - 1 of this tile
        const __amdgpu_buffer_rsrc_t orows = __builtin_amdgcn_make_buffer_rsrc(
            o0 + (size_t)t0 * BH * DV, 0,
            NARROW ? (int)(((uint32_t)(ct - 1) * (uint32_t)(BH * DV) + (uint32_t)DV) * 4u) : 0,
            0x00020000);
        const float ur[4] = {ut[0] * rr.x, ut[1] * rr.y, ut[2] * rr.z, ut[3] * rr.w};
        const float gmv[4] = {gm.x, gm.y, gm.z, gm.w}, rfv[4] = {rf.x, rf.y, rf.z, rf.w};

#pragma unroll
        for (int ib = 0; ib < IBW; ++ib) {
            const int i = 16 * (wv * IBW + ib) + cl;
            float vq[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) vq[r] = sh_v[(4 * g + r) * VS + i];   // V[q = 4 g + r][i]
            // 4. outputs O = Gam o (Q S^T - U F) + (U o R) V
            v4f uf = {0.f, 0.f, 0.f, 0.f}, uv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uf = mfma4(ua[r], fz[ib][r], uf);
                uv = mfma4(ur[r], vq[r], uv);
            }
            float ov[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ov[r] = gmv[r] * (qs[ib][r] - uf[r]) + uv[r];
            // keep these reads next to their chains rather than sunk into the stores below
            asm volatile("" ::"v"(ov[0]), "v"(ov[1]), "v"(ov[2]), "v"(ov[3]));
            if constexpr (NARROW) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    __builtin_amdgcn_raw_buffer_store_b32(
                        __float_as_uint(ov[r]), orows,
                        (int)(((uint32_t)(4 * g + r) * (uint32_t)(BH * DV) + (uint32_t)i) * 4u), 0, 0);
            } else {
                float *oc = o0 + (size_t)t0 * BH * DV + i;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * g + r < ct) oc[(size_t)(4 * g + r) * BH * DV] = ov[r];
            }
            // 5. fold of the chunk: Z = R[15] o V - gam F, C = T Z, S <- gam S + C^T K
            float zf[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) zf[r] = rfv[r] * vq[r] - gam * fz[ib][r];
            const float4 tv = ld4(sh_T + cl * kTS + 4 * g);                  // T[t = c][4 g + r]
            v4f cz = {0.f, 0.f, 0.f, 0.f};
            cz = mfma4(tv.x, zf[0], cz);
            cz = mfma4(tv.y, zf[1], cz);
            cz = mfma4(tv.z, zf[2], cz);
            cz = mfma4(tv.w, zf[3], cz);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                v4f u = {gam * s[ib][kb].x, gam * s[ib][kb].y, gam * s[ib][kb].z, gam * s[ib][kb].w};
                const float *kr = sh_k + (4 * g) * KS + 16 * kb + cl;          // K[t][16 kb + c]
                u = mfma4(kr[0], cz[0], u);
                u = mfma4(kr[KS], cz[1], u);
                u = mfma4(kr[2 * KS], cz[2], u);
                u = mfma4(kr[3 * KS], cz[3], u);
                s[ib][kb] = make_float4(u[0], u[1], u[2], u[3]);
            }
        }
        mfma_settle();
    }

    // the final state is the new checkpoint; the ring is empty
    ckpt_store<DV>(s, S0, t);
    if (h == 0 && t == 0) {
        a.bk.out[b] = a.bk.in[b];
        a.bk.out[B + b] = 0;
        a.bk.out[2 * B + b] = 0;
    }
}

template <int DV, int DK>
hipError_t go_gdn_prefill(const GdnPrefillArgs &a, hipStream_t s)
{
    const dim3 grid(a.d.B * a.d.H), block(GpShape<DV, DK>::TPB);
    const size_t lds = 4 * (size_t)gp_lds_floats<DV, DK>();
    // 16 token rows of the outputs within 4 GiB: unpredicated output stores
    if ((size_t)a.d.B * a.d.H * DV * 4 * kChunk <= 0xFFFFFFFFull)
        hipLaunchKernelGGL((k_gdn_prefill<DV, DK, true>), grid, block, lds, s, a);
    else
        hipLaunchKernelGGL((k_gdn_prefill<DV, DK, false>), grid, block, lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t gdn_prefill(const GdnPrefillArgs &a, hipStream_t s)
{
#define RSSM_C(v, k) if (a.d.DV == v && a.d.DK == k) return go_gdn_prefill<v, k>(a, s);
    RSSM_C(16, 16) RSSM_C(64, 64) RSSM_C(128, 128)
#undef RSSM_C
    return hipErrorInvalidValue;
}

}  // namespace rssm
