// kda_prefill.hip -- Kimi Delta Attention prefill into the checkpoint, in chunks of 16 tokens on
// the matrix cores (gfx950).
//
// Kimi Delta Attention is one of the layer types ReplaySSM targets (news.hamidun.com item "NVIDIA
// présente ReplaySSM...", section "Pourquoi les hybrides sont devenus la norme"); the pages give no
// formula, and the decode kernels' reading is kept: per (b, h) the d_v x d_k state follows
//     S_t = S_{t-1} diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t,
// with one gate per key channel. A prompt of T tokens runs through it, every output is written,
// and the final state becomes the checkpoint with an empty ring.
//
// Chunk form. Let S be the state at the chunk start and Gam_t = a_0 o a_1 o ... o a_t the gates'
// running product inside the chunk (per key channel). With u_t = beta_t (v_t - S_{t-1} (a_t o k_t))
// the step is S_t = S_{t-1} diag(a_t) + u_t k_t^T, so
//     S_t = S diag(Gam_t) + sum_{j<=t} u_j (k_j o Gam_t / Gam_j)^T.
// Put kh_t = k_t o Gam_t, kt_j = k_j / Gam_j, qh_t = q_t o Gam_t and A[t][j] = kh_t . kt_j (which
// carries the ratio Gam_t / Gam_j channel by channel). Then
//     u_t = beta_t (v_t - S kh_t - sum_{j<t} A[t][j] u_j),  i.e. U = T Z,  Z = V - Kh S^T,
// with T the lower-triangular factor of the delta rule's WY form (gdn_chunk.h) taken over A in
// place of the Gram block;
//     O = Qh S^T + M U,  M[t][j] = qh_t . kt_j for j <= t (else 0);
// and the chunk ends in S diag(Gam_15) + U^T Kb, Kb_j = kt_j o Gam_15, formed as
// (S + U^T Kt) diag(Gam_15). Every product is a
// v_mfma_f32_16x16x4_f32 chain on the register-resident tile of mfma_tile.h, as in the Gated
// DeltaNet prefill. Splitting Gam_t / Gam_j over the two operands needs 1 / Gam_j to stay finite: a
// chunk in which some channel's gate product falls below 2^-64 is applied token by token instead
// (the recurrence itself on the vector units), so any gate in [0, 1] is taken.
#include "dev_common.h"
#include "internal.h"
#include "gdn_chunk.h"
#include "gdn_layout.h"
#include "mfma_tile.h"

namespace rssm {
namespace {

// Waves per (b, h) workgroup: 4 at 128 x 128 (two i-blocks per wave, two workgroups per compute
// unit), else the tile's usual count.
template <int DV, int DK>
struct KpShape {
    static constexpr int NW = DV * DK >= 128 * 128 ? 4 : TileShape<DV, DK>::TPB / 64;
    static constexpr int TPB = 64 * NW;
};

// Smallest gate product over a chunk that the chunk form takes (then 1 / Gam_j <= 2^64).
constexpr float kMinGam = 0x1p-64f;

// LDS layout (floats). The chunk-form rows qh, kh, kt [16][d_k+4], beta [16] and Gam_15 [d_k] of
// two chunks (the next chunk's are written while the current one's are still read); the value rows
// [16][d_v+4]; the A, T and M blocks [16][20]; per chunk parity and wave a flag that sends the
// chunk to the token path.
template <int DV, int DK>
struct KpLds {
    static constexpr int KS = DK + 4, VS = DV + 4, R = kChunk * KS;
    static constexpr int rows(int p, int x) { return (3 * p + x) * R; }   // x: 0 qh, 1 kh, 2 kt
    static constexpr int v = 6 * R, be = v + kChunk * VS, gam = be + 2 * kChunk;
    static constexpr int A = gam + 2 * DK, T = A + kChunk * kTS, M = T + kChunk * kTS;
    static constexpr int flag = M + kChunk * kTS, floats = flag + 8;
    static_assert(R % 4 == 0 && be % 4 == 0 && gam % 4 == 0 && A % 4 == 0, "16-byte aligned rows");
};

__device__ __forceinline__ float4 mul4(float4 x, float4 y)
{
    return make_float4(x.x * y.x, x.y * y.y, x.z * y.z, x.w * y.w);
}

// The value of the lane D places lower in the same 16-lane row (a DPP row shift; lanes below D
// get 0).
template <int D>
__device__ __forceinline__ float4 row_shr4(float4 v)
{
    auto sh = [](float x) {
        const int r = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + D, 0xF, 0xF, true);
        return __int_as_float(r);
    };
    return make_float4(sh(v.x), sh(v.y), sh(v.z), sh(v.w));
}

// Step D of an inclusive product scan over groups of lanes aligned inside 16-lane rows (l = the
// lane's index in its group).
template <int D>
__device__ __forceinline__ void scan_mul_step(float4 &x, int l)
{
    const float4 y = row_shr4<D>(x);
    if (l >= D) x = mul4(x, y);
}

// The chunk's raw rows in registers between their load and their LDS store. Thread t holds the q,
// k and gate units of channels 4 cg .. 4 cg + 3 (cg = t / LPC) for TPT consecutive tokens, so
// that the LPC lanes of a channel group cover the chunk and the gate products are a scan across
// them; value units as VQ float4 in token-major order; beta of token t. The addresses are formed
// again for every chunk rather than kept in registers. Padding rows (tokens past the prompt) load
// as q = k = v = 0, gate 1, beta 0: they change nothing.
template <int DV, int DK>
struct KdaRows {
    static constexpr int TPB = KpShape<DV, DK>::TPB, KF = DK / 4, VF = DV / 4;
    static constexpr int TPT = kChunk * KF / TPB, LPC = kChunk / TPT;
    static constexpr int VQ = (kChunk * VF + TPB - 1) / TPB;
    static_assert(TPT * TPB == kChunk * KF && (TPT == 1 || TPT == 2) && (LPC == 8 || LPC == 16),
                  "row map: a channel group's lanes sit inside one 16-lane row");
    float4 q[TPT], k[TPT], a[TPT], v[VQ];
    float be;

    // tokens t0 .. t0 + ct - 1; the pointers are at token t0's row of this tile
    __device__ __forceinline__ void load(const float *qb, const float *kb, const float *ab,
                                         const float *vb, const float *bb, size_t BH, int ct, int t)
    {
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f), one = make_float4(1.f, 1.f, 1.f, 1.f);
        asm volatile("" : "+v"(t));        // the offsets are recomputed here
        const int cg = t / LPC, j0 = TPT * (t - cg * LPC);
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const bool in = j0 + i < ct;
            const size_t off = (size_t)(j0 + i) * BH * DK + 4 * cg;
            q[i] = in ? ld4(qb + off) : z;
            k[i] = in ? ld4(kb + off) : z;
            a[i] = in ? ld4(ab + off) : one;
        }
#pragma unroll
        for (int i = 0; i < VQ; ++i) {
            const int u = t + i * TPB, j = u / VF, o = (u - j * VF) * 4;
            v[i] = u < kChunk * VF && j < ct ? ld4(vb + (size_t)j * BH * DV + o) : z;
        }
        be = t < ct ? bb[(size_t)t * BH] : 0.f;
    }

    // The chunk-form rows of the held tokens into LDS buffer p: the gate products (over the
    // thread's tokens, then an exclusive product scan over the lanes of the channel group), qh,
    // kh and kt, beta; the group's last lane writes Gam_15 of its four channels and returns whether
    // one of them is below kMinGam or not a number.
    __device__ __forceinline__ bool derive(float *sm, int p, int t) const
    {
        using L = KpLds<DV, DK>;
        const int cg = t / LPC, l = t - cg * LPC, j0 = TPT * l;
        float4 pr[TPT];
        pr[0] = a[0];
#pragma unroll
        for (int i = 1; i < TPT; ++i) pr[i] = mul4(pr[i - 1], a[i]);
        float4 x = pr[TPT - 1];            // inclusive product scan over the group's lanes
        scan_mul_step<1>(x, l);
        scan_mul_step<2>(x, l);
        scan_mul_step<4>(x, l);
        if constexpr (LPC == 16) scan_mul_step<8>(x, l);
        float4 e = row_shr4<1>(x);         // exclusive: the earlier lanes' product
        if (l == 0) e = make_float4(1.f, 1.f, 1.f, 1.f);
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const float4 gm = mul4(e, pr[i]);
            const float4 rg = make_float4(__builtin_amdgcn_rcpf(gm.x), __builtin_amdgcn_rcpf(gm.y),
                                          __builtin_amdgcn_rcpf(gm.z), __builtin_amdgcn_rcpf(gm.w));
            const int o = (j0 + i) * L::KS + 4 * cg;
            st4(sm + L::rows(p, 0) + o, mul4(q[i], gm));
            st4(sm + L::rows(p, 1) + o, mul4(k[i], gm));
            st4(sm + L::rows(p, 2) + o, mul4(k[i], rg));
        }
        if (t < kChunk) sm[L::be + p * kChunk + t] = be;
        bool bad = false;
        if (l == LPC - 1) {
            st4(sm + L::gam + p * DK + 4 * cg, x);
            bad = !(x.x >= kMinGam && x.y >= kMinGam && x.z >= kMinGam && x.w >= kMinGam);
        }
        return bad;
    }

    __device__ __forceinline__ void store_v(float *sm, int t) const
    {
        using L = KpLds<DV, DK>;
#pragma unroll
        for (int i = 0; i < VQ; ++i) {
            const int u = t + i * TPB, j = u / VF, o = (u - j * VF) * 4;
            if (VQ * TPB == kChunk * VF || u < kChunk * VF) st4(sm + L::v + j * L::VS + o, v[i]);
        }
    }
};

// One token applied to the register tile by the recurrence itself (gate, key, query and value rows
// in LDS), then its output o = S q: per row the column scale, the dot with k, the rank-1 update and
// the dot with q; the four lanes that share a row add their parts by two exchanges.
template <typename F>
__device__ __forceinline__ void token_step(float4 (&s)[F::IBW][F::KB], const float *kr,
                                           const float *ar, const float *qr, const float *vr,
                                           float be, float *oj)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, cl = lane & 15;
#pragma unroll
    for (int ib = 0; ib < F::IBW; ++ib) {
        const int row = 16 * (wv * F::IBW + ib) + cl;
        float p = 0.f;
#pragma unroll
        for (int kb = 0; kb < F::KB; ++kb) {
            const float4 a4 = ld4(ar + 16 * kb + 4 * g), k4 = ld4(kr + 16 * kb + 4 * g);
            float4 &x = s[ib][kb];
            x.x *= a4.x; x.y *= a4.y; x.z *= a4.z; x.w *= a4.w;
            p += x.x * k4.x + x.y * k4.y + x.z * k4.z + x.w * k4.w;
        }
        p += bfly<16>(p);
        p += __shfl_xor(p, 32);
        const float cf = be * (vr[row] - p);
        float o = 0.f;
#pragma unroll
        for (int kb = 0; kb < F::KB; ++kb) {
            const float4 k4 = ld4(kr + 16 * kb + 4 * g), q4 = ld4(qr + 16 * kb + 4 * g);
            float4 &x = s[ib][kb];
            x.x += cf * k4.x; x.y += cf * k4.y; x.z += cf * k4.z; x.w += cf * k4.w;
            o += x.x * q4.x + x.y * q4.y + x.z * q4.z + x.w * q4.w;
        }
        o += bfly<16>(o);
        o += __shfl_xor(o, 32);
        if (g == 0) oj[row] = o;
    }
}

// NARROW: 16 token rows of the outputs span less than 4 GiB, so a chunk's output stores go
// through a buffer resource whose record range ends after the chunk's last real row: the stores of
// padding rows fall outside it and are dropped, and every store issues unpredicated (a predicated
// store leaves the compiler without a count of the stores in flight, and its wait for the next
// chunk's rows then covers those stores too).
template <int DV, int DK, bool NARROW>
__global__ void __launch_bounds__((KpShape<DV, DK>::TPB), 2) k_kda_prefill(GdnPrefillArgs a)
{
    using F = MfmaTile<DV, DK, KpShape<DV, DK>::NW>;
    using L = KpLds<DV, DK>;
    constexpr int NW = F::NW, IBW = F::IBW, KB = F::KB, KS = L::KS, VS = L::VS, KF = DK / 4;
    constexpr int NA = KB >= 2 ? 2 : KB;   // independent accumulators of the d_k products
    extern __shared__ float smem[];
    float *sh_v = smem + L::v, *sh_A = smem + L::A, *sh_T = smem + L::T, *sh_M = smem + L::M;
    int *sh_flag = reinterpret_cast<int *>(smem + L::flag);

    const int B = a.d.B, H = a.d.H, T = a.T;
    const int tile = blockIdx.x, b = tile / H, h = tile - b * H;
    const size_t bh = (size_t)tile, BH = (size_t)B * H;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6, g = lane >> 4, cl = lane & 15;

    const float *q0 = a.q + bh * DK, *k0 = a.k + bh * DK, *a0 = a.alpha + bh * DK;
    const float *v0 = a.v + bh * DV, *b0 = a.beta + bh;
    float *o0 = a.o + bh * DV;
    KdaRows<DV, DK> rows;
    rows.load(q0, k0, a0, v0, b0, BH, T < kChunk ? T : kChunk, t);
    float4 s[IBW][KB];
    float *S0 = a.S0 + bh * (size_t)(DV * DK);
    ckpt_load<DV>(s, S0, t);
    tile_loaded(s);
    auto derive = [&](int p) {
        const unsigned long long bad = __ballot(rows.derive(smem, p, t));
        if (lane == 0) sh_flag[4 * p + wv] = bad != 0;
    };
    derive(0);

    // Barriers per chunk: (1) the chunk-form rows, beta, Gam_15 and the flags of this chunk are in
    // LDS (written at the end of the previous one), and every wave is done with the previous chunk
    // (the value rows and the blocks may be rewritten); (2) the value rows and the A, T, M blocks
    // are in LDS. The next chunk's chunk-form rows go to the other buffer at the end of the chunk.
    for (int t0 = 0, n = 0; t0 < T; t0 += kChunk, ++n) {
        const int ct = T - t0 < kChunk ? T - t0 : kChunk, p = n & 1;
        __syncthreads();                                                             // (1)
        rows.store_v(smem, t);
        const bool more = t0 + kChunk < T;
        if (more) {                        // the next chunk's rows, in flight during this chunk
            const size_t t1 = t0 + kChunk;
            rows.load(q0 + t1 * BH * DK, k0 + t1 * BH * DK, a0 + t1 * BH * DK, v0 + t1 * BH * DV,
                      b0 + t1 * BH, BH, T - (int)t1 < kChunk ? T - (int)t1 : kChunk, t);
        }
        int slow = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) slow |= sh_flag[4 * p + w];
        const float *sh_qh = smem + L::rows(p, 0), *sh_kh = smem + L::rows(p, 1);
        const float *sh_kt = smem + L::rows(p, 2), *sh_be = smem + L::be + p * kChunk;
        const float *sh_gam = smem + L::gam + p * DK;

        if (slow) {
            // token path (some channel's gate product is below kMinGam): the raw q, k and gate rows
            // of the chunk go to this chunk's buffer in place of the chunk-form rows
            float *rq = smem + L::rows(p, 0), *rk = smem + L::rows(p, 1);
            float *ra = smem + L::rows(p, 2);
            for (int u = t; u < ct * KF; u += F::TPB) {
                const int j = u / KF, o = 4 * (u - j * KF);
                const size_t tk = (size_t)(t0 + j) * BH * DK + o;
                st4(rq + j * KS + o, ld4(q0 + tk));
                st4(rk + j * KS + o, ld4(k0 + tk));
                st4(ra + j * KS + o, ld4(a0 + tk));
            }
            __syncthreads();               // those rows and the value rows stored above
            for (int j = 0; j < ct; ++j)
                token_step<F>(s, rk + j * KS, ra + j * KS, rq + j * KS, sh_v + j * VS, sh_be[j],
                              o0 + (size_t)(t0 + j) * BH * DV);
        } else {
            // 2. the S-independent blocks first, so that their latency overlaps the other waves'
            //    matrix work: wave hv A and T, the next wave the masked M (one wave does both when
            //    alone); then every wave F = Kh S^T and Qs = Qh S^T for its i-blocks. The roles
            //    move from wave to wave with the chunk and the tile, so that the two workgroups on a
            //    compute unit do not both load the same SIMD with them. Wave hv's forward
            //    substitution sits in the same straight-line code as its products; its store of T
            //    comes after them.
            v4f fz[IBW], qs[IBW];
            auto products = [&]() {
#pragma unroll
                for (int ib = 0; ib < IBW; ++ib) {
                    v4f fp[NA], qp[NA];
#pragma unroll
                    for (int p = 0; p < NA; ++p) fp[p] = qp[p] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const float4 kv = ld4(sh_kh + cl * KS + 16 * kb + 4 * g);
                        const float4 qv = ld4(sh_qh + cl * KS + 16 * kb + 4 * g);
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
                    fz[ib] = tree_sum<NA>(fp);     // (S kh_q)[i] for q = 4 g + r, i = 16 ib' + c
                    qs[ib] = tree_sum<NA>(qp);     // (S qh_t)[i] for t = 4 g + r
                }
            };
            auto m_block = [&]() {
                const v4f m = row_dots16<KB, KS, NA, false>(sh_qh, sh_kt);   // qh_{4g+r} . kt_c
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sh_M[(4 * g + r) * kTS + cl] = cl <= 4 * g + r ? m[r] : 0.f;
            };
            const int hv = (n + tile) % NW;    // the wave with the extra roles this chunk
            if (wv == hv) {
                if constexpr (NW == 1) m_block();
                const v4f ak = row_dots16<KB, KS, NA, false>(sh_kh, sh_kt);  // kh_{4g+r} . kt_c
#pragma unroll
                for (int r = 0; r < 4; ++r) sh_A[(4 * g + r) * kTS + cl] = ak[r];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                float tq[kChunk];
                int q = cl;
                asm volatile("" : "+v"(q));
                t_solve_cols<kChunk, kTS>(sh_A, sh_be, tq, q);
                products();
                t_store_cols<kChunk, kTS>(tq, sh_T);
            } else {
                if (wv == (hv + 1) % NW) m_block();
                products();
            }
            mfma_settle();
            __syncthreads();                                                             // (2)

            // 3. M T, as (M T)^T = T^T M^T so that lane (g, c) ends with (M T)[t = c][q = 4 g + r],
            //    the A operand of the output chain
            v4f ut = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ut = mfma4(sh_T[(4 * g + r) * kTS + cl], sh_M[cl * kTS + 4 * g + r], ut);
            const float ua[4] = {ut[0], ut[1], ut[2], ut[3]};
            // the chunk's output rows; records end after row ct - 1 of this tile
            const __amdgpu_buffer_rsrc_t orows = __builtin_amdgcn_make_buffer_rsrc(
                o0 + (size_t)t0 * BH * DV, 0,
                NARROW ? (int)(((uint32_t)(ct - 1) * (uint32_t)(BH * DV) + (uint32_t)DV) * 4u) : 0,
                0x00020000);

#pragma unroll
            for (int ib = 0; ib < IBW; ++ib) {
                const int i = 16 * (wv * IBW + ib) + cl;
                float zq[4];                   // Z[q = 4 g + r][i] = v_q[i] - (S kh_q)[i]
#pragma unroll
                for (int r = 0; r < 4; ++r) zq[r] = sh_v[(4 * g + r) * VS + i] - fz[ib][r];
                // 4. outputs O = Qh S^T + (M T) Z
                v4f uz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < 4; ++r) uz = mfma4(ua[r], zq[r], uz);
                float ov[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) ov[r] = qs[ib][r] + uz[r];
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
                // 5. end of the chunk: U = T Z, S <- (S + U^T Kt) diag(Gam_15) (the column scale
                //    taken after the update, the same as S diag(Gam_15) + U^T Kb)
                const float4 tv = ld4(sh_T + cl * kTS + 4 * g);              // T[t = c][4 g + r]
                v4f cz = {0.f, 0.f, 0.f, 0.f};
                cz = mfma4(tv.x, zq[0], cz);
                cz = mfma4(tv.y, zq[1], cz);
                cz = mfma4(tv.z, zq[2], cz);
                cz = mfma4(tv.w, zq[3], cz);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    v4f u = {s[ib][kb].x, s[ib][kb].y, s[ib][kb].z, s[ib][kb].w};
                    const float *kr = sh_kt + (4 * g) * KS + 16 * kb + cl;     // kt[t][16 kb + c]
                    u = mfma4(kr[0], cz[0], u);
                    u = mfma4(kr[KS], cz[1], u);
                    u = mfma4(kr[2 * KS], cz[2], u);
                    u = mfma4(kr[3 * KS], cz[3], u);
                    const float4 gs = ld4(sh_gam + 16 * kb + 4 * g);   // Gam_15, lane's columns
                    s[ib][kb] = make_float4(gs.x * u[0], gs.y * u[1], gs.z * u[2], gs.w * u[3]);
                }
            }
            mfma_settle();
        }
        if (more) derive(p ^ 1);
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
hipError_t go_kda_prefill(const GdnPrefillArgs &a, hipStream_t s)
{
    const dim3 grid(a.d.B * a.d.H), block(KpShape<DV, DK>::TPB);
    const size_t lds = 4 * (size_t)KpLds<DV, DK>::floats;
    // 16 token rows of the outputs within 4 GiB: unpredicated output stores
    if ((size_t)a.d.B * a.d.H * DV * 4 * kChunk <= 0xFFFFFFFFull)
        hipLaunchKernelGGL((k_kda_prefill<DV, DK, true>), grid, block, lds, s, a);
    else
        hipLaunchKernelGGL((k_kda_prefill<DV, DK, false>), grid, block, lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t kda_prefill(const GdnPrefillArgs &a, hipStream_t s)
{
#define RSSM_C(v, k) if (a.d.DV == v && a.d.DK == k) return go_kda_prefill<v, k>(a, s);
    RSSM_C(16, 16) RSSM_C(64, 64) RSSM_C(128, 128)
#undef RSSM_C
    return hipErrorInvalidValue;
}

}  // namespace rssm
