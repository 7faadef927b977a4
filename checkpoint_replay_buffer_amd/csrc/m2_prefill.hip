// m2_prefill.hip -- Mamba-2 prefill into the checkpoint, on the matrix cores (gfx950).
//
// A prompt of T tokens is run through the recurrence S <- exp(dt A) S + dt x B^T, y = S C + D x
// (the conventional step the replay decode reproduces) and its final state becomes the checkpoint
// S0 with an empty ring: the persistent state the decode path starts from (ia.goatify.app article
// "NVIDIA y Princeton aceleran modelos híbridos...", paragraph "ReplaySSM cambia qué se
// almacena": a checkpoint plus the recent inputs). Every prompt token's output y_t is written too.
//
// The tokens go in chunks of 16. With S the state at the start of a chunk, dt_i the chunk's step
// sizes (zero past its last token) and, for tokens j <= t of the chunk,
//     w[t][j] = dt_j exp(A sum_{j<i<=t} dt_i),    Lam_t = exp(A sum_{i<=t} dt_i),
// the state after token t is Lam_t S + sum_{j<=t} w[t][j] x_j B_j^T, so
//     y_t = Lam_t (S C_t) + sum_{j<=t} w[t][j] (B_j . C_t) x_j + D x_t
//     S  <- Lam_15 S + sum_j w[15][j] x_j B_j^T                      (end of the chunk).
// The exponents are sums of the step sizes between the two tokens, not differences of running
// sums. S C^T, C B^T, M X (M[t][j] = w[t][j] (B_j . C_t)) and the rank-16 update are 16 x 16 x 4
// products on v_mfma_f32_16x16x4_f32; the tile stays in registers for the whole prompt, so the
// checkpoint is read and written once.
//
// Operand layouts of the instruction, lane l: A[l % 16][l / 16]; B[l / 16][l % 16]; accumulator
// register r holds D[4 (l / 16) + r][l % 16]. Lane (g, c) = (l / 16, l % 16) of wave w keeps, for
// each of its i-blocks ib (16 rows of S) and each k-block kb (16 columns), the float4
// S[16 ib' + c][16 kb + 4 g + r], ib' = w IBW + ib, r = 0..3. That float4 is the B operand of
// C S^T (inner index 16 kb + 4 g + r in step r of k-block kb) and the accumulator of B^T (w X),
// the transpose of the rank-16 update.
#include "dev_common.h"
#include "internal.h"

namespace rssm {
namespace {

constexpr int kChunk = 16;

template <int P, int N>
struct PrefillMap {
    static constexpr int TPB = TileShape<P, N>::TPB, NW = TPB / 64;
    static constexpr int IB = P / 16, KB = N / 16, IBW = IB / NW;   // i-blocks per wave
    static constexpr int XS = P + 4, BS = N + 4;                      // padded LDS row strides
    static_assert(IBW >= 1 && IBW * NW == IB, "prefill map");
};

// LDS floats: x [16][P+4], B and C [16][N+4], M [16][20], Lam, w[15][.] and dt [16] each
template <int P, int N>
__host__ __device__ constexpr int prefill_lds_floats()
{
    return kChunk * (P + 4) + 2 * kChunk * (N + 4) + kChunk * 20 + 3 * kChunk;
}

__device__ __forceinline__ v4f mfma4(float a, float b, v4f c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// The fp32 MFMA adds its four products to the accumulator in sequence, so a chain over d_state
// is a sequential sum of N terms. The long products (S C^T, C B^T) keep NA independent chains
// over interleaved k-blocks and add them as a tree: shorter sequential sums (the outputs of heads
// whose terms nearly cancel are sensitive to it), and independent work for the matrix cores.
template <int NA>
__device__ __forceinline__ v4f tree_sum(const v4f (&p)[NA])
{
    if constexpr (NA == 1) return p[0];
    else if constexpr (NA == 2) return p[0] + p[1];
    else return (p[0] + p[1]) + (p[2] + p[3]);
}

// Wait states after an MFMA chain whose accumulators are next read on the far side of a branch
// (the loop back-edge, the loop exit): 16 here, more than an 8-pass 16x16x4 f32 result needs, and
// the scheduling barriers keep the chain ahead of them.
__device__ __forceinline__ void mfma_settle()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int P, int N, bool BF16>
__global__ void __launch_bounds__((TileShape<P, N>::TPB)) k_m2_prefill(M2PrefillArgs a)
{
    using F = PrefillMap<P, N>;
    constexpr int TPB = F::TPB, IBW = F::IBW, KB = F::KB, XS = F::XS, BS = F::BS;
    constexpr int PF = P / 4, NF = N / 4, MS = 20;
    constexpr int NA = KB >= 4 ? 4 : KB;   // independent accumulators of the d_state products
    extern __shared__ float smem[];
    float *sh_x = smem;                    // [16][XS]
    float *sh_B = sh_x + kChunk * XS;      // [16][BS]
    float *sh_C = sh_B + kChunk * BS;      // [16][BS]
    float *sh_M = sh_C + kChunk * BS;      // [16][MS]  w[t][j] (B_j . C_t)
    float *sh_L = sh_M + kChunk * MS;      // [16]      Lam_t
    float *sh_wf = sh_L + kChunk;          // [16]      w[15][j]
    float *sh_dt = sh_wf + kChunk;         // [16]

    const int B = a.d.B, H = a.d.H, G = a.d.G, T = a.T;
    const int tile = blockIdx.x, b = tile / H, h = tile - b * H, g0 = h / (H / G);
    const size_t bh = (size_t)tile, bg = (size_t)b * G + g0;
    const size_t BH = (size_t)B * H, BG = (size_t)B * G;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6, g = lane >> 4, cl = lane & 15;
    const float Ah = a.A[h], Dh = a.D[h];

    float4 s[IBW][KB];
    float *S0 = a.S0 + bh * (size_t)(P * N);
    int off[IBW];
#pragma unroll
    for (int ib = 0; ib < IBW; ++ib) {
        off[ib] = (16 * (wv * IBW + ib) + cl) * N + 4 * g;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s[ib][kb] = ld4_nt(S0 + off[ib] + 16 * kb);
    }

    for (int t0 = 0; t0 < T; t0 += kChunk) {
        const int ct = T - t0 < kChunk ? T - t0 : kChunk;
        // 1. the chunk's rows (zero past its last token)
        for (int i = t; i < kChunk * (PF + 2 * NF); i += TPB) {
            if (i < kChunk * PF) {
                const int j = i / PF, o = (i - j * PF) * 4;
                st4(sh_x + j * XS + o, j < ct ? ld4(a.x + ((size_t)(t0 + j) * BH + bh) * P + o)
                                              : make_float4(0.f, 0.f, 0.f, 0.f));
            } else {
                const int i2 = i - kChunk * PF, which = i2 / (kChunk * NF);
                const int i3 = i2 - which * kChunk * NF, j = i3 / NF, o = (i3 - j * NF) * 4;
                const float *src = which == 0 ? a.Bm : a.C;
                st4((which == 0 ? sh_B : sh_C) + j * BS + o,
                    j < ct ? ld4(src + ((size_t)(t0 + j) * BG + bg) * N + o)
                           : make_float4(0.f, 0.f, 0.f, 0.f));
            }
        }
        if (t < kChunk) sh_dt[t] = t < ct ? a.dt[(size_t)(t0 + t) * BH + bh] : 0.f;
        __syncthreads();

        // 2. wave 0: the weights w[tt][j] (tt = 4 g + r, j = c) and Lam, then C B^T on the matrix
        //    cores and M = w o (C B^T); every wave: Z = C S^T for its i-blocks (S at the chunk start)
        if (wv == 0) {
            float w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tt = 4 * g + r, j = cl;
                float e = 0.f;
                for (int i = j + 1; i <= tt; ++i) e += sh_dt[i];
                w[r] = j <= tt ? sh_dt[j] * expf(Ah * e) : 0.f;
                if (j == 0) sh_L[tt] = expf(Ah * (e + sh_dt[0]));
                if (tt == kChunk - 1) sh_wf[j] = w[r];
            }
            v4f gp[NA];
#pragma unroll
            for (int q = 0; q < NA; ++q) gp[q] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const float4 cv = ld4(sh_C + cl * BS + 16 * kb + 4 * g);   // A: C[tt = c][k]
                const float4 bv = ld4(sh_B + cl * BS + 16 * kb + 4 * g);   // B: B[j = c][k]
                v4f &q = gp[kb % NA];
                q = mfma4(cv.x, bv.x, q);
                q = mfma4(cv.y, bv.y, q);
                q = mfma4(cv.z, bv.z, q);
                q = mfma4(cv.w, bv.w, q);
            }
            const v4f gc = tree_sum<NA>(gp);
#pragma unroll
            for (int r = 0; r < 4; ++r) sh_M[(4 * g + r) * MS + cl] = w[r] * gc[r];
        }
        v4f z[IBW];
#pragma unroll
        for (int ib = 0; ib < IBW; ++ib) {
            v4f zp[NA];
#pragma unroll
            for (int q = 0; q < NA; ++q) zp[q] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const float4 cv = ld4(sh_C + cl * BS + 16 * kb + 4 * g);
                v4f &q = zp[kb % NA];
                q = mfma4(cv.x, s[ib][kb].x, q);
                q = mfma4(cv.y, s[ib][kb].y, q);
                q = mfma4(cv.z, s[ib][kb].z, q);
                q = mfma4(cv.w, s[ib][kb].w, q);
            }
            z[ib] = tree_sum<NA>(zp);      // (S C_tt)[i] for tt = 4 g + r, i = 16 ib' + c
        }
        __syncthreads();

        // 3. outputs Y = Lam o Z + M X + D X; then S <- Lam_15 S + B^T (w X) (transposed form)
        const float lam_end = sh_L[kChunk - 1];
#pragma unroll
        for (int ib = 0; ib < IBW; ++ib) {
            const int i = 16 * (wv * IBW + ib) + cl;
            float xj[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) xj[r] = sh_x[(4 * g + r) * XS + i];   // X[j = 4 g + r][i]
            const float4 mv = ld4(sh_M + cl * MS + 4 * g);                    // M[tt = c][4 g + r]
            v4f acc = {0.f, 0.f, 0.f, 0.f};
            acc = mfma4(mv.x, xj[0], acc);
            acc = mfma4(mv.y, xj[1], acc);
            acc = mfma4(mv.z, xj[2], acc);
            acc = mfma4(mv.w, xj[3], acc);
            float yv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tt = 4 * g + r;
                yv[r] = sh_L[tt] * z[ib][r] + acc[r] + Dh * sh_x[tt * XS + i];
            }
            // keep the reads of the accumulator here, next to its chain, rather than sunk into the
            // conditional stores below
            asm volatile("" ::"v"(yv[0]), "v"(yv[1]), "v"(yv[2]), "v"(yv[3]));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tt = 4 * g + r;
                if (tt < ct) a.y[((size_t)(t0 + tt) * BH + bh) * P + i] = yv[r];
            }
            float wx[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) wx[r] = sh_wf[4 * g + r] * xj[r];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                v4f u = {lam_end * s[ib][kb].x, lam_end * s[ib][kb].y, lam_end * s[ib][kb].z,
                         lam_end * s[ib][kb].w};
                const float *br = sh_B + (4 * g) * BS + 16 * kb + cl;         // B[j][16 kb + c]
                u = mfma4(br[0], wx[0], u);
                u = mfma4(br[BS], wx[1], u);
                u = mfma4(br[2 * BS], wx[2], u);
                u = mfma4(br[3 * BS], wx[3], u);
                s[ib][kb] = make_float4(u[0], u[1], u[2], u[3]);
            }
        }
        mfma_settle();
        __syncthreads();
    }

    // the final state is the new checkpoint (and its bf16 read copy); the ring is empty
#pragma unroll
    for (int ib = 0; ib < IBW; ++ib) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            st4_nt(S0 + off[ib] + 16 * kb, s[ib][kb]);
            if constexpr (BF16) {
                uint2 w2;
                w2.x = pack_bf16x2(s[ib][kb].x, s[ib][kb].y);
                w2.y = pack_bf16x2(s[ib][kb].z, s[ib][kb].w);
                *reinterpret_cast<uint2 *>(a.S0b + bh * (size_t)(P * N) + off[ib] + 16 * kb) = w2;
            }
        }
    }
    if (h == 0 && t == 0) {
        a.bk.out[b] = a.bk.in[b];
        a.bk.out[B + b] = 0;
        a.bk.out[2 * B + b] = 0;
    }
}

template <int P, int N>
hipError_t go_prefill(const M2PrefillArgs &a, bool bf16, hipStream_t s)
{
    const dim3 grid(a.d.B * a.d.H), block(TileShape<P, N>::TPB);
    const size_t lds = 4 * (size_t)prefill_lds_floats<P, N>();
    if (bf16) hipLaunchKernelGGL((k_m2_prefill<P, N, true>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((k_m2_prefill<P, N, false>), grid, block, lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t m2_prefill(const M2PrefillArgs &a, bool bf16, hipStream_t s)
{
#define RSSM_C(p, n) if (a.d.P == p && a.d.N == n) return go_prefill<p, n>(a, bf16, s);
    RSSM_C(16, 16) RSSM_C(32, 32) RSSM_C(64, 64) RSSM_C(64, 128) RSSM_C(128, 128)
#undef RSSM_C
    return hipErrorInvalidValue;
}

}  // namespace rssm
