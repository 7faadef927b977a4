// gdn.hip -- Gated DeltaNet ReplaySSM decode kernels for gfx950.
//
// Per (b, h) the state S is d_v x d_k (row i = output channel) with the update
//     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t.
// Gated DeltaNet is one of the SSM layer types ReplaySSM targets (news.hamidun.com item
// "NVIDIA présente ReplaySSM...", section "Pourquoi les hybrides sont devenus la norme").
//
// Replay. For m buffered entries 0..m-1 (newest last), with the decay ratio
// d_j = prod_{i>j} alpha_i and gamma = prod_i alpha_i, unrolling the update applied to q gives
//     o = gamma S0 r + sum_j d_j beta_j c_j v_j,      r = q - sum_j beta_j c_j k_j,
// where the scalars c_j solve the triangular system
//     c_j = k_j . q - sum_{i>j} beta_i (k_j . k_i) c_i          (back substitution from j = m-1).
// The Gram entries and k_j . q are independent dot products; the solve is m steps of one wave.
// The checkpoint is read once (S0 r) and never written.
//
// Fold (WY form of the product of the rank-1 corrections). With G_it = k_i . k_t, the n x n
// lower-triangular T of the substitution y_t = beta_t (k_t - sum_{i<t} G_it y_i), i.e. y = T K,
// and d_q = prod_{i>q} alpha_i, gamma = prod_i alpha_i, the second recurrence
// u_t = beta_t (v_t - sum_{i<t} (gamma_t / gamma_i) G_it u_i) becomes the same substitution on
// the rows d_q v_q once u_t is scaled by d_t, so the folded state is
//     S0 <- gamma S0 + C^T K,     C = T Z,     Z_q = d_q v_q - gamma S0 k_q,
// in which every decay factor is at most 1. S0 K^T, T Z and C^T K run on the matrix cores.
#include "dev_common.h"
#include "internal.h"
#include "tile_order.h"
#include "mfma_tile.h"
#include "gdn_chunk.h"
#include "gdn_layout.h"

namespace rssm {
namespace {

struct GTile {
    int b, h, t, W;
    size_t bh, rh;
};

// The replay launches and the conventional comparator take runs of tiles per XCD; the launches
// that fold keep the identity order (contiguous ranges per XCD measured no faster there).
__device__ __forceinline__ GTile make_gtile(const GdnDims &d, TileOrder order)
{
    GTile c;
    const int tile = tile_of(blockIdx.x, d.B * d.H, order, run_tiles(d.DV * d.DK));
    c.b = tile / d.H;
    c.h = tile - c.b * d.H;
    c.t = threadIdx.x;
    c.W = d.W;
    c.bh = (size_t)tile;
    c.rh = c.bh * d.W;
    return c;
}

// Lanes per dot product and floats per lane for length-DK dots staged in LDS.
template <int DK>
struct DotMap {
    static constexpr int LPD = DK / 4 < 16 ? DK / 4 : 16;
    static constexpr int EPD = DK / LPD;
};

// Index (l, i), l < i, of the p-th strictly-upper pair in the order (0,1), (0,2), (1,2), ...
__device__ __forceinline__ void upper_pair(int p, int &l, int &i)
{
    i = 1;
    while (p >= i) {
        p -= i;
        ++i;
    }
    l = p;
}

template <int DK, int TPB>
__device__ __forceinline__ float lds_dot(const float *a, const float *b, int lane)
{
    constexpr int EPD = DotMap<DK>::EPD;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < EPD; e += 4) {
        const float4 x = ld4(a + lane * EPD + e), y = ld4(b + lane * EPD + e);
        s += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
    }
    return s;
}

// Gram entries G[l][i] = k_l . k_i (l < i < n), row stride W1; with q != nullptr also
// u_j = k_j . q into sh_u. Lane groups of LPD lanes take one dot each.
template <int DK, int TPB, int KSTR = DK>
__device__ __forceinline__ void gram_dots(const float *sh_k, const float *sh_q, int n, int W1,
                                          float *sh_G, float *sh_u, int t)
{
    constexpr int LPD = DotMap<DK>::LPD;
    const int grp = t / LPD, lane = t - grp * LPD;
    const int nq = sh_q ? n : 0;
    const int ndot = nq + n * (n - 1) / 2;
    for (int d = grp; d < ndot; d += TPB / LPD) {
        float s;
        int l, i = -1;
        if (d < nq) {
            l = d;
            s = lds_dot<DK, TPB>(sh_k + l * KSTR, sh_q, lane);
        } else {
            upper_pair(d - nq, l, i);
            s = lds_dot<DK, TPB>(sh_k + l * KSTR, sh_k + i * KSTR, lane);
        }
        s = group_sum<LPD>(s);
        if (lane == 0) {
            if (i < 0) sh_u[l] = s;
            else sh_G[l * W1 + i] = s;
        }
    }
}

// ------------------------------------------------------------------------------------------
// replay (the token does not fill the ring). Two barriers per tile.
// ------------------------------------------------------------------------------------------

// Exclusive suffix products across the lanes of a wave: lane l < n gets prod_{l<i<n} a_i (lane i
// holds a_i); `all` receives prod_{i<n} a_i on every lane. Every lane of the wave takes part.
__device__ __forceinline__ float wave_suffix_prod(float al, int n, float &all)
{
    const int lane = threadIdx.x & 63;
    const float v = lane < n ? al : 1.f;
    float e = __shfl_down(v, 1);
    if (lane == 63) e = 1.f;
    for (int off = 1; off < n; off <<= 1) {
        const float o = __shfl_down(e, off);
        if (lane + off < 64) e *= o;
    }
    all = __shfl(v * e, 0);
    return e;
}

__device__ __forceinline__ float lane_value(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// LDS floats of the replay: k and v rows of the W entries, q, the Gram entries [W][W+1], u [W],
// and per wave r [DK] and the value-sum coefficients [32].
template <int DV, int DK>
__host__ __device__ constexpr int gdn_replay_lds(int W)
{
    return W * (DK + DV) + DK + W * (W + 1) + W + (TileShape<DV, DK>::TPB / 64) * (DK + 32);
}

// The tile is held as in the fold (lane (g, c) of wave w keeps S[16 (w IBW + ib) + c][16 kb + 4 g
// .. +3]), which the checkpoint layout makes 1 KB per load instruction. LOAD = true: the tile is
// read here, after the ring loads went out (the ring position is known without a device read);
// LOAD = false: the caller already issued it.
template <int DV, int DK, bool LOAD>
__device__ __forceinline__ void gdn_replay(const GdnStepArgs &a, const GTile &c, int head, int len,
                                           float4 (&s)[MfmaTile<DV, DK>::IBW][MfmaTile<DV, DK>::KB],
                                           float *smem)
{
    using F = MfmaTile<DV, DK>;
    constexpr int TPB = F::TPB, IBW = F::IBW, KB = F::KB;
    constexpr int KF = DK / 4, VF = DV / 4;
    constexpr int XQ = (16 * (KF + VF) + TPB - 1) / TPB;   // float4 staged in registers (W <= 16)
    const int W = c.W, t = c.t, m = len + 1, W1 = W + 1, lane = t & 63, wv = t >> 6;
    const int g = lane >> 4, cl = lane & 15;
    float *sh_k = smem;                 // [m][DK]
    float *sh_v = sh_k + W * DK;        // [m][DV]
    float *sh_q = sh_v + W * DV;        // [DK]
    float *sh_G = sh_q + DK;            // [m][W1]  k_l . k_i, l < i
    float *sh_u = sh_G + W * W1;        // [m]      k_j . q
    float *sh_r = sh_u + W + wv * (DK + 32);   // [DK]  this wave's copy of r
    float *sh_cv = sh_r + DK;                  // [32]  d_j beta_j c_j, 0 past m

    const float *qt = a.q + c.bh * DK, *kt = a.k + c.bh * DK, *vt = a.v + c.bh * DV;
    const float bet = a.beta[c.bh], alt = a.alpha[c.bh];
    const int slot = (head + len) % W;
    // ring-side loads: beta / alpha of entry `lane` (every wave), k and v rows of all entries, q
    const float bel = lane < len ? a.ring.beta[c.rh + (head + lane) % W] : bet;
    const float all = lane < len ? a.ring.alpha[c.rh + (head + lane) % W] : alt;
    float4 xs[XQ];
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
        const int i = t + q * TPB;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < m * KF) {
            const int j = i / KF, o = (i - j * KF) * 4;
            v = j < len ? ld4(a.ring.k + (c.rh + (head + j) % W) * DK + o) : ld4(kt + o);
        } else if (i < m * (KF + VF)) {
            const int i2 = i - m * KF, j = i2 / VF, o = (i2 - j * VF) * 4;
            v = j < len ? ld4(a.ring.v + (c.rh + (head + j) % W) * DV + o) : ld4(vt + o);
        }
        xs[q] = v;
    }
    const float4 qv = t < KF ? ld4(qt + 4 * t) : make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (LOAD) ckpt_load<DV>(s, a.S0 + c.bh * (size_t)(DV * DK), t);
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
        const int i = t + q * TPB;
        if (i < m * KF) {
            const int j = i / KF, o = (i - j * KF) * 4;
            st4(sh_k + j * DK + o, xs[q]);
        } else if (i < m * (KF + VF)) {
            const int i2 = i - m * KF, j = i2 / VF, o = (i2 - j * VF) * 4;
            st4(sh_v + j * DV + o, xs[q]);
        }
    }
    for (int i = t + XQ * TPB; i < m * (KF + VF); i += TPB) {   // longer rings
        if (i < m * KF) {
            const int j = i / KF, o = (i - j * KF) * 4;
            st4(sh_k + j * DK + o, j < len ? ld4(a.ring.k + (c.rh + (head + j) % W) * DK + o) : ld4(kt + o));
        } else {
            const int i2 = i - m * KF, j = i2 / VF, o = (i2 - j * VF) * 4;
            st4(sh_v + j * DV + o, j < len ? ld4(a.ring.v + (c.rh + (head + j) % W) * DV + o) : ld4(vt + o));
        }
    }
    if (t < KF) st4(sh_q + 4 * t, qv);
    __syncthreads();
    gram_dots<DK, TPB>(sh_k, sh_q, m, W1, sh_G, sh_u, t);
    __syncthreads();

    // c_j by back substitution, in every wave (lane j ends with c_j): c_j = u_j - sum_{i>j}
    // beta_i G[j][i] c_i. The broadcast of c_i is a readlane, so the loop carries one FMA.
    float val = lane < m ? sh_u[lane] : 0.f;
    for (int i = m - 1; i >= 0; --i) {
        const float ci = lane_value(val, i) * lane_value(bel, i);
        if (lane < i) val -= sh_G[lane * W1 + i] * ci;
    }
    float gam;
    const float d = wave_suffix_prod(all, m, gam);        // prod_{i>j} alpha_i on lane j
    const float bc = bel * val;                           // beta_j c_j
    const float cv = d * bc;

    // r = q - sum_j beta_j c_j k_j into this wave's copy (CPL consecutive columns per lane) and
    // d_j beta_j c_j into the wave's coefficient row, both before the checkpoint is needed. The
    // loops run whole groups of eight entries without branches (coefficient 0 and a valid row past
    // m), so their LDS loads are in flight together.
    constexpr int CPL = DK >= 64 ? DK / 64 : 1;
    static_assert(CPL == 1 || CPL == 2, "r columns per lane");
    if (lane < 32) sh_cv[lane] = lane < m ? cv : 0.f;
    if (lane * CPL < DK) {
        const int col = lane * CPL;
        float r0 = sh_q[col], r1 = CPL == 2 ? sh_q[col + 1] : 0.f;
        for (int j0 = 0; j0 < m; j0 += 8) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int j = j0 + jj, jr = j < m ? j : m - 1;
                const float b = j < m ? lane_value(bc, j & 63) : 0.f;
                if constexpr (CPL == 2) {
                    const float2 kv = *reinterpret_cast<const float2 *>(sh_k + jr * DK + col);
                    r0 -= b * kv.x;
                    r1 -= b * kv.y;
                } else {
                    r0 -= b * sh_k[jr * DK + col];
                }
            }
        }
        if constexpr (CPL == 2) *reinterpret_cast<float2 *>(sh_r + col) = make_float2(r0, r1);
        else sh_r[col] = r0;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // o = gamma S0 r + sum_j d_j beta_j c_j v_j for the wave's rows: lane (g, c) takes its four
    // columns of each k-block and the entries j = g mod 4; the four lanes of a row are added by two
    // exchanges
#pragma unroll
    for (int ib = 0; ib < IBW; ++ib) {
        const int row = 16 * (wv * IBW + ib) + cl;
        float u = 0.f;
        for (int j0 = 0; j0 < m; j0 += 16) {
#pragma unroll
            for (int jj = 0; jj < 16; jj += 4) {
                const int j = j0 + jj + g, jr = j < m ? j : m - 1;
                u += sh_cv[j & 31] * sh_v[jr * DV + row];
            }
        }
        float p = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const float4 rq = ld4(sh_r + 16 * kb + 4 * g);
            p += s[ib][kb].x * rq.x + s[ib][kb].y * rq.y + s[ib][kb].z * rq.z + s[ib][kb].w * rq.w;
        }
        p = gam * p + u;
        p += __shfl_xor(p, 16);
        p += __shfl_xor(p, 32);
        if (g == 0) a.o[c.bh * DV + row] = p;
    }

    // Append the token as entry len (its slot is none of the entries read above); after the last
    // barrier, so no barrier waits for these stores.
    for (int i = t; i < KF; i += TPB) st4(a.ring.k + (c.rh + slot) * DK + 4 * i, ld4(sh_k + len * DK + 4 * i));
    for (int i = t; i < VF; i += TPB) st4(a.ring.v + (c.rh + slot) * DV + 4 * i, ld4(sh_v + len * DV + 4 * i));
    if (t == 0) {
        a.ring.beta[c.rh + slot] = bet;
        a.ring.alpha[c.rh + slot] = alt;
    }
}

// ------------------------------------------------------------------------------------------
// fold on the matrix cores (tile layout: mfma_tile.h). The accumulator of K S0^T is the B operand
// of T Z, and the accumulator of T Z the B operand of K^T C. Blocks of 16 entries; at most two
// (W <= 32).
// ------------------------------------------------------------------------------------------
template <int DV, int DK>
using FoldMap = MfmaTile<DV, DK>;

// Waves per SIMD the kernels that fold (and the verify) are compiled for: three 8-wave workgroups
// per compute unit at 128 x 128 with one entry block (at most 80 VGPRs), the compiler's choice
// otherwise.
template <int DV, int DK, int NTM>
struct FoldOcc {
    static constexpr int WPE = TileShape<DV, DK>::TPB == 512 && NTM == 1 ? 6 : 1;
};

// Entry blocks of the fold: one for W <= 16, two up to 32.
__host__ __device__ constexpr int fold_blocks(int W) { return W > 16 ? 2 : 1; }

template <int DV, int DK>
__host__ __device__ constexpr int gdn_fold_lds(int W)
{
    // K [NP][DK+4], V [NP][DV+4], beta [NP], decays d [NP], gamma [4], Gram and T [NP][NP+4]
    const int NP = 16 * fold_blocks(W);
    return NP * (DK + 4 + DV + 4) + 2 * NP + 4 + 2 * NP * (NP + 4);
}

// Fold n = nring (+1 with the token) entries, 1 <= n <= 16 NTM, (ring entries [0, nring) from
// slot `head`, then the token (kt, vt, bet, alt) if tok) into the tile, which is read from S0t
// (fold layout) after the entries' loads went out. All threads call it; two barriers. Wave 0
// forms the Gram blocks on the matrix cores and solves T in registers (gdn_chunk.h) while every
// wave forms Z = d o V - gamma K S0^T for its i-blocks; then C = T Z and S0 <- gamma S0 + C^T K.
//
// Every MFMA chain runs a compile-time number of steps (NTM blocks of 16 entries; rows past n are
// zero), and its accumulator is first read in the same straight-line code that issued the chain:
// a conditional chain followed by a read on the other side of a branch was given too few wait
// states by the compiler (the read saw a stale accumulator register), so no chain sits in a
// branch and no chain result is read across one (the Gram chains of wave 0 are read inside it).
template <int DV, int DK, int NTM, int IBW, int KB>
__device__ __forceinline__ void gdn_fold_mfma(float4 (&s)[IBW][KB], float *smem, const GdnRing &ring,
                                              const GTile &c, int head, int nring, bool tok,
                                              const float *kt, const float *vt, float bet,
                                              float alt, const float *S0t)
{
    using F = FoldMap<DV, DK>;
    static_assert(IBW == F::IBW && KB == F::KB, "fold block");
    static_assert(NTM == 1 || NTM == 2, "one or two 16-entry blocks");
    constexpr int TPB = F::TPB, KS = F::CS, VS = F::RS, KF = DK / 4, VF = DV / 4;
    constexpr int NP = 16 * NTM, PS = NP + 4;          // entry rows, zero past n
    constexpr int KQ = (NP * KF + TPB - 1) / TPB, VQ = (NP * VF + TPB - 1) / TPB;
    constexpr int NA = KB >= 2 ? 2 : 1;
    const int W = c.W, t = c.t, lane = t & 63, wv = t >> 6, g = lane >> 4, cl = lane & 15;
    const int n = nring + (tok ? 1 : 0);
    float *sh_k = smem;                 // [NP][KS]
    float *sh_v = sh_k + NP * KS;       // [NP][VS]
    float *sh_be = sh_v + NP * VS;      // [NP]
    float *sh_d = sh_be + NP;           // [NP]
    float *sh_g = sh_d + NP;            // gamma
    float *sh_G = sh_g + 4;             // [NP][PS]
    float *sh_T = sh_G + NP * PS;       // [NP][PS]

    // 1. the entries' loads, then the tile's; stage the entries (zero rows up to NP), beta, the
    //    decay ratios d_q and gamma (wave 0)
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 kr[KQ], vr[VQ];
#pragma unroll
    for (int i = 0; i < KQ; ++i) {
        const int u = t + i * TPB, j = u / KF, o = (u - j * KF) * 4;
        kr[i] = z4;
        if (u < NP * KF && j < n) kr[i] = j < nring ? ld4(ring.k + (c.rh + (head + j) % W) * DK + o) : ld4(kt + o);
    }
#pragma unroll
    for (int i = 0; i < VQ; ++i) {
        const int u = t + i * TPB, j = u / VF, o = (u - j * VF) * 4;
        vr[i] = z4;
        if (u < NP * VF && j < n) vr[i] = j < nring ? ld4(ring.v + (c.rh + (head + j) % W) * DV + o) : ld4(vt + o);
    }
    float bel = 0.f, all = 1.f;
    if (wv == 0) {
        bel = lane < nring ? ring.beta[c.rh + (head + lane) % W] : (lane < n ? bet : 0.f);
        all = lane < nring ? ring.alpha[c.rh + (head + lane) % W] : (lane < n ? alt : 1.f);
    }
    ckpt_load<DV>(s, S0t, t);
#pragma unroll
    for (int i = 0; i < KQ; ++i) {
        const int u = t + i * TPB, j = u / KF, o = (u - j * KF) * 4;
        if (u < NP * KF) st4(sh_k + j * KS + o, kr[i]);
    }
#pragma unroll
    for (int i = 0; i < VQ; ++i) {
        const int u = t + i * TPB, j = u / VF, o = (u - j * VF) * 4;
        if (u < NP * VF) st4(sh_v + j * VS + o, vr[i]);
    }
    if (wv == 0) {
        float gam;
        const float d = wave_suffix_prod(all, n, gam);
        if (lane < NP) {
            sh_be[lane] = bel;
            sh_d[lane] = lane < n ? d : 0.f;
        }
        if (lane == 0) sh_g[0] = gam;
    }
    __syncthreads();

    // 2. wave 0: the Gram blocks on the matrix cores, then T in registers; every wave:
    //    Z = d_q v_q - gamma S0 k_q for its i-blocks, with S0 k_q from K S0^T
    if (wv == 0) {
#pragma unroll
        for (int ib = 0; ib < NTM; ++ib) {
#pragma unroll
            for (int jb = 0; jb <= ib; ++jb) {
                const v4f gk = ib == jb
                    ? row_dots16<KB, KS, NA, true>(sh_k + 16 * ib * KS, sh_k + 16 * ib * KS)
                    : row_dots16<KB, KS, NA, false>(sh_k + 16 * ib * KS, sh_k + 16 * jb * KS);
#pragma unroll
                for (int r = 0; r < 4; ++r) sh_G[(16 * ib + 4 * g + r) * PS + 16 * jb + cl] = gk[r];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        t_solve_regs<NP, PS, PS>(sh_G, sh_be, sh_T);
    }
    const float gam = sh_g[0];
    v4f fz[IBW][NTM];
#pragma unroll
    for (int ib = 0; ib < IBW; ++ib) {
        const int i = 16 * (wv * IBW + ib) + cl;
#pragma unroll
        for (int tb = 0; tb < NTM; ++tb) {
            v4f fp[NA];
#pragma unroll
            for (int a = 0; a < NA; ++a) fp[a] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const float4 kv = ld4(sh_k + (16 * tb + cl) * KS + 16 * kb + 4 * g);
                v4f &f = fp[kb % NA];
                f = mfma4(kv.x, s[ib][kb].x, f);
                f = mfma4(kv.y, s[ib][kb].y, f);
                f = mfma4(kv.z, s[ib][kb].z, f);
                f = mfma4(kv.w, s[ib][kb].w, f);
            }
            const v4f acc = tree_sum<NA>(fp);
            // acc[r] = (S0 k_q)[i] for q = 16 tb + 4 g + r
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int q = 16 * tb + 4 * g + r;
                fz[ib][tb][r] = sh_d[q] * sh_v[q * VS + i] - gam * acc[r];
            }
        }
    }
    __syncthreads();

    // 3. C = T Z, then S0 <- gamma S0 + C^T K
#pragma unroll
    for (int ib = 0; ib < IBW; ++ib) {
        v4f cz[NTM];
#pragma unroll
        for (int tt = 0; tt < NTM; ++tt) {
            v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int tb = 0; tb <= tt; ++tb) {
                const float4 tv = ld4(sh_T + (16 * tt + cl) * PS + 16 * tb + 4 * g);
                acc = mfma4(tv.x, fz[ib][tb][0], acc);
                acc = mfma4(tv.y, fz[ib][tb][1], acc);
                acc = mfma4(tv.z, fz[ib][tb][2], acc);
                acc = mfma4(tv.w, fz[ib][tb][3], acc);
            }
            cz[tt] = acc;                // C[t][i] for t = 16 tt + 4 g + r, i = 16 ib' + c
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            v4f acc = {gam * s[ib][kb].x, gam * s[ib][kb].y, gam * s[ib][kb].z, gam * s[ib][kb].w};
#pragma unroll
            for (int tt = 0; tt < NTM; ++tt) {
                const float *kr = sh_k + (16 * tt + 4 * g) * KS + 16 * kb + cl;
#pragma unroll
                for (int r = 0; r < 4; ++r) acc = mfma4(kr[r * KS], cz[tt][r], acc);
            }
            s[ib][kb] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    }
}

// The tile, held in the operand layout, written row-major (materialisation).
template <int DV, int DK, int IBW, int KB>
__device__ __forceinline__ void store_rows(const float4 (&s)[IBW][KB], float *dst, int t)
{
#pragma unroll
    for (int ib = 0; ib < IBW; ++ib) {
        float *p = dst + mfma_tile_offset<DV, DK>(t, ib);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) st4_nt(p + 16 * kb, s[ib][kb]);
    }
}

// decode step whose token fills the ring: fold the ring and the token, store, o = S q (all in
// one straight-line region after the fold's MFMA chains)
template <int DV, int DK, int NTM>
__device__ __forceinline__ void gdn_fold_decode(const GdnStepArgs &a, const GTile &c, int head,
                                                int len, float *smem)
{
    using F = FoldMap<DV, DK>;
    const int t = c.t, lane = t & 63, g = lane >> 4;
    float *S0 = a.S0 + c.bh * (size_t)(DV * DK);
    const float *qt = a.q + c.bh * DK;
    float4 s[F::IBW][F::KB];
    gdn_fold_mfma<DV, DK, NTM>(s, smem, a.ring, c, head, len, true, a.k + c.bh * DK,
                               a.v + c.bh * DV, a.beta[c.bh], a.alpha[c.bh], S0);
    ckpt_store<DV>(s, S0, t);
#pragma unroll
    for (int ib = 0; ib < F::IBW; ++ib) {
        float p = 0.f;
#pragma unroll
        for (int kb = 0; kb < F::KB; ++kb) {
            const float4 qv = ld4(qt + 16 * kb + 4 * g);
            p += s[ib][kb].x * qv.x + s[ib][kb].y * qv.y + s[ib][kb].z * qv.z + s[ib][kb].w * qv.w;
        }
        p += __shfl_xor(p, 16);
        p += __shfl_xor(p, 32);
        if (g == 0) a.o[c.bh * DV + 16 * ((t >> 6) * F::IBW + ib) + (lane & 15)] = p;
    }
}

// Consolidation or materialisation of one tile: fold, then store (same straight-line region).
template <int DV, int DK, int NTM>
__device__ __forceinline__ void gdn_fold_tile(const GdnFoldArgs &a, const GTile &c, int head,
                                              int len, float *smem)
{
    using F = FoldMap<DV, DK>;
    float *S0 = a.S0 + c.bh * (size_t)(DV * DK);
    float4 s[F::IBW][F::KB];
    gdn_fold_mfma<DV, DK, NTM>(s, smem, a.ring, c, head, len, false, nullptr, nullptr, 0.f, 0.f, S0);
    mfma_settle();                      // the tile is read on either side of the branch below
    if (a.out) store_rows<DV, DK>(s, a.out + c.bh * (size_t)(DV * DK), c.t);
    else ckpt_store<DV>(s, S0, c.t);
}

// Decode variants, chosen on the host as for Mamba-2: 0 = every sequence at the ring position
// (a.uhead, a.ulen) with no fold (ring loads before the checkpoint read), 1 = no sequence folds
// (positions read from the device), 2 = any sequence may fold (NTM entry blocks: one kernel per
// block count, so that the one-block fold keeps its register budget).
template <int DV, int DK, int MODE, int NTM = 1>
__global__ void __launch_bounds__((TileShape<DV, DK>::TPB), (MODE == 2 ? FoldOcc<DV, DK, NTM>::WPE : 1))
k_gdn_decode(GdnStepArgs a)
{
    using F = MfmaTile<DV, DK>;
    extern __shared__ float smem[];
    const GTile c = make_gtile(a.d, MODE == 2 ? kIdentity : kRuns);
    const int B = a.d.B, W = c.W;
    float4 s[F::IBW][F::KB];
    int head, len;
    bool fold = false;
    if constexpr (MODE == 0) {
        head = a.uhead;
        len = a.ulen;
        gdn_replay<DV, DK, true>(a, c, head, len, s, smem);
    } else if constexpr (MODE == 1) {
        // the checkpoint tile first, then the ring position
        ckpt_load<DV>(s, a.S0 + c.bh * (size_t)(DV * DK), c.t);
        head = a.bk.in[c.b];
        len = a.bk.in[B + c.b];
        gdn_replay<DV, DK, false>(a, c, head, len, s, smem);
    } else {
        // the ring position first: the fold issues the entries' loads before the tile's
        head = a.bk.in[c.b];
        len = a.bk.in[B + c.b];
        fold = len + 1 >= W;
        if (!fold) gdn_replay<DV, DK, true>(a, c, head, len, s, smem);
        else gdn_fold_decode<DV, DK, NTM>(a, c, head, len, smem);
    }
    if (c.h == 0 && c.t == 0) {
        a.bk.out[c.b] = fold ? (head + len + 1) % W : head;
        a.bk.out[B + c.b] = fold ? 0 : len + 1;
        a.bk.out[2 * B + c.b] = 0;
    }
}

template <int DV, int DK, int NTM>
__global__ void __launch_bounds__((TileShape<DV, DK>::TPB), (FoldOcc<DV, DK, NTM>::WPE)) k_gdn_fold(GdnFoldArgs a)
{
    constexpr int TPB = TileShape<DV, DK>::TPB;
    extern __shared__ float smem[];
    const GTile c = make_gtile(a.d, kIdentity);
    const int B = a.d.B, W = c.W;
    const int head = a.bk.in[c.b];
    const int len = a.bk.in[B + c.b];
    const int nd = a.bk.in[2 * B + c.b];
    const bool fold = len >= (a.min_len > 1 ? a.min_len : 1);
    if (!a.out && c.h == 0 && c.t == 0) {
        a.bk.out[c.b] = fold ? (head + len) % W : head;
        a.bk.out[B + c.b] = fold ? 0 : len;
        a.bk.out[2 * B + c.b] = nd;
    }
    float *S0 = a.S0 + c.bh * (size_t)(DV * DK);
    if (!fold) {
        if (a.out) {
            float *dst = a.out + c.bh * (size_t)(DV * DK);
            for (int i = c.t; i < DV * DK / 4; i += TPB) {     // row-major from the checkpoint layout
                const int row = 4 * i / DK, col = 4 * i - row * DK;
                st4(dst + 4 * i, ld4(S0 + ckpt_offset(row, col, DV)));
            }
        }
        return;
    }
    gdn_fold_tile<DV, DK, NTM>(a, c, head, len, smem);
}

// conventional read-modify-write comparator
template <int DV, int DK>
__global__ void __launch_bounds__((TileShape<DV, DK>::TPB)) k_gdn_rmw(GdnRmwArgs a)
{
    using M = Map4<DV, DK>;
    constexpr int R = M::R, LPR = M::LPR;
    __shared__ float sh_sk[DV];
    const GTile c = make_gtile(a.d, kRuns);
    const int t = c.t;
    const int rg = t / LPR, cg = t - rg * LPR, c0 = cg * 4;
    const size_t BH = (size_t)a.d.B * a.d.H, VK = (size_t)DV * DK;
    const size_t lo = (size_t)(rg * R) * DK + c0;          // lane block within a tile
    const size_t off = c.bh * VK + lo;
    // source tile and the first snapshot tile (snapshot k is k * BH tiles further)
    // source (updated in place when there are no snapshots) and first snapshot
    float *src;
    float *snap0;
    if (a.slot_of) {
        const int sl = a.slot_of[c.b];
        src = a.state + ((size_t)sl * BH + c.bh) * VK + lo;
        snap0 = a.state + ((size_t)(sl < a.ntok ? a.ntok : 0) * BH + c.bh) * VK + lo;
    } else {
        src = a.seq ? a.seq[c.b] + (size_t)c.h * VK + lo : a.state + off;
        snap0 = a.snap ? a.snap + off : nullptr;
    }
    float4 S[R];
#pragma unroll
    for (int r = 0; r < R; ++r) S[r] = ld4_nt(src + (size_t)r * DK);
    for (int k = 0; k < a.ntok; ++k) {
        const size_t tk = k * BH + c.bh;
        const float be = a.beta[tk], al = a.alpha[tk];
        const float4 kv = ld4(a.k + tk * DK + c0);
        const float4 qv = ld4(a.q + tk * DK + c0);
        const float *vv = a.v + tk * DV;
        float part[R];
#pragma unroll
        for (int r = 0; r < R; ++r) part[r] = S[r].x * kv.x + S[r].y * kv.y + S[r].z * kv.z + S[r].w * kv.w;
        int rsel;
        const float sk = row_reduce_scatter<R, LPR, false>(part, cg, rsel);
        if (row_writer<R, LPR>(cg)) sh_sk[rg * R + rsel] = sk;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = rg * R + r;
            // alpha (S - beta (S k) k^T) + beta v k^T, one rank-1 term per row
            const float cf = be * vv[i] - al * be * sh_sk[i];
            S[r].x = al * S[r].x + cf * kv.x; S[r].y = al * S[r].y + cf * kv.y;
            S[r].z = al * S[r].z + cf * kv.z; S[r].w = al * S[r].w + cf * kv.w;
            part[r] = S[r].x * qv.x + S[r].y * qv.y + S[r].z * qv.z + S[r].w * qv.w;
        }
        __syncthreads();
        const float z = row_reduce_scatter<R, LPR, false>(part, cg, rsel);
        if (row_writer<R, LPR>(cg)) a.o[tk * DV + rg * R + rsel] = z;
        if (snap0) {
#pragma unroll
            for (int r = 0; r < R; ++r) st4_nt(snap0 + k * BH * VK + (size_t)r * DK, S[r]);
        }
    }
    if (!snap0) {
#pragma unroll
        for (int r = 0; r < R; ++r) st4_nt(src + (size_t)r * DK, S[r]);
    }
}

// ------------------------------------------------------------------------------------------
// speculative verify: K drafts per sequence, outputs only, checkpoint streamed once
// ------------------------------------------------------------------------------------------
// One block of 16 entries (W <= 16): sequences that fold stage their ring entries and their drafts
// in two separate blocks and fold the first inside the verify's own phases. Two blocks (W > 16):
// they fold first with the decode fold, then verify.
template <int NTM>
struct VerifySplit {
    static constexpr bool value = NTM == 1;
};

// LDS floats of the verify with NP = 16 NTM entry rows (two blocks of them when split): keys
// [.][d_k+4] and values [.][d_v+4] by entry position, the drafts' queries (then their r rows)
// [16][d_k+4], beta and alpha [.], the Gram and T [NP][NP+4] of the verified entries, A and the
// decay rows [16][NP+4], Gam [16]; when split also the Gram, T and decay rows of the folded block
// and its Gam.
template <int DV, int DK, int NTM>
__host__ __device__ constexpr int gdn_verify_lds()
{
    constexpr int NP = kChunk * NTM, PS = NP + 4, NR = VerifySplit<NTM>::value ? 2 * NP : NP;
    constexpr int base = NR * (DK + 4 + DV + 4) + kChunk * (DK + 4) + 2 * NR + 2 * NP * PS
                         + 2 * kChunk * PS + kChunk;
    return VerifySplit<NTM>::value ? base + 2 * NP * PS + kChunk * PS + kChunk : base;
}

// Drafts k = 0..K-1 become entries len_e + k, and draft k's output is the replay (top of this
// file) for q_k over the first m_k = len_e + k + 1 entries. Back substitution over a prefix is the
// leading block of the substitution that T solves (gdn_chunk.h), so with A[k][i] = q_k . k_i for
// i < m_k (else 0) and U = A T,
//     beta_j c_{k,j} = U[k][j],     r_k = q_k - sum_j U[k][j] k_j,
//     o_k = Gam_k S0 r_k + sum_j D[k][j] U[k][j] v_j,
// with D[k][j] = prod_{j<i<m_k} alpha_i and Gam_k = prod_{i<m_k} alpha_i. While the checkpoint
// streams in, one wave forms the Gram blocks and T, another A, a third the decays; then U, W = D o U
// and the rows r_k are 16-wide products on the matrix cores, and the outputs of all drafts are
// R S0^T + W V on the tile held in the layout of mfma_tile.h. The checkpoint is read once.
//
// Sequences whose ring cannot take the drafts (len + K > W) first fold their len entries into the
// checkpoint. Split (one block): the ring entries are a block of their own, folded in the same
// phases by the chunk fold of the prefill (F = K S0^T, C = T Z with Z_q = R[q] v_q - gam F_q,
// S0 <- gam S0 + C^T K) while the drafts' blocks are formed, and the new checkpoint is written.
template <int DV, int DK, int NTM>
__global__ void __launch_bounds__((TileShape<DV, DK>::TPB), (FoldOcc<DV, DK, NTM>::WPE)) k_gdn_verify(GdnStepArgs a)
{
    using F = FoldMap<DV, DK>;
    constexpr int TPB = F::TPB, NW = F::NW, IBW = F::IBW, KB = F::KB, KS = F::CS, VS = F::RS;
    constexpr bool SPLIT = VerifySplit<NTM>::value;
    constexpr int NP = kChunk * NTM, PS = NP + 4, NR = SPLIT ? 2 * NP : NP;
    constexpr int KF = DK / 4, VF = DV / 4;
    constexpr int KQ = (NR * KF + TPB - 1) / TPB, VQ = (NR * VF + TPB - 1) / TPB;
    constexpr int QQ = (kChunk * KF + TPB - 1) / TPB;
    constexpr int NA = KB >= 2 ? 2 : 1;
    static_assert(KB % NW == 0, "k-blocks of the r rows split evenly over the waves");
    extern __shared__ float smem[];
    const GTile c = make_gtile(a.d, kRuns);
    const int B = a.d.B, W = c.W, K = a.ntok, t = c.t, lane = t & 63, wv = t >> 6;
    const int g = lane >> 4, cl = lane & 15;
    const size_t BH = (size_t)B * a.d.H;
    const int head = a.bk.in[c.b], len = a.bk.in[B + c.b];
    const bool prefold = len + K > W;
    const bool fold_here = SPLIT && prefold;             // the ring block is folded below
    const int head_e = prefold ? (head + len) % W : head, len_e = prefold ? 0 : len;
    const int ne = len_e + K;
    const int nring = prefold && !SPLIT ? 0 : len;        // ring entries staged from slot `head`
    const int d0 = fold_here ? NP : nring;                // row of draft 0
    const int vb = fold_here ? NP : 0;                    // first row of the verified entries
    float *S0 = a.S0 + c.bh * (size_t)(DV * DK);
    float4 s[IBW][KB];
    if constexpr (!SPLIT) {
        if (prefold) {
            gdn_fold_mfma<DV, DK, NTM>(s, smem, a.ring, c, head, len, false, nullptr, nullptr, 0.f, 0.f, S0);
            ckpt_store<DV>(s, S0, t);
            mfma_settle();                  // the tile is read by the chains below
            __syncthreads();                // the fold's LDS is reused
        }
    }
    float *sh_k = smem;                     // [NR][KS]  entries by row
    float *sh_v = sh_k + NR * KS;           // [NR][VS]
    float *sh_q = sh_v + NR * VS;           // [16][KS]  q_k, then r_k
    float *sh_be = sh_q + kChunk * KS;      // [NR]
    float *sh_al = sh_be + NR;              // [NR]
    float *sh_G = sh_al + NR;               // [NP][PS]  G[t][i] = k_t . k_i, i <= t
    float *sh_T = sh_G + NP * PS;           // [NP][PS]
    float *sh_A = sh_T + NP * PS;           // [16][PS]
    float *sh_D = sh_A + kChunk * PS;       // [16][PS]
    float *sh_gam = sh_D + kChunk * PS;     // [16]
    float *sh_Gf = sh_gam + kChunk;         // [NP][PS]  the folded block (split only)
    float *sh_Tf = sh_Gf + NP * PS;         // [NP][PS]
    float *sh_Df = sh_Tf + NP * PS;         // [16][PS]
    float *sh_gf = sh_Df + kChunk * PS;     // [16]

    // 1. into registers: key and value of row j (ring entry j < nring, then the drafts from row
    //    d0, zero elsewhere), the query of draft k (zero from K), beta and alpha of row t (0 and 1
    //    on zero rows); then the checkpoint goes out; then the rows go to LDS
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 kr[KQ], vr[VQ], qr[QQ];
#pragma unroll
    for (int i = 0; i < KQ; ++i) {
        const int u = t + i * TPB, j = u / KF, o = (u - j * KF) * 4;
        kr[i] = z4;
        if (u < NR * KF) {
            if (j < nring) kr[i] = ld4(a.ring.k + (c.rh + (head + j) % W) * DK + o);
            else if (j >= d0 && j < d0 + K) kr[i] = ld4(a.k + ((j - d0) * BH + c.bh) * DK + o);
        }
    }
#pragma unroll
    for (int i = 0; i < VQ; ++i) {
        const int u = t + i * TPB, j = u / VF, o = (u - j * VF) * 4;
        vr[i] = z4;
        if (u < NR * VF) {
            if (j < nring) vr[i] = ld4(a.ring.v + (c.rh + (head + j) % W) * DV + o);
            else if (j >= d0 && j < d0 + K) vr[i] = ld4(a.v + ((j - d0) * BH + c.bh) * DV + o);
        }
    }
#pragma unroll
    for (int i = 0; i < QQ; ++i) {
        const int u = t + i * TPB, k = u / KF, o = (u - k * KF) * 4;
        qr[i] = u < kChunk * KF && k < K ? ld4(a.q + (k * BH + c.bh) * DK + o) : z4;
    }
    float be = 0.f, al = 1.f;
    if (t < NR) {
        if (t < nring) {
            const size_t sl = c.rh + (head + t) % W;
            be = a.ring.beta[sl];
            al = a.ring.alpha[sl];
        } else if (t >= d0 && t < d0 + K) {
            const size_t d = (t - d0) * BH + c.bh;
            be = a.beta[d];
            al = a.alpha[d];
        }
    }
    if (SPLIT || !prefold) ckpt_load<DV>(s, S0, t);
#pragma unroll
    for (int i = 0; i < KQ; ++i) {
        const int u = t + i * TPB, j = u / KF, o = (u - j * KF) * 4;
        if (u < NR * KF) st4(sh_k + j * KS + o, kr[i]);
    }
#pragma unroll
    for (int i = 0; i < VQ; ++i) {
        const int u = t + i * TPB, j = u / VF, o = (u - j * VF) * 4;
        if (u < NR * VF) st4(sh_v + j * VS + o, vr[i]);
    }
#pragma unroll
    for (int i = 0; i < QQ; ++i) {
        const int u = t + i * TPB, k = u / KF, o = (u - k * KF) * 4;
        if (u < kChunk * KF) st4(sh_q + k * KS + o, qr[i]);
    }
    if (t < NR) {
        sh_be[t] = be;
        sh_al[t] = al;
    }
    __syncthreads();

    // 2. the blocks that do not need the checkpoint, one role per wave (roles share a wave when
    //    there are fewer than four): the verified entries' Gram blocks and T; A; the decays (and
    //    those of the folded block); the folded block's Gram and T. Then, when folding, every wave
    //    forms F = K S0^T of the folded block for its i-blocks.
    const float *vk = sh_k + vb * KS;
    if (wv == 0) {
#pragma unroll
        for (int ib = 0; ib < NTM; ++ib) {
#pragma unroll
            for (int jb = 0; jb <= ib; ++jb) {
                const v4f gk = ib == jb
                    ? row_dots16<KB, KS, NA, true>(vk + 16 * ib * KS, vk + 16 * ib * KS)
                    : row_dots16<KB, KS, NA, false>(vk + 16 * ib * KS, vk + 16 * jb * KS);
#pragma unroll
                for (int r = 0; r < 4; ++r) sh_G[(16 * ib + 4 * g + r) * PS + 16 * jb + cl] = gk[r];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        t_solve_regs<NP, PS, PS>(sh_G, sh_be + vb, sh_T);
    }
    if (wv == 1 % NW) {
#pragma unroll
        for (int jb = 0; jb < NTM; ++jb) {
            const v4f qk = row_dots16<KB, KS, NA, false>(sh_q, vk + 16 * jb * KS);   // q_{4g+r} . k_{16jb+c}
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sh_A[(4 * g + r) * PS + 16 * jb + cl] = 16 * jb + cl <= len_e + 4 * g + r ? qk[r] : 0.f;
        }
    }
    if (wv == 3 % NW) {
        decay_row<NP, PS>(sh_al + vb, len_e + lane, sh_D, sh_gam);
        if (fold_here) decay_row<NP, PS>(sh_al, NP - 1, sh_Df, sh_gf);   // R[q] of the whole block
    }
    if constexpr (SPLIT) {
        if (fold_here) {
            if (wv == 2 % NW) {
                const v4f gk = row_dots16<KB, KS, NA, true>(sh_k, sh_k);
#pragma unroll
                for (int r = 0; r < 4; ++r) sh_Gf[(4 * g + r) * PS + cl] = gk[r];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                t_solve_regs<NP, PS, PS>(sh_Gf, sh_be, sh_Tf);
            }
        }
    }
    v4f fz[IBW];                            // F[q = 4 g + r][i = 16 ib' + c] of the folded block
    if constexpr (SPLIT) {
        if (fold_here) {
#pragma unroll
            for (int ib = 0; ib < IBW; ++ib) {
                v4f fp[NA];
#pragma unroll
                for (int n = 0; n < NA; ++n) fp[n] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const float4 kv = ld4(sh_k + cl * KS + 16 * kb + 4 * g);   // A: K[c][16 kb + 4 g + r]
                    v4f &f = fp[kb % NA];
                    f = mfma4(kv.x, s[ib][kb].x, f);
                    f = mfma4(kv.y, s[ib][kb].y, f);
                    f = mfma4(kv.z, s[ib][kb].z, f);
                    f = mfma4(kv.w, s[ib][kb].w, f);
                }
                fz[ib] = tree_sum<NA>(fp);
            }
            mfma_settle();
        }
    }
    __syncthreads();

    // 3. when folding: Z = R o V - gam F, C = T Z, S0 <- gam S0 + C^T K, and the new checkpoint
    //    goes out. Then U = A T as U^T = T^T A^T, so that lane (g, c) ends with
    //    U[k = c][j = 16 jb + 4 g + r], the A operand of the products below (T[i][j] = 0 for
    //    i < j); W = D o U; and the rows r_k = q_k - sum_j U[k][j] k_j of the wave's k-blocks,
    //    written over the queries
    if constexpr (SPLIT) {
        if (fold_here) {
            const float4 rf4 = ld4(sh_Df + 4 * g);                  // R[q = 4 g + r]
            const float rf[4] = {rf4.x, rf4.y, rf4.z, rf4.w};
            const float gf = sh_gf[0];
            const float4 tv = ld4(sh_Tf + cl * PS + 4 * g);         // T[t = c][4 g + r]
#pragma unroll
            for (int ib = 0; ib < IBW; ++ib) {
                const int i = 16 * (wv * IBW + ib) + cl;
                float zf[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) zf[r] = rf[r] * sh_v[(4 * g + r) * VS + i] - gf * fz[ib][r];
                v4f cz = {0.f, 0.f, 0.f, 0.f};
                cz = mfma4(tv.x, zf[0], cz);
                cz = mfma4(tv.y, zf[1], cz);
                cz = mfma4(tv.z, zf[2], cz);
                cz = mfma4(tv.w, zf[3], cz);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    v4f u = {gf * s[ib][kb].x, gf * s[ib][kb].y, gf * s[ib][kb].z, gf * s[ib][kb].w};
                    const float *kc = sh_k + (4 * g) * KS + 16 * kb + cl;   // K[t = 4 g + r][16 kb + c]
                    u = mfma4(kc[0], cz[0], u);
                    u = mfma4(kc[KS], cz[1], u);
                    u = mfma4(kc[2 * KS], cz[2], u);
                    u = mfma4(kc[3 * KS], cz[3], u);
                    s[ib][kb] = make_float4(u[0], u[1], u[2], u[3]);
                }
            }
            mfma_settle();
            ckpt_store<DV>(s, S0, t);
        }
    }
    float ua[NTM][4], wa[NTM][4];
#pragma unroll
    for (int jb = 0; jb < NTM; ++jb) {
        v4f ut = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ib = jb; ib < NTM; ++ib) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ut = mfma4(sh_T[(16 * ib + 4 * g + r) * PS + 16 * jb + cl], sh_A[cl * PS + 16 * ib + 4 * g + r], ut);
        }
        const float4 dv = ld4(sh_D + cl * PS + 16 * jb + 4 * g);
        const float dr[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            ua[jb][r] = ut[r];
            wa[jb][r] = ut[r] * dr[r];
        }
    }
#pragma unroll
    for (int n = 0; n < KB / NW; ++n) {
        const int kb = wv + n * NW;
        v4f rk;
#pragma unroll
        for (int r = 0; r < 4; ++r) rk[r] = sh_q[(4 * g + r) * KS + 16 * kb + cl];   // Q[4g+r][16kb+c]
#pragma unroll
        for (int jb = 0; jb < NTM; ++jb) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                rk = mfma4(-ua[jb][r], vk[(16 * jb + 4 * g + r) * KS + 16 * kb + cl], rk);
        }
        const float rv[4] = {rk[0], rk[1], rk[2], rk[3]};
        asm volatile("" ::"v"(rv[0]), "v"(rv[1]), "v"(rv[2]), "v"(rv[3]));
#pragma unroll
        for (int r = 0; r < 4; ++r) sh_q[(4 * g + r) * KS + 16 * kb + cl] = rv[r];
    }
    mfma_settle();
    __syncthreads();

    // 4. Z = R S0^T and the value sums W V on the matrix cores; o_k = Gam_k Z_k + (W V)_k
    const float4 gm4 = ld4(sh_gam + 4 * g);
    const float gm[4] = {gm4.x, gm4.y, gm4.z, gm4.w};
#pragma unroll
    for (int ib = 0; ib < IBW; ++ib) {
        const int i = 16 * (wv * IBW + ib) + cl;
        v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const float4 rv = ld4(sh_q + cl * KS + 16 * kb + 4 * g);   // A: R[c][16 kb + 4 g + r]
            z = mfma4(rv.x, s[ib][kb].x, z);
            z = mfma4(rv.y, s[ib][kb].y, z);
            z = mfma4(rv.z, s[ib][kb].z, z);
            z = mfma4(rv.w, s[ib][kb].w, z);
        }
        v4f u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jb = 0; jb < NTM; ++jb) {
            const float *vc = sh_v + (vb + 16 * jb + 4 * g) * VS + i;       // B: V[16 jb + 4 g + r][i]
#pragma unroll
            for (int r = 0; r < 4; ++r) u = mfma4(wa[jb][r], vc[r * VS], u);
        }
        float ov[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ov[r] = gm[r] * z[r] + u[r];   // draft k = 4 g + r, row i
        // the accumulators are read here, not inside the conditional stores
        asm volatile("" ::"v"(ov[0]), "v"(ov[1]), "v"(ov[2]), "v"(ov[3]));
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (4 * g + r < K) a.o[((size_t)(4 * g + r) * BH + c.bh) * DV + i] = ov[r];
    }

    // 5. append the drafts as entries len_e .. ne - 1 (every ring read is done), with non-temporal
    //    stores (measured faster here; the replay's single append measured no faster with them)
    const int dr0 = vb + len_e;             // row of draft 0
    for (int i = t; i < K * KF; i += TPB) {
        const int k = i / KF, o = (i - k * KF) * 4;
        st4_nt(a.ring.k + (c.rh + (head_e + len_e + k) % W) * DK + o, ld4(sh_k + (dr0 + k) * KS + o));
    }
    for (int i = t; i < K * VF; i += TPB) {
        const int k = i / VF, o = (i - k * VF) * 4;
        st4_nt(a.ring.v + (c.rh + (head_e + len_e + k) % W) * DV + o, ld4(sh_v + (dr0 + k) * VS + o));
    }
    for (int k = t; k < K; k += TPB) {
        const size_t slot = c.rh + (head_e + len_e + k) % W;
        a.ring.beta[slot] = sh_be[dr0 + k];
        a.ring.alpha[slot] = sh_al[dr0 + k];
    }
    if (c.h == 0 && t == 0) {
        a.bk.out[c.b] = head_e;
        a.bk.out[B + c.b] = len_e;
        a.bk.out[2 * B + c.b] = K;
    }
}

template <int DV, int DK>
size_t gdn_decode_lds(int W)
{
    const size_t replay = gdn_replay_lds<DV, DK>(W);
    const size_t fold = gdn_fold_lds<DV, DK>(W);
    return 4 * (replay > fold ? replay : fold);
}

template <int DV, int DK>
hipError_t go_decode(const GdnStepArgs &a, int mode, hipStream_t s)
{
    const dim3 grid(a.d.B * a.d.H), block(TileShape<DV, DK>::TPB);
    const size_t lds = gdn_decode_lds<DV, DK>(a.d.W);
    if (mode == 0) hipLaunchKernelGGL((k_gdn_decode<DV, DK, 0>), grid, block, lds, s, a);
    else if (mode == 1) hipLaunchKernelGGL((k_gdn_decode<DV, DK, 1>), grid, block, lds, s, a);
    else if (a.d.W > 16) hipLaunchKernelGGL((k_gdn_decode<DV, DK, 2, 2>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((k_gdn_decode<DV, DK, 2, 1>), grid, block, lds, s, a);
    return hipGetLastError();
}

template <int DV, int DK>
size_t gdn_verify_lds_bytes(int W)
{
    if (W <= 16) return 4 * (size_t)gdn_verify_lds<DV, DK, 1>();
    const size_t out = gdn_verify_lds<DV, DK, 2>(), fold = gdn_fold_lds<DV, DK>(W);
    return 4 * (out > fold ? out : fold);
}

template <int DV, int DK>
hipError_t go_verify(const GdnStepArgs &a, hipStream_t s)
{
    const dim3 grid(a.d.B * a.d.H), block(TileShape<DV, DK>::TPB);
    const size_t lds = gdn_verify_lds_bytes<DV, DK>(a.d.W);
    if (a.d.W > 16) hipLaunchKernelGGL((k_gdn_verify<DV, DK, 2>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((k_gdn_verify<DV, DK, 1>), grid, block, lds, s, a);
    return hipGetLastError();
}

template <int DV, int DK>
hipError_t go_fold(const GdnFoldArgs &a, hipStream_t s)
{
    const dim3 grid(a.d.B * a.d.H), block(TileShape<DV, DK>::TPB);
    const size_t lds = 4 * (size_t)gdn_fold_lds<DV, DK>(a.d.W);
    if (a.d.W > 16) hipLaunchKernelGGL((k_gdn_fold<DV, DK, 2>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((k_gdn_fold<DV, DK, 1>), grid, block, lds, s, a);
    return hipGetLastError();
}

template <int DV, int DK>
hipError_t go_rmw(const GdnRmwArgs &a, hipStream_t s)
{
    const dim3 grid(a.d.B * a.d.H), block(TileShape<DV, DK>::TPB);
    hipLaunchKernelGGL((k_gdn_rmw<DV, DK>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

// (d_v, d_k) pairs with compiled kernels.
#define RSSM_GDN_SHAPES(X) X(16, 16) X(64, 64) X(128, 128)

bool gdn_supported(int DV, int DK)
{
#define RSSM_C(v, k) if (DV == v && DK == k) return true;
    RSSM_GDN_SHAPES(RSSM_C)
#undef RSSM_C
    return false;
}

size_t gdn_lds_bytes(int DV, int DK, int W)
{
#define RSSM_C(v, k) if (DV == v && DK == k) { const size_t d = gdn_decode_lds<v, k>(W), \
    e = gdn_verify_lds_bytes<v, k>(W); return d > e ? d : e; }
    RSSM_GDN_SHAPES(RSSM_C)
#undef RSSM_C
    return 0;
}

hipError_t gdn_decode(const GdnStepArgs &a, int mode, hipStream_t s)
{
#define RSSM_C(v, k) if (a.d.DV == v && a.d.DK == k) return go_decode<v, k>(a, mode, s);
    RSSM_GDN_SHAPES(RSSM_C)
#undef RSSM_C
    return hipErrorInvalidValue;
}

hipError_t gdn_fold(const GdnFoldArgs &a, hipStream_t s)
{
#define RSSM_C(v, k) if (a.d.DV == v && a.d.DK == k) return go_fold<v, k>(a, s);
    RSSM_GDN_SHAPES(RSSM_C)
#undef RSSM_C
    return hipErrorInvalidValue;
}

hipError_t gdn_verify(const GdnStepArgs &a, hipStream_t s)
{
#define RSSM_C(v, k) if (a.d.DV == v && a.d.DK == k) return go_verify<v, k>(a, s);
    RSSM_GDN_SHAPES(RSSM_C)
#undef RSSM_C
    return hipErrorInvalidValue;
}

hipError_t gdn_rmw(const GdnRmwArgs &a, hipStream_t s)
{
#define RSSM_C(v, k) if (a.d.DV == v && a.d.DK == k) return go_rmw<v, k>(a, s);
    RSSM_GDN_SHAPES(RSSM_C)
#undef RSSM_C
    return hipErrorInvalidValue;
}

}  // namespace rssm
