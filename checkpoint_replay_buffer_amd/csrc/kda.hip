// kda.hip -- Kimi Delta Attention ReplaySSM decode kernels for gfx950.
//
// Kimi Delta Attention is the third SSM layer type of the hybrids ReplaySSM targets
// (news.hamidun.com item "NVIDIA présente ReplaySSM...", section "Pourquoi les hybrides sont
// devenus la norme"); the pages give no formula. Read as the Gated DeltaNet delta rule with one
// forget gate per key channel: per (b, h) the state S is d_v x d_k (row i = output channel) and
//     S_t = S_{t-1} diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t,
// with a_t in (0, 1]^{d_k}. The ring keeps each entry's k, v, beta and gate vector a.
//
// Replay. For m buffered entries 0..m-1 (newest last) the state is S0 M_0 ... M_{m-1} plus the
// entries' rank-1 terms carried through the later M_i, M_i = diag(a_i) (I - beta_i k_i k_i^T).
// Applied to q from the right: keep r (initially q); for j = m-1 down to 0 take c_j = k_j . r,
// note beta_j c_j, and replace r by a_j o (r - beta_j c_j k_j); then
//     o = S0 r + sum_j beta_j c_j v_j.
// The gates act on r channel by channel, so the recursion is m dependent steps of one wave (a
// dot over d_k and a vector update); every wave runs it on its own copy, before the checkpoint is
// needed. The checkpoint is read once (S0 r) and never written.
//
// Fold (consolidation). The entries are applied to the register-resident tile in order, each a
// column scaling by a_j, a row dot with k_j and a rank-1 update: the recurrence itself, on the
// vector units. Per (b, h) it reads and writes the tile once for all W entries.
//
// Tile map and checkpoint layout as the Gated DeltaNet kernels (mfma_tile.h, gdn_layout.h): lane
// (g, c) of wave w holds S[16 (w IBW + ib) + c][16 kb + 4 g .. +3], and a checkpoint tile is
// stored so that each of those float4 loads is part of a 1 KB contiguous wave access.
#include "dev_common.h"
#include "internal.h"
#include "tile_order.h"
#include "mfma_tile.h"
#include "gdn_layout.h"
#include "gdn_chunk.h"

namespace rssm {
namespace {

struct KTile {
    int b, h, t, W;
    size_t bh, rh;
};

// The lane's float4s of a d_v x d_k tile in the map of mfma_tile.h.
template <int DV, int DK>
using TileRegs = float4[MfmaTile<DV, DK>::IBW][MfmaTile<DV, DK>::KB];

__device__ __forceinline__ KTile make_ktile(const GdnDims &d, TileOrder order)
{
    KTile c;
    const int tile = tile_of(blockIdx.x, d.B * d.H, order, run_tiles(d.DV * d.DK));
    c.b = tile / d.H;
    c.h = tile - c.b * d.H;
    c.t = threadIdx.x;
    c.W = d.W;
    c.bh = (size_t)tile;
    c.rh = c.bh * d.W;
    return c;
}

__device__ __forceinline__ float lane_of(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over the 64 lanes of the wave, returned wave-uniform: the DPP butterfly inside each 16-lane
// row, then the four row sums read from lanes 0, 16, 32 and 48. No LDS crossbar round trip, which
// the dependent chain of such sums in the recursion below would otherwise wait on at every entry.
// Every lane must take part.
__device__ __forceinline__ float wave_sum(float v)
{
    v = group_sum<16>(v);
    const int b = __float_as_int(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

// Columns of r per lane in the recursion: lane l holds columns CPL l .. CPL l + CPL - 1 (lanes
// past d_k / CPL hold zeros).
template <int DK>
struct RCols {
    static constexpr int CPL = DK >= 64 ? DK / 64 : 1;
    static_assert(CPL == 1 || CPL == 2, "r columns per lane");
};

// r-recursion of one wave over entries m-1 .. 0 of the staged rows (key, gate rows of stride KS):
// r starts as the query (qrow, stride-1, d_k floats), lane j < m returns beta_j c_j in `bc`, and
// the final r is written to rout (d_k floats). bel holds beta_j on lane j. m is wave-uniform.
template <int DK>
__device__ __forceinline__ float kda_recursion(const float *sh_k, const float *sh_a, int KS,
                                               const float *qrow, float bel, int m, float *rout)
{
    constexpr int CPL = RCols<DK>::CPL;
    const int lane = threadIdx.x & 63, col = lane * CPL;
    const bool on = col < DK;
    float r0 = on ? qrow[col] : 0.f, r1 = (CPL == 2 && on) ? qrow[col + 1] : 0.f;
    float bc = 0.f;
    // the key and gate values of entry j, loaded one entry ahead of their use
    auto rows = [&](int j, float &k0, float &k1, float &a0, float &a1) {
        k0 = k1 = a0 = a1 = 0.f;
        if (on && j >= 0) {
            if constexpr (CPL == 2) {
                const float2 kv = *reinterpret_cast<const float2 *>(sh_k + j * KS + col);
                const float2 av = *reinterpret_cast<const float2 *>(sh_a + j * KS + col);
                k0 = kv.x; k1 = kv.y; a0 = av.x; a1 = av.y;
            } else {
                k0 = sh_k[j * KS + col];
                a0 = sh_a[j * KS + col];
            }
        }
    };
    float nk0, nk1, na0, na1;
    rows(m - 1, nk0, nk1, na0, na1);
    for (int j = m - 1; j >= 0; --j) {
        const float k0 = nk0, k1 = nk1, a0 = na0, a1 = na1;
        rows(j - 1, nk0, nk1, na0, na1);
        const float c = wave_sum(k0 * r0 + k1 * r1);
        const float b = lane_of(bel, j) * c;
        if (lane == j) bc = b;
        r0 = a0 * (r0 - b * k0);
        r1 = a1 * (r1 - b * k1);
    }
    if (on) {
        if constexpr (CPL == 2) *reinterpret_cast<float2 *>(rout + col) = make_float2(r0, r1);
        else rout[col] = r0;
    }
    return bc;
}

__device__ __forceinline__ void wave_sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Entry rows staged in LDS: key, gate and value rows of up to NE entries, with row strides KS and
// VS (padded), and beta per entry.
template <int DV, int DK>
struct Rows {
    static constexpr int KS = DK + 4, VS = DV + 4;
    static constexpr int floats(int ne) { return ne * (2 * KS + VS) + ne; }
};

// Float4 unit i of the rows of n entries (ring entries [0, nring) from slot `head`, then extra
// entries whose rows sit token-major in xk / xa / xv, `xstride` tiles apart): its global source
// and its LDS destination. Each entry has KF key, KF gate and VF value units, in that order.
template <int DV, int DK>
struct EntryRows {
    static constexpr int KF = DK / 4, VF = DV / 4, RF = 2 * KF + VF;
    const GdnRing &ring;
    const KTile &c;
    int head, nring;
    const float *xk, *xa, *xv;
    size_t xstride;
    float *sh_k, *sh_a, *sh_v;

    __device__ __forceinline__ const float *src(int i) const
    {
        const int j = i / RF, u = i - j * RF;
        const bool ringe = j < nring;
        const size_t rs = c.rh + (head + j) % c.W;            // ring slot row
        const size_t xr = (size_t)(j - nring) * xstride;      // extra entry, in tiles
        if (u < KF) return ringe ? ring.k + rs * DK + 4 * u : xk + xr * DK + 4 * u;
        if (u < 2 * KF) return ringe ? ring.alpha + rs * DK + 4 * (u - KF) : xa + xr * DK + 4 * (u - KF);
        return ringe ? ring.v + rs * DV + 4 * (u - 2 * KF) : xv + xr * DV + 4 * (u - 2 * KF);
    }
    __device__ __forceinline__ float *dst(int i) const
    {
        const int j = i / RF, u = i - j * RF;
        if (u < KF) return sh_k + j * Rows<DV, DK>::KS + 4 * u;
        if (u < 2 * KF) return sh_a + j * Rows<DV, DK>::KS + 4 * (u - KF);
        return sh_v + j * Rows<DV, DK>::VS + 4 * (u - 2 * KF);
    }
};

// Stage the rows of n entries into LDS. The units of the first 16 entries are loaded into
// registers, then `before_store` runs (the caller issues the checkpoint read there, so that it
// streams in while the rows are written to LDS: vector loads complete in issue order), then the
// rows go to LDS; entries past 16 are staged after it. All threads call it.
template <int DV, int DK, int TPB, typename Fn>
__device__ __forceinline__ void stage_rows(const EntryRows<DV, DK> &er, int n, Fn before_store)
{
    constexpr int RF = EntryRows<DV, DK>::RF;
    constexpr int XQ = (16 * RF + TPB - 1) / TPB;
    const int t = threadIdx.x, nu = n * RF;
    float4 xs[XQ];
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
        const int i = t + q * TPB;
        xs[q] = i < nu ? ld4(er.src(i)) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    before_store();
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
        const int i = t + q * TPB;
        if (i < nu) st4(er.dst(i), xs[q]);
    }
    for (int i = t + XQ * TPB; i < nu; i += TPB) st4(er.dst(i), ld4(er.src(i)));
}

// Waves per SIMD the kernels that fold are compiled for: three 8-wave workgroups per compute unit
// at 128 x 128 (at most 80 VGPRs), the compiler's choice otherwise.
template <int DV, int DK>
struct KdaFoldOcc {
    static constexpr int WPE = TileShape<DV, DK>::TPB == 512 ? 6 : 1;
};

// Fold entries 0..n-1 (staged in LDS, oldest first) into the register tile: for each entry,
// scale the columns by its gate, form (S k) per row, add beta (v - S k) k^T. No barrier.
template <int DV, int DK>
__device__ __forceinline__ void kda_fold_tile(TileRegs<DV, DK> &s,
                                              const float *sh_k, const float *sh_a, const float *sh_v,
                                              const float *sh_be, int n)
{
    using F = MfmaTile<DV, DK>;
    using RW = Rows<DV, DK>;
    constexpr int IBW = F::IBW, KB = F::KB;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, cl = lane & 15;
    for (int j = 0; j < n; ++j) {
        const float *kr = sh_k + j * RW::KS + 4 * g, *ar = sh_a + j * RW::KS + 4 * g;
        const float be = sh_be[j];
#pragma unroll
        for (int ib = 0; ib < IBW; ++ib) {
            const int row = 16 * (wv * IBW + ib) + cl;
            float p = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const float4 a4 = ld4(ar + 16 * kb), k4 = ld4(kr + 16 * kb);
                float4 &x = s[ib][kb];
                x.x *= a4.x; x.y *= a4.y; x.z *= a4.z; x.w *= a4.w;
                p += x.x * k4.x + x.y * k4.y + x.z * k4.z + x.w * k4.w;
            }
            p += bfly<16>(p);
            p += __shfl_xor(p, 32);
            const float cf = be * (sh_v[j * RW::VS + row] - p);
            int ko = j * RW::KS + 4 * g;
            asm volatile("" : "+v"(ko));
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const float4 k4 = ld4(sh_k + ko + 16 * kb);
                float4 &x = s[ib][kb];
                x.x += cf * k4.x; x.y += cf * k4.y; x.z += cf * k4.z; x.w += cf * k4.w;
            }
        }
    }
}

// The fold on the matrix cores. With Gam_j = a_0 o ... o a_j the gates' running product over the
// entries (per key channel), kh_j = k_j o Gam_j, kt_j = k_j / Gam_j and A[t][j] = kh_t . kt_j, the n
// entries applied in order give (the chunk form of the Kimi Delta Attention prefill)
//     S <- (S + U^T Kt) diag(Gam_{n-1}),   U = T (V - Kh S^T),
// with T the lower-triangular factor of the delta rule's WY form taken over A (gdn_chunk.h). The
// ratios Gam_t / Gam_j sit on the two operands, so the form is taken when every channel's product
// stays at or above 2^-64 (then 1 / Gam_j <= 2^64); otherwise, and for more than 16 entries, the
// entries are folded one by one on the vector units (kda_fold_tile).
constexpr float kMinGamFold = 0x1p-64f;

// LDS floats of the matrix-core fold beside the staged rows: kh and kt rows [16][d_k+4], beta of 16
// rows, the A and T blocks [16][20], Gam [d_k] and a flag per wave.
template <int DV, int DK>
__host__ __device__ constexpr int kda_mfold_floats()
{
    return 2 * kChunk * (DK + 4) + kChunk + 2 * kChunk * kTS + DK + 16;
}

// Fold entries 0..n-1 (rows staged in LDS as for kda_fold_tile, oldest first) into the register
// tile, then hand the tile to `done` (which stores it). mf: whether the matrix-core form may be used
// (its LDS `ext` of kda_mfold_floats floats is there); n and mf are uniform over the workgroup. All
// threads call it; it holds two barriers on the matrix-core path, one on the other. Each path ends
// in its own call of `done`, so that no tile value is live where the paths join (a join there
// kept two copies of the tile in registers).
template <int DV, int DK, typename Done>
__device__ __forceinline__ void kda_fold_any(TileRegs<DV, DK> &s, const float *sh_k,
                                             const float *sh_a, const float *sh_v,
                                             const float *sh_be, int n, bool mf, float *ext,
                                             Done done)
{
    using F = MfmaTile<DV, DK>;
    using RW = Rows<DV, DK>;
    constexpr int IBW = F::IBW, KB = F::KB, NW = F::NW, KS = RW::KS, VS = RW::VS;
    constexpr int NA = KB >= 2 ? 2 : 1;
    const int t = threadIdx.x, lane = t & 63, g = lane >> 4, cl = lane & 15;
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
    float *sh_kh = ext;                        // [16][KS]
    float *sh_kt = sh_kh + kChunk * KS;        // [16][KS]
    float *sh_b = sh_kt + kChunk * KS;         // [16]  beta, 0 past n
    float *sh_A = sh_b + kChunk;               // [16][kTS]
    float *sh_T = sh_A + kChunk * kTS;         // [16][kTS]
    float *sh_gam = sh_T + kChunk * kTS;       // [DK]
    int *sh_flag = reinterpret_cast<int *>(sh_gam + DK);   // [NW]

    // 1. one key channel per thread: the running product, kh and kt (zero rows past n), Gam_{n-1};
    //    then one call site of the vector fold (a second inlined copy costs registers)
    int slow = 1;
    if (mf && n <= kChunk) {
        bool bad = false;
        if (t < DK) {
            float gm = 1.f;
            for (int j = 0; j < kChunk; ++j) {
                float kh = 0.f, kt = 0.f;
                if (j < n) {
                    gm *= sh_a[j * KS + t];
                    const float kv = sh_k[j * KS + t];
                    kh = kv * gm;
                    kt = kv * __builtin_amdgcn_rcpf(gm);
                }
                sh_kh[j * KS + t] = kh;
                sh_kt[j * KS + t] = kt;
            }
            sh_gam[t] = gm;
            bad = !(gm >= kMinGamFold);
        }
        if (t < kChunk) sh_b[t] = t < n ? sh_be[t] : 0.f;
        const unsigned long long bw = __ballot(bad);
        if (lane == 0) sh_flag[wv] = bw != 0;
        __syncthreads();
        slow = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) slow |= sh_flag[w];
    }
    if (slow) {
        kda_fold_tile<DV, DK>(s, sh_k, sh_a, sh_v, sh_be, n);
        done(s);
        return;
    }

    // 2. wave 0: A = Kh Kt^T on the matrix cores and T in registers; every wave:
    //    Z = V - Kh S^T for its i-blocks (rows past n zero)
    if (wv == 0) {
        const v4f ak = row_dots16<KB, KS, NA, false>(sh_kh, sh_kt);      // kh_{4g+r} . kt_c
#pragma unroll
        for (int r = 0; r < 4; ++r) sh_A[(4 * g + r) * kTS + cl] = ak[r];
        wave_sync_lds();
        t_solve_regs<kChunk, kTS, kTS>(sh_A, sh_b, sh_T);
    }
    v4f fz[IBW];
#pragma unroll
    for (int ib = 0; ib < IBW; ++ib) {
        const int i = 16 * (wv * IBW + ib) + cl;
        v4f fp[NA];
#pragma unroll
        for (int p = 0; p < NA; ++p) fp[p] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const float4 kv = ld4(sh_kh + cl * KS + 16 * kb + 4 * g);
            v4f &f = fp[kb % NA];
            f = mfma4(kv.x, s[ib][kb].x, f);
            f = mfma4(kv.y, s[ib][kb].y, f);
            f = mfma4(kv.z, s[ib][kb].z, f);
            f = mfma4(kv.w, s[ib][kb].w, f);
        }
        const v4f acc = tree_sum<NA>(fp);      // (S kh_q)[i] for q = 4 g + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int q = 4 * g + r;
            fz[ib][r] = q < n ? sh_v[q * VS + i] - acc[r] : 0.f;
        }
    }
    __syncthreads();

    // 3. U = T Z, S <- (S + U^T Kt) diag(Gam_{n-1})
#pragma unroll
    for (int ib = 0; ib < IBW; ++ib) {
        const float4 tv = ld4(sh_T + cl * kTS + 4 * g);                    // T[t = c][4 g + r]
        v4f cz = {0.f, 0.f, 0.f, 0.f};
        cz = mfma4(tv.x, fz[ib][0], cz);
        cz = mfma4(tv.y, fz[ib][1], cz);
        cz = mfma4(tv.z, fz[ib][2], cz);
        cz = mfma4(tv.w, fz[ib][3], cz);       // U[t][i] for t = 4 g + r, i = 16 ib' + c
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            v4f u = {s[ib][kb].x, s[ib][kb].y, s[ib][kb].z, s[ib][kb].w};
            const float *kr = sh_kt + (4 * g) * KS + 16 * kb + cl;           // kt[t][16 kb + c]
            u = mfma4(kr[0], cz[0], u);
            u = mfma4(kr[KS], cz[1], u);
            u = mfma4(kr[2 * KS], cz[2], u);
            u = mfma4(kr[3 * KS], cz[3], u);
            const float4 gs = ld4(sh_gam + 16 * kb + 4 * g);
            s[ib][kb] = make_float4(gs.x * u[0], gs.y * u[1], gs.z * u[2], gs.w * u[3]);
        }
    }
    mfma_settle();
    done(s);
}

// o[row] = S r (r in LDS, d_k floats) for the wave's rows, plus extra[row] (added by the g = 0
// lane, which writes); the four lanes of a row are added by two exchanges.
template <int DV, int DK>
__device__ __forceinline__ float tile_gemv_row(const TileRegs<DV, DK> &s,
                                               int ib, const float *r)
{
    constexpr int KB = MfmaTile<DV, DK>::KB;
    const int g = (threadIdx.x & 63) >> 4;
    float p = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const float4 rq = ld4(r + 16 * kb + 4 * g);
        p += s[ib][kb].x * rq.x + s[ib][kb].y * rq.y + s[ib][kb].z * rq.z + s[ib][kb].w * rq.w;
    }
    return p;
}

// ------------------------------------------------------------------------------------------
// decode
// ------------------------------------------------------------------------------------------
// Start of the matrix-core fold's LDS after rows of `floats` floats (16-byte aligned).
__host__ __device__ constexpr int kda_ext_off(int floats) { return (floats + 3) & ~3; }

template <int DV, int DK>
__host__ __device__ constexpr int kda_decode_lds(int W, bool fold)
{
    // rows of up to W + 1 entries (a fold after a full commit takes the ring and the token); the
    // replay adds the query and per wave r [DK] and the coefficients [W + 1], the step that folds
    // the matrix-core fold's blocks (W <= 16)
    const int rows = Rows<DV, DK>::floats(W + 1);
    const int replay = rows + DK + (MfmaTile<DV, DK>::NW) * (DK + 36);
    const int mfold = kda_ext_off(rows) + (W <= kChunk ? kda_mfold_floats<DV, DK>() : 0);
    return fold && mfold > replay ? mfold : replay;
}

// Replay step (len + 1 < W). LOAD: read the tile here after the ring loads went out.
template <int DV, int DK, bool LOAD>
__device__ __forceinline__ void kda_replay(const GdnStepArgs &a, const KTile &c, int head, int len,
                                           TileRegs<DV, DK> &s,
                                           float *smem)
{
    using F = MfmaTile<DV, DK>;
    using RW = Rows<DV, DK>;
    constexpr int TPB = F::TPB, IBW = F::IBW, NW = F::NW;
    constexpr int KF = DK / 4, VF = DV / 4;
    const int W = c.W, t = c.t, m = len + 1, lane = t & 63;
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6), g = lane >> 4, cl = lane & 15;
    float *sh_k = smem;                          // [W+1][KS]
    float *sh_a = sh_k + (W + 1) * RW::KS;       // [W+1][KS]
    float *sh_v = sh_a + (W + 1) * RW::KS;       // [W+1][VS]
    float *sh_be = sh_v + (W + 1) * RW::VS;      // [W+1]
    float *sh_q = sh_be + (W + 1);               // [DK]
    float *sh_r = sh_q + DK + wv * (DK + 36);    // [DK]  this wave's r
    float *sh_cv = sh_r + DK;                    // [36]  this wave's beta_j c_j, 0 past m
    (void)NW;

    const float *qt = a.q + c.bh * DK, *kt = a.k + c.bh * DK, *vt = a.v + c.bh * DV;
    const float *at = a.alpha + c.bh * DK;
    const float bet = a.beta[c.bh];
    const int slot = (head + len) % W;
    const float bel = lane < len ? a.ring.beta[c.rh + (head + lane) % W] : (lane == len ? bet : 0.f);
    // the rows (ring entries and the token) are loaded first, the checkpoint after them
    const EntryRows<DV, DK> er{a.ring, c, head, len, kt, at, vt, 0, sh_k, sh_a, sh_v};
    stage_rows<DV, DK, TPB>(er, m, [&] {
        if constexpr (LOAD) ckpt_load<DV>(s, a.S0 + c.bh * (size_t)(DV * DK), t);
    });
    for (int i = t; i < KF; i += TPB) st4(sh_q + 4 * i, ld4(qt + 4 * i));
    __syncthreads();

    const float bc = kda_recursion<DK>(sh_k, sh_a, RW::KS, sh_q, bel, m, sh_r);
    if (lane < 36) sh_cv[lane] = lane < m ? bc : 0.f;
    wave_sync_lds();

    // o = S0 r + sum_j beta_j c_j v_j: lane (g, c) takes its columns of each k-block and the
    // entries j = g mod 4
#pragma unroll
    for (int ib = 0; ib < IBW; ++ib) {
        const int row = 16 * (wv * IBW + ib) + cl;
        float u = 0.f;
        for (int j = g; j < m; j += 4) u += sh_cv[j] * sh_v[j * RW::VS + row];
        float p = tile_gemv_row<DV, DK>(s, ib, sh_r) + u;
        p += bfly<16>(p);
        p += __shfl_xor(p, 32);
        if (g == 0) a.o[c.bh * DV + row] = p;
    }

    // append the token as entry len (its slot is none of the entries read above)
    for (int i = t; i < KF; i += TPB) {
        st4(a.ring.k + (c.rh + slot) * DK + 4 * i, ld4(sh_k + len * RW::KS + 4 * i));
        st4(a.ring.alpha + (c.rh + slot) * DK + 4 * i, ld4(sh_a + len * RW::KS + 4 * i));
    }
    for (int i = t; i < VF; i += TPB) st4(a.ring.v + (c.rh + slot) * DV + 4 * i, ld4(sh_v + len * RW::VS + 4 * i));
    if (t == 0) a.ring.beta[c.rh + slot] = bet;
}

// Decode step whose token fills the ring: fold the ring entries and the token, store, o = S q.
template <int DV, int DK>
__device__ __forceinline__ void kda_fold_decode(const GdnStepArgs &a, const KTile &c, int head,
                                                int len, float *smem)
{
    using F = MfmaTile<DV, DK>;
    using RW = Rows<DV, DK>;
    constexpr int TPB = F::TPB, IBW = F::IBW, KB = F::KB;
    const int W = c.W, t = c.t, n = len + 1, lane = t & 63, wv = t >> 6, g = lane >> 4, cl = lane & 15;
    float *sh_k = smem;
    float *sh_a = sh_k + (W + 1) * RW::KS;
    float *sh_v = sh_a + (W + 1) * RW::KS;
    float *sh_be = sh_v + (W + 1) * RW::VS;
    float *S0 = a.S0 + c.bh * (size_t)(DV * DK);
    const float *qt = a.q + c.bh * DK;
    for (int j = t; j < n; j += TPB) sh_be[j] = j < len ? a.ring.beta[c.rh + (head + j) % W] : a.beta[c.bh];
    float4 s[IBW][KB];
    const EntryRows<DV, DK> er{a.ring, c, head, len, a.k + c.bh * DK, a.alpha + c.bh * DK,
                               a.v + c.bh * DV, 0, sh_k, sh_a, sh_v};
    stage_rows<DV, DK, TPB>(er, n, [&] { ckpt_load<DV>(s, S0, t); });
    __syncthreads();
    kda_fold_any<DV, DK>(s, sh_k, sh_a, sh_v, sh_be, n, W <= kChunk,
                         smem + kda_ext_off(Rows<DV, DK>::floats(W + 1)), [&](TileRegs<DV, DK> &f) {
        ckpt_store<DV>(f, S0, t);
#pragma unroll
        for (int ib = 0; ib < IBW; ++ib) {
            float p = tile_gemv_row<DV, DK>(f, ib, qt);
            p += bfly<16>(p);
            p += __shfl_xor(p, 32);
            if (g == 0) a.o[c.bh * DV + 16 * (wv * IBW + ib) + cl] = p;
        }
    });
}

// Variants as the Gated DeltaNet decode: 0 = every sequence at (a.uhead, a.ulen), none folds;
// 1 = none folds (positions read from the device); 2 = any sequence may fold.
template <int DV, int DK, int MODE>
__global__ void __launch_bounds__((TileShape<DV, DK>::TPB), (MODE == 2 ? KdaFoldOcc<DV, DK>::WPE : 1)) k_kda_decode(GdnStepArgs a)
{
    using F = MfmaTile<DV, DK>;
    extern __shared__ float smem[];
    const KTile c = make_ktile(a.d, MODE == 2 ? kIdentity : kRuns);
    const int B = a.d.B, W = c.W;
    float4 s[F::IBW][F::KB];
    int head, len;
    bool fold = false;
    if constexpr (MODE == 0) {
        head = a.uhead;
        len = a.ulen;
        kda_replay<DV, DK, true>(a, c, head, len, s, smem);
    } else if constexpr (MODE == 1) {
        ckpt_load<DV>(s, a.S0 + c.bh * (size_t)(DV * DK), c.t);
        head = a.bk.in[c.b];
        len = a.bk.in[B + c.b];
        kda_replay<DV, DK, false>(a, c, head, len, s, smem);
    } else {
        head = a.bk.in[c.b];
        len = a.bk.in[B + c.b];
        fold = len + 1 >= W;
        if (!fold) kda_replay<DV, DK, true>(a, c, head, len, s, smem);
        else kda_fold_decode<DV, DK>(a, c, head, len, smem);
    }
    if (c.h == 0 && c.t == 0) {
        a.bk.out[c.b] = fold ? (head + len + 1) % W : head;
        a.bk.out[B + c.b] = fold ? 0 : len + 1;
        a.bk.out[2 * B + c.b] = 0;
    }
}

// ------------------------------------------------------------------------------------------
// consolidation / materialisation
// ------------------------------------------------------------------------------------------
template <int DV, int DK>
__host__ __device__ constexpr int kda_fold_lds(int W)
{
    return kda_ext_off(Rows<DV, DK>::floats(W)) + (W <= kChunk ? kda_mfold_floats<DV, DK>() : 0);
}

template <int DV, int DK>
__global__ void __launch_bounds__((TileShape<DV, DK>::TPB), (KdaFoldOcc<DV, DK>::WPE)) k_kda_fold(GdnFoldArgs a)
{
    using F = MfmaTile<DV, DK>;
    using RW = Rows<DV, DK>;
    constexpr int TPB = F::TPB, IBW = F::IBW, KB = F::KB;
    extern __shared__ float smem[];
    const KTile c = make_ktile(a.d, kIdentity);
    const int B = a.d.B, W = c.W, t = c.t;
    const int head = a.bk.in[c.b];
    const int len = a.bk.in[B + c.b];
    const int nd = a.bk.in[2 * B + c.b];
    const bool fold = len >= (a.min_len > 1 ? a.min_len : 1);
    if (!a.out && c.h == 0 && t == 0) {
        a.bk.out[c.b] = fold ? (head + len) % W : head;
        a.bk.out[B + c.b] = fold ? 0 : len;
        a.bk.out[2 * B + c.b] = nd;
    }
    float *S0 = a.S0 + c.bh * (size_t)(DV * DK);
    if (!fold) {
        if (a.out) {
            float *dst = a.out + c.bh * (size_t)(DV * DK);
            for (int i = t; i < DV * DK / 4; i += TPB) {     // row-major from the checkpoint layout
                const int row = 4 * i / DK, col = 4 * i - row * DK;
                st4(dst + 4 * i, ld4(S0 + ckpt_offset(row, col, DV)));
            }
        }
        return;
    }
    float *sh_k = smem;
    float *sh_a = sh_k + W * RW::KS;
    float *sh_v = sh_a + W * RW::KS;
    float *sh_be = sh_v + W * RW::VS;
    for (int j = t; j < len; j += TPB) sh_be[j] = a.ring.beta[c.rh + (head + j) % W];
    float4 s[IBW][KB];
    const EntryRows<DV, DK> er{a.ring, c, head, len, a.ring.k, a.ring.alpha, a.ring.v, 0, sh_k, sh_a, sh_v};
    stage_rows<DV, DK, TPB>(er, len, [&] { ckpt_load<DV>(s, S0, t); });
    __syncthreads();
    kda_fold_any<DV, DK>(s, sh_k, sh_a, sh_v, sh_be, len, W <= kChunk,
                         smem + kda_ext_off(Rows<DV, DK>::floats(W)), [&](TileRegs<DV, DK> &f) {
        if (a.out) {
#pragma unroll
            for (int ib = 0; ib < IBW; ++ib) {
                float *p = a.out + c.bh * (size_t)(DV * DK) + mfma_tile_offset<DV, DK>(t, ib);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) st4(p + 16 * kb, f[ib][kb]);
            }
        } else {
            ckpt_store<DV>(f, S0, t);
        }
    });
}

// ------------------------------------------------------------------------------------------
// speculative verify: K drafts, outputs only, checkpoint streamed once
// ------------------------------------------------------------------------------------------
// Drafts k = 0..K-1 become entries len_e + k; draft k's output is the replay over the first
// m_k = len_e + k + 1 entries with query q_k: one wave per draft runs the recursion, then the
// outputs of 16 drafts at a time are O = R S0^T + Cf V on the matrix cores, with R the rows r_k
// and Cf[k][j] = beta_j c_{k,j} (zero for j >= m_k). Sequences whose ring cannot take the drafts
// (len + K > W) first fold their len committed entries. NJB = 16-entry blocks of the ring.
template <int DV, int DK>
__host__ __device__ constexpr int kda_verify_lds(int W, int K)
{
    // rows of up to W entries (16 NJB, the value rows past the entries zeroed), the drafts'
    // queries (then their r rows) [K16][KS] and coefficients [K16][16 NJB + 4]; the fold of the
    // committed entries uses the same rows
    const int W16 = (W + 15) / 16 * 16, K16 = (K + 15) / 16 * 16;
    return Rows<DV, DK>::floats(W16) + K16 * (DK + 4) + K16 * (W16 + 4);
}

// Compiled for eight waves per SIMD at 128 x 128 (at most 64 VGPRs, no spills): four workgroups per
// compute unit, which its LDS allows at W <= 16 (three at 65 VGPRs).
template <int DV, int DK, int NJB>
__global__ void __launch_bounds__((TileShape<DV, DK>::TPB), (TileShape<DV, DK>::TPB == 512 ? 8 : 1)) k_kda_verify(GdnStepArgs a)
{
    using F = MfmaTile<DV, DK>;
    using RW = Rows<DV, DK>;
    constexpr int TPB = F::TPB, IBW = F::IBW, KB = F::KB, NW = F::NW;
    constexpr int KF = DK / 4, VF = DV / 4, QS = DK + 4;
    constexpr int NE = 16 * NJB, CS = NE + 4;   // entry rows on the matrix cores
    constexpr int NA = KB >= 2 ? 2 : 1;
    extern __shared__ float smem[];
    const KTile c = make_ktile(a.d, kRuns);
    const int B = a.d.B, W = c.W, K = a.ntok, t = c.t, lane = t & 63;
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6), g = lane >> 4, cl = lane & 15;
    const size_t BH = (size_t)B * a.d.H;
    const int head = a.bk.in[c.b], len = a.bk.in[B + c.b];
    const bool prefold = len + K > W;
    const int head_e = prefold ? (head + len) % W : head, len_e = prefold ? 0 : len;
    const int ne = len_e + K;
    const int K16 = (K + 15) & ~15;
    float *S0 = a.S0 + c.bh * (size_t)(DV * DK);
    float *sh_k = smem;                      // [NE][KS]
    float *sh_a = sh_k + NE * RW::KS;        // [NE][KS]
    float *sh_v = sh_a + NE * RW::KS;        // [NE][VS]
    float *sh_be = sh_v + NE * RW::VS;       // [NE]
    float *sh_q = sh_be + NE;                // [K16][QS]  q_k, then r_k
    float *sh_cf = sh_q + K16 * QS;          // [K16][CS]  beta_j c_{k,j}
    float4 s[IBW][KB];
    if (prefold) {
        for (int j = t; j < len; j += TPB) sh_be[j] = a.ring.beta[c.rh + (head + j) % W];
        const EntryRows<DV, DK> er{a.ring, c, head, len, a.ring.k, a.ring.alpha, a.ring.v, 0, sh_k, sh_a, sh_v};
        stage_rows<DV, DK, TPB>(er, len, [&] { ckpt_load<DV>(s, S0, t); });
        __syncthreads();
        kda_fold_tile<DV, DK>(s, sh_k, sh_a, sh_v, sh_be, len);
        ckpt_store<DV>(s, S0, t);
        __syncthreads();                     // the rows are restaged below
    }
    // committed entries [0, len_e) from the ring, then the K drafts (token-major, BH tiles apart);
    // the checkpoint is read after their loads went out (unless it was folded above); the value
    // rows past the entries are zeroed (their coefficients are zero, and 0 times stale LDS
    // contents could be a NaN)
    for (int j = t; j < ne; j += TPB)
        sh_be[j] = j < len_e ? a.ring.beta[c.rh + (head_e + j) % W] : a.beta[(size_t)(j - len_e) * BH + c.bh];
    const EntryRows<DV, DK> er{a.ring, c, head_e, len_e, a.k + c.bh * DK, a.alpha + c.bh * DK,
                               a.v + c.bh * DV, BH, sh_k, sh_a, sh_v};
    stage_rows<DV, DK, TPB>(er, ne, [&] { if (!prefold) ckpt_load<DV>(s, S0, t); });
    for (int i = t; i < (NE - ne) * VF; i += TPB) {
        const int j = i / VF, o = 4 * (i - j * VF);
        st4(sh_v + (ne + j) * RW::VS + o, make_float4(0.f, 0.f, 0.f, 0.f));
    }
    for (int i = t; i < K * KF; i += TPB) {
        const int k = i / KF, o = 4 * (i - k * KF);
        st4(sh_q + k * QS + o, ld4(a.q + ((size_t)k * BH + c.bh) * DK + o));
    }
    __syncthreads();

    // one wave per draft: r_k over the first m_k entries (written over q_k), coefficients
    const float bel = lane < ne ? sh_be[lane] : 0.f;
    for (int k = wv; k < K; k += NW) {
        const int mk = len_e + k + 1;
        const float bc = kda_recursion<DK>(sh_k, sh_a, RW::KS, sh_q + k * QS, bel, mk, sh_q + k * QS);
        if (lane < CS) sh_cf[k * CS + lane] = lane < mk ? bc : 0.f;
    }
    __syncthreads();

    // O = R S0^T + Cf V, 16 drafts at a time: lane (g, c) of i-block ib ends with draft
    // 16 db + 4 g + r, row i = 16 ib' + c (the rows of R and Cf past K only reach outputs past K)
    for (int db = 0; db < K16; db += 16) {
#pragma unroll
        for (int ib = 0; ib < IBW; ++ib) {
            const int i = 16 * (wv * IBW + ib) + cl;
            v4f zp[NA];
#pragma unroll
            for (int n = 0; n < NA; ++n) zp[n] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const float4 rv = ld4(sh_q + (db + cl) * QS + 16 * kb + 4 * g);   // A: R[c][16 kb + 4 g + r]
                v4f &z = zp[kb % NA];
                z = mfma4(rv.x, s[ib][kb].x, z);
                z = mfma4(rv.y, s[ib][kb].y, z);
                z = mfma4(rv.z, s[ib][kb].z, z);
                z = mfma4(rv.w, s[ib][kb].w, z);
            }
            v4f u = tree_sum<NA>(zp);
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const float *cf = sh_cf + (db + cl) * CS + 16 * jb + 4 * g;      // A: Cf[c][16 jb + 4 g + r]
                const float *vc = sh_v + (16 * jb + 4 * g) * RW::VS + i;       // B: V[16 jb + 4 g + r][i]
#pragma unroll
                for (int r = 0; r < 4; ++r) u = mfma4(cf[r], vc[r * RW::VS], u);
            }
            const float ov[4] = {u[0], u[1], u[2], u[3]};
            // the accumulators are read here, not inside the conditional stores
            asm volatile("" ::"v"(ov[0]), "v"(ov[1]), "v"(ov[2]), "v"(ov[3]));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int k = db + 4 * g + r;
                if (k < K) a.o[((size_t)k * BH + c.bh) * DV + i] = ov[r];
            }
        }
    }
    mfma_settle();

    // append the drafts as entries len_e .. ne - 1 (every ring read is done)
    for (int i = t; i < K * KF; i += TPB) {
        const int k = i / KF, o = 4 * (i - k * KF);
        const size_t slot = c.rh + (head_e + len_e + k) % W;
        st4_nt(a.ring.k + slot * DK + o, ld4(sh_k + (len_e + k) * RW::KS + o));
        st4_nt(a.ring.alpha + slot * DK + o, ld4(sh_a + (len_e + k) * RW::KS + o));
    }
    for (int i = t; i < K * VF; i += TPB) {
        const int k = i / VF, o = 4 * (i - k * VF);
        st4_nt(a.ring.v + (c.rh + (head_e + len_e + k) % W) * DV + o, ld4(sh_v + (len_e + k) * RW::VS + o));
    }
    for (int k = t; k < K; k += TPB) a.ring.beta[c.rh + (head_e + len_e + k) % W] = sh_be[len_e + k];
    if (c.h == 0 && t == 0) {
        a.bk.out[c.b] = head_e;
        a.bk.out[B + c.b] = len_e;
        a.bk.out[2 * B + c.b] = K;
    }
}

// ------------------------------------------------------------------------------------------
// conventional read-modify-write comparator (row-major state)
// ------------------------------------------------------------------------------------------
template <int DV, int DK>
__global__ void __launch_bounds__((TileShape<DV, DK>::TPB)) k_kda_rmw(GdnRmwArgs a)
{
    using M = Map4<DV, DK>;
    constexpr int R = M::R, LPR = M::LPR;
    __shared__ float sh_sk[DV];
    const KTile c = make_ktile(a.d, kRuns);
    const int t = c.t;
    const int rg = t / LPR, cg = t - rg * LPR, c0 = cg * 4;
    const size_t BH = (size_t)a.d.B * a.d.H, VK = (size_t)DV * DK;
    const size_t lo = (size_t)(rg * R) * DK + c0;          // lane block within a tile
    const size_t off = c.bh * VK + lo;
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
        const float be = a.beta[tk];
        const float4 kv = ld4(a.k + tk * DK + c0);
        const float4 qv = ld4(a.q + tk * DK + c0);
        const float4 av = ld4(a.alpha + tk * DK + c0);
        const float *vv = a.v + tk * DV;
        float part[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            S[r].x *= av.x; S[r].y *= av.y; S[r].z *= av.z; S[r].w *= av.w;
            part[r] = S[r].x * kv.x + S[r].y * kv.y + S[r].z * kv.z + S[r].w * kv.w;
        }
        int rsel;
        const float sk = row_reduce_scatter<R, LPR, false>(part, cg, rsel);
        if (row_writer<R, LPR>(cg)) sh_sk[rg * R + rsel] = sk;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = rg * R + r;
            const float cf = be * (vv[i] - sh_sk[i]);
            S[r].x += cf * kv.x; S[r].y += cf * kv.y; S[r].z += cf * kv.z; S[r].w += cf * kv.w;
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
// launchers
// ------------------------------------------------------------------------------------------
template <int DV, int DK>
hipError_t go_decode(const GdnStepArgs &a, int mode, hipStream_t s)
{
    const dim3 grid(a.d.B * a.d.H), block(TileShape<DV, DK>::TPB);
    const size_t lds = 4 * (size_t)kda_decode_lds<DV, DK>(a.d.W, mode == 2);
    if (mode == 0) hipLaunchKernelGGL((k_kda_decode<DV, DK, 0>), grid, block, lds, s, a);
    else if (mode == 1) hipLaunchKernelGGL((k_kda_decode<DV, DK, 1>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((k_kda_decode<DV, DK, 2>), grid, block, lds, s, a);
    return hipGetLastError();
}

template <int DV, int DK>
hipError_t go_fold(const GdnFoldArgs &a, hipStream_t s)
{
    const dim3 grid(a.d.B * a.d.H), block(TileShape<DV, DK>::TPB);
    const size_t lds = 4 * (size_t)kda_fold_lds<DV, DK>(a.d.W);
    hipLaunchKernelGGL((k_kda_fold<DV, DK>), grid, block, lds, s, a);
    return hipGetLastError();
}

template <int DV, int DK>
hipError_t go_verify(const GdnStepArgs &a, hipStream_t s)
{
    const dim3 grid(a.d.B * a.d.H), block(TileShape<DV, DK>::TPB);
    const size_t lds = 4 * (size_t)kda_verify_lds<DV, DK>(a.d.W, a.ntok);
    if (a.d.W > 16) hipLaunchKernelGGL((k_kda_verify<DV, DK, 2>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((k_kda_verify<DV, DK, 1>), grid, block, lds, s, a);
    return hipGetLastError();
}

template <int DV, int DK>
hipError_t go_rmw(const GdnRmwArgs &a, hipStream_t s)
{
    const dim3 grid(a.d.B * a.d.H), block(TileShape<DV, DK>::TPB);
    hipLaunchKernelGGL((k_kda_rmw<DV, DK>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

// (d_v, d_k) pairs with compiled kernels.
#define RSSM_KDA_SHAPES(X) X(16, 16) X(64, 64) X(128, 128)

bool kda_supported(int DV, int DK)
{
#define RSSM_C(v, k) if (DV == v && DK == k) return true;
    RSSM_KDA_SHAPES(RSSM_C)
#undef RSSM_C
    return false;
}

size_t kda_lds_bytes(int DV, int DK, int W, int K)
{
#define RSSM_C(v, k) if (DV == v && DK == k) { const size_t d = kda_decode_lds<v, k>(W, true), \
    e = kda_verify_lds<v, k>(W, K); return 4 * (d > e ? d : e); }
    RSSM_KDA_SHAPES(RSSM_C)
#undef RSSM_C
    return 0;
}

hipError_t kda_decode(const GdnStepArgs &a, int mode, hipStream_t s)
{
#define RSSM_C(v, k) if (a.d.DV == v && a.d.DK == k) return go_decode<v, k>(a, mode, s);
    RSSM_KDA_SHAPES(RSSM_C)
#undef RSSM_C
    return hipErrorInvalidValue;
}

hipError_t kda_fold(const GdnFoldArgs &a, hipStream_t s)
{
#define RSSM_C(v, k) if (a.d.DV == v && a.d.DK == k) return go_fold<v, k>(a, s);
    RSSM_KDA_SHAPES(RSSM_C)
#undef RSSM_C
    return hipErrorInvalidValue;
}

hipError_t kda_verify(const GdnStepArgs &a, hipStream_t s)
{
#define RSSM_C(v, k) if (a.d.DV == v && a.d.DK == k) return go_verify<v, k>(a, s);
    RSSM_KDA_SHAPES(RSSM_C)
#undef RSSM_C
    return hipErrorInvalidValue;
}

hipError_t kda_rmw(const GdnRmwArgs &a, hipStream_t s)
{
#define RSSM_C(v, k) if (a.d.DV == v && a.d.DK == k) return go_rmw<v, k>(a, s);
    RSSM_KDA_SHAPES(RSSM_C)
#undef RSSM_C
    return hipErrorInvalidValue;
}

}  // namespace rssm
