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
// Fold (WY form of the product of the rank-1 corrections), with gamma_t = prod_{i<=t} alpha_i:
//     y_t = beta_t (k_t - sum_{i<t} (k_i . k_t) y_i)
//     u_t = beta_t (v_t - sum_{i<t} (gamma_t / gamma_i) (k_i . k_t) u_i)
//     S0 <- gamma S0 + sum_t ((gamma / gamma_t) u_t - gamma S0 y_t) k_t^T.
// Both recurrences run down columns independently; S0 y_t uses the row reduce-scatter.
#include "dev_common.h"
#include "internal.h"

namespace rssm {
namespace {

struct GTile {
    int b, h, t, W;
    size_t bh, rh;
};

__device__ __forceinline__ GTile make_gtile(const GdnDims &d)
{
    GTile c;
    const int tile = blockIdx.x;
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

// Stage n entries (ring entries [0, nring) from slot `head`, then the token `tok` if given) of
// k, v, beta, alpha into LDS.
template <int DV, int DK, int TPB>
__device__ __forceinline__ void stage_entries(const GdnRing &ring, const GTile &c, int head, int nring,
                                              bool tok, const float *kt, const float *vt, float bet,
                                              float alt, float *sh_k, float *sh_v, float *sh_be,
                                              float *sh_al)
{
    const int W = c.W, t = c.t, n = nring + (tok ? 1 : 0);
    for (int j = t; j < n; j += TPB) {
        sh_be[j] = j < nring ? ring.beta[c.rh + (head + j) % W] : bet;
        sh_al[j] = j < nring ? ring.alpha[c.rh + (head + j) % W] : alt;
    }
    constexpr int KF = DK / 4, VF = DV / 4;
    for (int i = t; i < n * KF; i += TPB) {
        const int j = i / KF, q = (i - j * KF) * 4;
        st4(sh_k + j * DK + q, j < nring ? ld4(ring.k + (c.rh + (head + j) % W) * DK + q) : ld4(kt + q));
    }
    for (int i = t; i < n * VF; i += TPB) {
        const int j = i / VF, q = (i - j * VF) * 4;
        st4(sh_v + j * DV + q, j < nring ? ld4(ring.v + (c.rh + (head + j) % W) * DV + q) : ld4(vt + q));
    }
}

// Gram entries G[l][i] = k_l . k_i (l < i < n), row stride W1; with q != nullptr also
// u_j = k_j . q into sh_u. Lane groups of LPD lanes take one dot each.
template <int DK, int TPB>
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
            s = lds_dot<DK, TPB>(sh_k + l * DK, sh_q, lane);
        } else {
            upper_pair(d - nq, l, i);
            s = lds_dot<DK, TPB>(sh_k + l * DK, sh_k + i * DK, lane);
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

// LOAD = true: the checkpoint tile s is read here, after the ring loads went out (the ring position
// is known without a device read); LOAD = false: the caller already issued it.
template <int DV, int DK, int R, bool LOAD>
__device__ __forceinline__ void gdn_replay(const GdnStepArgs &a, const GTile &c, int head, int len,
                                           float4 (&s)[R], float *smem)
{
    constexpr int TPB = TileShape<DV, DK>::TPB;
    using M = Map4<DV, DK>;
    static_assert(R == M::R, "tile block");
    constexpr int LPR = M::LPR, DUP = LPR / R;
    constexpr int KF = DK / 4, VF = DV / 4;
    constexpr int XQ = (16 * (KF + VF) + TPB - 1) / TPB;   // float4 staged in registers (W <= 16)
    const int W = c.W, t = c.t, m = len + 1, W1 = W + 1, lane = t & 63;
    const int rg = t / LPR, cg = t - rg * LPR, c0 = cg * 4;
    float *sh_k = smem;                 // [m][DK]
    float *sh_v = sh_k + W * DK;        // [m][DV]
    float *sh_q = sh_v + W * DV;        // [DK]
    float *sh_G = sh_q + DK;            // [m][W1]  k_l . k_i, l < i
    float *sh_u = sh_G + W * W1;        // [m]      k_j . q

    const float *qt = a.q + c.bh * DK, *kt = a.k + c.bh * DK, *vt = a.v + c.bh * DV;
    const float bet = a.beta[c.bh], alt = a.alpha[c.bh];
    const int slot = (head + len) % W;
    // ring-side loads: beta / alpha of entry `lane` (every wave), k and v rows of all entries
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
    const float4 qv = ld4(qt + c0);
    if constexpr (LOAD) {
        const size_t off = c.bh * (size_t)(DV * DK) + (size_t)(rg * R) * DK + c0;
#pragma unroll
        for (int r = 0; r < R; ++r) s[r] = ld4_nt(a.S0 + off + (size_t)r * DK);
    }
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
    if (rg == 0) st4(sh_q + c0, qv);
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

    // r = q - sum_j beta_j c_j k_j on the lane's columns, then S0 r
    float4 rv = qv;
    for (int j = 0; j < m; ++j) {
        const float b = lane_value(bc, j);
        const float4 kj = ld4(sh_k + j * DK + c0);
        rv.x -= b * kj.x; rv.y -= b * kj.y; rv.z -= b * kj.z; rv.w -= b * kj.w;
    }
    float part[R];
#pragma unroll
    for (int r = 0; r < R; ++r) part[r] = s[r].x * rv.x + s[r].y * rv.y + s[r].z * rv.z + s[r].w * rv.w;
    int rsel;
    const float z = row_reduce_scatter<R, LPR>(part, cg, rsel);
    const int row = rg * R + rsel, k = cg & (DUP - 1);
    float acc = 0.f;
    for (int j = 0; j < m; ++j) {                         // split over the DUP lanes of the row
        const float w = lane_value(cv, j);
        if ((j & (DUP - 1)) == k) acc += w * sh_v[j * DV + row];
    }
    acc = group_sum<DUP>(acc);
    if (k == 0) a.o[c.bh * DV + row] = gam * z + acc;

    // Append the token as entry len (its slot is none of the entries read above); after the last
    // barrier, so no barrier waits for these stores.
    for (int i = t; i < KF; i += TPB) st4(a.ring.k + (c.rh + slot) * DK + 4 * i, ld4(sh_k + len * DK + 4 * i));
    for (int i = t; i < VF; i += TPB) st4(a.ring.v + (c.rh + slot) * DV + 4 * i, ld4(sh_v + len * DV + 4 * i));
    if (t == 0) {
        a.ring.beta[c.rh + slot] = bet;
        a.ring.alpha[c.rh + slot] = alt;
    }
}

template <int DV, int DK>
__host__ __device__ constexpr int gdn_fold_lds(int W)
{
    // k, v, Y, U: (W+1) rows each; e [DV][W+1]; G [(W+1)^2]; beta, alpha, decay ratios, gamma
    return (W + 1) * (2 * DK + 2 * DV) + DV * (W + 1) + (W + 1) * (W + 1) + 3 * (W + 1) + 4;
}

// Fold n entries (ring entries [0, nring) and optionally the token) into the lane's block of the
// checkpoint held in s. All threads call it.
template <int DV, int DK, int R>
__device__ __forceinline__ void gdn_fold_core(float4 (&s)[R], float *smem, const GdnRing &ring,
                                              const GTile &c, int head, int nring, bool tok,
                                              const float *kt, const float *vt, float bet, float alt)
{
    constexpr int TPB = TileShape<DV, DK>::TPB;
    using M = Map4<DV, DK>;
    static_assert(R == M::R, "fold block");
    constexpr int LPR = M::LPR;
    static_assert(TPB >= DK + DV, "one thread per Y / U column");
    const int W = c.W, t = c.t, W1 = W + 1;
    const int n = nring + (tok ? 1 : 0);
    const int rg = t / LPR, cg = t - rg * LPR, c0 = cg * 4;
    float *sh_k = smem;                 // [n][DK]
    float *sh_v = sh_k + W1 * DK;       // [n][DV]
    float *sh_Y = sh_v + W1 * DV;       // [n][DK]
    float *sh_U = sh_Y + W1 * DK;       // [n][DV]
    float *sh_e = sh_U + W1 * DV;       // [DV][W1]  (S0 y_t)
    float *sh_G = sh_e + DV * W1;       // [W1][W1]
    float *sh_be = sh_G + W1 * W1;      // [n]
    float *sh_al = sh_be + W1;          // [n]
    float *sh_dr = sh_al + W1;          // [n] prod_{i>t} alpha_i
    float *sh_g = sh_dr + W1;           // gamma

    stage_entries<DV, DK, TPB>(ring, c, head, nring, tok, kt, vt, bet, alt, sh_k, sh_v, sh_be, sh_al);
    __syncthreads();
    gram_dots<DK, TPB>(sh_k, nullptr, n, W1, sh_G, nullptr, t);
    for (int j = t; j < n; j += TPB) {
        float d = 1.f;
        for (int i = j + 1; i < n; ++i) d *= sh_al[i];
        sh_dr[j] = d;
    }
    if (t == TPB - 1) {
        float g = 1.f;
        for (int i = 0; i < n; ++i) g *= sh_al[i];
        sh_g[0] = g;
    }
    __syncthreads();
    if (t < DK) {                       // column t of Y
        for (int q = 0; q < n; ++q) {
            float y = sh_k[q * DK + t];
            for (int i = 0; i < q; ++i) y -= sh_G[i * W1 + q] * sh_Y[i * DK + t];
            sh_Y[q * DK + t] = sh_be[q] * y;
        }
    } else if (t < DK + DV) {           // column t - DK of U
        const int col = t - DK;
        for (int q = 0; q < n; ++q) {
            float u = sh_v[q * DV + col];
            float ratio = 1.f;          // gamma_q / gamma_i = prod_{i < i' <= q} alpha_i'
            for (int i = q - 1; i >= 0; --i) {
                ratio *= sh_al[i + 1];
                u -= ratio * sh_G[i * W1 + q] * sh_U[i * DV + col];
            }
            sh_U[q * DV + col] = sh_be[q] * u;
        }
    }
    __syncthreads();
    // e_t = S0 y_t for every t
    for (int q = 0; q < n; ++q) {
        const float4 y = ld4(sh_Y + q * DK + c0);
        float part[R];
#pragma unroll
        for (int r = 0; r < R; ++r) part[r] = s[r].x * y.x + s[r].y * y.y + s[r].z * y.z + s[r].w * y.w;
        int rsel;
        const float e = row_reduce_scatter<R, LPR>(part, cg, rsel);
        if (row_writer<R, LPR>(cg)) sh_e[(rg * R + rsel) * W1 + q] = e;
    }
    __syncthreads();
    const float g = sh_g[0];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        s[r].x *= g; s[r].y *= g; s[r].z *= g; s[r].w *= g;
    }
    for (int q = 0; q < n; ++q) {
        const float4 kq = ld4(sh_k + q * DK + c0);
        const float dq = sh_dr[q];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = rg * R + r;
            const float cf = dq * sh_U[q * DV + i] - g * sh_e[i * W1 + q];
            s[r].x += cf * kq.x; s[r].y += cf * kq.y; s[r].z += cf * kq.z; s[r].w += cf * kq.w;
        }
    }
}

template <int DV, int DK, int R>
__device__ __forceinline__ void gdn_store(const float4 (&s)[R], float *dst, int t)
{
    using M = Map4<DV, DK>;
    const int rg = t / M::LPR, c0 = (t - rg * M::LPR) * 4;
    const size_t off = (size_t)(rg * R) * DK + c0;
#pragma unroll
    for (int r = 0; r < R; ++r) st4_nt(dst + off + (size_t)r * DK, s[r]);
}

template <int DV, int DK, int R>
__device__ __forceinline__ void gdn_fold_decode(const GdnStepArgs &a, const GTile &c, int head,
                                                int len, float4 (&s)[R], float *smem)
{
    using M = Map4<DV, DK>;
    static_assert(R == M::R, "tile block");
    constexpr int LPR = M::LPR;
    const int t = c.t;
    const int rg = t / LPR, cg = t - rg * LPR, c0 = cg * 4;
    float *S0 = a.S0 + c.bh * (size_t)(DV * DK);
    const float *qt = a.q + c.bh * DK;
    const float4 qv = ld4(qt + c0);
    gdn_fold_core<DV, DK>(s, smem, a.ring, c, head, len, true, a.k + c.bh * DK, a.v + c.bh * DV,
                          a.beta[c.bh], a.alpha[c.bh]);
    gdn_store<DV, DK>(s, S0, t);
    float part[R];
#pragma unroll
    for (int r = 0; r < R; ++r) part[r] = s[r].x * qv.x + s[r].y * qv.y + s[r].z * qv.z + s[r].w * qv.w;
    int rsel;
    const float z = row_reduce_scatter<R, LPR>(part, cg, rsel);
    if (row_writer<R, LPR>(cg)) a.o[c.bh * DV + rg * R + rsel] = z;
}

// Decode variants, chosen on the host as for Mamba-2: 0 = every sequence at the ring position
// (a.uhead, a.ulen) with no fold (ring loads before the checkpoint read), 1 = no sequence folds
// (positions read from the device), 2 = any sequence may fold.
template <int DV, int DK, int MODE>
__global__ void __launch_bounds__((TileShape<DV, DK>::TPB))
k_gdn_decode(GdnStepArgs a)
{
    using M = Map4<DV, DK>;
    extern __shared__ float smem[];
    const GTile c = make_gtile(a.d);
    const int B = a.d.B, W = c.W;
    float4 s[M::R];
    int head, len;
    bool fold = false;
    if constexpr (MODE == 0) {
        head = a.uhead;
        len = a.ulen;
        gdn_replay<DV, DK, M::R, true>(a, c, head, len, s, smem);
    } else {
        // the checkpoint tile first: both paths read it with the same map
        const int rg = c.t / M::LPR, c0 = (c.t - rg * M::LPR) * 4;
        const size_t off = c.bh * (size_t)(DV * DK) + (size_t)(rg * M::R) * DK + c0;
#pragma unroll
        for (int r = 0; r < M::R; ++r) s[r] = ld4_nt(a.S0 + off + (size_t)r * DK);
        head = a.bk.in[c.b];
        len = a.bk.in[B + c.b];
        if constexpr (MODE == 2) fold = len + 1 >= W;
        if (fold) gdn_fold_decode<DV, DK>(a, c, head, len, s, smem);
        else gdn_replay<DV, DK, M::R, false>(a, c, head, len, s, smem);
    }
    if (c.h == 0 && c.t == 0) {
        a.bk.out[c.b] = fold ? (head + len + 1) % W : head;
        a.bk.out[B + c.b] = fold ? 0 : len + 1;
        a.bk.out[2 * B + c.b] = 0;
    }
}

template <int DV, int DK>
__global__ void __launch_bounds__((TileShape<DV, DK>::TPB)) k_gdn_fold(GdnFoldArgs a)
{
    constexpr int TPB = TileShape<DV, DK>::TPB;
    using M = Map4<DV, DK>;
    extern __shared__ float smem[];
    const GTile c = make_gtile(a.d);
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
            for (int i = c.t; i < DV * DK / 4; i += TPB) st4(dst + 4 * i, ld4(S0 + 4 * i));
        }
        return;
    }
    const int rg = c.t / M::LPR, c0 = (c.t - rg * M::LPR) * 4;
    float4 s[M::R];
    const size_t off = (size_t)(rg * M::R) * DK + c0;
#pragma unroll
    for (int r = 0; r < M::R; ++r) s[r] = ld4_nt(S0 + off + (size_t)r * DK);
    gdn_fold_core<DV, DK>(s, smem, a.ring, c, head, len, false, nullptr, nullptr, 0.f, 0.f);
    gdn_store<DV, DK>(s, a.out ? a.out + c.bh * (size_t)(DV * DK) : S0, c.t);
}

// conventional read-modify-write comparator
template <int DV, int DK>
__global__ void __launch_bounds__((TileShape<DV, DK>::TPB)) k_gdn_rmw(GdnRmwArgs a)
{
    using M = Map4<DV, DK>;
    constexpr int R = M::R, LPR = M::LPR;
    __shared__ float sh_sk[DV];
    const GTile c = make_gtile(a.d);
    const int t = c.t;
    const int rg = t / LPR, cg = t - rg * LPR, c0 = cg * 4;
    const size_t BH = (size_t)a.d.B * a.d.H;
    const size_t off = c.bh * (size_t)(DV * DK) + (size_t)(rg * R) * DK + c0;
    float4 S[R];
#pragma unroll
    for (int r = 0; r < R; ++r) S[r] = ld4_nt(a.state + off + (size_t)r * DK);
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
        if (a.snap) {
#pragma unroll
            for (int r = 0; r < R; ++r) st4_nt(a.snap + k * BH * (size_t)(DV * DK) + off + (size_t)r * DK, S[r]);
        }
    }
    if (!a.snap) {
#pragma unroll
        for (int r = 0; r < R; ++r) st4_nt(a.state + off + (size_t)r * DK, S[r]);
    }
}

template <int DV, int DK>
size_t gdn_decode_lds(int W)
{
    const size_t W1 = W + 1;
    const size_t replay = (size_t)W * (DK + DV) + DK + W * W1 + W;
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
    else hipLaunchKernelGGL((k_gdn_decode<DV, DK, 2>), grid, block, lds, s, a);
    return hipGetLastError();
}

template <int DV, int DK>
hipError_t go_fold(const GdnFoldArgs &a, hipStream_t s)
{
    const dim3 grid(a.d.B * a.d.H), block(TileShape<DV, DK>::TPB);
    const size_t lds = 4 * (size_t)gdn_fold_lds<DV, DK>(a.d.W);
    hipLaunchKernelGGL((k_gdn_fold<DV, DK>), grid, block, lds, s, a);
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
#define RSSM_C(v, k) if (DV == v && DK == k) return gdn_decode_lds<v, k>(W);
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

hipError_t gdn_rmw(const GdnRmwArgs &a, hipStream_t s)
{
#define RSSM_C(v, k) if (a.d.DV == v && a.d.DK == k) return go_rmw<v, k>(a, s);
    RSSM_GDN_SHAPES(RSSM_C)
#undef RSSM_C
    return hipErrorInvalidValue;
}

}  // namespace rssm
