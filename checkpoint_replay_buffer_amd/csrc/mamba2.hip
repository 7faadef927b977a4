// mamba2.hip -- Mamba-2 ReplaySSM decode kernels for gfx950.
//
// Per (sequence b, head h) the state is a P x N fp32 checkpoint S0 plus a ring of the last W
// tokens' inputs. Writing Lam_m = exp(A sum_{i<m} dt_i) for the decay over m buffered entries and
// w_j = dt_j exp(A sum_{i>j} dt_i) for entry j's weight, the state after the entries is
//     S = Lam_m S0 + sum_j w_j x_j B_j^T,
// so the output of the newest entry, y = S C + D x, is
//     y = Lam_m (S0 C) + sum_j w_j (B_j . C) x_j + D x                                   (replay)
// which reads S0 once and never writes it. Folding the entries (consolidation) writes that S
// back as the new S0. The normal step appends to the buffer and reads the checkpoint; only a
// full buffer is consolidated (ia.goatify.app article "NVIDIA y Princeton aceleran modelos
// híbridos...", paragraph "El checkpoint reduce escrituras de estado").
//
// One workgroup per (b, h) tile. The S0 stream is the only large traffic: its 16-byte loads are
// issued first, the small per-tile work (ring staging in LDS, decay weights, B_j . C dots with
// lane-group butterflies) runs while they are in flight, and the row sums of S0 C use a
// reduce-scatter butterfly over the lanes of a row.
#include "dev_common.h"
#include "internal.h"
#include "tile_order.h"

namespace rssm {
namespace {

__device__ __forceinline__ float dot_row(const float4 &v, const float *cc)
{
    return v.x * cc[0] + v.y * cc[1] + v.z * cc[2] + v.w * cc[3];
}
__device__ __forceinline__ float dot_row(const uint2 &v, const float *cc)
{
    return bf16_lo(v.x) * cc[0] + bf16_hi(v.x) * cc[1] + bf16_lo(v.y) * cc[2] + bf16_hi(v.y) * cc[3];
}
__device__ __forceinline__ float dot_row(const uint4 &v, const float *cc)
{
    return bf16_lo(v.x) * cc[0] + bf16_hi(v.x) * cc[1] + bf16_lo(v.y) * cc[2] + bf16_hi(v.y) * cc[3]
         + bf16_lo(v.z) * cc[4] + bf16_hi(v.z) * cc[5] + bf16_lo(v.w) * cc[6] + bf16_hi(v.w) * cc[7];
}

template <int EPL>
__device__ __forceinline__ void load_cols(float (&cc)[EPL], const float *src)
{
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
        const float4 v = ld4(src + e);
        cc[e] = v.x; cc[e + 1] = v.y; cc[e + 2] = v.z; cc[e + 3] = v.w;
    }
}

// Decode kernel variants, chosen on the host from what it knows about the ring fill:
//   kUniform  every sequence has the ring position (a.uhead, a.ulen) and none fills its ring:
//             no device read is needed before the ring loads, which go out before the checkpoint
//   kReplay   no sequence fills its ring; positions are read from the device, so the checkpoint
//             read is issued first and the ring loads after the positions arrive
//   kMayFold  any mix of replaying and folding sequences (positions read from the device)
//   kAllFold  every sequence has the position (a.uhead, a.ulen) and fills its ring: all fold
enum DecodeMode { kUniform = 0, kReplay = 1, kMayFold = 2, kAllFold = 3 };

// Threads per workgroup of the Mamba-2 kernels for a P x N tile. WIDE gives each thread about
// 4 float4 of the fp32 checkpoint (512 threads at 64 x 128), NARROW about 8 (256), SINGLE about
// 2 (1024, for the conventional kernel over a single token). The fp32 decode (every variant), the
// fold and the bf16 launches in which every tile folds take WIDE; verify and the bf16 launches in
// which most tiles replay (replay-only, or a mix) take NARROW; the conventional kernel chooses by
// token count (go_rmw). Each choice measured fastest in same-box comparisons.
template <int P, int N>
struct M2Threads {
    static constexpr int NF4 = P * N / 4;
    static constexpr int WIDE = NF4 / 4 < 64 ? 64 : (NF4 / 4 > 512 ? 512 : NF4 / 4);
    static constexpr int NARROW = TileShape<P, N>::TPB;
    static constexpr int SINGLE = NF4 / 2 < 64 ? 64 : (NF4 / 2 > 1024 ? 1024 : NF4 / 2);
    static constexpr int decode(bool bf16, int mode) { return bf16 && mode != kAllFold ? NARROW : WIDE; }
};

// bf16 read-copy layout: 16-byte loads (8 values) when the tile has enough of them for every
// lane, else 8-byte loads.
template <int P, int N, int TPB>
struct Bf16Epl {
    static constexpr int value = (P * N / 8 >= TPB) ? 8 : 4;
};

template <int EPL> struct RawBf16;
template <> struct RawBf16<8> { using type = uint4; };
template <> struct RawBf16<4> { using type = uint2; };

// Per-tile context of one (b, h) workgroup.
struct Tile {
    int b, h, g, t, W;
    size_t bh, bg;            // tile index and (b, group) index
    size_t rh, rg_;           // ring row bases: (b,h) and (b,g) times W
    bool own_group;           // first head of its group: writes the group's B / C ring rows
    float Ah, Dh;
};

// The launches that only read the checkpoint take runs of tiles per XCD, the launches that fold
// (read and write it) one contiguous range per XCD: each measured fastest in same-box A/B runs.
__device__ __forceinline__ Tile make_tile(const M2Dims &d, const float *A, const float *D,
                                          TileOrder order)
{
    Tile c;
    const int tile = tile_of(blockIdx.x, d.B * d.H, order, run_tiles(d.P * d.N));
    c.b = tile / d.H;
    c.h = tile - c.b * d.H;
    const int hpg = d.H / d.G;
    c.g = c.h / hpg;
    c.t = threadIdx.x;
    c.W = d.W;
    c.bh = (size_t)tile;
    c.bg = (size_t)c.b * d.G + c.g;
    c.rh = c.bh * d.W;
    c.rg_ = c.bg * d.W;
    c.own_group = (c.h - c.g * hpg) == 0;
    c.Ah = A ? A[c.h] : 0.f;
    c.Dh = D ? D[c.h] : 0.f;
    return c;
}

// LDS floats used by the fold core for a ring of length W (x and B rows of up to W+1 entries).
__host__ __device__ constexpr int fold_lds_floats(int W, int P, int N)
{
    return (W + 1) * (P + N);
}

// Decay weights of n <= 64 entries whose step sizes sit one per lane of the wave (lane l < n holds
// dt_l, oldest first): returns w_l = dt_l exp(A sum_{i>l} dt_i) on lane l (0 on lanes >= n), and
// the decay of the whole window exp(A sum_i dt_i) in `lam` on every lane. The suffix sums are a
// log-step scan with wave shuffles; every lane of the wave must take part.
__device__ __forceinline__ float wave_weights(float dtl, int n, float A, float &lam)
{
    const int lane = threadIdx.x & 63;
    const float v = lane < n ? dtl : 0.f;
    float e = __shfl_down(v, 1);        // sum over i > lane, built up by the scan below
    if (lane == 63) e = 0.f;
    for (int off = 1; off < n; off <<= 1) {
        const float o = __shfl_down(e, off);
        if (lane + off < 64) e += o;
    }
    lam = expf(A * __shfl(v + e, 0));
    return lane < n ? dtl * expf(A * e) : 0.f;
}

__device__ __forceinline__ float lane_value(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Fold n = nring (+1 with a current token) entries into the lane's R x 4 block of the
// checkpoint held in acc:  acc <- Lam_n acc + sum_j w_j x_j B_j^T.  Ring entries start at ring
// slot `head`; the current token (xt, Bt, dtt), if xt != nullptr, is the newest entry.
// n <= W + 1 <= 33 entries, so each wave holds every step size in its lanes. All threads of the
// workgroup must call it; it synchronises once.
template <int P, int N, int TPB, int R>
__device__ __forceinline__ void m2_fold_core(float4 (&acc)[R], float *smem, const M2Ring &ring,
                                             const Tile &c, int head, int nring, const float *xt,
                                             const float *Bt, float dtt)
{
    using M = RowMap<P, N, TPB, 4>;
    static_assert(R == M::R, "fold block");
    const int W = c.W, t = c.t, lane = t & 63;
    const int rg = t / M::LPR, c0 = (t - rg * M::LPR) * 4;
    const int n = nring + (xt ? 1 : 0);
    float *sh_x = smem;                     // [n][P]
    float *sh_B = sh_x + (W + 1) * P;       // [n][N]

    const float dtl = lane < nring ? ring.dt[c.rh + (head + lane) % W] : dtt;
    constexpr int PF = P / 4, NF = N / 4;
    for (int i = t; i < n * PF; i += TPB) {
        const int j = i / PF, q = (i - j * PF) * 4;
        st4(sh_x + j * P + q, j < nring ? ld4(ring.x + (c.rh + (head + j) % W) * P + q) : ld4(xt + q));
    }
    for (int i = t; i < n * NF; i += TPB) {
        const int j = i / NF, q = (i - j * NF) * 4;
        st4(sh_B + j * N + q, j < nring ? ld4(ring.B + (c.rg_ + (head + j) % W) * N + q) : ld4(Bt + q));
    }
    float lam;
    const float w = wave_weights(dtl, n, c.Ah, lam);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        acc[r].x *= lam; acc[r].y *= lam; acc[r].z *= lam; acc[r].w *= lam;
    }
    const int p0 = rg * R;
    for (int j = 0; j < n; ++j) {
        const float wj = lane_value(w, j);
        const float4 bv = ld4(sh_B + j * N + c0);
        const float *xj = sh_x + j * P + p0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float ur = wj * xj[r];
            acc[r].x += ur * bv.x; acc[r].y += ur * bv.y;
            acc[r].z += ur * bv.z; acc[r].w += ur * bv.w;
        }
    }
}

// Store the lane's block of a folded checkpoint (and its bf16 read copy).
template <int P, int N, int TPB, int R>
__device__ __forceinline__ void store_tile(const float4 (&acc)[R], float *dst, uint16_t *dstb, int t)
{
    using M = RowMap<P, N, TPB, 4>;
    static_assert(R == M::R, "fold block");
    const int rg = t / M::LPR, c0 = (t - rg * M::LPR) * 4;
    const size_t off = (size_t)(rg * M::R) * N + c0;
#pragma unroll
    for (int r = 0; r < M::R; ++r) st4_nt(dst + off + (size_t)r * N, acc[r]);
    if (dstb) {
#pragma unroll
        for (int r = 0; r < M::R; ++r) {
            uint2 w;
            w.x = pack_bf16x2(acc[r].x, acc[r].y);
            w.y = pack_bf16x2(acc[r].z, acc[r].w);
            *reinterpret_cast<uint2 *>(dstb + off + (size_t)r * N) = w;
        }
    }
}

// The lane's R rows x EPL columns of the checkpoint read: fp32 S0 or its bf16 copy.
template <int P, int N, int TPB, bool BF16>
struct ReadTile {
    static constexpr int EPL = BF16 ? Bf16Epl<P, N, TPB>::value : 4;
    using M = RowMap<P, N, TPB, EPL>;
    using RawT = typename std::conditional<BF16, typename RawBf16<EPL>::type, float4>::type;
    RawT v[M::R];

    __device__ __forceinline__ void load(const M2StepArgs &a, const Tile &c)
    {
        const int rg = c.t / M::LPR, c0 = (c.t - rg * M::LPR) * EPL;
        const size_t off = c.bh * (size_t)(P * N) + (size_t)(rg * M::R) * N + c0;
#pragma unroll
        for (int r = 0; r < M::R; ++r) {
            if constexpr (!BF16) v[r] = ld4_nt(a.S0 + off + (size_t)r * N);
            else if constexpr (EPL == 8) v[r] = ldu4_nt(a.S0b + off + (size_t)r * N);
            else v[r] = ldu2_nt(a.S0b + off + (size_t)r * N);
        }
    }
};

template <int P, int N, int TPB, int R>
__device__ __forceinline__ void load_fp32_tile(float4 (&acc)[R], const float *S0, const Tile &c)
{
    using M = RowMap<P, N, TPB, 4>;
    const int rg = c.t / M::LPR, c0 = (c.t - rg * M::LPR) * 4;
    const size_t off = c.bh * (size_t)(P * N) + (size_t)(rg * M::R) * N + c0;
#pragma unroll
    for (int r = 0; r < M::R; ++r) acc[r] = ld4_nt(S0 + off + (size_t)r * N);
}

// ------------------------------------------------------------------------------------------
// decode: replay path (the token does not fill the ring). One barrier per tile.
//
// Vector-load completions are waited for in issue order, so whatever is issued first can be
// consumed while later loads are still in flight. With EARLY = false the small ring-side loads go
// out first and the checkpoint read after them: the ring work (LDS staging, decay weights,
// B_j . C) then overlaps the checkpoint stream. EARLY = true means the caller already issued the
// checkpoint read (needed when the ring position must first be read from device memory).
// ------------------------------------------------------------------------------------------
template <int P, int N, int TPB, bool BF16, bool EARLY>
__device__ __forceinline__ void m2_replay_decode(const M2StepArgs &a, const Tile &c, int head,
                                                 int len, ReadTile<P, N, TPB, BF16> &tile, float *smem)
{
    using RT = ReadTile<P, N, TPB, BF16>;
    constexpr int EPL = RT::EPL;
    using M = typename RT::M;
    constexpr int R = M::R, LPR = M::LPR, RG = M::RG;
    constexpr int DUP = LPR / R;                          // lanes holding the same finished row
    constexpr int PF = P / 4;
    constexpr int XQ = (kMaxWindow * PF + TPB - 1) / TPB; // x-row float4 per thread, at most
    const int W = c.W, t = c.t, m = len + 1;
    const int rg = t / LPR, cg = t - rg * LPR, c0 = cg * EPL;
    float *sh_x = smem;            // [m][P]   x of the entries
    float *sh_cf = sh_x + W * P;   // [m]      w_j (B_j . C)
    const float *xt = a.x + c.bh * P;
    const float *Bt = a.Bm + c.bg * N;
    const float dtt = a.dt[c.bh];
    const int slot = (head + len) % W;

    // 1. ring-side loads: C columns, step sizes (one per lane), B rows of this row group's first
    //    two entries, x rows of every entry
    float cc[EPL];
    load_cols<EPL>(cc, a.C + c.bg * N + c0);
    const int lane = t & 63;
    const float dtl = lane < len ? a.ring.dt[c.rh + (head + lane) % W] : dtt;
    float4 bq[2][EPL / 4];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int j = rg + RG * q;
        const float *Bj = j < len ? a.ring.B + (c.rg_ + (head + j) % W) * N : Bt;
#pragma unroll
        for (int e = 0; e < EPL / 4; ++e)
            bq[q][e] = j < m ? ld4(Bj + c0 + 4 * e) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float4 xs[XQ];
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
        const int i = t + q * TPB, j = i / PF, o = (i - j * PF) * 4;
        xs[q] = i < m * PF ? (j < len ? ld4(a.ring.x + (c.rh + (head + j) % W) * P + o) : ld4(xt + o))
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // 2. the checkpoint read
    if constexpr (!EARLY) tile.load(a, c);

    // 3. ring work while the checkpoint streams in
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
        const int i = t + q * TPB, j = i / PF, o = (i - j * PF) * 4;
        if (i < m * PF) st4(sh_x + j * P + o, xs[q]);
    }
    float lam;
    const float w = wave_weights(dtl, m, c.Ah, lam);     // w_j on lane j of every wave
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int j = rg + RG * q;
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < EPL / 4; ++e)
            part += bq[q][e].x * cc[4 * e] + bq[q][e].y * cc[4 * e + 1] + bq[q][e].z * cc[4 * e + 2]
                  + bq[q][e].w * cc[4 * e + 3];
        const float sj = group_sum<LPR>(part);
        const float wj = __shfl(w, j);                   // all lanes active: j < 2 RG <= 64
        if (cg == 0 && j < m) sh_cf[j] = wj * sj;
    }
    for (int q = 2; q * RG < m; ++q) {                   // rings longer than 2 RG (trip count is
        const int j = rg + RG * q;                       // uniform, so every lane shuffles)
        const float *Bj = j < len ? a.ring.B + (c.rg_ + (head + j) % W) * N : Bt;
        float part = 0.f;
        if (j < m) {
#pragma unroll
            for (int e = 0; e < EPL; e += 4) {
                const float4 v = ld4(Bj + c0 + e);
                part += v.x * cc[e] + v.y * cc[e + 1] + v.z * cc[e + 2] + v.w * cc[e + 3];
            }
        }
        const float sj = group_sum<LPR>(part);
        const float wj = __shfl(w, j & 63);
        if (cg == 0 && j < m) sh_cf[j] = wj * sj;
    }
    __syncthreads();

    // 4. z = S0 C; y = Lam z + sum_j w_j (B_j . C) x_j + D x, the sum split over the DUP lanes
    //    that hold the same row
    float part[R];
#pragma unroll
    for (int r = 0; r < R; ++r) part[r] = dot_row(tile.v[r], cc);
    int rsel;
    const float z = row_reduce_scatter<R, LPR>(part, cg, rsel);
    const int p = rg * R + rsel, k = cg & (DUP - 1);
    float corr = 0.f;
    for (int j = k; j < m; j += DUP) corr += sh_cf[j] * sh_x[j * P + p];
    corr = group_sum<DUP>(corr);
    if (k == 0) a.y[c.bh * P + p] = lam * z + corr + c.Dh * sh_x[len * P + p];

    // 5. Append the token as entry len. Its slot is none of the entries read above. The stores
    //    come after the barrier: a workgroup barrier waits for the workgroup's outstanding
    //    stores, so stores issued before it would put their latency on every tile. They are
    //    non-temporal, which measured faster than write-back stores here and in verify.
    for (int i = t; i < PF; i += TPB) st4_nt(a.ring.x + (c.rh + slot) * P + 4 * i, ld4(sh_x + len * P + 4 * i));
    if (c.own_group) {
        // The B and C rows (in cache from the loads above) go out as LPR consecutive float4 per
        // instruction, whole 128-byte lines: a non-temporal store of part of a line costs a
        // write of the whole line.
        if (rg == len % RG) {
#pragma unroll
            for (int e = 0; e < EPL / 4; ++e) {
                const int q = 4 * (cg + e * LPR);
                st4_nt(a.ring.B + (c.rg_ + slot) * N + q, ld4(Bt + q));
            }
        }
        if (a.ring.C && rg == 0) {
#pragma unroll
            for (int e = 0; e < EPL / 4; ++e) {
                const int q = 4 * (cg + e * LPR);
                const float4 v = EPL == 4 ? make_float4(cc[0], cc[1], cc[2], cc[3]) : ld4(a.C + c.bg * N + q);
                st4_nt(a.ring.C + (c.rg_ + slot) * N + q, v);
            }
        }
    }
    if (t == 0) a.ring.dt[c.rh + slot] = dtt;
}

// ------------------------------------------------------------------------------------------
// decode: fold path (the token fills the ring; with len == W after a full commit the ring is
// already full and the token is the (W+1)-th entry)
// ------------------------------------------------------------------------------------------
template <int P, int N, int TPB, bool BF16, int R>
__device__ __forceinline__ void m2_fold_decode(const M2StepArgs &a, const Tile &c, int head, int len,
                                               float4 (&acc)[R], float *smem)
{
    using M = RowMap<P, N, TPB, 4>;
    static_assert(R == M::R, "fold block");
    constexpr int LPR = M::LPR;
    const int t = c.t;
    const int rg = t / LPR, cg = t - rg * LPR, c0 = cg * 4;
    const float *xt = a.x + c.bh * P;
    float cc[4];
    load_cols<4>(cc, a.C + c.bg * N + c0);
    m2_fold_core<P, N, TPB>(acc, smem, a.ring, c, head, len, xt, a.Bm + c.bg * N, a.dt[c.bh]);
    store_tile<P, N, TPB>(acc, a.S0 + c.bh * (size_t)(P * N), BF16 ? a.S0b + c.bh * (size_t)(P * N) : nullptr, t);
    float part[R];
#pragma unroll
    for (int r = 0; r < R; ++r) part[r] = dot_row(acc[r], cc);
    int rsel;
    const float z = row_reduce_scatter<R, LPR>(part, cg, rsel);
    if (row_writer<R, LPR>(cg)) {
        const int p = rg * R + rsel;
        a.y[c.bh * P + p] = z + c.Dh * xt[p];
    }
}

template <int P, int N, bool BF16, int MODE>
__global__ void __launch_bounds__((M2Threads<P, N>::decode(BF16, MODE))) k_m2_decode(M2StepArgs a)
{
    constexpr int TPB = M2Threads<P, N>::decode(BF16, MODE);
    extern __shared__ float smem[];
    // the launches that fold take contiguous tile ranges per XCD (mixed launches too), the
    // replay-only launches runs
    const Tile c = make_tile(a.d, a.A, a.D, MODE >= kMayFold ? kContiguous : kRuns);
    const int B = a.d.B, W = c.W;
    bool fold = false;
    int head, len;
    if constexpr (MODE == kUniform) {
        ReadTile<P, N, TPB, BF16> tile;
        head = a.uhead;
        len = a.ulen;
        m2_replay_decode<P, N, TPB, BF16, false>(a, c, head, len, tile, smem);
    } else if constexpr (MODE == kReplay) {
        ReadTile<P, N, TPB, BF16> tile;
        tile.load(a, c);
        head = a.bk.in[c.b];
        len = a.bk.in[B + c.b];
        m2_replay_decode<P, N, TPB, BF16, true>(a, c, head, len, tile, smem);
    } else if constexpr (MODE == kAllFold) {
        head = a.uhead;
        len = a.ulen;
        fold = true;
        float4 acc[RowMap<P, N, TPB, 4>::R];
        load_fp32_tile<P, N, TPB>(acc, a.S0, c);
        m2_fold_decode<P, N, TPB, BF16>(a, c, head, len, acc, smem);
    } else if constexpr (!BF16) {
        // a mix: the checkpoint read goes out before the position read, so the latter hides under
        // it; the fold and the replay both start from the fp32 tile
        ReadTile<P, N, TPB, false> tile;
        tile.load(a, c);
        head = a.bk.in[c.b];
        len = a.bk.in[B + c.b];
        fold = len + 1 >= W;
        if (fold) m2_fold_decode<P, N, TPB, false>(a, c, head, len, tile.v, smem);
        else m2_replay_decode<P, N, TPB, false, true>(a, c, head, len, tile, smem);
    } else {
        // a mix read from the bf16 copy: the position first (a folding tile reads the fp32 tile, a
        // replaying one the copy), then the tile, then the ring (the kReplay order)
        head = a.bk.in[c.b];
        len = a.bk.in[B + c.b];
        fold = len + 1 >= W;
        if (fold) {
            float4 acc[RowMap<P, N, TPB, 4>::R];
            load_fp32_tile<P, N, TPB>(acc, a.S0, c);
            m2_fold_decode<P, N, TPB, true>(a, c, head, len, acc, smem);
        } else {
            ReadTile<P, N, TPB, true> tile;
            tile.load(a, c);
            m2_replay_decode<P, N, TPB, true, true>(a, c, head, len, tile, smem);
        }
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
template <int P, int N, bool BF16>
__global__ void __launch_bounds__((M2Threads<P, N>::WIDE)) k_m2_fold(M2FoldArgs a)
{
    constexpr int TPB = M2Threads<P, N>::WIDE;
    using M = RowMap<P, N, TPB, 4>;
    extern __shared__ float smem[];
    const Tile c = make_tile(a.d, a.A, nullptr, kContiguous);
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
    float *S0 = a.S0 + c.bh * (size_t)(P * N);
    if (!fold) {
        if (a.out) {
            float *dst = a.out + c.bh * (size_t)(P * N);
            for (int i = c.t; i < P * N / 4; i += TPB) st4(dst + 4 * i, ld4(S0 + 4 * i));
        }
        return;
    }
    const int rg = c.t / M::LPR, c0 = (c.t - rg * M::LPR) * 4;
    float4 acc[M::R];
    const size_t off = (size_t)(rg * M::R) * N + c0;
#pragma unroll
    for (int r = 0; r < M::R; ++r) acc[r] = ld4_nt(S0 + off + (size_t)r * N);
    m2_fold_core<P, N, TPB>(acc, smem, a.ring, c, head, len, nullptr, nullptr, 0.f);
    if (a.out) store_tile<P, N, TPB>(acc, a.out + c.bh * (size_t)(P * N), nullptr, c.t);
    else store_tile<P, N, TPB>(acc, S0, BF16 ? a.S0b + c.bh * (size_t)(P * N) : nullptr, c.t);
}

// ------------------------------------------------------------------------------------------
// speculative verify: K drafts, outputs only, S0 streamed once
//
// The drafts become entries len_e .. len_e + K - 1 after the ring's len_e committed entries.
// Draft k sees the m_k = len_e + k + 1 entries up to and including itself (causal), so
//     y_k = Lam_{m_k} (S0 C_k) + sum_{j < m_k} w_{j,m_k} (B_j . C_k) x_j + D x_{len_e+k}.
// As in the replay decode, the ring and draft rows are loaded first and staged in LDS, and the
// checkpoint read is issued after them, so the decay weights, the B_j . C_k dots and the
// per-draft coefficients are computed while the checkpoint streams in. Two barriers per tile.
// ------------------------------------------------------------------------------------------

// LDS floats of the verify outputs: x [W][P], B [W][N], C [W][N] (K <= W drafts), the weights
// and coefficients [W][W] each, the window decays [W].
__host__ __device__ constexpr int verify_lds_floats(int W, int P, int N)
{
    return W * (P + 2 * N) + 2 * W * W + W;
}

// LOADED = true: the tile already holds the checkpoint (folded just before); otherwise it is read
// here after the ring and draft loads went out.
template <int P, int N, int TPB, bool BF16, bool LOADED>
__device__ __forceinline__ void m2_verify_outputs(const M2StepArgs &a, const Tile &c, int head_e,
                                                  int len_e, ReadTile<P, N, TPB, BF16> &tile, float *smem)
{
    using RT = ReadTile<P, N, TPB, BF16>;
    constexpr int EPL = RT::EPL;
    using M = typename RT::M;
    constexpr int R = M::R, LPR = M::LPR;
    constexpr int DUP = LPR / R;
    constexpr int PF = P / 4, NF = N / 4;
    constexpr int XQ = (kMaxWindow * PF + TPB - 1) / TPB;
    constexpr int BQ = (kMaxWindow * NF + TPB - 1) / TPB;
    const int W = c.W, t = c.t, K = a.ntok, ne = len_e + K;
    const int rg = t / LPR, cg = t - rg * LPR, c0 = cg * EPL;
    const size_t BH = (size_t)a.d.B * a.d.H, BG = (size_t)a.d.B * a.d.G;
    float *sh_x = smem;                // [ne][P]
    float *sh_B = sh_x + W * P;        // [ne][N]
    float *sh_C = sh_B + W * N;        // [K][N]
    float *sh_w = sh_C + W * N;        // [K][W]  w_{j, m_k}
    float *sh_cf = sh_w + W * W;       // [K][W]  w_{j, m_k} (B_j . C_k)
    float *sh_lam = sh_cf + W * W;     // [K]     Lam_{m_k}

    // 1. ring and draft rows, step sizes (entry j on lane j of every wave), then the checkpoint
    const int lane = t & 63;
    const float dtl = lane < len_e ? a.ring.dt[c.rh + (head_e + lane) % W]
                                   : (lane < ne ? a.dt[(lane - len_e) * BH + c.bh] : 0.f);
    float4 xs[XQ], bs[BQ], cs[BQ];
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
        const int i = t + q * TPB, j = i / PF, o = (i - j * PF) * 4;
        xs[q] = i >= ne * PF ? make_float4(0.f, 0.f, 0.f, 0.f)
              : (j < len_e ? ld4(a.ring.x + (c.rh + (head_e + j) % W) * P + o)
                           : ld4(a.x + ((j - len_e) * BH + c.bh) * P + o));
    }
#pragma unroll
    for (int q = 0; q < BQ; ++q) {
        const int i = t + q * TPB, j = i / NF, o = (i - j * NF) * 4;
        bs[q] = i >= ne * NF ? make_float4(0.f, 0.f, 0.f, 0.f)
              : (j < len_e ? ld4(a.ring.B + (c.rg_ + (head_e + j) % W) * N + o)
                           : ld4(a.Bm + ((j - len_e) * BG + c.bg) * N + o));
        cs[q] = i < K * NF ? ld4(a.C + (j * BG + c.bg) * N + o) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if constexpr (!LOADED) tile.load(a, c);

    // 2. staging and decay weights while the checkpoint is in flight
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
        const int i = t + q * TPB;
        if (i < ne * PF) st4(sh_x + 4 * i, xs[q]);
    }
#pragma unroll
    for (int q = 0; q < BQ; ++q) {
        const int i = t + q * TPB;
        if (i < ne * NF) st4(sh_B + 4 * i, bs[q]);
        if (i < K * NF) st4(sh_C + 4 * i, cs[q]);
    }
    constexpr int NW = TPB / 64;
    for (int k = t / 64; k < K; k += NW) {               // one wave per draft
        const int mk = len_e + k + 1;
        float lam;
        const float w = wave_weights(dtl, mk, c.Ah, lam);
        if (lane < mk) sh_w[k * W + lane] = w;
        if (lane == 0) sh_lam[k] = lam;
    }
    __syncthreads();

    // 3. coefficients w_{j, m_k} (B_j . C_k), j < m_k: one dot per lane group
    {
        constexpr int LPD = NF < 16 ? NF : 16;           // lanes per dot
        constexpr int EPD = N / LPD;                     // floats per lane, a multiple of 4
        const int grp = t / LPD, gl = t - grp * LPD;
        for (int d = grp; d < K * ne; d += TPB / LPD) {
            const int k = d / ne, j = d - k * ne;
            if (j <= len_e + k) {                        // uniform over the lane group
                const float *bj = sh_B + j * N + gl * EPD, *ck = sh_C + k * N + gl * EPD;
                float s = 0.f;
#pragma unroll
                for (int e = 0; e < EPD; e += 4) {
                    const float4 u = ld4(bj + e), v = ld4(ck + e);
                    s += u.x * v.x + u.y * v.y + u.z * v.z + u.w * v.w;
                }
                s = group_sum<LPD>(s);
                if (gl == 0) sh_cf[k * W + j] = sh_w[k * W + j] * s;
            }
        }
    }
    __syncthreads();

    // 4. per draft: z = S0 C_k (row reduce-scatter), the buffer sum split over the DUP lanes that
    //    hold the same row
    const int kd = cg & (DUP - 1);
    for (int k = 0; k < K; ++k) {
        float cc[EPL];
        load_cols<EPL>(cc, sh_C + k * N + c0);
        float part[R];
#pragma unroll
        for (int r = 0; r < R; ++r) part[r] = dot_row(tile.v[r], cc);
        int rsel;
        const float z = row_reduce_scatter<R, LPR>(part, cg, rsel);
        const int p = rg * R + rsel, mk = len_e + k + 1;
        float corr = 0.f;
        for (int j = kd; j < mk; j += DUP) corr += sh_cf[k * W + j] * sh_x[j * P + p];
        corr = group_sum<DUP>(corr);
        if (kd == 0) a.y[(k * BH + c.bh) * P + p] = sh_lam[k] * z + corr + c.Dh * sh_x[(len_e + k) * P + p];
    }

    // 5. append the drafts as entries len_e .. len_e + K - 1 (every ring read is done)
    for (int i = t; i < K * PF; i += TPB) {
        const int k = i / PF, q = (i - k * PF) * 4;
        st4_nt(a.ring.x + (c.rh + (head_e + len_e + k) % W) * P + q, ld4(sh_x + (len_e + k) * P + q));
    }
    if (c.own_group) {
        for (int i = t; i < K * NF; i += TPB) {
            const int k = i / NF, q = (i - k * NF) * 4;
            const size_t row = (c.rg_ + (head_e + len_e + k) % W) * N + q;
            st4_nt(a.ring.B + row, ld4(sh_B + (len_e + k) * N + q));
            if (a.ring.C) st4_nt(a.ring.C + row, ld4(sh_C + k * N + q));
        }
    }
    for (int k = t; k < K; k += TPB) a.ring.dt[c.rh + (head_e + len_e + k) % W] = a.dt[k * BH + c.bh];
}

template <int P, int N, bool BF16>
__global__ void __launch_bounds__((M2Threads<P, N>::NARROW)) k_m2_verify(M2StepArgs a)
{
    constexpr int TPB = M2Threads<P, N>::NARROW;
    extern __shared__ float smem[];
    const Tile c = make_tile(a.d, a.A, a.D, kRuns);
    const int B = a.d.B, W = c.W, K = a.ntok;
    const int head = a.bk.in[c.b];
    const int len = a.bk.in[B + c.b];
    const bool prefold = len + K > W;
    const int head_e = prefold ? (head + len) % W : head;
    const int len_e = prefold ? 0 : len;
    if (prefold) {
        // fold the committed entries first; the drafts then read the folded fp32 tile
        ReadTile<P, N, TPB, false> tile;
        load_fp32_tile<P, N, TPB>(tile.v, a.S0, c);
        m2_fold_core<P, N, TPB>(tile.v, smem, a.ring, c, head, len, nullptr, nullptr, 0.f);
        const size_t off0 = c.bh * (size_t)(P * N);
        store_tile<P, N, TPB>(tile.v, a.S0 + off0, BF16 ? a.S0b + off0 : nullptr, c.t);
        __syncthreads();
        m2_verify_outputs<P, N, TPB, false, true>(a, c, head_e, len_e, tile, smem);
    } else {
        ReadTile<P, N, TPB, BF16> tile;
        m2_verify_outputs<P, N, TPB, BF16, false>(a, c, head_e, len_e, tile, smem);
    }
    if (c.h == 0 && c.t == 0) {
        a.bk.out[c.b] = head_e;
        a.bk.out[B + c.b] = len_e;
        a.bk.out[2 * B + c.b] = K;
    }
}

// ------------------------------------------------------------------------------------------
// conventional read-modify-write comparator
// ------------------------------------------------------------------------------------------
template <int P, int N, int TPB>
__global__ void __launch_bounds__(TPB) k_m2_rmw(M2RmwArgs a)
{
    using M = RowMap<P, N, TPB, 4>;
    constexpr int R = M::R, LPR = M::LPR;
    const Tile c = make_tile(a.d, a.A, a.D, kRuns);
    const int t = c.t;
    const int rg = t / LPR, cg = t - rg * LPR, c0 = cg * 4;
    const size_t BH = (size_t)a.d.B * a.d.H, BG = (size_t)a.d.B * a.d.G, PN = (size_t)P * N;
    const size_t off = (size_t)(rg * R) * N + c0;       // lane block within a tile
    // source tile and the first snapshot tile (snapshot k is k * BH tiles further)
    // source tile (updated in place when there are no snapshots), and the first snapshot tile
    float *src;
    float *snap0;
    if (a.slot_of) {
        const int sl = a.slot_of[c.b];
        src = a.state + ((size_t)sl * BH + c.bh) * PN;
        snap0 = a.state + ((size_t)(sl < a.ntok ? a.ntok : 0) * BH + c.bh) * PN;
    } else {
        src = a.seq ? a.seq[c.b] + (size_t)c.h * PN : a.state + c.bh * PN;
        snap0 = a.snap ? a.snap + c.bh * PN : nullptr;
    }
    float4 S[R];
#pragma unroll
    for (int r = 0; r < R; ++r) S[r] = ld4_nt(src + off + (size_t)r * N);
    for (int k = 0; k < a.ntok; ++k) {
        const float dtv = a.dt[k * BH + c.bh];
        const float dec = expf(dtv * c.Ah);
        const float *xk = a.x + (k * BH + c.bh) * P;
        const float4 bv = ld4(a.Bm + (k * BG + c.bg) * N + c0);
        float cc[4];
        load_cols<4>(cc, a.C + (k * BG + c.bg) * N + c0);
        float part[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float coef = dtv * xk[rg * R + r];
            S[r].x = dec * S[r].x + coef * bv.x;
            S[r].y = dec * S[r].y + coef * bv.y;
            S[r].z = dec * S[r].z + coef * bv.z;
            S[r].w = dec * S[r].w + coef * bv.w;
            part[r] = dot_row(S[r], cc);
        }
        int rsel;
        const float z = row_reduce_scatter<R, LPR, false>(part, cg, rsel);
        if (row_writer<R, LPR>(cg)) {
            const int p = rg * R + rsel;
            a.y[(k * BH + c.bh) * P + p] = z + c.Dh * xk[p];
        }
        if (snap0) {
#pragma unroll
            for (int r = 0; r < R; ++r) st4_nt(snap0 + k * BH * PN + off + (size_t)r * N, S[r]);
        }
    }
    if (!snap0) {
#pragma unroll
        for (int r = 0; r < R; ++r) st4_nt(src + off + (size_t)r * N, S[r]);
    }
}

// ------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------
template <int P, int N>
size_t decode_lds(int W)
{
    const size_t replay = (size_t)W * P + W;
    const size_t fold = fold_lds_floats(W, P, N);
    return 4 * (replay > fold ? replay : fold);
}

template <int P, int N>
size_t verify_lds(int W)
{
    const size_t out = verify_lds_floats(W, P, N);
    const size_t fold = fold_lds_floats(W, P, N);
    return 4 * (out > fold ? out : fold);
}

template <int P, int N>
hipError_t go_decode(const M2StepArgs &a, bool bf16, int mode, hipStream_t s)
{
    const dim3 grid(a.d.B * a.d.H), block(M2Threads<P, N>::decode(bf16, mode));
    const size_t lds = decode_lds<P, N>(a.d.W);
#define RSSM_GO(b, md) hipLaunchKernelGGL((k_m2_decode<P, N, b, md>), grid, block, lds, s, a)
    if (bf16) {
        if (mode == kUniform) RSSM_GO(true, kUniform);
        else if (mode == kReplay) RSSM_GO(true, kReplay);
        else if (mode == kAllFold) RSSM_GO(true, kAllFold);
        else RSSM_GO(true, kMayFold);
    } else {
        if (mode == kUniform) RSSM_GO(false, kUniform);
        else if (mode == kReplay) RSSM_GO(false, kReplay);
        else if (mode == kAllFold) RSSM_GO(false, kAllFold);
        else RSSM_GO(false, kMayFold);
    }
#undef RSSM_GO
    return hipGetLastError();
}

template <int P, int N>
hipError_t go_verify(const M2StepArgs &a, bool bf16, hipStream_t s)
{
    const dim3 grid(a.d.B * a.d.H), block(M2Threads<P, N>::NARROW);
    const size_t lds = verify_lds<P, N>(a.d.W);
    if (bf16) hipLaunchKernelGGL((k_m2_verify<P, N, true>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((k_m2_verify<P, N, false>), grid, block, lds, s, a);
    return hipGetLastError();
}

template <int P, int N>
hipError_t go_fold(const M2FoldArgs &a, bool bf16, hipStream_t s)
{
    const dim3 grid(a.d.B * a.d.H), block(M2Threads<P, N>::WIDE);
    const size_t lds = 4 * (size_t)fold_lds_floats(a.d.W, P, N);
    if (bf16) hipLaunchKernelGGL((k_m2_fold<P, N, true>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((k_m2_fold<P, N, false>), grid, block, lds, s, a);
    return hipGetLastError();
}

// The conventional kernel over a few tokens is bound by the state stream and takes a wide
// workgroup, the widest for a single token over at least 16k tiles (with fewer tiles, as at
// batch 1 or 32 with 128 heads, the 512-thread one is faster); over long runs (a prompt) the
// per-token work of each lane dominates and the narrow one, with more rows per lane, is faster
// (measured at 1, 6 and 512 tokens and batch 1 to 512).
template <int P, int N>
hipError_t go_rmw(const M2RmwArgs &a, hipStream_t s)
{
    const dim3 grid(a.d.B * a.d.H);
    if (a.ntok == 1 && (long)a.d.B * a.d.H >= 16384) {
        constexpr int T = M2Threads<P, N>::SINGLE;
        hipLaunchKernelGGL((k_m2_rmw<P, N, T>), grid, dim3(T), 0, s, a);
    } else if (a.ntok <= 8) {
        constexpr int T = M2Threads<P, N>::WIDE;
        hipLaunchKernelGGL((k_m2_rmw<P, N, T>), grid, dim3(T), 0, s, a);
    } else {
        constexpr int T = M2Threads<P, N>::NARROW;
        hipLaunchKernelGGL((k_m2_rmw<P, N, T>), grid, dim3(T), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

// (head_dim P, d_state N) pairs with compiled kernels.
#define RSSM_M2_SHAPES(X) X(16, 16) X(32, 32) X(64, 64) X(64, 128) X(128, 128)

bool m2_supported(int P, int N)
{
#define RSSM_CASE(p, n) if (P == p && N == n) return true;
    RSSM_M2_SHAPES(RSSM_CASE)
#undef RSSM_CASE
    return false;
}

size_t m2_lds_bytes(int P, int N, int W)
{
    // the largest of the decode, verify and fold layouts (every kernel's is at most this)
    const size_t v = verify_lds_floats(W, P, N), f = fold_lds_floats(W, P, N), d = (size_t)W * P + W;
    const size_t m = v > f ? v : f;
    return 4 * (m > d ? m : d);
}

hipError_t m2_decode(const M2StepArgs &a, bool bf16, int mode, hipStream_t s)
{
#define RSSM_C(p, n) if (a.d.P == p && a.d.N == n) return go_decode<p, n>(a, bf16, mode, s);
    RSSM_M2_SHAPES(RSSM_C)
#undef RSSM_C
    return hipErrorInvalidValue;
}

hipError_t m2_verify(const M2StepArgs &a, bool bf16, hipStream_t s)
{
#define RSSM_C(p, n) if (a.d.P == p && a.d.N == n) return go_verify<p, n>(a, bf16, s);
    RSSM_M2_SHAPES(RSSM_C)
#undef RSSM_C
    return hipErrorInvalidValue;
}

hipError_t m2_fold(const M2FoldArgs &a, bool bf16, hipStream_t s)
{
#define RSSM_C(p, n) if (a.d.P == p && a.d.N == n) return go_fold<p, n>(a, bf16, s);
    RSSM_M2_SHAPES(RSSM_C)
#undef RSSM_C
    return hipErrorInvalidValue;
}

hipError_t m2_rmw(const M2RmwArgs &a, hipStream_t s)
{
#define RSSM_C(p, n) if (a.d.P == p && a.d.N == n) return go_rmw<p, n>(a, s);
    RSSM_M2_SHAPES(RSSM_C)
#undef RSSM_C
    return hipErrorInvalidValue;
}

}  // namespace rssm
