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
#include <type_traits>

#include "dev_common.h"
#include "internal.h"
#include "mfma_tile.h"

namespace rssm {
namespace {

constexpr int kChunk = 16;
constexpr int kMS = kChunk + 4;   // row stride of the 16 x 16 blocks in LDS

// Threads per workgroup (one (b, h) tile) and waves per SIMD the prefill is compiled for.
template <int P, int N>
struct PrefillShape {
    static constexpr int TPB = TileShape<P, N>::TPB, OCC = 4;
};

// LDS floats: two staging buffers of the rows read on both sides of the mid-chunk barrier, x
// [16][P+4] and B [16][N+4]; one buffer of those read before it only, C [16][N+4] and dt [16];
// then one 16 x 16 partial of B C^T per wave, the weights w[t][j] [16][20], w[15][j] [16] and
// Lam_t [16]. At 64 x 128 that is 40,640 bytes: four workgroups fit the 160 KB of a CU.
template <int P, int N>
__host__ __device__ constexpr int prefill_buf_floats()
{
    return kChunk * (P + 4) + kChunk * (N + 4);
}
template <int P, int N>
__host__ __device__ constexpr int prefill_lds_floats()
{
    return 2 * prefill_buf_floats<P, N>() + kChunk * (N + 4) + kChunk
         + (PrefillShape<P, N>::TPB / 64 + 1) * kChunk * kMS + 2 * kChunk;
}

// Inclusive prefix sum over the 16 lanes of each row of the wave (lanes 16 g .. 16 g + 15): four
// shifted adds across the row, the lanes shifted in from outside it reading zero.
__device__ __forceinline__ float row_scan16(float v)
{
#define RSSM_SHR(n) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + (n), 0xF, 0xF, true))
    v += RSSM_SHR(1);
    v += RSSM_SHR(2);
    v += RSSM_SHR(4);
    v += RSSM_SHR(8);
#undef RSSM_SHR
    return v;
}

// Decay weights of the chunk, spread over the NW waves of the workgroup; lane (g, c) of wave w
// takes t = c and j = 4 g + r for r = w, w + NW, ... < 4:
//     w[t][j] = dt_j exp(A sum_{j<i<=t} dt_i) (0 for j > t)  -> sh_wm[t][j]
//     w[15][j] = dt_j exp(A sum_{j<i<=15} dt_i)              -> sh_wf (lanes c = 15)
//     Lam_t = exp(A sum_{i<=t} dt_i)                        -> sh_lam (wave 0, lanes g = 0)
// Every exponent is a sum of the step sizes between the two tokens, formed as a prefix sum over
// the row of lanes c of dt_c masked to c > j: no differences of running sums.
template <int NW>
__device__ __forceinline__ void chunk_weights(const float *sh_dt, float Ah, float *sh_wm,
                                              float *sh_wf, float *sh_lam, int wv)
{
    const int lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
    const float dc = sh_dt[cl];
    for (int r = wv; r < 4; r += NW) {
        const int j = 4 * g + r;
        const float dj = sh_dt[j];
        const float e = row_scan16(cl > j ? dc : 0.f);   // sum_{j<i<=c} dt_i
        const float wm = j <= cl ? dj * expf(Ah * e) : 0.f;
        sh_wm[cl * kMS + j] = wm;
        if (cl == kChunk - 1) sh_wf[j] = wm;
    }
    if (wv == 0) {
        const float lam = expf(Ah * row_scan16(dc));
        if (g == 0) sh_lam[cl] = lam;
    }
}

// Sum of the per-wave partials of B C^T, as a pairwise tree.
template <int NW>
__device__ __forceinline__ float4 sum_partials(const float4 (&p)[NW])
{
    if constexpr (NW == 1) {
        return p[0];
    } else {
        float4 h[NW / 2];
#pragma unroll
        for (int w = 0; w < NW / 2; ++w)
            h[w] = make_float4(p[2 * w].x + p[2 * w + 1].x, p[2 * w].y + p[2 * w + 1].y,
                               p[2 * w].z + p[2 * w + 1].z, p[2 * w].w + p[2 * w + 1].w);
        return sum_partials<NW / 2>(h);
    }
}

// float4 at a byte offset from a base pointer: with a wave-uniform base the load takes the
// scalar-base form and the lane offset stays one 32-bit register.
__device__ __forceinline__ float4 ld4_at(const float *base, uint32_t off)
{
    return *reinterpret_cast<const float4 *>(reinterpret_cast<const char *>(base) + off);
}

// The chunk's rows of x, B, C and dt held in registers between their load and their LDS store.
// Lane t takes float4 i = t + q TPB of the chunk's rows (row i / PF of x, i / NF of B and C). The
// addresses are formed at each load from t and the (uniform) row bases, not kept in registers
// from one chunk to the next.
template <int P, int N>
struct ChunkRows {
    static constexpr int TPB = PrefillShape<P, N>::TPB, PF = P / 4, NF = N / 4;
    static constexpr int XQ = (kChunk * PF + TPB - 1) / TPB, BQ = (kChunk * NF + TPB - 1) / TPB;
    float4 x[XQ], b[BQ], c[BQ];
    float dt;

    // rows of tokens t0 .. t0 + ct - 1 (zeros past them); xb, bb, cb, db point at token t0's row
    // of this tile, rows BH (x, dt) or BG (B, C) apart. A full chunk (every chunk but a ragged
    // last one) loads without predicates.
    __device__ __forceinline__ void load(const float *xb, const float *bb, const float *cb,
                                         const float *db, size_t BH, size_t BG, int ct, int t)
    {
        asm volatile("" : "+v"(t));
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int q = 0; q < XQ; ++q) {
            const int i = t + q * TPB, j = i / PF, o = (i - j * PF) * 4;
            const bool in = (XQ * TPB == kChunk * PF || i < kChunk * PF) && (ct == kChunk || j < ct);
            x[q] = in ? ld4(xb + (size_t)j * BH * P + o) : z;
        }
#pragma unroll
        for (int q = 0; q < BQ; ++q) {
            const int i = t + q * TPB, j = i / NF, o = (i - j * NF) * 4;
            const bool in = (BQ * TPB == kChunk * NF || i < kChunk * NF) && (ct == kChunk || j < ct);
            const size_t e = (size_t)j * BG * N + o;
            b[q] = in ? ld4(bb + e) : z;
            c[q] = in ? ld4(cb + e) : z;
        }
        // a full chunk: lanes t >= 16 load a row too, and only lanes t < 16 keep theirs
        const int jt = ct == kChunk ? (t & (kChunk - 1)) : t;
        dt = ct == kChunk || t < ct ? db[(size_t)jt * BH] : 0.f;
    }

    // The same for a full chunk whose rows lie within 4 GiB of its first row: no predicates, and
    // every address is the (uniform) row base plus a 32-bit lane offset in bytes.
    __device__ __forceinline__ void load_full(const float *xb, const float *bb, const float *cb,
                                              const float *db, uint32_t BH, uint32_t BG, int t)
    {
        asm volatile("" : "+v"(t));
#pragma unroll
        for (int q = 0; q < XQ; ++q) {
            const int i = t + q * TPB, j = i / PF, o = (i - j * PF) * 16;
            if (XQ * TPB == kChunk * PF || i < kChunk * PF)
                x[q] = ld4_at(xb, (uint32_t)j * (BH * (4u * P)) + (uint32_t)o);
        }
#pragma unroll
        for (int q = 0; q < BQ; ++q) {
            const int i = t + q * TPB, j = i / NF, o = (i - j * NF) * 16;
            if (BQ * TPB == kChunk * NF || i < kChunk * NF) {
                const uint32_t e = (uint32_t)j * (BG * (4u * N)) + (uint32_t)o;
                b[q] = ld4_at(bb, e);
                c[q] = ld4_at(cb, e);
            }
        }
        // lanes t >= 16 load a row too, and only lanes t < 16 keep theirs
        dt = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(db) +
                                              (uint32_t)(t & (kChunk - 1)) * (4u * BH));
    }

    __device__ __forceinline__ void store(float *sh_x, float *sh_B, float *sh_C, float *sh_dt, int t) const
    {
        constexpr int XS = P + 4, BS = N + 4;
#pragma unroll
        for (int q = 0; q < XQ; ++q) {
            const int i = t + q * TPB, j = i / PF, o = (i - j * PF) * 4;
            if (XQ * TPB == kChunk * PF || i < kChunk * PF) st4(sh_x + j * XS + o, x[q]);
        }
#pragma unroll
        for (int q = 0; q < BQ; ++q) {
            const int i = t + q * TPB, j = i / NF, o = (i - j * NF) * 4;
            if (BQ * TPB == kChunk * NF || i < kChunk * NF) {
                st4(sh_B + j * BS + o, b[q]);
                st4(sh_C + j * BS + o, c[q]);
            }
        }
        if (t < kChunk) sh_dt[t] = dt;
    }
};

// Two barriers per chunk: the chunk's rows (prefetched into registers during the previous chunk)
// go to one of two LDS buffers; the waves then form the blocks that do not depend on the state
// (B C^T split over the waves by k-blocks, the decay weights) next to their C S^T products, and
// after the second barrier every wave has what it needs for its outputs and its part of the
// update.
template <int P, int N, bool BF16>
__global__ void __launch_bounds__((PrefillShape<P, N>::TPB), (PrefillShape<P, N>::OCC)) k_m2_prefill(M2PrefillArgs a)
{
    using F = MfmaTile<P, N, PrefillShape<P, N>::TPB / 64>;
    constexpr int NW = F::NW, IBW = F::IBW, KB = F::KB, XS = F::RS, BS = F::CS;
    constexpr int NA = KB >= 2 ? 2 : KB;   // independent accumulators of the d_state products
                                           // (two: the registers of four waves per SIMD)
    constexpr int KBW = KB / NW;           // k-blocks of B C^T per wave
    static_assert(KBW * NW == KB, "B C^T split");
    constexpr int BUF = prefill_buf_floats<P, N>();
    extern __shared__ float smem[];
    float *sh_C = smem + 2 * BUF;          // [16][BS]       C of the chunk
    float *sh_dt = sh_C + kChunk * BS;     // [16]           dt of the chunk
    float *sh_P = sh_dt + kChunk;          // [NW][16][kMS]  partials of B C^T
    float *sh_wm = sh_P + NW * kChunk * kMS;   // [16][kMS]  w[t][j] (0 for j > t)
    float *sh_wf = sh_wm + kChunk * kMS;   // [16]       w[15][j]
    float *sh_lam = sh_wf + kChunk;        // [16]       Lam_t

    const int B = a.d.B, H = a.d.H, G = a.d.G, T = a.T;
    const int tile = blockIdx.x, b = tile / H, h = tile - b * H, g0 = h / (H / G);
    const size_t bh = (size_t)tile, bg = (size_t)b * G + g0;
    const size_t BH = (size_t)B * H, BG = (size_t)B * G;
    // a chunk's rows span 16 token strides of B H (x, dt) or B G (B, C) rows: 32-bit byte
    // offsets reach them all
    const bool narrow = (BH * P > BG * N ? BH * P : BG * N) * 4 * kChunk <= 0xFFFFFFFFull;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6, g = lane >> 4, cl = lane & 15;
    const float Ah = a.A[h], Dh = a.D[h];

    // token-0 rows of this tile; a chunk adds t0 rows of stride BH (x, dt) or BG (B, C)
    const float *x0 = a.x + bh * P, *b0 = a.Bm + bg * N, *c0 = a.C + bg * N, *d0 = a.dt + bh;
    float *y0 = a.y + bh * P;
    ChunkRows<P, N> rows;
    rows.load(x0, b0, c0, d0, BH, BG, T < kChunk ? T : kChunk, t);
    float4 s[IBW][KB];
    float *S0 = a.S0 + bh * (size_t)(P * N);
    int off[IBW];
#pragma unroll
    for (int ib = 0; ib < IBW; ++ib) {
        off[ib] = (16 * (wv * IBW + ib) + cl) * N + 4 * g;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s[ib][kb] = ld4_nt(S0 + off[ib] + 16 * kb);
    }
    tile_loaded(s);

    // One chunk of tokens t0 .. t0 + ct - 1. FULL (ct = 16, every chunk but a ragged last one)
    // stores every output row without predicates, so the chunk is straight-line code. NEXT_FULL:
    // the next chunk is full too and its rows take the unpredicated 32-bit-offset load. Each
    // kind of load has its own copy of the chunk: a load path that joins the other one would make
    // the compiler wait, before the loads, for every memory operation still in flight (the
    // previous chunk's output stores among them).
    auto chunk = [&](auto full, auto next_full, int t0, int buf) {
        constexpr bool FULL = decltype(full)::value, NEXT_FULL = decltype(next_full)::value;
        const int ct = FULL ? kChunk : T - t0;
        float *sh_x = smem + buf * BUF;
        float *sh_B = sh_x + kChunk * XS;
        // C and dt are read before the mid-chunk barrier only: every wave is past it before any
        // wave stores the next chunk's, so they need one buffer; x and B are read after it too
        rows.store(sh_x, sh_B, sh_C, sh_dt, t);
        __syncthreads();
        const size_t t1 = t0 + kChunk;    // the next chunk's rows, in flight during this chunk
        if constexpr (NEXT_FULL)
            rows.load_full(x0 + t1 * BH * P, b0 + t1 * BG * N, c0 + t1 * BG * N, d0 + t1 * BH,
                           (uint32_t)BH, (uint32_t)BG, t);
        else if ((int)t1 < T)
            rows.load(x0 + t1 * BH * P, b0 + t1 * BG * N, c0 + t1 * BG * N, d0 + t1 * BH, BH, BG,
                      T - (int)t1 < kChunk ? T - (int)t1 : kChunk, t);

        // 1. S-independent blocks first: every wave its share of B C^T (k-blocks wv KBW ..
        //    wv KBW + KBW - 1) and of the decay weights of the chunk
        {
            v4f pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kq = 0; kq < KBW; ++kq) {
                const int kb = wv * KBW + kq;
                const float4 bv = ld4(sh_B + cl * BS + 16 * kb + 4 * g);   // A: B[j = c][k]
                const float4 cv = ld4(sh_C + cl * BS + 16 * kb + 4 * g);   // B: C[t = c][k]
                pp = mfma4(bv.x, cv.x, pp);
                pp = mfma4(bv.y, cv.y, pp);
                pp = mfma4(bv.z, cv.z, pp);
                pp = mfma4(bv.w, cv.w, pp);
            }
            // register r of lane (g, c) holds B_{4g+r} . C_c over this share: stored at
            // [c][4 g + r], where every wave's lane (g, c) reads it back
            st4(sh_P + wv * kChunk * kMS + cl * kMS + 4 * g, make_float4(pp[0], pp[1], pp[2], pp[3]));
        }
        chunk_weights<NW>(sh_dt, Ah, sh_wm, sh_wf, sh_lam, wv);
        //    every wave: Z = C S^T for its i-blocks (S at the chunk start)
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
            z[ib] = tree_sum<NA>(zp);        // (S C_tt)[i] for tt = 4 g + r, i = 16 ib' + c
        }
        mfma_settle();
        __syncthreads();

        // 2. M[t = c][j = 4 g + r] = w[t][j] (B_j . C_t), the A operand of M X; Lam of the output
        //    rows t = 4 g + r; the fold weights w[15][j = 4 g + r] and Lam_15
        float4 bcs[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) bcs[w] = ld4(sh_P + w * kChunk * kMS + cl * kMS + 4 * g);
        const float4 bc = sum_partials<NW>(bcs);
        const float4 wm = ld4(sh_wm + cl * kMS + 4 * g);
        const float ma[4] = {wm.x * bc.x, wm.y * bc.y, wm.z * bc.z, wm.w * bc.w};
        const float4 lm = ld4(sh_lam + 4 * g), wq = ld4(sh_wf + 4 * g);
        const float lam[4] = {lm.x, lm.y, lm.z, lm.w}, wf[4] = {wq.x, wq.y, wq.z, wq.w};
        const float lam_end = sh_lam[kChunk - 1];

#pragma unroll
        for (int ib = 0; ib < IBW; ++ib) {
            const int i = 16 * (wv * IBW + ib) + cl;
            // 3. Y = Lam o Z + M X + D X
            float xj[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) xj[r] = sh_x[(4 * g + r) * XS + i];   // X[j = 4 g + r][i]
            v4f acc = {0.f, 0.f, 0.f, 0.f};
            acc = mfma4(ma[0], xj[0], acc);
            acc = mfma4(ma[1], xj[1], acc);
            acc = mfma4(ma[2], xj[2], acc);
            acc = mfma4(ma[3], xj[3], acc);
            float yv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) yv[r] = lam[r] * z[ib][r] + acc[r] + Dh * xj[r];
            // keep the reads of the accumulators here, next to their chains, rather than sunk into
            // the conditional stores below
            asm volatile("" ::"v"(yv[0]), "v"(yv[1]), "v"(yv[2]), "v"(yv[3]));
            int iy = i;                     // the output address is formed here, each chunk
            asm volatile("" : "+v"(iy));
            float *yc = y0 + (size_t)(t0 + 4 * g) * BH * P + iy;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (FULL || 4 * g + r < ct) yc[(size_t)r * BH * P] = yv[r];
            // 4. S <- Lam_15 S + B^T (w X): B operand w[15][j] x_j[i] for j = 4 g + r
            float wx[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) wx[r] = wf[r] * xj[r];
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
    };
    int t0 = 0, buf = 0;
    if (narrow)
        for (; t0 + 2 * kChunk <= T; t0 += kChunk, buf ^= 1)
            chunk(std::true_type{}, std::true_type{}, t0, buf);
    for (; t0 + kChunk <= T; t0 += kChunk, buf ^= 1) chunk(std::true_type{}, std::false_type{}, t0, buf);
    if (t0 < T) chunk(std::false_type{}, std::false_type{}, t0, buf);

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
    const dim3 grid(a.d.B * a.d.H), block(PrefillShape<P, N>::TPB);
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
