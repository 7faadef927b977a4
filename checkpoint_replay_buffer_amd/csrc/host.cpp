// host.cpp -- the C ABI of librssm: argument checks, workspace layout, call-order state and
// kernel dispatch. Every entry point returns before launching anything when a check fails.
#include <hip/hip_runtime.h>

#include <new>

#include "../../include/rssm.h"
#include "internal.h"

using namespace rssm;

struct rssm_ctx {
    rssm_config cfg;
    char *ws;
    size_t ws_bytes;
    int32_t *bk[2];        // [3][B] head, len, ndraft; the live copy is bk[par]
    uint32_t *err;
    float *S0;
    uint16_t *S0b;
    M2Ring m2;
    GdnRing gdn;
    const float *A, *D;
    int par;
    bool pending;          // a verify awaits its commit / rollback
    bool initialized;      // a full rssm_init_checkpoint has run
    // Bounds lo <= len[b] <= hi over all sequences, kept on the host from the call sequence
    // (the device-resident commit / rollback arguments only widen them). A decode with
    // hi + 1 < W cannot fold any sequence and uses the replay-only kernel.
    int lo, hi;
    int pending_k;         // draft count of the pending verify
    // Every sequence is at the same ring position (uhead, ulen), known exactly on the host: true
    // from a full load until a masked load, a commit or a rollback (whose effect depends on
    // device-resident arguments). Such decodes pass the position as a kernel argument.
    bool uni;
    int uhead, ulen;
};

namespace {

constexpr size_t kAlign = 256;

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Layout {
    size_t bk, err, S0, S0b, r0, r1, r2, r3, total;
};

rssm_status check_config(const rssm_config *c)
{
    if (!c) return RSSM_E_ARG;
    if (c->kind != RSSM_MAMBA2 && c->kind != RSSM_GDN && c->kind != RSSM_KDA) return RSSM_E_ARG;
    if (c->batch < 1 || c->nheads < 1 || c->ngroups < 1 || c->dim_v < 1 || c->dim_k < 1)
        return RSSM_E_SHAPE;
    if (c->window < 1 || c->window > kMaxWindow) return RSSM_E_SHAPE;
    if (c->max_draft < 0 || c->max_draft > c->window) return RSSM_E_SHAPE;
    if (c->nheads % c->ngroups != 0) return RSSM_E_SHAPE;
    if (c->flags & ~(uint32_t)(RSSM_F_BF16_READ | RSSM_F_STORE_C)) return RSSM_E_ARG;
    if ((long long)c->batch * c->nheads > 0x7fffffffLL) return RSSM_E_SHAPE;
    if (c->kind == RSSM_GDN) {
        if (c->ngroups != c->nheads) return RSSM_E_SHAPE;
        if (c->flags != 0) return RSSM_E_UNSUPPORTED;
        if (!gdn_supported(c->dim_v, c->dim_k)) return RSSM_E_UNSUPPORTED;
        if (gdn_lds_bytes(c->dim_v, c->dim_k, c->window) > 65536) return RSSM_E_UNSUPPORTED;
    } else if (c->kind == RSSM_KDA) {
        if (c->ngroups != c->nheads) return RSSM_E_SHAPE;
        if (c->flags != 0) return RSSM_E_UNSUPPORTED;
        if (!kda_supported(c->dim_v, c->dim_k)) return RSSM_E_UNSUPPORTED;
        if (kda_lds_bytes(c->dim_v, c->dim_k, c->window, c->max_draft) > 65536) return RSSM_E_UNSUPPORTED;
    } else {
        if (!m2_supported(c->dim_v, c->dim_k)) return RSSM_E_UNSUPPORTED;
        // ring entries staged in LDS by the fold and verify kernels: within 64 KiB per workgroup
        if (m2_lds_bytes(c->dim_v, c->dim_k, c->window) > 65536) return RSSM_E_UNSUPPORTED;
    }
    return RSSM_OK;
}

Layout layout(const rssm_config *c)
{
    const size_t B = c->batch, H = c->nheads, G = c->ngroups, P = c->dim_v, N = c->dim_k,
                 W = c->window;
    Layout L{};
    size_t o = 0;
    L.bk = o;  o += up(2 * 3 * B * sizeof(int32_t));
    L.err = o; o += up(sizeof(uint32_t));
    L.S0 = o;  o += up(B * H * P * N * sizeof(float));
    L.S0b = o; o += (c->flags & RSSM_F_BF16_READ) ? up(B * H * P * N * 2) : 0;
    if (c->kind == RSSM_MAMBA2) {
        L.r0 = o; o += up(B * H * W * P * sizeof(float));                               // x
        L.r1 = o; o += up(B * G * W * N * sizeof(float));                               // B
        L.r2 = o; o += (c->flags & RSSM_F_STORE_C) ? up(B * G * W * N * sizeof(float)) : 0;  // C
        L.r3 = o; o += up(B * H * W * sizeof(float));                                   // dt
    } else {
        const size_t A = c->kind == RSSM_KDA ? N : 1;   // gate: one per key channel (KDA) or scalar
        L.r0 = o; o += up(B * H * W * N * sizeof(float));                               // k
        L.r1 = o; o += up(B * H * W * P * sizeof(float));                               // v
        L.r2 = o; o += up(B * H * W * sizeof(float));                                   // beta
        L.r3 = o; o += up(B * H * W * A * sizeof(float));                               // alpha
    }
    L.total = o;
    return L;
}

hipStream_t strm(void *s) { return reinterpret_cast<hipStream_t>(s); }

Bk flip(rssm_ctx *c) { return Bk{c->bk[c->par], c->bk[c->par ^ 1]}; }

rssm_status launched(rssm_ctx *c, hipError_t e, bool flips)
{
    if (e != hipSuccess) return RSSM_E_DEVICE;
    if (flips) c->par ^= 1;
    return RSSM_OK;
}

M2Dims m2dims(const rssm_config &c)
{
    return M2Dims{c.batch, c.nheads, c.ngroups, c.dim_v, c.dim_k, c.window};
}

GdnDims gdndims(const rssm_config &c)
{
    return GdnDims{c.batch, c.nheads, c.dim_v, c.dim_k, c.window};
}

rssm_status check_inputs(const rssm_config &c, const rssm_inputs *in)
{
    if (!in || in->ntok < 1) return RSSM_E_ARG;
    if (c.kind == RSSM_MAMBA2) {
        if (!aligned16(in->x) || !aligned16(in->B) || !aligned16(in->C) || !in->dt) return RSSM_E_ARG;
    } else {
        if (!aligned16(in->q) || !aligned16(in->k) || !aligned16(in->v) || !in->beta || !in->alpha)
            return RSSM_E_ARG;
        if (c.kind == RSSM_KDA && !aligned16(in->alpha)) return RSSM_E_ARG;   // gate rows read as float4
    }
    return RSSM_OK;
}

// len bounds after folding every sequence with len >= m (m >= 1)
void bounds_after_fold(rssm_ctx *c, int m)
{
    if (c->lo >= m) {
        c->lo = c->hi = 0;
    } else if (c->hi >= m) {
        c->lo = 0;
        c->hi = m - 1;
    }
}

rssm_status ready(const rssm_ctx *c)
{
    if (!c) return RSSM_E_ARG;
    if (!c->initialized) return RSSM_E_STATE;
    if (c->cfg.kind == RSSM_MAMBA2 && (!c->A || !c->D)) return RSSM_E_STATE;
    return RSSM_OK;
}

// The per-sequence segments of the workspace arrays and their packed-slot layout.
SeqCopyArgs seq_args(const rssm_ctx *c, int mode, int n, const int32_t *src, const int32_t *dst,
                     char *buf)
{
    const rssm_config &g = c->cfg;
    const size_t H = g.nheads, G = g.ngroups, P = g.dim_v, N = g.dim_k, W = g.window;
    SeqCopyArgs a{};
    a.mode = mode;
    a.n = n;
    a.B = g.batch;
    a.W = g.window;
    a.src = src;
    a.dst = dst;
    a.buf = buf;
    a.err = c->err;
    auto add = [&](void *base, size_t bytes) {
        if (!base) return;
        a.base[a.nseg] = static_cast<char *>(base);
        a.seg_bytes[a.nseg] = bytes;
        a.unit_log2[a.nseg] = bytes % 16 == 0 ? 4 : 2;
        ++a.nseg;
    };
    add(c->S0, H * P * N * sizeof(float));
    add(c->S0b, H * P * N * sizeof(uint16_t));
    if (g.kind == RSSM_MAMBA2) {
        add(c->m2.x, H * W * P * sizeof(float));
        add(c->m2.B, G * W * N * sizeof(float));
        add(c->m2.C, G * W * N * sizeof(float));
        add(c->m2.dt, H * W * sizeof(float));
    } else {
        add(c->gdn.k, H * W * N * sizeof(float));
        add(c->gdn.v, H * W * P * sizeof(float));
        add(c->gdn.beta, H * W * sizeof(float));
        add(c->gdn.alpha, H * W * (g.kind == RSSM_KDA ? N : 1) * sizeof(float));
    }
    uint64_t off = 0, units = 0;
    for (int k = 0; k < a.nseg; ++k) {
        a.pack_off[k] = off;
        off += (a.seg_bytes[k] + 15) / 16 * 16;
        a.unit_prefix[k] = units;
        units += a.seg_bytes[k] >> a.unit_log2[k];
    }
    a.unit_prefix[a.nseg] = units;
    a.pack_bytes = kSeqHeader + off;
    return a;
}

rssm_status seq_checks(const rssm_ctx *ctx, int32_t n, const void *idx, const void *buf, bool need_buf)
{
    rssm_status s = ready(ctx);
    if (s != RSSM_OK) return s;
    if (n < 0 || n > ctx->cfg.batch || n > 65535) return RSSM_E_ARG;
    if (n > 0 && !idx) return RSSM_E_ARG;
    if (need_buf && n > 0 && !aligned16(buf)) return RSSM_E_ARG;
    if (ctx->pending) return RSSM_E_STATE;
    return RSSM_OK;
}

// The conventional step over a contiguous state (state) or per-sequence tiles (seq, [B] device
// pointers, each to an [H,dim_v,dim_k] block); exactly one of them is given.
rssm_status step_baseline_impl(const rssm_config *cfg, float *state, float *const *seq,
                               const rssm_inputs *in, const float *A, const float *D, float *y,
                               float *snapshots, void *stream)
{
    rssm_status s = check_config(cfg);
    if (s != RSSM_OK) return s;
    if ((s = check_inputs(*cfg, in)) != RSSM_OK) return s;
    if (!aligned16(y) || (snapshots && !aligned16(snapshots))) return RSSM_E_ARG;
    if (cfg->kind == RSSM_MAMBA2) {
        if (!A || !D) return RSSM_E_ARG;
        M2RmwArgs a{m2dims(*cfg), state, snapshots, A, D, in->x, in->B, in->C, in->dt, y, in->ntok,
                    nullptr, seq};
        return m2_rmw(a, strm(stream)) == hipSuccess ? RSSM_OK : RSSM_E_DEVICE;
    }
    GdnRmwArgs a{gdndims(*cfg), state, snapshots, in->q, in->k, in->v, in->beta, in->alpha, y,
                 in->ntok, nullptr, seq};
    const hipError_t e = cfg->kind == RSSM_KDA ? kda_rmw(a, strm(stream)) : gdn_rmw(a, strm(stream));
    return e == hipSuccess ? RSSM_OK : RSSM_E_DEVICE;
}

}  // namespace

extern "C" {

rssm_status rssm_workspace_bytes(const rssm_config *cfg, size_t *bytes)
{
    const rssm_status s = check_config(cfg);
    if (s != RSSM_OK) return s;
    if (!bytes) return RSSM_E_ARG;
    *bytes = layout(cfg).total;
    return RSSM_OK;
}

rssm_status rssm_create(const rssm_config *cfg, void *dev_ws, size_t bytes, rssm_ctx **out)
{
    const rssm_status s = check_config(cfg);
    if (s != RSSM_OK) return s;
    if (!out || !dev_ws || (reinterpret_cast<uintptr_t>(dev_ws) & (kAlign - 1)) != 0) return RSSM_E_ARG;
    const Layout L = layout(cfg);
    if (bytes < L.total) return RSSM_E_SPACE;
    rssm_ctx *c = new (std::nothrow) rssm_ctx();
    if (!c) return RSSM_E_ARG;
    c->cfg = *cfg;
    c->ws = static_cast<char *>(dev_ws);
    c->ws_bytes = bytes;
    const size_t B = cfg->batch;
    c->bk[0] = reinterpret_cast<int32_t *>(c->ws + L.bk);
    c->bk[1] = c->bk[0] + 3 * B;
    c->err = reinterpret_cast<uint32_t *>(c->ws + L.err);
    c->S0 = reinterpret_cast<float *>(c->ws + L.S0);
    c->S0b = (cfg->flags & RSSM_F_BF16_READ) ? reinterpret_cast<uint16_t *>(c->ws + L.S0b) : nullptr;
    if (cfg->kind == RSSM_MAMBA2) {
        c->m2.x = reinterpret_cast<float *>(c->ws + L.r0);
        c->m2.B = reinterpret_cast<float *>(c->ws + L.r1);
        c->m2.C = (cfg->flags & RSSM_F_STORE_C) ? reinterpret_cast<float *>(c->ws + L.r2) : nullptr;
        c->m2.dt = reinterpret_cast<float *>(c->ws + L.r3);
    } else {
        c->gdn.k = reinterpret_cast<float *>(c->ws + L.r0);
        c->gdn.v = reinterpret_cast<float *>(c->ws + L.r1);
        c->gdn.beta = reinterpret_cast<float *>(c->ws + L.r2);
        c->gdn.alpha = reinterpret_cast<float *>(c->ws + L.r3);
    }
    *out = c;
    return RSSM_OK;
}

void rssm_destroy(rssm_ctx *ctx) { delete ctx; }

rssm_status rssm_set_params(rssm_ctx *ctx, const float *A, const float *D)
{
    if (!ctx || !A || !D) return RSSM_E_ARG;
    if (ctx->cfg.kind != RSSM_MAMBA2) return RSSM_E_UNSUPPORTED;
    ctx->A = A;
    ctx->D = D;
    return RSSM_OK;
}

rssm_status rssm_init_checkpoint(rssm_ctx *ctx, const float *state, const int32_t *seq_mask,
                                 void *stream)
{
    if (!ctx || !aligned16(state)) return RSSM_E_ARG;
    if (seq_mask && !ctx->initialized) return RSSM_E_STATE;   // the first load must cover all
    const rssm_config &c = ctx->cfg;
    const hipError_t e = init_checkpoint(ctx->S0, ctx->S0b, state, seq_mask, flip(ctx), ctx->err,
                                         c.batch, c.nheads, (long)c.dim_v * c.dim_k,
                                         c.kind == RSSM_MAMBA2 ? 0 : c.dim_v, strm(stream));
    const rssm_status s = launched(ctx, e, true);
    if (s == RSSM_OK) {
        ctx->initialized = true;
        ctx->pending = false;
        ctx->lo = 0;
        if (!seq_mask) ctx->hi = 0;
        ctx->uni = seq_mask == nullptr;
        ctx->uhead = ctx->ulen = 0;
    }
    return s;
}

rssm_status rssm_decode_step(rssm_ctx *ctx, const rssm_inputs *in, float *y, void *stream)
{
    rssm_status s = ready(ctx);
    if (s != RSSM_OK) return s;
    const rssm_config &c = ctx->cfg;
    if ((s = check_inputs(c, in)) != RSSM_OK) return s;
    if (in->ntok != 1 || !aligned16(y)) return RSSM_E_ARG;
    if (ctx->pending) return RSSM_E_STATE;
    const bool mayfold = ctx->hi + 1 >= c.window;
    if (c.kind == RSSM_MAMBA2) {
        M2StepArgs a{m2dims(c), flip(ctx), ctx->S0, ctx->S0b, ctx->m2, ctx->A, ctx->D,
                     in->x, in->B, in->C, in->dt, y, 1, ctx->uhead, ctx->ulen};
        // every sequence at one known position: none folds (0) or all fold (3); else 1 or 2
        const int mode = ctx->uni ? (ctx->ulen + 1 < c.window ? 0 : 3) : (mayfold ? 2 : 1);
        s = launched(ctx, m2_decode(a, ctx->S0b != nullptr, mode, strm(stream)), true);
    } else {
        GdnStepArgs a{gdndims(c), flip(ctx), ctx->S0, ctx->gdn, in->q, in->k, in->v, in->beta,
                      in->alpha, y, ctx->uhead, ctx->ulen};
        const int mode = (ctx->uni && ctx->ulen + 1 < c.window) ? 0 : (mayfold ? 2 : 1);
        s = launched(ctx, c.kind == RSSM_KDA ? kda_decode(a, mode, strm(stream))
                                             : gdn_decode(a, mode, strm(stream)), true);
    }
    if (s == RSSM_OK) {
        if (ctx->ulen + 1 >= c.window) {
            ctx->uhead = (ctx->uhead + ctx->ulen + 1) % c.window;
            ctx->ulen = 0;
        } else {
            ++ctx->ulen;
        }
        if (!mayfold) {
            ++ctx->lo;
            ++ctx->hi;
        } else if (ctx->lo + 1 >= c.window) {       // every sequence folded
            ctx->lo = ctx->hi = 0;
        } else {                                     // some may have folded, the rest < W
            ctx->lo = 0;
            ctx->hi = c.window - 1;
        }
    }
    return s;
}

rssm_status rssm_consolidate(rssm_ctx *ctx, int32_t min_len, void *stream)
{
    rssm_status s = ready(ctx);
    if (s != RSSM_OK) return s;
    if (ctx->pending) return RSSM_E_STATE;
    const rssm_config &c = ctx->cfg;
    if (c.kind == RSSM_MAMBA2) {
        M2FoldArgs a{m2dims(c), flip(ctx), ctx->S0, ctx->S0b, ctx->m2, ctx->A, min_len, nullptr};
        s = launched(ctx, m2_fold(a, ctx->S0b != nullptr, strm(stream)), true);
    } else {
        GdnFoldArgs a{gdndims(c), flip(ctx), ctx->S0, ctx->gdn, min_len, nullptr};
        s = launched(ctx, c.kind == RSSM_KDA ? kda_fold(a, strm(stream)) : gdn_fold(a, strm(stream)), true);
    }
    if (s == RSSM_OK) {
        const int m = min_len > 1 ? min_len : 1;
        bounds_after_fold(ctx, m);
        if (ctx->ulen >= m) {
            ctx->uhead = (ctx->uhead + ctx->ulen) % c.window;
            ctx->ulen = 0;
        }
    }
    return s;
}

rssm_status rssm_prefill(rssm_ctx *ctx, const rssm_inputs *in, float *y, void *stream)
{
    rssm_status s = ready(ctx);
    if (s != RSSM_OK) return s;
    const rssm_config &c = ctx->cfg;
    if ((s = check_inputs(c, in)) != RSSM_OK) return s;
    if (!aligned16(y)) return RSSM_E_ARG;
    if (ctx->pending) return RSSM_E_STATE;
    if (ctx->hi > 0 && (s = rssm_consolidate(ctx, 1, stream)) != RSSM_OK) return s;
    if (c.kind == RSSM_MAMBA2) {
        M2PrefillArgs a{m2dims(c), flip(ctx), ctx->S0, ctx->S0b, ctx->A, ctx->D,
                        in->x, in->B, in->C, in->dt, y, in->ntok};
        s = launched(ctx, m2_prefill(a, ctx->S0b != nullptr, strm(stream)), true);
    } else {
        GdnPrefillArgs a{gdndims(c), flip(ctx), ctx->S0, in->q, in->k, in->v, in->beta, in->alpha,
                         y, in->ntok};
        s = launched(ctx, c.kind == RSSM_KDA ? kda_prefill(a, strm(stream)) : gdn_prefill(a, strm(stream)),
                     true);
    }
    if (s == RSSM_OK) {
        ctx->lo = ctx->hi = 0;
        ctx->ulen = 0;
    }
    return s;
}

rssm_status rssm_verify(rssm_ctx *ctx, const rssm_inputs *in, float *y, void *stream)
{
    rssm_status s = ready(ctx);
    if (s != RSSM_OK) return s;
    const rssm_config &c = ctx->cfg;
    if ((s = check_inputs(c, in)) != RSSM_OK) return s;
    if (!aligned16(y)) return RSSM_E_ARG;
    if (in->ntok > c.max_draft || in->ntok > c.window) return RSSM_E_ARG;
    if (c.kind == RSSM_GDN && in->ntok > kGdnMaxDraft) return RSSM_E_ARG;
    if (ctx->pending) return RSSM_E_STATE;
    if (c.kind == RSSM_MAMBA2) {
        // With B / C shared by a group of heads (G < H), a sequence whose drafts do not fit
        // (len + K > W) cannot fold inside the verify launch: the group's first head appends the
        // drafts' B rows to slots that wrap onto committed slots, which the group's other heads,
        // in other workgroups of the same launch, still read for their own fold. Those sequences
        // are folded by a consolidation launch first, so the verify launch folds nothing and
        // every slot it writes is disjoint from every slot it reads.
        const int min_fold = c.window - in->ntok + 1;
        if (c.ngroups < c.nheads && ctx->hi >= min_fold) {
            M2FoldArgs f{m2dims(c), flip(ctx), ctx->S0, ctx->S0b, ctx->m2, ctx->A, min_fold, nullptr};
            if ((s = launched(ctx, m2_fold(f, ctx->S0b != nullptr, strm(stream)), true)) != RSSM_OK)
                return s;
            bounds_after_fold(ctx, min_fold);
            if (ctx->ulen >= min_fold) {
                ctx->uhead = (ctx->uhead + ctx->ulen) % c.window;
                ctx->ulen = 0;
            }
        }
        M2StepArgs a{m2dims(c), flip(ctx), ctx->S0, ctx->S0b, ctx->m2, ctx->A, ctx->D,
                     in->x, in->B, in->C, in->dt, y, in->ntok};
        s = launched(ctx, m2_verify(a, ctx->S0b != nullptr, strm(stream)), true);
    } else {
        GdnStepArgs a{gdndims(c), flip(ctx), ctx->S0, ctx->gdn, in->q, in->k, in->v, in->beta,
                      in->alpha, y, 0, 0, in->ntok};
        s = launched(ctx, c.kind == RSSM_KDA ? kda_verify(a, strm(stream)) : gdn_verify(a, strm(stream)),
                     true);
    }
    if (s == RSSM_OK) {
        ctx->pending = true;
        ctx->pending_k = in->ntok;
        bounds_after_fold(ctx, c.window - in->ntok + 1);   // sequences with len + K > W fold
        if (ctx->ulen + in->ntok > c.window) {
            ctx->uhead = (ctx->uhead + ctx->ulen) % c.window;
            ctx->ulen = 0;
        }
    }
    return s;
}

rssm_status rssm_verify_commit(rssm_ctx *ctx, const int32_t *accepted, void *stream)
{
    if (!ctx || !accepted) return RSSM_E_ARG;
    if (!ctx->pending) return RSSM_E_STATE;
    const rssm_status s = launched(ctx, bk_commit(flip(ctx), accepted, ctx->err, ctx->cfg.batch,
                                                  strm(stream)), true);
    if (s == RSSM_OK) {
        ctx->pending = false;
        ctx->hi = ctx->hi + ctx->pending_k < ctx->cfg.window ? ctx->hi + ctx->pending_k : ctx->cfg.window;
        ctx->uni = false;
    }
    return s;
}

rssm_status rssm_rollback(rssm_ctx *ctx, const int32_t *new_len, void *stream)
{
    if (!ctx || !new_len) return RSSM_E_ARG;
    if (!ctx->initialized) return RSSM_E_STATE;
    const rssm_status s = launched(ctx, bk_rollback(flip(ctx), new_len, ctx->err, ctx->cfg.batch,
                                                    strm(stream)), true);
    if (s == RSSM_OK) {
        ctx->pending = false;
        ctx->lo = 0;
        ctx->uni = false;
    }
    return s;
}

rssm_status rssm_step_baseline(const rssm_config *cfg, float *state, const rssm_inputs *in,
                               const float *A, const float *D, float *y, float *snapshots,
                               void *stream)
{
    if (!aligned16(state)) return RSSM_E_ARG;
    return step_baseline_impl(cfg, state, nullptr, in, A, D, y, snapshots, stream);
}

rssm_status rssm_step_baseline_seqs(const rssm_config *cfg, float *const *seq_state,
                                    const rssm_inputs *in, const float *A, const float *D, float *y,
                                    float *snapshots, void *stream)
{
    if (!seq_state) return RSSM_E_ARG;
    return step_baseline_impl(cfg, nullptr, seq_state, in, A, D, y, snapshots, stream);
}

rssm_status rssm_step_baseline_spec(const rssm_config *cfg, float *pool, const int32_t *slot_of,
                                    const rssm_inputs *in, const float *A, const float *D, float *y,
                                    void *stream)
{
    rssm_status s = check_config(cfg);
    if (s != RSSM_OK) return s;
    if ((s = check_inputs(*cfg, in)) != RSSM_OK) return s;
    if (!aligned16(pool) || !aligned16(y) || !slot_of) return RSSM_E_ARG;
    if (cfg->kind != RSSM_MAMBA2) {
        GdnRmwArgs a{gdndims(*cfg), pool, nullptr, in->q, in->k, in->v, in->beta, in->alpha, y,
                     in->ntok, slot_of};
        const hipError_t e = cfg->kind == RSSM_KDA ? kda_rmw(a, strm(stream)) : gdn_rmw(a, strm(stream));
        return e == hipSuccess ? RSSM_OK : RSSM_E_DEVICE;
    }
    if (!A || !D) return RSSM_E_ARG;
    M2RmwArgs a{m2dims(*cfg), pool, nullptr, A, D, in->x, in->B, in->C, in->dt, y, in->ntok, slot_of};
    return m2_rmw(a, strm(stream)) == hipSuccess ? RSSM_OK : RSSM_E_DEVICE;
}

rssm_status rssm_baseline_commit(const rssm_config *cfg, int32_t *slot_of, const int32_t *accepted,
                                 int32_t ndraft, void *stream)
{
    const rssm_status s = check_config(cfg);
    if (s != RSSM_OK) return s;
    if (!slot_of || !accepted || ndraft < 1) return RSSM_E_ARG;
    return slot_commit(slot_of, accepted, cfg->batch, ndraft, strm(stream)) == hipSuccess
               ? RSSM_OK : RSSM_E_DEVICE;
}

rssm_status rssm_materialize(rssm_ctx *ctx, float *state_out, void *stream)
{
    rssm_status s = ready(ctx);
    if (s != RSSM_OK) return s;
    if (!aligned16(state_out)) return RSSM_E_ARG;
    const rssm_config &c = ctx->cfg;
    const Bk bk{ctx->bk[ctx->par], nullptr};
    if (c.kind == RSSM_MAMBA2) {
        M2FoldArgs a{m2dims(c), bk, ctx->S0, nullptr, ctx->m2, ctx->A, 1, state_out};
        return launched(ctx, m2_fold(a, false, strm(stream)), false);
    }
    GdnFoldArgs a{gdndims(c), bk, ctx->S0, ctx->gdn, 1, state_out};
    return launched(ctx, c.kind == RSSM_KDA ? kda_fold(a, strm(stream)) : gdn_fold(a, strm(stream)), false);
}

rssm_status rssm_seq_state_bytes(const rssm_config *cfg, size_t *bytes)
{
    if (!cfg || !bytes) return RSSM_E_ARG;
    const rssm_status s = check_config(cfg);
    if (s != RSSM_OK) return s;
    rssm_ctx c{};
    c.cfg = *cfg;
    // any non-null bases give the segment sizes
    char dummy[16];
    c.S0 = reinterpret_cast<float *>(dummy);
    c.S0b = (cfg->flags & RSSM_F_BF16_READ) ? reinterpret_cast<uint16_t *>(dummy) : nullptr;
    float *f = reinterpret_cast<float *>(dummy);
    c.m2 = M2Ring{f, f, (cfg->flags & RSSM_F_STORE_C) ? f : nullptr, f};
    c.gdn = GdnRing{f, f, f, f};
    *bytes = seq_args(&c, kSeqExport, 0, nullptr, nullptr, nullptr).pack_bytes;
    return RSSM_OK;
}

rssm_status rssm_fork(rssm_ctx *ctx, const int32_t *src, const int32_t *dst, int32_t n, void *stream)
{
    rssm_status s = seq_checks(ctx, n, src, nullptr, false);
    if (s != RSSM_OK) return s;
    if (n > 0 && !dst) return RSSM_E_ARG;
    const SeqCopyArgs a = seq_args(ctx, kSeqFork, n, src, dst, nullptr);
    return launched(ctx, seq_copy(a, flip(ctx), strm(stream)), true);
}

rssm_status rssm_export(rssm_ctx *ctx, const int32_t *seq, int32_t n, void *buf, void *stream)
{
    rssm_status s = seq_checks(ctx, n, seq, buf, true);
    if (s != RSSM_OK) return s;
    const SeqCopyArgs a = seq_args(ctx, kSeqExport, n, seq, nullptr, static_cast<char *>(buf));
    return launched(ctx, seq_copy(a, Bk{ctx->bk[ctx->par], nullptr}, strm(stream)), false);
}

rssm_status rssm_import(rssm_ctx *ctx, const int32_t *seq, int32_t n, const void *buf, void *stream)
{
    rssm_status s = seq_checks(ctx, n, seq, buf, true);
    if (s != RSSM_OK) return s;
    const SeqCopyArgs a = seq_args(ctx, kSeqImport, n, nullptr, seq,
                                   const_cast<char *>(static_cast<const char *>(buf)));
    s = launched(ctx, seq_copy(a, flip(ctx), strm(stream)), true);
    if (s == RSSM_OK) {                       // the imported lengths are device data
        ctx->lo = 0;
        ctx->hi = ctx->cfg.window;
        ctx->uni = false;
    }
    return s;
}

rssm_status rssm_read_bookkeeping(rssm_ctx *ctx, int32_t *head, int32_t *len, int32_t *ndraft,
                                  uint32_t *dev_err, void *stream)
{
    if (!ctx) return RSSM_E_ARG;
    const hipStream_t st = strm(stream);
    const size_t B = ctx->cfg.batch;
    const int32_t *live = ctx->bk[ctx->par];
    hipError_t e = hipSuccess;
    if (head && e == hipSuccess) e = hipMemcpyAsync(head, live, B * 4, hipMemcpyDeviceToHost, st);
    if (len && e == hipSuccess) e = hipMemcpyAsync(len, live + B, B * 4, hipMemcpyDeviceToHost, st);
    if (ndraft && e == hipSuccess) e = hipMemcpyAsync(ndraft, live + 2 * B, B * 4, hipMemcpyDeviceToHost, st);
    if (dev_err && e == hipSuccess) e = hipMemcpyAsync(dev_err, ctx->err, 4, hipMemcpyDeviceToHost, st);
    if (dev_err && e == hipSuccess) e = clear_word(ctx->err, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    return e == hipSuccess ? RSSM_OK : RSSM_E_DEVICE;
}

const char *rssm_status_str(rssm_status s)
{
    switch (s) {
    case RSSM_OK: return "ok";
    case RSSM_E_ARG: return "invalid argument (null or misaligned pointer, bad value)";
    case RSSM_E_SHAPE: return "invalid or inconsistent dimensions";
    case RSSM_E_SPACE: return "workspace too small";
    case RSSM_E_STATE: return "call-order misuse";
    case RSSM_E_DEVICE: return "HIP launch or copy failed";
    case RSSM_E_UNSUPPORTED: return "shape or option without a compiled kernel";
    default: return "unknown status";
    }
}

}  // extern "C"
