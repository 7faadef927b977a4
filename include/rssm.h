/*
 * rssm.h -- C ABI of librssm, the ReplaySSM decode hot path for the SSM layers of hybrid
 * attention/SSM models, written for AMD MI355X (gfx950).
 *
 * The method (as described by five short web articles on ReplaySSM):
 *  - an SSM layer's per-sequence state is kept as a full-precision checkpoint S0 plus a short
 *    ring buffer of the last W tokens' inputs instead of being read and rewritten whole on every
 *    token (ia.goatify.app article "NVIDIA y Princeton aceleran modelos híbridos...", paragraph
 *    "ReplaySSM cambia qué se almacena"; newsverum.com item "NVIDIA e Princeton apresentam
 *    ReplaySSM...", lede);
 *  - a normal decode step appends its inputs to the buffer and computes its output from the
 *    read-only checkpoint; only a full buffer is consolidated into a new checkpoint
 *    (ia.goatify.app, paragraph "El checkpoint reduce escrituras de estado");
 *  - speculative decoding stores the drafts' inputs, evaluates outputs only, and accepts a prefix
 *    by moving a pointer, with no per-draft state copy (ia.goatify.app, paragraph "El retroceso
 *    usa un puntero del búfer"; fagnersouza.tech post "ReplaySSM: o ganho aparece na carga
 *    concorrente...", section "O que muda para quem desenvolve");
 *  - an optional lower-precision copy of the checkpoint may serve the reads while the recurrence
 *    stays in full precision (ia.goatify.app, paragraph "La precisión separa lectura y
 *    recurrencia"); here that copy is bf16;
 *  - the layer types are Mamba-2, Gated DeltaNet and Kimi Delta Attention (news.hamidun.com item
 *    "NVIDIA présente ReplaySSM...", section "Pourquoi les hybrides sont devenus la norme"; the
 *    pages give no formula for Kimi Delta Attention, read here as Gated DeltaNet with one forget
 *    gate per key channel).
 *
 * Recurrences (per sequence b and head h; the plain reading, since the pages print no formulas):
 *   Mamba-2, state S [P x N]:   S <- exp(dt A_h) S + dt x B^T,   y = S C + D_h x
 *   Gated DeltaNet, S [dv x dk]: S <- alpha S (I - beta k k^T) + beta v k^T,   o = S q
 *   Kimi Delta Attention, S [dv x dk]: S <- S diag(a) (I - beta k k^T) + beta v k^T,   o = S q
 * Outputs use the post-update state. ReplaySSM produces the same outputs up to rounding
 * (fagnersouza.tech post, section "Cuidados e limites").
 *
 * Conventions for every function:
 *  - Tensor pointers are DEVICE pointers unless marked HOST. All tensors are fp32, row-major and
 *    contiguous (last index fastest) and 16-byte aligned. Shapes use B batch, H heads, G B/C
 *    groups (H % G == 0, head h uses group h / (H / G)), P = dim_v, N = dim_k, W ring length.
 *  - Memory is caller-owned: the caller allocates one device workspace of
 *    rssm_workspace_bytes() bytes (it holds S0, the bf16 copy, the rings, the bookkeeping and the
 *    error word) and all inputs and outputs, and keeps them alive until the queued work finishes.
 *    The library allocates only its small host object; it never allocates or frees device memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work is asynchronous and
 *    stream-ordered; only rssm_read_bookkeeping synchronises. A context is used from one stream
 *    at a time and is not thread-safe.
 *  - Errors: problems the host can see return a negative rssm_status before anything is launched
 *    (bad pointer or alignment, bad shape, too small workspace, call-order misuse). Problems in
 *    device-resident arguments (commit / rollback lengths) set sticky bits in the device error
 *    word, read with rssm_read_bookkeeping. A failed launch returns RSSM_E_DEVICE. Nothing throws
 *    across the ABI.
 *  - Bookkeeping per sequence: head (ring slot of the oldest buffered entry), len (committed
 *    buffered entries, 0..W) and ndraft (drafts appended by the last verify). Logical entry j of
 *    sequence b lives in ring slot (head + j) mod W; a fold of n entries sets
 *    head <- (head + n) mod W and len <- 0.
 */
#ifndef RSSM_H
#define RSSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct rssm_ctx rssm_ctx;
typedef int32_t rssm_status;

enum {
    RSSM_OK = 0,
    RSSM_E_ARG = -1,          /* null / misaligned pointer, bad scalar argument */
    RSSM_E_SHAPE = -2,        /* inconsistent or non-positive dimensions */
    RSSM_E_SPACE = -3,        /* workspace smaller than rssm_workspace_bytes() */
    RSSM_E_STATE = -4,        /* call-order misuse (e.g. decode with drafts pending) */
    RSSM_E_DEVICE = -5,       /* HIP launch or copy failure */
    RSSM_E_UNSUPPORTED = -6   /* shape or option combination without a compiled kernel */
};

/* Device error word bits (sticky until read). */
enum {
    RSSM_DEV_COMMIT_RANGE = 1u,    /* accepted[b] outside [0, ndraft[b]]; len left unchanged */
    RSSM_DEV_ROLLBACK_RANGE = 2u,  /* new_len[b] outside [0, len[b]]; len left unchanged */
    RSSM_DEV_INDEX_RANGE = 8u,     /* a fork / export / import sequence index outside [0, B); that
                                      pair is skipped */
    RSSM_DEV_IMPORT_HEADER = 16u   /* an imported slot's header is not one an export writes (head
                                      outside [0, W), len outside [0, W] or pending drafts); that
                                      pair is skipped: the sequence keeps its state */
};

enum { RSSM_MAMBA2 = 1, RSSM_GDN = 2, RSSM_KDA = 3 };

enum {
    RSSM_F_BF16_READ = 1u,   /* keep a bf16 copy of S0 and read it for replayed outputs */
    RSSM_F_STORE_C = 2u      /* also store C in the ring (Mamba-2); kept but not read */
};

typedef struct {
    int32_t kind;        /* RSSM_MAMBA2, RSSM_GDN or RSSM_KDA */
    int32_t batch;       /* B */
    int32_t nheads;      /* H */
    int32_t ngroups;     /* G (Mamba-2 B/C groups; must be H for GDN and KDA) */
    int32_t dim_v;       /* P (Mamba-2 head_dim) or d_v (GDN, KDA) */
    int32_t dim_k;       /* N (Mamba-2 d_state) or d_k (GDN, KDA) */
    int32_t window;      /* W, ring length, 1..32 */
    int32_t max_draft;   /* largest K accepted by rssm_verify, 0..W (0 = no speculative use) */
    uint32_t flags;      /* RSSM_F_* */
} rssm_config;

/* Inputs of ntok consecutive tokens, token-major (leading axis ntok).
 * Mamba-2: x [ntok,B,H,P], B and C [ntok,B,G,N], dt [ntok,B,H] (dt > 0, already discretised).
 * GDN:     q and k [ntok,B,H,dk], v [ntok,B,H,dv], beta and alpha [ntok,B,H].
 * KDA:     as GDN, but alpha [ntok,B,H,dk] (one forget gate per key channel), 16-byte aligned.
 * Fields of the other kind are ignored and may be NULL. */
typedef struct {
    int32_t ntok;
    const float *x, *B, *C, *dt;
    const float *q, *k, *v, *beta, *alpha;
} rssm_inputs;

/* Bytes of device workspace needed for `cfg` (host only, no device call). */
rssm_status rssm_workspace_bytes(const rssm_config *cfg, size_t *bytes /* HOST */);

/* Create a context over a caller-owned workspace `dev_ws` of `bytes` bytes (256-byte aligned).
 * Nothing is launched; call rssm_init_checkpoint before any decode. */
rssm_status rssm_create(const rssm_config *cfg, void *dev_ws, size_t bytes, rssm_ctx **out /* HOST */);

/* Free the host object. The workspace stays the caller's. NULL is allowed. */
void rssm_destroy(rssm_ctx *ctx);

/* Mamba-2 per-head parameters A [H] (negative decay rate) and D [H] (skip weight), device
 * pointers kept by reference: they must stay valid while the context is used. */
rssm_status rssm_set_params(rssm_ctx *ctx, const float *A, const float *D);

/* The state of a sequence is a checkpoint plus a short buffer of its recent inputs (ia.goatify.app
 * article, paragraph "ReplaySSM cambia qué se almacena").
 * Load checkpoints: S0[b] <- state[b] ([B,H,dim_v,dim_k]) for every sequence b with
 * seq_mask[b] != 0 (seq_mask [B] int32, or NULL for all), refresh the bf16 copy, and reset those
 * sequences' bookkeeping to head = len = ndraft = 0. With seq_mask NULL the error word is cleared
 * too. Clears a pending verify. */
rssm_status rssm_init_checkpoint(rssm_ctx *ctx, const float *state, const int32_t *seq_mask,
                                 void *stream);

/* A normal step appends its inputs to the buffer and computes the output from the checkpoint;
 * only a full buffer is consolidated (ia.goatify.app article, paragraph "El checkpoint reduce
 * escrituras de estado").
 * One decode token (inputs->ntok must be 1) for every sequence; writes y [B,H,dim_v].
 * The token becomes logical entry len and its output is computed from the read-only checkpoint
 * and the buffered entries ("replay"). When the token fills the buffer (len + 1 >= W) the same
 * launch folds all buffered entries and the token into S0 and the output is read from the new
 * checkpoint; then len = 0. Requires no pending verify (RSSM_E_STATE). */
rssm_status rssm_decode_step(rssm_ctx *ctx, const rssm_inputs *in, float *y, void *stream);

/* Consolidation, the update of the persistent state from the buffered entries (ia.goatify.app
 * article, paragraph "El checkpoint reduce escrituras de estado").
 * Fold the buffered entries of every sequence with len >= max(min_len, 1) into its checkpoint.
 * Requires no pending verify. */
rssm_status rssm_consolidate(rssm_ctx *ctx, int32_t min_len, void *stream);

/* Prefill: run T = in->ntok prompt tokens (Mamba-2 in: x [T,B,H,P], B and C [T,B,G,N],
 * dt [T,B,H]; Gated DeltaNet in: q and k [T,B,H,dim_k], v [T,B,H,dim_v], beta and alpha [T,B,H];
 * Kimi Delta Attention in: the same with alpha [T,B,H,dim_k])
 * through the recurrence from each sequence's current state and make the final state
 * the checkpoint (ia.goatify.app article "NVIDIA y Princeton aceleran modelos hibridos...",
 * paragraph "ReplaySSM cambia que se almacena": the decode path starts from a checkpoint plus
 * recent inputs). y [T,B,H,dim_v] (required) receives every prompt token's output, the same as T
 * decode steps would give. Buffered entries are folded first (one consolidation launch when any
 * sequence may hold some); afterwards len = ndraft = 0 for every sequence and the bf16 read copy,
 * if any, is refreshed. The checkpoint is read and written once for the whole prompt. Requires no
 * pending verify (RSSM_E_STATE). Every layer type runs the prompt in 16-token chunks on the
 * matrix cores; a Kimi Delta Attention chunk in which some key channel's gate product falls below
 * 2^-64 is applied token by token instead. */
rssm_status rssm_prefill(rssm_ctx *ctx, const rssm_inputs *in, float *y, void *stream);

/* Speculative decoding stores the drafts' inputs and evaluates outputs only (ia.goatify.app
 * article, paragraph "El retroceso usa un puntero del búfer").
 * Speculative verify of K = in->ntok drafts (1 <= K <= max_draft), every layer type (Mamba-2
 * drafts: x, B, C, dt; Gated DeltaNet and Kimi Delta Attention drafts: q, k, v, beta, alpha, each
 * with a leading K axis):
 * sequences whose drafts would not fit (len + K > W) first fold their committed entries; the
 * drafts are then appended as entries len .. len+K-1 (ndraft = K) and y [K,B,H,dim_v] gets every
 * draft's output, draft k seeing the committed entries and drafts 0..k. S0 is streamed once for
 * all K outputs. Gated DeltaNet takes at most 16 drafts per call (RSSM_E_ARG beyond). With B / C
 * shared by groups of heads (G < H), sequences whose drafts do not fit are folded by a
 * consolidation launch queued before the verify launch. Requires no pending verify; afterwards
 * exactly one of commit / rollback must follow. */
rssm_status rssm_verify(rssm_ctx *ctx, const rssm_inputs *in, float *y, void *stream);

/* The accepted prefix is confirmed by moving a pointer to the last accepted token, with no state
 * copy per draft (ia.goatify.app article, paragraph "El retroceso usa un puntero del búfer";
 * fagnersouza.tech post, section "O que muda para quem desenvolve").
 * Accept accepted[b] ([B] int32, device) drafts per sequence: len += accepted[b] when
 * 0 <= accepted[b] <= ndraft[b], else RSSM_DEV_COMMIT_RANGE and len unchanged; ndraft = 0.
 * A pointer move only: no state or ring data is copied. Requires a pending verify. */
rssm_status rssm_verify_commit(rssm_ctx *ctx, const int32_t *accepted, void *stream);

/* Rollback by the same pointer (ia.goatify.app article, paragraph "El retroceso usa un puntero
 * del búfer").
 * Roll back to new_len[b] ([B] int32, device) committed entries: len = new_len[b] when
 * 0 <= new_len[b] <= len[b], else RSSM_DEV_ROLLBACK_RANGE and len unchanged; pending drafts are
 * discarded (ndraft = 0). The checkpoint is never rolled back. */
rssm_status rssm_rollback(rssm_ctx *ctx, const int32_t *new_len, void *stream);

/* Conventional decoding reads and rewrites the whole state matrix on every token
 * (fagnersouza.tech post "ReplaySSM: o ganho aparece na carga concorrente...", lede).
 * Conventional read-modify-write decode, the comparator: for each token of `in` in order,
 * state <- update(state) and y[t] <- output, per the recurrences above. state [B,H,dim_v,dim_k]
 * is updated in place when snapshots is NULL. Otherwise state is only read and the state after
 * token t is written to snapshots [ntok,B,H,dim_v,dim_k] (per-draft snapshots, the conventional
 * way to keep rollback possible). A and D [H] are used for Mamba-2 only. y [ntok,B,H,dim_v]. */
rssm_status rssm_step_baseline(const rssm_config *cfg, float *state, const rssm_inputs *in,
                               const float *A, const float *D, float *y, float *snapshots,
                               void *stream);

/* rssm_step_baseline over per-sequence state tiles: seq_state [B] (a DEVICE array of device
 * pointers, each 16-byte aligned) gives sequence b's [H,dim_v,dim_k] state, which the launch
 * updates in place when snapshots is NULL (snapshots, if given, stay one contiguous
 * [ntok,B,H,dim_v,dim_k] array). This is how a serving engine's conventional kernel reaches
 * states kept in per-sequence slots of a cache pool. The pointers are read on the device; they
 * must not alias each other. */
rssm_status rssm_step_baseline_seqs(const rssm_config *cfg, float *const *seq_state,
                                    const rssm_inputs *in, const float *A, const float *D,
                                    float *y, float *snapshots, void *stream);

/* Conventional speculative round, the comparator for rssm_verify + rssm_verify_commit (both layer
 * types; A and D are required for Mamba-2 and ignored for Gated DeltaNet).
 * Done conventionally, a rollback needs a copy of the state after every step (news.hamidun.com
 * item "NVIDIA présente ReplaySSM...", section "D'où vient le problème de l'état"); this keeps
 * one snapshot per draft and commits by pointer. `pool` holds 2K+1 state slots
 * [2K+1][B,H,dim_v,dim_k] (K = in->ntok); slot_of[b] ([B] int32, device, values 0..2K) names the
 * slot with sequence b's committed state. Each sequence runs the K drafts from that state and
 * writes the state after draft k to slot o_b + k, o_b = K if slot_of[b] < K else 0 (the half
 * that does not hold its committed state), and y [K,B,H,dim_v] receives every draft's output.
 * Slot values outside 0..2K are undefined behaviour (the caller owns slot_of). */
rssm_status rssm_step_baseline_spec(const rssm_config *cfg, float *pool, const int32_t *slot_of,
                                    const rssm_inputs *in, const float *A, const float *D,
                                    float *y, void *stream);

/* Commit of the conventional comparator: for every b with 1 <= accepted[b] <= ndraft, point
 * slot_of[b] at the snapshot after accepted[b] drafts (o_b + accepted[b] - 1, o_b as above);
 * 0 keeps the committed state. No state is copied. accepted [B] int32, device. */
rssm_status rssm_baseline_commit(const rssm_config *cfg, int32_t *slot_of, const int32_t *accepted,
                                 int32_t ndraft, void *stream);

/* Per-sequence state snapshots for prefix caching and continuous batching (news.hamidun.com item
 * "NVIDIA présente ReplaySSM...", sections "D'où vient le problème de l'état" and "Ce que les
 * ingénieurs d'inférence doivent vérifier"). A sequence's state is its checkpoint (and bf16 read
 * copy), its ring and its head / len / ndraft; copies of it need no recomputation. All three calls
 * require no pending verify (RSSM_E_STATE); 0 <= n <= min(batch, 65535) (RSSM_E_ARG); index
 * arrays are [n] int32 in device memory, and an index outside [0, batch) sets
 * RSSM_DEV_INDEX_RANGE and skips that pair. */

/* Bytes of one packed sequence slot (16-byte header with head, len, ndraft, then the state
 * arrays, each padded to 16 bytes); the layout is only meaningful to a context with the same
 * configuration. Host only. */
rssm_status rssm_seq_state_bytes(const rssm_config *cfg, size_t *bytes);

/* Make sequence dst[i] a copy of sequence src[i] (state and bookkeeping), i < n. The dst indices
 * must be distinct and none may be a src of another pair (otherwise the result is undefined). */
rssm_status rssm_fork(rssm_ctx *ctx, const int32_t *src, const int32_t *dst, int32_t n, void *stream);

/* Write the state of sequence seq[i] into packed slot i of buf (device, 16-byte aligned,
 * n * rssm_seq_state_bytes bytes, caller-owned). The context is not changed. */
rssm_status rssm_export(rssm_ctx *ctx, const int32_t *seq, int32_t n, void *buf, void *stream);

/* Replace the state of sequence seq[i] by packed slot i of buf (as written by rssm_export of a
 * context with the same configuration). seq indices must be distinct. A slot whose header an
 * export could not have written (head outside [0, W), len outside [0, W], ndraft != 0) is not
 * imported and sets RSSM_DEV_IMPORT_HEADER. */
rssm_status rssm_import(rssm_ctx *ctx, const int32_t *seq, int32_t n, const void *buf, void *stream);

/* The state a sequence represents is its checkpoint with its buffered entries applied
 * (ia.goatify.app article, paragraph "ReplaySSM cambia qué se almacena").
 * Write the current state of every sequence (S0 with its committed entries folded in) to
 * state_out [B,H,dim_v,dim_k] without changing the context. */
rssm_status rssm_materialize(rssm_ctx *ctx, float *state_out, void *stream);

/* The buffer pointers of every sequence (ia.goatify.app article, paragraph "El retroceso usa un
 * puntero del búfer").
 * Copy head, len, ndraft ([B] int32 each, HOST, any may be NULL) and the device error word
 * (HOST, may be NULL) to the host; synchronises `stream`. When dev_err is given, the error bits
 * it returns are cleared on the device; with dev_err NULL the word is left as it is. */
rssm_status rssm_read_bookkeeping(rssm_ctx *ctx, int32_t *head, int32_t *len, int32_t *ndraft,
                                  uint32_t *dev_err, void *stream);

/* Static description of a status code. */
const char *rssm_status_str(rssm_status s);

#ifdef __cplusplus
}
#endif
#endif /* RSSM_H */
