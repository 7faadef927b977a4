// internal.h -- kernel argument blocks and launcher entry points of librssm (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rssm {

constexpr int kMaxWindow = 32;   // largest ring length W (W + 1 entries fit one wave's lanes)
constexpr int kGdnMaxDraft = 16; // drafts of one Gated DeltaNet verify (one 16-row matrix-core block)

// Bookkeeping is double-buffered: every launch that changes it reads bk_in and writes bk_out
// (each [3][B] int32: head, len, ndraft). All head-workgroups of a sequence read bk_in while one
// of them writes bk_out, so no launch both reads and writes the same word.
struct Bk {
    const int32_t *in;
    int32_t *out;
};

struct M2Ring {
    float *x;     // [B,H,W,P]
    float *B;     // [B,G,W,N]
    float *C;     // [B,G,W,N] or nullptr (not stored)
    float *dt;    // [B,H,W]
};

struct M2Dims {
    int B, H, G, P, N, W;
};

// Mamba-2 decode / verify (ntok tokens, token-major inputs).
struct M2StepArgs {
    M2Dims d;
    Bk bk;
    float *S0;          // [B,H,P,N]
    uint16_t *S0b;      // bf16 copy or nullptr
    M2Ring ring;
    const float *A, *D; // [H]
    const float *x, *Bm, *C, *dt;
    float *y;
    int ntok;
    int uhead, ulen;    // ring position shared by every sequence (uniform decode mode only)
};

// Per-sequence state copies (fork, export to / import from a packed buffer).
enum SeqMode { kSeqFork = 0, kSeqExport = 1, kSeqImport = 2 };
constexpr int kSeqMaxSeg = 6;              // checkpoint, read copy and up to four ring arrays
constexpr size_t kSeqHeader = 16;          // packed slot: head, len, ndraft, 0, then the segments
constexpr uint32_t kDevIndexRange = 8u;    // device error bit: a sequence index out of range
constexpr uint32_t kDevImportHeader = 16u; // device error bit: an imported slot header out of range

struct SeqCopyArgs {
    int mode, n, B, W, nseg;
    const int32_t *src, *dst;              // fork: src[n], dst[n]; export: src = sequences; import: dst
    char *base[kSeqMaxSeg];                // array bases in the workspace
    uint64_t seg_bytes[kSeqMaxSeg];        // bytes of one sequence in each array
    uint64_t pack_off[kSeqMaxSeg];         // offsets of the segments in a packed slot (after the header)
    int unit_log2[kSeqMaxSeg];             // 4 (16-byte units) or 2 (4-byte units)
    uint64_t unit_prefix[kSeqMaxSeg + 1];  // cumulative units over the segments
    char *buf;                             // packed slots (export / import)
    uint64_t pack_bytes;                   // bytes of one packed slot
    uint32_t *err;
};

// Mamba-2 prefill of T prompt tokens (token-major inputs) into the checkpoint.
struct M2PrefillArgs {
    M2Dims d;
    Bk bk;
    float *S0;          // [B,H,P,N]
    uint16_t *S0b;      // bf16 copy or nullptr
    const float *A, *D; // [H]
    const float *x, *Bm, *C, *dt;
    float *y;           // [T,B,H,P]
    int T;
};

// Mamba-2 consolidation (write S0) or materialisation (write out).
struct M2FoldArgs {
    M2Dims d;
    Bk bk;
    float *S0;
    uint16_t *S0b;
    M2Ring ring;
    const float *A;
    int min_len;
    float *out;         // materialise target, nullptr when consolidating
};

struct M2RmwArgs {
    M2Dims d;
    float *state;       // [B,H,P,N]; with slot_of: the slot pool [2 ntok + 1][B,H,P,N]
    float *snap;        // nullptr = in place (ignored with slot_of)
    const float *A, *D;
    const float *x, *Bm, *C, *dt;
    float *y;
    int ntok;
    const int32_t *slot_of;   // [B] committed slot per sequence, or nullptr
    float *const *seq;        // [B] per-sequence state tiles [H,P,N] (instead of state), or nullptr
};

// Rings of the delta-rule layers (Gated DeltaNet; Kimi Delta Attention with a gate per key
// channel, alpha [B,H,W,dk]). The step arguments of both use the structs below, with alpha
// [ntok,B,H] for Gated DeltaNet and [ntok,B,H,dk] for Kimi Delta Attention.
struct GdnRing {
    float *k;      // [B,H,W,dk]
    float *v;      // [B,H,W,dv]
    float *beta;   // [B,H,W]
    float *alpha;  // [B,H,W] (Gated DeltaNet) or [B,H,W,dk] (Kimi Delta Attention)
};

struct GdnDims {
    int B, H, DV, DK, W;
};

struct GdnStepArgs {
    GdnDims d;
    Bk bk;
    float *S0;
    GdnRing ring;
    const float *q, *k, *v, *beta, *alpha;
    float *o;
    int uhead, ulen;    // ring position shared by every sequence (mode 0 only)
    int ntok;           // verify: drafts per sequence
};

struct GdnFoldArgs {
    GdnDims d;
    Bk bk;
    float *S0;
    GdnRing ring;
    int min_len;
    float *out;
};

// Gated DeltaNet prefill of T prompt tokens (token-major inputs) into the checkpoint.
struct GdnPrefillArgs {
    GdnDims d;
    Bk bk;
    float *S0;          // [B,H,dv,dk]
    const float *q, *k, *v, *beta, *alpha;
    float *o;           // [T,B,H,dv]
    int T;
};

struct GdnRmwArgs {
    GdnDims d;
    float *state;       // [B,H,dv,dk]; with slot_of: the slot pool [2 ntok + 1][B,H,dv,dk]
    float *snap;        // nullptr = in place (ignored with slot_of)
    const float *q, *k, *v, *beta, *alpha;
    float *o;
    int ntok;
    const int32_t *slot_of;   // [B] committed slot per sequence, or nullptr
    float *const *seq;        // [B] per-sequence state tiles [H,dv,dk] (instead of state), or nullptr
};

// ---- launchers (return hipSuccess or the launch error) ----
bool m2_supported(int P, int N);
// Decode kernel choice. 0: every sequence is at ring position (a.uhead, a.ulen) and none fills
// its ring; 1: no sequence fills its ring; 2: any sequence may fold; 3: every sequence is at
// (a.uhead, a.ulen) and fills its ring (Mamba-2 only).
hipError_t m2_decode(const M2StepArgs &a, bool bf16, int mode, hipStream_t s);
hipError_t m2_verify(const M2StepArgs &a, bool bf16, hipStream_t s);
size_t m2_lds_bytes(int P, int N, int W);   // dynamic LDS of the largest Mamba-2 kernel
hipError_t m2_prefill(const M2PrefillArgs &a, bool bf16, hipStream_t s);
hipError_t seq_copy(const SeqCopyArgs &a, Bk bk, hipStream_t s);
hipError_t m2_fold(const M2FoldArgs &a, bool bf16, hipStream_t s);
hipError_t m2_rmw(const M2RmwArgs &a, hipStream_t s);

bool gdn_supported(int DV, int DK);
size_t gdn_lds_bytes(int DV, int DK, int W);
hipError_t gdn_decode(const GdnStepArgs &a, int mode, hipStream_t s);   // mode as m2_decode
hipError_t gdn_fold(const GdnFoldArgs &a, hipStream_t s);
hipError_t gdn_rmw(const GdnRmwArgs &a, hipStream_t s);
hipError_t gdn_verify(const GdnStepArgs &a, hipStream_t s);
hipError_t gdn_prefill(const GdnPrefillArgs &a, hipStream_t s);

bool kda_supported(int DV, int DK);
size_t kda_lds_bytes(int DV, int DK, int W, int K);   // dynamic LDS of the largest KDA kernel
hipError_t kda_decode(const GdnStepArgs &a, int mode, hipStream_t s);   // mode as m2_decode
hipError_t kda_fold(const GdnFoldArgs &a, hipStream_t s);
hipError_t kda_rmw(const GdnRmwArgs &a, hipStream_t s);
hipError_t kda_verify(const GdnStepArgs &a, hipStream_t s);
hipError_t kda_prefill(const GdnPrefillArgs &a, hipStream_t s);

// ckpt_dv > 0: the tiles are Gated DeltaNet checkpoints with ckpt_dv rows, stored in the layout
// of gdn_layout.h; 0: row-major (Mamba-2).
hipError_t init_checkpoint(float *S0, uint16_t *S0b, const float *state, const int32_t *mask,
                           Bk bk, uint32_t *err, int B, int H, long tile_elems, int ckpt_dv,
                           hipStream_t s);
hipError_t bk_commit(Bk bk, const int32_t *accepted, uint32_t *err, int B, hipStream_t s);
hipError_t bk_rollback(Bk bk, const int32_t *new_len, uint32_t *err, int B, hipStream_t s);
hipError_t slot_commit(int32_t *slot_of, const int32_t *accepted, int B, int K, hipStream_t s);
hipError_t clear_word(uint32_t *w, hipStream_t s);

}  // namespace rssm
