// seqstate.hip -- per-sequence state copies: fork one sequence's state onto another slot, export it
// to a packed buffer, import it back (gfx950).
//
// A sequence's replay state is its checkpoint (and bf16 read copy), its ring and its head / len /
// ndraft. Prefix caching and continuous batching need to snapshot, restore or duplicate exactly
// that (news.hamidun.com item "NVIDIA présente ReplaySSM...", sections "D'où vient le problème de
// l'état" and "Ce que les ingénieurs d'inférence doivent vérifier": snapshots of the SSM state for
// speculative decoding, prefix caching and continuous batching). With the checkpoint + ring form
// a snapshot is a copy of those arrays at a moment with no pending drafts; nothing is recomputed.
//
// Every array of the workspace holds a sequence's data contiguously (sequence-major layout), so a
// sequence is a list of segments (one per array) at offset b * bytes_per_sequence. The copy kernel
// walks the concatenation of the segments in 16-byte units where a segment allows it (size a
// multiple of 16) and 4-byte units otherwise, one pair of sequences per grid row.
#include "dev_common.h"
#include "internal.h"

namespace rssm {
namespace {

__device__ __forceinline__ bool in_range(int v, int B) { return v >= 0 && v < B; }

// each byte is read and written once: streaming (non-temporal) 16-byte accesses
__device__ __forceinline__ void copy16_nt(char *dst, const char *src)
{
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(src));
    __builtin_nontemporal_store(v, reinterpret_cast<v4u *>(dst));
}

// A packed slot's header may come from anywhere: it is accepted only as an export writes it
// (ring head in [0, W), committed length in [0, W], no pending drafts), so that every later kernel
// sees ring indices in range.
__device__ __forceinline__ bool header_ok(const SeqCopyArgs &a, int slot)
{
    const int32_t *h = reinterpret_cast<const int32_t *>(a.buf + (size_t)slot * a.pack_bytes);
    return h[0] >= 0 && h[0] < a.W && h[1] >= 0 && h[1] <= a.W && h[2] == 0;
}

// source and destination (sequence or buffer slot) of pair p; false when an index is out of range
// or an imported header is invalid (the pair is then skipped whole: state and bookkeeping)
__device__ __forceinline__ bool pair_of(const SeqCopyArgs &a, int p, int &s, int &d)
{
    if (a.mode == kSeqFork) {
        s = a.src[p];
        d = a.dst[p];
        return in_range(s, a.B) && in_range(d, a.B);
    }
    if (a.mode == kSeqExport) {
        s = a.src[p];
        d = p;
        return in_range(s, a.B);
    }
    s = p;
    d = a.dst[p];
    return in_range(d, a.B) && header_ok(a, p);
}

__global__ void __launch_bounds__(256) k_seq_copy(SeqCopyArgs a)
{
    const int p = blockIdx.y;
    int s, d;
    if (!pair_of(a, p, s, d)) return;        // reported by k_seq_bk
    const uint64_t total = a.unit_prefix[a.nseg];
    const bool from_buf = a.mode == kSeqImport, to_buf = a.mode == kSeqExport;
    for (uint64_t u = (uint64_t)blockIdx.x * 256 + threadIdx.x; u < total;
         u += (uint64_t)gridDim.x * 256) {
        int k = 0;
        while (u >= a.unit_prefix[k + 1]) ++k;
        const uint64_t off = (u - a.unit_prefix[k]) << a.unit_log2[k];
        const char *src = from_buf ? a.buf + (size_t)s * a.pack_bytes + kSeqHeader + a.pack_off[k] + off
                                   : a.base[k] + (size_t)s * a.seg_bytes[k] + off;
        char *dst = to_buf ? a.buf + (size_t)d * a.pack_bytes + kSeqHeader + a.pack_off[k] + off
                           : a.base[k] + (size_t)d * a.seg_bytes[k] + off;
        if (a.unit_log2[k] == 4)
            copy16_nt(dst, src);
        else
            *reinterpret_cast<uint32_t *>(dst) = *reinterpret_cast<const uint32_t *>(src);
    }
}

// Bookkeeping of the copies, one workgroup. Fork / import: the new bookkeeping is the old one
// (bk.in -> bk.out) with the destinations' head / len / ndraft replaced. Export: each buffer
// slot's header gets its sequence's head / len / ndraft (bk.out unused).
__global__ void __launch_bounds__(256) k_seq_bk(SeqCopyArgs a, Bk bk)
{
    const int B = a.B, t = threadIdx.x;
    if (a.mode != kSeqExport) {
        for (int i = t; i < 3 * B; i += 256) bk.out[i] = bk.in[i];
        __syncthreads();
    }
    for (int p = t; p < a.n; p += 256) {
        int s, d;
        if (!pair_of(a, p, s, d)) {
            const bool index_ok = a.mode == kSeqImport ? in_range(a.dst[p], B)
                                : a.mode == kSeqExport ? in_range(a.src[p], B)
                                : in_range(a.src[p], B) && in_range(a.dst[p], B);
            atomicOr(a.err, index_ok ? kDevImportHeader : kDevIndexRange);
            continue;
        }
        if (a.mode == kSeqFork) {
            bk.out[d] = bk.in[s];
            bk.out[B + d] = bk.in[B + s];
            bk.out[2 * B + d] = bk.in[2 * B + s];
        } else if (a.mode == kSeqExport) {
            int32_t *h = reinterpret_cast<int32_t *>(a.buf + (size_t)d * a.pack_bytes);
            h[0] = bk.in[s];
            h[1] = bk.in[B + s];
            h[2] = bk.in[2 * B + s];
            h[3] = 0;
        } else {
            const int32_t *h = reinterpret_cast<const int32_t *>(a.buf + (size_t)s * a.pack_bytes);
            bk.out[d] = h[0];
            bk.out[B + d] = h[1];
            bk.out[2 * B + d] = h[2];
        }
    }
}

}  // namespace

hipError_t seq_copy(const SeqCopyArgs &a, Bk bk, hipStream_t s)
{
    if (a.n > 0) {
        const uint64_t total = a.unit_prefix[a.nseg];
        uint64_t nblk = (total + 255) / 256;
        if (nblk > 512) nblk = 512;
        if (nblk < 1) nblk = 1;
        hipLaunchKernelGGL(k_seq_copy, dim3((unsigned)nblk, (unsigned)a.n), dim3(256), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_seq_bk, dim3(1), dim3(256), 0, s, a, bk);
    return hipGetLastError();
}

}  // namespace rssm
