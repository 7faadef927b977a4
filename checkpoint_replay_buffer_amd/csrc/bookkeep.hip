// bookkeep.hip -- checkpoint loading and the pointer-only commit / rollback of speculative drafts.
//
// Accepting a prefix of the drafts only moves the committed length: no state and no ring data is
// copied (ia.goatify.app article "NVIDIA y Princeton aceleran modelos híbridos...", paragraph
// "El retroceso usa un puntero del búfer"). Bookkeeping words are [3][B] int32 (head, len,
// ndraft), read from bk.in and written to bk.out.
#include "dev_common.h"
#include "internal.h"
#include "gdn_layout.h"

namespace rssm {
namespace {

constexpr uint32_t kCommitRange = 1u;
constexpr uint32_t kRollbackRange = 2u;

// One workgroup per (b, h) tile: copy the initial state of selected sequences into S0 (and its
// bf16 copy) and reset their bookkeeping. ckpt_dv > 0: S0 in the layout of gdn_layout.h (tiles
// of ckpt_dv rows).
__global__ void __launch_bounds__(256) k_init(float *S0, uint16_t *S0b, const float *state,
                                              const int32_t *mask, Bk bk, uint32_t *err, int B,
                                              int H, long tile_elems, int ckpt_dv)
{
    const int tile = blockIdx.x;
    const int b = tile / H, h = tile - b * H;
    const bool sel = mask == nullptr || mask[b] != 0;
    if (h == 0 && threadIdx.x == 0) {
        bk.out[b] = sel ? 0 : bk.in[b];
        bk.out[B + b] = sel ? 0 : bk.in[B + b];
        bk.out[2 * B + b] = sel ? 0 : bk.in[2 * B + b];
        if (mask == nullptr && tile == 0) *err = 0u;
    }
    if (!sel) return;
    const size_t base = (size_t)tile * tile_elems;
    for (long i = threadIdx.x; i < tile_elems / 4; i += blockDim.x) {
        const float4 v = ld4_nt(state + base + 4 * i);
        if (ckpt_dv > 0) {
            const long cols = tile_elems / ckpt_dv;
            const int row = (int)(4 * i / cols), col = (int)(4 * i - row * cols);
            st4(S0 + base + ckpt_offset(row, col, ckpt_dv), v);
        } else {
            st4(S0 + base + 4 * i, v);
        }
        if (S0b) {
            uint2 w;
            w.x = pack_bf16x2(v.x, v.y);
            w.y = pack_bf16x2(v.z, v.w);
            *reinterpret_cast<uint2 *>(S0b + base + 4 * i) = w;
        }
    }
}

__global__ void __launch_bounds__(256) k_commit(Bk bk, const int32_t *accepted, uint32_t *err, int B)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int len = bk.in[B + b], nd = bk.in[2 * B + b], acc = accepted[b];
    const bool ok = acc >= 0 && acc <= nd;
    bk.out[b] = bk.in[b];
    bk.out[B + b] = ok ? len + acc : len;
    bk.out[2 * B + b] = 0;
    if (!ok) atomicOr(err, kCommitRange);
}

__global__ void __launch_bounds__(256) k_rollback(Bk bk, const int32_t *new_len, uint32_t *err, int B)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int len = bk.in[B + b], nl = new_len[b];
    const bool ok = nl >= 0 && nl <= len;
    bk.out[b] = bk.in[b];
    bk.out[B + b] = ok ? nl : len;
    bk.out[2 * B + b] = 0;
    if (!ok) atomicOr(err, kRollbackRange);
}

// Conventional speculative comparator: point each sequence at the snapshot taken after its
// accepted drafts (slot (slot_of < K ? K : 0) + accepted - 1); nothing is copied.
__global__ void __launch_bounds__(256) k_slot_commit(int32_t *slot_of, const int32_t *accepted, int B, int K)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int acc = accepted[b], sl = slot_of[b];
    if (acc >= 1 && acc <= K) slot_of[b] = (sl < K ? K : 0) + acc - 1;
}

__global__ void k_clear(uint32_t *w) { *w = 0u; }

}  // namespace

hipError_t init_checkpoint(float *S0, uint16_t *S0b, const float *state, const int32_t *mask,
                           Bk bk, uint32_t *err, int B, int H, long tile_elems, int ckpt_dv,
                           hipStream_t s)
{
    hipLaunchKernelGGL(k_init, dim3(B * H), dim3(256), 0, s, S0, S0b, state, mask, bk, err, B, H,
                       tile_elems, ckpt_dv);
    return hipGetLastError();
}

hipError_t bk_commit(Bk bk, const int32_t *accepted, uint32_t *err, int B, hipStream_t s)
{
    hipLaunchKernelGGL(k_commit, dim3((B + 255) / 256), dim3(256), 0, s, bk, accepted, err, B);
    return hipGetLastError();
}

hipError_t bk_rollback(Bk bk, const int32_t *new_len, uint32_t *err, int B, hipStream_t s)
{
    hipLaunchKernelGGL(k_rollback, dim3((B + 255) / 256), dim3(256), 0, s, bk, new_len, err, B);
    return hipGetLastError();
}

hipError_t slot_commit(int32_t *slot_of, const int32_t *accepted, int B, int K, hipStream_t s)
{
    hipLaunchKernelGGL(k_slot_commit, dim3((B + 255) / 256), dim3(256), 0, s, slot_of, accepted, B, K);
    return hipGetLastError();
}

hipError_t clear_word(uint32_t *w, hipStream_t s)
{
    hipLaunchKernelGGL(k_clear, dim3(1), dim3(1), 0, s, w);
    return hipGetLastError();
}

}  // namespace rssm
