// tile_order.h -- which (b, h) tile a workgroup takes (gfx950).
//
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup w runs on XCD w % 8), each with
// its own L2. The orders below keep an XCD's workgroups on neighbouring tiles; the tiles of a last
// incomplete round keep their own index, so every order is a bijection of [0, n):
//   kIdentity:   tile w;
//   kRuns:       XCD x takes runs of `run` consecutive tiles, the XCDs interleaved run by run;
//   kContiguous: XCD x takes one range of n / 8 consecutive tiles.
// Runs cover kRunBytes of fp32 checkpoint (64 tiles of 64 x 128, 32 tiles of 128 x 128): the
// length measured fastest for the launches that only read the checkpoint, for both layer types.
#pragma once

namespace rssm {

enum TileOrder { kIdentity = 0, kRuns = 1, kContiguous = 2 };
constexpr int kRunBytes = 2 << 20;

// tiles per run for a tile of `tile_floats` fp32 values
__device__ __forceinline__ int run_tiles(int tile_floats)
{
    const int r = kRunBytes / (4 * tile_floats);
    return r > 0 ? r : 1;
}

__device__ __forceinline__ int tile_of(int w, int n, TileOrder order, int run)
{
    if (order == kContiguous) {
        const int per = n / 8;
        return w < 8 * per ? (w % 8) * per + w / 8 : w;
    }
    if (order == kRuns) {
        const int full = n / (8 * run) * (8 * run), j = w / 8;
        return w < full ? ((j / run) * 8 + w % 8) * run + j % run : w;
    }
    return w;
}

}  // namespace rssm
