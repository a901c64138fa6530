// Block-mask builder: classify every q_block x kv_block tile by evaluating
// mask_mod on each of its cells, then emit ordered partial and full lists.
//
// What is computed follows the 2kiu "PyTorch Flex Attention complete guide"
// (section 3.1: a tile is skipped only when every element is masked;
// section 4.1: create_block_mask with full tiles kept in their own lists) and
// the charlestar blog "FlexAttention score_mod / BlockMask" (BlockMask
// section: empty / full / partial tiles).  Unlike the eager path the blog's
// cache section describes, no element-level dense mask is materialised: each
// wave counts visible cells of one tile in registers.
//
// Layout conventions: cells beyond L or S are not visible; each index row
// lists its tiles ascending, then the remaining tile indices ascending.
#include "internal.hpp"

namespace flexmi {

namespace {

constexpr int kBuildThreads = 512;
constexpr int kBuildWaves = kBuildThreads / 64;

enum : uint8_t { TILE_EMPTY = 0, TILE_PARTIAL = 1, TILE_FULL = 2 };

__global__ __launch_bounds__(kBuildThreads) void blockmask_build_kernel(BuildArgs a) {
    extern __shared__ uint8_t tile_class[];  // [nKB]
    const int qb = blockIdx.x;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row0 = qb * a.q_block;
    const int cells = a.q_block * a.kv_block;

    // Phase 1: one wave per tile; lanes sweep the tile row by row.
    for (int kb = wave; kb < a.nKB; kb += kBuildWaves) {
        const int col0 = kb * a.kv_block;
        int count = 0;
        for (int i = 0; i < a.q_block; ++i) {
            const int row = row0 + i;
            const bool row_in = row < a.L;
            const int p = row + a.mask.q_offset;
            for (int j0 = 0; j0 < a.kv_block; j0 += 64) {
                const int jj = j0 + lane;
                const int col = col0 + jj;
                const bool vis = row_in && jj < a.kv_block && col < a.S && mask_visible(a.mask, p, col);
                count += __popcll(__ballot(vis));
            }
        }
        if (lane == 0)
            tile_class[kb] = count == 0 ? TILE_EMPTY : (count == cells ? TILE_FULL : TILE_PARTIAL);
    }
    __syncthreads();

    // Phase 2: wave 0 writes the partial list, wave 1 the full list.
    if (wave > 1) return;
    const uint8_t want = wave == 0 ? TILE_PARTIAL : TILE_FULL;
    const int64_t row_id = ((int64_t)b * a.Hm + h) * a.nQB + qb;
    int* idx = (wave == 0 ? a.kv_idx : a.full_idx) + row_id * a.nKB;
    int* num = (wave == 0 ? a.kv_num : a.full_num) + row_id;

    int total = 0;
    for (int c0 = 0; c0 < a.nKB; c0 += 64) {
        const int kb = c0 + lane;
        total += __popcll(__ballot(kb < a.nKB && tile_class[kb] == want));
    }
    int hits = 0;    // listed tiles before this chunk
    int misses = 0;  // other tiles before this chunk
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int c0 = 0; c0 < a.nKB; c0 += 64) {
        const int kb = c0 + lane;
        const bool in = kb < a.nKB;
        const bool hit = in && tile_class[kb] == want;
        const uint64_t hit_mask = __ballot(hit);
        const uint64_t miss_mask = __ballot(in && !hit);
        if (hit) idx[hits + __popcll(hit_mask & below)] = kb;
        else if (in) idx[total + misses + __popcll(miss_mask & below)] = kb;
        hits += __popcll(hit_mask);
        misses += __popcll(miss_mask);
    }
    if (lane == 0) *num = total;
}

}  // namespace

hipError_t launch_blockmask_build(const BuildArgs& a, hipStream_t stream) {
    dim3 grid(a.nQB, a.Hm, a.Bm);
    hipLaunchKernelGGL(blockmask_build_kernel, grid, dim3(kBuildThreads), (size_t)a.nKB, stream, a);
    return hipGetLastError();
}

}  // namespace flexmi
