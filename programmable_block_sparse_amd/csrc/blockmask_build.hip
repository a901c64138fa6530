// Block-mask builder: classify every q_block x kv_block tile by evaluating
// mask_mod on each of its cells, then emit ordered partial and full lists.
//
// What is computed follows the 2kiu "PyTorch Flex Attention complete guide"
// (section 3.1: a tile is skipped only when every element is masked;
// section 4.1: create_block_mask with full tiles kept in their own lists) and
// the charlestar blog "FlexAttention score_mod / BlockMask" (BlockMask
// section: empty / full / partial tiles).  Unlike the eager path the blog's
// cache section describes, no element-level dense mask is materialised.
//
// Two launches on the caller's stream:
//   classify  one wave per tile; each lane owns a key column and the wave
//             walks the tile's rows, so one v_cmp + ballot evaluates 64 cells
//             and the visible-cell count accumulates in scalar registers.  The
//             tile class (0 empty, 1 partial, 2 full) is parked in the tile's
//             own kv_indices slot.
//   compact   one workgroup per Q-block row reads the row's classes into LDS
//             and rewrites kv_indices / full_kv_indices as ordered lists.
//
// Layout conventions: cells beyond L or S are not visible; each index row
// lists its tiles ascending, then the remaining tile indices ascending.
#include "internal.hpp"

namespace flexmi {

namespace {

constexpr int kClassifyWaves = 8;
constexpr int kCompactThreads = 256;

enum : int { TILE_EMPTY = 0, TILE_PARTIAL = 1, TILE_FULL = 2 };

// Ballot of the visible cells of one query position p over this lane's key
// column (branch-free within the row; col_ok folds the tile and S bounds).
template <int KIND>
__device__ __forceinline__ uint64_t row_ballot(const MaskArgs& m, int p, int col, bool col_ok, int doc_p,
                                               int doc_col) {
    bool v;
    if constexpr (KIND == MASK_NOOP) {
        v = col_ok;
    } else if constexpr (KIND == MASK_CAUSAL) {
        v = col_ok & (col <= p);
    } else if constexpr (KIND == MASK_CAUSAL_WINDOW_SINKS) {
        v = col_ok & (col <= p) & ((p - col < m.window) | (col < m.sinks));
    } else {
        v = col_ok & (col <= p) & (doc_p == doc_col);
    }
    return __ballot(v);
}

template <int KIND>
__global__ __launch_bounds__(kClassifyWaves * 64) void blockmask_classify(BuildArgs a) {
    const int lane = threadIdx.x & 63;
    const int kb = blockIdx.x * kClassifyWaves + (threadIdx.x >> 6);
    if (kb >= a.nKB) return;
    const int qb = blockIdx.y;
    const int bh = blockIdx.z;
    const int row0 = qb * a.q_block;
    const int rows = min(a.q_block, a.L - row0);
    const int64_t row_id = (int64_t)bh * a.nQB + qb;
    int64_t count = 0;
    for (int j0 = 0; j0 < a.kv_block; j0 += 64) {
        const int jj = j0 + lane;
        const int col = kb * a.kv_block + jj;
        const bool col_ok = (jj < a.kv_block) & (col < a.S);
        int doc_col = -1;
        if constexpr (KIND == MASK_DOC_CAUSAL)
            doc_col = (col_ok && col < a.mask.doc_len) ? __ldg(a.mask.doc_id + col) : -1;
        for (int i = 0; i < rows; ++i) {
            const int p = row0 + i + a.mask.q_offset;
            int doc_p = -2;
            if constexpr (KIND == MASK_DOC_CAUSAL)
                doc_p = (p >= 0 && p < a.mask.doc_len) ? __ldg(a.mask.doc_id + p) : -2;
            count += __popcll(row_ballot<KIND>(a.mask, p, col, col_ok, doc_p, doc_col));
        }
    }
    if (lane == 0) {
        const int64_t cells = (int64_t)a.q_block * a.kv_block;
        a.kv_idx[row_id * a.nKB + kb] = count == 0 ? TILE_EMPTY : (count == cells ? TILE_FULL : TILE_PARTIAL);
    }
}

__global__ __launch_bounds__(kCompactThreads) void blockmask_compact(BuildArgs a) {
    extern __shared__ uint8_t tile_class[];  // [nKB]
    const int qb = blockIdx.x;
    const int bh = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t row_id = (int64_t)bh * a.nQB + qb;
    for (int kb = threadIdx.x; kb < a.nKB; kb += kCompactThreads)
        tile_class[kb] = (uint8_t)a.kv_idx[row_id * a.nKB + kb];
    __syncthreads();
    if (wave > 1) return;

    // wave 0 writes the partial list, wave 1 the full list
    const uint8_t want = wave == 0 ? TILE_PARTIAL : TILE_FULL;
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

template <int KIND>
hipError_t launch_classify(const BuildArgs& a, hipStream_t stream) {
    dim3 grid((a.nKB + kClassifyWaves - 1) / kClassifyWaves, a.nQB, a.Bm * a.Hm);
    hipLaunchKernelGGL(blockmask_classify<KIND>, grid, dim3(kClassifyWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_blockmask_build(const BuildArgs& a, hipStream_t stream) {
    hipError_t e;
    switch (a.mask.kind) {
    case MASK_NOOP: e = launch_classify<MASK_NOOP>(a, stream); break;
    case MASK_CAUSAL: e = launch_classify<MASK_CAUSAL>(a, stream); break;
    case MASK_CAUSAL_WINDOW_SINKS: e = launch_classify<MASK_CAUSAL_WINDOW_SINKS>(a, stream); break;
    default: e = launch_classify<MASK_DOC_CAUSAL>(a, stream); break;
    }
    if (e != hipSuccess) return e;
    dim3 grid(a.nQB, a.Bm * a.Hm);
    hipLaunchKernelGGL(blockmask_compact, grid, dim3(kCompactThreads), (size_t)a.nKB, stream, a);
    return hipGetLastError();
}

}  // namespace flexmi
