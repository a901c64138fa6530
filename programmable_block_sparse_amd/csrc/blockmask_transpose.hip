// Q-side lists of a block mask: for every KV block (a column of the tile
// grid), the Q blocks whose tile with it is partial, then those whose tile is
// full.  The 2kiu "PyTorch Flex Attention complete guide", section 3.3, says the
// Q-side block information is derived from the KV-side lists by transposing
// them; the backward pass walks a column of tiles with it.
//
// One thread per column: it scans the Q-block rows in ascending order and
// looks its KV block up in each row's ascending lists by binary search, so the
// output is a pure function of the input lists (no atomics, no ordering
// races).  A first scan writes the listed rows, a second the completions
// (every other Q-block index, ascending), which keeps each index row a
// permutation of 0..nQB-1 like the KV-side lists.
#include "internal.hpp"

namespace flexmi {

namespace {

constexpr int kThreads = 256;

// True when the ascending list[0, n) holds x.
__device__ __forceinline__ bool sorted_contains(const int* __restrict__ list, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const int v = list[mid];
        if (v == x) return true;
        if (v < x) lo = mid + 1;
        else hi = mid;
    }
    return false;
}

// Tile class of (row, kb): 1 partial, 2 full, 0 empty.  Counts are clamped
// as the attention kernels clamp them; a block listed in both lists is
// partial.
__device__ __forceinline__ int tile_class(const TransposeArgs& a, int64_t row, int kb) {
    const int n_part = min(max(a.kv_num[row], 0), a.nKB);
    if (sorted_contains(a.kv_idx + row * a.nKB, n_part, kb)) return 1;
    const int n_full = min(max(a.full_num[row], 0), a.nKB - n_part);
    return sorted_contains(a.full_idx + row * a.nKB, n_full, kb) ? 2 : 0;
}

__global__ __launch_bounds__(kThreads) void blockmask_transpose(TransposeArgs a) {
    const int64_t col = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t n_cols = (int64_t)a.Bm * a.Hm * a.nKB;
    if (col >= n_cols) return;
    const int64_t bh = col / a.nKB;
    const int kb = (int)(col % a.nKB);
    const int64_t row0 = bh * a.nQB;
    int* __restrict__ qi = a.q_idx + col * a.nQB;
    int* __restrict__ fi = a.fq_idx + col * a.nQB;
    int n_part = 0, n_full = 0;
    for (int qb = 0; qb < a.nQB; ++qb) {
        const int c = tile_class(a, row0 + qb, kb);
        if (c == 1) qi[n_part++] = qb;
        else if (c == 2) fi[n_full++] = qb;
    }
    int pp = n_part, fp = n_full;
    for (int qb = 0; qb < a.nQB; ++qb) {
        const int c = tile_class(a, row0 + qb, kb);
        if (c != 1) qi[pp++] = qb;
        if (c != 2) fi[fp++] = qb;
    }
    a.q_num[col] = n_part;
    a.fq_num[col] = n_full;
}

}  // namespace

hipError_t launch_blockmask_transpose(const TransposeArgs& a, hipStream_t stream) {
    const int64_t n_cols = (int64_t)a.Bm * a.Hm * a.nKB;
    const int64_t blocks = (n_cols + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(blockmask_transpose, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace flexmi
