// Q-side lists of a block mask: for every KV block (a column of the tile
// grid), the Q blocks whose tile with it is partial, then those whose tile is
// full.  The 2kiu "PyTorch Flex Attention complete guide", section 3.3, says the
// Q-side block information is derived from the KV-side lists by transposing
// them; the backward pass walks a column of tiles with it.
//
// One wave per column: lane l takes Q-block row 64*i + l of chunk i, looks the
// column's KV block up in that row's ascending lists by binary search, and
// the wave places its rows with a ballot and a prefix count, so the output
// is a pure function of the input lists (no atomics, no ordering races) and
// the writes of a chunk are contiguous.  A first sweep counts the listed
// rows, a second writes them and then the completions (every other Q-block
// index, ascending), which keeps each index row a permutation of 0..nQB-1
// like the KV-side lists.
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

// Lanes of this wave below the calling lane whose bit is set in `bits`.
__device__ __forceinline__ int prefix_count(uint64_t bits) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
}

__global__ __launch_bounds__(kThreads) void blockmask_transpose(TransposeArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t col = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int64_t n_cols = (int64_t)a.Bm * a.Hm * a.nKB;
    if (col >= n_cols) return;   // wave-uniform
    const int64_t bh = col / a.nKB;
    const int kb = (int)(col % a.nKB);
    const int64_t row0 = bh * a.nQB;
    int* __restrict__ qi = a.q_idx + col * a.nQB;
    int* __restrict__ fi = a.fq_idx + col * a.nQB;
    // sweep 1: how many rows list this block as partial / full
    int n_part = 0, n_full = 0;
    for (int base = 0; base < a.nQB; base += 64) {
        const int qb = base + lane;
        const int c = qb < a.nQB ? tile_class(a, row0 + qb, kb) : 0;
        n_part += __popcll(__ballot(c == 1));
        n_full += __popcll(__ballot(c == 2));
    }
    // sweep 2: listed rows first, then the rest, both ascending
    int lp = 0, lf = 0, rp = n_part, rf = n_full;
    for (int base = 0; base < a.nQB; base += 64) {
        const int qb = base + lane;
        const bool in = qb < a.nQB;
        const int c = in ? tile_class(a, row0 + qb, kb) : 0;
        const uint64_t is_p = __ballot(in && c == 1), not_p = __ballot(in && c != 1);
        const uint64_t is_f = __ballot(in && c == 2), not_f = __ballot(in && c != 2);
        if (in) {
            if (c == 1) qi[lp + prefix_count(is_p)] = qb;
            else qi[rp + prefix_count(not_p)] = qb;
            if (c == 2) fi[lf + prefix_count(is_f)] = qb;
            else fi[rf + prefix_count(not_f)] = qb;
        }
        lp += __popcll(is_p);
        rp += __popcll(not_p);
        lf += __popcll(is_f);
        rf += __popcll(not_f);
    }
    if (lane == 0) {
        a.q_num[col] = n_part;
        a.fq_num[col] = n_full;
    }
}

}  // namespace

hipError_t launch_blockmask_transpose(const TransposeArgs& a, hipStream_t stream) {
    const int64_t n_cols = (int64_t)a.Bm * a.Hm * a.nKB;
    const int64_t blocks = (n_cols + kThreads / 64 - 1) / (kThreads / 64);
    hipLaunchKernelGGL(blockmask_transpose, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace flexmi
