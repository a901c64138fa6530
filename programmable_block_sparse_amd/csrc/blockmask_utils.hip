// BlockMask utilities of the 2kiu "PyTorch Flex Attention complete guide",
// section 3.3, on device arrays: the dense block view (to_dense), the pooled
// tile-class grid that to_string draws, sparsity, Q-block-row slicing
// (__getitem__) and cropping to new lengths (_adjust).
//
// Each kernel rebuilds a row's tile classes from its two ordered lists in an
// LDS bitmap (one bit per KV block, for the partial and for the full list),
// so a block listed twice counts once, and works from there with coalesced
// writes.  Counts are clamped as the attention kernels clamp them; a block in
// both lists is partial.
#include "internal.hpp"

namespace flexmi {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxWords = 65536 / 32;   // bitmap words for up to 65536 KV blocks

struct RowBits {
    uint32_t* part;   // LDS, ceil(nKB / 32) words
    uint32_t* full;
};

// Fills the two bitmaps of one row (entries below `ncols` only) and returns
// after a barrier.  All threads of the workgroup take part.
__device__ __forceinline__ void load_row_bits(const RowBits& rb, const UtilArgs& a, int64_t row, int ncols) {
    const int words = (ncols + 31) / 32;
    for (int w = threadIdx.x; w < words; w += kThreads) {
        rb.part[w] = 0u;
        rb.full[w] = 0u;
    }
    __syncthreads();
    const int n_part = min(max(a.kv_num[row], 0), a.nKB);
    const int n_full = min(max(a.full_num[row], 0), a.nKB - n_part);
    const int* pi = a.kv_idx + row * a.nKB;
    const int* fi = a.full_idx + row * a.nKB;
    for (int t = threadIdx.x; t < n_part; t += kThreads) {
        const int kb = pi[t];
        if (kb >= 0 && kb < ncols) atomicOr(rb.part + (kb >> 5), 1u << (kb & 31));
    }
    for (int t = threadIdx.x; t < n_full; t += kThreads) {
        const int kb = fi[t];
        if (kb >= 0 && kb < ncols) atomicOr(rb.full + (kb >> 5), 1u << (kb & 31));
    }
    __syncthreads();
}

// 1 partial, 2 full, 0 empty.
__device__ __forceinline__ int bit_class(const RowBits& rb, int kb) {
    const uint32_t m = 1u << (kb & 31);
    if (rb.part[kb >> 5] & m) return 1;
    return (rb.full[kb >> 5] & m) ? 2 : 0;
}

__global__ __launch_bounds__(kThreads) void blockmask_to_dense(UtilArgs a, int32_t* dense) {
    __shared__ uint32_t bits[2 * kMaxWords];
    const RowBits rb{bits, bits + kMaxWords};
    const int64_t row = blockIdx.x;
    load_row_bits(rb, a, row, a.nKB);
    for (int kb = threadIdx.x; kb < a.nKB; kb += kThreads) dense[row * a.nKB + kb] = bit_class(rb, kb) != 0;
}

// One workgroup per (batch, head, grid row): ORs, per window column, whether
// some tile of the window is not full (bit 0) and whether some is not empty
// (bit 1); sixteen windows per word.
__global__ __launch_bounds__(kThreads) void blockmask_grid(UtilArgs a, int wr, int wc, int gr, int gc, int8_t* grid) {
    __shared__ uint32_t bits[2 * kMaxWords];
    __shared__ uint32_t flags[65536 / 16];
    const RowBits rb{bits, bits + kMaxWords};
    const int64_t bh = blockIdx.x / gr;
    const int i = (int)(blockIdx.x % gr);
    for (int j = threadIdx.x; j < (gc + 15) / 16; j += kThreads) flags[j] = 0u;
    const int r_end = min((i + 1) * wr, a.nQB);
    for (int r = i * wr; r < r_end; ++r) {
        load_row_bits(rb, a, bh * a.nQB + r, a.nKB);
        for (int kb = threadIdx.x; kb < a.nKB; kb += kThreads) {
            const int c = bit_class(rb, kb);
            const int j = kb / wc;
            atomicOr(flags + (j >> 4), ((c != 2 ? 1u : 0u) | (c != 0 ? 2u : 0u)) << (2 * (j & 15)));
        }
        __syncthreads();
    }
    for (int j = threadIdx.x; j < gc; j += kThreads) {
        const uint32_t f = flags[j >> 4] >> (2 * (j & 15));
        grid[(bh * gr + i) * gc + j] = (int8_t)(!(f & 1u) ? 2 : (!(f & 2u) ? 0 : 1));
    }
}

// Sparsity: a zeroing pass, an integer count of the distinct listed tiles
// (order-independent, so the result is exact and repeatable), and the
// conversion to a percentage, all in the caller's 8 bytes.
__global__ void blockmask_count_zero(unsigned long long* acc) { *acc = 0ull; }

__global__ __launch_bounds__(kThreads) void blockmask_count(UtilArgs a, unsigned long long* acc) {
    __shared__ uint32_t bits[2 * kMaxWords];
    __shared__ unsigned int total;
    const RowBits rb{bits, bits + kMaxWords};
    if (threadIdx.x == 0) total = 0u;
    load_row_bits(rb, a, blockIdx.x, a.nKB);
    unsigned int n = 0;
    for (int w = threadIdx.x; w < (a.nKB + 31) / 32; w += kThreads) n += __popc(rb.part[w] | rb.full[w]);
    atomicAdd(&total, n);
    __syncthreads();
    if (threadIdx.x == 0) atomicAdd(acc, (unsigned long long)total);
}

__global__ void blockmask_count_finish(unsigned long long* acc, double tiles) {
    const unsigned long long n = *acc;
    *reinterpret_cast<double*>(acc) = 100.0 * (1.0 - (double)n / tiles);
}

__global__ __launch_bounds__(kThreads) void blockmask_slice(UtilArgs a, SliceArgs s, UtilOut o) {
    const int64_t out_row = blockIdx.x;
    const int r = (int)(out_row % s.rows);
    const int64_t bh = out_row / s.rows;
    const int h = (int)(bh % s.heads), b = (int)(bh / s.heads);
    const int64_t in_row = ((int64_t)(s.b0 + b) * a.Hm + (s.h0 + h)) * a.nQB + (s.r0 + r);
    if (threadIdx.x == 0) {
        o.kv_num[out_row] = a.kv_num[in_row];
        o.full_num[out_row] = a.full_num[in_row];
    }
    for (int t = threadIdx.x; t < a.nKB; t += kThreads) {
        o.kv_idx[out_row * a.nKB + t] = a.kv_idx[in_row * a.nKB + t];
        o.full_idx[out_row * a.nKB + t] = a.full_idx[in_row * a.nKB + t];
    }
}

// Position of this thread's set bit among the workgroup's set bits below it,
// and the workgroup's count (all threads take part).
__device__ __forceinline__ int block_rank(bool flag, int& count, unsigned int* scratch) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t bal = __ballot(flag);
    const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (lane == 0) scratch[wave] = (unsigned int)__popcll(bal);
    __syncthreads();
    int before = 0;
    count = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
        before += w < wave ? (int)scratch[w] : 0;
        count += (int)scratch[w];
    }
    __syncthreads();
    return before + below;
}

// Cropping: row r of the output keeps the blocks below nk of input row r; a
// full tile on the cut row (edge_row) or in the cut column (edge_col) becomes
// partial; the lists are written ascending and then completed ascending.
__global__ __launch_bounds__(kThreads) void blockmask_adjust(UtilArgs a, int nq, int nk, int edge_row, int edge_col,
                                                             UtilOut o) {
    __shared__ uint32_t bits[2 * kMaxWords];
    __shared__ unsigned int scratch[kThreads / 64];
    const RowBits rb{bits, bits + kMaxWords};
    const int64_t out_row = blockIdx.x;
    const int r = (int)(out_row % nq);
    const int64_t bh = out_row / nq;
    load_row_bits(rb, a, bh * a.nQB + r, nk);
    const bool cut_row = edge_row && r == nq - 1;
    // totals first (class of every block after the reclassification)
    int n_part = 0, n_full = 0;
    for (int base = 0; base < nk; base += kThreads) {
        const int kb = base + (int)threadIdx.x;
        int c = kb < nk ? bit_class(rb, kb) : 0;
        if (c == 2 && (cut_row || (edge_col && kb == nk - 1))) c = 1;
        int cnt;
        block_rank(c == 1, cnt, scratch);
        n_part += cnt;
        block_rank(c == 2, cnt, scratch);
        n_full += cnt;
    }
    int lp = 0, lf = 0, rp = n_part, rf = n_full;
    for (int base = 0; base < nk; base += kThreads) {
        const int kb = base + (int)threadIdx.x;
        const bool in = kb < nk;
        int c = in ? bit_class(rb, kb) : 0;
        if (c == 2 && (cut_row || (edge_col && kb == nk - 1))) c = 1;
        int c_is_p, c_not_p, c_is_f, c_not_f;
        const int k_is_p = block_rank(in && c == 1, c_is_p, scratch);
        const int k_not_p = block_rank(in && c != 1, c_not_p, scratch);
        const int k_is_f = block_rank(in && c == 2, c_is_f, scratch);
        const int k_not_f = block_rank(in && c != 2, c_not_f, scratch);
        if (in) {
            o.kv_idx[out_row * nk + (c == 1 ? lp + k_is_p : rp + k_not_p)] = kb;
            o.full_idx[out_row * nk + (c == 2 ? lf + k_is_f : rf + k_not_f)] = kb;
        }
        lp += c_is_p;
        rp += c_not_p;
        lf += c_is_f;
        rf += c_not_f;
    }
    if (threadIdx.x == 0) {
        o.kv_num[out_row] = n_part;
        o.full_num[out_row] = n_full;
    }
}

}  // namespace

hipError_t launch_blockmask_to_dense(const UtilArgs& a, int32_t* dense, hipStream_t stream) {
    const int64_t rows = (int64_t)a.Bm * a.Hm * a.nQB;
    hipLaunchKernelGGL(blockmask_to_dense, dim3((unsigned)rows), dim3(kThreads), 0, stream, a, dense);
    return hipGetLastError();
}

hipError_t launch_blockmask_grid(const UtilArgs& a, int wr, int wc, int8_t* grid, hipStream_t stream) {
    const int gr = (a.nQB + wr - 1) / wr, gc = (a.nKB + wc - 1) / wc;
    const int64_t blocks = (int64_t)a.Bm * a.Hm * gr;
    hipLaunchKernelGGL(blockmask_grid, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, wr, wc, gr, gc, grid);
    return hipGetLastError();
}

hipError_t launch_blockmask_sparsity(const UtilArgs& a, double* percent, hipStream_t stream) {
    unsigned long long* acc = reinterpret_cast<unsigned long long*>(percent);
    hipLaunchKernelGGL(blockmask_count_zero, dim3(1), dim3(1), 0, stream, acc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)a.Bm * a.Hm * a.nQB;
    hipLaunchKernelGGL(blockmask_count, dim3((unsigned)rows), dim3(kThreads), 0, stream, a, acc);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(blockmask_count_finish, dim3(1), dim3(1), 0, stream, acc, (double)rows * (double)a.nKB);
    return hipGetLastError();
}

hipError_t launch_blockmask_slice(const UtilArgs& a, const SliceArgs& s, const UtilOut& o, hipStream_t stream) {
    const int64_t rows = (int64_t)s.batches * s.heads * s.rows;
    hipLaunchKernelGGL(blockmask_slice, dim3((unsigned)rows), dim3(kThreads), 0, stream, a, s, o);
    return hipGetLastError();
}

hipError_t launch_blockmask_adjust(const UtilArgs& a, int nq, int nk, int edge_row, int edge_col, const UtilOut& o,
                                   hipStream_t stream) {
    const int64_t rows = (int64_t)a.Bm * a.Hm * nq;
    hipLaunchKernelGGL(blockmask_adjust, dim3((unsigned)rows), dim3(kThreads), 0, stream, a, nq, nk, edge_row,
                       edge_col, o);
    return hipGetLastError();
}

}  // namespace flexmi
