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
// One launch, one workgroup per Q-block row:
//   classify  waves take the row's tiles in turn.  Where the mask's rule is
//             monotone in (q, kv) -- the causal part kv <= q, the window
//             q - kv < W, the sink kv < sinks and the L/S bounds -- the class
//             is read off the tile's corner cells, which gives exactly the
//             class that counting would; otherwise each lane owns a key column
//             and counts the visible cells of its column in closed form (the
//             window and sinks bound an interval of rows; for documents the
//             block's rows are cut into runs of equal id, so the count is a sum
//             over the runs that carry the column's id), and a wave reduction
//             gives the tile count.  Classes go to LDS, two bits per tile.
//   compact   wave 0 writes the ordered partial list, wave 1 the full list.
//
// Layout conventions: cells beyond L or S are not visible; each index row
// lists its tiles ascending, then the remaining tile indices ascending.
#include <climits>

#include "internal.hpp"

namespace flexmi {

namespace {

constexpr int kMaxQBlock = 1024;

enum : int { TILE_EMPTY = 0, TILE_PARTIAL = 1, TILE_FULL = 2, TILE_COUNT = 3 };

// Class of a tile decided from its corners, or TILE_COUNT when the cells have
// to be counted.  Rows [r0, r1] (logical positions p0 = r0 + off, p1), columns
// [c0, c1], all clipped to L and S; `clipped` tells whether the tile extends
// past L or S (then it cannot be full).
// Three-valued truth of a PROGRAM predicate over the rectangle of positions
// [p0, p1] x keys [c0, c1] at head h: all cells true, all false, or mixed /
// not known without counting.
enum : int { TRI_FALSE = 0, TRI_TRUE = 1, TRI_MIXED = 2 };

__device__ __forceinline__ int floor_div_i64(int64_t a, int64_t b) {
    const int64_t q = a / b;
    return (int)((a % b != 0 && a < 0) ? q - 1 : q);
}

__device__ __forceinline__ int pred_over_tile(int kind, int arg, int p0, int p1, int c0, int c1, int h) {
    switch (kind) {
    case PRED_CAUSAL:                                   // j <= p
        return c1 <= p0 ? TRI_TRUE : (c0 > p1 ? TRI_FALSE : TRI_MIXED);
    case PRED_WINDOW:                                   // p - j < arg
        return (int64_t)p1 - c0 < arg ? TRI_TRUE : ((int64_t)p0 - c1 >= arg ? TRI_FALSE : TRI_MIXED);
    case PRED_KV_LT:                                    // j < arg
        return c1 < arg ? TRI_TRUE : (c0 >= arg ? TRI_FALSE : TRI_MIXED);
    case PRED_CHUNK: {                                  // floor(p/arg) == floor(j/arg)
        const int fp0 = floor_div_i64(p0, arg), fp1 = floor_div_i64(p1, arg);
        const int fc0 = floor_div_i64(c0, arg), fc1 = floor_div_i64(c1, arg);
        if (fp0 == fp1 && fc0 == fc1 && fp0 == fc0) return TRI_TRUE;
        return (fp1 < fc0 || fc1 < fp0) ? TRI_FALSE : TRI_MIXED;
    }
    case PRED_STRIDE: return arg == 1 ? TRI_TRUE : TRI_MIXED;
    case PRED_DOC: return TRI_MIXED;
    default: return h < arg ? TRI_TRUE : TRI_FALSE;     // PRED_HEAD_LT
    }
}

// Kleene AND over clauses of Kleene ORs: a tile is decided when the program is
// true (false) on every cell; otherwise its cells are counted.
__device__ __forceinline__ int program_over_tile(const MaskProgram& pg, int p0, int p1, int c0, int c1, int h) {
    int all = TRI_TRUE;
#pragma unroll
    for (int c = 0; c < kMaxClauses; ++c) {
        if (c >= pg.n_clauses) break;
        int any = TRI_FALSE;
#pragma unroll
        for (int l = 0; l < kMaxLiterals; ++l) {
            if (l >= pg.n_lits[c]) break;
            const int t = pred_over_tile(pg.kind[c][l], pg.arg[c][l], p0, p1, c0, c1, h);
            if (t == TRI_TRUE) any = TRI_TRUE;
            else if (t == TRI_MIXED && any == TRI_FALSE) any = TRI_MIXED;
        }
        if (any == TRI_FALSE) return TRI_FALSE;
        if (any == TRI_MIXED) all = TRI_MIXED;
    }
    return all;
}

// Visible cells of key column j over the block's rows, for a PROGRAM mask.
// For a fixed column every predicate is an interval of positions p (causal:
// p >= j; window: p <= j + W - 1; chunk: the chunk of j; kv_lt and head_lt:
// everything or nothing), except stride (an interval plus p = j mod arg,
// tracked incrementally) and doc (a per-run comparison).  The rows are then
// scanned with compares only, run by run.
__device__ __forceinline__ int count_program_column(const MaskProgram& pg, int j, int h, int doc_j, int p0,
                                                    const int* run_start, const int* run_doc, int runs) {
    constexpr int kInterval = 0, kStride = 1, kDoc = 2;
    int lo[kMaxClauses][kMaxLiterals], hi[kMaxClauses][kMaxLiterals], kind[kMaxClauses][kMaxLiterals];
    int modk[kMaxClauses][kMaxLiterals], res[kMaxClauses][kMaxLiterals];
    const int p_first = p0 + run_start[0];
#pragma unroll
    for (int c = 0; c < kMaxClauses; ++c)
#pragma unroll
        for (int l = 0; l < kMaxLiterals; ++l) {
            int L = INT_MIN, H = INT_MAX, K = kInterval, mk = 1, rs = 0;
            if (c < pg.n_clauses && l < pg.n_lits[c]) {
                const int arg = pg.arg[c][l];
                switch (pg.kind[c][l]) {
                case PRED_CAUSAL: L = j; break;
                case PRED_WINDOW: H = (int)min<int64_t>((int64_t)j + arg - 1, INT_MAX); break;
                case PRED_KV_LT: if (!(j < arg)) { L = 1; H = 0; } break;
                case PRED_CHUNK: {
                    const int64_t c0 = (int64_t)(j / arg) * arg;     // j >= 0
                    L = (int)c0;
                    H = (int)min<int64_t>(c0 + arg - 1, INT_MAX);
                    break;
                }
                case PRED_STRIDE: {
                    K = kStride;
                    mk = arg;
                    int r = (int)(((int64_t)p_first - j) % arg);
                    rs = r < 0 ? r + arg : r;                        // (p - j) mod arg at the first row
                    break;
                }
                case PRED_DOC: K = kDoc; break;
                default: if (!(h < arg)) { L = 1; H = 0; } break;   // PRED_HEAD_LT
                }
            }
            lo[c][l] = L; hi[c][l] = H; kind[c][l] = K; modk[c][l] = mk; res[c][l] = rs;
        }
    bool has_stride = false;
#pragma unroll
    for (int c = 0; c < kMaxClauses; ++c)
#pragma unroll
        for (int l = 0; l < kMaxLiterals; ++l) has_stride = has_stride || kind[c][l] == kStride;
    // program value at position p of a run whose document equality is same_doc
    auto holds = [&](int p, bool same_doc) {
        bool all = true;
#pragma unroll
        for (int c = 0; c < kMaxClauses; ++c) {
            if (c >= pg.n_clauses) break;
            bool any = false;
#pragma unroll
            for (int l = 0; l < kMaxLiterals; ++l) {
                if (l >= pg.n_lits[c]) break;
                bool v = p >= lo[c][l] && p <= hi[c][l];
                if (kind[c][l] == kDoc) v = v && same_doc;
                any = any || v;
            }
            all = all && any;
        }
        return all;
    };
    int count = 0;
    if (!has_stride && runs <= 8) {
        // Without stride predicates the program is constant between interval
        // end points, so each run is cut at those points and each piece is
        // evaluated once.
        for (int r = 0; r < runs; ++r) {
            const bool same_doc = run_doc[r] == doc_j;
            const int a0 = p0 + run_start[r], a1 = p0 + run_start[r + 1];   // [a0, a1)
            int b = a0;
            while (b < a1) {
                int next = a1;   // smallest boundary above b
#pragma unroll
                for (int c = 0; c < kMaxClauses; ++c)
#pragma unroll
                    for (int l = 0; l < kMaxLiterals; ++l) {
                        const int e0 = lo[c][l];
                        const int64_t e1 = (int64_t)hi[c][l] + 1;
                        if (e0 > b && e0 < next) next = e0;
                        if (e1 > b && e1 < next) next = (int)e1;
                    }
                if (holds(b, same_doc)) count += next - b;
                b = next;
            }
        }
        return count;
    }
    for (int r = 0; r < runs; ++r) {
        const int dp = run_doc[r];
        const bool same_doc = dp == doc_j;
        for (int p = p0 + run_start[r]; p < p0 + run_start[r + 1]; ++p) {
            bool all = true;
#pragma unroll
            for (int c = 0; c < kMaxClauses; ++c) {
                if (c >= pg.n_clauses) break;
                bool any = false;
#pragma unroll
                for (int l = 0; l < kMaxLiterals; ++l) {
                    if (l >= pg.n_lits[c]) break;
                    bool v = p >= lo[c][l] && p <= hi[c][l];
                    if (kind[c][l] == kStride) v = v && res[c][l] == 0;
                    else if (kind[c][l] == kDoc) v = v && same_doc;
                    any = any || v;
                }
                all = all && any;
            }
            count += all ? 1 : 0;
#pragma unroll
            for (int c = 0; c < kMaxClauses; ++c)
#pragma unroll
                for (int l = 0; l < kMaxLiterals; ++l)
                    if (kind[c][l] == kStride && ++res[c][l] == modk[c][l]) res[c][l] = 0;
        }
    }
    return count;
}

template <int KIND>
__device__ __forceinline__ int corner_class(const MaskArgs& m, int p0, int p1, int c0, int c1, bool clipped, int h) {
    if constexpr (KIND == MASK_PROGRAM) {
        const int t = program_over_tile(m.prog, p0, p1, c0, c1, h);
        if (t == TRI_FALSE) return TILE_EMPTY;
        if (t == TRI_TRUE) return clipped ? TILE_PARTIAL : TILE_FULL;
        return TILE_COUNT;
    } else if constexpr (KIND == MASK_NOOP) {
        return clipped ? TILE_PARTIAL : TILE_FULL;
    } else {
        if (c0 > p1) return TILE_EMPTY;                       // every kv > every q: causal part fails
        if constexpr (KIND == MASK_CAUSAL) {
            if (c1 <= p0) return clipped ? TILE_PARTIAL : TILE_FULL;
            return TILE_PARTIAL;                              // both visible and hidden cells exist
        } else if constexpr (KIND == MASK_CAUSAL_WINDOW_SINKS) {
            // hidden everywhere: beyond the window for every cell and past the sinks
            if (p0 - c1 >= m.window && c0 >= m.sinks) return TILE_EMPTY;
            // visible everywhere: causal for every cell and inside the window or a sink
            if (c1 <= p0 && (p1 - c0 < m.window || c1 < m.sinks)) return clipped ? TILE_PARTIAL : TILE_FULL;
            return TILE_COUNT;
        } else {
            return TILE_COUNT;                                // document ids have to be compared
        }
    }
}

// Document id of a position, or `none` outside the id array (such positions
// belong to no document).
__device__ __forceinline__ int doc_at(const MaskArgs& m, int p, int none) {
    return (p >= 0 && p < m.doc_len) ? __ldg(m.doc_id + p) : none;
}

__device__ __forceinline__ int class_of(const uint32_t* words, int kb) {
    return (int)((words[kb >> 4] >> (2 * (kb & 15))) & 3u);
}

// Masks that count cells use 16 waves; the others only need the two that
// write the lists.
template <int KIND>
constexpr int build_threads() {
    return (KIND == MASK_CAUSAL_WINDOW_SINKS || KIND == MASK_DOC_CAUSAL || KIND == MASK_PROGRAM) ? 1024 : 128;
}
constexpr int kCountBatch = 8;

template <int KIND>
__global__ __launch_bounds__(build_threads<KIND>()) void blockmask_build(BuildArgs a) {
    constexpr int kBuildThreads = build_threads<KIND>();
    constexpr int kBuildWaves = kBuildThreads / 64;
    // Document runs of this block's rows: maximal stretches of equal id.
    __shared__ int run_start[kMaxQBlock + 1];
    __shared__ int run_doc[kMaxQBlock];
    __shared__ int run_count;
    extern __shared__ uint32_t tile_class[];  // 2 bits per tile, 16 tiles per word
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int qb = blockIdx.x;
    const int bh = blockIdx.y;
    const int row0 = qb * a.q_block;
    const int rows = min(a.q_block, a.L - row0);
    const int64_t row_id = (int64_t)bh * a.nQB + qb;
    const int h = bh % a.Hm;   // query head of this mask row (0 when broadcast)
    const int bb = bh / a.Hm;  // batch of this mask row
    // per-batch logical offset of row 0 and valid key count (clamped into range)
    const int q_offset = a.mask.q_offsets ? min(max(a.mask.q_offsets[bb], -(1 << 30)), 1 << 30) : a.mask.q_offset;
    const int S = a.mask.kv_lens ? min(max(a.mask.kv_lens[bb], 0), a.S) : a.S;
    const int p0 = row0 + q_offset, p1 = p0 + rows - 1;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if constexpr (KIND == MASK_PROGRAM) {
        if (!a.mask.uses_doc && threadIdx.x == 0) {
            // one run holding every row, with no document
            run_start[0] = 0;
            run_start[1] = rows;
            run_doc[0] = -2;
            run_count = 1;
        }
    }
    if (KIND == MASK_DOC_CAUSAL || (KIND == MASK_PROGRAM && a.mask.uses_doc)) {
        if (wave == 0) {
            int runs = 0;
            for (int i0 = 0; i0 < rows; i0 += 64) {
                const int i = i0 + lane;
                const int d = i < rows ? doc_at(a.mask, p0 + i, -2) : 0;
                const int prev = (i > 0 && i < rows) ? doc_at(a.mask, p0 + i - 1, -2) : 0;
                const bool start = i < rows && (i == 0 || d != prev);
                const uint64_t starts = __ballot(start);
                if (start) {
                    const int r = runs + __popcll(starts & below);
                    run_start[r] = i;
                    run_doc[r] = d;
                }
                runs += __popcll(starts);
            }
            if (lane == 0) {
                run_start[runs] = rows;
                run_count = runs;
            }
        }
    }

    // Phase 1: classify.  Corner rules first (one tile per thread, the 2-bit
    // classes OR-ed into their LDS words), then the tiles that need counting,
    // one per wave.
    const int words = (a.nKB + 15) >> 4;
    for (int w = threadIdx.x; w < words; w += kBuildThreads) tile_class[w] = 0u;
    __syncthreads();
    for (int kb = threadIdx.x; kb < a.nKB; kb += kBuildThreads) {
        const int c0 = kb * a.kv_block;
        const int c1 = min(c0 + a.kv_block, S) - 1;
        const bool clipped = rows < a.q_block || c0 + a.kv_block > S;
        // tiles past the valid keys are empty
        const int cls = c0 >= S ? TILE_EMPTY : corner_class<KIND>(a.mask, p0, p1, c0, c1, clipped, h);
        if (cls != 0) atomicOr(&tile_class[kb >> 4], (uint32_t)cls << (2 * (kb & 15)));
    }
    __syncthreads();
    if constexpr (KIND == MASK_CAUSAL_WINDOW_SINKS || KIND == MASK_DOC_CAUSAL || KIND == MASK_PROGRAM) {
        // A wave takes kCountBatch of its tiles at a time so that the column id
        // loads of the batch are in flight together.
        const int runs = (KIND == MASK_DOC_CAUSAL || KIND == MASK_PROGRAM) ? run_count : 0;
        for (int kb0 = wave; kb0 < a.nKB; kb0 += kBuildWaves * kCountBatch) {
            bool todo[kCountBatch];
            bool any = false;
#pragma unroll
            for (int u = 0; u < kCountBatch; ++u) {
                const int kb = kb0 + u * kBuildWaves;
                todo[u] = kb < a.nKB && class_of(tile_class, kb) == TILE_COUNT;   // wave-uniform
                any |= todo[u];
            }
            if (!any) continue;
            int count[kCountBatch];   // visible cells of this lane's columns, per tile
#pragma unroll
            for (int u = 0; u < kCountBatch; ++u) count[u] = 0;
            for (int j0 = 0; j0 < a.kv_block; j0 += 64) {
                const int jj = j0 + lane;
                int doc_col[kCountBatch];
                if (KIND == MASK_DOC_CAUSAL || (KIND == MASK_PROGRAM && a.mask.uses_doc)) {
#pragma unroll
                    for (int u = 0; u < kCountBatch; ++u) {
                        const int col = (kb0 + u * kBuildWaves) * a.kv_block + jj;
                        doc_col[u] = (todo[u] && jj < a.kv_block && col < S) ? doc_at(a.mask, col, -1) : -1;
                    }
                }
#pragma unroll
                for (int u = 0; u < kCountBatch; ++u) {
                    const int col = (kb0 + u * kBuildWaves) * a.kv_block + jj;
                    if (!todo[u] || jj >= a.kv_block || col >= S) continue;
                    // rows of this column that pass the causal part: p in [max(p0, col), p1]
                    const int lo = max(p0, col);
                    if constexpr (KIND == MASK_CAUSAL_WINDOW_SINKS) {
                        // a sink column is seen by every later row; any other
                        // column by rows p < col + window
                        const int hi = (col < a.mask.sinks || a.mask.window > p1 - col) ? p1 : col + a.mask.window - 1;
                        count[u] += max(0, hi - lo + 1);
                    } else if constexpr (KIND == MASK_PROGRAM) {
                        const int dc = a.mask.uses_doc ? doc_col[u] : -1;
                        count[u] += count_program_column(a.mask.prog, col, h, dc, p0, run_start, run_doc, runs);
                    } else {
                        // rows of a run with the column's document, at or after the column
                        for (int r = 0; r < runs; ++r) {
                            if (run_doc[r] != doc_col[u]) continue;
                            const int s0 = max(p0 + run_start[r], lo);
                            count[u] += max(0, p0 + run_start[r + 1] - s0);
                        }
                    }
                }
            }
            const int cells = a.q_block * a.kv_block;
#pragma unroll
            for (int u = 0; u < kCountBatch; ++u) {
                if (!todo[u]) continue;
                int c = count[u];
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
                const int kb = kb0 + u * kBuildWaves;
                const uint32_t cls = c == 0 ? TILE_EMPTY : (c == cells ? TILE_FULL : TILE_PARTIAL);
                // the tile's two bits read TILE_COUNT (both set): clear the ones cls lacks
                if (lane == 0) atomicAnd(&tile_class[kb >> 4], ~((TILE_COUNT & ~cls) << (2 * (kb & 15))));
            }
        }
        __syncthreads();
    }
    if (wave > 1) return;

    // Phase 2: wave 0 writes the partial list, wave 1 the full list.
    const int want = wave == 0 ? TILE_PARTIAL : TILE_FULL;
    int* idx = (wave == 0 ? a.kv_idx : a.full_idx) + row_id * a.nKB;
    int* num = (wave == 0 ? a.kv_num : a.full_num) + row_id;
    int total = 0;
    for (int c0 = 0; c0 < a.nKB; c0 += 64) {
        const int kb = c0 + lane;
        total += __popcll(__ballot(kb < a.nKB && class_of(tile_class, kb) == want));
    }
    int hits = 0;    // listed tiles before this chunk
    int misses = 0;  // other tiles before this chunk
    for (int c0 = 0; c0 < a.nKB; c0 += 64) {
        const int kb = c0 + lane;
        const bool in = kb < a.nKB;
        const bool hit = in && class_of(tile_class, kb) == want;
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
hipError_t launch_build(const BuildArgs& a, hipStream_t stream) {
    dim3 grid(a.nQB, a.Bm * a.Hm);
    const size_t lds = (size_t)((a.nKB + 15) >> 4) * sizeof(uint32_t);
    hipLaunchKernelGGL(blockmask_build<KIND>, grid, dim3(build_threads<KIND>()), lds, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_blockmask_build(const BuildArgs& a, hipStream_t stream) {
    switch (a.mask.kind) {
    case MASK_NOOP: return launch_build<MASK_NOOP>(a, stream);
    case MASK_CAUSAL: return launch_build<MASK_CAUSAL>(a, stream);
    case MASK_CAUSAL_WINDOW_SINKS: return launch_build<MASK_CAUSAL_WINDOW_SINKS>(a, stream);
    case MASK_PROGRAM: return launch_build<MASK_PROGRAM>(a, stream);
    default: return launch_build<MASK_DOC_CAUSAL>(a, stream);
    }
}

}  // namespace flexmi
