// Block-sparse attention backward for gfx950 (CDNA4): dq, dk, dv.
//
// What is computed: the gradients of sum(out * dout) through the forward
// definition (scaled score, score_mod g, -inf where mask_mod is false, row
// softmax, weighted sum of values).  The charlestar blog "FlexAttention
// score_mod / BlockMask" calls backward on the summed output of its example;
// the 2kiu "PyTorch Flex Attention complete guide" (section 3.3) has the
// backward walk Q-side lists obtained by transposing the KV-side lists, and
// (sections 4.1 and 5.1) offers a deterministic dQ write order.  With
// P = exp(z - lse) from the forward's lse and D_i = dout_i . out_i:
//
//   dS = P * (dout v^T - D) * g'(s) * scale,  g' = 1 - tanh(s/cap)^2 or 1
//   dv = P^T dout,   dk = dS^T q,   dq = dS k
//
// How it maps onto CDNA4 (design of this library, not of the pages):
//   * A row pass writes D_i and the base-2 lse per row (rows padded to a
//     multiple of 128, +inf for rows that saw no key, so their P is 0).
//   * Key-major pass (dk, dv): a workgroup owns 64 keys of one K/V head and
//     walks their KV block's Q-side lists, for each query head of the GQA
//     group in turn, so dk and dv of the K/V head are summed in registers.
//     Wave (kh, qh) takes key half kh (32 keys) and query half qh of every
//     64-query tile.  Scores are computed S = Q K^T, so each lane holds one key
//     and 16 query rows: K and V rows stay in registers as the MFMA B operands
//     of S and dP = dO V^T, the Q and dO tiles (with the rows' lse, D and
//     document ids) stream through LDS, and P and dS feed dv^T += dO^T P and
//     dk^T += Q^T dS straight from registers, the A operands coming from
//     transposing LDS reads of the same tiles.  The two query halves are added
//     once at the end.
//   * Query-major pass (dq): the forward's layout.  A workgroup owns 64 query
//     rows; wave (rg, kh) takes row group rg and key half kh of every K/V tile
//     of the row block's KV-side lists.  S^T = K Q^T and dP^T = V dO^T with Q
//     and dO rows in registers, so each lane holds one query row and its lse
//     and D are per-lane scalars; dq^T += K^T dS^T.  The key halves are added
//     once at the end.
//   * Both passes recompute the scores, so nothing is accumulated with
//     atomics: every output element is written once, by one workgroup, and
//     the results do not depend on scheduling.
//   * bf16 tiles arrive by LDS-DMA into a double buffer in the forward's
//     swizzled layout; fp32 tiles are staged through registers into padded
//     rows.
#pragma once

#include "attn_fwd_impl.hpp"

namespace flexmi {

namespace {

// The LDS array seen in its own address space: DMA destinations are formed
// there, so no generic-to-LDS conversion of a constant address is needed.
typedef __attribute__((address_space(3))) char lds_char_t;

// LDS geometry of one ring buffer of the backward passes: two row-major
// 64-row tiles (Q and dO, or K and V), then the tile rows' base-2 lse and D
// (key-major pass) and document ids.  bf16 rows are unpadded and swizzled as
// in the forward (filled by LDS-DMA); fp32 rows are padded by four floats.
template <typename T, int D> struct BwdTiles {
    static constexpr int kStride = sizeof(T) == 2 ? D : D + Elem<float>::kPadK;   // elements per row
    static constexpr int kTileBytes = kTileN * kStride * (int)sizeof(T);
    static constexpr int kStatsOffset = 2 * kTileBytes;
    static constexpr int kDocOffset = kStatsOffset + 2 * kTileN * 4;
    static constexpr int kBufBytes = kDocOffset + kTileN * 4;
    static_assert(kStride == Tiles<T, D>::kStrideK, "qk_block reads the first tile with this row stride");
};

// LDS-DMA fill of a 64-row bf16 tile in the forward's swizzled layout (see
// dma_plan): wave w's instruction i writes the 64 contiguous 16-byte chunks
// (i*4 + w)*64 .. +63, lane l the one at position l.  The chunk a lane loads
// depends on its row only modulo 16, and instruction i + 1 is 2048/D rows
// further, so one per-lane byte offset serves every instruction; the row step
// goes into the scalar offset.
template <int D>
__device__ __forceinline__ int dma_lane_offset(int row_bytes, int wave, int lane) {
    constexpr int kChunksPerRow = D / 8;
    const int pos = wave * 64 + lane;
    const int row = pos / kChunksPerRow;
    const int chunk = (pos % kChunksPerRow) ^ swz<D>(row);
    return row * row_bytes + chunk * 16;
}
constexpr int dma_rows_per_inst(int D) { return 2048 / D; }

// Waves per SIMD the backward kernels are compiled for.
template <typename T, int D> struct BwdOccupancy {
    static constexpr int kKeys = sizeof(T) == 2 ? 2 : 1;
    static constexpr int kRows = sizeof(T) == 2 ? 2 : 1;
};

// Per-head constants of the score rule, base-2 units.
struct BwdConsts {
    ScoreConsts sc;   // mul (NONE / ALIBI: scale*log2e; soft-cap: 2*scale*log2e/cap), c2 = cap*log2e, polynomials
    float scale;
    float gk;         // scale / c2^2: g'(s) * scale = scale - gk * (capped base-2 score)^2
    float alpha2;     // distance-bias slope * log2e of the query head (0 without bias)
};

__device__ __forceinline__ BwdConsts bwd_consts(const BwdArgs& a, int hq) {
    BwdConsts c;
    c.sc = a.sc;
    c.scale = a.scale;
    c.gk = a.scale / (a.sc.c2 * a.sc.c2);
    c.alpha2 = 0.0f;
    if (a.score_kind == SCORE_SOFTCAP_ALIBI || a.score_kind == SCORE_ALIBI)
        c.alpha2 = __builtin_amdgcn_exp2f(-(a.alibi_m * (float)(hq + 1)) / (float)a.Hq) * kLog2e;
    return c;
}

// Base-2 scores z[r] = g(s) * log2e of the accumulators s[r] (= q.k) plus the
// distance bias bias0 + step * acc_row(r, 0) (ALiBi kinds), and gs[r] =
// g'(s) * scale.  The soft-cap tanh uses the forward's polynomials when every
// |s| of the wave is in their range (wave-uniform choice; their error, at
// most 7.9e-6 of the cap, is far inside the bf16 bounds), else the exact form
// cap - 2 cap / (1 + e^{2y}); the fp32 path always takes the exact form.
template <int SCORE, bool PRECISE>
__device__ __forceinline__ void scores2(const f32x16_t& s, float bias0, float step, const BwdConsts& c, float (&z)[16],
                                        float (&gs)[16]) {
    constexpr bool kBias = SCORE == SCORE_ALIBI || SCORE == SCORE_SOFTCAP_ALIBI;
    auto bias = [&](int r) __attribute__((always_inline)) {
        return kBias ? __builtin_fmaf(step, (float)acc_row(r, 0), bias0) : 0.0f;
    };
    if constexpr (SCORE == SCORE_NONE || SCORE == SCORE_ALIBI) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            z[r] = kBias ? __builtin_fmaf(s[r], c.sc.mul, bias(r)) : s[r] * c.sc.mul;
            gs[r] = c.scale;
        }
        return;
    } else {
        int tier = 2;   // 0 cubic, 1 quintic, 2 exact
        if constexpr (!PRECISE) {
            float amax = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(s[r]));
            tier = !__any(amax > c.sc.amax1) ? 0 : (!__any(amax > c.sc.amax) ? 1 : 2);
        }
        if (tier == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) z[r] = s[r] * __builtin_fmaf(s[r] * s[r], c.sc.j1, c.sc.j0);
        } else if (tier == 1) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float w = s[r] * s[r];
                z[r] = s[r] * __builtin_fmaf(w, __builtin_fmaf(w, c.sc.k2, c.sc.k1), c.sc.k0);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = __builtin_amdgcn_exp2f(s[r] * c.sc.mul);
                z[r] = __builtin_fmaf(-2.0f * c.sc.c2, __builtin_amdgcn_rcpf(1.0f + e), c.sc.c2);
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            gs[r] = __builtin_fmaf(-c.gk * z[r], z[r], c.scale);
            if constexpr (kBias) z[r] += bias(r);
        }
    }
}

// S and dP blocks of one 32-row block of two LDS tiles against two register
// operands (bf16), with the two MFMA chains interleaved so neither waits on
// its own previous result.
template <int D>
__device__ __forceinline__ void qk2_block_bf16(const QRegs<__bf16, D>& ra, const QRegs<__bf16, D>& rb,
                                               const char* __restrict__ ta, const char* __restrict__ tb,
                                               const LdsAddr<__bf16, D>& la, f32x16_t& sa, f32x16_t& sb) {
    sa = f32x16_t{};
    sb = f32x16_t{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        const bf16x8_t xa = *reinterpret_cast<const bf16x8_t*>(ta + la.k[s]);
        const bf16x8_t xb = *reinterpret_cast<const bf16x8_t*>(tb + la.k[s]);
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, ra.x[s], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xb, rb.x[s], sb, 0, 0, 0);
    }
}

template <typename T, int D>
__device__ __forceinline__ void qk2_block(const QRegs<T, D>& ra, const QRegs<T, D>& rb, const char* ta, const char* tb,
                                          const LdsAddr<T, D>& la, int kb2, int lane, f32x16_t& sa, f32x16_t& sb) {
    if constexpr (sizeof(T) == 2) {
        qk2_block_bf16<D>(ra, rb, ta, tb, la, sa, sb);
    } else {
        sa = qk_block<T, D>(ra, ta, la, kb2, lane);
        sb = qk_block<T, D>(rb, tb, la, kb2, lane);
    }
}

// Visibility in the key-major orientation: bit o of the result says whether
// this lane's key `key` is visible from query row qr0 + o (qr0 includes the
// lane half's row offset; the rows used are o = acc_row(r, 0)).  Rows past L
// and keys past S (the batch's filled length) are hidden.  q_off is the
// batch's position of query row 0.  doc_rows holds the document ids of rows
// qr0 + 0..27 (LDS); a row whose position lies outside doc_id has no document.
template <bool EXT>
__device__ __forceinline__ uint32_t mask_bits_keys(const MaskArgs& m, int key, int S, int L, int qr0, int q_off,
                                                   int hq, int doc_k, const int* __restrict__ doc_rows) {
    const int p0i = qr0 + q_off;                             // position of row offset 0, in [-2^30, 2^31)
    const int64_t p0 = (int64_t)qr0 + q_off;
    uint32_t keep = key < S ? range_bits(0, (int64_t)L - qr0) : 0u;
    const uint32_t causal = range_bits((int64_t)key - p0, 32);  // key <= p0 + o
    auto doc_bits = [&]() __attribute__((always_inline)) -> uint32_t {
        uint32_t bits = 0;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int4 d4 = *reinterpret_cast<const int4*>(doc_rows + 8 * g);
            const int dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) bits |= (dv[e] == doc_k) ? (1u << (8 * g + e)) : 0u;
        }
        return bits & range_bits(-p0, (int64_t)m.doc_len - p0);
    };
    switch (m.kind) {
    case MASK_NOOP: break;
    case MASK_CAUSAL: keep &= causal; break;
    case MASK_CAUSAL_WINDOW_SINKS: {
        // p0 + o - key < window  <=>  o < key + window - p0
        const uint32_t near = key < m.sinks ? ~0u : range_bits(0, (int64_t)key + m.window - p0);
        keep &= causal & near;
        break;
    }
    case MASK_PROGRAM: {
        if constexpr (!EXT) break;   // program masks run in the extended kernels only
        const uint32_t docb = m.uses_doc ? doc_bits() : 0u;
#pragma unroll
        for (int c = 0; c < kMaxClauses; ++c) {
            if (c >= m.prog.n_clauses) break;
            uint32_t any = 0;
#pragma unroll
            for (int l = 0; l < kMaxLiterals; ++l) {
                if (l >= m.prog.n_lits[c]) break;
                const int arg = m.prog.arg[c][l];
                switch (m.prog.kind[c][l]) {
                case PRED_CAUSAL: any |= causal; break;
                case PRED_WINDOW: any |= range_bits(0, (int64_t)key + arg - p0); break;
                case PRED_KV_LT: any |= key < arg ? ~0u : 0u; break;
                case PRED_CHUNK: {                                      // p in key's chunk
                    const int64_t lo = (int64_t)floor_div(key, arg) * arg;
                    any |= range_bits(lo - p0, lo + arg - p0);
                    break;
                }
                case PRED_STRIDE: {                                     // o = key - p0 (mod arg)
                    // 32-bit residues (key >= 0, -2^30 <= p0 < 2^31): key - p0
                    // itself may not fit in 32 bits
                    int p0m = p0i % arg;
                    if (p0m < 0) p0m += arg;
                    int rm = key % arg - p0m;
                    if (rm < 0) rm += arg;
                    uint32_t bits = 0;
                    if (arg >= 32) bits = rm < 32 ? 1u << rm : 0u;
                    else
                        for (int o = rm; o < 32; o += arg) bits |= 1u << o;
                    any |= bits;
                    break;
                }
                case PRED_DOC: any |= docb; break;
                default: any |= hq < arg ? ~0u : 0u; break;             // h < arg
                }
            }
            keep &= any;
        }
        break;
    }
    default: keep &= causal & doc_bits(); break;   // DOC_CAUSAL
    }
    return keep;
}

// fp32: O^T += X^T P over rows [kb2*32, kb2*32 + 32) of a row-major padded
// tile X (rows = the contracted index).  Lane (column c = lane & 31, half hf)
// supplies P for row acc_row(r, hf) at step r, so the A operand is X[that
// row][32*db + lane & 31]: consecutive lanes read consecutive floats.
template <int D>
__device__ __forceinline__ void xtp_f32(f32x16_t (&o)[D / 32], const float (&p)[16], const float* __restrict__ X,
                                        int kb2, int lane) {
    constexpr int kStride = BwdTiles<float, D>::kStride;
    const int hf = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        const float* col = X + kb2 * 32 * kStride + db * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r)
            o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(col[acc_row(r, hf) * kStride], p[r], o[db], 0, 0, 0);
    }
}

// O^T += X^T P for either dtype (X a row-major tile in LDS, 32-row block kb2).
template <typename T, int D>
__device__ __forceinline__ void xtp(f32x16_t (&o)[D / 32], const float (&p)[16], const char* __restrict__ X,
                                    const LdsAddr<T, D>& la, int kb2, int lane) {
    if constexpr (sizeof(T) == 2) {
        bf16x8_t pb[2];
        pack_p(pb, p);
        pv_bf16<D>(o, pb, X, la, kb2);
    } else {
        xtp_f32<D>(o, p, reinterpret_cast<const float*>(X), kb2, lane);
    }
}

// fp32 staging of one tile's rows [row0, row0 + 64) of a slice with `rows`
// valid rows (others read as zero) into a padded LDS tile.
template <int D>
__device__ __forceinline__ void fill_tile_f32(float* __restrict__ dst, const float* __restrict__ src, int64_t sr,
                                              int row0, int rows, int tid) {
    constexpr int kChunks = D / 4;
    constexpr int kUnits = kTileN * kChunks / kThreads;
    constexpr int kStride = BwdTiles<float, D>::kStride;
    float4 v[kUnits];
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
        const int c = tid + u * kThreads;
        const int r = c / kChunks, ch = c % kChunks;
        v[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (row0 + r < rows) v[u] = *reinterpret_cast<const float4*>(src + (int64_t)(row0 + r) * sr + ch * 4);
    }
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
        const int c = tid + u * kThreads;
        const int r = c / kChunks, ch = c % kChunks;
        *reinterpret_cast<float4*>(dst + r * kStride + ch * 4) = v[u];
    }
}

// Walks n tiles through a two-buffer LDS ring.  desc(t, masked) gives the
// first row of tile t and whether its tile is partial; issue(buffer, row0)
// starts filling ring buffer 0 or 1 (bf16: LDS-DMA, asynchronous; fp32:
// through registers, done on return); compute(buf, row0, masked) consumes a
// published buffer.  Per tile: wait for this wave's loads, barrier (publishes
// the tile and frees the buffer computed last), refill that buffer with the
// next tile, compute.
template <bool DMA, class Desc, class Issue, class Compute>
__device__ __forceinline__ void walk_ring(int n, Desc&& desc, Issue&& issue, Compute&& compute, const char* lds,
                                          int buf_bytes) {
    if (n <= 0) return;
    int row[2] = {0, 0};
    bool msk[2] = {false, false};
    row[0] = desc(0, msk[0]);
    issue(std::integral_constant<int, 0>{}, row[0]);
    auto step = [&](auto bc, int t) __attribute__((always_inline)) {
        constexpr int B = decltype(bc)::value;
        if constexpr (DMA) {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            __builtin_amdgcn_s_barrier();
        } else {
            __syncthreads();
        }
        if (t + 1 < n) {
            row[1 - B] = desc(t + 1, msk[1 - B]);
            issue(std::integral_constant<int, 1 - B>{}, row[1 - B]);
        }
        compute(lds + B * buf_bytes, row[B], msk[B]);
    };
    for (int t = 0; t < n; t += 2) {
        step(std::integral_constant<int, 0>{}, t);
        if (t + 1 < n) step(std::integral_constant<int, 1>{}, t + 1);
    }
    // every wave is done with the ring before the LDS is reused
    __syncthreads();
}

// ------------------------------------------------------------------ row pass
// lse2 = lse * log2(e) (+inf for rows with no visible key and padding rows)
// and D_i = dout_i . out_i, for rows [0, Lp) of every (batch, query head).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attn_bwd_rows(BwdArgs a) {
    constexpr int kChunk = 16 / (int)sizeof(T);
    constexpr int kLanes = D / kChunk;                 // lanes per row
    constexpr int kRowsPerBlock = kThreads / kLanes;
    const int64_t n_rows = (int64_t)a.B * a.Hq * a.Lp;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanes;
    const int c = threadIdx.x % kLanes;
    const bool in = row < n_rows;
    const int64_t bh = in ? row / a.Lp : 0;
    const int r = in ? (int)(row % a.Lp) : a.Lp;
    float acc = 0.0f;
    if (r < a.L) {
        const int64_t off = (bh * a.L + r) * D + c * kChunk;
        const uint4 o4 = *reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(a.out) + off);
        const uint4 d4 = *reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(a.dout) + off);
        if constexpr (sizeof(T) == 2) {
            const bf16x8_t ov = __builtin_bit_cast(bf16x8_t, o4), dv = __builtin_bit_cast(bf16x8_t, d4);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)ov[e], (float)dv[e], acc);
        } else {
            acc = __uint_as_float(o4.x) * __uint_as_float(d4.x);
            acc = __builtin_fmaf(__uint_as_float(o4.y), __uint_as_float(d4.y), acc);
            acc = __builtin_fmaf(__uint_as_float(o4.z), __uint_as_float(d4.z), acc);
            acc = __builtin_fmaf(__uint_as_float(o4.w), __uint_as_float(d4.w), acc);
        }
    }
#pragma unroll
    for (int m = kLanes / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m);
    if (in && c == 0) {
        float l2 = __builtin_inff();
        if (r < a.L) {
            const float lse = a.lse[bh * a.L + r];
            if (lse > kNegInf) l2 = lse * kLog2e;
        }
        a.ws_lse2[row] = l2;
        a.ws_dsum[row] = r < a.L ? acc : 0.0f;
    }
}

// Position of query row 0 and the filled key length of batch b: the mask's
// per-batch arrays when it carries them (values clamped as in the forward),
// else its scalar offset and the capacity S.
__device__ __forceinline__ int batch_q_offset(const MaskArgs& m, int b) {
    return m.q_offsets != nullptr ? min(max(scalar_load(m.q_offsets + b), -(1 << 30)), 1 << 30) : m.q_offset;
}
__device__ __forceinline__ int batch_kv_len(const MaskArgs& m, int b, int S) {
    return m.kv_lens != nullptr ? min(max(scalar_load(m.kv_lens + b), 0), S) : S;
}

// Where the K/V rows of logical keys [kv0, kv0 + 64) of batch b and K/V
// head hkv live: the head slice of a contiguous cache, or the page holding
// them in a paged pool (a page holds whole 64-key tiles).  base points at
// row 0 of that slice or page, row0 is kv0's row in it and rows bounds the
// valid rows: keys at or past the batch's filled length S_b read as zeros,
// whatever the cache holds there.  Page-table entries are clamped into the
// pool.
struct KvSlice {
    const char* kbase;
    const char* vbase;
    int row0, rows;
};

template <typename T>
__device__ __forceinline__ KvSlice kv_slice(const BwdArgs& a, int b, int hkv, int kv0, int S_b) {
    const char* k = reinterpret_cast<const char*>(a.k);
    const char* v = reinterpret_cast<const char*>(a.v);
    KvSlice sl;
    if (a.page_table == nullptr) {
        sl.kbase = k + ((int64_t)b * a.k_sb + (int64_t)hkv * a.k_sh) * (int64_t)sizeof(T);
        sl.vbase = v + ((int64_t)b * a.v_sb + (int64_t)hkv * a.v_sh) * (int64_t)sizeof(T);
        sl.row0 = kv0;
        sl.rows = S_b;
    } else {
        // a tile of a wide KV block can start past the last page: its rows
        // are then all past S and read as zeros
        const int lp = min(kv0 >> a.page_shift, a.max_pages - 1);
        int page = scalar_load(a.page_table + (int64_t)b * a.max_pages + lp);
        page = min(max(page, 0), a.num_pages - 1);
        sl.kbase = k + ((int64_t)page * a.k_sb + (int64_t)hkv * a.k_sh) * (int64_t)sizeof(T);
        sl.vbase = v + ((int64_t)page * a.v_sb + (int64_t)hkv * a.v_sh) * (int64_t)sizeof(T);
        sl.row0 = kv0 - (lp << a.page_shift);
        sl.rows = min(1 << a.page_shift, S_b - (lp << a.page_shift));
    }
    return sl;
}

// --------------------------------------------------------- key-major pass
// Tiles of query head hq's Q-side list for KV block kvb (64-row tiles).
__device__ __forceinline__ int bwd_head_tiles(const BwdArgs& a, int b, int hq, int kvb) {
    const int bm_b = a.Bm > 1 ? b : 0, bm_h = a.Hm > 1 ? hq : 0;
    const int64_t col_id = ((int64_t)bm_b * a.Hm + bm_h) * a.nKB + kvb;
    const int n_part = min(max(scalar_load(a.q_num + col_id), 0), a.nQB);
    const int n_full = min(max(scalar_load(a.fq_num + col_id), 0), a.nQB - n_part);
    return (n_part + n_full) * (a.q_block / kTileN);
}

// Number of workgroups that share the key-major work of (batch b, K/V head
// hkv, KV block kvb): its tile count over the group's query heads in units of
// chunk_tiles, at most kv_splits.
__device__ __forceinline__ int bwd_key_splits(const BwdArgs& a, int b, int hkv, int kvb) {
    if (a.kv_splits <= 1) return 1;
    int n = 0;
    for (int g = 0; g < a.group; ++g) n += bwd_head_tiles(a, b, hkv * a.group + g, kvb);
    return min(max((n + a.chunk_tiles - 1) / a.chunk_tiles, 1), a.kv_splits);
}

// Most workgroups that share one 64-key column (the host's bwd_kv_splits
// caps the split count at this; launch_bwd_passes rejects more).
constexpr int kBwdMaxSplits = 4;

// fp32 partial sums of split `split` of 64-key column `col` (bh * per_bh + kt):
// 64 x D for dk, then 64 x D for dv.
__device__ __forceinline__ float* bwd_partial(const BwdArgs& a, int split, int col, int D) {
    const int64_t cols = (int64_t)a.B * a.Hkv * a.nKB * (a.kv_block / kTileN);
    return a.ws_part + ((int64_t)split * cols + col) * (2 * 64 * (int64_t)D);
}

template <typename T, int D> struct DkdvLds {
    static constexpr int kMergeBytes = 2 * 64 * D * 4;
    static constexpr int value =
        2 * BwdTiles<T, D>::kBufBytes > kMergeBytes ? 2 * BwdTiles<T, D>::kBufBytes : kMergeBytes;
};

template <typename T, int D, int SCORE, bool EXT>
__device__ __forceinline__ void dkdv_body(const BwdArgs& a, char* lds, lds_char_t* lds3, int block) {
    using G = BwdTiles<T, D>;
    constexpr bool kDma = sizeof(T) == 2;

    // Work item (K/V head slice bh, 64-key tile kt) and split of its Q-side
    // tile sequence.  Workgroup i runs on XCD i % 8: when the items split
    // evenly, each XCD takes whole K/V heads (their Q / dO tiles then stay in
    // one L2) and walks them lowest key tile first (under causal-type masks it
    // has the longest Q list).
    const int subs = a.kv_block / kTileN;
    const int per_bh = a.nKB * subs;
    const int BH = a.B * a.Hkv;
    const int items = BH * per_bh;
    const int split = block / items;
    const int n = block % items;
    int bh, kt;
    if (items % 8 == 0 && (items / 8) % per_bh == 0) {
        const int hpx = items / 8 / per_bh, k = n >> 3;
        kt = k / hpx;
        bh = (n & 7) * hpx + k % hpx;
    } else {
        kt = n / BH;
        bh = n % BH;
    }
    const int b = bh / a.Hkv, hkv = bh % a.Hkv;
    const int q_off = batch_q_offset(a.mask, b), S_b = batch_kv_len(a.mask, b, a.S);
    const int kvb = kt / subs;
    const int kv0 = kt * kTileN;
    // Splits past the ones this column needs have no work: leave before the
    // K/V rows are loaded (and, at head dim 128, partly spilled to scratch).
    // Only split launches have such workgroups; without splits the count is
    // taken below, after the loads are issued.
    if (a.kv_splits > 1 && split >= bwd_key_splits(a, b, hkv, kvb)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), hf = lane >> 5;
    const int kh = wave & 1, qh = wave >> 1;
    const int key = kv0 + 32 * kh + (lane & 31);
    const bool key_ok = key < a.S;
    const bool with_doc = a.mask.uses_doc != 0;

    // this workgroup's 64 keys lie in one slice or page; keys past the
    // batch's filled length load as zeros (and the mask hides them)
    const KvSlice ksl = kv_slice<T>(a, b, hkv, kv0, S_b);
    const int krow = ksl.row0 + key - kv0;
    QRegs<T, D> kr, vr;
    load_q<T, D>(kr, reinterpret_cast<const T*>(ksl.kbase) + (int64_t)krow * a.k_sr, key < S_b, hf);
    load_q<T, D>(vr, reinterpret_cast<const T*>(ksl.vbase) + (int64_t)krow * a.v_sr, key < S_b, hf);
    const int doc_k = (with_doc && key_ok) ? __ldg(a.mask.doc_id + key) : -3;

    f32x16_t dk[D / 32], dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        dk[db] = f32x16_t{};
        dv[db] = f32x16_t{};
    }
    // bf16 LDS operand offsets with this wave's query half folded in
    const LdsAddr<T, D> la = [&] {
        if constexpr (sizeof(T) == 2) return lds_addr_bf16<D>(lane, qh);
        else return LdsAddr<T, D>{};
    }();
    const int kb2 = sizeof(T) == 2 ? 0 : qh;
    const int qsubs = a.q_block / kTileN;

    // The column's tiles over all query heads of the group, as one sequence;
    // a long one is cut into up to kv_splits contiguous ranges of about
    // chunk_tiles tiles, one per workgroup (their partial sums are added in
    // split order by attn_bwd_dkdv_reduce).
    const int nch = bwd_key_splits(a, b, hkv, kvb);
    if (split >= nch) return;
    int n_col = 0;
    for (int g = 0; g < a.group; ++g) n_col += bwd_head_tiles(a, b, hkv * a.group + g, kvb);
    const int t_lo = (int)((int64_t)n_col * split / nch), t_hi = (int)((int64_t)n_col * (split + 1) / nch);

    int base = 0;
    for (int g = 0; g < a.group; ++g) {
        const int hq = hkv * a.group + g;
        const int bm_b = a.Bm > 1 ? b : 0, bm_h = a.Hm > 1 ? hq : 0;
        const int64_t col_id = ((int64_t)bm_b * a.Hm + bm_h) * a.nKB + kvb;
        const int n_part = min(max(scalar_load(a.q_num + col_id), 0), a.nQB);
        const int n_full = min(max(scalar_load(a.fq_num + col_id), 0), a.nQB - n_part);
        const int head_tiles = (n_part + n_full) * qsubs;
        const int lo = max(t_lo - base, 0), hi = min(t_hi - base, head_tiles);
        base += head_tiles;
        if (lo >= hi) continue;
        const int n_tiles = hi - lo;
        const int* part_idx = a.q_idx + col_id * a.nQB;
        const int* full_idx = a.fq_idx + col_id * a.nQB;
        const BwdConsts bc = bwd_consts(a, hq);

        const T* qslice = reinterpret_cast<const T*>(a.q) + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh;
        const T* dslice = reinterpret_cast<const T*>(a.dout) + ((int64_t)b * a.Hq + hq) * a.L * D;
        const float* lslice = a.ws_lse2 + ((int64_t)b * a.Hq + hq) * a.Lp;
        const float* sslice = a.ws_dsum + ((int64_t)b * a.Hq + hq) * a.Lp;

        auto desc = [&](int t, bool& masked) __attribute__((always_inline)) -> int {
            t += lo;
            const int blk = qsubs == 1 ? t : t / qsubs;
            const int sub = t - blk * qsubs;
            int qb;
            if (blk < n_part) {
                qb = scalar_load(part_idx + blk);
                masked = true;
            } else {
                qb = scalar_load(full_idx + (blk - n_part));
                masked = false;
            }
            qb = min(max(qb, 0), a.nQB - 1);
            return qb * a.q_block + sub * kTileN;
        };

        auto compute = [&](const char* cur, int q0, bool masked) __attribute__((always_inline)) {
            const int qr0 = q0 + 32 * qh + 4 * hf;
            f32x16_t s, dp;
            qk2_block<T, D>(kr, vr, cur, cur + G::kTileBytes, la, kb2, lane, s, dp);
            float z[16], pg[16];
            scores2<SCORE, Precise<T>::value>(s, bc.alpha2 * (float)(key - (qr0 + q_off)), -bc.alpha2, bc, z, pg);
            if (masked) {
                const uint32_t keep =
                    mask_bits_keys<EXT>(a.mask, key, S_b, a.L, qr0, q_off, hq, doc_k,
                                        reinterpret_cast<const int*>(cur + G::kDocOffset) + 32 * qh + 4 * hf);
#pragma unroll
                for (int r = 0; r < 16; ++r) z[r] = (keep >> acc_row(r, 0)) & 1u ? z[r] : kNegInf;
            }
            // P = exp2(z - lse2) and dS = P (dP - D) g' scale, per row of the block
            const float* st = reinterpret_cast<const float*>(cur + G::kStatsOffset) + 32 * qh + 4 * hf;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const float4 l4 = *reinterpret_cast<const float4*>(st + 8 * gq);
                const float4 d4 = *reinterpret_cast<const float4*>(st + 64 + 8 * gq);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dsv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * gq + e;
                    z[r] = __builtin_amdgcn_exp2f(z[r] - lv[e]);
                    pg[r] *= z[r] * (dp[r] - dsv[e]);
                }
            }
            xtp<T, D>(dv, z, cur + G::kTileBytes, la, kb2, lane);   // dv^T += dO^T P
            xtp<T, D>(dk, pg, cur, la, kb2, lane);                 // dk^T += Q^T dS
        };

        if constexpr (kDma) {
            const int q_row_bytes = (int)(a.q_sr * (int64_t)sizeof(T));
            const int d_row_bytes = D * (int)sizeof(T);
            const __amdgpu_buffer_rsrc_t rq = slice_rsrc(qslice, q_row_bytes, a.L);
            const __amdgpu_buffer_rsrc_t rd = slice_rsrc(dslice, d_row_bytes, a.L);
            const __amdgpu_buffer_rsrc_t rl = slice_rsrc(lslice, 4, a.Lp);
            const __amdgpu_buffer_rsrc_t rs = slice_rsrc(sslice, 4, a.Lp);
            const __amdgpu_buffer_rsrc_t rdoc = slice_rsrc(a.mask.doc_id, 4, with_doc ? a.mask.doc_len : 0);
            const int oq = dma_lane_offset<D>(q_row_bytes, wave, lane);
            const int od = dma_lane_offset<D>(d_row_bytes, wave, lane);
            auto issue = [&](auto bi, int q0) __attribute__((always_inline)) {
                lds_char_t* buf = lds3 + decltype(bi)::value * G::kBufBytes;
#pragma unroll
                for (int i = 0; i < D / 32; ++i)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void_t*)(buf + (i * 4 + wave) * 1024), 16, oq,
                                                             (q0 + i * dma_rows_per_inst(D)) * q_row_bytes, 0, 0);
#pragma unroll
                for (int i = 0; i < D / 32; ++i)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rd, (lds_void_t*)(buf + G::kTileBytes + (i * 4 + wave) * 1024), 16, od,
                        (q0 + i * dma_rows_per_inst(D)) * d_row_bytes, 0, 0);
                const int l4 = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) * 4;
                if (wave == 0)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void_t*)(buf + G::kStatsOffset), 4, l4, q0 * 4,
                                                             0, 0);
                else if (wave == 1)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(buf + G::kStatsOffset + 256), 4, l4,
                                                             q0 * 4, 0, 0);
                else if (wave == 2 && with_doc) {
                    // rows whose position is outside doc_id read 0 (out of
                    // range); mask_bits_keys hides them
                    const int pos = q0 + q_off + l4 / 4;
                    const int voff = (pos >= 0 && pos < a.mask.doc_len) ? pos * 4 : 0x7ffffff0;   // doc_len < 2^29
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rdoc, (lds_void_t*)(buf + G::kDocOffset), 4, voff, 0, 0,
                                                             0);
                }
            };
            walk_ring<true>(n_tiles, desc, issue, compute, lds, G::kBufBytes);
        } else {
            auto issue = [&](auto bi, int q0) __attribute__((always_inline)) {
                char* buf = lds + decltype(bi)::value * G::kBufBytes;
                fill_tile_f32<D>(reinterpret_cast<float*>(buf), reinterpret_cast<const float*>(qslice), a.q_sr, q0,
                                 a.L, tid);
                fill_tile_f32<D>(reinterpret_cast<float*>(buf + G::kTileBytes), reinterpret_cast<const float*>(dslice),
                                 D, q0, a.L, tid);
                if (tid < 64) {
                    reinterpret_cast<float*>(buf + G::kStatsOffset)[tid] = lslice[q0 + tid];
                } else if (tid < 128) {
                    reinterpret_cast<float*>(buf + G::kStatsOffset)[tid] = sslice[q0 + tid - 64];
                } else if (tid < 192) {
                    const int pos = q0 + (tid - 128) + q_off;
                    int d = -1;
                    if (with_doc && pos >= 0 && pos < a.mask.doc_len) d = a.mask.doc_id[pos];
                    reinterpret_cast<int*>(buf + G::kDocOffset)[tid - 128] = d;
                }
            };
            walk_ring<false>(n_tiles, desc, issue, compute, lds, G::kBufBytes);
        }
    }

    // Add the two query halves (qh = 1 hands its sums to qh = 0) and store.
    float* slot = reinterpret_cast<float*>(lds) + (kh * 64 + lane) * D;
    if (qh == 1) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                *reinterpret_cast<float4*>(slot + db * 16 + 4 * g) =
                    make_float4(dk[db][4 * g], dk[db][4 * g + 1], dk[db][4 * g + 2], dk[db][4 * g + 3]);
                *reinterpret_cast<float4*>(slot + D / 2 + db * 16 + 4 * g) =
                    make_float4(dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2], dv[db][4 * g + 3]);
            }
    }
    __syncthreads();
    if (qh == 0 && key_ok) {
        if (nch == 1) {
            const int64_t orow = (((int64_t)b * a.Hkv + hkv) * a.S + key) * D;
            T* dkrow = reinterpret_cast<T*>(a.dk) + orow;
            T* dvrow = reinterpret_cast<T*>(a.dv) + orow;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 k4 = *reinterpret_cast<const float4*>(slot + db * 16 + 4 * g);
                    const float4 v4 = *reinterpret_cast<const float4*>(slot + D / 2 + db * 16 + 4 * g);
                    const int d0 = db * 32 + 8 * g + 4 * hf;
                    store_out4<T>(dkrow + d0, dk[db][4 * g] + k4.x, dk[db][4 * g + 1] + k4.y,
                                  dk[db][4 * g + 2] + k4.z, dk[db][4 * g + 3] + k4.w);
                    store_out4<T>(dvrow + d0, dv[db][4 * g] + v4.x, dv[db][4 * g + 1] + v4.y,
                                  dv[db][4 * g + 2] + v4.z, dv[db][4 * g + 3] + v4.w);
                }
        } else {
            // fp32 partial sums of this split: [key][D] for dk, then for dv
            float* part = bwd_partial(a, split, bh * per_bh + kt, D) + (key - kv0) * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 k4 = *reinterpret_cast<const float4*>(slot + db * 16 + 4 * g);
                    const float4 v4 = *reinterpret_cast<const float4*>(slot + D / 2 + db * 16 + 4 * g);
                    const int d0 = db * 32 + 8 * g + 4 * hf;
                    *reinterpret_cast<float4*>(part + d0) =
                        make_float4(dk[db][4 * g] + k4.x, dk[db][4 * g + 1] + k4.y, dk[db][4 * g + 2] + k4.z,
                                    dk[db][4 * g + 3] + k4.w);
                    *reinterpret_cast<float4*>(part + 64 * D + d0) =
                        make_float4(dv[db][4 * g] + v4.x, dv[db][4 * g + 1] + v4.y, dv[db][4 * g + 2] + v4.z,
                                    dv[db][4 * g + 3] + v4.w);
                }
        }
    }
}

template <typename T, int D, int SCORE, bool EXT>
__global__ __launch_bounds__(kThreads, (BwdOccupancy<T, D>::kKeys)) void attn_bwd_dkdv(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[DkdvLds<T, D>::value];
    dkdv_body<T, D, SCORE, EXT>(a, lds, (lds_char_t*)lds, (int)blockIdx.x);
}

// Adds the split partial sums of the columns the key-major pass cut, in
// split order, and writes dk, dv (one workgroup per 64-key column).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attn_bwd_dkdv_reduce(BwdArgs a) {
    const int subs = a.kv_block / kTileN;
    const int per_bh = a.nKB * subs;
    const int col = blockIdx.x;
    const int bh = col / per_bh, kt = col % per_bh;
    const int b = bh / a.Hkv, hkv = bh % a.Hkv;
    const int nch = bwd_key_splits(a, b, hkv, kt / subs);
    if (nch == 1) return;
    const int kv0 = kt * kTileN;
    // Each thread owns kPer float4 positions of the column.  Every partial of
    // two positions is loaded before any is added, so a thread waits on memory
    // once per pair of positions instead of once per load; the sums still run
    // in split order.  Positions past S are loaded (the partial arrays cover
    // all 64 keys of a column) but not stored.
    constexpr int kPer = 64 * D / (kThreads * 4);
    static_assert(kPer % 2 == 0, "positions go in pairs");
#pragma unroll 1
    for (int i0 = 0; i0 < kPer; i0 += 2) {
        float4 pk[2][kBwdMaxSplits], pv[2][kBwdMaxSplits];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = (threadIdx.x + (i0 + i) * kThreads) * 4;
#pragma unroll
            for (int sp = 0; sp < kBwdMaxSplits; ++sp) {
                if (sp < nch) {
                    const float* part = bwd_partial(a, sp, col, D);
                    pk[i][sp] = *reinterpret_cast<const float4*>(part + e);
                    pv[i][sp] = *reinterpret_cast<const float4*>(part + 64 * D + e);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = (threadIdx.x + (i0 + i) * kThreads) * 4;
            const int key = kv0 + e / D, d = e % D;
            if (key >= a.S) continue;
            float4 sk = make_float4(0.0f, 0.0f, 0.0f, 0.0f), sv = sk;
#pragma unroll
            for (int sp = 0; sp < kBwdMaxSplits; ++sp) {
                if (sp < nch) {
                    sk.x += pk[i][sp].x; sk.y += pk[i][sp].y; sk.z += pk[i][sp].z; sk.w += pk[i][sp].w;
                    sv.x += pv[i][sp].x; sv.y += pv[i][sp].y; sv.z += pv[i][sp].z; sv.w += pv[i][sp].w;
                }
            }
            const int64_t o = ((int64_t)bh * a.S + key) * D + d;
            store_out4<T>(reinterpret_cast<T*>(a.dk) + o, sk.x, sk.y, sk.z, sk.w);
            store_out4<T>(reinterpret_cast<T*>(a.dv) + o, sv.x, sv.y, sv.z, sv.w);
        }
    }
}

// ------------------------------------------------------- query-major pass
template <typename T, int D> struct DqLds {
    static constexpr int kMergeBytes = 2 * 64 * (D / 2) * 4;
    static constexpr int value =
        2 * BwdTiles<T, D>::kBufBytes > kMergeBytes ? 2 * BwdTiles<T, D>::kBufBytes : kMergeBytes;
};

template <typename T, int D, int SCORE, bool EXT>
__device__ __forceinline__ void dq_body(const BwdArgs& a, char* lds, lds_char_t* lds3, int block) {
    using G = BwdTiles<T, D>;
    constexpr bool kDma = sizeof(T) == 2;

    // Highest Q block first (under causal-type masks it holds the most tiles);
    // under GQA the query heads of one K/V head are kept on one XCD, as in the
    // forward.
    const int BH = a.B * a.Hq;
    const int parts = a.q_block / 64;
    const int qb = a.nQB - 1 - block / (BH * parts);
    const int rem = block % (BH * parts);
    const int part = rem / BH;
    int bh = rem % BH;
    if (a.group > 1 && BH % (8 * a.group) == 0) {
        const int xcd = bh & 7, k = bh >> 3;
        bh = (xcd + 8 * (k / a.group)) * a.group + k % a.group;
    }
    const int b = bh / a.Hq, hq = bh % a.Hq, hkv = hq / a.group;
    const int S_b = batch_kv_len(a.mask, b, a.S);
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), hf = lane >> 5;
    const int rg = wave & 1, kh = wave >> 1;
    const bool with_doc = a.mask.uses_doc != 0;

    LaneRow row;
    row.q_row = qb * a.q_block + part * 64 + rg * 32 + (lane & 31);
    row.ok = row.q_row < a.L;
    row.q_pos = row.q_row + batch_q_offset(a.mask, b);
    row.hq = hq;
    row.doc_q = lane_doc(a.mask, row.q_pos);

    const T* qbase = reinterpret_cast<const T*>(a.q) + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh;
    const T* dslice = reinterpret_cast<const T*>(a.dout) + ((int64_t)b * a.Hq + hq) * a.L * D;
    QRegs<T, D> qr, dor;
    load_q<T, D>(qr, qbase + (int64_t)row.q_row * a.q_sr, row.ok, hf);
    load_q<T, D>(dor, dslice + (int64_t)row.q_row * D, row.ok, hf);
    const int64_t srow = ((int64_t)b * a.Hq + hq) * a.Lp + min(row.q_row, a.Lp - 1);
    const float lse2 = row.ok ? a.ws_lse2[srow] : __builtin_inff();
    const float dsum = row.ok ? a.ws_dsum[srow] : 0.0f;
    const BwdConsts bc = bwd_consts(a, hq);

    const int bm_b = a.Bm > 1 ? b : 0, bm_h = a.Hm > 1 ? hq : 0;
    const int64_t row_id = ((int64_t)bm_b * a.Hm + bm_h) * a.nQB + qb;
    const int n_part = min(max(scalar_load(a.kv_num + row_id), 0), a.nKB);
    const int n_full = min(max(scalar_load(a.full_num + row_id), 0), a.nKB - n_part);
    const int ksubs = a.kv_block / kTileN;
    const int n_tiles = (n_part + n_full) * ksubs;
    const int* part_idx = a.kv_idx + row_id * a.nKB;
    const int* full_idx = a.full_idx + row_id * a.nKB;

    f32x16_t dq[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dq[db] = f32x16_t{};
    const LdsAddr<T, D> la = [&] {
        if constexpr (sizeof(T) == 2) return lds_addr_bf16<D>(lane, kh);
        else return LdsAddr<T, D>{};
    }();
    const int kb2 = sizeof(T) == 2 ? 0 : kh;

    auto desc = [&](int t, bool& masked) __attribute__((always_inline)) -> int {
        const int blk = ksubs == 1 ? t : t / ksubs;
        const int sub = t - blk * ksubs;
        int kb;
        if (blk < n_part) {
            kb = scalar_load(part_idx + blk);
            masked = true;
        } else {
            kb = scalar_load(full_idx + (blk - n_part));
            masked = false;
        }
        kb = min(max(kb, 0), a.nKB - 1);
        return kb * a.kv_block + sub * kTileN;
    };

    auto compute = [&](const char* cur, int kv0, bool masked) __attribute__((always_inline)) {
        f32x16_t s, dp;
        qk2_block<T, D>(qr, dor, cur, cur + G::kTileBytes, la, kb2, lane, s, dp);
        const int key_base = kv0 + 32 * kh + 4 * hf;
        float z[16], ds[16];
        scores2<SCORE, Precise<T>::value>(s, bc.alpha2 * (float)(key_base - row.q_pos), bc.alpha2, bc, z, ds);
        if (masked) apply_mask<EXT>(z, a.mask, kv0, S_b, row, reinterpret_cast<const int*>(cur + G::kDocOffset), kh, hf);
#pragma unroll
        for (int r = 0; r < 16; ++r) ds[r] *= __builtin_amdgcn_exp2f(z[r] - lse2) * (dp[r] - dsum);
        xtp<T, D>(dq, ds, cur, la, kb2, lane);   // dq^T += K^T dS^T
    };

    if constexpr (kDma) {
        const int k_row_bytes = (int)(a.k_sr * (int64_t)sizeof(T));
        const int v_row_bytes = (int)(a.v_sr * (int64_t)sizeof(T));
        const __amdgpu_buffer_rsrc_t rdoc = slice_rsrc(a.mask.doc_id, 4, with_doc ? a.mask.doc_len : 0);
        const int ok_ = dma_lane_offset<D>(k_row_bytes, wave, lane);
        const int ov = dma_lane_offset<D>(v_row_bytes, wave, lane);
        auto issue = [&](auto bi, int kv0) __attribute__((always_inline)) {
            lds_char_t* buf = lds3 + decltype(bi)::value * G::kBufBytes;
            const KvSlice sl = kv_slice<T>(a, b, hkv, kv0, S_b);
            const __amdgpu_buffer_rsrc_t rk = slice_rsrc(sl.kbase, k_row_bytes, sl.rows);
            const __amdgpu_buffer_rsrc_t rv = slice_rsrc(sl.vbase, v_row_bytes, sl.rows);
#pragma unroll
            for (int i = 0; i < D / 32; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(buf + (i * 4 + wave) * 1024), 16, ok_,
                                                         (sl.row0 + i * dma_rows_per_inst(D)) * k_row_bytes, 0, 0);
#pragma unroll
            for (int i = 0; i < D / 32; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(buf + G::kTileBytes + (i * 4 + wave) * 1024),
                                                         16, ov, (sl.row0 + i * dma_rows_per_inst(D)) * v_row_bytes, 0,
                                                         0);
            if (with_doc && wave == 0) {
                const int l4 = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) * 4;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rdoc, (lds_void_t*)(buf + G::kDocOffset), 4, l4, kv0 * 4, 0,
                                                         0);
            }
        };
        walk_ring<true>(n_tiles, desc, issue, compute, lds, G::kBufBytes);
    } else {
        auto issue = [&](auto bi, int kv0) __attribute__((always_inline)) {
            char* buf = lds + decltype(bi)::value * G::kBufBytes;
            const KvSlice sl = kv_slice<T>(a, b, hkv, kv0, S_b);
            fill_tile_f32<D>(reinterpret_cast<float*>(buf), reinterpret_cast<const float*>(sl.kbase), a.k_sr, sl.row0,
                             sl.rows, tid);
            fill_tile_f32<D>(reinterpret_cast<float*>(buf + G::kTileBytes), reinterpret_cast<const float*>(sl.vbase),
                             a.v_sr, sl.row0, sl.rows, tid);
            if (tid < 64) {
                const int pos = kv0 + tid;
                int d = -1;
                if (with_doc && pos < a.mask.doc_len) d = a.mask.doc_id[pos];
                reinterpret_cast<int*>(buf + G::kDocOffset)[tid] = d;
            }
        };
        walk_ring<false>(n_tiles, desc, issue, compute, lds, G::kBufBytes);
    }

    // Add the two key halves (kh = 1 hands its sums to kh = 0) and store.
    float* slot = reinterpret_cast<float*>(lds) + (rg * 64 + lane) * (D / 2);
    if (kh == 1) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<float4*>(slot + db * 16 + 4 * g) =
                    make_float4(dq[db][4 * g], dq[db][4 * g + 1], dq[db][4 * g + 2], dq[db][4 * g + 3]);
    }
    __syncthreads();
    if (kh == 0 && row.ok) {
        T* dqrow = reinterpret_cast<T*>(a.dq) + (((int64_t)b * a.Hq + hq) * a.L + row.q_row) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 x = *reinterpret_cast<const float4*>(slot + db * 16 + 4 * g);
                const int d0 = db * 32 + 8 * g + 4 * hf;
                store_out4<T>(dqrow + d0, dq[db][4 * g] + x.x, dq[db][4 * g + 1] + x.y, dq[db][4 * g + 2] + x.z,
                              dq[db][4 * g + 3] + x.w);
            }
    }
}

template <typename T, int D, int SCORE, bool EXT>
__global__ __launch_bounds__(kThreads, (BwdOccupancy<T, D>::kRows)) void attn_bwd_dq(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[DqLds<T, D>::value];
    dq_body<T, D, SCORE, EXT>(a, lds, (lds_char_t*)lds, (int)blockIdx.x);
}

// Both major passes in one launch: workgroups [0, kv_blocks) take the
// key-major work, the rest the query-major work, so query-major workgroups
// run on CUs beside key-major ones instead of after the whole key-major pass
// (the key-major kernel at head dim 128 spills and waits on memory, which the
// query-major MFMA work then fills).
template <typename T, int D> struct FusedOccupancy {
    static constexpr int value =
        BwdOccupancy<T, D>::kKeys < BwdOccupancy<T, D>::kRows ? BwdOccupancy<T, D>::kKeys : BwdOccupancy<T, D>::kRows;
};

template <typename T, int D, int SCORE, bool EXT>
__global__ __launch_bounds__(kThreads, (FusedOccupancy<T, D>::value)) void attn_bwd_fused(BwdArgs a, int kv_blocks) {
    __shared__ __attribute__((aligned(16)))
    char lds[DkdvLds<T, D>::value > DqLds<T, D>::value ? DkdvLds<T, D>::value : DqLds<T, D>::value];
    if ((int)blockIdx.x < kv_blocks) dkdv_body<T, D, SCORE, EXT>(a, lds, (lds_char_t*)lds, (int)blockIdx.x);
    else dq_body<T, D, SCORE, EXT>(a, lds, (lds_char_t*)lds, (int)blockIdx.x - kv_blocks);
}

// ------------------------------------------------------------------ launch
template <typename T, int D, int SCORE, bool EXT>
hipError_t launch_bwd_passes(const BwdArgs& a, hipStream_t stream) {
    const int64_t kv_items = (int64_t)a.B * a.Hkv * a.nKB * (a.kv_block / kTileN);
    const int64_t q_items = (int64_t)a.B * a.Hq * a.nQB * (a.q_block / 64);
    if (a.kv_splits > kBwdMaxSplits) return hipErrorInvalidValue;   // the reduce sums at most that many
    hipError_t e;
    // one launch for GQA at head dim 128 (bf16, element-rule masks); two
    // otherwise: at head dim 64 the query-major pass alone runs at a higher
    // occupancy than in the shared kernel, and without GQA or with program
    // masks the single launch measured no faster
    if constexpr (sizeof(T) == 2 && D == 128 && !EXT) {
        if (a.group > 1) {
            hipLaunchKernelGGL((attn_bwd_fused<T, D, SCORE, EXT>), dim3((unsigned)(kv_items * a.kv_splits + q_items)),
                               dim3(kThreads), 0, stream, a, (int)(kv_items * a.kv_splits));
            e = hipGetLastError();
            if (e != hipSuccess || a.kv_splits <= 1) return e;
            hipLaunchKernelGGL((attn_bwd_dkdv_reduce<T, D>), dim3((unsigned)kv_items), dim3(kThreads), 0, stream, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((attn_bwd_dkdv<T, D, SCORE, EXT>), dim3((unsigned)(kv_items * a.kv_splits)), dim3(kThreads), 0,
                       stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.kv_splits > 1) {
        hipLaunchKernelGGL((attn_bwd_dkdv_reduce<T, D>), dim3((unsigned)kv_items), dim3(kThreads), 0, stream, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((attn_bwd_dq<T, D, SCORE, EXT>), dim3((unsigned)q_items), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int D, bool EXT>
hipError_t bwd_dispatch_score(const BwdArgs& a, hipStream_t stream) {
    switch (a.score_kind) {
    case SCORE_NONE: return launch_bwd_passes<T, D, SCORE_NONE, EXT>(a, stream);
    case SCORE_SOFTCAP: return launch_bwd_passes<T, D, SCORE_SOFTCAP, EXT>(a, stream);
    case SCORE_SOFTCAP_ALIBI: return launch_bwd_passes<T, D, SCORE_SOFTCAP_ALIBI, EXT>(a, stream);
    case SCORE_ALIBI: return launch_bwd_passes<T, D, SCORE_ALIBI, EXT>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

// Row pass, then the key-major and query-major passes (program masks run in
// separately compiled extended kernels, as in the forward).
template <typename T, int D>
hipError_t bwd_dispatch(const BwdArgs& a, hipStream_t stream) {
    constexpr int kRowsPerBlock = kThreads / (D / (16 / (int)sizeof(T)));
    const int64_t rows = (int64_t)a.B * a.Hq * a.Lp;
    hipLaunchKernelGGL((attn_bwd_rows<T, D>), dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)),
                       dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.mask.kind == MASK_PROGRAM) return bwd_dispatch_score<T, D, true>(a, stream);
    return bwd_dispatch_score<T, D, false>(a, stream);
}

}  // namespace

}  // namespace flexmi
