// Block-sparse attention forward for gfx950 (CDNA4): the prefill kernel, the
// GQA-packed split-KV decode kernel and its combine pass.
//
// What is computed: the charlestar blog "FlexAttention score_mod / BlockMask",
// section on what one connection goes through (scaled score, score_mod g,
// -inf where mask_mod is false, softmax-weighted sum of values), its BlockMask
// section (empty tiles skipped, full tiles computed without the element mask
// but with score_mod, partial tiles computed then masked) and its template
// section (tiles with an online softmax, no score matrix in memory).  The
// quant67 "Causal Mask" article, section 7, describes the same running
// statistics for FlashAttention's block skipping; its section 4 the
// bottom-right alignment used for short query blocks against long caches.
//
// How it maps onto CDNA4 (design of this library, not of the pages):
//   * A workgroup of 4 wave64s owns up to 128 query rows, 32 per wave, and
//     walks the row block's partial list then its full list, 64 keys per
//     step, K and V^T tiles double-buffered in LDS.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (fp32 inputs: v_mfma_f32_32x32x2f32): each
//     lane holds one query row (lane & 31) and 16 keys per 32-key block, so
//     row reductions are in-lane plus one v_permlane32_swap.  O^T = V^T P^T
//     keeps that orientation: probabilities feed the MFMA B operand straight
//     from registers and per-row factors are per-lane scalars.
//   * The score pipeline is VALU-bound at head dim 64, so it is kept short:
//     base-2 units with log2(e) folded into the constants; the soft-cap tanh
//     is an odd polynomial on |y| <= kTanhRange with a wave-uniform exact
//     (exp + rcp) fallback for tiles holding larger scores; when the soft-cap
//     bounds every visible score (soft-cap alone, or soft-cap plus a
//     non-positive distance bias under a causal-type mask) the softmax
//     reference is a fixed constant, so there is no running max or rescale;
//     otherwise the reference moves only when a tile maximum exceeds it by
//     more than kRescaleSlack.  Mask bounds are precomputed per tile so a
//     partial tile costs a compare and a select per score.
//   * fp32 inputs take a precise path (double scores and reference, accurate
//     tanh / exp) so results stay within a few fp32 ulps of the definition.
//   * Short query blocks under GQA (decode / verify) pack the G query heads
//     that share a K/V head into the row dimension of one workgroup, so each
//     K/V byte is read once, and split the key range across workgroups; a
//     combine kernel merges the partial (numerator, reference, denominator)
//     triples with the usual log-sum-exp rule.
#pragma once

#include <type_traits>

#include "internal.hpp"

namespace flexmi {

namespace {

constexpr int kThreads = 256;     // 4 waves
constexpr int kTileN = 64;        // keys per step
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;
constexpr float kNegInf = -__builtin_inff();

// Soft-cap polynomials: odd cubic and quintic approximations of tanh(y) on
// [0, Y], minimax in absolute error, fitted on the host for each cap with the
// largest range Y <= kTanhRange whose error times the cap stays below
// kPolyScoreErr, a quarter of the 1e-3 lse tolerance (score_consts).
constexpr double kTanhRange = 0.4;
constexpr double kPolyScoreErr = 2.5e-4;



template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kChunk = 4;     // elements per 16-byte load
    static constexpr int kPadK = 4;      // K row pad (elements)
    static constexpr int kPadV = 1;      // V^T row pad (elements)
};
template <> struct Elem<__bf16> {
    static constexpr int kChunk = 8;
    static constexpr int kPadK = 8;
    static constexpr int kPadV = 4;
};

// LDS geometry of one pipeline buffer: K[key][d], V, doc ids[key].  bf16 keeps
// K and V row-major and unpadded, filled by LDS-DMA buffer loads, with the
// 16-byte chunks of each row permuted (swz below) so that neither the K
// operand reads nor the ds_read_b64_tr_b16 V reads collide in LDS banks; fp32
// stages through registers into padded K[key][d] and V^T[d][key].
template <typename T, int D> struct Tiles {
    static constexpr bool kVRowMajor = sizeof(T) == 2;
    static constexpr int kStrideK = sizeof(T) == 2 ? D : D + Elem<T>::kPadK;
    static constexpr int kStrideV = kVRowMajor ? D : kTileN + Elem<T>::kPadV;
    static constexpr int kElemsK = kTileN * kStrideK;
    static constexpr int kElemsV = kVRowMajor ? kTileN * kStrideV : D * kStrideV;
    static constexpr int kDocOffset = (kElemsK + kElemsV) * (int)sizeof(T);   // bytes
    static constexpr int kBufBytes = kDocOffset + kTileN * 4;
    static_assert(kDocOffset % 16 == 0, "doc ids must stay 16-byte aligned");
};

// Key (within a 32-key block) held by accumulator register r in lane half hf
// for a 32x32 MFMA output tile: rows (r&3) + 8*(r>>2) + 4*hf.
__device__ __forceinline__ constexpr int acc_row(int r, int hf) { return (r & 3) + 8 * (r >> 2) + 4 * hf; }
// Offset of score z[i] (i = kb2*16 + r) within the tile, lane half 0.
__device__ __forceinline__ constexpr int z_off(int i) { return (i >> 4) * 32 + acc_row(i & 15, 0); }

__device__ __forceinline__ float wave_half_max(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float wave_half_sum(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <typename T> struct Precise { static constexpr bool value = sizeof(T) == 4; };

// Load of a wave-uniform address through the constant address space, which
// the compiler serves with a scalar load (lgkmcnt), so it never waits behind
// the vector-memory counter that tracks the tile DMA.
__device__ __forceinline__ int scalar_load(const int* p) {
    return *reinterpret_cast<const __attribute__((address_space(4))) int*>(
        reinterpret_cast<uintptr_t>(p));
}

// Wave index within the workgroup as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Per-lane constants of the score rule.
struct TileConsts {
    float mul;        // NONE: scale*log2e; soft-cap exact path: 2*scale*log2e/cap
    float c2;         // cap*log2e
    float k0, k1, k2; // quintic path: g2 = acc*(k0 + k1*w + k2*w^2), w = acc^2
    float amax;       // quintic valid while |acc| <= amax
    float j0, j1;     // cubic path: g2 = acc*(j0 + j1*w)
    float amax1;      // cubic valid while |acc| <= amax1 (amax1 <= amax)
    float alpha2;     // distance-bias slope * log2e of this lane's query head
    float ref_fixed;  // fixed base-2 reference
    double scale_d, cap_d, alpha_d;
    bool want_max;    // track the row maxima (max_scores requested; the reference is then never fixed)
};

template <bool PRECISE>
__device__ __forceinline__ TileConsts make_consts(const FwdArgs& a, int hq) {
    TileConsts c;
    c.mul = a.sc.mul;
    c.c2 = a.sc.c2;
    c.k0 = a.sc.k0;
    c.k1 = a.sc.k1;
    c.k2 = a.sc.k2;
    c.amax = a.sc.amax;
    c.j0 = a.sc.j0;
    c.j1 = a.sc.j1;
    c.amax1 = a.sc.amax1;
    c.ref_fixed = a.ref_fixed;
    c.want_max = a.max_scores != nullptr;
    c.scale_d = a.scale;
    c.cap_d = a.cap;
    c.alpha_d = 0.0;
    c.alpha2 = 0.0f;
    if (a.score_kind == SCORE_SOFTCAP_ALIBI || a.score_kind == SCORE_ALIBI) {
        // slope 2^(-m (h+1) / Hq) of this query head; the bf16 path needs it in
        // fp32 only (its relative error scales the bias, so it is smallest
        // where the weights are largest), the precise path in double
        if constexpr (PRECISE) {
            c.alpha_d = exp2(-(double)a.alibi_m * (double)(hq + 1) / (double)a.Hq);
        } else {
            const float e = -(a.alibi_m * (float)(hq + 1)) / (float)a.Hq;
            c.alpha2 = __builtin_amdgcn_exp2f(e) * kLog2e;
        }
    }
    return c;
}

// Registers staged from global memory for one K/V tile (+ doc ids).
template <typename T, int D> struct Stage;
template <int D> struct Stage<__bf16, D> {
    static constexpr int kKUnits = kTileN * D / 8 / kThreads;          // 16-byte K chunks per thread
    static constexpr int kVUnits = kKUnits;                            // same for V (row-major)
    uint4 k[kKUnits];
    uint4 v[kVUnits];
    int doc;
};
template <int D> struct Stage<float, D> {
    static constexpr int kKUnits = kTileN * D / 4 / kThreads;
    static constexpr int kVUnits = kTileN * D / 4 / kThreads;
    uint4 k[kKUnits];
    uint4 v[kVUnits];
    int doc;
};

// Buffer resource over rows [0, S) of one K/V (or doc-id) slice; a tile is
// addressed with a scalar byte offset.  Loads past the end of the range return
// zeros in hardware, so tiles need no bounds branches, and a stale or corrupt
// tile index can only read zeros or rows of the same slice.  The host keeps
// every slice below 2^31 bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const void* base, int64_t row_bytes, int rows) {
    const int64_t bytes = min((int64_t)max(rows, 0) * row_bytes, (int64_t)0x7FFFFFF0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// The three descriptors of a workgroup's K/V head (doc ids only for DOC_CAUSAL).
struct SliceRsrc {
    __amdgpu_buffer_rsrc_t k, v, doc;
    int k_row_bytes, v_row_bytes;
};

// Per-thread byte offsets of the staged chunks within a tile (fixed per kernel).
template <typename T, int D> struct StageOffsets {
    int k[Stage<T, D>::kKUnits];
    int v[Stage<T, D>::kVUnits];
};

template <typename T, int D>
__device__ __forceinline__ StageOffsets<T, D> stage_offsets(int64_t k_sr, int64_t v_sr, int tid) {
    constexpr int kChunks = D / Elem<T>::kChunk;
    StageOffsets<T, D> so;
#pragma unroll
    for (int u = 0; u < Stage<T, D>::kKUnits; ++u) {
        const int c = tid + u * kThreads;
        so.k[u] = (int)((c / kChunks) * k_sr * (int64_t)sizeof(T)) + (c % kChunks) * 16;
    }
#pragma unroll
    for (int u = 0; u < Stage<T, D>::kVUnits; ++u) {
        const int c = tid + u * kThreads;
        so.v[u] = (int)((c / kChunks) * v_sr * (int64_t)sizeof(T)) + (c % kChunks) * 16;
    }
    return so;
}

// K/V layouts a kernel is compiled for: contiguous (B, Hkv, S, D) caches;
// contiguous caches with per-batch query offsets and filled lengths; paged
// pools (with or without the per-batch arrays).  Each has its own kernels, so
// a paged kernel keeps no contiguous descriptors live and a contiguous one no
// page-table state.
constexpr int kKvContig = 0, kKvPerBatch = 1, kKvPaged = 2;

// Where the K and V rows of the tile starting at logical key kv0 live: buffer
// descriptors and byte offsets.  A contiguous cache uses the head slice's
// descriptors.  A paged cache (kKvPaged kernels) sends the logical page
// kv0 >> page_shift through the batch's page-table row to a physical page of
// the pool; masks and biases keep using the logical position kv0.  As in a
// contiguous slice, rows at or past the batch's valid length S read as zeros
// (a partly filled page may hold anything there).
struct TileAddr {
    __amdgpu_buffer_rsrc_t k, v;
    int ko, vo;
};

template <typename T, int KVL>
__device__ __forceinline__ TileAddr tile_addr(const FwdArgs& a, const SliceRsrc& sr, const T* kbase, const T* vbase,
                                              int b, int kv0, int S) {
    if constexpr (KVL == kKvPaged) {
        // a tile of a wide KV block can start past the last page: its rows
        // are then all past S and read as zeros
        const int lp = min(kv0 >> a.page_shift, a.max_pages - 1);
        int page = scalar_load(a.page_table + (int64_t)b * a.max_pages + lp);
        page = min(max(page, 0), a.num_pages - 1);       // a bad entry reads another page, never outside the pool
        const int in_page = kv0 - (lp << a.page_shift);
        const int page_rows = min(1 << a.page_shift, S - (lp << a.page_shift));
        return TileAddr{slice_rsrc(kbase + (int64_t)page * a.k_sb, sr.k_row_bytes, page_rows),
                        slice_rsrc(vbase + (int64_t)page * a.v_sb, sr.v_row_bytes, page_rows), in_page * sr.k_row_bytes,
                        in_page * sr.v_row_bytes};
    }
    return TileAddr{sr.k, sr.v, kv0 * sr.k_row_bytes, kv0 * sr.v_row_bytes};
}

template <typename T, int D>
__device__ __forceinline__ void stage_load(Stage<T, D>& st, const StageOffsets<T, D>& so, const TileAddr& ta,
                                           const SliceRsrc& sr, int kv0, bool with_doc, int tid) {
#pragma unroll
    for (int u = 0; u < Stage<T, D>::kKUnits; ++u)
        st.k[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ta.k, so.k[u], ta.ko, 0));
#pragma unroll
    for (int u = 0; u < Stage<T, D>::kVUnits; ++u)
        st.v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ta.v, so.v[u], ta.vo, 0));
    if (with_doc && tid < kTileN) st.doc = __builtin_amdgcn_raw_buffer_load_b32(sr.doc, tid * 4, kv0 * 4, 0);
}

template <typename T, int D>
__device__ __forceinline__ void stage_store(const Stage<T, D>& st, char* __restrict__ buf, bool with_doc, int tid) {
    using G = Tiles<T, D>;
    constexpr int kChunks = D / Elem<T>::kChunk;
    T* Ks = reinterpret_cast<T*>(buf);
    T* Vt = Ks + G::kElemsK;
#pragma unroll
    for (int u = 0; u < Stage<T, D>::kKUnits; ++u) {
        const int c = tid + u * kThreads;
        const int key = c / kChunks, ch = c % kChunks;
        *reinterpret_cast<uint4*>(Ks + key * G::kStrideK + ch * Elem<T>::kChunk) = st.k[u];
    }
    if constexpr (G::kVRowMajor) {
#pragma unroll
        for (int u = 0; u < Stage<T, D>::kVUnits; ++u) {
            const int c = tid + u * kThreads;
            const int key = c / kChunks, ch = c % kChunks;
            *reinterpret_cast<uint4*>(Vt + key * G::kStrideV + ch * Elem<T>::kChunk) = st.v[u];
        }
    } else {
#pragma unroll
        for (int u = 0; u < Stage<T, D>::kVUnits; ++u) {
            const int c = tid + u * kThreads;
            const int key = c / kChunks, ch = c % kChunks;
            const float f[4] = {__uint_as_float(st.v[u].x), __uint_as_float(st.v[u].y),
                                __uint_as_float(st.v[u].z), __uint_as_float(st.v[u].w)};
#pragma unroll
            for (int e = 0; e < 4; ++e) Vt[(ch * 4 + e) * G::kStrideV + key] = f[e];
        }
    }
    if (with_doc && tid < kTileN) reinterpret_cast<int*>(buf + G::kDocOffset)[tid] = st.doc;
}

// bf16 tiles: 16-byte chunk c of LDS row r (a key) holds the row's chunk
// c ^ swz(r).  swz depends on r mod 16 only, so row offsets that are
// multiples of 16 stay immediate offsets.  Both patterns were checked for
// 32 and 64 LDS banks against the two read shapes: eight or sixteen lanes
// reading one chunk of consecutive rows (K operand, ds_read_b128) and four
// consecutive rows x two or four chunks (V, ds_read_b64_tr_b16).
template <int D> __device__ __forceinline__ constexpr int swz(int r) {
    return D == 64 ? ((2 * (r & 15) + ((r & 15) >> 2)) & 7) : ((5 * r) & 15);
}

// Per-lane LDS byte offsets of the bf16 operand reads within a buffer (fixed
// per lane): K operand step s of key block kb2_base (add 32 rows per further
// block), and V chunk pairs for dims 32*db.. at rows 4*hf + j/4 (+8 for hi) of
// the first 16-row group of that block.
template <typename T, int D> struct LdsAddr {};
template <int D> struct LdsAddr<__bf16, D> {
    int k[D / 16];
    int v[D / 32][2];
};

template <int D> __device__ __forceinline__ LdsAddr<__bf16, D> lds_addr_bf16(int lane, int kb2_base) {
    constexpr int kRowBytes = 2 * D, kChunkMask = D / 8 - 1;
    LdsAddr<__bf16, D> la;
    const int hf = lane >> 5, r = lane & 31;
    const int g = hf ^ swz<D>(r);
    const int blk = kb2_base * 32 * kRowBytes;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) la.k[s] = blk + r * kRowBytes + (((2 * s) ^ g) & kChunkMask) * 16;
    const int j = lane & 15;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = 4 * hf + (j >> 2) + 8 * h;
            const int c = 4 * db + 2 * ((lane >> 4) & 1) + ((j & 3) >> 1);
            la.v[db][h] = blk + row * kRowBytes + ((c ^ swz<D>(row)) & kChunkMask) * 16 + (j & 1) * 8;
        }
    return la;
}

// LDS-DMA fill of one bf16 tile: wave w's instruction i writes the 64
// contiguous chunks (i*4 + w)*64 .. +63 of the K (then V) area, lane l the
// chunk at position l; the lane loads the global chunk that the swizzle puts
// there.  Offsets are bytes within the tile's rows.
template <int D> struct DmaPlan {
    static constexpr int kInsts = D / 32;   // per wave, for K and again for V
    int k[kInsts];
    int v[kInsts];
};

template <int D>
__device__ __forceinline__ DmaPlan<D> dma_plan(int k_row_bytes, int v_row_bytes, int wave, int lane) {
    constexpr int kChunksPerRow = D / 8;
    DmaPlan<D> pl;
#pragma unroll
    for (int i = 0; i < DmaPlan<D>::kInsts; ++i) {
        const int pos = (i * 4 + wave) * 64 + lane;
        const int row = pos / kChunksPerRow;
        const int chunk = (pos % kChunksPerRow) ^ swz<D>(row);
        pl.k[i] = row * k_row_bytes + chunk * 16;
        pl.v[i] = row * v_row_bytes + chunk * 16;
    }
    return pl;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Q operand (MFMA B operand, one query row per lane & 31).
template <typename T, int D> struct QRegs;
template <int D> struct QRegs<__bf16, D> {
    bf16x8_t x[D / 16];   // step s: dims 16*s + 8*hf .. +7
};
template <int D> struct QRegs<float, D> {
    float x[D / 2];       // step s: dim hf*(D/2) + s
};

template <typename T, int D>
__device__ __forceinline__ void load_q(QRegs<T, D>& qr, const T* __restrict__ qrow, bool valid, int hf) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (valid) x = *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * hf);
            qr.x[s] = __builtin_bit_cast(bf16x8_t, x);
        }
    } else {
#pragma unroll
        for (int s = 0; s < D / 8; ++s) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (valid) x = *reinterpret_cast<const uint4*>(qrow + hf * (D / 2) + 4 * s);
            qr.x[4 * s + 0] = __uint_as_float(x.x);
            qr.x[4 * s + 1] = __uint_as_float(x.y);
            qr.x[4 * s + 2] = __uint_as_float(x.z);
            qr.x[4 * s + 3] = __uint_as_float(x.w);
        }
    }
}

// S^T block (32 keys x 32 queries) for keys [kb2*32, kb2*32+32) of the LDS tile.
template <typename T, int D>
__device__ __forceinline__ f32x16_t qk_block(const QRegs<T, D>& qr, const char* __restrict__ buf,
                                             const LdsAddr<T, D>& la, int kb2, int lane) {
    using G = Tiles<T, D>;
    const int hf = lane >> 5;
    f32x16_t acc = {};
    if constexpr (sizeof(T) == 2) {
        const char* kblk = buf + kb2 * 32 * 2 * D;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kblk + la.k[s]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr.x[s], acc, 0, 0, 0);
        }
    } else {
        const T* krow = reinterpret_cast<const T*>(buf) + (kb2 * 32 + (lane & 31)) * G::kStrideK;
#pragma unroll
        for (int s4 = 0; s4 < D / 8; ++s4) {
            const f32x4_t a4 = *reinterpret_cast<const f32x4_t*>(krow + hf * (D / 2) + 4 * s4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[e], qr.x[4 * s4 + e], acc, 0, 0, 0);
        }
    }
    return acc;
}

// Probabilities p[r] of keys kb2*32 + acc_row(r, hf) (one 32-key half), rounded
// to bf16 (nearest even) and packed as the two 8-key MFMA B operands.
__device__ __forceinline__ void pack_p(bf16x8_t (&pb)[2], const float (&p)[16]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[t][e] = (__bf16)p[8 * t + e];
}

// acc plus the sum of the rounded probabilities (two per v_dot2 against a
// pair of ones; SPLIT: in two independent chains, one register more).
template <bool SPLIT>
__device__ __forceinline__ float sum_packed(const bf16x8_t (&pb)[2], float acc) {
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    float part[2] = {acc, 0.0f};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bf16x2_t pair = {pb[t][2 * e], pb[t][2 * e + 1]};
            float& dst = SPLIT ? part[t] : part[0];
            dst = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, dst, false);
        }
    return SPLIT ? part[0] + part[1] : part[0];
}

typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

// O^T += V^T P^T over keys [kb2*32, kb2*32 + 32) (bf16).  V is row-major in LDS;
// each 16-lane group issues ds_read_b64_tr_b16 with source lane j pointing at
// row keybase + j/4, dims d0 + 4*(j%4), which hands lane j the four values
// V[keybase + e][d0 + j], e = 0..3: the A-operand slots of V^T for the keys
// whose probabilities the same lane holds in pb (keys 16t + 4hf + e and
// 16t + 8 + 4hf + e, t = 2*kb2 + tt).  The swizzled byte offsets of those
// source addresses are in la.v.
template <int D>
__device__ __forceinline__ void pv_bf16(f32x16_t (&o)[D / 32], const bf16x8_t (&pb)[2], const char* __restrict__ Vs,
                                        const LdsAddr<__bf16, D>& la, int kb2) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const char* grp = Vs + (16 * (2 * kb2 + tt)) * 2 * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(grp + la.v[db][0]));
            const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(grp + la.v[db][1]));
            const bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[tt], o[db], 0, 0, 0);
        }
    }
}

// O^T += V^T P^T over keys [kb2*32, kb2*32 + 32) (fp32; V^T in LDS).
template <int D>
__device__ __forceinline__ void pv_f32(f32x16_t (&o)[D / 32], const float (&p)[16], const float* __restrict__ Vt,
                                       int kb2, int lane) {
    using G = Tiles<float, D>;
    const int hf = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        const float* vrow = Vt + (db * 32 + (lane & 31)) * G::kStrideV + kb2 * 32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float a = vrow[acc_row(r, hf)];
            o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[r], o[db], 0, 0, 0);
        }
    }
}

// Online-softmax state for this lane's query row (both lane halves keep
// their own partial sums; they are added at the end).  ref is -inf until the
// row has seen a finite score; base 2 (float) on the bf16 path, natural units
// (double) on the precise path.  l sums the probabilities as computed (it
// gives lse); lr sums them as rounded for the PV product, and out is divided
// by lr so the weights applied to V sum to one exactly (on the fp32 path the
// two are the same).
template <bool P> struct RowState;
template <> struct RowState<false> {
    float ref;
    float l;
    float lr;
    float mx;     // largest visible score (base 2, absolute), kept only when asked for
};
template <> struct RowState<true> {
    double ref;
    float l;
    float lr;
    double mx;    // largest visible score (natural units), kept only when asked for
};

// Per-lane row description.
struct LaneRow {
    int q_row;    // query index within [0, L) (may be out of range when !ok)
    int q_pos;    // logical position q_row + q_offset
    int hq;       // query head
    int doc_q;    // document id of q_pos (DOC_CAUSAL), -2 when out of range
    bool ok;      // row exists and is written
};

// Offsets o in [lo, hi) of a 32-key half as a bit mask (bounds clamped).
__device__ __forceinline__ uint32_t range_bits(int64_t lo64, int64_t hi64) {
    const int lo = (int)max<int64_t>(lo64, 0);
    const int hi = (int)min<int64_t>(hi64, 32);
    if (hi <= lo) return 0u;
    const uint32_t upto_hi = hi >= 32 ? ~0u : ((1u << hi) - 1u);
    return upto_hi & ~((1u << lo) - 1u);
}

// Sets z[r] = -inf for the cells of half kb2 that the element mask hides
// (partial tiles only).  Bounds are folded into per-half integers so each
// score costs a compare and a select (two compares for the window rule).
template <bool EXT>
__device__ __forceinline__ void apply_mask(float (&z)[16], const MaskArgs& m, int kv0, int S, const LaneRow& row,
                                           const int* __restrict__ doc_lds, int kb2, int hf) {
    const int key_base = kv0 + 32 * kb2 + 4 * hf;
    const int in_s = S - key_base;                               // off < in_s  <=>  kv < S
    const int causal = min(row.q_pos - key_base + 1, in_s);     // off < causal <=> kv <= q_pos && kv < S
    switch (m.kind) {
    case MASK_NOOP:
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = acc_row(r, 0) < in_s ? z[r] : kNegInf;
        break;
    case MASK_CAUSAL:
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = acc_row(r, 0) < causal ? z[r] : kNegInf;
        break;
    case MASK_CAUSAL_WINDOW_SINKS: {
        const int lo = row.q_pos - m.window - key_base;          // off > lo  <=> q_pos - kv < window
        const int sk = m.sinks - key_base;                       // off < sk  <=> kv < sinks
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int off = acc_row(r, 0);
            z[r] = (off < causal && (off > lo || off < sk)) ? z[r] : kNegInf;
        }
        break;
    }
    case MASK_PROGRAM: {
        if constexpr (!EXT) break;   // program masks run in the extended kernels only
        // bit o of `keep` (o = key offset from key_base, 0..31) says whether
        // the program holds for this lane's row and that key; each predicate
        // is a range or a residue class of offsets, or a per-key document test
        uint32_t keep = range_bits(0, in_s);
        const int p = row.q_pos, kb = key_base;
        uint32_t doc_bits = 0;
        if (m.uses_doc) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int4 d4 = *reinterpret_cast<const int4*>(doc_lds + 32 * kb2 + 8 * g + 4 * hf);
                const int dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    doc_bits |= (row.doc_q != -2 && dv[e] == row.doc_q) ? (1u << acc_row(4 * g + e, 0)) : 0u;
            }
        }
#pragma unroll
        for (int c = 0; c < kMaxClauses; ++c) {
            if (c >= m.prog.n_clauses) break;
            uint32_t any = 0;
#pragma unroll
            for (int l = 0; l < kMaxLiterals; ++l) {
                if (l >= m.prog.n_lits[c]) break;
                const int arg = m.prog.arg[c][l];
                switch (m.prog.kind[c][l]) {
                case PRED_CAUSAL: any |= range_bits(0, (int64_t)p - kb + 1); break;             // j <= p
                case PRED_WINDOW: any |= range_bits((int64_t)p - kb - arg + 1, 32); break;      // p - j < arg
                case PRED_KV_LT: any |= range_bits(0, (int64_t)arg - kb); break;                // j < arg
                case PRED_CHUNK: {                                                              // same chunk as p
                    const int64_t lo = (int64_t)floor_div(p, arg) * arg;
                    any |= range_bits(lo - kb, lo + arg - kb);
                    break;
                }
                case PRED_STRIDE: {                                                             // (p - j) % arg == 0
                    int rm = (p - kb) % arg;
                    if (rm < 0) rm += arg;
                    uint32_t bits = 0;
                    if (arg >= 32) bits = rm < 32 ? 1u << rm : 0u;
                    else
                        for (int o = rm; o < 32; o += arg) bits |= 1u << o;
                    any |= bits;
                    break;
                }
                case PRED_DOC: any |= doc_bits; break;
                default: any |= row.hq < arg ? ~0u : 0u; break;                       // h < arg
                }
            }
            keep &= any;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = (keep >> acc_row(r, 0)) & 1u ? z[r] : kNegInf;
        break;
    }
    default: {
        const int lim = row.doc_q == -2 ? -1 : causal;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int4 d4 = *reinterpret_cast<const int4*>(doc_lds + 32 * kb2 + 8 * g + 4 * hf);
            const int dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g + e;
                z[r] = (acc_row(r, 0) < lim && dv[e] == row.doc_q) ? z[r] : kNegInf;
            }
        }
        break;
    }
    }
}

// One 32-key half (kb2) of a 64-key tile after QK^T: score_mod, the element
// mask on partial tiles (wave-uniform branch), softmax update, PV with the V
// tile and document ids in buf.  mid() runs between the mask and the
// exponentials, so that work placed there (QK^T of the tile's other key half)
// shares a basic block with the exponentials and PV and its MFMAs overlap
// their VALU work.
template <typename T, int D, int SCORE, bool FIXED, bool EXT, bool CUBIC_FIRST, typename Mid>
__device__ __forceinline__ void tile_update(const f32x16_t& s, const char* __restrict__ buf,
                                            const LdsAddr<T, D>& la, f32x16_t (&o)[D / 32],
                                            RowState<Precise<T>::value>& st, const TileConsts& tc,
                                            const MaskArgs& mask, bool masked, int kv0, int S, const LaneRow& row,
                                            int kb2, int kb2_lds, int lane, Mid&& mid) {
    using G = Tiles<T, D>;
    constexpr bool P = Precise<T>::value;
    using RefT = typename std::conditional<P, double, float>::type;
    const int hf = lane >> 5;
    const T* Vs = reinterpret_cast<const T*>(buf) + G::kElemsK;
    const int* doc_lds = reinterpret_cast<const int*>(buf + G::kDocOffset);
    {
        float z[16];
        const RefT ref_sub = FIXED ? (RefT)tc.ref_fixed : ((st.ref == (RefT)kNegInf) ? (RefT)0 : st.ref);
        const int key_base = kv0 + 32 * kb2 + 4 * hf;
        if constexpr (P) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                double g = (double)s[r] * tc.scale_d;
                if constexpr (SCORE == SCORE_SOFTCAP || SCORE == SCORE_SOFTCAP_ALIBI) g = tc.cap_d * tanh(g / tc.cap_d);
                if constexpr (SCORE == SCORE_SOFTCAP_ALIBI || SCORE == SCORE_ALIBI)
                    g = fma(tc.alpha_d, (double)(key_base + acc_row(r, 0) - row.q_pos), g);
                z[r] = (float)(g - ref_sub);
            }
        } else if constexpr (SCORE == SCORE_NONE) {
#pragma unroll
            for (int r = 0; r < 16; ++r) z[r] = __builtin_fmaf(s[r], tc.mul, -ref_sub);
        } else if constexpr (SCORE == SCORE_ALIBI) {
            // z = s*scale*log2e + alpha2*(kv - q_pos) - ref
            const float base = __builtin_fmaf(tc.alpha2, (float)(key_base - row.q_pos), -ref_sub);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                z[r] = __builtin_fmaf(s[r], tc.mul, __builtin_fmaf(tc.alpha2, (float)acc_row(r, 0), base));
        } else {
            // base-2 score minus reference: z = c2*tanh(y) [+ alpha2*(kv - q_pos)] - ref
            float base = -ref_sub;
            if constexpr (SCORE == SCORE_SOFTCAP_ALIBI)
                base = __builtin_fmaf(tc.alpha2, (float)(key_base - row.q_pos), base);
            float amax = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(s[r]));
            // polynomial tanh (cubic or quintic), or the exact form
            // cap - 2*cap / (1 + e^{2y}) when a score of the half is out of the
            // polynomials' range (wave-uniform choice).  With CUBIC_FIRST the
            // cubic, the common case, is evaluated first in place and the other
            // forms overwrite it: the compiler then does not give the cubic a
            // branch of its own, whose results it copies (eight v_mov_b64 per
            // half); the empty asm keeps it from sinking the cubic back into one.
            // Kernels with less register room keep the plain three-way branch.
            if constexpr (CUBIC_FIRST) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = base;
                    if constexpr (SCORE == SCORE_SOFTCAP_ALIBI) x = __builtin_fmaf(tc.alpha2, (float)acc_row(r, 0), base);
                    const float acc = s[r];
                    const float poly = __builtin_fmaf(acc * acc, tc.j1, tc.j0);
                    z[r] = __builtin_fmaf(acc, poly, x);
                    asm volatile("" : "+v"(z[r]));
                }
            }
            if (!__any(amax > tc.amax1)) {
                if constexpr (!CUBIC_FIRST) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float x = base;
                        if constexpr (SCORE == SCORE_SOFTCAP_ALIBI)
                            x = __builtin_fmaf(tc.alpha2, (float)acc_row(r, 0), base);
                        const float acc = s[r];
                        const float poly = __builtin_fmaf(acc * acc, tc.j1, tc.j0);
                        z[r] = __builtin_fmaf(acc, poly, x);
                    }
                }
            } else if (!__any(amax > tc.amax)) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = base;
                    if constexpr (SCORE == SCORE_SOFTCAP_ALIBI) x = __builtin_fmaf(tc.alpha2, (float)acc_row(r, 0), base);
                    const float acc = s[r];
                    const float w = acc * acc;
                    const float poly = __builtin_fmaf(w, __builtin_fmaf(w, tc.k2, tc.k1), tc.k0);
                    z[r] = __builtin_fmaf(acc, poly, x);
                }
            } else {
                const float base_c = base + tc.c2;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = base_c;
                    if constexpr (SCORE == SCORE_SOFTCAP_ALIBI) x = __builtin_fmaf(tc.alpha2, (float)acc_row(r, 0), base_c);
                    const float e2y = __builtin_amdgcn_exp2f(s[r] * tc.mul);
                    const float rcp = __builtin_amdgcn_rcpf(1.0f + e2y);
                    z[r] = __builtin_fmaf(-2.0f * tc.c2, rcp, x);
                }
            }
        }
        if (masked) apply_mask<EXT>(z, mask, kv0, S, row, doc_lds, kb2, hf);

        if constexpr (!FIXED) {
            // Move the reference when the half's max exceeds it by more than the
            // slack, or when the row sees its first finite score (wave-uniform).
            float tmax = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, z[r]);
            tmax = wave_half_max(tmax);
            if (EXT && tc.want_max && tmax != kNegInf) {
                const RefT m = ref_sub + (RefT)tmax;
                st.mx = st.mx > m ? st.mx : m;
            }
            const bool need = (tmax > kRescaleSlack) || (st.ref == (RefT)kNegInf && tmax != kNegInf);
            if (__builtin_expect(__any(need), 0)) {
                const RefT tile_max_abs = ref_sub + (RefT)tmax;
                const RefT new_ref = st.ref > tile_max_abs ? st.ref : tile_max_abs;
                const RefT new_sub = (new_ref == (RefT)kNegInf) ? (RefT)0 : new_ref;
                float factor;
                if constexpr (P) factor = (st.ref == (RefT)kNegInf) ? 0.0f : expf((float)(st.ref - new_ref));
                else factor = (st.ref == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(st.ref - new_ref);
                const float shift = (float)(new_sub - ref_sub);
                st.l *= factor;
                st.lr *= factor;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) o[db] *= factor;
                st.ref = new_ref;
#pragma unroll
                for (int r = 0; r < 16; ++r) z[r] -= shift;
            }
        }

        mid();
        float lsum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if constexpr (P) z[r] = expf(z[r]);
            else z[r] = __builtin_amdgcn_exp2f(z[r]);
            if constexpr (!CUBIC_FIRST) lsum += z[r];
        }
        if constexpr (CUBIC_FIRST) {
            // pairwise sum: fifteen adds in four dependent steps
            float t[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) t[r] = z[2 * r] + z[2 * r + 1];
#pragma unroll
            for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
                for (int r = 0; r < w; ++r) t[r] += t[r + w];
            lsum = t[0];
        }
        st.l += lsum;
        if constexpr (P) {
            st.lr += lsum;
            pv_f32<D>(o, z, Vs, kb2, lane);
        } else {
            bf16x8_t pb[2];
            pack_p(pb, z);
            st.lr = sum_packed<CUBIC_FIRST>(pb, st.lr);
            pv_bf16<D>(o, pb, reinterpret_cast<const char*>(Vs), la, kb2_lds);
        }
    }
}

// One 32-key half (kb2) of a 64-key tile: QK^T, then tile_update.  The two
// halves of every tile go to two different waves that own the same query
// rows (their partial states are merged once at the end, merge_key_halves),
// or both to one wave (process_tile_pair).
template <typename T, int D, int SCORE, bool FIXED, bool EXT>
__device__ __forceinline__ void process_tile(const QRegs<T, D>& qr, const char* __restrict__ buf,
                                             const LdsAddr<T, D>& la, f32x16_t (&o)[D / 32],
                                             RowState<Precise<T>::value>& st, const TileConsts& tc,
                                             const MaskArgs& mask, bool masked, int kv0, int S, const LaneRow& row,
                                             int kb2, int kb2_lds, int lane) {
    const f32x16_t s = qk_block<T, D>(qr, buf, la, sizeof(T) == 2 ? kb2_lds : kb2, lane);
    tile_update<T, D, SCORE, FIXED, EXT, false>(s, buf, la, o, st, tc, mask, masked, kv0, S, row, kb2, kb2_lds, lane,
                                                [] {});
}

// Both 32-key halves of a 64-key tile in one wave: QK^T of the second half is
// issued inside the first half's exponential/PV block.
template <typename T, int D, int SCORE, bool FIXED, bool EXT>
__device__ __forceinline__ void process_tile_pair(const QRegs<T, D>& qr, const char* __restrict__ buf,
                                                  const LdsAddr<T, D>& la, f32x16_t (&o)[D / 32],
                                                  RowState<Precise<T>::value>& st, const TileConsts& tc,
                                                  const MaskArgs& mask, bool masked, int kv0, int S,
                                                  const LaneRow& row, int lane) {
    constexpr bool kCubicFirst = D == 64 && FIXED && !EXT;
    const f32x16_t s0 = qk_block<T, D>(qr, buf, la, 0, lane);
    f32x16_t s1;
    tile_update<T, D, SCORE, FIXED, EXT, kCubicFirst>(s0, buf, la, o, st, tc, mask, masked, kv0, S, row, 0, 0, lane,
                                                      [&] { s1 = qk_block<T, D>(qr, buf, la, 1, lane); });
    tile_update<T, D, SCORE, FIXED, EXT, kCubicFirst>(s1, buf, la, o, st, tc, mask, masked, kv0, S, row, 1, 1, lane,
                                                      [] {});
}

// True when a wave whose 32 rows start at query position q_lo sees no key of
// the 32-key half starting at k0 (wave-uniform and conservative): every key
// is at or past S, above every row's diagonal under a causal-type mask, or
// (window + sinks) outside every row's window and past the sinks.  Skipping
// such a half of a partial tile is exact: all its weights are zero.
__device__ __forceinline__ bool half_dead(const MaskArgs& m, int k0, int S, int q_lo) {
    if (k0 >= S) return true;
    const bool causal_kind =
        m.kind == MASK_CAUSAL || m.kind == MASK_CAUSAL_WINDOW_SINKS || m.kind == MASK_DOC_CAUSAL;
    if (causal_kind && k0 > q_lo + 31) return true;
    return m.kind == MASK_CAUSAL_WINDOW_SINKS && k0 >= m.sinks && q_lo - (k0 + 31) >= m.window;
}

// Calls f(integral_constant<int, I>) for I = FIRST .. LAST - 1.
template <int FIRST, int LAST> struct Unroll {
    template <class F> __device__ __forceinline__ static void run(F&& f) {
        f(std::integral_constant<int, FIRST>{});
        Unroll<FIRST + 1, LAST>::run(f);
    }
};
template <int LAST> struct Unroll<LAST, LAST> {
    template <class F> __device__ __forceinline__ static void run(F&&) {}
};

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// bf16 tile walk: tiles arrive by LDS-DMA (no staging registers) into a ring of
// STAGES buffers, STAGES - 1 tiles ahead of the one being computed; the loop is
// unrolled over the ring so every LDS operand address is a per-lane constant
// plus an immediate.  Per tile: wait for this wave's part of the tile, barrier
// (publishes the tile and frees the buffer computed last), refill that buffer
// with the tile STAGES - 1 ahead, compute.
template <int D, int SCORE, bool FIXED, bool KSPLIT, bool EXT, int STAGES, int KVL>
__device__ __forceinline__ void attend_rows_dma(const FwdArgs& a, const __bf16* __restrict__ kbase,
                                                const __bf16* __restrict__ vbase, const QRegs<__bf16, D>& qr,
                                                const int* __restrict__ part_idx, int n_part,
                                                const int* __restrict__ full_idx, int tile_lo, int tile_hi,
                                                const TileConsts& tc, const LaneRow& row, bool wave_active, int kh,
                                                f32x16_t (&o)[D / 32], RowState<false>& st, char* lds, int S, int b,
                                                int rot = 0) {
    using G = Tiles<__bf16, D>;
    static_assert(STAGES >= 2, "at least double buffering");
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = wave_id();
    const int sub_per_block = a.kv_block / kTileN;
    const bool with_doc = a.mask.uses_doc != 0;

    // tiles are walked starting `rot` tiles into the range, wrapping around
    // (any order gives the same result up to rounding)
    const int n_range = tile_hi - tile_lo;
    auto tile_kv0 = [&](int t, bool& masked) -> int {
        if (rot != 0) {
            int u = t - tile_lo + rot;
            if (u >= n_range) u -= n_range;
            t = tile_lo + u;
        }
        const int blk = sub_per_block == 1 ? t : t / sub_per_block;
        const int sub = t - blk * sub_per_block;
        int kb;
        if (blk < n_part) { kb = scalar_load(part_idx + blk); masked = true; }
        else { kb = scalar_load(full_idx + (blk - n_part)); masked = false; }
        return kb * a.kv_block + sub * kTileN;
    };

    if (tile_lo >= tile_hi) return;
    SliceRsrc sr;
    sr.k_row_bytes = (int)(a.k_sr * (int64_t)sizeof(__bf16));
    sr.v_row_bytes = (int)(a.v_sr * (int64_t)sizeof(__bf16));
    sr.k = slice_rsrc(kbase, sr.k_row_bytes, S);
    sr.v = slice_rsrc(vbase, sr.v_row_bytes, S);
    sr.doc = slice_rsrc(a.mask.doc_id, 4, with_doc ? a.mask.doc_len : 0);
    const DmaPlan<D> pl = dma_plan<D>(sr.k_row_bytes, sr.v_row_bytes, wave, lane);
    // key-split waves read only their own key half: fold it into the offsets
    const LdsAddr<__bf16, D> la = lds_addr_bf16<D>(lane, KSPLIT ? kh : 0);

    // K and V instructions per wave and tile (wave 0 adds one doc-id load).
    constexpr int kPerTile = 2 * DmaPlan<D>::kInsts;
    auto issue = [&](char* buf, int kv0) {
        const TileAddr ta = tile_addr<__bf16, KVL>(a, sr, kbase, vbase, b, kv0, S);
#pragma unroll
        for (int i = 0; i < DmaPlan<D>::kInsts; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ta.k, (lds_void_t*)(buf + (i * 4 + wave) * 1024), 16, pl.k[i],
                                                     ta.ko, 0, 0);
#pragma unroll
        for (int i = 0; i < DmaPlan<D>::kInsts; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ta.v, (lds_void_t*)(buf + G::kElemsK * 2 + (i * 4 + wave) * 1024),
                                                     16, pl.v[i], ta.vo, 0, 0);
        if (with_doc && wave == 0) {
            // lane id from mbcnt: cheap to recompute, so it is not kept live
            const int l4 = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) * 4;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(sr.doc, (lds_void_t*)(buf + G::kDocOffset), 4, l4, kv0 * 4, 0, 0);
        }
    };

    // first query position of this wave's rows (lane 0 holds the lowest row)
    const int q_lo = __builtin_amdgcn_readfirstlane(row.q_pos);

    // Tile descriptors of the ring (static indices after unrolling).
    int ring_kv0[STAGES];
    bool ring_masked[STAGES];
#pragma unroll
    for (int i = 0; i < STAGES - 1; ++i) {
        ring_masked[i] = false;
        ring_kv0[i] = 0;
        if (tile_lo + i < tile_hi) {
            ring_kv0[i] = tile_kv0(tile_lo + i, ring_masked[i]);
            issue(lds + i * G::kBufBytes, ring_kv0[i]);
        }
    }
    auto step = [&](auto bufc, int t) {
        constexpr int B = decltype(bufc)::value;
        constexpr int R = (B + STAGES - 1) % STAGES;     // buffer computed last, refilled now
        // Tiles t+1 .. t+STAGES-2 may stay in flight (DMA completes in order;
        // wave 0's doc loads make it wait a little longer than needed).
        if (t + STAGES - 2 < tile_hi) __builtin_amdgcn_s_waitcnt(vmcnt_imm((STAGES - 2) * kPerTile));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        // A bare barrier: the waves' LDS reads of the buffer refilled below were
        // consumed (waited on) before they got here, and a fenced barrier would
        // also drain the DMA still in flight for later tiles.
        __builtin_amdgcn_s_barrier();
        if (t + STAGES - 1 < tile_hi) {
            ring_kv0[R] = tile_kv0(t + STAGES - 1, ring_masked[R]);
            issue(lds + R * G::kBufBytes, ring_kv0[R]);
        }
        const char* cur = lds + B * G::kBufBytes;
        const int kv0 = ring_kv0[B];
        const bool masked = ring_masked[B];
        if (wave_active) {
            // Halves of a partial tile that none of this wave's rows can see are
            // skipped (element-rule masks; mask programs keep the plain walk,
            // where the test only cost time).
            const bool may_skip = !EXT && masked;
            if constexpr (KSPLIT) {
                if (!(may_skip && half_dead(a.mask, kv0 + 32 * kh, S, q_lo)))
                    process_tile<__bf16, D, SCORE, FIXED, EXT>(qr, cur, la, o, st, tc, a.mask, masked, kv0, S, row,
                                                              kh, 0, lane);
            } else {
                // both halves at once: a lone-half path would cost registers in the common case
                if (!(may_skip && half_dead(a.mask, kv0, S, q_lo) && half_dead(a.mask, kv0 + 32, S, q_lo)))
                    process_tile_pair<__bf16, D, SCORE, FIXED, EXT>(qr, cur, la, o, st, tc, a.mask, masked, kv0, S,
                                                                    row, lane);
            }
        }
    };
    for (int t = tile_lo; t < tile_hi; t += STAGES) {
        Unroll<0, STAGES>::run([&](auto ic) {
            constexpr int I = decltype(ic)::value;
            if (t + I < tile_hi) step(ic, t + I);
        });
    }
    // every wave is done with the ring before the caller reuses the LDS
    __syncthreads();
}

// Walk tiles [tile_lo, tile_hi) of one row block's lists: partial tiles (masked)
// first, then full tiles.  All waves load; active waves compute either key half
// kh of every tile (KSPLIT) or both halves.
template <typename T, int D, int SCORE, bool FIXED, bool KSPLIT, bool EXT, int STAGES = 2, int KVL = kKvContig>
__device__ __forceinline__ void attend_rows(const FwdArgs& a, const T* __restrict__ kbase, const T* __restrict__ vbase,
                                            const QRegs<T, D>& qr, const int* __restrict__ part_idx, int n_part,
                                            const int* __restrict__ full_idx, int tile_lo, int tile_hi,
                                            const TileConsts& tc, const LaneRow& row, bool wave_active, int kh,
                                            f32x16_t (&o)[D / 32], RowState<Precise<T>::value>& st, char* lds, int S,
                                            int b, int rot = 0) {
    if constexpr (sizeof(T) == 2) {
        attend_rows_dma<D, SCORE, FIXED, KSPLIT, EXT, STAGES, KVL>(a, kbase, vbase, qr, part_idx, n_part, full_idx, tile_lo,
                                                         tile_hi, tc, row, wave_active, kh, o, st, lds, S, b, rot);
    } else {
    using G = Tiles<T, D>;
    const LdsAddr<T, D> la{};
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int sub_per_block = a.kv_block / kTileN;
    const bool with_doc = a.mask.uses_doc != 0;

    auto tile_kv0 = [&](int t, bool& masked) -> int {
        const int blk = sub_per_block == 1 ? t : t / sub_per_block;
        const int sub = t - blk * sub_per_block;
        int kb;
        if (blk < n_part) { kb = scalar_load(part_idx + blk); masked = true; }
        else { kb = scalar_load(full_idx + (blk - n_part)); masked = false; }
        return kb * a.kv_block + sub * kTileN;
    };

    if (tile_lo >= tile_hi) return;
    const StageOffsets<T, D> so = stage_offsets<T, D>(a.k_sr, a.v_sr, tid);
    SliceRsrc sr;
    sr.k_row_bytes = (int)(a.k_sr * (int64_t)sizeof(T));
    sr.v_row_bytes = (int)(a.v_sr * (int64_t)sizeof(T));
    sr.k = slice_rsrc(kbase, sr.k_row_bytes, S);
    sr.v = slice_rsrc(vbase, sr.v_row_bytes, S);
    sr.doc = slice_rsrc(a.mask.doc_id, 4, with_doc ? a.mask.doc_len : 0);
    Stage<T, D> stage;
    bool masked;
    int kv0 = tile_kv0(tile_lo, masked);
    stage_load<T, D>(stage, so, tile_addr<T, KVL>(a, sr, kbase, vbase, b, kv0, S), sr, kv0, with_doc, tid);
    stage_store<T, D>(stage, lds, with_doc, tid);
    __syncthreads();
    for (int t = tile_lo; t < tile_hi; ++t) {
        const int buf = (t - tile_lo) & 1;
        bool next_masked = false;
        int next_kv0 = 0;
        const bool has_next = t + 1 < tile_hi;
        if (has_next) {
            next_kv0 = tile_kv0(t + 1, next_masked);
            stage_load<T, D>(stage, so, tile_addr<T, KVL>(a, sr, kbase, vbase, b, next_kv0, S), sr, next_kv0, with_doc,
                             tid);
        }
        const char* cur = lds + buf * G::kBufBytes;
        if (wave_active) {
            if constexpr (KSPLIT) {
                process_tile<T, D, SCORE, FIXED, EXT>(qr, cur, la, o, st, tc, a.mask, masked, kv0, S, row, kh, kh, lane);
            } else {
                process_tile<T, D, SCORE, FIXED, EXT>(qr, cur, la, o, st, tc, a.mask, masked, kv0, S, row, 0, 0, lane);
                process_tile<T, D, SCORE, FIXED, EXT>(qr, cur, la, o, st, tc, a.mask, masked, kv0, S, row, 1, 1, lane);
            }
        }
        if (has_next) stage_store<T, D>(stage, lds + (buf ^ 1) * G::kBufBytes, with_doc, tid);
        __syncthreads();
        kv0 = next_kv0;
        masked = next_masked;
    }
    }
}

// Merge the two key halves of every query row: the kh = 1 wave of each row
// group hands (numerator, reference, sums) to the kh = 0 wave through LDS,
// which rescales both to the larger reference and adds them.  Called by all
// threads after the tile loop (the LDS tiles are no longer read).
template <typename T, int D, bool FIXED>
__device__ __forceinline__ void merge_key_halves(f32x16_t (&o)[D / 32], RowState<Precise<T>::value>& st, char* lds,
                                                 int rg, int kh, int lane, bool active) {
    constexpr bool P = Precise<T>::value;
    constexpr int kSlot = D / 2 + 6;       // floats per lane: numerator, reference (2), l, lr, max (2)
    float* slot = reinterpret_cast<float*>(lds) + (rg * 64 + lane) * kSlot;
    if (kh == 1 && active) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<float4*>(slot + db * 16 + 4 * g) =
                    make_float4(o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
        const double ref = (double)st.ref;
        *reinterpret_cast<double*>(slot + D / 2) = ref;
        slot[D / 2 + 2] = st.l;
        slot[D / 2 + 3] = st.lr;
        *reinterpret_cast<double*>(slot + D / 2 + 4) = (double)st.mx;
    }
    __syncthreads();
    if (kh == 0 && active) {
        const double ref_b = *reinterpret_cast<const double*>(slot + D / 2);
        const float l_b = slot[D / 2 + 2], lr_b = slot[D / 2 + 3];
        const double mx_b = *reinterpret_cast<const double*>(slot + D / 2 + 4);
        if ((double)st.mx < mx_b) st.mx = (typename std::conditional<P, double, float>::type)mx_b;
        float fa = 1.0f, fb = 1.0f;
        if constexpr (!FIXED) {
            const double ref_a = (double)st.ref;
            const double m = ref_a > ref_b ? ref_a : ref_b;
            if (m == -__builtin_inf()) {
                fa = 0.0f;
                fb = 0.0f;
            } else if constexpr (P) {
                fa = ref_a == -__builtin_inf() ? 0.0f : expf((float)(ref_a - m));
                fb = ref_b == -__builtin_inf() ? 0.0f : expf((float)(ref_b - m));
            } else {
                fa = ref_a == -__builtin_inf() ? 0.0f : __builtin_amdgcn_exp2f((float)(ref_a - m));
                fb = ref_b == -__builtin_inf() ? 0.0f : __builtin_amdgcn_exp2f((float)(ref_b - m));
            }
            st.ref = (typename std::conditional<P, double, float>::type)m;
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 v = *reinterpret_cast<const float4*>(slot + db * 16 + 4 * g);
                o[db][4 * g] = __builtin_fmaf(fb, v.x, fa * o[db][4 * g]);
                o[db][4 * g + 1] = __builtin_fmaf(fb, v.y, fa * o[db][4 * g + 1]);
                o[db][4 * g + 2] = __builtin_fmaf(fb, v.z, fa * o[db][4 * g + 2]);
                o[db][4 * g + 3] = __builtin_fmaf(fb, v.w, fa * o[db][4 * g + 3]);
            }
        st.l = __builtin_fmaf(fb, l_b, fa * st.l);
        st.lr = __builtin_fmaf(fb, lr_b, fa * st.lr);
    }
}

template <typename T> __device__ __forceinline__ void store_out4(T* dst, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store_out4<float>(float* dst, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}
template <> __device__ __forceinline__ void store_out4<__bf16>(__bf16* dst, float a, float b, float c, float d) {
    bf16x4_t v;
    v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
    *reinterpret_cast<bf16x4_t*>(dst) = v;
}

__device__ __forceinline__ int lane_doc(const MaskArgs& m, int q_pos) {
    if (!m.uses_doc) return 0;
    return (q_pos >= 0 && q_pos < m.doc_len) ? __ldg(m.doc_id + q_pos) : -2;
}

// Per-batch view of the call (paged / per-batch kernels only): the logical position of
// query row 0 and the number of valid keys of batch b, when the mask carries
// per-batch arrays (values clamped into range), and the K/V base of the head
// (a paged pool has no batch term: pages carry it).
struct BatchView {
    int q_offset;
    int S;
};

template <int KVL>
__device__ __forceinline__ BatchView batch_view(const FwdArgs& a, int b) {
    BatchView v{a.mask.q_offset, a.S};
    if constexpr (KVL != kKvContig) {
        if (a.mask.q_offsets != nullptr)
            v.q_offset = min(max(scalar_load(a.mask.q_offsets + b), -(1 << 30)), 1 << 30);
        if (a.mask.kv_lens != nullptr) v.S = min(max(scalar_load(a.mask.kv_lens + b), 0), a.S);
    }
    return v;
}

template <typename T, int KVL>
__device__ __forceinline__ const T* kv_head_base(const void* base, int64_t sb, int64_t sh, const FwdArgs& a, int b,
                                                 int hkv) {
    const int64_t off = KVL == kKvPaged ? (int64_t)hkv * sh : (int64_t)b * sb + (int64_t)hkv * sh;
    return reinterpret_cast<const T*>(base) + off;
}

// Waves per SIMD the prefill kernel is compiled for: four for bf16 key-split
// workgroups at head dim 64 (the score pipeline is VALU-bound there, so more
// waves hide MFMA and LDS latency behind each other's VALU work), otherwise
// as many as the registers of the wider tiles allow.  The extended kernels
// (mask programs, max_scores) at head dim 64 need more than the 168 registers
// of three waves and would spill, so they take two; the key-split paged and
// per-batch ones need more than the 128 of four and take three.
template <typename T, int D, bool KSPLIT, bool EXT, int KVL = kKvContig> struct PrefillOccupancy {
    static constexpr int value =
        sizeof(T) == 2 ? (D == 64 ? (KSPLIT ? (EXT ? 2 : (KVL != kKvContig ? 3 : 4)) : (EXT ? 2 : 3)) : 2) : (D == 64 ? 2 : 1);
};



// The Q block of rank j in a longest-first order of the row blocks of mask
// row 0 that keeps packed documents together.  Under a packed-document mask
// a document's row blocks have non-decreasing tile counts, so each block is
// keyed by the count at the end of its non-decreasing run (about its
// document's length) and blocks are ordered by that key, largest first, then
// by higher block index.  Long documents run first, each with its blocks
// together (they share its K/V tiles in L2), and short ones fill the tail.
// Run ends are found through a bitmap of the blocks where a run ends (one
// ballot per wave), so no thread walks a run.  The ranks are a permutation of
// 0 .. nQB-1, so exactly one block matches.  Needs nQB <= kThreads; every
// thread returns the block; uses the first 8 * nQB + 40 bytes of lds.
__device__ __forceinline__ int longest_first_block(const FwdArgs& a, int j, char* lds) {
    int* cnt = reinterpret_cast<int*>(lds);
    int* key = cnt + a.nQB;
    uint64_t* ends = reinterpret_cast<uint64_t*>(key + a.nQB);     // 8-byte aligned: nQB ints twice
    int* pick = reinterpret_cast<int*>(ends + kThreads / 64);
    const int q = threadIdx.x;
    if (q < a.nQB) cnt[q] = min(max(a.kv_num[q], 0), a.nKB) + min(max(a.full_num[q], 0), a.nKB);
    __syncthreads();
    const bool end = q < a.nQB && (q + 1 == a.nQB || cnt[q + 1] < cnt[q]);
    const uint64_t m = __ballot(end);
    if ((q & 63) == 0) ends[q >> 6] = m;
    __syncthreads();
    if (q < a.nQB) {
        int w = q >> 6;
        uint64_t mm = ends[w] & (~0ull << (q & 63));
        while (mm == 0) mm = ends[++w];      // block nQB - 1 always ends a run
        key[q] = cnt[w * 64 + __builtin_ctzll(mm)];
    }
    __syncthreads();
    if (q < a.nQB) {
        const int c = key[q];
        int rank = 0;
        for (int q2 = 0; q2 < a.nQB; ++q2) {
            const int c2 = key[q2];
            rank += (c2 > c || (c2 == c && q2 > q)) ? 1 : 0;
        }
        if (rank == j) *pick = q;
    }
    __syncthreads();
    const int qb = *pick;
    __syncthreads();   // the tile walk reuses lds
    return qb;
}
static_assert(kLongestFirstMaxBlocks <= kThreads, "one Q block per thread when ordering documents");

// Prefill: one workgroup per (row part of a Q block, query head, batch),
// highest Q block index first (under causal-type masks it holds the most
// tiles), or longest document first (longest_first: packed documents).
// KSPLIT: a part is 64 rows and wave w handles row group w & 1 (32
// rows) and key half w >> 1 of every tile, which halves the tile loop of a
// workgroup (short critical path when a few Q blocks hold most of the work);
// otherwise a part is 128 rows, one 32-row group per wave, both key halves.
template <typename T, int D, int SCORE, bool FIXED, bool KSPLIT, bool EXT, int KVL>
__global__ __launch_bounds__(kThreads, (PrefillOccupancy<T, D, KSPLIT, EXT, KVL>::value)) void attn_fwd_prefill(FwdArgs a) {
    using G = Tiles<T, D>;
    __shared__ __attribute__((aligned(16))) char lds[2 * G::kBufBytes];
    constexpr int kRows = KSPLIT ? 64 : 128;
    const int BH = a.B * a.Hq;
    const int parts = (a.q_block + kRows - 1) / kRows;
    const int order = (int)(blockIdx.x / (BH * parts));
    const int qb = a.longest_first ? longest_first_block(a, order, lds) : a.nQB - 1 - order;
    const int rem = (int)(blockIdx.x % (BH * parts));
    const int part = rem / BH;
    int bh = rem % BH;
    // Workgroup i runs on XCD i % 8, each XCD with its own L2.  Under GQA the
    // ids are permuted so that the `group` query heads of one K/V head land on
    // the same XCD (and stay there for every Q block), so their K/V tiles are
    // fetched into one L2 instead of `group`.
    if (a.group > 1 && BH % (8 * a.group) == 0) {
        const int xcd = bh & 7, k = bh >> 3;
        bh = (xcd + 8 * (k / a.group)) * a.group + k % a.group;
    }
    const int b = bh / a.Hq, hq = bh % a.Hq, hkv = hq / a.group;
    const int lane = threadIdx.x & 63, wave = wave_id(), hf = lane >> 5;
    const int rg = KSPLIT ? (wave & 1) : wave, kh = KSPLIT ? (wave >> 1) : 0;
    const int r_in_blk = part * kRows + rg * 32 + (lane & 31);

    LaneRow row;
    row.q_row = qb * a.q_block + r_in_blk;
    row.ok = r_in_blk < a.q_block && row.q_row < a.L;
    const BatchView bv = batch_view<KVL>(a, b);
    row.q_pos = row.q_row + bv.q_offset;
    row.hq = hq;
    row.doc_q = lane_doc(a.mask, row.q_pos);
    const bool wave_active = part * kRows + rg * 32 < a.q_block;

    const T* qbase = reinterpret_cast<const T*>(a.q) + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh;
    const T* kbase = kv_head_base<T, KVL>(a.k, a.k_sb, a.k_sh, a, b, hkv);
    const T* vbase = kv_head_base<T, KVL>(a.v, a.v_sb, a.v_sh, a, b, hkv);

    QRegs<T, D> qr;
    load_q<T, D>(qr, qbase + (int64_t)row.q_row * a.q_sr, row.ok, hf);

    const int bm_b = a.Bm > 1 ? b : 0, bm_h = a.Hm > 1 ? hq : 0;
    const int64_t row_id = ((int64_t)bm_b * a.Hm + bm_h) * a.nQB + qb;
    const int n_part = min(max(scalar_load(a.kv_num + row_id), 0), a.nKB);
    const int n_full = min(max(scalar_load(a.full_num + row_id), 0), a.nKB - n_part);
    const int n_tiles = (n_part + n_full) * (a.kv_block / kTileN);

    const TileConsts tc = make_consts<Precise<T>::value>(a, hq);
    f32x16_t o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
    RowState<Precise<T>::value> st{kNegInf, 0.0f, 0.0f, kNegInf};
    attend_rows<T, D, SCORE, FIXED, KSPLIT, EXT, 2, KVL>(a, kbase, vbase, qr, a.kv_idx + row_id * a.nKB, n_part,
                                            a.full_idx + row_id * a.nKB, 0, n_tiles, tc, row, wave_active, kh, o, st,
                                            lds, bv.S, b);
    if constexpr (KSPLIT) merge_key_halves<T, D, FIXED>(o, st, lds, rg, kh, lane, wave_active);

    // Epilogue: out = acc / lr (0 for rows that saw no key), lse = ln(sum).
    const float l = wave_half_sum(st.l);
    const float lr = wave_half_sum(st.lr);
    const bool live = l > 0.0f;
    const float inv = (live && lr > 0.0f) ? 1.0f / lr : 0.0f;
    if (row.ok && kh == 0) {
        T* orow = reinterpret_cast<T*>(a.out) + (((int64_t)b * a.Hq + hq) * a.L + row.q_row) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + 8 * g + 4 * hf;
                store_out4<T>(orow + d0, o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                              o[db][4 * g + 3] * inv);
            }
        if (a.lse != nullptr && hf == 0) {
            float lse = kNegInf;
            if (live) {
                const double ref = FIXED ? (double)tc.ref_fixed : (double)st.ref;
                lse = Precise<T>::value ? (float)(ref + log((double)l))
                                        : (float)((ref + (double)__log2f(l)) * 0.6931471805599453);
            }
            a.lse[((int64_t)b * a.Hq + hq) * a.L + row.q_row] = lse;
        }
        if (a.max_scores != nullptr && hf == 0) {
            float ms = kNegInf;
            if (live) ms = Precise<T>::value ? (float)st.mx : (float)((double)st.mx * 0.6931471805599453);
            a.max_scores[((int64_t)b * a.Hq + hq) * a.L + row.q_row] = ms;
        }
    }
}

// Decode streams K/V once, so it is bound by HBM latency x bytes in flight:
// a ring of four tile buffers keeps three tiles (96 KiB at head dim 128) in
// flight per workgroup, which fills the LDS of a CU at one workgroup (two at
// head dim 64).
template <int D> struct DecodeShape {
    static constexpr int kStages = 4;
    static constexpr int kWgsPerCu = D == 64 ? 2 : 1;
    static constexpr int kWavesPerSimd = kWgsPerCu;   // 4 waves per workgroup, one per SIMD
};

// Decode / verify: one workgroup per (split, Q block, K/V head, batch).  Rows
// are the G query heads sharing the K/V head times the Q block's queries
// (row r -> head hkv*G + r / q_block, query qb*q_block + r % q_block), so every
// K/V tile is read once for all of them.  The key tiles of the row block are
// divided into `splits` contiguous ranges; each workgroup writes its partial
// numerator, base-2 reference and denominator.  bf16 only; the block mask must
// be the same for every head (H = 1).
template <int D, int SCORE, bool FIXED, bool EXT, int KVL>
__global__ __launch_bounds__(kThreads, DecodeShape<D>::kWavesPerSimd) void attn_fwd_decode(FwdArgs a) {
    using T = __bf16;
    using G = Tiles<T, D>;
    __shared__ __attribute__((aligned(16))) char lds[DecodeShape<D>::kStages * G::kBufBytes];
    const int split = blockIdx.x % a.splits;
    const int unit = blockIdx.x / a.splits;
    const int qb = unit % a.nQB;
    const int bk = unit / a.nQB;
    const int b = bk / a.Hkv, hkv = bk % a.Hkv;
    const int lane = threadIdx.x & 63, wave = wave_id(), hf = lane >> 5;
    const int rg = wave & 1, kh = wave >> 1;
    const int r = rg * 32 + (lane & 31);
    const int rows = a.group * a.q_block;

    LaneRow row;
    const int g = min(r / a.q_block, a.group - 1);
    row.q_row = qb * a.q_block + r % a.q_block;
    row.hq = hkv * a.group + g;
    row.ok = r < rows && row.q_row < a.L;
    const BatchView bv = batch_view<KVL>(a, b);
    row.q_pos = row.q_row + bv.q_offset;
    row.doc_q = lane_doc(a.mask, row.q_pos);
    const bool wave_active = rg * 32 < rows;

    const T* qrow = reinterpret_cast<const T*>(a.q) + (int64_t)b * a.q_sb + (int64_t)row.hq * a.q_sh +
                    (int64_t)row.q_row * a.q_sr;
    const T* kbase = kv_head_base<T, KVL>(a.k, a.k_sb, a.k_sh, a, b, hkv);
    const T* vbase = kv_head_base<T, KVL>(a.v, a.v_sb, a.v_sh, a, b, hkv);
    QRegs<T, D> qr;
    load_q<T, D>(qr, qrow, row.ok, hf);

    const int bm_b = a.Bm > 1 ? b : 0;
    const int64_t row_id = (int64_t)bm_b * a.nQB + qb;
    const int n_part = min(max(scalar_load(a.kv_num + row_id), 0), a.nKB);
    const int n_full = min(max(scalar_load(a.full_num + row_id), 0), a.nKB - n_part);
    const int n_tiles = (n_part + n_full) * (a.kv_block / kTileN);
    const int t_lo = (int)((int64_t)n_tiles * split / a.splits);
    const int t_hi = (int)((int64_t)n_tiles * (split + 1) / a.splits);

    const TileConsts tc = make_consts<false>(a, row.hq);
    f32x16_t o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
    RowState<false> st{kNegInf, 0.0f, 0.0f, kNegInf};
    // each workgroup starts its key range at a different tile, so the
    // workgroups streaming at the same pace do not read addresses a whole
    // range apart at the same moment
    const int n_rng = t_hi - t_lo;
    const int rot = n_rng > 1 ? (int)(((uint32_t)blockIdx.x * 2654435761u >> 12) % (uint32_t)n_rng) : 0;
    attend_rows<T, D, SCORE, FIXED, true, EXT, DecodeShape<D>::kStages, KVL>(a, kbase, vbase, qr, a.kv_idx + row_id * a.nKB,
                                                                   n_part, a.full_idx + row_id * a.nKB, t_lo, t_hi,
                                                                   tc, row, wave_active, kh, o, st, lds, bv.S, b, rot);
    merge_key_halves<T, D, FIXED>(o, st, lds, rg, kh, lane, wave_active);

    const float l = wave_half_sum(st.l);
    const float lr = wave_half_sum(st.lr);
    if (row.ok && kh == 0) {
        const int64_t slot = (((int64_t)split * a.B + b) * a.Hq + row.hq) * a.L + row.q_row;
        float* dst = a.ws_acc + slot * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *reinterpret_cast<float4*>(dst + db * 32 + 8 * q4 + 4 * hf) =
                    make_float4(o[db][4 * q4], o[db][4 * q4 + 1], o[db][4 * q4 + 2], o[db][4 * q4 + 3]);
        if (hf == 0)
            *reinterpret_cast<float4*>(a.ws_ml + slot * 4) = make_float4(FIXED ? tc.ref_fixed : st.ref, l, lr, st.mx);
    }
}

// Merge the split partials of every (batch, head, query) row: one wave per row.
template <int D>
__global__ __launch_bounds__(kThreads) void attn_fwd_combine(FwdArgs a) {
    const int64_t n_rows = (int64_t)a.B * a.Hq * a.L;
    const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const int lane = threadIdx.x & 63;
    const int64_t stride = n_rows;   // slots between consecutive splits
    float ref_max = kNegInf;
    for (int s = 0; s < a.splits; ++s) {
        const float4 ml = *reinterpret_cast<const float4*>(a.ws_ml + (s * stride + row) * 4);
        if (ml.y > 0.0f) ref_max = fmaxf(ref_max, ml.x);
    }
    constexpr int kPer = D / 64;
    float acc[kPer] = {};
    float l = 0.0f, lr = 0.0f;
    if (ref_max != kNegInf) {
        for (int s = 0; s < a.splits; ++s) {
            const float4 ml = *reinterpret_cast<const float4*>(a.ws_ml + (s * stride + row) * 4);
            if (!(ml.y > 0.0f)) continue;
            const float w = __builtin_amdgcn_exp2f(ml.x - ref_max);
            l = __builtin_fmaf(w, ml.y, l);
            lr = __builtin_fmaf(w, ml.z, lr);
            const float* src = a.ws_acc + (s * stride + row) * D + lane * kPer;
#pragma unroll
            for (int e = 0; e < kPer; ++e) acc[e] = __builtin_fmaf(w, src[e], acc[e]);
        }
    }
    const bool live = l > 0.0f;
    const float inv = (live && lr > 0.0f) ? 1.0f / lr : 0.0f;
    if (a.max_scores != nullptr && lane == 0) {
        float mx = kNegInf;
        for (int s = 0; s < a.splits; ++s) {
            const float4 ml = *reinterpret_cast<const float4*>(a.ws_ml + (s * stride + row) * 4);
            if (ml.y > 0.0f) mx = fmaxf(mx, ml.w);
        }
        a.max_scores[row] = live ? (float)((double)mx * 0.6931471805599453) : kNegInf;
    }
    __bf16* out = reinterpret_cast<__bf16*>(a.out) + row * D + lane * kPer;
#pragma unroll
    for (int e = 0; e < kPer; ++e) out[e] = (__bf16)(acc[e] * inv);
    if (a.lse != nullptr && lane == 0)
        a.lse[row] = live ? (float)(((double)ref_max + (double)__log2f(l)) * 0.6931471805599453) : kNegInf;
}

template <typename T, int D, int SCORE, bool FIXED, bool EXT, int KVL>
hipError_t launch_prefill(const FwdArgs& a, hipStream_t stream) {
    const int rows = a.ksplit ? 64 : 128;
    const int64_t blocks = (int64_t)a.nQB * ((a.q_block + rows - 1) / rows) * a.B * a.Hq;
    if constexpr (D == 64 && sizeof(T) == 4) {
        // fp32 at head dim 64 always uses key-split workgroups (prefill_ksplit)
        if (!a.ksplit) return hipErrorInvalidValue;
        hipLaunchKernelGGL((attn_fwd_prefill<T, D, SCORE, FIXED, true, EXT, KVL>), dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, a);
    } else {
        if (a.ksplit)
            hipLaunchKernelGGL((attn_fwd_prefill<T, D, SCORE, FIXED, true, EXT, KVL>), dim3((unsigned)blocks),
                               dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((attn_fwd_prefill<T, D, SCORE, FIXED, false, EXT, KVL>), dim3((unsigned)blocks),
                               dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

template <int D, int SCORE, bool FIXED, bool EXT, int KVL>
hipError_t launch_decode(const FwdArgs& a, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.B * a.Hkv * a.nQB * a.splits;
    hipLaunchKernelGGL((attn_fwd_decode<D, SCORE, FIXED, EXT, KVL>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)a.B * a.Hq * a.L;
    const int64_t cblocks = (rows + kThreads / 64 - 1) / (kThreads / 64);
    hipLaunchKernelGGL((attn_fwd_combine<D>), dim3((unsigned)cblocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int D, bool DECODE, bool EXT, int KVL>
hipError_t dispatch_ext(const FwdArgs& a, hipStream_t stream) {
    const bool fixed = a.ref_mode == 1;
    if constexpr (DECODE) {
        switch (a.score_kind) {
        case SCORE_NONE: return launch_decode<D, SCORE_NONE, false, EXT, KVL>(a, stream);
        case SCORE_SOFTCAP:
            return fixed ? launch_decode<D, SCORE_SOFTCAP, true, EXT, KVL>(a, stream)
                         : launch_decode<D, SCORE_SOFTCAP, false, EXT, KVL>(a, stream);
        case SCORE_SOFTCAP_ALIBI:
            return fixed ? launch_decode<D, SCORE_SOFTCAP_ALIBI, true, EXT, KVL>(a, stream)
                         : launch_decode<D, SCORE_SOFTCAP_ALIBI, false, EXT, KVL>(a, stream);
        case SCORE_ALIBI: return launch_decode<D, SCORE_ALIBI, false, EXT, KVL>(a, stream);
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (a.score_kind) {
        case SCORE_NONE: return launch_prefill<T, D, SCORE_NONE, false, EXT, KVL>(a, stream);
        case SCORE_SOFTCAP:
            if constexpr (sizeof(T) == 2)
                if (fixed) return launch_prefill<T, D, SCORE_SOFTCAP, true, EXT, KVL>(a, stream);
            return launch_prefill<T, D, SCORE_SOFTCAP, false, EXT, KVL>(a, stream);
        case SCORE_SOFTCAP_ALIBI:
            if constexpr (sizeof(T) == 2)
                if (fixed) return launch_prefill<T, D, SCORE_SOFTCAP_ALIBI, true, EXT, KVL>(a, stream);
            return launch_prefill<T, D, SCORE_SOFTCAP_ALIBI, false, EXT, KVL>(a, stream);
        case SCORE_ALIBI: return launch_prefill<T, D, SCORE_ALIBI, false, EXT, KVL>(a, stream);
        default: return hipErrorInvalidValue;
        }
    }
}

// Program masks and the max_scores output run in separately compiled
// "extended" kernels, so the common kernels keep their register budget.
// Paged pools (tiles remapped through the page table) and contiguous caches
// with per-batch offsets and lengths (per-batch values read per workgroup)
// have kernels of their own, lean or extended by the same rule.
template <typename T, int D, bool DECODE>
hipError_t dispatch(const FwdArgs& a, hipStream_t stream) {
    const bool ext = a.mask.kind == MASK_PROGRAM || a.max_scores != nullptr;
    if (a.page_table != nullptr)
        return ext ? dispatch_ext<T, D, DECODE, true, kKvPaged>(a, stream)
                   : dispatch_ext<T, D, DECODE, false, kKvPaged>(a, stream);
    if (a.mask.q_offsets != nullptr || a.mask.kv_lens != nullptr)
        return ext ? dispatch_ext<T, D, DECODE, true, kKvPerBatch>(a, stream)
                   : dispatch_ext<T, D, DECODE, false, kKvPerBatch>(a, stream);
    if (ext) return dispatch_ext<T, D, DECODE, true, kKvContig>(a, stream);
    return dispatch_ext<T, D, DECODE, false, kKvContig>(a, stream);
}

}  // namespace

}  // namespace flexmi
