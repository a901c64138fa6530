// Block-sparse attention forward for gfx950 (CDNA4): the prefill kernel and
// the split-KV decode kernel with its combine pass.
//
// What is computed: the charlestar blog "FlexAttention score_mod / BlockMask",
// section on what one connection goes through (scaled score, score_mod g,
// -inf where mask_mod is false, softmax-weighted sum of values), its BlockMask
// section (empty tiles skipped, full tiles computed without the element mask
// but with score_mod, partial tiles computed then masked) and its template
// section (tiles with an online softmax, no score matrix in memory).  The
// quant67 "Causal Mask" article, section 7, describes the same running
// statistics for FlashAttention's block skipping.
//
// How it maps onto CDNA4 (design of this library, not of the pages):
//   * A workgroup of 4 wave64s owns one Q block (<= 128 query rows, 32 per
//     wave).  It walks the block's partial list then its full list, 64 keys
//     per step, K and V tiles double-buffered in LDS.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (fp32 inputs: v_mfma_f32_32x32x2f32): the
//     accumulator then holds one query row per lane (lane & 31) and 16 keys
//     per 32-key block in registers, so the row max / sum is in-lane plus one
//     v_permlane32_swap across the two lane halves.
//   * The same orientation is kept for O^T = V^T P^T: the probabilities feed
//     the MFMA B operand straight from registers (no LDS round trip), and the
//     per-row rescale and the final 1/l are per-lane scalars.
//   * Softmax works in base 2 with the log2(e) factor folded into the score
//     constants.  The running reference is only moved when a row's tile
//     maximum exceeds it by more than kRescaleSlack (probabilities up to
//     2^kRescaleSlack are exact in fp32 and bf16), and the move is a
//     wave-uniform branch, so most tiles skip the accumulator rescale.
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

// LDS tile geometry for one buffer.
template <typename T, int D> struct Tiles {
    static constexpr int kStrideK = D + Elem<T>::kPadK;        // K[key][d]
    static constexpr int kStrideV = kTileN + Elem<T>::kPadV;   // V^T[d][key]
    static constexpr int kElemsK = kTileN * kStrideK;
    static constexpr int kElemsV = D * kStrideV;
    static constexpr int kElems = kElemsK + kElemsV;
};

// Key (within a 32-key block) held by accumulator register r in lane half hf
// for a 32x32 MFMA output tile: rows (r&3) + 8*(r>>2) + 4*hf.
__device__ __forceinline__ constexpr int acc_row(int r, int hf) { return (r & 3) + 8 * (r >> 2) + 4 * hf; }

__device__ __forceinline__ float wave_half_max(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float wave_half_sum(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Per-workgroup constants of the score rule.  The bf16 path works in base-2
// units (log2(e) folded in); the fp32 path keeps natural units in double.
struct ScoreConsts {
    float mul;      // NONE: scale*log2e; SOFTCAP*: 2*scale*log2e/cap
    float c2;       // cap*log2e
    float alpha2;   // ALiBi slope * log2e (0 if unused)
    double scale_d, cap_d, alpha_d;
};

// fp32 inputs take the precise path: scores, references and the softmax
// exponent argument in double / accurate library functions, so results stay
// within a few fp32 ulps of the float64 definition even for large scores.
template <typename T> struct Precise { static constexpr bool value = sizeof(T) == 4; };

// Registers staged from global memory for one K/V tile.
template <typename T, int D> struct Stage;

template <int D> struct Stage<__bf16, D> {
    static constexpr int kKUnits = kTileN * D / 8 / kThreads;       // 16-byte K chunks per thread
    static constexpr int kVUnits = (kTileN / 2) * (D / 8) / kThreads;  // key pairs x 8 dims per thread
    uint4 k[kKUnits];
    uint4 v[kVUnits][2];
};
template <int D> struct Stage<float, D> {
    static constexpr int kKUnits = kTileN * D / 4 / kThreads;
    static constexpr int kVUnits = kTileN * D / 4 / kThreads;
    uint4 k[kKUnits];
    uint4 v[kVUnits];
};

template <typename T, int D>
__device__ __forceinline__ void stage_load(Stage<T, D>& st, const T* __restrict__ kbase, const T* __restrict__ vbase,
                                           int64_t k_sr, int64_t v_sr, int kv0, int S, int tid) {
    constexpr int kChunks = D / Elem<T>::kChunk;  // 16-byte chunks per row
#pragma unroll
    for (int u = 0; u < Stage<T, D>::kKUnits; ++u) {
        const int c = tid + u * kThreads;
        const int key = c / kChunks, ch = c % kChunks;
        const int kv = kv0 + key;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (kv >= 0 && kv < S) x = *reinterpret_cast<const uint4*>(kbase + (int64_t)kv * k_sr + ch * Elem<T>::kChunk);
        st.k[u] = x;
    }
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int u = 0; u < Stage<T, D>::kVUnits; ++u) {
            const int c = tid + u * kThreads;
            const int pair = c / kChunks, ch = c % kChunks;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int kv = kv0 + 2 * pair + e;
                uint4 x = make_uint4(0, 0, 0, 0);
                if (kv >= 0 && kv < S) x = *reinterpret_cast<const uint4*>(vbase + (int64_t)kv * v_sr + ch * 8);
                st.v[u][e] = x;
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < Stage<T, D>::kVUnits; ++u) {
            const int c = tid + u * kThreads;
            const int key = c / kChunks, ch = c % kChunks;
            const int kv = kv0 + key;
            uint4 x = make_uint4(0, 0, 0, 0);
            if (kv >= 0 && kv < S) x = *reinterpret_cast<const uint4*>(vbase + (int64_t)kv * v_sr + ch * 4);
            st.v[u] = x;
        }
    }
}

template <typename T, int D>
__device__ __forceinline__ void stage_store(const Stage<T, D>& st, T* __restrict__ lds, int tid) {
    using G = Tiles<T, D>;
    constexpr int kChunks = D / Elem<T>::kChunk;
    T* Ks = lds;
    T* Vt = lds + G::kElemsK;
#pragma unroll
    for (int u = 0; u < Stage<T, D>::kKUnits; ++u) {
        const int c = tid + u * kThreads;
        const int key = c / kChunks, ch = c % kChunks;
        *reinterpret_cast<uint4*>(Ks + key * G::kStrideK + ch * Elem<T>::kChunk) = st.k[u];
    }
    if constexpr (sizeof(T) == 2) {
        // Two consecutive keys x 8 dims -> 8 dwords of V^T, each (key, key+1) for one dim.
#pragma unroll
        for (int u = 0; u < Stage<T, D>::kVUnits; ++u) {
            const int c = tid + u * kThreads;
            const int pair = c / kChunks, ch = c % kChunks;
            const uint32_t a[4] = {st.v[u][0].x, st.v[u][0].y, st.v[u][0].z, st.v[u][0].w};
            const uint32_t b[4] = {st.v[u][1].x, st.v[u][1].y, st.v[u][1].z, st.v[u][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t w = __builtin_amdgcn_perm(b[e >> 1], a[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
                *reinterpret_cast<uint32_t*>(Vt + (ch * 8 + e) * G::kStrideV + 2 * pair) = w;
            }
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
}

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
__device__ __forceinline__ f32x16_t qk_block(const QRegs<T, D>& qr, const T* __restrict__ Ks, int kb2, int lane) {
    using G = Tiles<T, D>;
    const int hf = lane >> 5;
    const T* krow = Ks + (kb2 * 32 + (lane & 31)) * G::kStrideK;
    f32x16_t acc = {};
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(krow + 16 * s + 8 * hf);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr.x[s], acc, 0, 0, 0);
        }
    } else {
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

// O^T += V^T P^T over the 64 keys of the tile.  p[kb2][r] holds the
// probability of key kb2*32 + acc_row(r, hf) for this lane's query.
template <typename T, int D>
__device__ __forceinline__ void pv_tile(f32x16_t (&o)[D / 32], const float (&p)[2][16], const T* __restrict__ Vt, int lane) {
    using G = Tiles<T, D>;
    const int hf = lane >> 5;
    if constexpr (sizeof(T) == 2) {
        bf16x8_t pb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[t][e] = (__bf16)p[t >> 1][8 * (t & 1) + e];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const T* vrow = Vt + (db * 32 + (lane & 31)) * G::kStrideV;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                // keys 16t + 4hf + {0..3} and 16t + 8 + 4hf + {0..3}: the same keys, in the
                // same order, as registers 8(t&1)..8(t&1)+7 of block t>>1 hold in pb[t].
                const bf16x4_t lo = *reinterpret_cast<const bf16x4_t*>(vrow + 16 * t + 4 * hf);
                const bf16x4_t hi = *reinterpret_cast<const bf16x4_t*>(vrow + 16 * t + 8 + 4 * hf);
                const bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[t], o[db], 0, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const T* vrow = Vt + (db * 32 + (lane & 31)) * G::kStrideV;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float a = vrow[kb2 * 32 + acc_row(r, hf)];
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[kb2][r], o[db], 0, 0, 0);
                }
        }
    }
}

// Online-softmax state for this lane's query row (both lane halves keep
// their own partial denominator; they are added at the end).  ref is -inf
// until the row has seen a finite score; base 2 (float) on the bf16 path,
// natural units (double) on the precise path.
template <bool P> struct RowState;
template <> struct RowState<false> {
    float ref;
    float l;
};
template <> struct RowState<true> {
    double ref;
    float l;
};

// One 64-key tile: scores, score_mod, optional mask, softmax update, PV.
template <typename T, int D, int SCORE, bool MASKED>
__device__ __forceinline__ void process_tile(const QRegs<T, D>& qr, const T* __restrict__ lds, f32x16_t (&o)[D / 32],
                                             RowState<Precise<T>::value>& st, const ScoreConsts& sc,
                                             const MaskArgs& mask, int kv0, int S, int q_pos, int lane) {
    using G = Tiles<T, D>;
    constexpr bool P = Precise<T>::value;
    using RefT = typename std::conditional<P, double, float>::type;
    const int hf = lane >> 5;
    f32x16_t s[2];
    s[0] = qk_block<T, D>(qr, lds, 0, lane);
    s[1] = qk_block<T, D>(qr, lds, 1, lane);

    // score minus the current reference (base 2 or natural), and its row maximum.
    const RefT ref_sub = (st.ref == (RefT)kNegInf) ? (RefT)0 : st.ref;
    float z[2][16];
    float tmax = kNegInf;
    const int key_base = kv0 + 4 * hf;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float acc = s[kb2][r];
            const int kv = key_base + kb2 * 32 + acc_row(r, 0);
            float x;
            if constexpr (P) {
                double g = (double)acc * sc.scale_d;
                if constexpr (SCORE != SCORE_NONE) g = sc.cap_d * tanh(g / sc.cap_d);
                if constexpr (SCORE == SCORE_SOFTCAP_ALIBI) g = fma(sc.alpha_d, (double)(kv - q_pos), g);
                x = (float)(g - ref_sub);
            } else if constexpr (SCORE == SCORE_NONE) {
                x = __builtin_fmaf(acc, sc.mul, -ref_sub);
            } else {
                // cap*tanh(y) = cap - 2*cap / (1 + e^{2y}),  y = scale*acc/cap
                const float e2y = __builtin_amdgcn_exp2f(acc * sc.mul);
                const float rcp = __builtin_amdgcn_rcpf(1.0f + e2y);
                float base = sc.c2 - ref_sub;
                if constexpr (SCORE == SCORE_SOFTCAP_ALIBI) base = __builtin_fmaf(sc.alpha2, (float)(kv - q_pos), base);
                x = __builtin_fmaf(-2.0f * sc.c2, rcp, base);
            }
            if constexpr (MASKED) {
                const bool vis = (kv < S) && mask_visible(mask, q_pos, kv);
                x = vis ? x : kNegInf;
            }
            z[kb2][r] = x;
            tmax = fmaxf(tmax, x);
        }
    tmax = wave_half_max(tmax);

    // Move the reference when the tile max exceeds it by more than the slack,
    // or when the row sees its first finite score.  Wave-uniform branch.
    const bool need = (tmax > kRescaleSlack) || (st.ref == (RefT)kNegInf && tmax != kNegInf);
    float shift = 0.0f;
    if (__builtin_expect(__any(need), 0)) {
        const RefT tile_max_abs = ref_sub + (RefT)tmax;             // -inf if nothing visible yet
        const RefT new_ref = st.ref > tile_max_abs ? st.ref : tile_max_abs;
        const RefT new_sub = (new_ref == (RefT)kNegInf) ? (RefT)0 : new_ref;
        float factor;
        if constexpr (P) factor = (st.ref == (RefT)kNegInf) ? 0.0f : expf((float)(st.ref - new_ref));
        else factor = (st.ref == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(st.ref - new_ref);
        shift = (float)(new_sub - ref_sub);
        st.l *= factor;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] *= factor;
        st.ref = new_ref;
    }

    float p[2][16];
    float lsum = 0.0f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float e;
            if constexpr (P) e = expf(z[kb2][r] - shift);
            else e = __builtin_amdgcn_exp2f(z[kb2][r] - shift);
            p[kb2][r] = e;
            lsum += e;
        }
    st.l += lsum;
    pv_tile<T, D>(o, p, lds + G::kElemsK, lane);
}

template <typename T, int D, int SCORE>
__device__ __forceinline__ void attend_rows(const FwdArgs& a, const T* __restrict__ kbase, const T* __restrict__ vbase,
                                            const QRegs<T, D>& qr, const int* __restrict__ part_idx, int n_part,
                                            const int* __restrict__ full_idx, int n_full, int tile_lo, int tile_hi,
                                            const ScoreConsts& sc, int q_pos, bool wave_active,
                                            f32x16_t (&o)[D / 32], RowState<Precise<T>::value>& st, T* lds) {
    using G = Tiles<T, D>;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int sub_per_block = a.kv_block / kTileN;

    auto tile_kv0 = [&](int t, bool& masked) -> int {
        const int blk = t / sub_per_block, sub = t - blk * sub_per_block;
        int kb;
        if (blk < n_part) { kb = part_idx[blk]; masked = true; }
        else { kb = full_idx[blk - n_part]; masked = false; }
        return kb * a.kv_block + sub * kTileN;
    };

    if (tile_lo >= tile_hi) return;
    Stage<T, D> stage;
    bool masked;
    int kv0 = tile_kv0(tile_lo, masked);
    stage_load<T, D>(stage, kbase, vbase, a.k_sr, a.v_sr, kv0, a.S, tid);
    stage_store<T, D>(stage, lds, tid);
    __syncthreads();
    for (int t = tile_lo; t < tile_hi; ++t) {
        const int buf = (t - tile_lo) & 1;
        bool next_masked = false;
        int next_kv0 = 0;
        const bool has_next = t + 1 < tile_hi;
        if (has_next) {
            next_kv0 = tile_kv0(t + 1, next_masked);
            stage_load<T, D>(stage, kbase, vbase, a.k_sr, a.v_sr, next_kv0, a.S, tid);
        }
        const T* cur = lds + buf * G::kElems;
        if (wave_active) {
            if (masked)
                process_tile<T, D, SCORE, true>(qr, cur, o, st, sc, a.mask, kv0, a.S, q_pos, lane);
            else
                process_tile<T, D, SCORE, false>(qr, cur, o, st, sc, a.mask, kv0, a.S, q_pos, lane);
        }
        if (has_next) stage_store<T, D>(stage, lds + (buf ^ 1) * G::kElems, tid);
        __syncthreads();
        kv0 = next_kv0;
        masked = next_masked;
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

__device__ __forceinline__ ScoreConsts make_consts(const FwdArgs& a, int hq) {
    ScoreConsts sc;
    if (a.score_kind == SCORE_NONE) {
        sc.mul = a.scale * kLog2e;
        sc.c2 = 0.0f;
    } else {
        sc.mul = 2.0f * a.scale * kLog2e / a.cap;
        sc.c2 = a.cap * kLog2e;
    }
    sc.alpha2 = 0.0f;
    sc.scale_d = (double)a.scale;
    sc.cap_d = (double)a.cap;
    sc.alpha_d = 0.0;
    if (a.score_kind == SCORE_SOFTCAP_ALIBI) {
        sc.alpha_d = exp2(-(double)a.alibi_m * (double)(hq + 1) / (double)a.Hq);
        sc.alpha2 = (float)(sc.alpha_d * 1.4426950408889634);
    }
    return sc;
}

// Prefill: one workgroup per (Q block, query head, batch), heaviest Q blocks
// (highest index) first.
template <typename T, int D, int SCORE>
__global__ __launch_bounds__(kThreads) void attn_fwd_prefill(FwdArgs a) {
    using G = Tiles<T, D>;
    __shared__ __attribute__((aligned(16))) T lds[2 * G::kElems];
    const int BH = a.B * a.Hq;
    const int qb = a.nQB - 1 - (int)(blockIdx.x / BH);
    const int bh = blockIdx.x % BH;
    const int b = bh / a.Hq, hq = bh % a.Hq, hkv = hq / a.group;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hf = lane >> 5;
    const int r_in_blk = wave * 32 + (lane & 31);
    const int q_row = qb * a.q_block + r_in_blk;
    const bool row_ok = r_in_blk < a.q_block && q_row < a.L;
    const bool wave_active = wave * 32 < a.q_block;
    const int q_pos = q_row + a.mask.q_offset;

    const T* qbase = reinterpret_cast<const T*>(a.q) + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh;
    const T* kbase = reinterpret_cast<const T*>(a.k) + (int64_t)b * a.k_sb + (int64_t)hkv * a.k_sh;
    const T* vbase = reinterpret_cast<const T*>(a.v) + (int64_t)b * a.v_sb + (int64_t)hkv * a.v_sh;

    QRegs<T, D> qr;
    load_q<T, D>(qr, qbase + (int64_t)q_row * a.q_sr, row_ok, hf);

    const int bm_b = a.Bm > 1 ? b : 0, bm_h = a.Hm > 1 ? hq : 0;
    const int64_t row_id = ((int64_t)bm_b * a.Hm + bm_h) * a.nQB + qb;
    const int n_part = min(max(a.kv_num[row_id], 0), a.nKB);
    const int n_full = min(max(a.full_num[row_id], 0), a.nKB - n_part);
    const int* part_idx = a.kv_idx + row_id * a.nKB;
    const int* full_idx = a.full_idx + row_id * a.nKB;
    const int n_tiles = (n_part + n_full) * (a.kv_block / kTileN);

    const ScoreConsts sc = make_consts(a, hq);
    f32x16_t o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
    RowState<Precise<T>::value> st{kNegInf, 0.0f};
    attend_rows<T, D, SCORE>(a, kbase, vbase, qr, part_idx, n_part, full_idx, n_full, 0, n_tiles, sc, q_pos,
                             wave_active, o, st, lds);

    // Epilogue: out = acc / l (0 for rows that saw no key), lse = ln(sum).
    const float l = wave_half_sum(st.l);
    const bool live = l > 0.0f;
    const float inv = live ? 1.0f / l : 0.0f;
    if (row_ok) {
        T* orow = reinterpret_cast<T*>(a.out) + (((int64_t)b * a.Hq + hq) * a.L + q_row) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + 8 * g + 4 * hf;
                store_out4<T>(orow + d0, o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                              o[db][4 * g + 3] * inv);
            }
        if (a.lse != nullptr && hf == 0)
            a.lse[((int64_t)b * a.Hq + hq) * a.L + q_row] = !live ? kNegInf
                : Precise<T>::value ? (float)((double)st.ref + log((double)l)) : (float)((st.ref + __log2f(l)) * kLn2);
    }
}

template <typename T, int D, int SCORE>
hipError_t launch_prefill(const FwdArgs& a, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.nQB * a.B * a.Hq;
    hipLaunchKernelGGL((attn_fwd_prefill<T, D, SCORE>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t dispatch_score(const FwdArgs& a, hipStream_t stream) {
    switch (a.score_kind) {
    case SCORE_NONE: return launch_prefill<T, D, SCORE_NONE>(a, stream);
    case SCORE_SOFTCAP: return launch_prefill<T, D, SCORE_SOFTCAP>(a, stream);
    case SCORE_SOFTCAP_ALIBI: return launch_prefill<T, D, SCORE_SOFTCAP_ALIBI>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t attn_fwd_workspace_bytes(int, int, int, int, int, int, int, int, int, int, int, int) { return 0; }

hipError_t launch_attn_fwd(int dtype, int D, const FwdArgs& a, hipStream_t stream) {
    if (dtype == 1 && D == 64) return dispatch_score<__bf16, 64>(a, stream);
    if (dtype == 1 && D == 128) return dispatch_score<__bf16, 128>(a, stream);
    if (dtype == 0 && D == 64) return dispatch_score<float, 64>(a, stream);
    if (dtype == 0 && D == 128) return dispatch_score<float, 128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace flexmi
