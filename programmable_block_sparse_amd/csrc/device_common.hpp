// Device-side helpers shared by the block-mask builder and the attention
// kernels: vector types for gfx950 MFMA operands and the mask_mod menu.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flexmi {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

enum MaskKind : int {
    MASK_NOOP = 0,
    MASK_CAUSAL = 1,
    MASK_CAUSAL_WINDOW_SINKS = 2,
    MASK_DOC_CAUSAL = 3,
    MASK_PROGRAM = 4
};
enum ScoreKind : int { SCORE_NONE = 0, SCORE_SOFTCAP = 1, SCORE_SOFTCAP_ALIBI = 2, SCORE_ALIBI = 3 };
enum PredKind : int {
    PRED_CAUSAL = 0,
    PRED_WINDOW = 1,
    PRED_KV_LT = 2,
    PRED_CHUNK = 3,
    PRED_STRIDE = 4,
    PRED_DOC = 5,
    PRED_HEAD_LT = 6
};

constexpr int kMaxClauses = 4;
constexpr int kMaxLiterals = 2;

// A PROGRAM mask: the AND of n_clauses clauses, clause c the OR of n_lits[c]
// predicates (kind, arg).
struct MaskProgram {
    int n_clauses;
    int n_lits[kMaxClauses];
    int kind[kMaxClauses][kMaxLiterals];
    int arg[kMaxClauses][kMaxLiterals];
};

// mask_mod arguments in device-friendly form.  Positions fit in int32 (the
// host rejects lengths and offsets that would not).
struct MaskArgs {
    int kind;
    int window;
    int sinks;
    int q_offset;
    const int* doc_id;
    int doc_len;
    int uses_doc;    // the mask compares document ids (DOC_CAUSAL, or a DOC predicate)
    MaskProgram prog;
    const int* q_offsets;   // per batch: logical position of query row 0 (NULL: q_offset)
    const int* kv_lens;     // per batch: valid keys, positions [0, kv_lens[b]) (NULL: S)
};

// floor(a / b) for b > 0.
__device__ __forceinline__ int floor_div(int a, int b) {
    const int q = a / b;
    return (a % b != 0 && a < 0) ? q - 1 : q;
}

// One predicate of a PROGRAM mask at query position p, key j, query head h;
// doc_p and doc_j are the positions' document ids (distinct sentinels when a
// position has none).
__device__ __forceinline__ bool pred_holds(int kind, int arg, int p, int j, int h, int doc_p, int doc_j) {
    switch (kind) {
    case PRED_CAUSAL: return j <= p;
    case PRED_WINDOW: return p - j < arg;
    case PRED_KV_LT: return j < arg;
    case PRED_CHUNK: return floor_div(p, arg) == floor_div(j, arg);
    case PRED_STRIDE: return (p - j) % arg == 0;
    case PRED_DOC: return doc_p == doc_j;
    default: return h < arg;   // PRED_HEAD_LT
    }
}

// (Loops run over the fixed maxima with early exits so that every index is a
// compile-time constant and the program stays in scalar registers.)
__device__ __forceinline__ bool program_holds(const MaskProgram& pg, int p, int j, int h, int doc_p, int doc_j) {
    bool all = true;
#pragma unroll
    for (int c = 0; c < kMaxClauses; ++c) {
        if (c >= pg.n_clauses) break;
        bool any = false;
#pragma unroll
        for (int l = 0; l < kMaxLiterals; ++l) {
            if (l >= pg.n_lits[c]) break;
            any = any || pred_holds(pg.kind[c][l], pg.arg[c][l], p, j, h, doc_p, doc_j);
        }
        all = all && any;
    }
    return all;
}

}  // namespace flexmi
