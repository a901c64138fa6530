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

enum MaskKind : int { MASK_NOOP = 0, MASK_CAUSAL = 1, MASK_CAUSAL_WINDOW_SINKS = 2, MASK_DOC_CAUSAL = 3 };
enum ScoreKind : int { SCORE_NONE = 0, SCORE_SOFTCAP = 1, SCORE_SOFTCAP_ALIBI = 2 };

// mask_mod arguments in device-friendly form.  Positions fit in int32 (the
// host rejects lengths and offsets that would not).
struct MaskArgs {
    int kind;
    int window;
    int sinks;
    int q_offset;
    const int* doc_id;
    int doc_len;
};

// True when logical query position p may attend key j (true = attend).  The
// menu: NOOP; CAUSAL j <= p; CAUSAL_WINDOW_SINKS j <= p and (p - j < window or
// j < sinks); DOC_CAUSAL j <= p and doc[p] == doc[j].  Positions outside the
// document-id array belong to no document.
__device__ __forceinline__ bool mask_visible(const MaskArgs& m, int p, int j) {
    switch (m.kind) {
    case MASK_NOOP:
        return true;
    case MASK_CAUSAL:
        return j <= p;
    case MASK_CAUSAL_WINDOW_SINKS:
        return (j <= p) && ((p - j < m.window) || (j < m.sinks));
    default: {
        if (!(j <= p)) return false;
        if (p < 0 || p >= m.doc_len || j < 0 || j >= m.doc_len) return false;
        return __ldg(m.doc_id + p) == __ldg(m.doc_id + j);
    }
    }
}

}  // namespace flexmi
