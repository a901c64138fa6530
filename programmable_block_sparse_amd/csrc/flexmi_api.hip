// C ABI of the library (declared in include/flexmi.h): argument checks on the
// host, then dispatch to the kernel launchers.  No entry point allocates,
// synchronises or keeps state; every check runs before the first HIP call.
//
// The checks restate the 2kiu "PyTorch Flex Attention complete guide",
// section 1.3 (4-D inputs, Hq == Hkv unless grouped, Hq % Hkv == 0, block mask
// sized to the query and key lengths: "too small / too large"), plus the
// limits of this implementation (head dims, tile shapes, alignment).
#include <cmath>
#include <cstdio>
#include <cstdarg>
#include <mutex>
#include <string>

#include "flexmi.h"
#include "internal.hpp"

using namespace flexmi;

namespace {

thread_local std::string g_last_error;

flex_status fail(flex_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

constexpr int64_t kMaxLen = int64_t(1) << 30;   // positions and offsets fit in int32

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// True when a PROGRAM mask has a predicate of this kind.
bool program_uses(const flex_mask_params* m, int pred) {
    if (m->kind != FLEX_MASK_PROGRAM) return false;
    for (int c = 0; c < m->n_clauses && c < FLEX_MAX_CLAUSES; ++c)
        for (int l = 0; l < m->clause[c].n && l < FLEX_MAX_LITERALS; ++l)
            if (m->clause[c].lit[l].kind == pred) return true;
    return false;
}

// True when every visible cell has j <= p: the mask is causal-type (CAUSAL,
// the causal window, DOC_CAUSAL, or a PROGRAM with a clause that is CAUSAL
// alone).
bool mask_implies_causal(const flex_mask_params* m) {
    if (m->kind == FLEX_MASK_CAUSAL || m->kind == FLEX_MASK_CAUSAL_WINDOW_SINKS || m->kind == FLEX_MASK_DOC_CAUSAL)
        return true;
    if (m->kind != FLEX_MASK_PROGRAM) return false;
    for (int c = 0; c < m->n_clauses; ++c)
        if (m->clause[c].n == 1 && m->clause[c].lit[0].kind == FLEX_PRED_CAUSAL) return true;
    return false;
}

// True when every row that sees a key also sees its own diagonal key j = p
// (whenever p is a valid key): each clause of a PROGRAM holds a predicate that
// is true at j = p (causal, window, chunk, stride or same document).  kv_lt and
// head_lt are not: a clause made of them alone can hide the diagonal while
// leaving far keys visible.
bool mask_keeps_diagonal(const flex_mask_params* m) {
    if (m->kind != FLEX_MASK_PROGRAM) return true;
    for (int c = 0; c < m->n_clauses; ++c) {
        bool has = false;
        for (int l = 0; l < m->clause[c].n; ++l) {
            const int k = m->clause[c].lit[l].kind;
            has = has || k == FLEX_PRED_CAUSAL || k == FLEX_PRED_WINDOW || k == FLEX_PRED_CHUNK ||
                  k == FLEX_PRED_STRIDE || k == FLEX_PRED_DOC;
        }
        if (!has) return false;
    }
    return true;
}

flex_status check_mask(const flex_mask_params* m, int64_t L, int64_t S) {
    if (m->kind < FLEX_MASK_NOOP || m->kind > FLEX_MASK_PROGRAM)
        return fail(FLEX_ERR_PARAM, "unknown mask kind %d", m->kind);
    if (m->q_offset <= -kMaxLen || m->q_offset >= kMaxLen || m->q_offset + L >= kMaxLen)
        return fail(FLEX_ERR_PARAM, "q_offset %lld out of range for L=%lld", (long long)m->q_offset, (long long)L);
    if (m->kind == FLEX_MASK_CAUSAL_WINDOW_SINKS) {
        if (m->window < 1) return fail(FLEX_ERR_PARAM, "window must be >= 1 (got %d)", m->window);
        if (m->sinks < 0) return fail(FLEX_ERR_PARAM, "sinks must be >= 0 (got %d)", m->sinks);
    }
    if (m->kind == FLEX_MASK_PROGRAM) {
        if (m->n_clauses < 1 || m->n_clauses > FLEX_MAX_CLAUSES)
            return fail(FLEX_ERR_PARAM, "a mask program needs 1..%d clauses (got %d)", FLEX_MAX_CLAUSES, m->n_clauses);
        for (int c = 0; c < m->n_clauses; ++c) {
            const flex_mask_clause& cl = m->clause[c];
            if (cl.n < 1 || cl.n > FLEX_MAX_LITERALS)
                return fail(FLEX_ERR_PARAM, "clause %d needs 1..%d predicates (got %d)", c, FLEX_MAX_LITERALS, cl.n);
            for (int l = 0; l < cl.n; ++l) {
                const int kind = cl.lit[l].kind, arg = cl.lit[l].arg;
                if (kind < FLEX_PRED_CAUSAL || kind > FLEX_PRED_HEAD_LT)
                    return fail(FLEX_ERR_PARAM, "clause %d: unknown predicate kind %d", c, kind);
                const bool positive = kind == FLEX_PRED_WINDOW || kind == FLEX_PRED_CHUNK || kind == FLEX_PRED_STRIDE;
                const bool non_negative = kind == FLEX_PRED_KV_LT || kind == FLEX_PRED_HEAD_LT;
                if ((positive && arg < 1) || (non_negative && arg < 0))
                    return fail(FLEX_ERR_PARAM, "clause %d: predicate %d argument %d out of range", c, kind, arg);
            }
        }
    }
    if ((reinterpret_cast<uintptr_t>(m->q_offsets) & 3u) || (reinterpret_cast<uintptr_t>(m->kv_lens) & 3u))
        return fail(FLEX_ERR_LAYOUT, "q_offsets and kv_lens must be 4-byte aligned");
    if (m->kind == FLEX_MASK_DOC_CAUSAL || program_uses(m, FLEX_PRED_DOC)) {
        if (m->doc_id == nullptr) return fail(FLEX_ERR_NULL, "a document mask needs doc_id");
        if (m->q_offset < 0 && !m->q_offsets) return fail(FLEX_ERR_PARAM, "a document mask needs q_offset >= 0");
        const int64_t need = std::max<int64_t>(S, m->q_offset + L);
        if (m->doc_len < need)
            return fail(FLEX_ERR_PARAM, "doc_len %lld must cover max(S, q_offset + L) = %lld",
                        (long long)m->doc_len, (long long)need);
        // the kernels address doc_id through 2 GiB buffer descriptors
        if (m->doc_len >= (int64_t(1) << 29))
            return fail(FLEX_ERR_PARAM, "doc_len %lld must stay below 2^29", (long long)m->doc_len);
        if (reinterpret_cast<uintptr_t>(m->doc_id) & 3u)
            return fail(FLEX_ERR_LAYOUT, "doc_id must be 4-byte aligned");
    }
    return FLEX_OK;
}

MaskArgs to_mask_args(const flex_mask_params* m) {
    MaskArgs a{};
    a.kind = m->kind;
    a.window = m->window;
    a.sinks = m->sinks;
    a.q_offset = (int)m->q_offset;
    a.doc_id = m->doc_id;
    a.doc_len = (int)std::min<int64_t>(m->doc_len, kMaxLen - 1);
    a.uses_doc = (m->kind == FLEX_MASK_DOC_CAUSAL || program_uses(m, FLEX_PRED_DOC)) ? 1 : 0;
    if (m->kind == FLEX_MASK_PROGRAM) {
        a.prog.n_clauses = m->n_clauses;
        for (int c = 0; c < m->n_clauses; ++c) {
            a.prog.n_lits[c] = m->clause[c].n;
            for (int l = 0; l < m->clause[c].n; ++l) {
                a.prog.kind[c][l] = m->clause[c].lit[l].kind;
                a.prog.arg[c][l] = m->clause[c].lit[l].arg;
            }
        }
    }
    if (!a.uses_doc) a.doc_len = 0;
    a.q_offsets = m->q_offsets;
    a.kv_lens = m->kv_lens;
    return a;
}

bool per_batch(const flex_mask_params* m) { return m->q_offsets != nullptr || m->kv_lens != nullptr; }

flex_status check_bm_arrays(const flex_block_mask* bm) {
    if (!bm->kv_num_blocks || !bm->kv_indices || !bm->full_kv_num_blocks || !bm->full_kv_indices)
        return fail(FLEX_ERR_NULL, "block mask arrays must not be NULL");
    return FLEX_OK;
}

flex_status check_bm_dims(const flex_block_mask* bm, int64_t L, int64_t S) {
    if (bm->q_block < 1 || bm->kv_block < 1 || bm->q_block > 1024 || bm->kv_block > 1024)
        return fail(FLEX_ERR_BLOCKMASK, "block sizes must be in [1, 1024] (got %d x %d)", bm->q_block, bm->kv_block);
    const int64_t nqb = ceil_div(L, bm->q_block), nkb = ceil_div(S, bm->kv_block);
    if (bm->num_q_blocks != nqb)
        return fail(FLEX_ERR_BLOCKMASK, "block mask has %d Q blocks, L=%lld needs %lld (mask too %s)",
                    bm->num_q_blocks, (long long)L, (long long)nqb, bm->num_q_blocks < nqb ? "small" : "large");
    if (bm->num_kv_blocks != nkb)
        return fail(FLEX_ERR_BLOCKMASK, "block mask has %d KV blocks, S=%lld needs %lld (mask too %s)",
                    bm->num_kv_blocks, (long long)S, (long long)nkb, bm->num_kv_blocks < nkb ? "small" : "large");
    if (bm->B < 1 || bm->H < 1 || bm->B > 65535 || bm->H > 65535)
        return fail(FLEX_ERR_BLOCKMASK, "block mask B=%d H=%d out of range", bm->B, bm->H);
    return FLEX_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

namespace {

flex_status check_util_bm(const flex_block_mask* bm) {
    if (!bm) return fail(FLEX_ERR_NULL, "bm must not be NULL");
    if (flex_status s = check_bm_arrays(bm)) return s;
    if (bm->B < 1 || bm->H < 1 || bm->num_q_blocks < 1 || bm->num_kv_blocks < 1 || bm->q_block < 1 ||
        bm->kv_block < 1 || bm->B > 65535 || bm->H > 65535)
        return fail(FLEX_ERR_BLOCKMASK, "block mask dims out of range");
    if (bm->num_kv_blocks > 65536)
        return fail(FLEX_ERR_UNSUPPORTED, "at most 65536 KV blocks per row (got %d)", bm->num_kv_blocks);
    if ((int64_t)bm->B * bm->H * bm->num_q_blocks >= (int64_t(1) << 31) ||
        (int64_t)bm->B * bm->H * bm->num_q_blocks * bm->num_kv_blocks >= (int64_t(1) << 40))
        return fail(FLEX_ERR_UNSUPPORTED, "block mask too large");
    return FLEX_OK;
}

UtilArgs util_args(const flex_block_mask* bm) {
    UtilArgs a;
    a.kv_num = bm->kv_num_blocks;
    a.kv_idx = bm->kv_indices;
    a.full_num = bm->full_kv_num_blocks;
    a.full_idx = bm->full_kv_indices;
    a.Bm = bm->B;
    a.Hm = bm->H;
    a.nQB = bm->num_q_blocks;
    a.nKB = bm->num_kv_blocks;
    return a;
}

UtilOut util_out(const flex_block_mask* o) { return UtilOut{o->kv_num_blocks, o->kv_indices, o->full_kv_num_blocks, o->full_kv_indices}; }

flex_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(FLEX_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return FLEX_OK;
}

}  // namespace

extern "C" {

const char* flex_status_string(int32_t s) {
    switch (s) {
    case FLEX_OK: return "FLEX_OK";
    case FLEX_ERR_NULL: return "FLEX_ERR_NULL";
    case FLEX_ERR_SHAPE: return "FLEX_ERR_SHAPE";
    case FLEX_ERR_GQA: return "FLEX_ERR_GQA";
    case FLEX_ERR_BLOCKMASK: return "FLEX_ERR_BLOCKMASK";
    case FLEX_ERR_UNSUPPORTED: return "FLEX_ERR_UNSUPPORTED";
    case FLEX_ERR_LAYOUT: return "FLEX_ERR_LAYOUT";
    case FLEX_ERR_WORKSPACE: return "FLEX_ERR_WORKSPACE";
    case FLEX_ERR_HIP: return "FLEX_ERR_HIP";
    case FLEX_ERR_PARAM: return "FLEX_ERR_PARAM";
    default: return "FLEX_ERR_UNKNOWN";
    }
}

const char* flex_last_error(void) { return g_last_error.c_str(); }

flex_status flex_blockmask_build(const flex_mask_params* mask, int64_t L, int64_t S, const flex_block_mask* bm,
                                 void* stream) {
    g_last_error.clear();
    if (!mask || !bm) return fail(FLEX_ERR_NULL, "mask and bm must not be NULL");
    if (flex_status s = check_bm_arrays(bm)) return s;
    if (L < 1 || S < 1 || L >= kMaxLen || S >= kMaxLen)
        return fail(FLEX_ERR_SHAPE, "L=%lld S=%lld must be in [1, 2^30)", (long long)L, (long long)S);
    if (flex_status s = check_bm_dims(bm, L, S)) return s;
    if (bm->num_kv_blocks > 65536)
        return fail(FLEX_ERR_UNSUPPORTED, "at most 65536 KV blocks per row (got %d)", bm->num_kv_blocks);
    if (bm->num_q_blocks > 65535 || (int64_t)bm->B * bm->H > 65535)
        return fail(FLEX_ERR_UNSUPPORTED, "at most 65535 Q blocks and 65535 (B x H) mask rows (got %d, %d x %d)",
                    bm->num_q_blocks, bm->B, bm->H);
    if (flex_status s = check_mask(mask, L, S)) return s;

    BuildArgs a;
    a.mask = to_mask_args(mask);
    a.L = (int)L;
    a.S = (int)S;
    a.q_block = bm->q_block;
    a.kv_block = bm->kv_block;
    a.nQB = bm->num_q_blocks;
    a.nKB = bm->num_kv_blocks;
    a.Bm = bm->B;
    a.Hm = bm->H;
    a.kv_num = bm->kv_num_blocks;
    a.kv_idx = bm->kv_indices;
    a.full_num = bm->full_kv_num_blocks;
    a.full_idx = bm->full_kv_indices;
    (void)hipGetLastError();
    hipError_t e = launch_blockmask_build(a, as_stream(stream));
    if (e != hipSuccess) return fail(FLEX_ERR_HIP, "block mask build launch failed: %s", hipGetErrorString(e));
    return FLEX_OK;
}

static flex_status check_fwd(const void* q, const void* k, const void* v, int32_t dtype, int32_t B, int32_t Hq,
                             int32_t Hkv, int64_t L, int64_t S, int32_t D, const int64_t* qs, const int64_t* ks,
                             const int64_t* vs, const flex_score_params* score, const flex_mask_params* mask,
                             const flex_block_mask* bm, const void* out, const float* lse) {
    if (!q || !k || !v || !out) return fail(FLEX_ERR_NULL, "q, k, v and out must not be NULL");
    if (!qs || !ks || !vs) return fail(FLEX_ERR_NULL, "stride arrays must not be NULL");
    if (!score || !mask || !bm) return fail(FLEX_ERR_NULL, "score, mask and bm must not be NULL");
    if (flex_status s = check_bm_arrays(bm)) return s;
    if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || S < 1 || L >= kMaxLen || S >= kMaxLen)
        return fail(FLEX_ERR_SHAPE, "sizes must be positive and L, S < 2^30 (B=%d Hq=%d Hkv=%d L=%lld S=%lld)", B,
                    Hq, Hkv, (long long)L, (long long)S);
    if (Hq % Hkv != 0) return fail(FLEX_ERR_GQA, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (dtype != FLEX_F32 && dtype != FLEX_BF16) return fail(FLEX_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
    if (D != 64 && D != 128) return fail(FLEX_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", D);
    if (flex_status s = check_bm_dims(bm, L, S)) return s;
    if (bm->B != 1 && bm->B != B) return fail(FLEX_ERR_BLOCKMASK, "block mask B=%d must be 1 or %d", bm->B, B);
    if (bm->H != 1 && bm->H != Hq) return fail(FLEX_ERR_BLOCKMASK, "block mask H=%d must be 1 or Hq=%d", bm->H, Hq);
    if (bm->q_block != 16 && bm->q_block != 32 && bm->q_block != 64 && bm->q_block != 128)
        return fail(FLEX_ERR_UNSUPPORTED, "q_block %d not supported (16, 32, 64, 128)", bm->q_block);
    if (bm->kv_block % 64 != 0) return fail(FLEX_ERR_UNSUPPORTED, "kv_block %d must be a multiple of 64", bm->kv_block);
    if ((int64_t)bm->num_q_blocks * B * Hq >= 2147483647LL)
        return fail(FLEX_ERR_SHAPE, "too many (Q block, head, batch) work items");
    const int64_t chunk = dtype == FLEX_BF16 ? 8 : 4;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(FLEX_ERR_LAYOUT, "q, k, v and out must be 16-byte aligned");
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(FLEX_ERR_LAYOUT, "lse must be 4-byte aligned");
    for (int i = 0; i < 3; ++i)
        if (qs[i] % chunk || ks[i] % chunk || vs[i] % chunk || qs[i] < 0 || ks[i] < 0 || vs[i] < 0)
            return fail(FLEX_ERR_LAYOUT, "strides must be non-negative multiples of %lld elements", (long long)chunk);
    const int64_t elem = dtype == FLEX_BF16 ? 2 : 4;
    if (ks[2] * elem * 64 >= (int64_t(1) << 31) || vs[2] * elem * 64 >= (int64_t(1) << 31))
        return fail(FLEX_ERR_UNSUPPORTED, "K/V row strides above 2^25 bytes are not supported");
    if (S * std::max(ks[2], (int64_t)D) * elem >= (int64_t(1) << 31) ||
        S * std::max(vs[2], (int64_t)D) * elem >= (int64_t(1) << 31))
        return fail(FLEX_ERR_UNSUPPORTED, "one K or V head slice (S x row stride) must stay below 2 GiB");
    if (score->kind < FLEX_SCORE_NONE || score->kind > FLEX_SCORE_ALIBI)
        return fail(FLEX_ERR_PARAM, "unknown score kind %d", score->kind);
    const bool capped = score->kind == FLEX_SCORE_SOFTCAP || score->kind == FLEX_SCORE_SOFTCAP_ALIBI;
    const bool alibi = score->kind == FLEX_SCORE_SOFTCAP_ALIBI || score->kind == FLEX_SCORE_ALIBI;
    if (capped && !(score->cap > 0.0f && std::isfinite(score->cap)))
        return fail(FLEX_ERR_PARAM, "soft-cap needs a finite cap > 0");
    if (alibi && !std::isfinite(score->alibi_m)) return fail(FLEX_ERR_PARAM, "alibi_m must be finite");
    if (flex_status s = check_mask(mask, L, S)) return s;
    if (program_uses(mask, FLEX_PRED_HEAD_LT) && bm->H != Hq)
        return fail(FLEX_ERR_BLOCKMASK, "the mask reads the query head: block mask H=%d must be Hq=%d", bm->H, Hq);
    if (per_batch(mask) && bm->B != B)
        return fail(FLEX_ERR_BLOCKMASK, "per-batch offsets or lengths: block mask B=%d must be B=%d", bm->B, B);
    return FLEX_OK;
}

size_t flex_attn_fwd_workspace_bytes(int32_t dtype, int32_t B, int32_t Hq, int32_t Hkv, int64_t L, int64_t S,
                                     int32_t D, const flex_block_mask* bm) {
    if (!bm || B < 1 || Hq < 1 || Hkv < 1 || L < 1 || S < 1 || L >= kMaxLen || S >= kMaxLen || Hq % Hkv) return 0;
    if ((dtype != FLEX_F32 && dtype != FLEX_BF16) || (D != 64 && D != 128)) return 0;
    return attn_fwd_workspace_bytes(dtype, B, Hq, Hkv, (int)L, (int)S, D, bm->q_block, bm->kv_block,
                                    bm->num_kv_blocks, bm->B, bm->H);
}

flex_status flex_attn_fwd(const void* q, const void* k, const void* v, int32_t dtype, int32_t B, int32_t Hq,
                          int32_t Hkv, int64_t L, int64_t S, int32_t D, const int64_t q_strides[3],
                          const int64_t k_strides[3], const int64_t v_strides[3], float scale,
                          const flex_score_params* score, const flex_mask_params* mask, const flex_block_mask* bm,
                          void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    return flex_attn_fwd_aux(q, k, v, dtype, B, Hq, Hkv, L, S, D, q_strides, k_strides, v_strides, scale, score, mask,
                             bm, out, lse, nullptr, workspace, workspace_bytes, stream);
}

// Page geometry of a paged K/V pool (both passes); page_shift = log2(page_size).
static flex_status check_pages(const flex_kv_pages* pages, int32_t dtype, int32_t B, int64_t S, int32_t D,
                               const int64_t k_strides[3], const int64_t v_strides[3], int* page_shift) {
    if (!pages->page_table) return fail(FLEX_ERR_NULL, "page_table must not be NULL");
    if (reinterpret_cast<uintptr_t>(pages->page_table) & 3u)
        return fail(FLEX_ERR_LAYOUT, "page_table must be 4-byte aligned");
    const int32_t ps = pages->page_size;
    if (ps < 64 || ps > (1 << 20) || (ps & (ps - 1)))
        return fail(FLEX_ERR_PARAM, "page_size must be a power of two in [64, 2^20] (got %d)", ps);
    *page_shift = 0;
    while ((1 << *page_shift) < ps) ++*page_shift;
    if (pages->num_pages < 1 || pages->max_pages < 1 || (int64_t)pages->max_pages * ps < S)
        return fail(FLEX_ERR_PARAM, "max_pages * page_size must cover S and num_pages be >= 1");
    if ((int64_t)B * pages->max_pages >= (int64_t(1) << 31)) return fail(FLEX_ERR_PARAM, "page table too large");
    const int64_t elem = dtype == FLEX_BF16 ? 2 : 4;
    if ((int64_t)ps * std::max(k_strides[2], (int64_t)D) * elem >= (int64_t(1) << 31) ||
        (int64_t)ps * std::max(v_strides[2], (int64_t)D) * elem >= (int64_t(1) << 31))
        return fail(FLEX_ERR_UNSUPPORTED, "one page of one head must stay below 2 GiB");
    return FLEX_OK;
}

static flex_status fwd_common(const void* q, const void* k, const void* v, int32_t dtype, int32_t B, int32_t Hq,
                              int32_t Hkv, int64_t L, int64_t S, int32_t D, const int64_t q_strides[3],
                              const int64_t k_strides[3], const int64_t v_strides[3], float scale,
                              const flex_score_params* score, const flex_mask_params* mask,
                              const flex_block_mask* bm, const flex_kv_pages* pages, void* out, float* lse,
                              float* max_scores, void* workspace, size_t workspace_bytes, void* stream) {
    if (flex_status s = check_fwd(q, k, v, dtype, B, Hq, Hkv, L, S, D, q_strides, k_strides, v_strides, score, mask,
                                  bm, out, lse))
        return s;
    int page_shift = 0;
    if (pages)
        if (flex_status s = check_pages(pages, dtype, B, S, D, k_strides, v_strides, &page_shift)) return s;
    if (!std::isfinite(scale)) return fail(FLEX_ERR_PARAM, "scale must be finite");
    if (max_scores && (reinterpret_cast<uintptr_t>(max_scores) & 3u))
        return fail(FLEX_ERR_LAYOUT, "max_scores must be 4-byte aligned");
    const size_t need = attn_fwd_workspace_bytes(dtype, B, Hq, Hkv, (int)L, (int)S, D, bm->q_block, bm->kv_block,
                                                 bm->num_kv_blocks, bm->B, bm->H);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(FLEX_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
    if (need > 0 && !aligned16(workspace)) return fail(FLEX_ERR_LAYOUT, "workspace must be 16-byte aligned");

    FwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    a.max_scores = max_scores;
    a.q_sb = q_strides[0]; a.q_sh = q_strides[1]; a.q_sr = q_strides[2];
    a.k_sb = k_strides[0]; a.k_sh = k_strides[1]; a.k_sr = k_strides[2];
    a.v_sb = v_strides[0]; a.v_sh = v_strides[1]; a.v_sr = v_strides[2];
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.L = (int)L;
    a.S = (int)S;
    a.group = Hq / Hkv;
    a.scale = scale > 0.0f ? scale : 1.0f / std::sqrt((float)D);
    a.score_kind = score->kind;
    const bool capped = score->kind == FLEX_SCORE_SOFTCAP || score->kind == FLEX_SCORE_SOFTCAP_ALIBI;
    a.cap = capped ? score->cap : 1.0f;
    a.alibi_m = score->alibi_m;
    a.sc = score_consts(a.scale, a.cap, a.score_kind);
    a.mask = to_mask_args(mask);
    a.kv_num = bm->kv_num_blocks;
    a.kv_idx = bm->kv_indices;
    a.full_num = bm->full_kv_num_blocks;
    a.full_idx = bm->full_kv_indices;
    a.Bm = bm->B;
    a.Hm = bm->H;
    a.nQB = bm->num_q_blocks;
    a.nKB = bm->num_kv_blocks;
    a.q_block = bm->q_block;
    a.kv_block = bm->kv_block;
    // Fixed softmax reference when the soft-cap bounds every visible score:
    // g < cap always, and a distance bias alpha*(kv - q) <= 0 under causal-type
    // masks.  With the bias, a row's largest weight must also stay in range:
    // that holds when every row that sees a key keeps its own (bias 0) key,
    // which needs q_offset + L <= S and a mask whose every clause is true on
    // the diagonal; the range [ref - 120, ref + 64] (base 2) then loses
    // nothing.  A mask that can hide the diagonal while showing far keys (for
    // example causal AND kv < 4) takes the moving reference instead.
    a.ref_mode = 0;
    a.ref_fixed = 0.0f;
    if (dtype == FLEX_BF16 && capped && max_scores == nullptr) {
        const double c2 = (double)score->cap * 1.4426950408889634;
        bool ok = c2 <= 92.0;
        if (score->kind == FLEX_SCORE_SOFTCAP_ALIBI)
            ok = ok && mask_implies_causal(mask) && mask_keeps_diagonal(mask) && mask->q_offset + L <= S &&
                 !per_batch(mask);
        if (ok) {
            a.ref_mode = 1;
            a.ref_fixed = (float)(c2 <= 63.0 ? c2 : 120.0 - c2);
        }
    }
    a.page_table = pages ? pages->page_table : nullptr;
    a.page_shift = page_shift;
    a.max_pages = pages ? pages->max_pages : 0;
    a.num_pages = pages ? pages->num_pages : 0;
    a.ksplit = prefill_ksplit(dtype, B, Hq, bm->num_q_blocks, bm->q_block, D);
    // Packed documents give Q blocks tile counts that do not follow the block
    // index; launching the longest documents first shortens the tail of the
    // grid.  Not for mask programs: on the chunked workload a longest-first
    // order spread the resident blocks over every chunk and was 3.5 % slower.
    // One shared list of row blocks only (B = H = 1 masks).
    a.longest_first = mask->kind == FLEX_MASK_DOC_CAUSAL && bm->B == 1 && bm->H == 1 &&
                      bm->num_q_blocks <= kLongestFirstMaxBlocks;
    a.splits = decode_splits(dtype, B, Hq, Hkv, (int)L, D, bm->q_block, bm->kv_block, bm->num_kv_blocks, bm->H);
    a.ws_acc = nullptr;
    a.ws_ml = nullptr;
    if (a.splits > 0) {
        const size_t rows = (size_t)a.splits * B * Hq * L;
        a.ws_acc = reinterpret_cast<float*>(workspace);
        a.ws_ml = a.ws_acc + rows * D;
    }
    (void)hipGetLastError();
    hipError_t e = launch_attn_fwd(dtype, D, a, as_stream(stream));
    if (e != hipSuccess) return fail(FLEX_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
    return FLEX_OK;
}

flex_status flex_attn_fwd_aux(const void* q, const void* k, const void* v, int32_t dtype, int32_t B, int32_t Hq,
                              int32_t Hkv, int64_t L, int64_t S, int32_t D, const int64_t q_strides[3],
                              const int64_t k_strides[3], const int64_t v_strides[3], float scale,
                              const flex_score_params* score, const flex_mask_params* mask,
                              const flex_block_mask* bm, void* out, float* lse, float* max_scores, void* workspace,
                              size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    return fwd_common(q, k, v, dtype, B, Hq, Hkv, L, S, D, q_strides, k_strides, v_strides, scale, score, mask, bm,
                      nullptr, out, lse, max_scores, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// The forward without a caller workspace, for callers that cannot allocate.
// The split-KV decode partials go to a file-scope device array instead; each
// GPU holds its own copy, found once per device through hipGetSymbolAddress.
// Nothing in it must start at zero: every decode workgroup writes all of its
// rows' partials (zero-tile splits write an empty partial) before the combine
// kernel, later on the same stream, reads them.
namespace {

constexpr size_t kScratchBytes = FLEX_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (set up on the first call
// per device, with that device current).
flex_status scratch_for_device(int dev, void** ptr) {
    if (dev < 0 || dev >= kMaxDevices) return fail(FLEX_ERR_PARAM, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void* p = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur >= 0 && cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess || p == nullptr)
            return fail(FLEX_ERR_HIP, "scratch array of device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return FLEX_OK;
}

}  // namespace

flex_status flex_attn_fwd_noalloc(const void* q, const void* k, const void* v, int32_t dtype, int32_t B, int32_t Hq,
                                  int32_t Hkv, int64_t L, int64_t S, int32_t D, const int64_t q_strides[3],
                                  const int64_t k_strides[3], const int64_t v_strides[3], float scale,
                                  const flex_score_params* score, const flex_mask_params* mask,
                                  const flex_block_mask* bm, void* out, float* lse, void* stream) {
    g_last_error.clear();
    if (flex_status s = check_fwd(q, k, v, dtype, B, Hq, Hkv, L, S, D, q_strides, k_strides, v_strides, score, mask,
                                  bm, out, lse))
        return s;
    const size_t need = attn_fwd_workspace_bytes(dtype, B, Hq, Hkv, (int)L, (int)S, D, bm->q_block, bm->kv_block,
                                                 bm->num_kv_blocks, bm->B, bm->H);
    if (need > kScratchBytes)
        return fail(FLEX_ERR_WORKSPACE, "this call needs %zu bytes of scratch, above the %zu of the no-allocation entry",
                    need, kScratchBytes);
    void* ws = nullptr;
    if (need > 0) {
        int dev = -1;
        hipError_t e = stream ? hipStreamGetDevice(as_stream(stream), &dev) : hipGetDevice(&dev);
        if (e != hipSuccess) return fail(FLEX_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
        if (flex_status st = scratch_for_device(dev, &ws)) return st;
    }
    return fwd_common(q, k, v, dtype, B, Hq, Hkv, L, S, D, q_strides, k_strides, v_strides, scale, score, mask, bm,
                      nullptr, out, lse, nullptr, ws, need > 0 ? kScratchBytes : 0, stream);
}

flex_status flex_attn_fwd_paged(const void* q, const void* k, const void* v, int32_t dtype, int32_t B, int32_t Hq,
                                int32_t Hkv, int64_t L, int64_t S, int32_t D, const int64_t q_strides[3],
                                const int64_t k_strides[3], const int64_t v_strides[3], float scale,
                                const flex_score_params* score, const flex_mask_params* mask,
                                const flex_block_mask* bm, const flex_kv_pages* pages, void* out, float* lse,
                                float* max_scores, void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    if (!pages) return fail(FLEX_ERR_NULL, "pages must not be NULL");
    return fwd_common(q, k, v, dtype, B, Hq, Hkv, L, S, D, q_strides, k_strides, v_strides, scale, score, mask, bm,
                      pages, out, lse, max_scores, workspace, workspace_bytes, stream);
}

flex_status flex_blockmask_transpose(const flex_block_mask* bm, const flex_block_mask_q* bmq, void* stream) {
    g_last_error.clear();
    if (!bm || !bmq) return fail(FLEX_ERR_NULL, "bm and bmq must not be NULL");
    if (flex_status s = check_bm_arrays(bm)) return s;
    if (!bmq->q_num_blocks || !bmq->q_indices || !bmq->full_q_num_blocks || !bmq->full_q_indices)
        return fail(FLEX_ERR_NULL, "Q-side block mask arrays must not be NULL");
    if (bm->B < 1 || bm->H < 1 || bm->B > 65535 || bm->H > 65535 || bm->num_q_blocks < 1 || bm->num_kv_blocks < 1 ||
        bm->q_block < 1 || bm->kv_block < 1)
        return fail(FLEX_ERR_BLOCKMASK, "block mask dims out of range");
    if (bmq->B != bm->B || bmq->H != bm->H || bmq->q_block != bm->q_block || bmq->kv_block != bm->kv_block ||
        bmq->num_q_blocks != bm->num_q_blocks || bmq->num_kv_blocks != bm->num_kv_blocks)
        return fail(FLEX_ERR_BLOCKMASK, "Q-side block mask dims differ from the block mask's");
    if ((int64_t)bm->B * bm->H * bm->num_kv_blocks * bm->num_q_blocks >= (int64_t(1) << 31))
        return fail(FLEX_ERR_BLOCKMASK, "block mask lists above 2^31 entries are not supported");
    TransposeArgs a;
    a.kv_num = bm->kv_num_blocks;
    a.kv_idx = bm->kv_indices;
    a.full_num = bm->full_kv_num_blocks;
    a.full_idx = bm->full_kv_indices;
    a.q_num = bmq->q_num_blocks;
    a.q_idx = bmq->q_indices;
    a.fq_num = bmq->full_q_num_blocks;
    a.fq_idx = bmq->full_q_indices;
    a.Bm = bm->B;
    a.Hm = bm->H;
    a.nQB = bm->num_q_blocks;
    a.nKB = bm->num_kv_blocks;
    (void)hipGetLastError();
    hipError_t e = launch_blockmask_transpose(a, as_stream(stream));
    if (e != hipSuccess) return fail(FLEX_ERR_HIP, "block mask transpose launch failed: %s", hipGetErrorString(e));
    return FLEX_OK;
}

size_t flex_attn_bwd_workspace_bytes(int32_t dtype, int32_t B, int32_t Hq, int32_t Hkv, int64_t L, int64_t S,
                                     int32_t D, const flex_block_mask* bm) {
    if (!bm || B < 1 || Hq < 1 || Hkv < 1 || L < 1 || S < 1 || L >= kMaxLen || S >= kMaxLen || Hq % Hkv) return 0;
    if ((dtype != FLEX_F32 && dtype != FLEX_BF16) || (D != 64 && D != 128)) return 0;
    if ((bm->q_block != 64 && bm->q_block != 128) || bm->kv_block < 64 || bm->kv_block % 64) return 0;
    return attn_bwd_workspace_bytes(B, Hq, Hkv, (int)L, (int)S, D, bm->q_block, bm->kv_block, bm->num_q_blocks,
                                    bm->num_kv_blocks);
}

static flex_status bwd_common(const void* q, const void* k, const void* v, const flex_kv_pages* pages,
                              const void* out, const void* dout, const float* lse, int32_t dtype, int32_t B,
                              int32_t Hq, int32_t Hkv, int64_t L, int64_t S, int32_t D, const int64_t q_strides[3],
                              const int64_t k_strides[3], const int64_t v_strides[3], float scale,
                              const flex_score_params* score, const flex_mask_params* mask, const flex_block_mask* bm,
                              const flex_block_mask_q* bmq, void* dq, void* dk, void* dv, void* workspace,
                              size_t workspace_bytes, void* stream) {
    if (flex_status s = check_fwd(q, k, v, dtype, B, Hq, Hkv, L, S, D, q_strides, k_strides, v_strides, score, mask,
                                  bm, out, lse))
        return s;
    int page_shift = 0;
    if (pages)
        if (flex_status s = check_pages(pages, dtype, B, S, D, k_strides, v_strides, &page_shift)) return s;
    if (!dout || !lse || !dq || !dk || !dv) return fail(FLEX_ERR_NULL, "dout, lse, dq, dk and dv must not be NULL");
    if (!bmq) return fail(FLEX_ERR_NULL, "bmq must not be NULL");
    if (!bmq->q_num_blocks || !bmq->q_indices || !bmq->full_q_num_blocks || !bmq->full_q_indices)
        return fail(FLEX_ERR_NULL, "Q-side block mask arrays must not be NULL");
    if (bmq->B != bm->B || bmq->H != bm->H || bmq->q_block != bm->q_block || bmq->kv_block != bm->kv_block ||
        bmq->num_q_blocks != bm->num_q_blocks || bmq->num_kv_blocks != bm->num_kv_blocks)
        return fail(FLEX_ERR_BLOCKMASK, "Q-side block mask dims differ from the block mask's");
    if (bm->q_block != 64 && bm->q_block != 128)
        return fail(FLEX_ERR_UNSUPPORTED, "the backward pass needs q_block 64 or 128 (got %d)", bm->q_block);
    if (!std::isfinite(scale)) return fail(FLEX_ERR_PARAM, "scale must be finite");
    if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return fail(FLEX_ERR_LAYOUT, "dout, dq, dk and dv must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(FLEX_ERR_LAYOUT, "lse must be 4-byte aligned");
    const int64_t elem = dtype == FLEX_BF16 ? 2 : 4;
    if (L * std::max(q_strides[2], (int64_t)D) * elem >= (int64_t(1) << 31) || L * D * elem >= (int64_t(1) << 31))
        return fail(FLEX_ERR_UNSUPPORTED, "one Q or dout head slice (L x row stride) must stay below 2 GiB");
    if (q_strides[2] * elem * 128 >= (int64_t(1) << 31))
        return fail(FLEX_ERR_UNSUPPORTED, "Q row strides above 2^24 bytes are not supported");
    const size_t need = attn_bwd_workspace_bytes(B, Hq, Hkv, (int)L, (int)S, D, bm->q_block, bm->kv_block,
                                                 bm->num_q_blocks, bm->num_kv_blocks);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(FLEX_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
    if (!aligned16(workspace)) return fail(FLEX_ERR_LAYOUT, "workspace must be 16-byte aligned");

    BwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.dout = dout;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.Lp = (int)((L + 127) / 128 * 128);
    a.ws_lse2 = reinterpret_cast<float*>(workspace);
    a.ws_dsum = a.ws_lse2 + (size_t)B * Hq * a.Lp;
    a.kv_splits = bwd_kv_splits(Hq / Hkv, bm->num_q_blocks, bm->q_block);
    a.chunk_tiles = kBwdChunkTiles;
    a.ws_part = a.kv_splits > 1 ? a.ws_dsum + (size_t)B * Hq * a.Lp : nullptr;
    a.q_sb = q_strides[0]; a.q_sh = q_strides[1]; a.q_sr = q_strides[2];
    a.k_sb = k_strides[0]; a.k_sh = k_strides[1]; a.k_sr = k_strides[2];
    a.v_sb = v_strides[0]; a.v_sh = v_strides[1]; a.v_sr = v_strides[2];
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.L = (int)L;
    a.S = (int)S;
    a.group = Hq / Hkv;
    a.scale = scale > 0.0f ? scale : 1.0f / std::sqrt((float)D);
    a.score_kind = score->kind;
    a.alibi_m = score->alibi_m;
    const bool capped = score->kind == FLEX_SCORE_SOFTCAP || score->kind == FLEX_SCORE_SOFTCAP_ALIBI;
    a.sc = score_consts(a.scale, capped ? score->cap : 1.0f, score->kind);
    a.mask = to_mask_args(mask);
    a.kv_num = bm->kv_num_blocks;
    a.kv_idx = bm->kv_indices;
    a.full_num = bm->full_kv_num_blocks;
    a.full_idx = bm->full_kv_indices;
    a.q_num = bmq->q_num_blocks;
    a.q_idx = bmq->q_indices;
    a.fq_num = bmq->full_q_num_blocks;
    a.fq_idx = bmq->full_q_indices;
    a.Bm = bm->B;
    a.Hm = bm->H;
    a.nQB = bm->num_q_blocks;
    a.nKB = bm->num_kv_blocks;
    a.q_block = bm->q_block;
    a.kv_block = bm->kv_block;
    a.page_table = pages ? pages->page_table : nullptr;
    a.page_shift = page_shift;
    a.max_pages = pages ? pages->max_pages : 0;
    a.num_pages = pages ? pages->num_pages : 0;
    (void)hipGetLastError();
    hipError_t e = launch_attn_bwd(dtype, D, a, as_stream(stream));
    if (e != hipSuccess) return fail(FLEX_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
    return FLEX_OK;
}

flex_status flex_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                          const float* lse, int32_t dtype, int32_t B, int32_t Hq, int32_t Hkv, int64_t L, int64_t S,
                          int32_t D, const int64_t q_strides[3], const int64_t k_strides[3],
                          const int64_t v_strides[3], float scale, const flex_score_params* score,
                          const flex_mask_params* mask, const flex_block_mask* bm, const flex_block_mask_q* bmq,
                          void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    return bwd_common(q, k, v, nullptr, out, dout, lse, dtype, B, Hq, Hkv, L, S, D, q_strides, k_strides, v_strides,
                      scale, score, mask, bm, bmq, dq, dk, dv, workspace, workspace_bytes, stream);
}

flex_status flex_attn_bwd_paged(const void* q, const void* k, const void* v, const flex_kv_pages* pages,
                                const void* out, const void* dout, const float* lse, int32_t dtype, int32_t B,
                                int32_t Hq, int32_t Hkv, int64_t L, int64_t S, int32_t D, const int64_t q_strides[3],
                                const int64_t k_strides[3], const int64_t v_strides[3], float scale,
                                const flex_score_params* score, const flex_mask_params* mask,
                                const flex_block_mask* bm, const flex_block_mask_q* bmq, void* dq, void* dk, void* dv,
                                void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    if (!pages) return fail(FLEX_ERR_NULL, "pages must not be NULL");
    return bwd_common(q, k, v, pages, out, dout, lse, dtype, B, Hq, Hkv, L, S, D, q_strides, k_strides, v_strides,
                      scale, score, mask, bm, bmq, dq, dk, dv, workspace, workspace_bytes, stream);
}

flex_status flex_blockmask_to_dense(const flex_block_mask* bm, int32_t* dense, void* stream) {
    g_last_error.clear();
    if (flex_status s = check_util_bm(bm)) return s;
    if (!dense) return fail(FLEX_ERR_NULL, "dense must not be NULL");
    (void)hipGetLastError();
    return launched(launch_blockmask_to_dense(util_args(bm), dense, as_stream(stream)), "to_dense");
}

flex_status flex_blockmask_grid(const flex_block_mask* bm, int32_t grid_rows, int32_t grid_cols, int8_t* grid,
                                void* stream) {
    g_last_error.clear();
    if (flex_status s = check_util_bm(bm)) return s;
    if (!grid) return fail(FLEX_ERR_NULL, "grid must not be NULL");
    if (grid_rows < 1 || grid_cols < 1) return fail(FLEX_ERR_SHAPE, "grid_rows and grid_cols must be >= 1");
    const int wr = (int)ceil_div(bm->num_q_blocks, grid_rows), wc = (int)ceil_div(bm->num_kv_blocks, grid_cols);
    (void)hipGetLastError();
    return launched(launch_blockmask_grid(util_args(bm), wr, wc, grid, as_stream(stream)), "grid");
}

flex_status flex_blockmask_sparsity(const flex_block_mask* bm, double* percent, void* stream) {
    g_last_error.clear();
    if (flex_status s = check_util_bm(bm)) return s;
    if (!percent) return fail(FLEX_ERR_NULL, "percent must not be NULL");
    if (reinterpret_cast<uintptr_t>(percent) & 7u) return fail(FLEX_ERR_LAYOUT, "percent must be 8-byte aligned");
    (void)hipGetLastError();
    return launched(launch_blockmask_sparsity(util_args(bm), percent, as_stream(stream)), "sparsity");
}

flex_status flex_blockmask_slice(const flex_block_mask* bm, const int32_t ranges[6], const flex_block_mask* out,
                                 void* stream) {
    g_last_error.clear();
    if (flex_status s = check_util_bm(bm)) return s;
    if (!ranges || !out) return fail(FLEX_ERR_NULL, "ranges and out must not be NULL");
    if (flex_status s = check_bm_arrays(out)) return s;
    const int32_t* r = ranges;
    if (r[0] < 0 || r[1] > bm->B || r[0] >= r[1] || r[2] < 0 || r[3] > bm->H || r[2] >= r[3] || r[4] < 0 ||
        r[5] > bm->num_q_blocks || r[4] >= r[5])
        return fail(FLEX_ERR_BLOCKMASK, "slice ranges [%d,%d) x [%d,%d) x [%d,%d) are empty or outside %d x %d x %d",
                    r[0], r[1], r[2], r[3], r[4], r[5], bm->B, bm->H, bm->num_q_blocks);
    if (out->B != r[1] - r[0] || out->H != r[3] - r[2] || out->num_q_blocks != r[5] - r[4] ||
        out->num_kv_blocks != bm->num_kv_blocks || out->q_block != bm->q_block || out->kv_block != bm->kv_block)
        return fail(FLEX_ERR_BLOCKMASK, "out dims do not match the slice");
    SliceArgs sa{r[0], r[2], r[4], r[1] - r[0], r[3] - r[2], r[5] - r[4]};
    (void)hipGetLastError();
    return launched(launch_blockmask_slice(util_args(bm), sa, util_out(out), as_stream(stream)), "slice");
}

flex_status flex_blockmask_adjust(const flex_block_mask* bm, int64_t new_L, int64_t new_S, const flex_block_mask* out,
                                  void* stream) {
    g_last_error.clear();
    if (flex_status s = check_util_bm(bm)) return s;
    if (!out) return fail(FLEX_ERR_NULL, "out must not be NULL");
    if (flex_status s = check_bm_arrays(out)) return s;
    if (new_L < 1 || new_S < 1) return fail(FLEX_ERR_SHAPE, "new lengths must be positive");
    const int64_t nq = ceil_div(new_L, bm->q_block), nk = ceil_div(new_S, bm->kv_block);
    if (nq > bm->num_q_blocks || nk > bm->num_kv_blocks)
        return fail(FLEX_ERR_BLOCKMASK, "cropping to %lld x %lld needs %lld x %lld blocks, the mask has %d x %d",
                    (long long)new_L, (long long)new_S, (long long)nq, (long long)nk, bm->num_q_blocks,
                    bm->num_kv_blocks);
    if (out->B != bm->B || out->H != bm->H || out->q_block != bm->q_block || out->kv_block != bm->kv_block ||
        out->num_q_blocks != nq || out->num_kv_blocks != nk)
        return fail(FLEX_ERR_BLOCKMASK, "out dims do not match the cropped lengths");
    (void)hipGetLastError();
    return launched(launch_blockmask_adjust(util_args(bm), (int)nq, (int)nk, new_L % bm->q_block != 0,
                                            new_S % bm->kv_block != 0, util_out(out), as_stream(stream)),
                    "adjust");
}

}  // extern "C"
