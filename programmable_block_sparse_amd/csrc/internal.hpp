// Internal launch interfaces between the C-ABI layer (flexmi_api.hip) and the
// kernel translation units.  Everything here has been validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace flexmi {

struct BuildArgs {
    MaskArgs mask;
    int L, S;
    int q_block, kv_block;
    int nQB, nKB;
    int Bm, Hm;
    int* kv_num;
    int* kv_idx;
    int* full_num;
    int* full_idx;
};

hipError_t launch_blockmask_build(const BuildArgs& a, hipStream_t stream);

// Q-side lists of a block mask (the KV-side lists transposed).
struct TransposeArgs {
    const int* kv_num;
    const int* kv_idx;
    const int* full_num;
    const int* full_idx;
    int* q_num;
    int* q_idx;
    int* fq_num;
    int* fq_idx;
    int Bm, Hm, nQB, nKB;
};

hipError_t launch_blockmask_transpose(const TransposeArgs& a, hipStream_t stream);

// BlockMask utilities (blockmask_utils.hip): input lists, output lists, and
// the ranges of a slice.
struct UtilArgs {
    const int* kv_num;
    const int* kv_idx;
    const int* full_num;
    const int* full_idx;
    int Bm, Hm, nQB, nKB;
};
struct UtilOut {
    int* kv_num;
    int* kv_idx;
    int* full_num;
    int* full_idx;
};
struct SliceArgs {
    int b0, h0, r0;
    int batches, heads, rows;
};

hipError_t launch_blockmask_to_dense(const UtilArgs& a, int32_t* dense, hipStream_t stream);
hipError_t launch_blockmask_grid(const UtilArgs& a, int wr, int wc, int8_t* grid, hipStream_t stream);
hipError_t launch_blockmask_sparsity(const UtilArgs& a, double* percent, hipStream_t stream);
hipError_t launch_blockmask_slice(const UtilArgs& a, const SliceArgs& s, const UtilOut& o, hipStream_t stream);
hipError_t launch_blockmask_adjust(const UtilArgs& a, int nq, int nk, int edge_row, int edge_col, const UtilOut& o,
                                   hipStream_t stream);

// Constants of the score rule that depend only on scale and cap (computed on
// the host in double, rounded once).  Base-2 units: log2(e) is folded in.
struct ScoreConsts {
    float mul;        // NONE: scale*log2e; soft-cap exact path: 2*scale*log2e/cap
    float c2;         // cap*log2e
    float k0, k1, k2; // quintic path: g2 = acc*(k0 + k1*w + k2*w^2), w = acc^2
    float amax;       // quintic valid while |acc| <= amax
    float j0, j1;     // cubic path: g2 = acc*(j0 + j1*w)
    float amax1;      // cubic valid while |acc| <= amax1 (amax1 <= amax)
};

// Forward pass arguments (element strides; last dim contiguous).
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;
    float* max_scores;   // optional row maxima of the visible scores (natural units)
    int64_t q_sb, q_sh, q_sr;
    int64_t k_sb, k_sh, k_sr;
    int64_t v_sb, v_sh, v_sr;
    int B, Hq, Hkv, L, S, group;
    float scale;
    // score_mod
    int score_kind;
    float cap;
    float alibi_m;
    ScoreConsts sc;
    // mask_mod
    MaskArgs mask;
    // block mask
    const int* kv_num;
    const int* kv_idx;
    const int* full_num;
    const int* full_idx;
    int Bm, Hm, nQB, nKB, q_block, kv_block;
    // softmax reference: 0 = running (moved lazily), 1 = fixed at ref_fixed
    // (base 2), used when the soft-cap bounds every visible score
    int ref_mode;
    float ref_fixed;
    // prefill row layout: 1 = 64-row workgroups, key halves split across waves
    int ksplit;
    // prefill launch order: 1 = Q blocks of mask row 0 by tile count, largest
    // first (ties: higher block first); 0 = by block index, highest first
    int longest_first;
    // paged K/V pool (page_table == NULL: contiguous (B, Hkv, S, D) caches):
    // k, v point at pools of num_pages pages, k_sb / v_sb the page strides;
    // page_table[b][p] is the physical page of logical page p of batch b
    const int* page_table;
    int page_shift;     // log2(page size); a power of two >= 64
    int max_pages;
    int num_pages;
    // split-KV decode (splits == 0: prefill kernel)
    float* ws_acc;      // [splits][B][Hq][L][D] partial numerators
    float* ws_ml;       // [splits][B][Hq][L][4]  partial (base-2 reference, sum p, sum rounded p, max score)
    int splits;
};

// Prefill row layout for these sizes (see attn_fwd.hip): 1 = key-split.
int prefill_ksplit(int dtype, int B, int Hq, int nQB, int q_block, int D);
// Most Q blocks the prefill still orders longest document first (one block
// per thread of a workgroup).
constexpr int kLongestFirstMaxBlocks = 256;

// Number of key-range splits of the GQA-packed decode kernel for these sizes,
// or 0 when the prefill kernel is used.
// Host-side constants of the score rule for this scale and cap.
ScoreConsts score_consts(float scale, float cap, int score_kind);

int decode_splits(int dtype, int B, int Hq, int Hkv, int L, int D, int q_block, int kv_block, int nKB, int Hm);

// Per dtype / head-dimension launchers (one translation unit each).
hipError_t launch_attn_fwd_bf16_d64(const FwdArgs& a, hipStream_t stream);
hipError_t launch_attn_fwd_bf16_d128(const FwdArgs& a, hipStream_t stream);
hipError_t launch_attn_fwd_f32_d64(const FwdArgs& a, hipStream_t stream);
hipError_t launch_attn_fwd_f32_d128(const FwdArgs& a, hipStream_t stream);

// dtype: 0 fp32, 1 bf16.  Returns hipErrorInvalidValue for an unsupported
// combination (the host validated the combination before).
hipError_t launch_attn_fwd(int dtype, int D, const FwdArgs& a, hipStream_t stream);

// Workspace bytes for the split-KV path; 0 when the prefill kernel is used.
size_t attn_fwd_workspace_bytes(int dtype, int B, int Hq, int Hkv, int L, int S, int D,
                                int q_block, int kv_block, int nKB, int Bm, int Hm);

// Backward pass arguments.  q, k, v use element strides (last dim
// contiguous); out, dout, dq are contiguous (B, Hq, L, D), dk, dv contiguous
// (B, Hkv, S, D).
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* out;
    const void* dout;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    float* ws_lse2;     // [B][Hq][Lp] lse * log2(e); +inf for rows with no key and padding rows
    float* ws_dsum;     // [B][Hq][Lp] D_i = dout_i . out_i (0 for padding rows)
    float* ws_part;     // [kv_splits][B*Hkv*S/64 columns][2][64][D] fp32 partial dk, dv (kv_splits > 1)
    int Lp;             // L rounded up to a multiple of 128
    int kv_splits;      // most workgroups sharing one 64-key column of the key-major pass
    int chunk_tiles;    // Q-side tiles per share
    int64_t q_sb, q_sh, q_sr;
    int64_t k_sb, k_sh, k_sr;
    int64_t v_sb, v_sh, v_sr;
    int B, Hq, Hkv, L, S, group;
    float scale;
    int score_kind;
    float alibi_m;
    ScoreConsts sc;     // base-2 constants of the score rule (as for the forward)
    MaskArgs mask;
    const int* kv_num;  // KV-side lists (the query-major pass)
    const int* kv_idx;
    const int* full_num;
    const int* full_idx;
    const int* q_num;   // Q-side lists (the key-major pass)
    const int* q_idx;
    const int* fq_num;
    const int* fq_idx;
    int Bm, Hm, nQB, nKB, q_block, kv_block;
    // paged K/V (NULL page_table: contiguous): k, v are pools, k_sb / v_sb
    // the page strides; logical key j of batch b is row j % page_size of
    // page page_table[b * max_pages + j / page_size]
    const int* page_table;
    int page_shift, max_pages, num_pages;
};

// Q-side tiles one workgroup of the key-major pass takes before a column is
// shared: a column longer than that (keys every query sees, such as attention
// sinks or a prefix) would otherwise set the length of the whole pass.
constexpr int kBwdChunkTiles = 128;

// Key-major split bound and workspace bytes for these sizes (see attn_bwd.hip).
int bwd_kv_splits(int group, int nQB, int q_block);
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int L, int S, int D, int q_block, int kv_block, int nQB,
                                int nKB);

hipError_t launch_attn_bwd_bf16_d64(const BwdArgs& a, hipStream_t stream);
hipError_t launch_attn_bwd_bf16_d128(const BwdArgs& a, hipStream_t stream);
hipError_t launch_attn_bwd_f32_d64(const BwdArgs& a, hipStream_t stream);
hipError_t launch_attn_bwd_f32_d128(const BwdArgs& a, hipStream_t stream);
hipError_t launch_attn_bwd(int dtype, int D, const BwdArgs& a, hipStream_t stream);

}  // namespace flexmi
