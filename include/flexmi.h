/*
 * flexmi.h -- C ABI of the MI355X (gfx950) block-sparse attention library.
 *
 * The library computes the forward pass of programmable block-sparse attention
 * (the FlexAttention formulation) and its gradients:
 *
 *   s_ij  = scale * q_i . k_j
 *   z_ij  = g(s_ij, b, h, p_i, j)   if M(b, h, p_i, j)        else -inf
 *   o_i   = sum_j softmax_j(z_ij) v_j,   lse_i = log sum_j exp(z_ij)
 *
 * where g is a score_mod, M a mask_mod (true = attend) and p_i = i + q_offset
 * the logical position of query row i.  Source: charlestar blog "FlexAttention
 * score_mod / BlockMask", section on what one connection goes through (the
 * formula and the order: scaled score, then g, then visibility, then the
 * normalised sum of values) and its decode section (logical query position).
 * The call shape follows the 2kiu "PyTorch Flex Attention complete guide",
 * section 1.1 (query (B,Hq,L,E), key (B,Hkv,S,E), value (B,Hkv,S,Ev), scale,
 * GQA, output (B,Hq,L,Ev)) and section 2 (lse of shape (B,Hq,L)).
 *
 * score_mod and mask_mod are not arbitrary programs here: they are chosen from
 * a fixed menu (the enums below) with run-time parameters.
 *
 * Conventions for every entry point
 *   - Pointers named as device pointers must be HIP device memory (or memory
 *     the device can access); parameter structs are host memory read during
 *     the call only.  The caller owns every buffer.  The library keeps no
 *     state between calls, never allocates and never synchronises: work is
 *     enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *   - All argument checks run on the host before any HIP call, so an invalid
 *     call returns an error code and enqueues nothing.  A failing kernel
 *     launch returns FLEX_ERR_HIP.  flex_last_error() gives a one-line reason
 *     for the last failure on the calling thread.
 *   - Sizes are element counts; strides are element strides.
 */
#ifndef FLEXMI_H
#define FLEXMI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FLEX_OK = 0,
    FLEX_ERR_NULL = 1,         /* a required pointer is NULL */
    FLEX_ERR_SHAPE = 2,        /* non-positive or out-of-range size */
    FLEX_ERR_GQA = 3,          /* Hq is not a multiple of Hkv */
    FLEX_ERR_BLOCKMASK = 4,    /* block mask dims do not match L, S, B, Hq */
    FLEX_ERR_UNSUPPORTED = 5,  /* dtype, head dim, tile shape or menu entry not provided */
    FLEX_ERR_LAYOUT = 6,       /* pointer or stride not 16-byte aligned */
    FLEX_ERR_WORKSPACE = 7,    /* workspace missing or smaller than required */
    FLEX_ERR_HIP = 8,          /* a HIP call or kernel launch failed */
    FLEX_ERR_PARAM = 9         /* invalid mask or score parameter */
} flex_status;

typedef enum { FLEX_F32 = 0, FLEX_BF16 = 1 } flex_dtype;

/* mask_mod menu.  Each returns true when query position p may attend key j.
 *   NOOP                 always true (2kiu guide, section 4.4)
 *   CAUSAL               j <= p (quant67 "Causal Mask" article; with
 *                        q_offset = S - L this is the bottom-right alignment of
 *                        its section 4)
 *   CAUSAL_WINDOW_SINKS  j <= p and (p - j < window or j < sinks): a causal
 *                        window of `window` keys counting the query itself
 *                        (charlestar blog, pinned-version example) plus the
 *                        first `sinks` keys (tensorcad "Attention expressions",
 *                        Examples, sink window)
 *   DOC_CAUSAL           j <= p and doc_id[p] == doc_id[j] (charlestar blog,
 *                        packing section; quant67 article section 7 demo)
 *   PROGRAM              an AND of up to FLEX_MAX_CLAUSES clauses, each an OR
 *                        of up to FLEX_MAX_LITERALS predicates from the
 *                        flex_pred_kind list below: the and_masks / or_masks
 *                        composition of the 2kiu guide, section 4.3 (an AND
 *                        folds from true, an OR from false), which expresses
 *                        the mask column of the tensorcad "Attention
 *                        expressions" Examples table (prefix-LM, sink window,
 *                        chunked, every k-th key, half the heads global) */
typedef enum {
    FLEX_MASK_NOOP = 0,
    FLEX_MASK_CAUSAL = 1,
    FLEX_MASK_CAUSAL_WINDOW_SINKS = 2,
    FLEX_MASK_DOC_CAUSAL = 3,
    FLEX_MASK_PROGRAM = 4
} flex_mask_kind;

/* Predicates of a PROGRAM mask, on query position p (= row + q_offset), key j
 * and query head h:
 *   CAUSAL   j <= p
 *   WINDOW   p - j < arg                      (arg >= 1)
 *   KV_LT    j < arg                          (arg >= 0)
 *   CHUNK    floor(p / arg) == floor(j / arg) (arg >= 1, floor division)
 *   STRIDE   (p - j) mod arg == 0             (arg >= 1)
 *   DOC      doc_id[p] == doc_id[j]; positions outside doc_id are in no
 *            document (doc_id and doc_len as for DOC_CAUSAL, q_offset >= 0)
 *   HEAD_LT  h < arg                          (arg >= 0); a mask that uses it
 *            reads the head, so its BlockMask must have H = Hq */
typedef enum {
    FLEX_PRED_CAUSAL = 0,
    FLEX_PRED_WINDOW = 1,
    FLEX_PRED_KV_LT = 2,
    FLEX_PRED_CHUNK = 3,
    FLEX_PRED_STRIDE = 4,
    FLEX_PRED_DOC = 5,
    FLEX_PRED_HEAD_LT = 6
} flex_pred_kind;

#define FLEX_MAX_CLAUSES 4
#define FLEX_MAX_LITERALS 2

typedef struct {
    int32_t kind;   /* a flex_pred_kind */
    int32_t arg;
} flex_mask_pred;

/* A clause holds when any of its n (1..FLEX_MAX_LITERALS) predicates does. */
typedef struct {
    int32_t n;
    flex_mask_pred lit[FLEX_MAX_LITERALS];
} flex_mask_clause;

/* score_mod menu, applied to the already scaled score s of every computed cell
 * (full and partial tiles alike) before the mask.
 *   NONE            g = s
 *   SOFTCAP         g = cap * tanh(s / cap)   (tensorcad Examples, Gemma-2 cap)
 *   SOFTCAP_ALIBI   g = cap * tanh(s / cap) + alpha_h * (j - p),
 *                   alpha_h = 2^(-alibi_m * (h + 1) / Hq), h the query head
 *                   (charlestar blog, score_mod ordering section: cap first,
 *                   bias after; tensorcad Examples, ALiBi slope)
 *   ALIBI           g = s + alpha_h * (j - p), alpha_h as above, no cap
 *                   (tensorcad Examples, the ALiBi row) */
typedef enum {
    FLEX_SCORE_NONE = 0,
    FLEX_SCORE_SOFTCAP = 1,
    FLEX_SCORE_SOFTCAP_ALIBI = 2,
    FLEX_SCORE_ALIBI = 3
} flex_score_kind;

/* Mask parameters (host struct).
 *   kind      a flex_mask_kind
 *   window    CAUSAL_WINDOW_SINKS: window length, >= 1
 *   sinks     CAUSAL_WINDOW_SINKS: number of always-visible leading keys, >= 0
 *   q_offset  logical position of query row 0 (S - L aligns the causal
 *             diagonal bottom-right; 0 aligns it top-left)
 *   doc_id    DOC_CAUSAL and the DOC predicate: device int32[doc_len],
 *             document index per position
 *   doc_len   must then cover every key and query position, i.e.
 *             doc_len >= max(S, q_offset + L) with q_offset >= 0, and stay
 *             below 2^29
 *   n_clauses, clause   PROGRAM: 1 <= n_clauses <= FLEX_MAX_CLAUSES clauses,
 *             all of which must hold
 *   q_offsets optional device int32[B]: the logical position of query row 0
 *             per batch, in place of q_offset (values clamped to
 *             [-2^30, 2^30]); a position outside doc_id has no document
 *   kv_lens   optional device int32[B]: the valid keys per batch, positions
 *             [0, kv_lens[b]) of a cache of capacity S (values clamped to
 *             [0, S]); keys at or past it are hidden whatever the mask says
 *             (charlestar blog, decode section: capacity is not the filled
 *             length)
 *   Either array makes the mask differ between batches: its BlockMask must
 *   then have B equal to the batch count (build it with B rows). */
typedef struct {
    int32_t kind;
    int32_t window;
    int32_t sinks;
    int32_t reserved;
    int64_t q_offset;
    const int32_t* doc_id;
    int64_t doc_len;
    int32_t n_clauses;
    flex_mask_clause clause[FLEX_MAX_CLAUSES];
    const int32_t* q_offsets;
    const int32_t* kv_lens;
} flex_mask_params;

/* Score parameters (host struct).  cap > 0 for the SOFTCAP kinds; alibi_m
 * (the slope exponent, 8 in the pages' examples) for the ALiBi kinds. */
typedef struct {
    int32_t kind;
    float cap;
    float alibi_m;
} flex_score_params;

/* BlockMask (2kiu guide, sections 3.1-3.2 and 4.1).  Tiles are
 * q_block x kv_block cells; num_q_blocks = ceil(L / q_block),
 * num_kv_blocks = ceil(S / kv_block).  B and H are 1 (the mask is the same for
 * every batch / head and is broadcast) or the full batch / query-head count.
 * Device arrays, int32, C order:
 *   kv_num_blocks       [B][H][num_q_blocks]   number of partial tiles per row
 *   kv_indices          [B][H][num_q_blocks][num_kv_blocks]
 *                       the partial tiles' kv-block indices ascending, then the
 *                       remaining indices ascending
 *   full_kv_num_blocks  same shape as kv_num_blocks, full tiles
 *   full_kv_indices     same layout as kv_indices, full tiles
 * A tile is full when every one of its cells is visible, empty when none is
 * and partial otherwise; cells beyond L or S count as not visible. */
typedef struct {
    int32_t B, H;
    int32_t q_block, kv_block;
    int32_t num_q_blocks, num_kv_blocks;
    int32_t* kv_num_blocks;
    int32_t* kv_indices;
    int32_t* full_kv_num_blocks;
    int32_t* full_kv_indices;
} flex_block_mask;

/* Build a BlockMask from a mask_mod by evaluating it on every cell of every
 * tile (2kiu guide, section 4.1, create_block_mask with separate full blocks;
 * charlestar blog, BlockMask section, for the three tile classes).  No dense
 * element mask is ever formed.
 *   mask  mask parameters (q_offset, doc_id as for flex_attn_fwd)
 *   L, S  query and key lengths, 1 <= L, S < 2^30
 *   bm    dims filled in by the caller (B, H in {1, ...}, 1 <= q_block,
 *         kv_block <= 1024, num_q_blocks, num_kv_blocks as above) and the four
 *         caller-allocated device arrays, all written by this call
 * Errors: NULL, SHAPE, BLOCKMASK (dims), PARAM (mask parameters), HIP. */
flex_status flex_blockmask_build(const flex_mask_params* mask, int64_t L, int64_t S,
                                 const flex_block_mask* bm, void* stream);

/* Bytes of device workspace flex_attn_fwd needs for these sizes (0 when the
 * call needs none).  Returns 0 for arguments flex_attn_fwd would reject. */
size_t flex_attn_fwd_workspace_bytes(int32_t dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                     int64_t L, int64_t S, int32_t D,
                                     const flex_block_mask* bm);

/* Block-sparse attention forward.
 *   q, k, v      device tensors of `dtype` (FLEX_F32 or FLEX_BF16) with shapes
 *                q (B,Hq,L,D), k and v (B,Hkv,S,D); the last dimension is
 *                contiguous, the other three use the given element strides
 *                (q_strides = {batch, head, row}); base pointers and strides
 *                must be 16-byte aligned
 *   D            head dimension, 64 or 128
 *   Hq % Hkv     must be 0; query head h reads K/V head h / (Hq / Hkv)
 *   scale        multiplier of q.k; scale <= 0 selects 1/sqrt(D) (2kiu guide,
 *                section 6.2), computed in fp32
 *   score, mask  menu entries and their parameters
 *   bm           BlockMask built for the same mask parameters and (L, S);
 *                q_block in {16, 32, 64, 128}, kv_block a multiple of 64.
 *                It must be rebuilt whenever q_offset or doc_id changes
 *                (charlestar blog, decode and cache sections): the library
 *                trusts the lists and cannot detect a stale mask.
 *   out          device, (B,Hq,L,D) contiguous, dtype `dtype` (bf16 is
 *                rounded to nearest even)
 *   lse          device float32 (B,Hq,L) contiguous, or NULL when not wanted
 *   workspace    device scratch of at least flex_attn_fwd_workspace_bytes()
 *                (may be NULL when that is 0)
 * Rows with no visible key get out = 0 and lse = -inf.
 * Errors: NULL, SHAPE, GQA, BLOCKMASK, UNSUPPORTED, LAYOUT, WORKSPACE, PARAM,
 * HIP. */
flex_status flex_attn_fwd(const void* q, const void* k, const void* v, int32_t dtype,
                          int32_t B, int32_t Hq, int32_t Hkv, int64_t L, int64_t S, int32_t D,
                          const int64_t q_strides[3], const int64_t k_strides[3],
                          const int64_t v_strides[3], float scale,
                          const flex_score_params* score, const flex_mask_params* mask,
                          const flex_block_mask* bm, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/* flex_attn_fwd with the auxiliary outputs of the 2kiu guide, section 2:
 *   max_scores   device float32 (B,Hq,L) contiguous, or NULL: the largest
 *                visible score g(s) of each row (natural units, after
 *                score_mod and the mask), -inf for rows with no visible key
 * Every other argument is as for flex_attn_fwd, which is this call with
 * max_scores = NULL. */
flex_status flex_attn_fwd_aux(const void* q, const void* k, const void* v, int32_t dtype,
                              int32_t B, int32_t Hq, int32_t Hkv, int64_t L, int64_t S, int32_t D,
                              const int64_t q_strides[3], const int64_t k_strides[3],
                              const int64_t v_strides[3], float scale,
                              const flex_score_params* score, const flex_mask_params* mask,
                              const flex_block_mask* bm, void* out, float* lse, float* max_scores,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Q-side (transposed) BlockMask, used by the backward pass.  For every KV
 * block it lists the Q blocks whose tile with it is partial, then (separately)
 * full: the column view of the same tiles (2kiu guide, section 3.3:
 * from_kv_blocks derives Q-side block information by transposing the KV-side
 * lists).  Dims as in flex_block_mask.  Device arrays, int32, C order:
 *   q_num_blocks       [B][H][num_kv_blocks]   number of partial tiles per column
 *   q_indices          [B][H][num_kv_blocks][num_q_blocks]
 *                      the partial tiles' Q-block indices ascending, then the
 *                      remaining indices ascending
 *   full_q_num_blocks  same shape as q_num_blocks, full tiles
 *   full_q_indices     same layout as q_indices, full tiles */
typedef struct {
    int32_t B, H;
    int32_t q_block, kv_block;
    int32_t num_q_blocks, num_kv_blocks;
    int32_t* q_num_blocks;
    int32_t* q_indices;
    int32_t* full_q_num_blocks;
    int32_t* full_q_indices;
} flex_block_mask_q;

/* Fill the Q-side lists of a BlockMask (see flex_block_mask_q).
 *   bm    a BlockMask as flex_blockmask_build writes it: the first
 *         kv_num_blocks entries of each kv_indices row ascending (likewise the
 *         full lists); counts are clamped to [0, num_kv_blocks] and a KV block
 *         listed as both partial and full counts as partial
 *   bmq   dims equal to bm's and the four caller-allocated device arrays, all
 *         written by this call
 * Errors: NULL, BLOCKMASK (dims differ or out of range), HIP. */
flex_status flex_blockmask_transpose(const flex_block_mask* bm, const flex_block_mask_q* bmq, void* stream);

/* BlockMask utilities (2kiu guide, section 3.3).  Each reads a BlockMask as
 * flex_blockmask_build writes it (counts clamped to [0, num_kv_blocks]; a block
 * in both lists counts as partial, a block listed twice once) and writes
 * caller-allocated device memory; at most 65536 KV blocks per row.
 * Errors: NULL, BLOCKMASK (dims or ranges), UNSUPPORTED, HIP. */

/* to_dense: dense[b][h][qb][kb] = 1 where the lists name tile (qb, kb), as
 * partial or full, else 0 (int32, B*H*num_q_blocks*num_kv_blocks entries; the
 * row-wise rebuild of the guide's section 3.2). */
flex_status flex_blockmask_to_dense(const flex_block_mask* bm, int32_t* dense, void* stream);

/* The picture to_string draws: tile classes pooled into windows of
 * wr = ceil(num_q_blocks / grid_rows) by wc = ceil(num_kv_blocks / grid_cols)
 * tiles (the last ones cut); grid[b][h][i][j] = 2 when every tile of window
 * (i, j) is full, 0 when every tile is empty, 1 otherwise.  int8 device array
 * of B*H*ceil(num_q_blocks / wr)*ceil(num_kv_blocks / wc) entries; grid_rows,
 * grid_cols >= 1 (a grid no smaller than the tile grid gives the tile
 * classes themselves). */
flex_status flex_blockmask_grid(const flex_block_mask* bm, int32_t grid_rows, int32_t grid_cols, int8_t* grid,
                                void* stream);

/* sparsity: 100 * (1 - listed tiles / all tiles) over the whole
 * B x H x num_q_blocks x num_kv_blocks grid, written as one double to device
 * memory `percent` (8-byte aligned; also used as the counter while the call
 * runs). */
flex_status flex_blockmask_sparsity(const flex_block_mask* bm, double* percent, void* stream);

/* __getitem__: the rows of batches [r[0], r[1]), heads [r[2], r[3]) and Q-block
 * rows [r[4], r[5]) (ranges non-empty and inside the dims; the third range
 * indexes rows of the tile grid, not query tokens).  out: B = r[1]-r[0],
 * H = r[3]-r[2], num_q_blocks = r[5]-r[4], the same block sizes and
 * num_kv_blocks, and four caller-allocated arrays.  The slice serves queries
 * r[4]*q_block onwards, with the logical position q_offset + r[4]*q_block for
 * its first row. */
flex_status flex_blockmask_slice(const flex_block_mask* bm, const int32_t ranges[6], const flex_block_mask* out,
                                 void* stream);

/* _adjust: crop to the top-left lengths new_L x new_S, with
 * ceil(new_L / q_block) <= num_q_blocks and ceil(new_S / kv_block) <=
 * num_kv_blocks.  Each kept row keeps its listed blocks below the new column
 * count, in order; a full tile that now reaches past new_L or new_S becomes
 * partial (cells past the lengths are not visible).  The result equals a
 * rebuild when the cut falls on tile boundaries and the mask does not depend
 * on the lengths; otherwise it is conservative: every tile a rebuild would
 * visit is visited, and a tile is skipped its element mask only if a rebuild
 * would call it full.  out: dims for the new lengths and four arrays. */
flex_status flex_blockmask_adjust(const flex_block_mask* bm, int64_t new_L, int64_t new_S, const flex_block_mask* out,
                                  void* stream);

/* Bytes of device workspace flex_attn_bwd needs for these sizes: per (batch,
 * query head, row, rows padded to a multiple of 128) the base-2 lse and
 * D_i = dO_i . O_i as float32, plus, when one KV block's Q-side tiles may be
 * shared by several workgroups (long columns: keys that every query sees),
 * float32 partial sums of dk and dv for each share.  Returns 0 for arguments
 * flex_attn_bwd would reject. */
size_t flex_attn_bwd_workspace_bytes(int32_t dtype, int32_t B, int32_t Hq, int32_t Hkv, int64_t L, int64_t S,
                                     int32_t D, const flex_block_mask* bm);

/* Block-sparse attention backward: the gradients of sum(out * dout) with
 * respect to q, k and v for the forward of flex_attn_fwd (the charlestar blog
 * "FlexAttention score_mod / BlockMask" runs its example and then calls
 * backward on the summed output; the gradients are the chain rule through the
 * forward definition at the top of this file):
 *   P = exp(z - lse),  D_i = dout_i . out_i,
 *   dS = P (dout v^T - D) g'(s) scale,
 *   dq = dS k,  dk = dS^T q,  dv = P^T dout
 * where g' = 1 - tanh(s / cap)^2 for the soft-cap kinds and 1 otherwise; under
 * GQA dk and dv of a K/V head sum over its query heads.
 *   q, k, v, dtype, B, Hq, Hkv, L, S, D, strides, scale, score, mask
 *                as for the flex_attn_fwd call that produced out and lse
 *   out, dout    device (B,Hq,L,D) contiguous, dtype `dtype`: the forward
 *                output and the gradient flowing into it
 *   lse          device float32 (B,Hq,L) contiguous from that forward call
 *                (-inf rows, which saw no key, receive zero gradients)
 *   bm, bmq      the BlockMask of that call and its Q-side lists
 *                (flex_blockmask_transpose); q_block 64 or 128, kv_block a
 *                multiple of 64 (UNSUPPORTED otherwise); contiguous K/V
 *                (paged pools: flex_attn_bwd_paged)
 *   mask         may carry per-batch q_offsets / kv_lens as in the forward
 *                (the BlockMask then has B rows); keys at or past a batch's
 *                kv_lens are visible to no row and get zero dk, dv
 *   dq           device (B,Hq,L,D) contiguous, dtype `dtype`
 *   dk, dv       device (B,Hkv,S,D) contiguous, dtype `dtype`
 *   workspace    device scratch of at least flex_attn_bwd_workspace_bytes(),
 *                16-byte aligned
 * No output is accumulated with atomics: dq and, for most columns, dk and dv
 * are written once by one workgroup; a long column's dk, dv partial sums are
 * added in a fixed order.  Results do not depend on scheduling.  bf16 outputs are rounded to nearest even from
 * float32 accumulators.
 * Errors: NULL, SHAPE, GQA, BLOCKMASK, UNSUPPORTED, LAYOUT, WORKSPACE, PARAM,
 * HIP. */
flex_status flex_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                          const float* lse, int32_t dtype, int32_t B, int32_t Hq, int32_t Hkv, int64_t L,
                          int64_t S, int32_t D, const int64_t q_strides[3], const int64_t k_strides[3],
                          const int64_t v_strides[3], float scale, const flex_score_params* score,
                          const flex_mask_params* mask, const flex_block_mask* bm, const flex_block_mask_q* bmq,
                          void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream);

/* A paged K/V cache (charlestar blog, decode section: paged or circular
 * layouts store keys away from their logical positions, and those positions,
 * not the storage ones, are what masks and distance biases see).  K and V are
 * pools of num_pages pages of shape (Hkv, page_size, D); logical key j of
 * batch b lives in row j % page_size of page page_table[b][j / page_size].
 * A circular (rolling) buffer is the page table p -> p mod (pages in the
 * ring), with a mask that hides the positions the ring has overwritten.
 *   page_table  device int32 [B][max_pages]; entries outside [0, num_pages)
 *               are clamped (the row then reads another page, never past the
 *               pool)
 *   page_size   keys per page: a power of two, at least 64
 *   max_pages   entries per row, max_pages * page_size >= S
 *   num_pages   pages in each pool */
typedef struct {
    const int32_t* page_table;
    int32_t page_size;
    int32_t max_pages;
    int32_t num_pages;
    int32_t reserved;
} flex_kv_pages;

/* flex_attn_fwd_aux over a paged K/V cache.  k and v point at the pools;
 * k_strides and v_strides are {page, head, row} element strides of the pools;
 * S is the logical capacity of every batch's cache (with kv_lens giving the
 * filled length per batch).  Every other argument is as for flex_attn_fwd_aux.
 * Errors: as flex_attn_fwd_aux, plus NULL (pages, page_table), PARAM (page
 * geometry). */
flex_status flex_attn_fwd_paged(const void* q, const void* k, const void* v, int32_t dtype,
                                int32_t B, int32_t Hq, int32_t Hkv, int64_t L, int64_t S, int32_t D,
                                const int64_t q_strides[3], const int64_t k_strides[3],
                                const int64_t v_strides[3], float scale,
                                const flex_score_params* score, const flex_mask_params* mask,
                                const flex_block_mask* bm, const flex_kv_pages* pages, void* out, float* lse,
                                float* max_scores, void* workspace, size_t workspace_bytes, void* stream);

/* flex_attn_bwd over a paged K/V cache: the gradients for a forward run by
 * flex_attn_fwd_paged (same pools, pages, strides, S and mask).  The
 * key-major pass reads each 64-key tile's K and V rows from the page holding
 * them, the query-major pass stages its tiles from there, as the forward does.
 * dk and dv are the gradients of the LOGICAL keys and values: device
 * (B, Hkv, S, D) contiguous, row j of batch b for logical key j (a caller
 * that trains through a pool scatters them back through its page table, where
 * pages shared between batches add up).  Every other argument is as for
 * flex_attn_bwd.
 * Errors: as flex_attn_bwd, plus NULL (pages, page_table), PARAM (page
 * geometry). */
flex_status flex_attn_bwd_paged(const void* q, const void* k, const void* v, const flex_kv_pages* pages,
                                const void* out, const void* dout, const float* lse, int32_t dtype, int32_t B,
                                int32_t Hq, int32_t Hkv, int64_t L, int64_t S, int32_t D,
                                const int64_t q_strides[3], const int64_t k_strides[3],
                                const int64_t v_strides[3], float scale, const flex_score_params* score,
                                const flex_mask_params* mask, const flex_block_mask* bm,
                                const flex_block_mask_q* bmq, void* dq, void* dk, void* dv, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Size of the device scratch array behind flex_attn_fwd_noalloc (per GPU). */
#define FLEX_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* flex_attn_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace: the split-KV decode partials that flex_attn_fwd keeps
 * in the caller's workspace go to a file-scope device array of
 * FLEX_NOALLOC_SCRATCH_BYTES inside the library instead (one per GPU, held
 * until the process ends; set up on the first call on each device).  The call
 * allocates nothing and frees nothing.  Every argument is as for
 * flex_attn_fwd; inputs and outputs are still the caller's.
 * All calls on one GPU share its array: calls that overlap in time on that
 * GPU (different streams, or threads without ordering) race and must not be
 * issued.  Calls queued in order on one stream are safe.
 * Errors: as flex_attn_fwd; WORKSPACE when the call would need more than
 * FLEX_NOALLOC_SCRATCH_BYTES of scratch (flex_attn_fwd_workspace_bytes
 * gives the need); HIP when the array's device address cannot be found. */
flex_status flex_attn_fwd_noalloc(const void* q, const void* k, const void* v, int32_t dtype,
                                  int32_t B, int32_t Hq, int32_t Hkv, int64_t L, int64_t S, int32_t D,
                                  const int64_t q_strides[3], const int64_t k_strides[3],
                                  const int64_t v_strides[3], float scale,
                                  const flex_score_params* score, const flex_mask_params* mask,
                                  const flex_block_mask* bm, void* out, float* lse, void* stream);

/* Static name of a status code. */
const char* flex_status_string(int32_t status);

/* Reason for the failure of the calling thread's last library call ("" if it
 * succeeded).  The pointer stays valid until the thread's next library call. */
const char* flex_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FLEXMI_H */
