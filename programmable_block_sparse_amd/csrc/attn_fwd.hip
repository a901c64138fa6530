// Host side of the forward pass: score-rule constants, the prefill row layout
// and split-KV heuristics, the workspace size, and the launch entry that
// picks the translation unit compiled for the dtype and head dimension.
#include "attn_fwd_impl.hpp"

namespace flexmi {

ScoreConsts score_consts(float scale_f, float cap_f, int score_kind) {
    ScoreConsts c{};
    const double scale = scale_f, cap = cap_f, l2e = 1.4426950408889634;
    const bool capped = score_kind == SCORE_SOFTCAP || score_kind == SCORE_SOFTCAP_ALIBI;
    c.mul = capped ? (float)(2.0 * scale * l2e / cap) : (float)(scale * l2e);
    c.c2 = (float)(cap * l2e);
    const double r = scale / cap;
    c.k0 = (float)(scale * l2e * kTanh0);
    c.k1 = (float)(scale * l2e * kTanh1 * r * r);
    c.k2 = (float)(scale * l2e * kTanh2 * r * r * r * r);
    c.amax = (float)(kTanhRange / r);
    c.j0 = (float)(scale * l2e * kLin0);
    c.j1 = (float)(scale * l2e * kLin1 * r * r);
    c.amax1 = cap * kLinErr <= kPolyScoreErr ? (float)(kLinRange / r) : 0.0f;
    return c;
}

// Row layout of the prefill kernel: 64-row workgroups with key halves split
// across waves when the 128-row work items are too few to fill the chip, else
// 128-row workgroups (each K/V tile staged in LDS then serves twice the rows,
// and a wave's two key halves overlap one's QK^T with the other's softmax).
// Head dim 128: 128-row items from three per slot at two workgroups per CU;
// bf16 head dim 64: from one per slot at three per CU; fp32 head dim 64
// always splits.
int prefill_ksplit(int dtype, int B, int Hq, int nQB, int q_block, int D) {
    if (q_block <= 64) return 1;
    const int64_t items = (int64_t)B * Hq * nQB;
    if (D == 64) return (dtype != 1 || items < 256 * 3) ? 1 : 0;
    return items < 2 * 256 * 3 ? 1 : 0;
}

int decode_splits(int dtype, int B, int Hq, int Hkv, int L, int D, int q_block, int kv_block, int nKB, int Hm) {
    if (dtype != 1 || Hm != 1 || Hq % Hkv != 0) return 0;
    const int group = Hq / Hkv;
    if ((int64_t)group * q_block > 64 || q_block > 32) return 0;
    const int64_t n_qb = ((int64_t)L + q_block - 1) / q_block;
    const int64_t units = (int64_t)B * Hkv * n_qb;
    const int64_t tiles = (int64_t)nKB * (kv_block / kTileN);
    if (units >= 1024 || tiles < 32) return 0;
    // one workgroup per resident slot of the chip (256 CUs)
    const int64_t slots = 256 * (D == 64 ? DecodeShape<64>::kWgsPerCu : DecodeShape<128>::kWgsPerCu);
    int64_t splits = slots / units;
    splits = std::min<int64_t>(splits, tiles / 16);
    splits = std::max<int64_t>(std::min<int64_t>(splits, 256), 1);
    return (int)splits;
}

size_t attn_fwd_workspace_bytes(int dtype, int B, int Hq, int Hkv, int L, int S, int D, int q_block, int kv_block,
                                int nKB, int Bm, int Hm) {
    (void)S;
    (void)Bm;
    const int splits = decode_splits(dtype, B, Hq, Hkv, L, D, q_block, kv_block, nKB, Hm);
    if (splits == 0) return 0;
    const size_t rows = (size_t)splits * B * Hq * L;
    return rows * D * sizeof(float) + rows * 4 * sizeof(float);
}

hipError_t launch_attn_fwd(int dtype, int D, const FwdArgs& a, hipStream_t stream) {
    if (dtype == 1 && D == 64) return launch_attn_fwd_bf16_d64(a, stream);
    if (dtype == 1 && D == 128) return launch_attn_fwd_bf16_d128(a, stream);
    if (a.splits > 0) return hipErrorInvalidValue;    // split-KV decode is bf16 only
    if (dtype == 0 && D == 64) return launch_attn_fwd_f32_d64(a, stream);
    if (dtype == 0 && D == 128) return launch_attn_fwd_f32_d128(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace flexmi
