// Host side of the forward pass: score-rule constants, the prefill row layout
// and split-KV heuristics, the workspace size, and the launch entry that
// picks the translation unit compiled for the dtype and head dimension.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "attn_fwd_impl.hpp"

namespace flexmi {

namespace {

// Odd polynomial y * (a[0] + a[1] y^2 + ... + a[n-1] y^(2n-2)) approximating
// tanh(y) on [0, Y] with the least maximum absolute error, by Remez exchange
// on n + 1 alternation points (the last one at Y); err is that maximum.
struct TanhFit {
    double a[3];
    double err;
};

double odd_poly(const double* a, int n, double y) {
    const double w = y * y;
    double p = a[n - 1];
    for (int j = n - 2; j >= 0; --j) p = p * w + a[j];
    return y * p;
}

// Solves the (n+1) x (n+1) system M x = rhs in place (partial pivoting).
void solve_small(double (*M)[5], double* x, int m) {
    for (int c = 0; c < m; ++c) {
        int piv = c;
        for (int r = c + 1; r < m; ++r)
            if (std::fabs(M[r][c]) > std::fabs(M[piv][c])) piv = r;
        for (int k = 0; k <= m; ++k) std::swap(M[c][k], M[piv][k]);
        for (int r = 0; r < m; ++r) {
            if (r == c) continue;
            const double f = M[r][c] / M[c][c];
            for (int k = c; k <= m; ++k) M[r][k] -= f * M[c][k];
        }
    }
    for (int r = 0; r < m; ++r) x[r] = M[r][m] / M[r][r];
}

TanhFit fit_tanh(int n, double Y) {
    const double pi = 3.14159265358979323846;
    double y[4];
    for (int i = 0; i <= n; ++i) y[i] = Y * std::sin(0.5 * pi * (i + 1) / (n + 1));
    TanhFit f{};
    for (int it = 0; it < 16; ++it) {
        // a . (y_i, y_i^3, ...) + (-1)^i E = tanh(y_i)
        double M[4][5], x[4];
        for (int i = 0; i <= n; ++i) {
            double yp = y[i];
            for (int j = 0; j < n; ++j, yp *= y[i] * y[i]) M[i][j] = yp;
            M[i][n] = (i % 2) ? -1.0 : 1.0;
            M[i][n + 1] = std::tanh(y[i]);
        }
        solve_small(M, x, n + 1);
        for (int j = 0; j < n; ++j) f.a[j] = x[j];
        // move each interior point to the nearby extremum of the error
        // e = tanh - p (Newton on e' = 0); the last point stays at Y
        for (int i = 0; i < n; ++i) {
            double t = y[i];
            for (int k = 0; k < 20; ++k) {
                const double th = std::tanh(t), s2 = 1.0 - th * th, w = t * t;
                double d1 = s2, d2 = -2.0 * th * s2, wp = 1.0;
                for (int j = 0; j < n; ++j, wp *= w) {
                    d1 -= (2 * j + 1) * f.a[j] * wp;
                    if (j > 0) d2 -= (2 * j + 1) * (2 * j) * f.a[j] * wp / t;
                }
                if (d2 == 0.0) break;
                const double nt = std::min(std::max(t - d1 / d2, 0.5 * t), 0.5 * (t + Y));
                if (std::fabs(nt - t) < 1e-15 * Y) break;
                t = nt;
            }
            y[i] = t;
        }
        std::sort(y, y + n);
    }
    f.err = 0.0;
    for (int k = 1; k <= 512; ++k) {
        const double t = Y * k / 512.0;
        f.err = std::max(f.err, std::fabs(std::tanh(t) - odd_poly(f.a, n, t)));
    }
    return f;
}

// The widest range Y <= kTanhRange on which the n-term fit keeps
// cap * error <= kPolyScoreErr, with its coefficients.
double fit_for_cap(int n, double cap, TanhFit* out) {
    double Y = kTanhRange;
    for (int k = 0; k < 200; ++k, Y *= 0.97) {
        *out = fit_tanh(n, Y);
        if (out->err * cap <= kPolyScoreErr) return Y;
    }
    return Y;
}

struct CapFits {
    float cap;
    double Yc, Yq;
    TanhFit cubic, quintic;
};

// The fits depend on the cap alone; a small cache keeps repeated calls cheap.
CapFits cap_fits(float cap) {
    static std::mutex mu;
    static CapFits cache[16];
    static int used = 0, next = 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < used; ++i)
            if (cache[i].cap == cap) return cache[i];
    }
    CapFits c{};
    c.cap = cap;
    c.Yq = fit_for_cap(3, cap, &c.quintic);
    c.Yc = std::min(fit_for_cap(2, cap, &c.cubic), c.Yq);
    std::lock_guard<std::mutex> lock(mu);
    cache[next] = c;
    next = (next + 1) % 16;
    used = std::min(used + 1, 16);
    return c;
}

}  // namespace

ScoreConsts score_consts(float scale_f, float cap_f, int score_kind) {
    ScoreConsts c{};
    const double scale = scale_f, cap = cap_f, l2e = 1.4426950408889634;
    const bool capped = score_kind == SCORE_SOFTCAP || score_kind == SCORE_SOFTCAP_ALIBI;
    c.mul = capped ? (float)(2.0 * scale * l2e / cap) : (float)(scale * l2e);
    c.c2 = (float)(cap * l2e);
    if (!capped) return c;
    // g2 = cap*log2e*tanh(y) with y = acc*r: the fit in y becomes a polynomial
    // in the raw score acc with coefficients scale*log2e*a_j*r^(2j)
    const double r = scale / cap;
    const CapFits f = cap_fits(cap_f);
    c.k0 = (float)(scale * l2e * f.quintic.a[0]);
    c.k1 = (float)(scale * l2e * f.quintic.a[1] * r * r);
    c.k2 = (float)(scale * l2e * f.quintic.a[2] * r * r * r * r);
    c.amax = (float)(f.Yq / r);
    c.j0 = (float)(scale * l2e * f.cubic.a[0]);
    c.j1 = (float)(scale * l2e * f.cubic.a[1] * r * r);
    c.amax1 = (float)(f.Yc / r);
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
