// GPT-2 training-step oracle: a plain, slow, obviously-correct CPU model.
//
// TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls
// this file; only the tests, the smoke check and the benchmark's cpu_baseline
// leg do. It shares no source with the HIP library: its own parameter layout,
// its own math, its own loops.
//
// What it computes follows the pages as follows (page titles abbreviated):
//   [minigpt]  "从零实现一个最小GPT：代码讲解 + 知识点全解" (myblog.yourun.site),
//              section 二 (the full minigpt.py) and the walkthrough of section 三.
//   [karpathy] "两小时手搓GPT-2" (aipmzone.com), sections on the state dict and
//              on Attention/MLP/GELU.
//   [nanogpt]  "4.1 GPT-2 124M 复现" (aiknowledge.cn), section 2.3 (train_gpt2.py).
//   [llmc]     "手写训练脚本" (yunpans.com), section 二 (flat buffer, LayerNorm
//              forward and backward by hand).
// Readings where the pages are silent or disagree (tanh GELU, tied head,
// LayerNorm eps 1e-5, AdamW constants, the LR schedule, clipping) are listed
// with the reason in the design notes of the repository.
//
// Every function is templated on the scalar type R. The float instantiation is
// the fp32 oracle; the double instantiation is used for parity references and
// finite-difference self-checks. Matrix loops keep the summation index in
// plain sequential order; OpenMP only splits independent outputs.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <cstddef>
#include <vector>
#include <algorithm>
#include <omp.h>

extern "C" {
typedef struct {
    int32_t vocab;       // V
    int32_t block_size;  // maximum T (rows of the position table)
    int32_t n_embd;      // C
    int32_t n_head;      // H, head size d = C / H
    int32_t n_layer;     // L
    int32_t mlp_hidden;  // F (4C in every config on the pages)
    int32_t bias;        // 1: Linear layers carry biases
    int32_t variant;     // bit 0: exact erf GELU; bit 1: untied lm_head (ORACLE_* below)
    double ln_eps;       // LayerNorm epsilon
    double dropout;      // training-mode dropout probability p (0: none)
    uint64_t seed;       // dropout stream key (see keep() below)
} oracle_cfg;
}

// The minigpt page's literal model differs from the GPT-2 readings in three ways
// the oracle can follow on request: nn.GELU() with its default exact erf form,
// an lm_head Linear of its own instead of the tied embedding, and dropout
// (cfg.dropout, three sites per block, see model_step).
enum { ORACLE_GELU_ERF = 1, ORACLE_UNTIED = 2 };

// Dropout sites of a block in minigpt.py: the attention weights after the
// softmax (Head.forward), the attention projection's output
// (MultiHeadAttention.forward) and the FeedForward's last Linear (its
// nn.Dropout). Embeddings have none.
enum { DROP_ATTN = 0, DROP_PROJ = 1, DROP_FC2 = 2 };

namespace {

// ---------------------------------------------------------------- dropout stream
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC 2011): a 128-bit counter and a 64-bit key; each of ten rounds
// multiplies words 0 and 2 by fixed 32-bit constants into 64-bit products and
// rebuilds the four words from the product halves, the two other words and the
// key, which is advanced by two Weyl constants between rounds.
static void philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * x0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0;
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1;
        const uint32_t n3 = (uint32_t)p0;
        x0 = n0; x1 = n1; x2 = n2; x3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

// The keep decision for element e of a dropout site (nn.Dropout keeps each
// element independently with probability 1 - p). The pages fix no generator;
// the reading adopted: element e of site `site` in layer `layer` takes 16-bit
// half (e mod 8) of Philox4x32-10 at counter (e / 8 low and high words, site,
// layer) under key (seed low, seed high) -- halves numbered low then high
// within words 0..3 -- and is kept when that half is at least
// round(p * 65536). Element order: attention ((b H + h) T + i) T + j for query
// i and key j of head h in sequence b; the residual sites m C + c.
static uint32_t drop_threshold(double p) {
    double t = std::floor(p * 65536.0 + 0.5);
    return (uint32_t)std::min(t, 65536.0);
}
static bool keep(uint64_t seed, int site, int layer, uint64_t e, uint32_t thr) {
    const uint64_t n = e >> 3;
    const uint32_t ctr[4] = {(uint32_t)n, (uint32_t)(n >> 32), (uint32_t)site, (uint32_t)layer};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t r[4];
    philox4x32_10(ctr, key, r);
    const int h = (int)(e & 7);
    const uint32_t half = (h & 1) ? (r[h >> 1] >> 16) : (r[h >> 1] & 0xFFFFu);
    return half >= thr;
}

// Tensor kinds of the oracle's own canonical layout.
enum Kind {
    K_WTE = 0, K_WPE, K_LN1_G, K_LN1_B, K_W_QKV, K_B_QKV, K_W_PROJ, K_B_PROJ,
    K_LN2_G, K_LN2_B, K_W_FC, K_B_FC, K_W_FC2, K_B_FC2, K_LNF_G, K_LNF_B, K_LM_HEAD
};

struct LayerOff {
    size_t ln1_g, ln1_b, w_qkv, b_qkv, w_proj, b_proj, ln2_g, ln2_b, w_fc, b_fc, w_fc2, b_fc2;
};
struct Layout {
    size_t wte, wpe, lnf_g, lnf_b, lm_head, total;
    std::vector<LayerOff> layer;
};
static const size_t NONE = (size_t)-1;

// Compact layout, tensors back to back in the order the minigpt module
// registers them (token embedding, position embedding, blocks, ln_f), with the
// three per-head Q/K/V Linears of a block fused into one [3C, C] matrix whose
// rows are [Q heads 0..H-1 | K heads | V heads] (the fused QKV concatenation
// the karpathy page asks about). The head is tied to wte and has no tensor of
// its own, unless the untied variant asks for minigpt's separate lm_head [V, C]
// (registered last, after ln_f, as in minigpt.py).
static Layout make_layout(const oracle_cfg& c) {
    Layout lo;
    size_t o = 0;
    const size_t V = c.vocab, T = c.block_size, C = c.n_embd, F = c.mlp_hidden;
    auto take = [&](size_t n) { size_t r = o; o += n; return r; };
    lo.wte = take(V * C);
    lo.wpe = take(T * C);
    for (int l = 0; l < c.n_layer; ++l) {
        LayerOff L;
        L.ln1_g = take(C); L.ln1_b = take(C);
        L.w_qkv = take(3 * C * C); L.b_qkv = c.bias ? take(3 * C) : NONE;
        L.w_proj = take(C * C);    L.b_proj = c.bias ? take(C) : NONE;
        L.ln2_g = take(C); L.ln2_b = take(C);
        L.w_fc = take(F * C);      L.b_fc = c.bias ? take(F) : NONE;
        L.w_fc2 = take(C * F);     L.b_fc2 = c.bias ? take(C) : NONE;
        lo.layer.push_back(L);
    }
    lo.lnf_g = take(C); lo.lnf_b = take(C);
    lo.lm_head = (c.variant & ORACLE_UNTIED) ? take(V * C) : lo.wte;
    lo.total = o;
    return lo;
}

static bool cfg_ok(const oracle_cfg& c) {
    if (!(c.dropout >= 0.0 && c.dropout < 1.0)) return false;
    return c.vocab > 0 && c.block_size > 0 && c.n_embd > 0 && c.n_head > 0 &&
           c.n_layer >= 0 && c.mlp_hidden > 0 && c.n_embd % c.n_head == 0 &&
           (c.variant & ~(ORACLE_GELU_ERF | ORACLE_UNTIED)) == 0;
}

// ---------------------------------------------------------------- LayerNorm
// y = (x - mean) / sqrt(var + eps) * g + b over the last axis, biased variance
// (nn.LayerNorm as used by Block and ln_f in minigpt.py; the backward formula
// is the hand derivation the llm.c page describes).
template <class R>
void layernorm_fwd(int64_t rows, int C, const R* x, const R* g, const R* b, double eps,
                   R* y, R* mean, R* rstd) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const R* xr = x + r * C;
        R s = 0;
        for (int c = 0; c < C; ++c) s += xr[c];
        R mu = s / (R)C;
        R v = 0;
        for (int c = 0; c < C; ++c) { R d = xr[c] - mu; v += d * d; }
        v /= (R)C;
        R rs = (R)1 / std::sqrt(v + (R)eps);
        for (int c = 0; c < C; ++c) y[r * C + c] = (xr[c] - mu) * rs * g[c] + b[c];
        if (mean) mean[r] = mu;
        if (rstd) rstd[r] = rs;
    }
}

// dx += rstd * (g*dy - mean(g*dy) - xhat * mean(g*dy*xhat)); dg += sum dy*xhat; db += sum dy
template <class R>
void layernorm_bwd(int64_t rows, int C, const R* dy, const R* x, const R* mean, const R* rstd,
                   const R* g, R* dx, R* dg, R* db) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const R* xr = x + r * C;
        const R* dyr = dy + r * C;
        R mu = mean[r], rs = rstd[r];
        R a = 0, bb = 0;
        for (int c = 0; c < C; ++c) {
            R xh = (xr[c] - mu) * rs;
            R gd = g[c] * dyr[c];
            a += gd;
            bb += gd * xh;
        }
        a /= (R)C; bb /= (R)C;
        for (int c = 0; c < C; ++c) {
            R xh = (xr[c] - mu) * rs;
            dx[r * C + c] += rs * (g[c] * dyr[c] - a - xh * bb);
        }
    }
    // parameter gradients: rows summed in order, columns split across threads
#pragma omp parallel for schedule(static)
    for (int c = 0; c < C; ++c) {
        R sg = 0, sb = 0;
        for (int64_t r = 0; r < rows; ++r) {
            R xh = (x[r * C + c] - mean[r]) * rstd[r];
            sg += dy[r * C + c] * xh;
            sb += dy[r * C + c];
        }
        dg[c] += sg;
        db[c] += sb;
    }
}

// ---------------------------------------------------------------- Linear
// Y[M,N] = X[M,K] . W[N,K]^T (+ b), the nn.Linear convention of minigpt.py.
template <class R>
void linear_fwd(int64_t M, int N, int K, const R* X, const R* W, const R* b, R* Y) {
    std::vector<R> Wt((size_t)K * N);
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k) Wt[(size_t)k * N + n] = W[(size_t)n * K + k];
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        R* y = Y + m * N;
        for (int n = 0; n < N; ++n) y[n] = b ? b[n] : (R)0;
        const R* x = X + m * K;
        for (int k = 0; k < K; ++k) {
            const R xk = x[k];
            const R* wt = Wt.data() + (size_t)k * N;
            for (int n = 0; n < N; ++n) y[n] += xk * wt[n];
        }
    }
}

// dX = dY . W (overwrites), dW += dY^T . X, db += column sums of dY.
template <class R>
void linear_bwd(int64_t M, int N, int K, const R* dY, const R* X, const R* W,
                R* dX, R* dW, R* db) {
    if (dX) {
#pragma omp parallel for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            R* dx = dX + m * K;
            for (int k = 0; k < K; ++k) dx[k] = 0;
            const R* dy = dY + m * N;
            for (int n = 0; n < N; ++n) {
                const R d = dy[n];
                const R* w = W + (size_t)n * K;
                for (int k = 0; k < K; ++k) dx[k] += d * w[k];
            }
        }
    }
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        R* dw = dW + (size_t)n * K;
        R sb = 0;
        for (int64_t m = 0; m < M; ++m) {
            const R d = dY[m * N + n];
            sb += d;
            const R* x = X + m * K;
            for (int k = 0; k < K; ++k) dw[k] += d * x[k];
        }
        if (db) db[n] += sb;
    }
}

// ---------------------------------------------------------------- GELU
// The tanh approximation of GELU that the karpathy page says GPT-2 uses
// (Hendrycks & Gimpel): 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))).
// With erf_form, the exact definition nn.GELU() computes by default in
// minigpt.py: u Phi(u) = 0.5 u (1 + erf(u / sqrt 2)), whose derivative is
// Phi(u) + u phi(u) with phi the standard normal density.
template <class R>
R gelu(R u, bool erf_form = false) {
    if (erf_form) return (R)0.5 * u * ((R)1 + std::erf(u * (R)0.7071067811865476));
    const R k0 = (R)0.7978845608028654;  // sqrt(2/pi)
    const R k1 = (R)0.044715;
    return (R)0.5 * u * ((R)1 + std::tanh(k0 * (u + k1 * u * u * u)));
}
template <class R>
R gelu_grad(R u, bool erf_form = false) {
    if (erf_form) {
        const R Phi = (R)0.5 * ((R)1 + std::erf(u * (R)0.7071067811865476));
        const R phi = (R)0.3989422804014327 * std::exp((R)-0.5 * u * u);  // 1/sqrt(2 pi)
        return Phi + u * phi;
    }
    const R k0 = (R)0.7978845608028654;
    const R k1 = (R)0.044715;
    R w = k0 * (u + k1 * u * u * u);
    R t = std::tanh(w);
    return (R)0.5 * ((R)1 + t) + (R)0.5 * u * ((R)1 - t * t) * k0 * ((R)1 + (R)3 * k1 * u * u);
}

// ---------------------------------------------------------------- attention
// One causal head, the Head.forward of minigpt.py written out: scores
// q_i.k_j / sqrt(d), -inf for j > i, softmax over j, out_i = sum_j P_ij v_j.
// Rows of q, k, v, out are `stride` apart. P (T x T, may be null) receives the
// probabilities with exact zeros above the diagonal. With `kp` (T x T keep
// flags, may be null) the attention weights pass through dropout before they
// weight the values: P_ij kp_ij / (1 - p), with dscale = 1 / (1 - p).
template <class R>
void head_fwd(int T, int d, const R* q, const R* k, const R* v, int64_t stride, R* out,
              int64_t ostride, R* P, R* srow, const uint8_t* kp = nullptr, R dscale = 1) {
    const R scale = (R)1 / std::sqrt((R)d);
    for (int i = 0; i < T; ++i) {
        R mx = -INFINITY;
        for (int j = 0; j <= i; ++j) {
            R s = 0;
            for (int c = 0; c < d; ++c) s += q[(int64_t)i * stride + c] * k[(int64_t)j * stride + c];
            s *= scale;
            srow[j] = s;
            mx = std::max(mx, s);
        }
        R sum = 0;
        for (int j = 0; j <= i; ++j) { srow[j] = std::exp(srow[j] - mx); sum += srow[j]; }
        for (int j = 0; j <= i; ++j) srow[j] /= sum;
        R* o = out + (int64_t)i * ostride;
        for (int c = 0; c < d; ++c) o[c] = 0;
        for (int j = 0; j <= i; ++j) {
            const R w = kp ? (kp[(int64_t)i * T + j] ? srow[j] * dscale : (R)0) : srow[j];
            for (int c = 0; c < d; ++c) o[c] += w * v[(int64_t)j * stride + c];
        }
        if (P) {
            for (int j = 0; j < T; ++j) P[(int64_t)i * T + j] = j <= i ? srow[j] : (R)0;
        }
    }
}

// Backward of head_fwd with P recomputed from q and k:
//   dV_j = sum_i P_ij dO_i, dP_ij = dO_i . v_j, dS_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij'),
//   dQ_i = sum_j dS_ij k_j / sqrt(d), dK_j = sum_i dS_ij q_i / sqrt(d).
// With dropout (kp, dscale as in head_fwd) the values are weighted by the
// dropped weights W_ij = P_ij kp_ij dscale: dV_j = sum_i W_ij dO_i, and the
// softmax sees dP_ij = kp_ij dscale (dO_i . v_j).
// dq, dk, dv are overwritten.
template <class R>
void head_bwd(int T, int d, const R* q, const R* k, const R* v, int64_t stride, const R* dout,
              int64_t ostride, R* dq, R* dk, R* dv, R* prow, R* dprow, const uint8_t* kp = nullptr,
              R dscale = 1) {
    const R scale = (R)1 / std::sqrt((R)d);
    for (int i = 0; i < T; ++i)
        for (int c = 0; c < d; ++c) {
            dq[(int64_t)i * stride + c] = 0; dk[(int64_t)i * stride + c] = 0; dv[(int64_t)i * stride + c] = 0;
        }
    for (int i = 0; i < T; ++i) {
        // recompute row i of P
        R mx = -INFINITY;
        for (int j = 0; j <= i; ++j) {
            R s = 0;
            for (int c = 0; c < d; ++c) s += q[(int64_t)i * stride + c] * k[(int64_t)j * stride + c];
            s *= scale;
            prow[j] = s;
            mx = std::max(mx, s);
        }
        R sum = 0;
        for (int j = 0; j <= i; ++j) { prow[j] = std::exp(prow[j] - mx); sum += prow[j]; }
        for (int j = 0; j <= i; ++j) prow[j] /= sum;
        const R* doi = dout + (int64_t)i * ostride;
        R rowdot = 0;
        for (int j = 0; j <= i; ++j) {
            R s = 0;
            for (int c = 0; c < d; ++c) s += doi[c] * v[(int64_t)j * stride + c];
            if (kp) s = kp[(int64_t)i * T + j] ? s * dscale : (R)0;
            dprow[j] = s;
            rowdot += prow[j] * s;
        }
        for (int j = 0; j <= i; ++j) {
            R ds = prow[j] * (dprow[j] - rowdot);
            const R w = kp ? (kp[(int64_t)i * T + j] ? prow[j] * dscale : (R)0) : prow[j];
            for (int c = 0; c < d; ++c) {
                dq[(int64_t)i * stride + c] += ds * k[(int64_t)j * stride + c] * scale;
                dk[(int64_t)j * stride + c] += ds * q[(int64_t)i * stride + c] * scale;
                dv[(int64_t)j * stride + c] += w * doi[c];
            }
        }
    }
}

// Multi-head causal attention over a fused qkv [B*T, 3C] activation. Head h uses
// columns [h*d, (h+1)*d) of each third; outputs are concatenated head 0 first
// (torch.cat over heads in MultiHeadAttention.forward).
// Dropout of one model step: the probability and key, and the layer whose
// masks are wanted (p = 0: no dropout).
struct Drop {
    double p = 0.0;
    uint64_t seed = 0;
    int layer = 0;
    bool on() const { return p > 0.0; }
};
// keep flags of head (b, h): kp[i T + j] for the attention site
static void head_keep(const Drop& dr, int b, int h, int H, int T, uint8_t* kp) {
    const uint32_t thr = drop_threshold(dr.p);
    for (int i = 0; i < T; ++i)
        for (int j = 0; j < T; ++j)
            kp[(int64_t)i * T + j] = keep(dr.seed, DROP_ATTN, dr.layer,
                                          (((uint64_t)b * H + h) * T + i) * T + j, thr);
}

template <class R>
void attention_fwd(int B, int T, int C, int H, const R* qkv, R* out, const Drop& dr = Drop()) {
    const int d = C / H;
    const R dscale = dr.on() ? (R)(1.0 / (1.0 - dr.p)) : (R)1;
#pragma omp parallel
    {
        std::vector<R> srow(T);
        std::vector<uint8_t> kp(dr.on() ? (size_t)T * T : 0);
#pragma omp for schedule(dynamic)
        for (int bh = 0; bh < B * H; ++bh) {
            int b = bh / H, h = bh % H;
            if (dr.on()) head_keep(dr, b, h, H, T, kp.data());
            const R* base = qkv + (int64_t)b * T * 3 * C;
            head_fwd<R>(T, d, base + h * d, base + C + h * d, base + 2 * C + h * d, 3 * C,
                        out + (int64_t)b * T * C + h * d, C, nullptr, srow.data(),
                        dr.on() ? kp.data() : nullptr, dscale);
        }
    }
}
template <class R>
void attention_bwd(int B, int T, int C, int H, const R* qkv, const R* dout, R* dqkv, const Drop& dr = Drop()) {
    const int d = C / H;
    const R dscale = dr.on() ? (R)(1.0 / (1.0 - dr.p)) : (R)1;
#pragma omp parallel
    {
        std::vector<R> prow(T), dprow(T);
        std::vector<uint8_t> kp(dr.on() ? (size_t)T * T : 0);
#pragma omp for schedule(dynamic)
        for (int bh = 0; bh < B * H; ++bh) {
            int b = bh / H, h = bh % H;
            if (dr.on()) head_keep(dr, b, h, H, T, kp.data());
            const R* base = qkv + (int64_t)b * T * 3 * C;
            R* dbase = dqkv + (int64_t)b * T * 3 * C;
            head_bwd<R>(T, d, base + h * d, base + C + h * d, base + 2 * C + h * d, 3 * C,
                        dout + (int64_t)b * T * C + h * d, C,
                        dbase + h * d, dbase + C + h * d, dbase + 2 * C + h * d,
                        prow.data(), dprow.data(), dr.on() ? kp.data() : nullptr, dscale);
        }
    }
}

// Residual-branch dropout in place: y[m C + c] = keep ? y / (1 - p) : 0
// (also the backward: the same mask and scale on the incoming gradient).
template <class R>
void residual_dropout(const Drop& dr, int site, int64_t M, int C, R* y) {
    if (!dr.on()) return;
    const uint32_t thr = drop_threshold(dr.p);
    const R dscale = (R)(1.0 / (1.0 - dr.p));
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M * C; ++i) y[i] = keep(dr.seed, site, dr.layer, (uint64_t)i, thr) ? y[i] * dscale : (R)0;
}

// ---------------------------------------------------------------- cross-entropy
// F.cross_entropy with mean reduction, written per row: loss_r = lse(z_r) - z_r[y_r],
// lse = max + log sum exp(z - max). dlogits (optional) = (softmax - onehot) * scale.
template <class R>
void cross_entropy(int64_t rows, int V, const R* z, const int32_t* y, R* loss_rows, R* dz, R scale) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const R* zr = z + r * V;
        R mx = -INFINITY;
        for (int j = 0; j < V; ++j) mx = std::max(mx, zr[j]);
        R s = 0;
        for (int j = 0; j < V; ++j) s += std::exp(zr[j] - mx);
        R lse = mx + std::log(s);
        loss_rows[r] = lse - zr[y[r]];
        if (dz) {
            for (int j = 0; j < V; ++j) dz[r * V + j] = std::exp(zr[j] - lse) * scale;
            dz[r * V + y[r]] -= scale;
        }
    }
}

// ---------------------------------------------------------------- the model
template <class R>
struct Acts {
    std::vector<R> x0;                                  // embedding output [M,C]
    std::vector<std::vector<R>> xin, ln1, m1, r1, qkv, att, xmid, ln2, m2, r2, u, g;
    std::vector<R> xL, lnf, mf, rf, logits;
};

// Forward (and backward when grads != null) of the whole model of minigpt.py with
// the readings adopted for GPT-2: pre-LN blocks, fused QKV, tanh GELU, weight-tied
// head. Returns the mean loss over B*T rows (accumulated in double), or NaN when
// targets is null. grads are accumulated into (zero them to start fresh).
// cf.dropout > 0 is the training-mode model (model.train()): dropout after the
// softmax of every head, on the projection output and on the fc2 output.
template <class R>
double model_step(const oracle_cfg& cf, int B, int T, const R* p, const int32_t* idx,
                  const int32_t* tgt, R* grads, double loss_scale, R* logits_out, R* loss_rows_out) {
    const Layout lo = make_layout(cf);
    const int C = cf.n_embd, H = cf.n_head, F = cf.mlp_hidden, V = cf.vocab, L = cf.n_layer;
    const int64_t M = (int64_t)B * T;
    const size_t MC = (size_t)M * C;
    const bool erf_gelu = (cf.variant & ORACLE_GELU_ERF) != 0;
    Drop dr;
    dr.p = cf.dropout;
    dr.seed = cf.seed;
    Acts<R> a;
    auto vec = [](size_t n) { return std::vector<R>(n); };

    // 1) token + position embedding (MiniGPT.forward)
    a.x0 = vec(MC);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const int t = (int)(m % T);
        const R* te = p + lo.wte + (size_t)idx[m] * C;
        const R* pe = p + lo.wpe + (size_t)t * C;
        for (int c = 0; c < C; ++c) a.x0[m * C + c] = te[c] + pe[c];
    }
    // 2) blocks: x = x + sa(ln1(x)); x = x + ffwd(ln2(x))
    std::vector<R> x = a.x0;
    for (int l = 0; l < L; ++l) {
        const LayerOff& W = lo.layer[l];
        a.xin.push_back(x);
        auto h1 = vec(MC), m1 = vec(M), r1 = vec(M);
        layernorm_fwd<R>(M, C, x.data(), p + W.ln1_g, p + W.ln1_b, cf.ln_eps, h1.data(), m1.data(), r1.data());
        auto qkv = vec((size_t)M * 3 * C);
        linear_fwd<R>(M, 3 * C, C, h1.data(), p + W.w_qkv, W.b_qkv == NONE ? nullptr : p + W.b_qkv, qkv.data());
        dr.layer = l;
        auto att = vec(MC);
        attention_fwd<R>(B, T, C, H, qkv.data(), att.data(), dr);
        auto pr = vec(MC);
        linear_fwd<R>(M, C, C, att.data(), p + W.w_proj, W.b_proj == NONE ? nullptr : p + W.b_proj, pr.data());
        residual_dropout<R>(dr, DROP_PROJ, M, C, pr.data());
        for (size_t i = 0; i < MC; ++i) x[i] += pr[i];
        a.xmid.push_back(x);
        auto h2 = vec(MC), m2 = vec(M), r2 = vec(M);
        layernorm_fwd<R>(M, C, x.data(), p + W.ln2_g, p + W.ln2_b, cf.ln_eps, h2.data(), m2.data(), r2.data());
        auto u = vec((size_t)M * F);
        linear_fwd<R>(M, F, C, h2.data(), p + W.w_fc, W.b_fc == NONE ? nullptr : p + W.b_fc, u.data());
        auto gg = vec((size_t)M * F);
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < M * F; ++i) gg[i] = gelu<R>(u[i], erf_gelu);
        auto mo = vec(MC);
        linear_fwd<R>(M, C, F, gg.data(), p + W.w_fc2, W.b_fc2 == NONE ? nullptr : p + W.b_fc2, mo.data());
        residual_dropout<R>(dr, DROP_FC2, M, C, mo.data());
        for (size_t i = 0; i < MC; ++i) x[i] += mo[i];
        if (grads) {
            a.ln1.push_back(std::move(h1)); a.m1.push_back(std::move(m1)); a.r1.push_back(std::move(r1));
            a.qkv.push_back(std::move(qkv)); a.att.push_back(std::move(att));
            a.ln2.push_back(std::move(h2)); a.m2.push_back(std::move(m2)); a.r2.push_back(std::move(r2));
            a.u.push_back(std::move(u)); a.g.push_back(std::move(gg));
        }
    }
    // 3) final LayerNorm and the head: logits = ln_f(x) . lm_head^T (lm_head is
    //    wte itself when tied)
    a.xL = x;
    a.lnf = vec(MC); a.mf = vec(M); a.rf = vec(M);
    layernorm_fwd<R>(M, C, x.data(), p + lo.lnf_g, p + lo.lnf_b, cf.ln_eps, a.lnf.data(), a.mf.data(), a.rf.data());
    a.logits = vec((size_t)M * V);
    linear_fwd<R>(M, V, C, a.lnf.data(), p + lo.lm_head, nullptr, a.logits.data());
    if (logits_out) std::memcpy(logits_out, a.logits.data(), sizeof(R) * (size_t)M * V);
    if (!tgt) return NAN;

    // 4) loss: mean over all B*T positions
    std::vector<R> lrows(M);
    std::vector<R> dz;
    if (grads) dz = vec((size_t)M * V);
    const R scale = (R)(loss_scale / (double)M);
    cross_entropy<R>(M, V, a.logits.data(), tgt, lrows.data(), grads ? dz.data() : nullptr, scale);
    double loss = 0;
    for (int64_t m = 0; m < M; ++m) loss += (double)lrows[m];
    loss /= (double)M;
    if (loss_rows_out) std::memcpy(loss_rows_out, lrows.data(), sizeof(R) * M);
    if (!grads) return loss;

    // 5) backward, layer by layer in reverse
    R* gp = grads;
    auto dxf = vec(MC);
    linear_bwd<R>(M, V, C, dz.data(), a.lnf.data(), p + lo.lm_head, dxf.data(), gp + lo.lm_head, nullptr);
    dz.clear(); dz.shrink_to_fit();
    std::vector<R> dx(MC, (R)0);  // gradient of the residual stream
    layernorm_bwd<R>(M, C, dxf.data(), a.xL.data(), a.mf.data(), a.rf.data(), p + lo.lnf_g, dx.data(),
                     gp + lo.lnf_g, gp + lo.lnf_b);
    for (int l = L - 1; l >= 0; --l) {
        const LayerOff& W = lo.layer[l];
        dr.layer = l;
        // x_out = x_mid + drop(fc2(gelu(fc(ln2(x_mid)))))
        std::vector<R> dmo = dx;
        residual_dropout<R>(dr, DROP_FC2, M, C, dmo.data());
        auto dg = vec((size_t)M * F);
        linear_bwd<R>(M, C, F, dmo.data(), a.g[l].data(), p + W.w_fc2, dg.data(), gp + W.w_fc2,
                      W.b_fc2 == NONE ? nullptr : gp + W.b_fc2);
        auto& u = a.u[l];
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < M * F; ++i) dg[i] *= gelu_grad<R>(u[i], erf_gelu);
        auto dh2 = vec(MC);
        linear_bwd<R>(M, F, C, dg.data(), a.ln2[l].data(), p + W.w_fc, dh2.data(), gp + W.w_fc,
                      W.b_fc == NONE ? nullptr : gp + W.b_fc);
        layernorm_bwd<R>(M, C, dh2.data(), a.xmid[l].data(), a.m2[l].data(), a.r2[l].data(), p + W.ln2_g,
                         dx.data(), gp + W.ln2_g, gp + W.ln2_b);
        // x_mid = x_in + drop(proj(attn(ln1(x_in))))
        std::vector<R> dpr = dx;
        residual_dropout<R>(dr, DROP_PROJ, M, C, dpr.data());
        auto datt = vec(MC);
        linear_bwd<R>(M, C, C, dpr.data(), a.att[l].data(), p + W.w_proj, datt.data(), gp + W.w_proj,
                      W.b_proj == NONE ? nullptr : gp + W.b_proj);
        auto dqkv = vec((size_t)M * 3 * C);
        attention_bwd<R>(B, T, C, H, a.qkv[l].data(), datt.data(), dqkv.data(), dr);
        auto dh1 = vec(MC);
        linear_bwd<R>(M, 3 * C, C, dqkv.data(), a.ln1[l].data(), p + W.w_qkv, dh1.data(), gp + W.w_qkv,
                      W.b_qkv == NONE ? nullptr : gp + W.b_qkv);
        layernorm_bwd<R>(M, C, dh1.data(), a.xin[l].data(), a.m1[l].data(), a.r1[l].data(), p + W.ln1_g,
                         dx.data(), gp + W.ln1_g, gp + W.ln1_b);
        // free this layer's saved activations
        a.g[l].clear(); a.g[l].shrink_to_fit(); a.u[l].clear(); a.u[l].shrink_to_fit();
        a.qkv[l].clear(); a.qkv[l].shrink_to_fit();
    }
    // 6) embedding backward: dwte[idx[m]] += dx[m] in position order, dwpe[t] += sum_b dx[b,t]
#pragma omp parallel for schedule(static)
    for (int c = 0; c < C; ++c) {
        for (int64_t m = 0; m < M; ++m) {
            gp[lo.wte + (size_t)idx[m] * C + c] += dx[m * C + c];
            gp[lo.wpe + (size_t)(m % T) * C + c] += dx[m * C + c];
        }
    }
    return loss;
}

// ---------------------------------------------------------------- optimiser
// Decoupled weight decay Adam (torch.optim.AdamW as the minigpt loop uses it):
// p *= 1 - lr*wd; m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2;
// p -= lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).
template <class R>
void adamw(int64_t n, R* p, const R* g, R* m, R* v, double lr, double b1, double b2, double eps,
           double wd, int t, const uint8_t* decay) {
    const R bc1 = (R)(1.0 - std::pow(b1, t));
    const R bc2 = (R)(1.0 - std::pow(b2, t));
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        if (!decay || decay[i]) p[i] *= (R)(1.0 - lr * wd);
        m[i] = (R)b1 * m[i] + (R)(1.0 - b1) * g[i];
        v[i] = (R)b2 * v[i] + (R)(1.0 - b2) * g[i] * g[i];
        R mh = m[i] / bc1;
        R vh = v[i] / bc2;
        p[i] -= (R)lr * mh / (std::sqrt(vh) + (R)eps);
    }
}

// Global L2 norm over all gradients (accumulated in double); if clip > 0 and the
// norm exceeds it, every gradient is scaled by clip / (norm + 1e-6).
template <class R>
double clip_grads(int64_t n, R* g, double clip) {
    double s = 0;
    for (int64_t i = 0; i < n; ++i) s += (double)g[i] * (double)g[i];
    double norm = std::sqrt(s);
    if (clip > 0 && norm > clip) {
        const R coef = (R)(clip / (norm + 1e-6));
        for (int64_t i = 0; i < n; ++i) g[i] *= coef;
    }
    return norm;
}

}  // namespace

// ============================================================ C entry points
extern "C" {

void oracle_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
int oracle_max_threads(void) { return omp_get_max_threads(); }

// Number of parameters of the oracle's compact layout (a tied head counted once).
int64_t oracle_n_params(const oracle_cfg* c) {
    if (!c || !cfg_ok(*c)) return -1;
    return (int64_t)make_layout(*c).total;
}

// Fills out[5*i .. 5*i+4] = {kind, layer, offset, rows, cols} for every tensor of
// the compact layout (layer = -1 for global tensors). Returns the tensor count.
int oracle_param_table(const oracle_cfg* c, int64_t* out, int cap) {
    if (!c || !cfg_ok(*c)) return -1;
    Layout lo = make_layout(*c);
    const int64_t V = c->vocab, T = c->block_size, C = c->n_embd, F = c->mlp_hidden;
    int n = 0;
    auto put = [&](int kind, int layer, size_t off, int64_t r, int64_t cc) {
        if (off == NONE) return;
        if (n < cap) { int64_t* e = out + 5 * n; e[0] = kind; e[1] = layer; e[2] = (int64_t)off; e[3] = r; e[4] = cc; }
        ++n;
    };
    put(K_WTE, -1, lo.wte, V, C);
    put(K_WPE, -1, lo.wpe, T, C);
    for (int l = 0; l < c->n_layer; ++l) {
        const LayerOff& L = lo.layer[l];
        put(K_LN1_G, l, L.ln1_g, 1, C); put(K_LN1_B, l, L.ln1_b, 1, C);
        put(K_W_QKV, l, L.w_qkv, 3 * C, C); put(K_B_QKV, l, L.b_qkv, 1, 3 * C);
        put(K_W_PROJ, l, L.w_proj, C, C); put(K_B_PROJ, l, L.b_proj, 1, C);
        put(K_LN2_G, l, L.ln2_g, 1, C); put(K_LN2_B, l, L.ln2_b, 1, C);
        put(K_W_FC, l, L.w_fc, F, C); put(K_B_FC, l, L.b_fc, 1, F);
        put(K_W_FC2, l, L.w_fc2, C, F); put(K_B_FC2, l, L.b_fc2, 1, C);
    }
    put(K_LNF_G, -1, lo.lnf_g, 1, C); put(K_LNF_B, -1, lo.lnf_b, 1, C);
    if (c->variant & ORACLE_UNTIED) put(K_LM_HEAD, -1, lo.lm_head, V, C);
    return n;
}

#define ORACLE_STEP(SUF, R)                                                                       \
    double oracle_step_##SUF(const oracle_cfg* c, int B, int T, const R* params, const int32_t* idx, \
                             const int32_t* tgt, R* grads, double loss_scale, R* logits_out,       \
                             R* loss_rows_out) {                                                   \
        if (!c || !cfg_ok(*c) || B < 1 || T < 1 || T > c->block_size) return NAN;                 \
        for (int64_t m = 0; m < (int64_t)B * T; ++m)                                               \
            if (idx[m] < 0 || idx[m] >= c->vocab || (tgt && (tgt[m] < 0 || tgt[m] >= c->vocab)))  \
                return NAN;                                                                       \
        return model_step<R>(*c, B, T, params, idx, tgt, grads, loss_scale, logits_out,          \
                             loss_rows_out);                                                       \
    }
ORACLE_STEP(f32, float)
ORACLE_STEP(f64, double)

#define ORACLE_UNITS(SUF, R)                                                                      \
    void oracle_layernorm_##SUF(int64_t rows, int C, const R* x, const R* g, const R* b, double eps, \
                                R* y, R* mean, R* rstd) {                                          \
        layernorm_fwd<R>(rows, C, x, g, b, eps, y, mean, rstd);                                   \
    }                                                                                              \
    void oracle_layernorm_bwd_##SUF(int64_t rows, int C, const R* dy, const R* x, const R* mean,   \
                                    const R* rstd, const R* g, R* dx, R* dg, R* db) {              \
        layernorm_bwd<R>(rows, C, dy, x, mean, rstd, g, dx, dg, db);                              \
    }                                                                                              \
    void oracle_linear_##SUF(int64_t M, int N, int K, const R* X, const R* W, const R* b, R* Y) {  \
        linear_fwd<R>(M, N, K, X, W, b, Y);                                                        \
    }                                                                                              \
    void oracle_linear_bwd_##SUF(int64_t M, int N, int K, const R* dY, const R* X, const R* W,     \
                                 R* dX, R* dW, R* db) {                                            \
        linear_bwd<R>(M, N, K, dY, X, W, dX, dW, db);                                              \
    }                                                                                              \
    void oracle_gelu_##SUF(int64_t n, const R* u, R* y, R* dy, int erf_form) {                     \
        for (int64_t i = 0; i < n; ++i) {                                                          \
            if (y) y[i] = gelu<R>(u[i], erf_form != 0);                                            \
            if (dy) dy[i] = gelu_grad<R>(u[i], erf_form != 0);                                     \
        }                                                                                          \
    }                                                                                              \
    void oracle_head_attention_##SUF(int T, int d, const R* q, const R* k, const R* v, R* out,     \
                                     R* P) {                                                       \
        std::vector<R> srow(T > 0 ? T : 1);                                                        \
        head_fwd<R>(T, d, q, k, v, d, out, d, P, srow.data());                                     \
    }                                                                                              \
    void oracle_attention_##SUF(int B, int T, int C, int H, const R* qkv, R* out) {                \
        attention_fwd<R>(B, T, C, H, qkv, out);                                                    \
    }                                                                                              \
    void oracle_attention_bwd_##SUF(int B, int T, int C, int H, const R* qkv, const R* dout,       \
                                    R* dqkv) {                                                     \
        attention_bwd<R>(B, T, C, H, qkv, dout, dqkv);                                             \
    }                                                                                              \
    void oracle_cross_entropy_##SUF(int64_t rows, int V, const R* z, const int32_t* y, R* loss_rows, \
                                    R* dz, double scale) {                                         \
        cross_entropy<R>(rows, V, z, y, loss_rows, dz, (R)scale);                                  \
    }                                                                                              \
    void oracle_adamw_##SUF(int64_t n, R* p, const R* g, R* m, R* v, double lr, double b1,         \
                            double b2, double eps, double wd, int t, const uint8_t* decay) {       \
        adamw<R>(n, p, g, m, v, lr, b1, b2, eps, wd, t, decay);                                    \
    }                                                                                              \
    double oracle_clip_##SUF(int64_t n, R* g, double clip) { return clip_grads<R>(n, g, clip); }
ORACLE_UNITS(f32, float)
ORACLE_UNITS(f64, double)

// Linear warmup to max_lr over `warmup` iterations, then cosine decay to min_lr
// at max_iters, min_lr afterwards (the knobs of train_gpt2.py on the nanogpt page;
// the formula is the reading adopted for the shape it leaves unstated).
double oracle_lr(int64_t it, double max_lr, double min_lr, int64_t warmup, int64_t max_iters) {
    const double pi = 3.14159265358979323846;
    if (it < warmup) return max_lr * (double)(it + 1) / (double)warmup;
    if (it >= max_iters) return min_lr;
    double ratio = (double)(it - warmup) / (double)(max_iters - warmup);
    return min_lr + 0.5 * (1.0 + std::cos(pi * ratio)) * (max_lr - min_lr);
}

// Philox4x32-10 itself (for its known-answer vectors) and the keep flags of
// elements e0 .. e0 + n - 1 of one dropout site (1 = kept).
void oracle_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out) { philox4x32_10(ctr, key, out); }
void oracle_dropout_keep(double p, uint64_t seed, int site, int layer, uint64_t e0, int64_t n, uint8_t* out) {
    const uint32_t thr = drop_threshold(p);
    for (int64_t i = 0; i < n; ++i) out[i] = keep(seed, site, layer, e0 + (uint64_t)i, thr) ? 1 : 0;
}

// Row argmax with the lowest index winning ties.
void oracle_argmax_f32(int64_t rows, int V, const float* z, int32_t* out) {
    for (int64_t r = 0; r < rows; ++r) {
        int best = 0;
        for (int j = 1; j < V; ++j)
            if (z[r * V + j] > z[r * V + best]) best = j;
        out[r] = best;
    }
}

}  // extern "C"
