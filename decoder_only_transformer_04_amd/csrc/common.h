// Internal declarations shared by the host plan and the HIP kernels of the
// GPT-2 training-step library (gfx950 only).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/gpt2.h"

#ifdef __HIPCC__
#include <hip/hip_runtime.h>
#endif

namespace g2 {

typedef uint16_t bf16_t;  // bf16 bit pattern in memory

// --------------------------------------------------------------- layout of the flat buffers
static const int64_t kParamAlign = 256;  // every tensor starts on a 256-element boundary
static const int64_t kVocabPad = 128;    // wte rows reserved up to a multiple of this

struct TensorDesc {
    std::string name;
    int layer;
    int decay;
    int64_t offset, rows, cols, reserved;
};

struct LayerW {
    int64_t ln1_g, ln1_b, w_qkv, b_qkv, w_proj, b_proj, ln2_g, ln2_b, w_fc, b_fc, w_fc2, b_fc2;  // -1: absent
};

struct ParamLayout {
    int64_t wte, wpe, lnf_g, lnf_b;
    int64_t lm_head;  // the head's weight: wte's offset when tied
    std::vector<LayerW> layer;
    std::vector<TensorDesc> tensors;
    int64_t n_flat;   // total elements incl. padding (multiple of kParamAlign)
    int64_t n_real;   // exact parameter count
    int64_t vocab_pad;
};

int validate_config(const gpt2_config* c);
ParamLayout make_param_layout(const gpt2_config& c);

// --------------------------------------------------------------- arena plan
struct Region {
    size_t off = 0, bytes = 0;
};

struct ArenaPlan {
    int M, B, T, mode;
    size_t act_bytes;  // 2 (bf16) or 4 (f32)
    Region scalars;    // status word, clip coefficient, loss
    Region wlp;        // low-precision weights (bf16 mode)
    Region decay_tab;  // one byte per kParamAlign chunk of the flat buffers
    Region norm_part;  // grad-norm partial sums (double)
    // forward activations, per layer (eval mode: one slot reused)
    std::vector<Region> x, xmid, ln1, m1, r1, qkv, att, lse, ln2, m2, r2, fch, fcg;
    Region xL, xf, mf, rf, logits, loss_rows;
    // generation: per-layer key and value caches [B, block_size, C] (activation
    // type); logits are fp32 [B, Vp] there, for the sampler
    std::vector<Region> kc, vc;
    // backward scratch
    // dres_act / dres_act2: activation-type copies of the residual gradient,
    // written alternately (LayerNorm-f and LN1 backward, LN2 backward) so a
    // weight gradient reading one has a whole sub-layer to finish before the
    // next write to it
    Region dres, dres_act, dres_act2, dtmp, dF, dqkv, datt, attD;
    // training-mode dropout keep masks (all layers; empty without dropout)
    Region dm_attn, dm_proj, dm_fc2;
    int64_t dm_attn_words = 0, dm_res_words = 0;  // 64-bit words per layer
    int dm_tw = 0;                                // words per attention row
    // parameter-gradient partials, one buffer per producer so that all of them
    // are reduced by one launch at the end of the backward: LayerNorm backward
    // calls in issue order (ln_f, then ln2 and ln1 of each layer from the top),
    // and per layer the fc and the qkv bias partials
    std::vector<Region> ln_part, bias_part;
    Region colsum_jobs;  // the ColsumJob table of those reductions
    Region enc_count, enc_start, enc_segstart, enc_order, enc_segtok;
    size_t total = 0;
    int ln_part_rows = 0;    // partial rows of the LayerNorm parameter-gradient reduction
    int bias_part_rows = 0;  // partial rows of the bias-gradient reduction
    int norm_blocks = 0;
};

ArenaPlan make_arena_plan(const gpt2_config& c, const ParamLayout& pl, int B, int T, int mode);

// --------------------------------------------------------------- scalars region (int32/float slots)
enum ScalarSlot {
    SLOT_STATUS = 0,   // uint32 sticky status bits
    SLOT_COEF = 1,     // float clip coefficient for AdamW
    SLOT_NORM = 2,     // float gradient norm
    SLOT_LOSS = 3,     // float mean loss (when the caller passes no loss pointer)
    SLOT_NSEG = 4,     // int32 number of token segments (embedding backward)
    SLOT_GEN = 5       // int32 [3]: generation step state (column, position, prompt length)
};

// --------------------------------------------------------------- GEMM
enum Epilogue {
    EPI_STORE = 0,      // C(act) = alpha*acc + bias
    EPI_GELU = 1,       // u = acc + bias: C(act) = gelu_tanh'(u), C2(act) = gelu_tanh(u)
    EPI_RESID = 2,      // C(f32) = R(f32) + acc + bias      (C may alias R)
    EPI_F32 = 3,        // C(f32) = alpha*acc (+ C if accumulate)
    EPI_GELU_BWD = 4    // C(act) = acc * R(act), R the GELU derivative EPI_GELU wrote
};

struct GemmArgs {
    int64_t M;
    int N, K;
    const void* A; int64_t lda; bool a_kc;  // a_kc: A(m,k) = A[m*lda+k], else A[k*lda+m]
    const void* B; int64_t ldb; bool b_kc;  // b_kc: B(k,n) = B[n*ldb+k], else B[k*ldb+n]
    int epi;
    float alpha;
    const float* bias;
    void* C; int64_t ldc;
    void* C2; int64_t ldc2;
    const void* R; int64_t ldr;
    int accumulate;
    int gelu_erf;  // EPI_GELU: exact erf form instead of the tanh approximation
    // few-row products (at most 16 rows, K <= 1024, EPI_STORE or EPI_GELU): when
    // ln_g is set, A is fp32 and the operand is its LayerNorm with ln_g, ln_b, ln_eps
    const float* ln_g;
    const float* ln_b;
    float ln_eps;
    void* split_buf; size_t split_bytes;  // fp32 scratch for split-K partials (nullable)
    // EPI_GELU_BWD only (nullable): column sums of the output over each 64-row
    // block, written to colsum_part[(m / 64) * N + n] (the bias gradient's partials)
    float* colsum_part;
    // EPI_RESID only (nullable): dropout of the branch, C = R + keep(m N + n) *
    // dscale * (acc + bias), keep bits LSB-first in bytes (see dropout_masks_res)
    const uint8_t* dmask;
    float dscale;
};

#ifdef __HIPCC__
// launchers (return hipError_t of the launch)
hipError_t gemm(int dtype, const GemmArgs& a, hipStream_t s);

hipError_t encoder_fwd(int dtype, const int32_t* idx, const float* wte32, const bf16_t* wte16,
                       const float* wpe32, const bf16_t* wpe16, float* x, int M, int T, int C, int V,
                       uint32_t* status, hipStream_t s);
hipError_t layernorm_fwd(int dtype, const float* x, const float* g, const float* b, float eps, void* y,
                         float* mean, float* rstd, int64_t rows, int C, hipStream_t s);
// with_res: the partial rows also carry the column sums of the updated dres
// (layout per partial row: dg[C], db[C], dres[C]; else dg[C], db[C])
// dmask (nullable): the activation copy and the dres column sums are of the
// dropped residual gradient keep(row C + c) * dscale * dres (the gradient of the
// dropout branch that feeds dres); dres itself is never masked
hipError_t layernorm_bwd(int dtype, const float* dy, const float* x, const float* mean, const float* rstd,
                         const float* g, float* dres, void* dres_act, float* part, int part_rows, int64_t rows, int C,
                         int add, int with_res, hipStream_t s, const uint8_t* dmask = nullptr, float dscale = 1.0f);
int ln_bwd_partial_rows(int64_t rows);  // partial rows layernorm_bwd writes
hipError_t colsum_finish2(const float* part, int part_rows, int ld, float* out_a, int na, float* out_b, int nb,
                          int accumulate, hipStream_t s);
hipError_t colsum_finish3(const float* part, int part_rows, int ld, float* out_a, int na, float* out_b, int nb,
                          float* out_c, int nc, int accumulate, hipStream_t s);
// One deferred column-sum reduction: out (+)= sums over prows rows of `part`
// (row stride ld) of its first na + nb + nc columns, split over up to three
// outputs as colsum_finish3 does; blk0 is the job's first block in the batch.
struct ColsumJob {
    const float* part;
    float* out_a;
    float* out_b;
    float* out_c;
    int prows, ld, na, nb, nc, blk0;
    int pad[2];
};
bool colsum_job_vector(const ColsumJob& j);  // the batched kernel needs multiples of 4
int colsum_job_blocks(const ColsumJob& j);
hipError_t colsum_jobs(const ColsumJob* d_jobs, int njobs, int nblocks, int accumulate, hipStream_t s);
int bias_partial_rows(int64_t rows, int N);  // partial rows bias_partials writes
hipError_t bias_partials(int dtype, const void* dY, int64_t rows, int N, float* part, int part_rows, hipStream_t s);
hipError_t bias_grad(int dtype, const void* dY, int64_t rows, int N, float* part, int part_rows, float* db,
                     int accumulate, hipStream_t s);
// dmask (nullable): dropout of the attention weights, keep bit of query i, key j
// of (b, h) at bit j % 64 of word ((b H + h) T + i) Tw + j / 64, Tw = ceil(T / 64);
// the weights P_ij * keep * dscale multiply v_j (lse stays that of P)
hipError_t attention_fwd(int dtype, int B, int T, int C, int H, const void* qkv, void* out, float* lse,
                         hipStream_t s, const uint64_t* dmask = nullptr, float dscale = 1.0f);
// attention backward runs as two launches on the MFMA path: dQ (which also forms
// D = rowsum(dO*O) and writes it with lse in base 2 to Dbuf) and then dK/dV;
// `stages` selects which of them to enqueue (the scalar path takes both only).
// Dbuf: 2 B H T floats (D, then lse in base 2).
enum { ATT_BWD_DQ = 2, ATT_BWD_DKDV = 4, ATT_BWD_ALL = 6 };
bool attention_bwd_staged(int dtype, int C, int H);
hipError_t attention_bwd(int dtype, int B, int T, int C, int H, const void* qkv, const void* out,
                         const float* lse, const void* dout, void* dqkv, float* Dbuf, hipStream_t s,
                         int stages = ATT_BWD_ALL, const uint64_t* dmask = nullptr, float dscale = 1.0f);

// --------------------------------------------------------------- dropout
// Keep masks from Philox4x32-10 (Salmon et al., SC 2011) under key `seed`:
// element e of site `site`, layer l takes 16-bit half e % 8 (low half of word 0
// first) of the generator at counter (e / 8 low, e / 8 high, site, l) and is
// kept when that half is >= thr (round(p 65536)). Bits are written LSB-first,
// 64 per word, one block of words_per_layer words per layer, for layers
// layer0 .. layer0 + L - 1 (bits points at layer0's block).
enum { DROP_ATTN = 0, DROP_PROJ = 1, DROP_FC2 = 2 };
// attention site: e = (bh T + i) T + j, stored at bit j % 64 of word (bh T + i) Tw + j / 64;
// words wholly above the diagonal (64 (j / 64) > i) are written as zero
hipError_t dropout_masks_attn(uint64_t* bits, int layer0, int L, int64_t words_per_layer, int BH, int T, int Tw,
                              uint64_t seed, uint32_t thr, hipStream_t s);
// residual sites: e = m C + c over n_elem elements, stored at bit e % 64 of word e / 64
hipError_t dropout_masks_res(uint64_t* bits, int layer0, int L, int64_t words_per_layer, int64_t n_elem, int site,
                             uint64_t seed, uint32_t thr, hipStream_t s);
hipError_t cross_entropy(int dtype, void* logits, int64_t rows, int V, int ld, const int32_t* targets,
                         float* loss_rows, int32_t* argmax, int write_grad, uint32_t* status, hipStream_t s);
hipError_t mean_loss(const float* loss_rows, int64_t rows, float* out, uint32_t* status, hipStream_t s);
hipError_t encoder_bwd(const int32_t* idx, const float* dres, float* dwte, float* dwpe, int M, int T, int C,
                       int V, int32_t* count, int32_t* start, int32_t* seg_start, int32_t* order, int32_t* seg_tok,
                       int32_t* nseg_total, float* seg_part, int accumulate_wpe, hipStream_t s);
hipError_t cast_f32_bf16(const float* src, bf16_t* dst, int64_t n, hipStream_t s);
hipError_t fill_zero(void* p, size_t bytes, hipStream_t s);

// --------------------------------------------------------------- generation
constexpr int kGenMaxCache = 8192;  // longest key/value cache (block_size) gpt2_generate takes
// The step's position is device state cp[3] = {col: sequence column of the token
// fed, pos: its model position, T0: prompt length}, set by gen_set and moved on by
// one by gen_advance, so a captured step replays unchanged.
hipError_t gen_set(int32_t* cp, int col, int pos, int T0, hipStream_t s);
hipError_t gen_advance(int32_t* cp, hipStream_t s);
// x[b] = wte[seq[b * seq_ld + col]] + wpe[pos] for B rows (fp32 tables); an id
// outside [0, V) sets GPT2_STATUS_TOKEN_RANGE and embeds token 0
hipError_t gen_embed(const int32_t* seq, int64_t seq_ld, const int32_t* cp, const float* wte, const float* wpe,
                     float* x, int B, int C, int V, uint32_t* status, hipStream_t s);
// per (b, h): store this step's key and value (qkv [B, 3C]) at position pos of
// the caches [B, Tc, C], then out[b, h] = softmax_j(q . k_j / sqrt(d)) v_j over j <= pos
hipError_t gen_attention(int dtype, const void* qkv, void* kc, void* vc, int Tc, const int32_t* cp, void* out, int B,
                         int C, int H, hipStream_t s);
// per row b: the smallest k whose cumulative softmax(logits[b, :V] / temperature)
// probability exceeds u[b * u_ld + (col + 1 - T0)]; written to seq[b * seq_ld + col + 1]
hipError_t gen_sample(const float* logits, int Vp, int V, float temperature, const float* u, int64_t u_ld,
                      const int32_t* cp, int32_t* seq, int64_t seq_ld, int B, hipStream_t s);
hipError_t grad_norm(const float* g, int64_t n, double* part, int nblocks, float clip, float* norm_out,
                     float* coef_out, float* user_norm, uint32_t* status, hipStream_t s);
hipError_t adamw(float* p, const float* g, float* m, float* v, bf16_t* p16, int64_t n, float lr, float b1,
                 float b2, float eps, float decay_mul, float bc1, float bc2, const uint8_t* decay_tab,
                 const float* coef, hipStream_t s);
#endif

}  // namespace g2
