// Host-only planning: configuration checks, the flat parameter layout and the
// activation arena. No device code; compiled into the same shared library.
#include <cmath>
#include <cstring>

#include "common.h"

namespace g2 {

static int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int validate_config(const gpt2_config* c) {
    if (!c) return GPT2_EINVAL;
    if (c->vocab < 1 || c->block_size < 1 || c->n_embd < 1 || c->n_head < 1 || c->n_layer < 1 ||
        c->mlp_hidden < 1)
        return GPT2_EINVAL;
    // d_model must split evenly across heads (the assert in MultiHeadAttention)
    if (c->n_embd % c->n_head != 0) return GPT2_EINVAL;
    if (c->bias != 0 && c->bias != 1) return GPT2_EINVAL;
    if (c->dtype != GPT2_DTYPE_F32 && c->dtype != GPT2_DTYPE_BF16) return GPT2_EINVAL;
    if (!(c->ln_eps > 0.0f) || !std::isfinite(c->ln_eps)) return GPT2_EINVAL;
    if ((c->gelu_erf != 0 && c->gelu_erf != 1) || (c->untied_head != 0 && c->untied_head != 1)) return GPT2_EINVAL;
    if (!(c->dropout >= 0.0f && c->dropout < 1.0f)) return GPT2_EINVAL;
    const int d = c->n_embd / c->n_head;
    if (d > 128) return GPT2_EINVAL;
    if (c->dtype == GPT2_DTYPE_BF16) {
        // 16-byte vector loads of bf16 rows
        if (c->n_embd % 8 != 0 || c->mlp_hidden % 8 != 0 || d % 8 != 0) return GPT2_EINVAL;
    }
    // flat-buffer offsets stay well inside int64 and per-row indexing inside int32
    if ((int64_t)c->vocab * c->n_embd > (int64_t)1 << 40) return GPT2_EINVAL;
    return GPT2_OK;
}

ParamLayout make_param_layout(const gpt2_config& c) {
    ParamLayout pl;
    const int64_t V = c.vocab, T = c.block_size, C = c.n_embd, F = c.mlp_hidden;
    pl.vocab_pad = round_up(V, kVocabPad);
    int64_t off = 0;
    int64_t n_real = 0;
    auto take = [&](const std::string& name, int layer, int decay, int64_t rows, int64_t cols,
                    int64_t reserve_rows) -> int64_t {
        TensorDesc t;
        t.name = name;
        t.layer = layer;
        t.decay = decay;
        t.offset = off;
        t.rows = rows;
        t.cols = cols;
        t.reserved = round_up(reserve_rows * cols, kParamAlign);
        pl.tensors.push_back(t);
        off += t.reserved;
        n_real += rows * cols;
        return t.offset;
    };
    // the embedding table keeps its rows padded to a multiple of kVocabPad (zero
    // rows), so the head's GEMMs see whole tiles; padded logits are ignored
    pl.wte = take("wte", -1, 1, V, C, pl.vocab_pad);
    pl.wpe = take("wpe", -1, 1, T, C, T);
    for (int l = 0; l < c.n_layer; ++l) {
        LayerW w;
        const std::string p = "h" + std::to_string(l) + ".";
        w.ln1_g = take(p + "ln1_g", l, 0, 1, C, 1);
        w.ln1_b = take(p + "ln1_b", l, 0, 1, C, 1);
        w.w_qkv = take(p + "w_qkv", l, 1, 3 * C, C, 3 * C);
        w.b_qkv = c.bias ? take(p + "b_qkv", l, 0, 1, 3 * C, 1) : -1;
        w.w_proj = take(p + "w_proj", l, 1, C, C, C);
        w.b_proj = c.bias ? take(p + "b_proj", l, 0, 1, C, 1) : -1;
        w.ln2_g = take(p + "ln2_g", l, 0, 1, C, 1);
        w.ln2_b = take(p + "ln2_b", l, 0, 1, C, 1);
        w.w_fc = take(p + "w_fc", l, 1, F, C, F);
        w.b_fc = c.bias ? take(p + "b_fc", l, 0, 1, F, 1) : -1;
        w.w_fc2 = take(p + "w_fc2", l, 1, C, F, C);
        w.b_fc2 = c.bias ? take(p + "b_fc2", l, 0, 1, C, 1) : -1;
        pl.layer.push_back(w);
    }
    pl.lnf_g = take("lnf_g", -1, 0, 1, C, 1);
    pl.lnf_b = take("lnf_b", -1, 0, 1, C, 1);
    // untied: the head's own weight, rows padded like wte's; tied: wte itself
    pl.lm_head = c.untied_head ? take("lm_head", -1, 1, V, C, pl.vocab_pad) : pl.wte;
    pl.n_flat = off;
    pl.n_real = n_real;
    return pl;
}

ArenaPlan make_arena_plan(const gpt2_config& c, const ParamLayout& pl, int B, int T, int mode) {
    ArenaPlan a;
    const bool gen = mode == GPT2_MODE_GENERATE;
    // generation runs one position of B sequences at a time; T is the cache length
    a.M = gen ? B : B * T;
    a.B = B;
    a.T = T;
    a.mode = mode;
    a.act_bytes = c.dtype == GPT2_DTYPE_BF16 ? 2 : 4;
    const size_t M = (size_t)a.M, C = c.n_embd, F = c.mlp_hidden, H = c.n_head;
    const size_t Vp = (size_t)pl.vocab_pad;
    const size_t ab = a.act_bytes;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        Region r;
        r.off = off;
        r.bytes = bytes;
        off += (bytes + 255) / 256 * 256;
        return r;
    };
    a.scalars = take(256);
    a.wlp = take(c.dtype == GPT2_DTYPE_BF16 ? (size_t)pl.n_flat * 2 : 0);
    a.decay_tab = take((size_t)(pl.n_flat / kParamAlign));
    a.norm_blocks = 1024;
    a.norm_part = take(sizeof(double) * a.norm_blocks);
    const bool train = mode == GPT2_MODE_TRAIN;
    const int slots = train ? c.n_layer : 1;
    for (int l = 0; l < slots; ++l) {
        a.x.push_back(take(M * C * 4));
        a.ln1.push_back(take(M * C * ab));
        a.m1.push_back(take(M * 4));
        a.r1.push_back(take(M * 4));
        a.qkv.push_back(take(M * 3 * C * ab));
        a.att.push_back(take(M * C * ab));
        a.lse.push_back(take((size_t)B * H * (gen ? 1 : T) * 4));
        a.xmid.push_back(take(M * C * 4));
        a.ln2.push_back(take(M * C * ab));
        a.m2.push_back(take(M * 4));
        a.r2.push_back(take(M * 4));
        a.fch.push_back(take(M * F * ab));
        a.fcg.push_back(take(M * F * ab));
    }
    a.xL = take(M * C * 4);
    a.xf = take(M * C * ab);
    a.mf = take(M * 4);
    a.rf = take(M * 4);
    a.logits = take(M * Vp * (gen ? 4 : ab));
    if (gen)
        for (int l = 0; l < c.n_layer; ++l) {
            a.kc.push_back(take((size_t)B * T * C * ab));
            a.vc.push_back(take((size_t)B * T * C * ab));
        }
    a.loss_rows = take(M * 4);
    if (train) {
        a.dres = take(M * C * 4);
        a.dres_act = take(M * C * ab);
        a.dres_act2 = take(M * C * ab);
        a.dtmp = take(M * C * 4);
        a.dF = take(M * F * ab);
        a.dqkv = take(M * 3 * C * ab);
        a.datt = take(M * C * ab);
        a.attD = take((size_t)B * H * T * 4 * 2);  // D and base-2 lse for the attention backward
        a.ln_part_rows = (int)((M + 15) / 16);
        for (int i = 0; i < 2 * c.n_layer + 1; ++i)
            a.ln_part.push_back(take((size_t)a.ln_part_rows * 3 * C * 4));  // dg, db and the dres column sums
        size_t maxN = 3 * C > F ? 3 * C : F;
        a.bias_part_rows = (int)((M + 63) / 64);
        for (int i = 0; i < 2 * c.n_layer; ++i) a.bias_part.push_back(take((size_t)a.bias_part_rows * maxN * 4));
        a.colsum_jobs = take((size_t)(4 * c.n_layer + 1) * sizeof(ColsumJob));
        a.enc_count = take(Vp * 4);
        a.enc_start = take(Vp * 4);
        a.enc_segstart = take(Vp * 4);
        a.enc_order = take(M * 4);
        a.enc_segtok = take(M * 4);
        if (c.dropout > 0.0f) {
            a.dm_tw = (T + 63) / 64;
            a.dm_attn_words = (int64_t)B * H * T * a.dm_tw;
            a.dm_res_words = (int64_t)((M * C + 63) / 64);
            a.dm_attn = take((size_t)c.n_layer * a.dm_attn_words * 8);
            a.dm_proj = take((size_t)c.n_layer * a.dm_res_words * 8);
            a.dm_fc2 = take((size_t)c.n_layer * a.dm_res_words * 8);
        }
    }
    a.total = off;
    return a;
}

}  // namespace g2
