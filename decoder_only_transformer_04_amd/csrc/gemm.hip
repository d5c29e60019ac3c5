// Dense contractions of the training step: every Linear forward (X . W^T),
// its input gradient (dY . W) and its weight gradient (dY^T . X).
//
// bf16 path: v_mfma_f32_32x32x16_bf16 on LDS-staged 64-deep K tiles, fp32
// accumulation, 4 waves per workgroup in a 2 x 2 arrangement. Operands whose
// contraction index is contiguous in memory ("KC") are staged as [row][64 k]
// with a 16-byte XOR swizzle and read with 128-bit LDS loads; operands whose
// contraction index is strided (dgrad's W, wgrad's dY and X) are staged in
// their natural [k][row] orientation (rows padded by 32 elements) and read
// with the gfx950 LDS transpose load ds_read_b64_tr_b16, so no operand is
// ever transposed in memory. Fused epilogues: bias, tanh-GELU (writing both
// pre- and post-activation), residual add into the fp32 stream, GELU
// derivative, fp32 (accumulating) stores and split-K partials.
//
// fp32 path: a plain LDS-tiled FMA kernel with the same epilogues, used by the
// fp32 mode.
#include <algorithm>

#include "device.h"

#ifndef G2_GEMM_SCHED
#define G2_GEMM_SCHED 0
#endif

#ifndef G2_GEMM_IGLP
#define G2_GEMM_IGLP -1
#endif

namespace g2 {

struct GP {
    const void* A;
    const void* B;
    int64_t lda, ldb;
    int64_t M;
    int N, K;
    int k_per_split;
    float alpha;
    const float* bias;
    void* C;
    int64_t ldc;
    int64_t c_split_stride;
    void* C2;
    int64_t ldc2;
    const void* R;
    int64_t ldr;
    int accumulate;
    int gelu_erf;  // EPI_GELU: exact erf form
    float* cpart;  // GELU_BWD: per-64-row column sums of the output (nullable)
    const float* ln_g;  // skinny products: A is fp32 and the operand is its LayerNorm (nullable)
    const float* ln_b;
    float ln_eps;
    const uint8_t* dmask;  // EPI_RESID: dropout keep bits of the branch (nullable)
    float dscale;
};

// ------------------------------------------------------------------ epilogue
template <int EPI, class T>
__device__ __forceinline__ void epi_apply(const GP& p, int64_t m, int n, float v) {
    const float bias = p.bias ? p.bias[n] : 0.0f;
    if constexpr (EPI == EPI_STORE) {
        Act<T>::st((T*)p.C, m * p.ldc + n, p.alpha * v + bias);
    } else if constexpr (EPI == EPI_GELU) {
        float g, dg;
        if (p.gelu_erf) gelu_erf_and_grad(v + bias, g, dg);
        else gelu_tanh_and_grad(v + bias, g, dg);
        Act<T>::st((T*)p.C, m * p.ldc + n, dg);
        Act<T>::st((T*)p.C2, m * p.ldc2 + n, g);
    } else if constexpr (EPI == EPI_RESID) {
        float r = ((const float*)p.R)[m * p.ldr + n];
        float y = v + bias;
        if (p.dmask) {
            const int64_t e = m * p.N + n;
            y = ((p.dmask[e >> 3] >> (e & 7)) & 1) ? y * p.dscale : 0.0f;
        }
        ((float*)p.C)[m * p.ldc + n] = r + y;
    } else if constexpr (EPI == EPI_F32) {
        float* c = (float*)p.C + (int64_t)blockIdx.z * p.c_split_stride + m * p.ldc + n;
        float o = p.alpha * v;
        if (p.accumulate) o += *c;
        *c = o;
    } else if constexpr (EPI == EPI_GELU_BWD) {
        Act<T>::st((T*)p.C, m * p.ldc + n, v * Act<T>::ld((const T*)p.R, m * p.ldr + n));
    }
}

// Eight consecutive columns n..n+7 of row m (n % 8 == 0, N % 8 == 0): vector
// loads of bias / residual / GELU derivative and 16- or 32-byte stores.
__device__ __forceinline__ uint4 pack8(const float (&o)[8]) {
    uint4 r;
    r.x = pack2bf(o[0], o[1]);
    r.y = pack2bf(o[2], o[3]);
    r.z = pack2bf(o[4], o[5]);
    r.w = pack2bf(o[6], o[7]);
    return r;
}
__device__ __forceinline__ void unpack8(uint4 u, float (&o)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        o[2 * k] = bf2f((bf16_t)(w[k] & 0xffffu));
        o[2 * k + 1] = bf2f((bf16_t)(w[k] >> 16));
    }
}
__device__ __forceinline__ void ld8f(const float* p, float (&o)[8]) {
    const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void st8f(float* p, const float (&o)[8]) {
    *(float4*)p = make_float4(o[0], o[1], o[2], o[3]);
    *(float4*)(p + 4) = make_float4(o[4], o[5], o[6], o[7]);
}

template <int EPI>
__device__ __forceinline__ void epi_apply8(const GP& p, int64_t m, int n, const float (&v)[8], float (&o)[8]) {
    float bv[8];
    if (p.bias) ld8f(p.bias + n, bv);
    else {
#pragma unroll
        for (int k = 0; k < 8; ++k) bv[k] = 0.0f;
    }
    if constexpr (EPI == EPI_STORE) {
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = p.alpha * v[k] + bv[k];
        *(uint4*)((bf16_t*)p.C + m * p.ldc + n) = pack8(o);
    } else if constexpr (EPI == EPI_GELU) {
        float gl[8];
        if (p.gelu_erf) {
#pragma unroll
            for (int k = 0; k < 8; ++k) gelu_erf_and_grad(v[k] + bv[k], gl[k], o[k]);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) gelu_tanh_and_grad(v[k] + bv[k], gl[k], o[k]);
        }
        *(uint4*)((bf16_t*)p.C + m * p.ldc + n) = pack8(o);
        *(uint4*)((bf16_t*)p.C2 + m * p.ldc2 + n) = pack8(gl);
    } else if constexpr (EPI == EPI_RESID) {
        float r[8];
        ld8f((const float*)p.R + m * p.ldr + n, r);
        if (p.dmask) {
            // eight consecutive elements from a multiple of 8 (N % 8 == 0): one byte of keep bits
            const uint32_t kb = p.dmask[(m * p.N + n) >> 3];
#pragma unroll
            for (int k = 0; k < 8; ++k) o[k] = r[k] + (((kb >> k) & 1) ? (v[k] + bv[k]) * p.dscale : 0.0f);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) o[k] = r[k] + v[k] + bv[k];
        }
        st8f((float*)p.C + m * p.ldc + n, o);
    } else if constexpr (EPI == EPI_F32) {
        float* c = (float*)p.C + (int64_t)blockIdx.z * p.c_split_stride + m * p.ldc + n;
        float prev[8];
        if (p.accumulate) ld8f(c, prev);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = p.alpha * v[k] + (p.accumulate ? prev[k] : 0.0f);
        st8f(c, o);
    } else if constexpr (EPI == EPI_GELU_BWD) {
        float dg[8];
        unpack8(*(const uint4*)((const bf16_t*)p.R + m * p.ldr + n), dg);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = v[k] * dg[k];
        *(uint4*)((bf16_t*)p.C + m * p.ldc + n) = pack8(o);
    }
}

// ------------------------------------------------------------------ bf16 MFMA kernel
template <int R, bool KC, int BK = 64, int NT = 256>
struct TileCfg {
    static constexpr int BYTES = R * BK * 2;
    static constexpr int CHUNKS = BYTES / 16 / NT;   // 16-byte chunks per thread per stage (NT threads)
    static constexpr int PITCH = KC ? BK * 2 : R * 2;  // bytes per tile row
    static constexpr int CPR = PITCH / 16;           // 16-byte chunks per tile row
};

// LDS placement of 16-byte chunk `ch` of tile row `row`.
// KC tiles ([R][BK k]): the chunk index is XOR-ed with a function of the row so
// that the 128-bit fragment reads (16 consecutive rows, one chunk) hit 16
// distinct 16-byte bank groups. Transposed tiles ([BK k][R]) are read four
// consecutive rows by four consecutive chunks at a time. With 256- or 512-byte
// rows (R = 128, 256) every row starts on bank 0 and chunk ^ 4 (row mod 4)
// spreads the four rows over the 64 banks. With 384-byte rows (R = 192) odd rows
// already start half-way round, so only bit 2 of the chunk is flipped, by bit 1
// of the row, which keeps every chunk inside its row.
template <int R, bool KC, int BK = 64>
__device__ __forceinline__ int slot_of(int row, int ch) {
    if constexpr (KC) {
        if constexpr (BK == 64) return row * 8 + (ch ^ ((row >> 1) & 7));
        else return row * 4 + (ch ^ ((row >> 2) & 3));
    } else if constexpr (R % 128 == 0) {
        return row * (R / 8) + (ch ^ (4 * (row & 3)));
    } else {
        static_assert(R == 192, "transposed tile width");
        return row * (R / 8) + (ch ^ (4 * ((row >> 1) & 1)));
    }
}

// Global -> registers for one BK-deep stage, zero-filling out-of-range chunks.
// KC: tile rows r0.. (< rmax), k in [k0, kmax); not KC: k rows k0.. (< kmax),
// contiguous rows r0.. (< rmax). kmax (KC) and rmax (not KC) are multiples of
// 8, so a 16-byte chunk is either wholly in bounds or wholly zero-filled.
template <int R, bool KC, int BK, int NT>
__device__ __forceinline__ void tile_gload(uint4 (&regs)[R * BK / (8 * NT)], const bf16_t* base,
                                           int64_t ld, int64_t r0, int64_t rmax, int k0, int kmax, int tid) {
    constexpr int CPR = TileCfg<R, KC, BK>::CPR;
#pragma unroll
    for (int i = 0; i < R * BK / (8 * NT); ++i) {
        const int c = tid + NT * i;
        uint4 v = make_uint4(0, 0, 0, 0);
        if constexpr (KC) {
            const int row = c / CPR;
            const int k = k0 + (c % CPR) * 8;
            const int64_t gr = r0 + row;
            if (gr < rmax && k < kmax) v = *(const uint4*)(base + gr * ld + k);
        } else {
            const int k = k0 + c / CPR;
            const int64_t gr = r0 + (c % CPR) * 8;
            if (k < kmax && gr < rmax) v = *(const uint4*)(base + (int64_t)k * ld + gr);
        }
        regs[i] = v;
    }
}

// Global -> registers for a whole BK-deep stage (no k bound); rows (KC) or
// column chunks (not KC) past rmax are clamped to valid memory, like the DMA
// path: their products land only in discarded outputs.
template <int R, bool KC, int BK, int NT>
__device__ __forceinline__ void tile_gload_full(uint4 (&regs)[R * BK / (8 * NT)], const bf16_t* base, int64_t ld,
                                                int64_t r0, int64_t rmax, int k0, int tid) {
    constexpr int CPR = TileCfg<R, KC, BK>::CPR;
#pragma unroll
    for (int i = 0; i < R * BK / (8 * NT); ++i) {
        const int c = tid + NT * i;
        if constexpr (KC) {
            const int64_t gr = min(r0 + c / CPR, rmax - 1);
            regs[i] = *(const uint4*)(base + gr * ld + k0 + (c % CPR) * 8);
        } else {
            const int64_t gc = min(r0 + (c % CPR) * 8, rmax - 8);
            regs[i] = *(const uint4*)(base + (int64_t)(k0 + c / CPR) * ld + gc);
        }
    }
}

template <int R, bool KC, int BK, int NT>
__device__ __forceinline__ void tile_sstore(char* lds, const uint4 (&regs)[R * BK / (8 * NT)], int tid) {
    constexpr int CPR = TileCfg<R, KC, BK>::CPR;
#pragma unroll
    for (int i = 0; i < R * BK / (8 * NT); ++i) {
        const int c = tid + NT * i;
        *(uint4*)(lds + 16 * slot_of<R, KC, BK>(c / CPR, c % CPR)) = regs[i];
    }
}

// Direct global -> LDS for whole 64-deep stages (gfx950 global_load_lds_dwordx4):
// each wave instruction fills 1 KB of LDS, lane i at +16 i, so every lane
// fetches the global chunk that belongs at its slot. The per-lane source
// pointers are computed once per tile and advanced by one stage per issue.
// Rows past rmax are clamped to valid memory (their products land only in
// discarded output rows or columns); a stage that would cross the end of K
// takes the register path instead, which zero-fills the tail.
template <int R, bool KC, int BK, int NW = 4>
struct DmaPlan {
    static constexpr int NI = TileCfg<R, KC, BK>::BYTES / (1024 * NW);  // 1 KB instructions per wave (NW waves)
    static_assert(NI * 1024 * NW == TileCfg<R, KC, BK>::BYTES, "stage must split evenly over the waves");
    static constexpr int CPR = TileCfg<R, KC, BK>::CPR;
    const bf16_t* src[NI];
    int64_t step;
    __device__ __forceinline__ void init(const bf16_t* base, int64_t ld, int64_t r0, int64_t rmax, int k0, int wave,
                                         int lane) {
        step = KC ? BK : (int64_t)BK * ld;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int slot = (wave * NI + i) * 64 + lane;
            const int row = slot / CPR;
            // the logical chunk whose swizzled position is this slot (XOR is an involution)
            const int ch = slot_of<R, KC, BK>(row, slot % CPR) - row * CPR;
            if constexpr (KC) {
                const int64_t gr = min(r0 + row, rmax - 1);
                src[i] = base + gr * ld + k0 + 8 * ch;
            } else {
                const int64_t gc = min(r0 + 8 * ch, rmax - 8);
                src[i] = base + (int64_t)(k0 + row) * ld + gc;
            }
        }
    }
    // load the current stage into `lds` and move to the next stage
    __device__ __forceinline__ void issue(char* lds, int wave) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
#if defined(__HIP_DEVICE_COMPILE__)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src[i],
                                             (G2_LDS void*)(lds + (wave * NI + i) * 1024), 16, 0, 0);
#endif
            src[i] += step;
        }
    }
    __device__ __forceinline__ void skip() {
#pragma unroll
        for (int i = 0; i < NI; ++i) src[i] += step;
    }
    // instruction i of the current stage (no advance; call skip() after all NI)
    __device__ __forceinline__ void issue_one(char* lds, int wave, int i) {
#if defined(__HIP_DEVICE_COMPILE__)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src[i],
                                         (G2_LDS void*)(lds + (wave * NI + i) * 1024), 16, 0, 0);
#endif
    }
};

// MFMA operand fragment: lane l holds rows rb + (l & 31), k = 16 kk + 8 (l >> 5) + 0..7.
template <int R, bool KC, int BK>
__device__ __forceinline__ bf16x8 tile_frag(const char* lds, int rb, int kk, int lane) {
    if constexpr (KC) {
        const int row = rb + (lane & 31);
        const int ch = kk * 2 + (lane >> 5);
        return *(const bf16x8*)(lds + 16 * slot_of<R, KC, BK>(row, ch));
    } else {
        // each 16-lane group reads a 4 (k) x 16 (rows) block; lane i of the group
        // receives the 4 k-values of row i
        const int g = lane >> 4, j = lane & 15;
        const int k = kk * 16 + 8 * (g >> 1) + (j >> 2);
        const int r = rb + 16 * (g & 1) + 4 * (j & 3);
        // rows k and k + 4 share the swizzle (it depends on k mod 4)
        const char* p0 = lds + 16 * slot_of<R, KC, BK>(k, r >> 3) + (r & 7) * 2;
        return lds_tr_pair(p0, 4 * TileCfg<R, KC, BK>::PITCH);
    }
}

// One BK-deep stage from LDS: BK/16 steps of 16, every wave multiplying its
// FM x FN grid of 32x32 fragments (a WM x WN block at (wm, wn)). With KS wave
// groups splitting the contraction, group ks takes steps ks, ks + KS, ... The
// fragments of the next step are read while the MFMAs of the current one run
// (two register sets), so each step waits only for its own LDS reads.
// `dma(d)` issues the d-th of the next stage's ND load instructions of this
// wave, spread evenly between the MFMAs (ND = 0: the caller issued them before)
template <int BM, int BN, bool AKC, bool BKC, int BK, int FM, int FN, int WM, int WN, int KS, int ND, class Dma>
__device__ __forceinline__ void mma_stage(const char* cur, f32x16 (&acc)[FM][FN], int wm, int wn, int ks,
                                          int lane, Dma&& dma) {
    constexpr int ABYTES = TileCfg<BM, AKC, BK>::BYTES;
    constexpr int KK = BK / 16 / KS;
    constexpr int NMF = KK * FM * FN;
    constexpr int EVERY = ND > 0 ? (NMF / ND > 0 ? NMF / ND : 1) : 1;
#if G2_GEMM_IGLP >= 0
    __builtin_amdgcn_iglp_opt(G2_GEMM_IGLP);
#endif
    bf16x8 af[2][FM], bv[2][FN];
    auto load = [&](int buf, int kk) {
#pragma unroll
        for (int i = 0; i < FM; ++i) af[buf][i] = tile_frag<BM, AKC, BK>(cur, wm * WM + i * 32, kk, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) bv[buf][j] = tile_frag<BN, BKC, BK>(cur + ABYTES, wn * WN + j * 32, kk, lane);
    };
    load(0, ks);
#if G2_GEMM_SCHED
    __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);  // DS reads of step 0
#endif
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) load((kk + 1) & 1, ks + (kk + 1) * KS);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1][i], bv[kk & 1][j], acc[i][j], 0, 0, 0);
                const int q = (kk * FM + i) * FN + j;  // constant after unrolling
                if (ND > 0 && q % EVERY == 0 && q / EVERY < ND) dma(q / EVERY);
            }
#if G2_GEMM_SCHED
        // Keep the next step's fragment reads ahead of this step's MFMAs. Left
        // alone, the scheduler sinks each read to just before its first use (to
        // shorten live ranges), which puts an LDS round trip in front of every
        // few MFMAs; pinned here, a read has a whole step of MFMAs to land.
        if (kk + 1 < KK) {
#if G2_GEMM_SCHED == 1
            __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);  // DS reads of step kk + 1
            __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);  // MFMAs of step kk
#else
            // one read after each MFMA
#pragma unroll
            for (int q = 0; q < FM * FN; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (q < FM + FN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
#endif
        } else {
            __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);  // MFMAs of the last step
        }
#endif
    }
    if constexpr (ND > 0) {
        // any instructions the spread did not reach
#pragma unroll
        for (int d = NMF / EVERY; d < ND; ++d) dma(d);
    }
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (vmcnt only; LDS and export counters untouched). Loads, including the LDS DMA
// loads, retire in issue order, so this waits for all but the newest N.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the stage ring. __syncthreads() (and any fence) makes
// the compiler drain every outstanding vector-memory operation first (vmcnt(0)),
// including the LDS DMA loads of later stages that must stay in flight across
// the barrier. Here each wave has already waited (wait_vmcnt) for its own share
// of the stage about to be read, so the barrier only needs the wave's LDS
// operations complete (lgkmcnt(0)); the empty asm statements keep the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

#ifndef G2_GEMM_GROUP
#define G2_GEMM_GROUP 8
#endif
// Output tile of this workgroup (1-D grid of nm x nn tiles per split). The
// dispatcher deals workgroups round-robin to the 8 XCDs, each with its own L2;
// when the tile count is a multiple of 8, XCD x takes the x-th contiguous
// eighth of the tile sequence, so the tiles resident on one XCD are neighbours.
// The sequence walks G row-panels at a time, column by column, so a wave of
// concurrent tiles covers a compact block and each A and B panel it needs is
// fetched into that L2 once.
__device__ __forceinline__ void tile_coords(int nm, int nn, int& tm, int& tn) {
    const int ntiles = nm * nn;
    int t = (int)blockIdx.x;
    constexpr int G = G2_GEMM_GROUP;
    if constexpr (G == 0) {  // plain row-major raster (experiments)
        tm = t / nn;
        tn = t - tm * nn;
        return;
    }
    if ((ntiles & 7) == 0) t = (t & 7) * (ntiles >> 3) + (t >> 3);
    const int per_group = G * nn;
    const int group = t / per_group;
    const int first = group * G;
    const int gsize = min(nm - first, G);
    const int r = t - group * per_group;
    tm = first + r % gsize;
    tn = r / gsize;
}

// Tile BM x BN, BK-deep stages in an NS-deep LDS ring. Waves form a WGM x WGN
// grid over the tile (each a WM x WN block of 32x32 fragments), times KS groups
// that split every stage's contraction steps; the KS partial sums are added
// through LDS before the epilogue.
// SPREAD: the next stage's loads are issued between the MFMAs instead of before them.
// REGLOAD: operands go global -> registers -> LDS (one stage ahead in
// registers, two LDS buffers) instead of by DMA.
template <int BM, int BN, int BK, bool AKC, bool BKC, int EPI, int NS, int WGM = 2, int WGN = 2, int KS = 1,
          bool SPREAD = false, bool REGLOAD = false>
__global__ __launch_bounds__(64 * WGM * WGN * KS) void gemm_bf16_kernel(GP p) {
    static_assert(NS >= 2 && NS <= 4, "pipeline depth");
    static_assert(KS == 1 || KS == 2, "contraction split");
    constexpr int NWQ = WGM * WGN;      // waves per group
    constexpr int NW = NWQ * KS;        // waves per workgroup
    constexpr int NT = 64 * NW;
    constexpr int ABYTES = TileCfg<BM, AKC, BK>::BYTES;
    constexpr int BBYTES = TileCfg<BN, BKC, BK>::BYTES;
    constexpr int STAGE = ABYTES + BBYTES;
    constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
    static_assert(FM * 32 == WM && FN * 32 == WN && (BK / 16) % KS == 0, "wave tiling");
    constexpr int SP = WN + 4;  // epilogue: staged floats per row (padding spreads banks)
    constexpr int EPI_BYTES = NWQ * 32 * SP * 4;
    constexpr int NSB = REGLOAD ? 2 : NS;  // LDS stage buffers
    constexpr int SMEM = NSB * STAGE > EPI_BYTES ? NSB * STAGE : EPI_BYTES;
    constexpr int DMA_OPS = DmaPlan<BM, AKC, BK, NW>::NI + DmaPlan<BN, BKC, BK, NW>::NI;  // per wave per stage
    __shared__ __attribute__((aligned(16))) char smem[SMEM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ks = wave / NWQ, wq = wave - ks * NWQ;
    const int wm = wq / WGN, wn = wq - (wq / WGN) * WGN;
    int tm, tn;
    tile_coords((p.M + BM - 1) / BM, (p.N + BN - 1) / BN, tm, tn);
    const int64_t m0 = (int64_t)tm * BM;
    const int n0 = tn * BN;
    const int kbeg = blockIdx.z * p.k_per_split;
    const int kend = min(p.K, kbeg + p.k_per_split);
    const int nk = (kend - kbeg + BK - 1) / BK;
    const bf16_t* A = (const bf16_t*)p.A;
    const bf16_t* B = (const bf16_t*)p.B;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // NS-deep ring of LDS stages: while stage t is multiplied out of LDS, the
    // next NS - 1 stages stream straight from global memory into their LDS
    // slots (no staging registers). A stage that would cross the end of K takes
    // the register path, which zero-fills the tail and completes before it
    // returns, so only whole stages are ever in flight.
    DmaPlan<BM, AKC, BK, NW> dA;
    DmaPlan<BN, BKC, BK, NW> dB;
    dA.init(A, p.lda, m0, p.M, kbeg, wave, lane);
    dB.init(B, p.ldb, n0, p.N, kbeg, wave, lane);
    auto issue = [&](char* buf, int kt) {
        const int k0 = kbeg + kt * BK;
        if (k0 + BK <= kend) {
            dA.issue(buf, wave);
            dB.issue(buf + ABYTES, wave);
        } else {
            uint4 ra[BM * BK / (8 * NT)], rb[BN * BK / (8 * NT)];
            tile_gload<BM, AKC, BK, NT>(ra, A, p.lda, m0, p.M, k0, kend, tid);
            tile_gload<BN, BKC, BK, NT>(rb, B, p.ldb, n0, p.N, k0, kend, tid);
            tile_sstore<BM, AKC, BK, NT>(buf, ra, tid);
            tile_sstore<BN, BKC, BK, NT>(buf + ABYTES, rb, tid);
            dA.skip();
            dB.skip();
        }
    };
    if constexpr (REGLOAD) {
        uint4 ra[BM * BK / (8 * NT)], rb[BN * BK / (8 * NT)];
        auto gload = [&](int kt) {
            const int k0 = kbeg + kt * BK;
            if (k0 + BK <= kend) {
                tile_gload_full<BM, AKC, BK, NT>(ra, A, p.lda, m0, p.M, k0, tid);
                tile_gload_full<BN, BKC, BK, NT>(rb, B, p.ldb, n0, p.N, k0, tid);
            } else {
                tile_gload<BM, AKC, BK, NT>(ra, A, p.lda, m0, p.M, k0, kend, tid);
                tile_gload<BN, BKC, BK, NT>(rb, B, p.ldb, n0, p.N, k0, kend, tid);
            }
        };
        auto sstore = [&](char* buf) {
            tile_sstore<BM, AKC, BK, NT>(buf, ra, tid);
            tile_sstore<BN, BKC, BK, NT>(buf + ABYTES, rb, tid);
        };
        if (nk > 0) {
            gload(0);
            sstore(smem);
        }
        if (nk > 1) gload(1);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            // registers hold stage kt+1; its LDS buffer was last read in
            // iteration kt-1, before the barrier that ended it
            if (kt + 1 < nk) sstore(smem + ((kt + 1) & 1) * STAGE);
            if (kt + 2 < nk) gload(kt + 2);
            mma_stage<BM, BN, AKC, BKC, BK, FM, FN, WM, WN, KS, 0>(smem + (kt & 1) * STAGE, acc, wm, wn, ks, lane,
                                                                   [](int) {});
            lds_barrier();  // stage kt+1 is in LDS; stage kt is free (loads in flight target registers)
        }
    } else {
    // stages [0, nfull) are whole BK-deep stages loaded by DMA
    const int nfull = (kend - kbeg) / BK;
#pragma unroll
    for (int t = 0; t < NS - 1; ++t)
        if (t < nk) issue(smem + t * STAGE, t);
    for (int kt = 0; kt < nk; ++kt) {
        // stage kt must have landed: the DMA stages issued after it may stay in flight
        const int newer = min(nk - 1, kt + NS - 2) - kt;        // stages issued after kt
        const int newer_dma = max(0, min(nfull - 1, kt + NS - 2) - kt);
        if (newer_dma == newer) {
            if constexpr (NS >= 4) {
                if (newer >= 2) wait_vmcnt<2 * DMA_OPS>();
                else if (newer == 1) wait_vmcnt<DMA_OPS>();
                else wait_vmcnt<0>();
            } else if constexpr (NS == 3) {
                if (newer >= 1) wait_vmcnt<DMA_OPS>();
                else wait_vmcnt<0>();
            } else {
                wait_vmcnt<0>();
            }
        } else {
            wait_vmcnt<0>();
        }
        lds_barrier();  // every wave's share of stage kt is in LDS; stage kt-1 is free
        const int knext = kt + NS - 1;
        char* nbuf = smem + (knext % NS) * STAGE;
        const bool spread = SPREAD && knext < nk && kbeg + knext * BK + BK <= kend;
        if (!spread && knext < nk) issue(nbuf, knext);
        constexpr int NIA = DmaPlan<BM, AKC, BK, NW>::NI, NIB = DmaPlan<BN, BKC, BK, NW>::NI;
        mma_stage<BM, BN, AKC, BKC, BK, FM, FN, WM, WN, KS, SPREAD ? NIA + NIB : 0>(
            smem + (kt % NS) * STAGE, acc, wm, wn, ks, lane, [&](int d) {
                if (!spread) return;
                if (d < NIA) dA.issue_one(nbuf, wave, d);
                else dB.issue_one(nbuf + ABYTES, wave, d - NIA);
            });
        if (spread) {
            dA.skip();
            dB.skip();
        }
    }
    }
    __syncthreads();  // the epilogue reuses the stage buffers
    // Epilogue: each wave of group 0 stages one 32-row strip of its block at a
    // time through LDS (reusing the main-loop buffers) so that lanes then own 8
    // consecutive columns of a row; with KS = 2, group 1 first leaves its partial
    // sums in the same slots and group 0 adds them in. Accumulator (i, j, r) of
    // lane l sits at row 8 (r/4) + 4 (l/32) + r%4 and column l%32 of fragment (i, j).
    // Every wave reaches every barrier.
    constexpr int LPR = WN / 8;                   // lanes per staged row
    constexpr int RPP = 64 / LPR;                 // rows per pass
    constexpr int NPASS = (32 + RPP - 1) / RPP;   // passes per 32-row strip
    float* st = (float*)smem + wq * 32 * SP;
    const int srow = 4 * (lane >> 5), scol = lane & 31;
    // GELU_BWD with column sums: each lane sums its 8 output columns over the
    // rows it writes; lanes holding the same columns are combined below
    constexpr bool CSUM = EPI == EPI_GELU_BWD && KS == 1 && WM == 64 && (LPR & (LPR - 1)) == 0 && RPP * LPR == 64;
    float csum[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) csum[k] = 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        if constexpr (KS > 1) {
            if (ks == 1) {
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        st[(8 * (r >> 2) + srow + (r & 3)) * SP + j * 32 + scol] = acc[i][j][r];
            }
            __syncthreads();
        }
        if (ks == 0) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float* q = st + (8 * (r >> 2) + srow + (r & 3)) * SP + j * 32 + scol;
                    *q = KS > 1 ? *q + acc[i][j][r] : acc[i][j][r];
                }
        }
        __syncthreads();
        if (ks == 0) {
#pragma unroll
            for (int pass = 0; pass < NPASS; ++pass) {
                const int rr = pass * RPP + lane / LPR;
                const int cc = (lane % LPR) * 8;
                if (lane < RPP * LPR && rr < 32) {  // WN = 96 leaves lanes 60..63 idle
                    float v[8], o[8];
                    ld8f(st + rr * SP + cc, v);
                    const int64_t m = m0 + wm * WM + i * 32 + rr;
                    const int n = n0 + wn * WN + cc;
                    if (m < p.M && n < p.N) {
                        epi_apply8<EPI>(p, m, n, v, o);
                        if constexpr (CSUM) {
#pragma unroll
                            for (int k = 0; k < 8; ++k) csum[k] += o[k];
                        }
                    }
                }
            }
        }
        __syncthreads();
    }
    if constexpr (CSUM) {
        if (p.cpart && ks == 0) {
            // lanes l, l + LPR, l + 2 LPR, ... hold the same 8 columns
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
                for (int k = 0; k < 8; ++k) csum[k] += __shfl_xor(csum[k], off, 64);
            const int n = n0 + wn * WN + lane * 8;
            // one partial row per 64-row block that starts inside the matrix
            if (lane < LPR && n < p.N && m0 + wm * WM < p.M) {
                float* dst = p.cpart + ((m0 + wm * WM) / 64) * p.N + n;
                st8f(dst, csum);
            }
        }
    }
}

// ------------------------------------------------------------------ fp32 kernel
template <bool AKC, bool BKC, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GP p) {
    __shared__ float As[16][64 + 4];
    __shared__ float Bs[16][64 + 4];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int64_t m0 = (int64_t)blockIdx.y * 64;
    const int n0 = blockIdx.x * 64;
    const int kbeg = blockIdx.z * p.k_per_split;
    const int kend = min(p.K, kbeg + p.k_per_split);
    const float* A = (const float*)p.A;
    const float* B = (const float*)p.B;
    float acc[4][4] = {};
    for (int k0 = kbeg; k0 < kend; k0 += 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + 256 * i;
            int mm, kk;
            if (AKC) { mm = e >> 4; kk = e & 15; } else { kk = e >> 6; mm = e & 63; }
            const int64_t gm = m0 + mm;
            const int gk = k0 + kk;
            float v = 0.0f;
            if (gm < p.M && gk < kend) v = AKC ? A[gm * p.lda + gk] : A[(int64_t)gk * p.lda + gm];
            As[kk][mm] = v;
            int nn;
            if (BKC) { nn = e >> 4; kk = e & 15; } else { kk = e >> 6; nn = e & 63; }
            const int gn = n0 + nn;
            const int gk2 = k0 + kk;
            float w = 0.0f;
            if (gn < p.N && gk2 < kend) w = BKC ? B[(int64_t)gn * p.ldb + gk2] : B[(int64_t)gk2 * p.ldb + gn];
            Bs[kk][nn] = w;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t m = m0 + ty * 4 + i;
            const int n = n0 + tx * 4 + j;
            if (m < p.M && n < p.N) epi_apply<EPI, float>(p, m, n, acc[i][j]);
        }
}

// ------------------------------------------------------------------ skinny products
// Y = X W^T with at most kSkinnyRows rows of X, both contraction-contiguous
// (generation runs one position of a few sequences at a time). Tiles of 128+
// rows would leave all but a few CUs idle; here every wave owns one output
// column n, streams row n of W once with 16-byte loads (8 bf16 or 4 fp32 per
// lane), and keeps one partial sum per row of X, whose rows come through LDS in
// kSkinnyChunk-wide pieces of the contraction. A wave reduction leaves the M
// sums of column n; the tiled kernel's epilogues finish them. Summation order is
// fixed. (Reading X straight from the caches instead, several columns per wave,
// measured slower.) Every workgroup stages the whole X chunk, so a workgroup of
// eight waves (eight columns) stages it half as often as one of four: 11.9k
// against 11.0k generated tokens per second at 12 sequences (16 waves: 11.8k).
constexpr int kSkinnyRows = 16;
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyChunk = 1024;

template <int E>
__device__ __forceinline__ void skinny_unpack(uint4 v, float (&o)[E]) {
    if constexpr (E == 8) {
        unpack8(v, o);
    } else {
        o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
        o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
    }
}

// LNX: X is the fp32 residual stream and the product's operand is its
// LayerNorm (gain p.ln_g, bias p.ln_b, epsilon p.ln_eps, biased variance, the
// same two-pass statistics as the LayerNorm kernel), formed while staging; the
// contraction then fits one chunk (K <= kSkinnyChunk).
template <int EPI, class T, bool LNX>
__global__ __launch_bounds__(64 * kSkinnyWaves) void gemm_skinny_kernel(GP p) {
    constexpr int E = 16 / sizeof(T);  // elements per 16-byte load
    __shared__ __attribute__((aligned(16))) T xs[kSkinnyRows * kSkinnyChunk];
    const int M = (int)p.M, K = p.K, N = p.N;
    const T* W = (const T*)p.B;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = blockIdx.x * kSkinnyWaves + wave;
    const T* wr = W + (int64_t)min(n, N - 1) * p.ldb;
    float acc[kSkinnyRows];
#pragma unroll
    for (int m = 0; m < kSkinnyRows; ++m) acc[m] = 0.0f;
    // Loads are issued all together before their results are used (the weight
    // row's piece first, then every 16-byte piece of X this thread stages), so a
    // chunk costs about one memory round trip rather than one per piece.
    constexpr int NWR = kSkinnyChunk / (64 * E);                               // weight pieces per lane
    constexpr int NXR = kSkinnyRows * kSkinnyChunk / (64 * kSkinnyWaves * E);  // X pieces per thread
    for (int kc = 0; kc < K; kc += kSkinnyChunk) {
        const int kn = min(kSkinnyChunk, K - kc);
        uint4 wv[NWR];
#pragma unroll
        for (int r = 0; r < NWR; ++r) {
            const int k = (lane + 64 * r) * E;
            wv[r] = k < kn ? *(const uint4*)(wr + kc + k) : make_uint4(0, 0, 0, 0);
        }
        if constexpr (LNX) {
            // wave w normalises rows w, w + kSkinnyWaves, ...: every row's float4
            // pieces are loaded up front (one round trip), then mean, variance
            // about it and the normalised row come from registers
            constexpr int RPW = kSkinnyRows / kSkinnyWaves;  // rows per wave
            constexpr int NJ = kSkinnyChunk / 256;           // float4 pieces per lane per row
            const float4* Xf = (const float4*)p.A;
            const int K4 = K / 4;
            float4 v[RPW][NJ];
#pragma unroll
            for (int ri = 0; ri < RPW; ++ri) {
                const int m = wave + kSkinnyWaves * ri;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int c4 = lane + 64 * j;
                    v[ri][j] = m < M && c4 < K4 ? Xf[(int64_t)m * (p.lda / 4) + c4] : make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
#pragma unroll
            for (int ri = 0; ri < RPW; ++ri) {
                const int m = wave + kSkinnyWaves * ri;
                if (m >= M) continue;  // uniform across the wave
                float sum = 0.0f;
#pragma unroll
                for (int j = 0; j < NJ; ++j) sum += (v[ri][j].x + v[ri][j].y) + (v[ri][j].z + v[ri][j].w);
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
                const float mu = sum / (float)K;
                float q = 0.0f;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    if (lane + 64 * j < K4) {
                        const float a = v[ri][j].x - mu, b = v[ri][j].y - mu, c = v[ri][j].z - mu, d = v[ri][j].w - mu;
                        q += (a * a + b * b) + (c * c + d * d);
                    }
                }
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) q += __shfl_xor(q, off, 64);
                const float rs = 1.0f / sqrtf(q / (float)K + p.ln_eps);
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int c4 = lane + 64 * j;
                    if (c4 < K4) {
                        const float4 gg = ((const float4*)p.ln_g)[c4], bb = ((const float4*)p.ln_b)[c4];
                        const int o = m * kSkinnyChunk + 4 * c4;
                        Act<T>::st(xs, o + 0, (v[ri][j].x - mu) * rs * gg.x + bb.x);
                        Act<T>::st(xs, o + 1, (v[ri][j].y - mu) * rs * gg.y + bb.y);
                        Act<T>::st(xs, o + 2, (v[ri][j].z - mu) * rs * gg.z + bb.z);
                        Act<T>::st(xs, o + 3, (v[ri][j].w - mu) * rs * gg.w + bb.w);
                    }
                }
            }
            __syncthreads();
        } else {
            const T* X = (const T*)p.A;
            uint4 xv[NXR];
#pragma unroll
            for (int r = 0; r < NXR; ++r) {
                const int i = (threadIdx.x + 64 * kSkinnyWaves * r) * E;
                xv[r] = make_uint4(0, 0, 0, 0);
                if (i < M * kn) {
                    const int m = i / kn, k = i - m * kn;  // kn is a multiple of E
                    xv[r] = *(const uint4*)(X + (int64_t)m * p.lda + kc + k);
                }
            }
            __syncthreads();  // the previous chunk is no longer read
#pragma unroll
            for (int r = 0; r < NXR; ++r) {
                const int i = (threadIdx.x + 64 * kSkinnyWaves * r) * E;
                if (i < M * kn) {
                    const int m = i / kn, k = i - m * kn;
                    *(uint4*)(xs + m * kSkinnyChunk + k) = xv[r];
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int r = 0; r < NWR; ++r) {
            const int k = (lane + 64 * r) * E;
            if (k < kn) {
                float w[E];
                skinny_unpack<E>(wv[r], w);
#pragma unroll
                for (int m = 0; m < kSkinnyRows; ++m) {
                    if (m < M) {
                        float xx[E];
                        skinny_unpack<E>(*(const uint4*)(xs + m * kSkinnyChunk + k), xx);
#pragma unroll
                        for (int e = 0; e < E; ++e) acc[m] = fmaf(w[e], xx[e], acc[m]);
                    }
                }
            }
        }
    }
    // every lane ends with the column's M sums; lane m finishes row m
    float v = 0.0f;
#pragma unroll
    for (int m = 0; m < kSkinnyRows; ++m) {
        if (m < M) {
            float a = acc[m];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) a += __shfl_xor(a, off, 64);
            if (lane == m) v = a;
        }
    }
    if (n < N && lane < M) epi_apply<EPI, T>(p, lane, n, v);
}

template <int EPI, bool LNX>
static hipError_t launch_skinny(int dtype, const GP& p, hipStream_t s) {
    const dim3 grid((unsigned)((p.N + kSkinnyWaves - 1) / kSkinnyWaves));
    if (dtype == GPT2_DTYPE_BF16)
        hipLaunchKernelGGL((gemm_skinny_kernel<EPI, bf16_t, LNX>), grid, dim3(64 * kSkinnyWaves), 0, s, p);
    else
        hipLaunchKernelGGL((gemm_skinny_kernel<EPI, float, LNX>), grid, dim3(64 * kSkinnyWaves), 0, s, p);
    return hipGetLastError();
}

// forward products the skinny kernel takes: few rows, 16-byte aligned rows of X and W
static bool skinny_ok(int dtype, const GemmArgs& a) {
    const int E = dtype == GPT2_DTYPE_BF16 ? 8 : 4;
    const int eb = dtype == GPT2_DTYPE_BF16 ? 2 : 4;
    // (vocabulary-wide outputs keep the tiled kernel, measured faster there)
    return a.M <= kSkinnyRows && a.N < 8192 && a.K > 0 && a.K % E == 0 && a.lda % E == 0 && a.ldb % E == 0 &&
           ((uintptr_t)a.A % 16) == 0 && ((uintptr_t)a.B % 16) == 0 && (a.epi == EPI_STORE || a.epi == EPI_GELU ||
           a.epi == EPI_RESID || a.epi == EPI_F32) && eb > 0;
}

// ------------------------------------------------------------------ split-K reduction
// out[i] = sum_s part[s][i] (in s order) (+ out[i] if accumulate)
__global__ void splitk_reduce_kernel(const float* part, int splits, int64_t n, float* out, int64_t rows,
                                     int cols, int64_t ldo, int accumulate) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float s = 0.0f;
    for (int k = 0; k < splits; ++k) s += part[(int64_t)k * n + i];
    const int64_t r = i / cols;
    const int c = (int)(i % cols);
    float* o = out + r * ldo + c;
    *o = accumulate ? *o + s : s;
    (void)rows;
}

// float4 form (cols and ldo multiples of 4)
__global__ void splitk_reduce4_kernel(const float* part, int splits, int64_t n, float* out, int cols, int64_t ldo,
                                      int accumulate) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i >= n) return;
    float4 s = *(const float4*)(part + i);
    for (int k = 1; k < splits; ++k) {
        const float4 v = *(const float4*)(part + (int64_t)k * n + i);
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    const int64_t r = i / cols;
    const int c = (int)(i - r * cols);
    float4* o = (float4*)(out + r * ldo + c);
    if (accumulate) {
        const float4 q = *o;
        s.x += q.x; s.y += q.y; s.z += q.z; s.w += q.w;
    }
    *o = s;
}

// ------------------------------------------------------------------ launchers
#ifndef G2_GEMM_NS
#define G2_GEMM_NS 2
#endif
template <int BM, int BN, bool AKC, bool BKC, int EPI, int BK = 64, int NS = G2_GEMM_NS, int WGM = 2, int WGN = 2,
          int KS = 1, bool SPREAD = false, bool REGLOAD = false>
static hipError_t launch_bf16(const GP& p, int splits, hipStream_t s) {
    const int64_t tiles = (int64_t)((p.N + BN - 1) / BN) * ((p.M + BM - 1) / BM);
    if (tiles > INT32_MAX) return hipErrorInvalidValue;
    dim3 grid((unsigned)tiles, 1, splits);
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, AKC, BKC, EPI, NS, WGM, WGN, KS, SPREAD, REGLOAD>), grid,
                       dim3(64 * WGM * WGN * KS), 0, s, p);
    return hipGetLastError();
}

template <bool AKC, bool BKC, int EPI>
static hipError_t pick_tile_bf16(const GP& p, int splits, hipStream_t s) {
#if defined(G2_FORCE_TILE)  // tile experiments only: one configuration for every product
#if G2_FORCE_TILE == 40
    return launch_bf16<128, 128, AKC, BKC, EPI, AKC ? 32 : 64>(p, splits, s);
#elif G2_FORCE_TILE == 41
    return launch_bf16<192, 192, AKC, BKC, EPI, 64, 2, 2, 2, 2>(p, splits, s);
#elif G2_FORCE_TILE == 42
    return launch_bf16<256, 256, AKC, BKC, EPI, 64, 2, 2, 4, 1>(p, splits, s);
#elif G2_FORCE_TILE == 43
    return launch_bf16<128, 128, AKC, BKC, EPI, AKC ? 32 : 64, 2, 2, 2, 1, false, true>(p, splits, s);
#elif G2_FORCE_TILE == 44
    return launch_bf16<192, 192, AKC, BKC, EPI, 64, 2, 2, 2, 2, false, true>(p, splits, s);
#elif G2_FORCE_TILE == 45
    return launch_bf16<256, 256, AKC, BKC, EPI, 64, 2, 2, 4, 1, false, true>(p, splits, s);
#endif
#endif
    // Tile policy from per-product timings inside the 124M training step (M = 12288
    // tokens; each of the six configurations forced on every product in turn):
    //  - weight gradients (both operands transposed, K = tokens): operands staged
    //    through registers; 256 x 256 tiles for the vocabulary-wide one (unsplit),
    //    128 x 128 with split-K for the others;
    //  - input gradients (B transposed) onto at most 1536 columns that split into
    //    192-wide tiles: 192 x 192, eight waves in two groups splitting each stage's
    //    k-steps, operands staged through registers; the GELU-derivative product,
    //    whose epilogue takes per-64-row column sums, keeps 128 x 128;
    //  - forward products: 256 x 256 (eight waves, DMA) for the vocabulary-wide
    //    one; 128 x 128 with 64-deep stages and eight waves (32 x 64 each) for
    //    short contractions onto 2048..8191 columns; 192 x 192 (DMA) for long
    //    contractions onto <= 1536 columns; else 128 x 128, operands streamed
    //    global -> LDS by DMA (32-deep stages). A 64-deep stage reads whole
    //    128-byte rows: L2 serves half-line (64-byte) row reads at about half
    //    the rate of whole lines.
    if constexpr (!AKC) {
        if (!BKC && p.M >= 8192 && splits == 1 && p.K % 64 == 0)
            return launch_bf16<256, 256, AKC, BKC, EPI, 64, 2, 2, 4, 1, false, true>(p, splits, s);
        return launch_bf16<128, 128, AKC, BKC, EPI, 64, 2, 2, 2, 1, false, true>(p, splits, s);
    } else if constexpr (!BKC) {
        if constexpr (EPI == EPI_GELU_BWD)
            if (p.cpart) return launch_bf16<128, 128, AKC, BKC, EPI, 32>(p, splits, s);
        if (p.N % 192 == 0 && p.N <= 1536 && splits == 1)
            return launch_bf16<192, 192, AKC, BKC, EPI, 64, 2, 2, 2, 2, false, true>(p, splits, s);
        return launch_bf16<128, 128, AKC, BKC, EPI, 32>(p, splits, s);
    } else {
        if (p.N >= 2048 && p.N < 8192 && p.K <= 1024 && p.K % 64 == 0)
            return launch_bf16<128, 128, AKC, BKC, EPI, 64, 2, 4, 2, 1>(p, splits, s);
        if (p.N >= 8192) return launch_bf16<256, 256, AKC, BKC, EPI, 64, 2, 2, 4, 1>(p, splits, s);
        if (p.N % 192 == 0 && p.N <= 1536 && p.K >= 2048 && splits == 1)
            return launch_bf16<192, 192, AKC, BKC, EPI, 64, 2, 2, 2, 2>(p, splits, s);
        return launch_bf16<128, 128, AKC, BKC, EPI, 32>(p, splits, s);
    }
}

template <bool AKC, bool BKC, int EPI>
static hipError_t launch_f32(const GP& p, int splits, hipStream_t s) {
    dim3 grid((p.N + 63) / 64, (unsigned)((p.M + 63) / 64), splits);
    hipLaunchKernelGGL((gemm_f32_kernel<AKC, BKC, EPI>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

template <bool AKC, bool BKC, int EPI>
static hipError_t dispatch(int dtype, const GP& p, int splits, hipStream_t s) {
    if (dtype == GPT2_DTYPE_BF16) return pick_tile_bf16<AKC, BKC, EPI>(p, splits, s);
    return launch_f32<AKC, BKC, EPI>(p, splits, s);
}

#ifndef G2_WG_BIG
#define G2_WG_BIG 1
#endif
// 256 x 256 weight-gradient tiles (one workgroup per CU, half the operand
// traffic per FLOP of 128 x 128) for outputs of at least 2304 x 768; smaller
// outputs would need so many splits that the partial sums cost more than the
// larger tile saves.
static bool wgrad_big_tile(const GemmArgs& a) {
    if (!G2_WG_BIG) return false;
    return a.M % 256 == 0 && a.N % 256 == 0 && a.M * a.N >= (int64_t)2304 * 768;
}

// Weight gradient (both operands with the contraction index strided) over
// BM x BN register-staged tiles. `slots` is how many such workgroups should run
// at once; the contraction is split into as many 64-aligned pieces as
// fill them (at least MINK deep each, and within the partial-sum buffer), each
// piece writes its own fp32 partial, and one launch sums the partials in split
// order into dW (adding to it when accumulating).
template <int BM, int BN, int WGM, int WGN, int MINK>
static hipError_t wgrad_split(const GemmArgs& a, const GP& p, int slots, hipStream_t s) {
    const int64_t tiles = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    int splits = 1;
    if (tiles < slots) {
        splits = (int)std::min<int64_t>(std::max<int64_t>(1, slots / tiles), a.K / MINK);
        while (splits > 1 && (size_t)splits * a.M * a.N * 4 > a.split_bytes) --splits;
    }
    if (splits <= 1) return pick_tile_bf16<false, false, EPI_F32>(p, 1, s);
    int kps = (int)(((a.K + splits - 1) / splits + 63) / 64 * 64);
    splits = (a.K + kps - 1) / kps;
    GP q = p;
    q.k_per_split = kps;
    q.C = a.split_buf;
    q.ldc = a.N;
    q.c_split_stride = (int64_t)a.M * a.N;
    q.accumulate = 0;
    hipError_t e = launch_bf16<BM, BN, false, false, EPI_F32, 64, 2, WGM, WGN, 1, false, true>(q, splits, s);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)a.M * a.N;
    if (a.N % 4 == 0 && a.ldc % 4 == 0 && ((uintptr_t)a.C & 15) == 0)
        hipLaunchKernelGGL(splitk_reduce4_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s,
                           (const float*)a.split_buf, splits, n, (float*)a.C, a.N, a.ldc, a.accumulate);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           (const float*)a.split_buf, splits, n, (float*)a.C, a.M, a.N, a.ldc, a.accumulate);
    return hipGetLastError();
}

hipError_t gemm(int dtype, const GemmArgs& a, hipStream_t s) {
    GP p;
    p.A = a.A; p.B = a.B; p.lda = a.lda; p.ldb = a.ldb;
    p.M = a.M; p.N = a.N; p.K = a.K;
    p.k_per_split = a.K;
    p.alpha = a.alpha; p.bias = a.bias;
    p.C = a.C; p.ldc = a.ldc; p.c_split_stride = 0;
    p.C2 = a.C2; p.ldc2 = a.ldc2; p.R = a.R; p.ldr = a.ldr;
    p.accumulate = a.accumulate;
    p.gelu_erf = a.gelu_erf;
    p.cpart = a.epi == EPI_GELU_BWD ? a.colsum_part : nullptr;
    p.ln_g = a.ln_g;
    p.ln_b = a.ln_b;
    p.ln_eps = a.ln_eps;
    p.dmask = a.epi == EPI_RESID ? a.dmask : nullptr;
    p.dscale = a.dscale;
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    if (a.K <= 0) {
        // empty contraction: the product is zero
        if (a.epi != EPI_F32) return hipErrorInvalidValue;
        p.K = 0;
    }
    const bool kc11 = a.a_kc && a.b_kc, kc10 = a.a_kc && !a.b_kc, kc00 = !a.a_kc && !a.b_kc;
    if (a.ln_g) {
        // LayerNorm folded into a skinny product only (fp32 A rows, one chunk)
        if (!kc11 || !a.ln_b || a.K > kSkinnyChunk || !skinny_ok(GPT2_DTYPE_F32, a) || (a.K % 8) != 0)
            return hipErrorInvalidValue;
        switch (a.epi) {
            case EPI_STORE: return launch_skinny<EPI_STORE, true>(dtype, p, s);
            case EPI_GELU: return launch_skinny<EPI_GELU, true>(dtype, p, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (kc11 && skinny_ok(dtype, a)) {
        switch (a.epi) {
            case EPI_STORE: return launch_skinny<EPI_STORE, false>(dtype, p, s);
            case EPI_GELU: return launch_skinny<EPI_GELU, false>(dtype, p, s);
            case EPI_RESID: return launch_skinny<EPI_RESID, false>(dtype, p, s);
            case EPI_F32: return launch_skinny<EPI_F32, false>(dtype, p, s);
        }
    }
    if (kc11) {
        switch (a.epi) {
            case EPI_STORE: return dispatch<true, true, EPI_STORE>(dtype, p, 1, s);
            case EPI_GELU: return dispatch<true, true, EPI_GELU>(dtype, p, 1, s);
            case EPI_RESID: return dispatch<true, true, EPI_RESID>(dtype, p, 1, s);
            case EPI_F32: return dispatch<true, true, EPI_F32>(dtype, p, 1, s);
        }
    } else if (kc10) {
        switch (a.epi) {
            case EPI_STORE: return dispatch<true, false, EPI_STORE>(dtype, p, 1, s);
            case EPI_F32: return dispatch<true, false, EPI_F32>(dtype, p, 1, s);
            case EPI_GELU_BWD: return dispatch<true, false, EPI_GELU_BWD>(dtype, p, 1, s);
        }
    } else if (kc00 && a.epi == EPI_F32) {
        // weight gradients: contraction over all tokens; split K when the output
        // alone would not fill the GPU, reducing the partials in fixed order
        if (dtype != GPT2_DTYPE_BF16 || !a.split_buf || a.K < 1024) return dispatch<false, false, EPI_F32>(dtype, p, 1, s);
        // The training step runs weight gradients on a stream of their own beside
        // the backward's input-gradient chain, so they are split to fill about
        // half the GPU (128 CUs' worth of workgroups), not all of it: fewer
        // partial sums to write and reduce, and the step measured fastest there
        // (splitting for 256 CUs was 0.5 ms slower per step, for 96 CUs 1.4 ms).
        constexpr int kSlots = 128;
        if (wgrad_big_tile(a)) return wgrad_split<256, 256, 2, 4, 1024>(a, p, kSlots, s);
        return wgrad_split<128, 128, 2, 2, 512>(a, p, 2 * kSlots, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace g2
