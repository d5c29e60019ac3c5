// Causal flash attention for head size 64 on bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Forward (one workgroup = 128 queries of one (batch, head), 4 waves x 32
// queries; K/V tiles of 64 keys double-buffered in LDS): the scores are formed
// transposed, S^T = K Q^T, so each lane owns one query row and 16 of its key
// columns; the online softmax (running max and sum, base-2 exponent with the
// 1/sqrt(d) scale folded in) needs one cross-lane exchange per tile. The
// probabilities go straight from the accumulators into the next MFMA as the
// B operand of O^T += V^T P^T; the key order inside each 16-key step is the
// accumulator's row order, matched on the V side by the gfx950 LDS transpose
// load (ds_read_b64_tr_b16). Saves lse = max + log(sum) per query.
//
// Backward (P recomputed from lse): D_i = dO_i . O_i; a dQ kernel with the
// forward's structure (S^T, dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T +=
// K^T dS^T) and a dK/dV kernel owning 128 keys per workgroup that walks query
// tiles of 64 (S = Q K^T, dP = dO V^T, dV += P^T dO, dK += dS^T Q). No atomics:
// every output element is written by exactly one lane, so results are
// deterministic.
//
// Dropout (training mode, DROP): the keep bits of the attention weights are
// read from a mask written beforehand (one 64-bit word per query row and
// 64-key tile). The forward weights v_j by P_ij keep_ij and scales O by
// 1 / (1 - p) at the end, the sum l stays that of P, so lse is unchanged; the
// backward uses W = P keep / (1 - p) for dV and dP_ij = keep_ij / (1 - p)
// dO_i . v_j for dS = P (dP - D), where D = dO . O with the dropped O.
//
// LDS tiles are [rows][64] bf16 (128 B per row) with the 16-byte chunk index
// XOR-ed by a bit-reversal of (row / 2) mod 8: conflict-free both for 128-bit
// row reads (MFMA operands with the contraction index along the row) and for
// transpose reads (contraction index down the rows).
#include <cmath>
#include <type_traits>

#include "device.h"

namespace g2 {

hipError_t attention_fwd_simple(int dtype, int B, int Tn, int C, int H, const void* qkv, void* out, float* lse,
                                hipStream_t s, const uint64_t* dmask, float dscale);
hipError_t attention_bwd_simple(int dtype, int B, int Tn, int C, int H, const void* qkv, const void* out,
                                const float* lse, const void* dout, void* dqkv, float* Dbuf, hipStream_t s,
                                const uint64_t* dmask, float dscale);

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTileBytes = 64 * 128;  // 64 rows x 64 bf16

__device__ __forceinline__ int swz(int row) {
    const int x = (row >> 1) & 7;
    return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1);
}
__device__ __forceinline__ int toff(int row, int col) {
    return row * 128 + ((((col >> 3) ^ swz(row))) << 4) + ((col & 7) << 1);
}

// 64 rows (r0.., < rmax zero-filled) x 64 columns of a row-major bf16 matrix,
// two 16-byte chunks per thread (256 threads)
struct TileRegs {
    uint4 v[2];
};
__device__ __forceinline__ void tile_load(TileRegs& t, const bf16_t* g, int64_t ld, int r0, int rmax, int tid) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i;
        const int row = c >> 3, ch = c & 7;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r0 + row < rmax) v = *(const uint4*)(g + (int64_t)(r0 + row) * ld + ch * 8);
        t.v[i] = v;
    }
}
__device__ __forceinline__ void tile_store(char* lds, const TileRegs& t, int tid) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i;
        const int row = c >> 3, ch = c & 7;
        *(uint4*)(lds + row * 128 + ((ch ^ swz(row)) << 4)) = t.v[i];
    }
}

// 64 x 64 bf16 tile streamed straight into LDS (gfx950 global_load_lds_dwordx4):
// wave w fills rows 16 w .. 16 w + 15 with two 1 KB instructions; lane l of
// instruction i lands at row 16 w + 8 i + l / 8, slot l % 8, so it fetches the
// chunk that the swizzle places there. Rows past the end are clamped to the
// last row (finite data; every consumer masks those keys or queries).
struct TileDma {
    int roff[2];  // tile row of this lane's chunk in each instruction
    int coff[2];  // element offset of the chunk within the row
    __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = 16 * w + 8 * i + (lane >> 3);
            roff[i] = row;
            coff[i] = ((lane & 7) ^ swz(row)) * 8;
        }
    }
    __device__ __forceinline__ void issue(char* lds, const bf16_t* g, int64_t ld, int r0, int rmax, int w) const {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const bf16_t* src = g + (int64_t)min(r0 + roff[i], rmax - 1) * ld + coff[i];
#if defined(__HIP_DEVICE_COMPILE__)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                             (G2_LDS void*)(lds + (2 * w + i) * 1024), 16, 0, 0);
#endif
        }
    }
};

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void att_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// keep words of one 64-key tile for the 32 query rows of wave w, streamed into
// LDS like the K/V tiles (one 4-byte global_load_lds per wave: lane l fetches
// half l % 2 of row l / 2's word), so they ride in the same vmcnt-ordered
// stream as the tiles. dst: the ring slot's 128 words; rows past T read row T - 1.
__device__ __forceinline__ void mask_dma(uint64_t* dst, const uint64_t* rows, int Tw, int kt, int r0, int T, int w,
                                         int lane) {
    const int row = min(r0 + 32 * w + (lane >> 1), T - 1);
    const uint32_t* src = (const uint32_t*)(rows + (int64_t)row * Tw + kt) + (lane & 1);
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (G2_LDS void*)(dst + 32 * w), 4, 0, 0);
#endif
}

// workgroup barrier ordering LDS only (a __syncthreads() would also drain the
// DMA loads still in flight for later tiles)
__device__ __forceinline__ void att_lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// operand with the contraction index along the tile row: lane l holds row
// rbase + (l & 31), columns 16 kk + 8 (l >> 5) + 0..7
__device__ __forceinline__ bf16x8 frag_row(const char* lds, int rbase, int kk, int lane) {
    const int row = rbase + (lane & 31);
    const int ch = kk * 2 + (lane >> 5);
    return *(const bf16x8*)(lds + row * 128 + ((ch ^ swz(row)) << 4));
}

// operand with the contraction index down the tile rows: lane l holds column
// cbase + (l & 31), rows kbase + 4 (l >> 5) + {0..3} and kbase + 8 + 4 (l >> 5) + {0..3}
__device__ __forceinline__ bf16x8 frag_col(const char* lds, int kbase, int cbase, int lane) {
    const int G = lane >> 4, j = lane & 15;
    const int row = kbase + 4 * (G >> 1) + (j >> 2);
    const int col = cbase + 16 * (G & 1) + 4 * (j & 3);
    return lds_tr2(lds + toff(row, col), lds + toff(row + 8, col));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.0f;
    return z;
}

__device__ __forceinline__ bf16x8 load8(const bf16_t* p, bool ok) {
    if (!ok) {
        bf16x8 z;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.0f;
        return z;
    }
    return *(const bf16x8*)p;
}

// 2^x on the hardware exp unit; every argument here is <= 0 (scores minus their
// running maximum), where flushing a denormal result to zero is harmless
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// accumulator register r of lane l sits at row 8 (r/4) + 4 (l/32) + r%4
__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// 1-D grid over (128-row block, head, batch), ordered by decreasing causal work:
// query blocks from the last (longest rows) down, key blocks from the first
// (most query tiles) up, so the dispatcher schedules longest jobs first. When
// H B is a multiple of 8, all blocks of one (batch, head) share blockIdx mod 8,
// which keeps them on one XCD and its L2.
__device__ __forceinline__ void block_coords(int T, int H, bool late_first, int& blk, int& h, int& b) {
    const int nblk = (T + 127) / 128;
    const int hb_n = (int)gridDim.x / nblk;  // H * B
    const int bid = (int)blockIdx.x;
    const int rank = bid / hb_n, hb = bid - rank * hb_n;
    blk = late_first ? nblk - 1 - rank : rank;
    h = hb % H;
    b = hb / H;
}

}  // namespace

// ------------------------------------------------------------------ forward
// Lazy rescaling: the running maximum m (scaled, base 2) only moves when some
// lane's tile maximum exceeds it by more than kLazy; otherwise the stale m is
// kept and probabilities may reach 2^kLazy. O and l use the same m throughout,
// so the final O / l and lse = m + log2(l) are exact up to rounding.
constexpr float kLazy = 8.0f;

#ifndef G2_ATT_FWD_OCC
#define G2_ATT_FWD_OCC 3
#endif
// three workgroups (waves per SIMD) per CU: registers capped at 168. K/V tiles
// stream into a three-deep LDS ring (48 KB) by DMA, two tiles ahead.
// (with dropout: two per CU, the keep bits' registers do not fit in 168)
template <bool DROP>
__global__ __launch_bounds__(256, DROP ? 2 : G2_ATT_FWD_OCC) void attn_fwd_d64(const bf16_t* qkv, bf16_t* out, float* lse, int T,
                                                                    int C, int H, float sl2, const uint64_t* dmask,
                                                                    int Tw, float dscale) {
    __shared__ __attribute__((aligned(16))) char smem[3][2][kTileBytes];
    __shared__ __attribute__((aligned(16))) uint64_t smask[DROP ? 3 : 1][128];  // keep words per query row
    int qb, h, b;
    block_coords(T, H, true, qb, h, b);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5;
    const int64_t rs = 3 * (int64_t)C;
    const bf16_t* base = qkv + (int64_t)b * T * rs;
    const bf16_t* Qg = base + h * 64;
    const bf16_t* Kg = base + C + h * 64;
    const bf16_t* Vg = base + 2 * C + h * 64;
    const int q0 = qb * 128 + w * 32;
    const int qi = q0 + (lane & 31);
    const int kend = min(T, qb * 128 + 128);
    const int nkt = (kend + 63) / 64;
    const uint64_t* mrows = DROP ? dmask + ((int64_t)b * H + h) * T * Tw : nullptr;
    TileDma dma;
    dma.init(w, lane);
    auto issue = [&](int kt) {
        char* buf = smem[kt % 3][0];
        dma.issue(buf, Kg, rs, kt * 64, T, w);
        dma.issue(buf + kTileBytes, Vg, rs, kt * 64, T, w);
        if constexpr (DROP) mask_dma(smask[kt % 3], mrows, Tw, kt, qb * 128, T, w, lane);
    };
    issue(0);
    if (nkt > 1) issue(1);
    bf16x8 qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[kk] = load8(Qg + (int64_t)qi * rs + 16 * kk + 8 * g, qi < T);
    f32x16 o[2] = {zero16(), zero16()};
    // m is shared by the two half-waves (they hold different keys of the same
    // query); l is kept per half-wave and combined at the end
    float m = -INFINITY, l = 0.0f;
    for (int kt = 0; kt < nkt; ++kt) {
        // tile kt has landed once at most the next tile's 4 loads (5 with the
        // keep words) are pending (the Q loads above were issued after tiles 0
        // and 1 and are waited for by the compiler before their first use)
        if (kt + 1 < nkt) att_wait_vmcnt<DROP ? 5 : 4>();
        else att_wait_vmcnt<0>();
        att_lds_barrier();  // every wave's share of tile kt is in LDS; tile kt-1's slot is free
        uint64_t mw = 0;
        if constexpr (DROP) mw = smask[kt % 3][32 * w + (lane & 31)];
        if (kt + 2 < nkt) issue(kt + 2);
        const int k0 = kt * 64;
        const char* Ks = smem[kt % 3][0];
        const char* Vs = smem[kt % 3][1];
        if (k0 <= q0 + 31) {
            f32x16 s[2];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                s[kh] = zero16();
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) s[kh] = mfma(frag_row(Ks, 32 * kh, kk, lane), qf[kk], s[kh]);
            }
            // causal mask only on tiles that reach past this wave's first query
            if (k0 + 63 > q0) {
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    const int lim = qi - (k0 + 32 * kh + 4 * g);  // row offset allowed up to lim
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (8 * (r >> 2) + (r & 3) > lim) s[kh][r] = -INFINITY;
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kh][r]);
            const float mt = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sl2;  // raw scores scale by sl2 > 0
            if (__any(mt > m + kLazy)) {
                const float mn = fmaxf(m, mt);
                const float corr = fexp2(m - mn);
                l *= corr;
#pragma unroll
                for (int dt = 0; dt < 2; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[dt][r] *= corr;
                m = mn;
            }
            bf16x8 pk[4];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fexp2(fmaf(s[kh][r], sl2, -m));
                    l += p;
                    float pv = p;
                    if constexpr (DROP) pv = ((mw >> (32 * kh + 4 * g + 8 * (r >> 2) + (r & 3))) & 1) ? p : 0.0f;
                    pk[2 * kh + (r >> 3)][r & 7] = (__bf16)pv;
                }
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
#pragma unroll
                for (int u = 0; u < 4; ++u) o[dt] = mfma(frag_col(Vs, 16 * u, 32 * dt, lane), pk[u], o[dt]);
        }
    }
    l += __shfl_xor(l, 32, 64);
    if (qi < T) {
        const float inv = (DROP ? dscale : 1.0f) / l;
        bf16_t* orow = out + ((int64_t)b * T + qi) * C + h * 64;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int d = 32 * dt + 8 * rq + 4 * g;
                uint2 pk2;
                pk2.x = pack2bf(o[dt][4 * rq + 0] * inv, o[dt][4 * rq + 1] * inv);
                pk2.y = pack2bf(o[dt][4 * rq + 2] * inv, o[dt][4 * rq + 3] * inv);
                *(uint2*)(orow + d) = pk2;
            }
        if (g == 0) lse[((int64_t)b * H + h) * T + qi] = (m + log2f(l)) * kLn2;
    }
}

// ------------------------------------------------------------------ backward: dQ
// D_i = dO_i . O_i is formed here from the dO rows already in registers and
// written, with lse in base 2, to Dbuf for the dK/dV kernel that runs next.
template <bool DROP>
__global__ __launch_bounds__(256) void attn_bwd_dq_d64(const bf16_t* qkv, const bf16_t* outp, const bf16_t* dout,
                                                       const float* lse, float* Dbuf, bf16_t* dqkv, int T, int C,
                                                       int H, float sl2, float scale, const uint64_t* dmask, int Tw,
                                                       float dscale) {
    __shared__ __attribute__((aligned(16))) char smem[3][2][kTileBytes];
    __shared__ __attribute__((aligned(16))) uint64_t smask[DROP ? 3 : 1][128];  // keep words per query row
    int qb, h, b;
    block_coords(T, H, true, qb, h, b);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5;
    const int64_t rs = 3 * (int64_t)C;
    const bf16_t* base = qkv + (int64_t)b * T * rs;
    const bf16_t* Qg = base + h * 64;
    const bf16_t* Kg = base + C + h * 64;
    const bf16_t* Vg = base + 2 * C + h * 64;
    const bf16_t* dOg = dout + (int64_t)b * T * C + h * 64;
    const int q0 = qb * 128 + w * 32;
    const int qi = q0 + (lane & 31);
    const bool qok = qi < T;
    const int kend = min(T, qb * 128 + 128);
    const int nkt = (kend + 63) / 64;
    const uint64_t* mrows = DROP ? dmask + ((int64_t)b * H + h) * T * Tw : nullptr;
    // K/V tiles (and the keep words) stream into a three-deep LDS ring by DMA, two tiles ahead
    TileDma dma;
    dma.init(w, lane);
    auto issue = [&](int kt) {
        char* buf = smem[kt % 3][0];
        dma.issue(buf, Kg, rs, kt * 64, T, w);
        dma.issue(buf + kTileBytes, Vg, rs, kt * 64, T, w);
        if constexpr (DROP) mask_dma(smask[kt % 3], mrows, Tw, kt, qb * 128, T, w, lane);
    };
    issue(0);
    if (nkt > 1) issue(1);
    const bf16_t* Og = outp + (int64_t)b * T * C + h * 64;
    bf16x8 qf[4], df[4];
    float dpart = 0.0f;  // this half-wave's share of dO . O
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        qf[kk] = load8(Qg + (int64_t)qi * rs + 16 * kk + 8 * g, qok);
        df[kk] = load8(dOg + (int64_t)qi * C + 16 * kk + 8 * g, qok);
        const bf16x8 of = load8(Og + (int64_t)qi * C + 16 * kk + 8 * g, qok);
#pragma unroll
        for (int e = 0; e < 8; ++e) dpart = fmaf((float)df[kk][e], (float)of[e], dpart);
    }
    const int64_t lb = ((int64_t)b * H + h) * T;
    float* L2 = Dbuf + (int64_t)gridDim.x / ((T + 127) / 128) * T;  // lse * log2 e after the B H T values of D
    const float lse2 = qok ? lse[lb + qi] * kLog2e : 0.0f;
    const float Dq = dpart + __shfl_xor(dpart, 32, 64);
    if (qok && g == 0) {
        Dbuf[lb + qi] = Dq;
        L2[lb + qi] = lse2;
    }
    f32x16 dq[2] = {zero16(), zero16()};
    for (int kt = 0; kt < nkt; ++kt) {
        if (kt + 1 < nkt) att_wait_vmcnt<DROP ? 5 : 4>();
        else att_wait_vmcnt<0>();
        att_lds_barrier();  // every wave's share of tile kt is in LDS; tile kt-1's slot is free
        uint64_t mw = 0;
        if constexpr (DROP) mw = smask[kt % 3][32 * w + (lane & 31)];
        if (kt + 2 < nkt) issue(kt + 2);
        const int k0 = kt * 64;
        const char* Ks = smem[kt % 3][0];
        const char* Vs = smem[kt % 3][1];
        if (k0 <= q0 + 31) {
            f32x16 s[2], dp[2];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                s[kh] = zero16();
                dp[kh] = zero16();
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    s[kh] = mfma(frag_row(Ks, 32 * kh, kk, lane), qf[kk], s[kh]);
                    dp[kh] = mfma(frag_row(Vs, 32 * kh, kk, lane), df[kk], dp[kh]);
                }
            }
            bf16x8 dsk[4];
            const bool diag = k0 + 63 > q0;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const int lim = qi - (k0 + 32 * kh + 4 * g);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = fexp2(fmaf(s[kh][r], sl2, -lse2));
                    if (diag && 8 * (r >> 2) + (r & 3) > lim) p = 0.0f;
                    float dpk = dp[kh][r];
                    if constexpr (DROP)
                        dpk = ((mw >> (32 * kh + 4 * g + 8 * (r >> 2) + (r & 3))) & 1) ? dpk * dscale : 0.0f;
                    dsk[2 * kh + (r >> 3)][r & 7] = (__bf16)(p * (dpk - Dq));
                }
            }
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
#pragma unroll
                for (int u = 0; u < 4; ++u) dq[dt] = mfma(frag_col(Ks, 16 * u, 32 * dt, lane), dsk[u], dq[dt]);
        }
    }
    if (qok) {
        bf16_t* drow = dqkv + ((int64_t)b * T + qi) * rs + h * 64;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int d = 32 * dt + 8 * rq + 4 * g;
                uint2 pk2;
                pk2.x = pack2bf(dq[dt][4 * rq + 0] * scale, dq[dt][4 * rq + 1] * scale);
                pk2.y = pack2bf(dq[dt][4 * rq + 2] * scale, dq[dt][4 * rq + 3] * scale);
                *(uint2*)(drow + d) = pk2;
            }
    }
}

// ------------------------------------------------------------------ backward: dK, dV
template <bool DROP>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_d64(const bf16_t* qkv, const bf16_t* dout, const float* lse,
                                                         const float* Dbuf, bf16_t* dqkv, int T, int C, int H,
                                                         float sl2, float scale, const uint64_t* dmask, int Tw,
                                                         float dscale) {
    __shared__ __attribute__((aligned(16))) char smem[2][2][kTileBytes];
    __shared__ float sL[2][64], sD[2][64];
    // keep bits of the query tile against this workgroup's 128 keys: two words
    // per query row (keys kb 128 .. + 63 and + 64 .. + 127)
    __shared__ uint64_t sM[2][64][2];
    int kb, h, b;
    block_coords(T, H, false, kb, h, b);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5;
    const int64_t rs = 3 * (int64_t)C;
    const bf16_t* base = qkv + (int64_t)b * T * rs;
    const bf16_t* Qg = base + h * 64;
    const bf16_t* Kg = base + C + h * 64;
    const bf16_t* Vg = base + 2 * C + h * 64;
    const bf16_t* dOg = dout + (int64_t)b * T * C + h * 64;
    const int64_t lb = ((int64_t)b * H + h) * T;
    const float* L2 = Dbuf + (int64_t)gridDim.x / ((T + 127) / 128) * T;  // lse * log2 e after the B H T values of D
    const int k0w = kb * 128 + w * 32;
    const int kj = k0w + (lane & 31);
    bf16x8 kf[4], vf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        kf[kk] = load8(Kg + (int64_t)kj * rs + 16 * kk + 8 * g, kj < T);
        vf[kk] = load8(Vg + (int64_t)kj * rs + 16 * kk + 8 * g, kj < T);
    }
    f32x16 dk[2] = {zero16(), zero16()}, dv[2] = {zero16(), zero16()};
    const int qt0 = (kb * 128) / 64;
    const int nqt = (T + 63) / 64;
    TileRegs rq, rd;
    float pl = 0.0f, pd = 0.0f;
    uint64_t pm = 0;
    auto fetch = [&](int qt) {
        tile_load(rq, Qg, rs, qt * 64, T, tid);
        tile_load(rd, dOg, C, qt * 64, T, tid);
        if (tid < 64) {
            const int q = qt * 64 + tid;
            pl = q < T ? L2[lb + q] : INFINITY;  // rows past T get probability 0
            pd = q < T ? Dbuf[lb + q] : 0.0f;
        }
        if constexpr (DROP) {
            if (tid < 128) {
                const int q = qt * 64 + (tid >> 1), wd = 2 * kb + (tid & 1);
                pm = (q < T && wd < Tw) ? dmask[(lb + q) * Tw + wd] : 0;
            }
        }
    };
    auto put = [&](int buf) {
        tile_store(smem[buf][0], rq, tid);
        tile_store(smem[buf][1], rd, tid);
        if (tid < 64) {
            sL[buf][tid] = pl;
            sD[buf][tid] = pd;
        }
        if constexpr (DROP) {
            if (tid < 128) sM[buf][tid >> 1][tid & 1] = pm;
        }
    };
    const int kbit = kj & 63;  // this lane's key within its mask word (word w / 2 of the pair)
    if (qt0 < nqt) {
        fetch(qt0);
        put(0);
    }
    __syncthreads();
    for (int qt = qt0; qt < nqt; ++qt) {
        const int buf = (qt - qt0) & 1;
        const bool more = qt + 1 < nqt;
        if (more) fetch(qt + 1);
        const int q0t = qt * 64;
        const char* Qs = smem[buf][0];
        const char* dOs = smem[buf][1];
        if (q0t + 63 >= k0w) {
            bf16x8 pt[4], dst[4];
#pragma unroll
            for (int qh = 0; qh < 2; ++qh) {
                f32x16 s = zero16(), dp = zero16();
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    s = mfma(frag_row(Qs, 32 * qh, kk, lane), kf[kk], s);
                    dp = mfma(frag_row(dOs, 32 * qh, kk, lane), vf[kk], dp);
                }
                // queries of this half are q0t + 32 qh + acc_row(r, g); keep q >= kj
                const bool diag = q0t + 32 * qh < k0w + 32;
                const int lim = kj - (q0t + 32 * qh + 4 * g);  // row offset must be >= lim
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int ql = 32 * qh + acc_row(r, g);
                    float p = fexp2(fmaf(s[r], sl2, -sL[buf][ql]));
                    if (diag && 8 * (r >> 2) + (r & 3) < lim) p = 0.0f;
                    if constexpr (DROP) {
                        const bool kp = (sM[buf][ql][w >> 1] >> kbit) & 1;
                        pt[2 * qh + (r >> 3)][r & 7] = (__bf16)(kp ? p * dscale : 0.0f);
                        dst[2 * qh + (r >> 3)][r & 7] = (__bf16)(p * ((kp ? dp[r] * dscale : 0.0f) - sD[buf][ql]));
                    } else {
                        pt[2 * qh + (r >> 3)][r & 7] = (__bf16)p;
                        dst[2 * qh + (r >> 3)][r & 7] = (__bf16)(p * (dp[r] - sD[buf][ql]));
                    }
                }
            }
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    dv[dt] = mfma(pt[u], frag_col(dOs, 16 * u, 32 * dt, lane), dv[dt]);
                    dk[dt] = mfma(dst[u], frag_col(Qs, 16 * u, 32 * dt, lane), dk[dt]);
                }
        }
        if (more) put(buf ^ 1);
        __syncthreads();
    }
    // lane l holds column d = 32 dt + (l & 31), keys k0w + acc_row(r, g)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0w + acc_row(r, g);
            if (key < T) {
                bf16_t* drow = dqkv + ((int64_t)b * T + key) * rs + h * 64 + 32 * dt + (lane & 31);
                drow[C] = f2bf(dk[dt][r] * scale);
                drow[2 * C] = f2bf(dv[dt][r]);
            }
        }
}

// ------------------------------------------------------------------ dispatch
hipError_t attention_fwd(int dtype, int B, int Tn, int C, int H, const void* qkv, void* out, float* lse,
                         hipStream_t s, const uint64_t* dmask, float dscale) {
    if (B == 0 || Tn == 0) return hipSuccess;
    const int Tw = (Tn + 63) / 64;
    if (dtype == GPT2_DTYPE_BF16 && C / H == 64) {
        const float sl2 = kLog2e / 8.0f;  // 1/sqrt(64) in base 2
        const dim3 grid((unsigned)((Tn + 127) / 128 * H * B));
        if (dmask)
            hipLaunchKernelGGL(attn_fwd_d64<true>, grid, dim3(256), 0, s, (const bf16_t*)qkv, (bf16_t*)out, lse, Tn, C,
                               H, sl2, dmask, Tw, dscale);
        else
            hipLaunchKernelGGL(attn_fwd_d64<false>, grid, dim3(256), 0, s, (const bf16_t*)qkv, (bf16_t*)out, lse, Tn,
                               C, H, sl2, nullptr, Tw, 1.0f);
        return hipGetLastError();
    }
    return attention_fwd_simple(dtype, B, Tn, C, H, qkv, out, lse, s, dmask, dscale);
}

bool attention_bwd_staged(int dtype, int C, int H) { return dtype == GPT2_DTYPE_BF16 && C / H == 64; }

hipError_t attention_bwd(int dtype, int B, int Tn, int C, int H, const void* qkv, const void* out, const float* lse,
                         const void* dout, void* dqkv, float* Dbuf, hipStream_t s, int stages, const uint64_t* dmask,
                         float dscale) {
    if (B == 0 || Tn == 0) return hipSuccess;
    const int Tw = (Tn + 63) / 64;
    if (attention_bwd_staged(dtype, C, H)) {
        const float sl2 = kLog2e / 8.0f;
        const float scale = 0.125f;
        const dim3 grid((unsigned)((Tn + 127) / 128 * H * B));
        if (stages & ATT_BWD_DQ) {
            if (dmask)
                hipLaunchKernelGGL(attn_bwd_dq_d64<true>, grid, dim3(256), 0, s, (const bf16_t*)qkv, (const bf16_t*)out,
                                   (const bf16_t*)dout, lse, Dbuf, (bf16_t*)dqkv, Tn, C, H, sl2, scale, dmask, Tw,
                                   dscale);
            else
                hipLaunchKernelGGL(attn_bwd_dq_d64<false>, grid, dim3(256), 0, s, (const bf16_t*)qkv,
                                   (const bf16_t*)out, (const bf16_t*)dout, lse, Dbuf, (bf16_t*)dqkv, Tn, C, H, sl2,
                                   scale, nullptr, Tw, 1.0f);
        }
        if (stages & ATT_BWD_DKDV) {
            if (dmask)
                hipLaunchKernelGGL(attn_bwd_dkdv_d64<true>, grid, dim3(256), 0, s, (const bf16_t*)qkv,
                                   (const bf16_t*)dout, lse, (const float*)Dbuf, (bf16_t*)dqkv, Tn, C, H, sl2, scale,
                                   dmask, Tw, dscale);
            else
                hipLaunchKernelGGL(attn_bwd_dkdv_d64<false>, grid, dim3(256), 0, s, (const bf16_t*)qkv,
                                   (const bf16_t*)dout, lse, (const float*)Dbuf, (bf16_t*)dqkv, Tn, C, H, sl2, scale,
                                   nullptr, Tw, 1.0f);
        }
        return hipGetLastError();
    }
    if (stages != ATT_BWD_ALL) return hipErrorInvalidValue;
    return attention_bwd_simple(dtype, B, Tn, C, H, qkv, out, lse, dout, dqkv, Dbuf, s, dmask, dscale);
}

}  // namespace g2
