// Dropout keep masks for training mode (the minigpt page's model, section 二:
// nn.Dropout on every head's attention weights, on the attention projection's
// output and on the FeedForward's output).
//
// The bits come from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011), a counter-based generator:
// element e of a site is a pure function of (seed, site, layer, e), so the
// masks are generated once per forward by these kernels, one thread per 64-bit
// word, and every consumer (the attention kernels, the residual epilogues, the
// LayerNorm backward) reads the stored bits instead of drawing its own. One
// call gives four 32-bit words = eight 16-bit draws, so a word of mask bits
// costs eight calls (~10 integer multiply rounds each).
#include "device.h"

namespace g2 {

namespace {

// ten rounds: words 0 and 2 are multiplied by the two round constants into
// 64-bit products whose halves, xor-ed with words 1 and 3 and the round key,
// form the next state; the key advances by the two Weyl constants per round
__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                              uint32_t k1, uint32_t (&r)[4]) {
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        // one 32 x 32 -> 64-bit product per multiplication (v_mad_u64_u32)
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c0 = n0;
        c1 = (uint32_t)p1;
        c2 = n2;
        c3 = (uint32_t)p0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    r[0] = c0;
    r[1] = c1;
    r[2] = c2;
    r[3] = c3;
}

// 16-bit half h (0..7) of one call: low half of word h / 2 first
__device__ __forceinline__ uint32_t half16(const uint32_t (&r)[4], int h) {
    const uint32_t w = r[h >> 1];
    return (h & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// keep bits of elements [e_lo, e_hi) (at most 64), bit (e - e_lo)
__device__ __forceinline__ uint64_t keep_bits(uint64_t e_lo, uint64_t e_hi, uint32_t site, uint32_t layer,
                                              uint32_t k0, uint32_t k1, uint32_t thr) {
    uint64_t bits = 0;
    for (uint64_t n = e_lo >> 3; (n << 3) < e_hi; ++n) {
        uint32_t r[4];
        philox4x32_10((uint32_t)n, (uint32_t)(n >> 32), site, layer, k0, k1, r);
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            const uint64_t e = (n << 3) + h;
            if (e >= e_lo && e < e_hi && half16(r, h) >= thr) bits |= (uint64_t)1 << (e - e_lo);
        }
    }
    return bits;
}

__global__ __launch_bounds__(256) void drop_attn_kernel(uint64_t* bits, int64_t words, int T, int Tw, uint32_t k0,
                                                        uint32_t k1, uint32_t thr, int layer0) {
    const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (w >= words) return;
    const int layer = layer0 + (int)blockIdx.y;
    const int64_t row = w / Tw;  // (b H + h) T + i
    const int kw = (int)(w - row * Tw);
    const int i = (int)(row % T);
    uint64_t out = 0;
    if (64 * kw <= i) {
        // keys 64 kw .. up to the diagonal (later keys are masked by causality)
        const uint64_t e0 = (uint64_t)row * T + 64 * kw;
        const int jend = min(64 * kw + 64, i + 1);
        out = keep_bits(e0, (uint64_t)row * T + jend, DROP_ATTN, (uint32_t)layer, k0, k1, thr);
    }
    bits[(int64_t)blockIdx.y * words + w] = out;
}

__global__ __launch_bounds__(256) void drop_res_kernel(uint64_t* bits, int64_t words, int64_t n_elem, int site,
                                                       uint32_t k0, uint32_t k1, uint32_t thr, int layer0) {
    const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (w >= words) return;
    const int layer = layer0 + (int)blockIdx.y;
    const uint64_t e0 = (uint64_t)w * 64;
    const uint64_t e1 = min(e0 + 64, (uint64_t)n_elem);
    bits[(int64_t)blockIdx.y * words + w] = keep_bits(e0, e1, (uint32_t)site, (uint32_t)layer, k0, k1, thr);
}

}  // namespace

hipError_t dropout_masks_attn(uint64_t* bits, int layer0, int L, int64_t words_per_layer, int BH, int T, int Tw,
                              uint64_t seed, uint32_t thr, hipStream_t s) {
    if (L <= 0 || words_per_layer <= 0) return hipSuccess;
    if (words_per_layer != (int64_t)BH * T * Tw || Tw != (T + 63) / 64) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((words_per_layer + 255) / 256), (unsigned)L);
    hipLaunchKernelGGL(drop_attn_kernel, grid, dim3(256), 0, s, bits, words_per_layer, T, Tw, (uint32_t)seed,
                       (uint32_t)(seed >> 32), thr, layer0);
    return hipGetLastError();
}

hipError_t dropout_masks_res(uint64_t* bits, int layer0, int L, int64_t words_per_layer, int64_t n_elem, int site,
                             uint64_t seed, uint32_t thr, hipStream_t s) {
    if (L <= 0 || words_per_layer <= 0) return hipSuccess;
    if (words_per_layer != (n_elem + 63) / 64) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((words_per_layer + 255) / 256), (unsigned)L);
    hipLaunchKernelGGL(drop_res_kernel, grid, dim3(256), 0, s, bits, words_per_layer, n_elem, site, (uint32_t)seed,
                       (uint32_t)(seed >> 32), thr, layer0);
    return hipGetLastError();
}

}  // namespace g2
