// Causal multi-head attention, scalar-FMA kernels (any head size <= 128, fp32
// or bf16 activations). One thread per query (forward, dQ) or per key (dK, dV),
// K/V or Q/dO tiles of 64 rows staged in LDS, online softmax over key tiles.
// Used for the fp32 mode and for head sizes the MFMA kernels do not cover.
//
// Forward: S = q k^T / sqrt(d) with j <= i, P = softmax_j S, o = P v; saves
// lse = max + log(sum exp) per row. Backward (P recomputed from lse):
// D_i = dO_i . O_i, dV_j = sum_i P_ij dO_i, dS_ij = P_ij (dO_i . v_j - D_i),
// dQ_i = sum_j dS_ij k_j / sqrt(d), dK_j = sum_i dS_ij q_i / sqrt(d).
// Dropout (dm non-null): the keep bit of (i, j) is bit j % 64 of word
// ((b H + h) T + i) Tw + j / 64; the forward weights v_j by P_ij keep_ij and
// scales o by dscale = 1 / (1 - p); the backward uses P keep dscale for dV and
// keep dscale (dO_i . v_j) in place of dO_i . v_j in dS.
#include <cmath>

#include "device.h"

namespace g2 {

template <class T, int DM>
__global__ __launch_bounds__(64) void attn_fwd_simple(const T* qkv, T* out, float* lse, int Tn, int C, int H,
                                                      const uint64_t* dm, int Tw, float dscale) {
    __shared__ float Ks[64][DM + 1], Vs[64][DM + 1];
    const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int d = C / H;
    const float scale = 1.0f / sqrtf((float)d);
    const int i = qb * 64 + lane;
    const int64_t rs = 3 * (int64_t)C;
    const T* base = qkv + (int64_t)b * Tn * rs;
    float q[DM], o[DM];
#pragma unroll
    for (int c = 0; c < DM; ++c) {
        q[c] = (i < Tn && c < d) ? Act<T>::ld(base, (int64_t)i * rs + h * d + c) : 0.0f;
        o[c] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    const uint64_t* mrow = dm ? dm + (((int64_t)b * H + h) * Tn + min(i, Tn - 1)) * Tw : nullptr;
    for (int kb = 0; kb <= qb; ++kb) {
        const int j0 = kb * 64;
        const uint64_t mw = mrow ? mrow[kb] : ~(uint64_t)0;
        {
            const int j = j0 + lane;
#pragma unroll
            for (int c = 0; c < DM; ++c) {
                const bool ok = j < Tn && c < d;
                Ks[lane][c] = ok ? Act<T>::ld(base, (int64_t)j * rs + C + h * d + c) : 0.0f;
                Vs[lane][c] = ok ? Act<T>::ld(base, (int64_t)j * rs + 2 * C + h * d + c) : 0.0f;
            }
        }
        __syncthreads();
        float s[64];
        float mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < 64; ++r) {
            const int j = j0 + r;
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < DM; ++c) acc += q[c] * Ks[r][c];
            s[r] = (j < Tn && j <= i) ? acc * scale : -INFINITY;
            mt = fmaxf(mt, s[r]);
        }
        const float mn = fmaxf(m, mt);
        if (mn != -INFINITY) {
            const float corr = m == -INFINITY ? 0.0f : expf(m - mn);
            l *= corr;
#pragma unroll
            for (int c = 0; c < DM; ++c) o[c] *= corr;
#pragma unroll
            for (int r = 0; r < 64; ++r) {
                const float p = s[r] == -INFINITY ? 0.0f : expf(s[r] - mn);
                l += p;
                const float pv = ((mw >> r) & 1) ? p : 0.0f;
#pragma unroll
                for (int c = 0; c < DM; ++c) o[c] += pv * Vs[r][c];
            }
            m = mn;
        }
        __syncthreads();
    }
    if (i < Tn) {
        const float inv = (dm ? dscale : 1.0f) / l;
        T* orow = out + ((int64_t)b * Tn + i) * C + h * d;
#pragma unroll
        for (int c = 0; c < DM; ++c)
            if (c < d) Act<T>::st(orow, c, o[c] * inv);
        lse[((int64_t)b * H + h) * Tn + i] = m + logf(l);
    }
}

// D[b,h,i] = sum_c dO[b,i,h*d+c] * O[b,i,h*d+c]
template <class T>
__global__ void attn_bwd_D(const T* out, const T* dout, float* Dbuf, int B, int Tn, int C, int H) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)B * H * Tn) return;
    const int i = (int)(t % Tn);
    const int h = (int)((t / Tn) % H);
    const int b = (int)(t / ((int64_t)Tn * H));
    const int d = C / H;
    const int64_t off = ((int64_t)b * Tn + i) * C + h * d;
    float s = 0.0f;
    for (int c = 0; c < d; ++c) s += Act<T>::ld(dout, off + c) * Act<T>::ld(out, off + c);
    Dbuf[t] = s;
}

template <class T, int DM>
__global__ __launch_bounds__(64) void attn_bwd_dkdv_simple(const T* qkv, const float* lse, const T* dout,
                                                           const float* Dbuf, T* dqkv, int Tn, int C, int H,
                                                           const uint64_t* dm, int Tw, float dscale) {
    __shared__ float Kown[64][DM + 1], Vown[64][DM + 1];
    __shared__ float Qs[64][DM + 1], dOs[64][DM + 1];
    __shared__ float Ls[64], Ds[64];
    __shared__ uint64_t Ms[64];  // keep words of the query tile for this key block
    const int kb = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int d = C / H;
    const float scale = 1.0f / sqrtf((float)d);
    const int j = kb * 64 + lane;
    const int64_t rs = 3 * (int64_t)C;
    const T* base = qkv + (int64_t)b * Tn * rs;
    const T* dob = dout + (int64_t)b * Tn * C;
    const int64_t lb = ((int64_t)b * H + h) * Tn;
#pragma unroll
    for (int c = 0; c < DM; ++c) {
        const bool ok = j < Tn && c < d;
        Kown[lane][c] = ok ? Act<T>::ld(base, (int64_t)j * rs + C + h * d + c) : 0.0f;
        Vown[lane][c] = ok ? Act<T>::ld(base, (int64_t)j * rs + 2 * C + h * d + c) : 0.0f;
    }
    float dk[DM], dv[DM];
#pragma unroll
    for (int c = 0; c < DM; ++c) { dk[c] = 0.0f; dv[c] = 0.0f; }
    const int nqb = (Tn + 63) / 64;
    for (int qb = kb; qb < nqb; ++qb) {
        __syncthreads();
        {
            const int i = qb * 64 + lane;
#pragma unroll
            for (int c = 0; c < DM; ++c) {
                const bool ok = i < Tn && c < d;
                Qs[lane][c] = ok ? Act<T>::ld(base, (int64_t)i * rs + h * d + c) : 0.0f;
                dOs[lane][c] = ok ? Act<T>::ld(dob, (int64_t)i * C + h * d + c) : 0.0f;
            }
            Ls[lane] = i < Tn ? lse[lb + i] : 0.0f;
            Ds[lane] = i < Tn ? Dbuf[lb + i] : 0.0f;
            Ms[lane] = (dm && i < Tn) ? dm[(lb + i) * Tw + kb] : ~(uint64_t)0;
        }
        __syncthreads();
        if (j < Tn) {
            for (int r = 0; r < 64; ++r) {
                const int i = qb * 64 + r;
                if (i >= Tn) break;
                if (j > i) continue;
                float s = 0.0f, dp = 0.0f;
#pragma unroll
                for (int c = 0; c < DM; ++c) {
                    s += Qs[r][c] * Kown[lane][c];
                    dp += dOs[r][c] * Vown[lane][c];
                }
                const float p = expf(s * scale - Ls[r]);
                const bool kp = (Ms[r] >> lane) & 1;
                const float pv = dm ? (kp ? p * dscale : 0.0f) : p;
                const float ds = p * ((dm ? (kp ? dp * dscale : 0.0f) : dp) - Ds[r]);
#pragma unroll
                for (int c = 0; c < DM; ++c) {
                    dv[c] += pv * dOs[r][c];
                    dk[c] += ds * Qs[r][c] * scale;
                }
            }
        }
    }
    if (j < Tn) {
        T* drow = dqkv + ((int64_t)b * Tn + j) * rs;
#pragma unroll
        for (int c = 0; c < DM; ++c)
            if (c < d) {
                Act<T>::st(drow, C + h * d + c, dk[c]);
                Act<T>::st(drow, 2 * C + h * d + c, dv[c]);
            }
    }
}

template <class T, int DM>
__global__ __launch_bounds__(64) void attn_bwd_dq_simple(const T* qkv, const float* lse, const T* dout,
                                                         const float* Dbuf, T* dqkv, int Tn, int C, int H,
                                                         const uint64_t* dm, int Tw, float dscale) {
    __shared__ float Ks[64][DM + 1], Vs[64][DM + 1];
    const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int d = C / H;
    const float scale = 1.0f / sqrtf((float)d);
    const int i = qb * 64 + lane;
    const int64_t rs = 3 * (int64_t)C;
    const T* base = qkv + (int64_t)b * Tn * rs;
    const int64_t lb = ((int64_t)b * H + h) * Tn;
    float q[DM], dO[DM], dq[DM];
#pragma unroll
    for (int c = 0; c < DM; ++c) {
        const bool ok = i < Tn && c < d;
        q[c] = ok ? Act<T>::ld(base, (int64_t)i * rs + h * d + c) : 0.0f;
        dO[c] = ok ? Act<T>::ld(dout, ((int64_t)b * Tn + i) * C + h * d + c) : 0.0f;
        dq[c] = 0.0f;
    }
    const float Li = i < Tn ? lse[lb + i] : 0.0f;
    const float Di = i < Tn ? Dbuf[lb + i] : 0.0f;
    const uint64_t* mrow = dm ? dm + (lb + min(i, Tn - 1)) * Tw : nullptr;
    for (int kb = 0; kb <= qb; ++kb) {
        const uint64_t mw = mrow ? mrow[kb] : ~(uint64_t)0;
        __syncthreads();
        {
            const int j = kb * 64 + lane;
#pragma unroll
            for (int c = 0; c < DM; ++c) {
                const bool ok = j < Tn && c < d;
                Ks[lane][c] = ok ? Act<T>::ld(base, (int64_t)j * rs + C + h * d + c) : 0.0f;
                Vs[lane][c] = ok ? Act<T>::ld(base, (int64_t)j * rs + 2 * C + h * d + c) : 0.0f;
            }
        }
        __syncthreads();
        if (i < Tn) {
            for (int r = 0; r < 64; ++r) {
                const int j = kb * 64 + r;
                if (j > i || j >= Tn) break;
                float s = 0.0f, dp = 0.0f;
#pragma unroll
                for (int c = 0; c < DM; ++c) {
                    s += q[c] * Ks[r][c];
                    dp += dO[c] * Vs[r][c];
                }
                const float p = expf(s * scale - Li);
                const float dpk = dm ? (((mw >> r) & 1) ? dp * dscale : 0.0f) : dp;
                const float ds = p * (dpk - Di) * scale;
#pragma unroll
                for (int c = 0; c < DM; ++c) dq[c] += ds * Ks[r][c];
            }
        }
    }
    if (i < Tn) {
        T* drow = dqkv + ((int64_t)b * Tn + i) * rs;
#pragma unroll
        for (int c = 0; c < DM; ++c)
            if (c < d) Act<T>::st(drow, h * d + c, dq[c]);
    }
}

template <class T, int DM>
static hipError_t fwd_simple(int B, int Tn, int C, int H, const void* qkv, void* out, float* lse, hipStream_t s,
                             const uint64_t* dm, float dscale) {
    dim3 grid((Tn + 63) / 64, H, B);
    hipLaunchKernelGGL((attn_fwd_simple<T, DM>), grid, dim3(64), 0, s, (const T*)qkv, (T*)out, lse, Tn, C, H, dm,
                       (Tn + 63) / 64, dscale);
    return hipGetLastError();
}

template <class T, int DM>
static hipError_t bwd_simple(int B, int Tn, int C, int H, const void* qkv, const void* out, const float* lse,
                             const void* dout, void* dqkv, float* Dbuf, hipStream_t s, const uint64_t* dm,
                             float dscale) {
    const int Tw = (Tn + 63) / 64;
    const int64_t n = (int64_t)B * H * Tn;
    hipLaunchKernelGGL((attn_bwd_D<T>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const T*)out,
                       (const T*)dout, Dbuf, B, Tn, C, H);
    dim3 grid((Tn + 63) / 64, H, B);
    hipLaunchKernelGGL((attn_bwd_dkdv_simple<T, DM>), grid, dim3(64), 0, s, (const T*)qkv, lse, (const T*)dout,
                       (const float*)Dbuf, (T*)dqkv, Tn, C, H, dm, Tw, dscale);
    hipLaunchKernelGGL((attn_bwd_dq_simple<T, DM>), grid, dim3(64), 0, s, (const T*)qkv, lse, (const T*)dout,
                       (const float*)Dbuf, (T*)dqkv, Tn, C, H, dm, Tw, dscale);
    return hipGetLastError();
}

hipError_t attention_fwd_simple(int dtype, int B, int Tn, int C, int H, const void* qkv, void* out, float* lse,
                                hipStream_t s, const uint64_t* dm, float dscale) {
    const int d = C / H;
    if (dtype == GPT2_DTYPE_BF16) {
        if (d <= 32) return fwd_simple<bf16_t, 32>(B, Tn, C, H, qkv, out, lse, s, dm, dscale);
        if (d <= 64) return fwd_simple<bf16_t, 64>(B, Tn, C, H, qkv, out, lse, s, dm, dscale);
        return fwd_simple<bf16_t, 128>(B, Tn, C, H, qkv, out, lse, s, dm, dscale);
    }
    if (d <= 32) return fwd_simple<float, 32>(B, Tn, C, H, qkv, out, lse, s, dm, dscale);
    if (d <= 64) return fwd_simple<float, 64>(B, Tn, C, H, qkv, out, lse, s, dm, dscale);
    return fwd_simple<float, 128>(B, Tn, C, H, qkv, out, lse, s, dm, dscale);
}

hipError_t attention_bwd_simple(int dtype, int B, int Tn, int C, int H, const void* qkv, const void* out,
                                const float* lse, const void* dout, void* dqkv, float* Dbuf, hipStream_t s,
                                const uint64_t* dm, float dscale) {
    const int d = C / H;
    if (dtype == GPT2_DTYPE_BF16) {
        if (d <= 32) return bwd_simple<bf16_t, 32>(B, Tn, C, H, qkv, out, lse, dout, dqkv, Dbuf, s, dm, dscale);
        if (d <= 64) return bwd_simple<bf16_t, 64>(B, Tn, C, H, qkv, out, lse, dout, dqkv, Dbuf, s, dm, dscale);
        return bwd_simple<bf16_t, 128>(B, Tn, C, H, qkv, out, lse, dout, dqkv, Dbuf, s, dm, dscale);
    }
    if (d <= 32) return bwd_simple<float, 32>(B, Tn, C, H, qkv, out, lse, dout, dqkv, Dbuf, s, dm, dscale);
    if (d <= 64) return bwd_simple<float, 64>(B, Tn, C, H, qkv, out, lse, dout, dqkv, Dbuf, s, dm, dscale);
    return bwd_simple<float, 128>(B, Tn, C, H, qkv, out, lse, dout, dqkv, Dbuf, s, dm, dscale);
}

}  // namespace g2
