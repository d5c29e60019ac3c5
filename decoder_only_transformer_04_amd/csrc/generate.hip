// Autoregressive generation, one position of B sequences per step, the loop of
// MiniGPT.generate on the minigpt page (section 二; walkthrough 3.8): crop to the
// last block_size tokens, forward, last position's logits over the temperature,
// softmax, one draw, append. The forward of one position reuses the training
// step's LayerNorm and GEMM kernels with M = B rows; what is new here is
//  - the embedding of one position (gen_embed),
//  - attention of the new query over a cache of the keys and values of the
//    window so far (gen_attention), which also appends this position's k and v,
//  - the draw (gen_sample): the smallest token whose cumulative probability, in
//    index order, exceeds a caller-supplied uniform number u in [0, 1).
#include <cfloat>

#include "device.h"

namespace g2 {
namespace {

// The position of a step lives in device memory, cp[0] = sequence column of the
// token fed, cp[1] = its model position, cp[2] = prompt length, so one captured
// graph of a step serves every step: its last node moves the column and position on.
__global__ void gen_set_kernel(int32_t* cp, int col, int pos, int T0) {
    cp[0] = col;
    cp[1] = pos;
    cp[2] = T0;
}
__global__ void gen_advance_kernel(int32_t* cp) {
    cp[0] += 1;
    cp[1] += 1;
}

__global__ void gen_embed_kernel(const int32_t* seq, int64_t seq_ld, const int32_t* cp, const float* wte,
                                 const float* wpe, float* x, int C, int V, uint32_t* status) {
    const int b = blockIdx.x;
    const int col = cp[0], pos = cp[1];
    int tok = seq[(int64_t)b * seq_ld + col];
    if (tok < 0 || tok >= V) {
        if (threadIdx.x == 0) atomicOr(status, (uint32_t)GPT2_STATUS_TOKEN_RANGE);
        tok = 0;
    }
    const float* te = wte + (int64_t)tok * C;
    const float* pe = wpe + (int64_t)pos * C;
    float* xr = x + (int64_t)b * C;
    for (int c = threadIdx.x; c < C; c += blockDim.x) xr[c] = te[c] + pe[c];
}

constexpr int kAttThreads = 256;

// one 16-byte piece of an activation row as floats (8 bf16 or 4 fp32)
__device__ __forceinline__ void load16f(const bf16_t* p, float (&o)[8]) { unpack8f(*(const uint4*)p, o); }
__device__ __forceinline__ void load16f(const float* p, float (&o)[4]) {
    const float4 v = *(const float4*)p;
    o[0] = v.x;
    o[1] = v.y;
    o[2] = v.z;
    o[3] = v.w;
}

// One workgroup per (sequence b, head h); d = C / H <= 128, pos < Tc <= kGenMaxCache.
// Scores go to LDS (one float per cached position), then max, exponentials and
// their sum; the output sums p_j v_j with each thread owning one dimension of
// one of 256 / d interleaved slices of the positions, reduced in fixed order.
template <class T>
__global__ __launch_bounds__(kAttThreads) void gen_attn_kernel(const T* qkv, T* kc, T* vc, int Tc, const int32_t* cp,
                                                               T* out, int C, int H, float scale) {
    extern __shared__ float sm[];  // scores[Tc] | q[d] | partial outputs[kAttThreads] | reduction[kAttThreads]
    const int pos = cp[1];
    if (pos < 0 || pos >= Tc) return;  // the host keeps the window inside the cache
    const int b = blockIdx.x / H, h = blockIdx.x % H;
    const int d = C / H;
    const int tid = threadIdx.x;
    float* sc = sm;
    float* q = sm + Tc;
    float* part = q + d;
    float* red = part + kAttThreads;
    const T* row = qkv + (int64_t)b * 3 * C;
    T* kb = kc + (int64_t)b * Tc * C + h * d;
    T* vb = vc + (int64_t)b * Tc * C + h * d;
    // this position's query, and its key and value appended to the caches
    for (int c = tid; c < d; c += kAttThreads) {
        q[c] = Act<T>::ld(row, h * d + c);
        kb[(int64_t)pos * C + c] = row[C + h * d + c];
        vb[(int64_t)pos * C + c] = row[2 * C + h * d + c];
    }
    __syncthreads();  // the appended k and v are visible to the whole workgroup
    // scores of the positions j <= pos (causal: the new query sees the window so far);
    // a key row is read as 16-byte pieces when the head's columns allow it
    constexpr int E = 16 / sizeof(T);
    const bool vec = d % E == 0 && ((h * d) % E) == 0 && C % E == 0;
    float mx = -FLT_MAX;
    for (int j = tid; j <= pos; j += kAttThreads) {
        const T* kr = kb + (int64_t)j * C;
        float s = 0.0f;
        if (vec) {
            for (int c0 = 0; c0 < d; c0 += E) {
                float kv[E];
                load16f(kr + c0, kv);
#pragma unroll
                for (int e = 0; e < E; ++e) s = fmaf(q[c0 + e], kv[e], s);
            }
        } else {
            for (int c = 0; c < d; ++c) s = fmaf(q[c], Act<T>::ld(kr, c), s);
        }
        s *= scale;
        sc[j] = s;
        mx = fmaxf(mx, s);
    }
    // block maximum and sum: a wave reduction, then the four wave results
    constexpr int NWV = kAttThreads / 64;
    const int lane = tid & 63, wv = tid >> 6;
    mx = wave_max(mx);
    if (lane == 0) red[wv] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int k = 1; k < NWV; ++k) mx = fmaxf(mx, red[k]);
    float sum = 0.0f;
    for (int j = tid; j <= pos; j += kAttThreads) {
        const float e = __expf(sc[j] - mx);
        sc[j] = e;
        sum += e;
    }
    sum = wave_sum(sum);
    __syncthreads();  // every wave has read the maxima before they are overwritten
    if (lane == 0) red[wv] = sum;
    __syncthreads();
    float tot = red[0];
#pragma unroll
    for (int k = 1; k < NWV; ++k) tot += red[k];
    const float inv = 1.0f / tot;
    // out[c] = sum_j p_j v_j[c]: slice `sl` of the positions (j = sl, sl + ns, ...)
    const int ns = kAttThreads / d;  // d <= 128, so ns >= 2
    const int c = tid % d, sl = tid / d;
    float acc = 0.0f;
    if (sl < ns)
        for (int j = sl; j <= pos; j += ns) acc = fmaf(sc[j], Act<T>::ld(vb + (int64_t)j * C, c), acc);
    part[tid] = acc;
    __syncthreads();
    if (tid < d) {
        float o = 0.0f;
        for (int k = 0; k < ns; ++k) o += part[k * d + tid];
        Act<T>::st(out, (int64_t)b * C + h * d + tid, o * inv);
    }
}

constexpr int kSampleThreads = 1024;
constexpr int kSampleVec = 13;  // float4 pieces per thread: rows of up to 50k-odd logits (GPT-2: 50257)

// One workgroup per row. Thread t owns the contiguous chunk [t * ch, (t + 1) * ch)
// of the vocabulary (ch a multiple of 4), loaded once into registers as float4
// pieces; chunk sums of exp((z - max) / temperature) are scanned in index order,
// and the thread whose chunk holds u * total walks it to the first token whose
// running sum exceeds it.
__global__ __launch_bounds__(kSampleThreads) void gen_sample_kernel(const float* logits, int Vp, int V,
                                                                    float inv_temp, const float* u, int64_t u_ld,
                                                                    const int32_t* cp, int32_t* seq, int64_t seq_ld) {
    // the new token goes after the last one fed; it is new token number col + 1 - T0
    const int col = cp[0] + 1, ucol = cp[0] + 1 - cp[2];
    __shared__ float red[kSampleThreads];
    __shared__ float scan[kSampleThreads + 1];
    __shared__ float wsum[kSampleThreads / 64];
    __shared__ int pick;
    const int b = blockIdx.x, tid = threadIdx.x;
    const float* z = logits + (int64_t)b * Vp;
    const int ch = ((V + kSampleThreads - 1) / kSampleThreads + 3) / 4 * 4;
    const int lo = min(V, tid * ch), hi = min(V, lo + ch);
    float zv[kSampleVec * 4];
#pragma unroll
    for (int j = 0; j < kSampleVec; ++j) {
        const int k = lo + 4 * j;
        // whole pieces inside the padded row (Vp is a multiple of 4); tokens >= V are not used
        const float4 v = (4 * j < ch && k + 4 <= Vp) ? *(const float4*)(z + k) : make_float4(0.f, 0.f, 0.f, 0.f);
        zv[4 * j] = v.x; zv[4 * j + 1] = v.y; zv[4 * j + 2] = v.z; zv[4 * j + 3] = v.w;
    }
    float mx = -FLT_MAX;
#pragma unroll
    for (int i = 0; i < kSampleVec * 4; ++i)
        if (lo + i < hi) mx = fmaxf(mx, zv[i]);
    red[tid] = mx;
    if (tid == 0) pick = -1;
    __syncthreads();
    for (int w = kSampleThreads / 2; w > 0; w >>= 1) {
        if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
        __syncthreads();
    }
    mx = red[0];
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kSampleVec * 4; ++i)
        if (lo + i < hi) s += __expf((zv[i] - mx) * inv_temp);
    // prefix sums of the chunk sums in index order: within each wave by shuffles,
    // then the wave totals (one wave scans them), then each wave's offset added
    const int lane = tid & 63, wv = tid >> 6;
    float inc = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float t = __shfl_up(inc, off, 64);
        if (lane >= off) inc += t;
    }
    if (lane == 63) wsum[wv] = inc;
    __syncthreads();
    if (wv == 0) {
        float w = lane < kSampleThreads / 64 ? wsum[lane] : 0.0f;
#pragma unroll
        for (int off = 1; off < kSampleThreads / 64; off <<= 1) {
            const float t = __shfl_up(w, off, 64);
            if (lane >= off) w += t;
        }
        if (lane < kSampleThreads / 64) wsum[lane] = w;  // inclusive prefix of the wave totals
    }
    __syncthreads();
    scan[tid + 1] = inc + (wv > 0 ? wsum[wv - 1] : 0.0f);
    if (tid == 0) scan[0] = 0.0f;
    __syncthreads();
    const float target = u[(int64_t)b * u_ld + ucol] * scan[kSampleThreads];
    if (target >= scan[tid] && target < scan[tid + 1]) {
        // one thread walks its chunk (the exponentials recomputed as summed above)
        float run = scan[tid];
        int k = hi - 1;  // rounding can leave the walk just short of target: the chunk's last token
        for (int i = lo; i < hi; ++i) {
            run += __expf((z[i] - mx) * inv_temp);
            if (run > target) {
                k = i;
                break;
            }
        }
        atomicMax(&pick, k);  // one chunk holds the target; max keeps it unique
    }
    __syncthreads();
    if (tid == 0) {
        int k = pick;
        if (k < 0) {  // u * total at or past the rounded total: the last token with p > 0
            k = V - 1;
            while (k > 0 && __expf((z[k] - mx) * inv_temp) == 0.0f) --k;
        }
        seq[(int64_t)b * seq_ld + col] = k;
    }
}

}  // namespace

hipError_t gen_set(int32_t* cp, int col, int pos, int T0, hipStream_t s) {
    hipLaunchKernelGGL(gen_set_kernel, dim3(1), dim3(1), 0, s, cp, col, pos, T0);
    return hipGetLastError();
}

hipError_t gen_advance(int32_t* cp, hipStream_t s) {
    hipLaunchKernelGGL(gen_advance_kernel, dim3(1), dim3(1), 0, s, cp);
    return hipGetLastError();
}

hipError_t gen_embed(const int32_t* seq, int64_t seq_ld, const int32_t* cp, const float* wte, const float* wpe,
                     float* x, int B, int C, int V, uint32_t* status, hipStream_t s) {
    hipLaunchKernelGGL(gen_embed_kernel, dim3(B), dim3(256), 0, s, seq, seq_ld, cp, wte, wpe, x, C, V, status);
    return hipGetLastError();
}

hipError_t gen_attention(int dtype, const void* qkv, void* kc, void* vc, int Tc, const int32_t* cp, void* out, int B,
                         int C, int H, hipStream_t s) {
    const int d = C / H;
    if (d > 128 || Tc > kGenMaxCache) return hipErrorInvalidValue;
    const size_t lds = (size_t)(Tc + d + 2 * kAttThreads) * sizeof(float);
    const float scale = 1.0f / sqrtf((float)d);
    if (dtype == GPT2_DTYPE_BF16)
        hipLaunchKernelGGL(gen_attn_kernel<bf16_t>, dim3(B * H), dim3(kAttThreads), lds, s, (const bf16_t*)qkv,
                           (bf16_t*)kc, (bf16_t*)vc, Tc, cp, (bf16_t*)out, C, H, scale);
    else
        hipLaunchKernelGGL(gen_attn_kernel<float>, dim3(B * H), dim3(kAttThreads), lds, s, (const float*)qkv,
                           (float*)kc, (float*)vc, Tc, cp, (float*)out, C, H, scale);
    return hipGetLastError();
}

hipError_t gen_sample(const float* logits, int Vp, int V, float temperature, const float* u, int64_t u_ld,
                      const int32_t* cp, int32_t* seq, int64_t seq_ld, int B, hipStream_t s) {
    const int ch = ((V + kSampleThreads - 1) / kSampleThreads + 3) / 4 * 4;  // the kernel's chunk length
    if (ch > 4 * kSampleVec || Vp % 4 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gen_sample_kernel, dim3(B), dim3(kSampleThreads), 0, s, logits, Vp, V, 1.0f / temperature, u,
                       u_ld, cp, seq, seq_ld);
    return hipGetLastError();
}

}  // namespace g2
