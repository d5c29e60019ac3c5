// Character-level data path of the minigpt page (prepare_data and get_batch in
// minigpt.py, section 二; walkthrough 3.2): a byte tokenizer on the host, and the
// batch windows gathered on the device from a token stream resident in HBM, so
// a training loop never copies batches from the host.
#include <cmath>
#include <cstring>

#include "device.h"

namespace {

// x[b, t] = data[off_b + t], y[b, t] = data[off_b + t + 1] for t < T; a start
// outside [0, n - T - 1] zeroes row b and raises GPT2_STATUS_WINDOW_RANGE
__global__ void batch_windows_kernel(const int32_t* data, int64_t n, const int64_t* off, int T, int32_t* x,
                                     int32_t* y, uint32_t* status) {
    const int b = blockIdx.x;
    const int64_t o = off[b];
    const bool ok = o >= 0 && o + T + 1 <= n;
    if (!ok && threadIdx.x == 0 && status) atomicOr(status, (uint32_t)GPT2_STATUS_WINDOW_RANGE);
    for (int t = threadIdx.x; t < T; t += blockDim.x) {
        x[(int64_t)b * T + t] = ok ? data[o + t] : 0;
        y[(int64_t)b * T + t] = ok ? data[o + t + 1] : 0;
    }
}

}  // namespace

extern "C" {

int32_t gpt2_char_vocab(const uint8_t* text, int64_t n, uint8_t* chars) {
    if (!chars || n < 0 || (n > 0 && !text)) return GPT2_EINVAL;
    bool seen[256] = {};
    for (int64_t i = 0; i < n; ++i) seen[text[i]] = true;
    int32_t v = 0;
    for (int c = 0; c < 256; ++c)
        if (seen[c]) chars[v++] = (uint8_t)c;  // ascending: the sorted set
    return v;
}

int gpt2_char_encode(const uint8_t* text, int64_t n, const uint8_t* chars, int32_t vocab, int32_t* ids) {
    if (n < 0 || (n > 0 && (!text || !ids)) || !chars || vocab < 1 || vocab > 256) return GPT2_EINVAL;
    int32_t stoi[256];
    for (int c = 0; c < 256; ++c) stoi[c] = -1;
    for (int32_t i = 0; i < vocab; ++i) stoi[chars[i]] = i;
    for (int64_t i = 0; i < n; ++i) {
        if (stoi[text[i]] < 0) return GPT2_EINVAL;
        ids[i] = stoi[text[i]];
    }
    return GPT2_OK;
}

int gpt2_char_decode(const int32_t* ids, int64_t n, const uint8_t* chars, int32_t vocab, uint8_t* text) {
    if (n < 0 || (n > 0 && (!text || !ids)) || !chars || vocab < 1 || vocab > 256) return GPT2_EINVAL;
    for (int64_t i = 0; i < n; ++i) {
        if (ids[i] < 0 || ids[i] >= vocab) return GPT2_EINVAL;
        text[i] = chars[ids[i]];
    }
    return GPT2_OK;
}

int64_t gpt2_split_point(int64_t n, double ratio) {
    if (n < 0 || !(ratio >= 0.0 && ratio <= 1.0)) return GPT2_EINVAL;
    return (int64_t)(ratio * (double)n);  // int(ratio * n), as prepare_data
}

int gpt2_batch_windows(const int32_t* d_data, int64_t n, const int64_t* d_offsets, int32_t B, int32_t T,
                       int32_t* d_x, int32_t* d_y, uint32_t* d_status, void* hip_stream) {
    if (B < 0 || T < 1 || n < 0 || (B > 0 && (!d_data || !d_offsets || !d_x || !d_y))) return GPT2_EINVAL;
    if (B == 0) return GPT2_OK;
    hipLaunchKernelGGL(batch_windows_kernel, dim3(B), dim3(256), 0, (hipStream_t)hip_stream, d_data, n, d_offsets, T,
                       d_x, d_y, d_status);
    return hipGetLastError() == hipSuccess ? GPT2_OK : GPT2_EHIP;
}

}  // extern "C"
