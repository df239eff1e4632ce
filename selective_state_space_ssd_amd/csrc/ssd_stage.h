// ssd_stage.h -- LDS staging helpers shared by the chunked-scan kernels.
#pragma once

#include "ssd_device.h"

namespace ssd {

constexpr int kThreads = 256;

__host__ __device__ constexpr int round_up(int v, int m) { return (v + m - 1) / m * m; }

// LDS row stride (elements) of a tile whose rows are contiguous in `len`
// elements: rounded up to the 32-element MFMA k-step, plus 16 bytes so that
// consecutive rows start in different banks.
template <typename IO>
__host__ __device__ constexpr int lds_stride(int len) {
    return round_up(len, 32) + 16 / int(sizeof(IO));
}

constexpr size_t kScalarLds = (2 * kThreads + 8) * sizeof(float);

template <typename IO>
__device__ __forceinline__ IO elem(const uint4 &v, int j) {
    if constexpr (std::is_same_v<IO, float>) {
        return __uint_as_float((&v.x)[j]);
    } else {
        return bf16_bits(((&v.x)[j >> 1] >> (16 * (j & 1))) & 0xffffu);
    }
}

// Discretisation and in-chunk decay scan shared by the chunk kernels.
// acum[t] = log2(e) * sum_{r<=t} dt_r A_h over the chunk (t < qlen), dts[t] = dt_t;
// both are 0 for t >= qlen.  Returns this thread's dt.
__device__ __forceinline__ float chunk_cumsum(const float *__restrict__ dt, float A_h, int bi,
                                              int L, int H, int h, int t0, int qlen,
                                              float *acum, float *tmp) {
    const int tid = threadIdx.x;
    float d = 0.f;
    if (tid < qlen) d = dt[(size_t(bi) * L + t0 + tid) * H + h];
    const float cs = block_inclusive_scan_256(d * A_h * kLog2e, tmp);
    acum[tid] = tid < qlen ? cs : 0.f;
    return d;
}

// Stage a [Q tokens][W channels] slice of a [.., token, .., channel] tensor into
// LDS transposed, dst[w * stride + t], optionally scaling token t by scale[t].
// Tokens >= qlen are written as zeros.  Works on token pairs so every LDS store
// writes two adjacent tokens.
template <typename IO, bool kScale>
__device__ __forceinline__ void stage_transposed(const IO *__restrict__ src, size_t tok_stride,
                                                 int W, int Q, int qlen, IO *dst, int stride,
                                                 const float *scale) {
    constexpr int VW = 16 / sizeof(IO);
    const int vpr = W / VW;
    const int items = (Q / 2) * vpr;
    for (int it = threadIdx.x; it < items; it += kThreads) {
        const int tp = (it / vpr) * 2, w0 = (it % vpr) * VW;
        uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
        if (tp < qlen) v0 = *reinterpret_cast<const uint4 *>(src + size_t(tp) * tok_stride + w0);
        if (tp + 1 < qlen)
            v1 = *reinterpret_cast<const uint4 *>(src + size_t(tp + 1) * tok_stride + w0);
        float s0 = 1.f, s1 = 1.f;
        if constexpr (kScale) {
            s0 = scale[tp];
            s1 = scale[tp + 1];
        }
#pragma unroll
        for (int j = 0; j < VW; ++j) {
            IO *d = dst + (w0 + j) * stride + tp;
            if constexpr (std::is_same_v<IO, float>) {
                *reinterpret_cast<float2 *>(d) =
                    make_float2(elem<IO>(v0, j) * s0, elem<IO>(v1, j) * s1);
            } else if constexpr (kScale) {
                *reinterpret_cast<uint32_t *>(d) = pack_bf16x2(
                    bf16_to_f32(elem<IO>(v0, j)) * s0, bf16_to_f32(elem<IO>(v1, j)) * s1);
            } else {
                *reinterpret_cast<uint32_t *>(d) =
                    uint32_t(elem<IO>(v0, j)) | (uint32_t(elem<IO>(v1, j)) << 16);
            }
        }
    }
}

// Stage `rows` rows of `W` contiguous elements (row i at src + i * row_stride) into
// LDS in natural layout, dst[i * stride + w]; columns [W, stride) up to the next
// multiple of 32 and rows >= valid_rows are zero.
template <typename IO>
__device__ __forceinline__ void stage_rows(const IO *__restrict__ src, size_t row_stride,
                                           int rows, int valid_rows, int W, IO *dst,
                                           int stride) {
    constexpr int VW = 16 / sizeof(IO);
    const int vpr = round_up(W, 32) / VW;
    const int items = rows * vpr;
    for (int it = threadIdx.x; it < items; it += kThreads) {
        const int r = it / vpr, w0 = (it % vpr) * VW;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < valid_rows && w0 < W)
            v = *reinterpret_cast<const uint4 *>(src + size_t(r) * row_stride + w0);
        *reinterpret_cast<uint4 *>(dst + r * stride + w0) = v;
    }
}

}  // namespace ssd
