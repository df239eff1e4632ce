// ssd_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Element types: I/O tensors are either float or bfloat16 stored as uint16 bit
// patterns.  Matrix-core tiles use the 16x16 MFMA shapes of CDNA4 with wave64:
//   lane l: column/row index r16 = l & 15, lane group g4 = l >> 4 (0..3)
//   accumulator (4 floats): element i is D[row 4*g4 + i][col r16]
//   bf16 16x16x32: each lane supplies 8 bf16 of A (row r16) and 8 of B (col r16);
//                  the k index of element j in lane group g4 is the same
//                  function for A and B, so any consistent k assignment works
//   fp32 16x16x4:  each lane supplies A[r16][k = g4] and B[k = g4][r16]
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ssd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

typedef uint16_t bf16_bits;

__device__ __forceinline__ float bf16_to_f32(bf16_bits v) {
    return __uint_as_float(uint32_t(v) << 16);
}

// float -> bfloat16 with the hardware conversion (v_cvt_pk_bf16_f32: round to
// nearest even in the default rounding mode; NaN stays NaN).
__device__ __forceinline__ bf16_bits f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_bits, static_cast<__bf16>(f));
}

template <typename IO>
__device__ __forceinline__ float to_f32(IO v) {
    if constexpr (std::is_same_v<IO, float>) return v;
    else return bf16_to_f32(v);
}

template <typename IO>
__device__ __forceinline__ IO from_f32(float v) {
    if constexpr (std::is_same_v<IO, float>) return v;
    else return f32_to_bf16(v);
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// A buffer resource over `bytes` bytes from `base` (raw addressing, stride 0): a
// buffer access at a byte offset >= bytes is dropped (store) or reads 0 (load) by the
// hardware range check, so accesses need no branch around them.  The last word is the
// gfx9-family default (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, int(bytes), 0x00020000);
}
constexpr int kBufNonTemporal = 2;           // cache-policy bits of a buffer access: nt
constexpr uint32_t kBufOutOfRange = 0x7ffffff0u;   // a byte offset past any view

// 16 bytes of bf16 bit patterns as an MFMA operand.
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two 8-byte halves (4 bf16 each) as one MFMA operand.
__device__ __forceinline__ bf16x8 as_bf16x8(uint2 lo, uint2 hi) {
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Pack two floats into a 32-bit pair of bf16 (first value in the low half), one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// The low / high bf16 of a packed pair, widened exactly to float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Transpose an 8 x 8 block of 16-bit values: in[r] holds row r (8 values, element j
// in half (j & 1) of word j / 2); out[j] receives column j.  32 byte permutes.
__device__ __forceinline__ void transpose8x8_b16(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t a = (&in[2 * k].x)[j >> 1], b = (&in[2 * k + 1].x)[j >> 1];
            w[k] = __builtin_amdgcn_perm(b, a, sel);
        }
        out[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Transpose a 4 x 8 block of 16-bit values: in[r] holds row r (8 values); out[j]
// receives column j (4 values, row r in half (r & 1) of word r / 2).  16 permutes.
__device__ __forceinline__ void transpose4x8_b16(const uint4 (&in)[4], uint2 (&out)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t a0 = (&in[0].x)[j >> 1], a1 = (&in[1].x)[j >> 1];
        const uint32_t a2 = (&in[2].x)[j >> 1], a3 = (&in[3].x)[j >> 1];
        out[j] = make_uint2(__builtin_amdgcn_perm(a1, a0, sel), __builtin_amdgcn_perm(a3, a2, sel));
    }
}

// Sum over the 16 lanes of a DPP row; every lane of the row ends with the total.
__device__ __forceinline__ float row16_sum(float v) {
    constexpr int kQuadSwap1 = 0xB1, kQuadSwap2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140;
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kQuadSwap1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kQuadSwap2, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kRowHalfMirror, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kRowMirror, 0xF, 0xF, false));
    return v;
}

// v[l] + v[l ^ 16] in every lane l, on the vector ALU: v_permlane16_swap of v with
// itself trades the odd rows (16 lanes each) of one copy for the even rows of the
// other, so each lane holds its own value and its partner's (no LDS round trip, as a
// lane shuffle through ds_bpermute would take).  Addition commutes, so every lane
// gets the same bits as with the shuffle.
__device__ __forceinline__ float xor16_sum(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// v[l] + v[l ^ 32] in every lane l (v_permlane32_swap: the upper half of one copy for
// the lower half of the other).
__device__ __forceinline__ float xor32_sum(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// The value of lane `src` (the same for the whole wave) in every lane (v_readlane).
__device__ __forceinline__ float lane_value(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// Sum over the 64 lanes of a wave; every lane ends with the total.
__device__ __forceinline__ float wave_sum(float v) {
    return xor32_sum(xor16_sum(row16_sum(v)));
}

// Sum over the 4 lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48) of a wave.
__device__ __forceinline__ float group4_sum(float v) {
    return xor32_sum(xor16_sum(v));
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves (no LDS
// traffic): a Hillis-Steele scan inside each row of 16 lanes (shift right by 1, 2,
// 4, 8; lanes shifted in from outside the row add 0), then the total of row 0 is
// added to rows 1 and 3 and the total of rows 0-1 to rows 2 and 3.
__device__ __forceinline__ float wave_inclusive_scan(float v) {
    constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
    constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
    auto shifted = [](float x, auto ctrl) {
        return __int_as_float(
            __builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xF, 0xF, true));
    };
    v += shifted(v, std::integral_constant<int, kRowShr1>{});
    v += shifted(v, std::integral_constant<int, kRowShr2>{});
    v += shifted(v, std::integral_constant<int, kRowShr4>{});
    v += shifted(v, std::integral_constant<int, kRowShr8>{});
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kRowBcast15, 0xA, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kRowBcast31, 0xC, 0xF, false));
    return v;
}

// Inclusive prefix sum over the first 64 * kWaves threads of the block (the other
// waves only take part in the barriers).  `tmp` is LDS scratch of at least kWaves
// floats; the call contains two block barriers.
template <int kWaves>
__device__ __forceinline__ float block_inclusive_scan(float v, float *tmp) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        float o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    if (lane == 63 && wave < kWaves) tmp[wave] = v;
    __syncthreads();
    float add = 0.f;
    for (int w = 0; w < wave && w < kWaves; ++w) add += tmp[w];
    __syncthreads();
    return v + add;
}

// Inclusive prefix sum over a 256-thread block (4 waves).  `tmp` is LDS scratch
// of at least 4 floats; the call contains two block barriers.
__device__ __forceinline__ float block_inclusive_scan_256(float v, float *tmp) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        float o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    if (lane == 63) tmp[wave] = v;
    __syncthreads();
    float add = 0.f;
    for (int w = 0; w < wave; ++w) add += tmp[w];
    __syncthreads();
    return v + add;
}

}  // namespace ssd
