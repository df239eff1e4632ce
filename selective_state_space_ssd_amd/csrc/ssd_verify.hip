// ssd_verify.hip -- verify step of speculative decoding on gfx950.
//
// K draft tokens are applied to an existing state per (batch, head); outputs are
// written for every position and the state after the accepted number of tokens is
// kept ("如何将 Llama 变成 Mamba？研究人员推出新工作并提高推理速度", «推测解码»:
// Mamba holds only its current state, so the verifier must keep the state at the
// position where the draft stops matching).
//
// The work is a stream over the state: every element is read once from HBM, updated
// K times in registers and written once (plus once per position when all states are
// requested).  Layout of the work: a row p of the P x N state is spread over LR
// consecutive lanes, each holding J float4 chunks whose columns interleave so that
// one load instruction of the wave covers whole 128-byte row segments; the
// reduction y = C . h over N is an in-lane sum followed by DPP lane moves.  B and C
// of the K tokens are shared by every row of a block and are staged once into LDS.
#include <algorithm>

#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

template <int N>
struct VerifyShape {
    static constexpr int LR = (N >= 32) ? 8 : N / 4;   // lanes per state row
    static constexpr int J = N / (4 * LR);             // float4 chunks per lane
    static constexpr int RW = 64 / LR;                 // rows per wave
    static constexpr int RB = 4 * RW;                  // rows per 256-thread block
    static_assert(J >= 1 && LR >= 1 && (N % (4 * LR)) == 0, "unsupported N");
};

// Sum over the LR consecutive lanes of a state row (LR in {4, 8}) with DPP lane
// moves inside the VALU: swap neighbours, swap pairs, then (LR = 8) fold the two
// quads of the 8-lane row half onto each other.
template <int LR>
__device__ __forceinline__ float row_sum(float v) {
    static_assert(LR == 4 || LR == 8, "row_sum covers 4 or 8 lanes");
    constexpr int kQuadSwap1 = 0xB1;        // quad_perm [1, 0, 3, 2]
    constexpr int kQuadSwap2 = 0x4E;        // quad_perm [2, 3, 0, 1]
    constexpr int kRowHalfMirror = 0x141;   // lane i <-> lane 7 - i within 8 lanes
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kQuadSwap1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kQuadSwap2, 0xF, 0xF, false));
    if constexpr (LR == 8)
        v += __int_as_float(
            __builtin_amdgcn_update_dpp(0, __float_as_int(v), kRowHalfMirror, 0xF, 0xF, false));
    return v;
}

template <typename IO>
__device__ __forceinline__ float4 load4(const IO *p) {
    if constexpr (std::is_same_v<IO, float>) {
        return *reinterpret_cast<const float4 *>(p);
    } else {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                           __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
    }
}

// Step activation fused into the kernel: softplus(v) = ln(1 + e^v), evaluated as
// max(v, 0) + ln(1 + e^{-|v|}) so that it cannot overflow.
__device__ __forceinline__ float softplus(float v) {
    return fmaxf(v, 0.f) + log1pf(expf(-fabsf(v)));
}

// B and C of the K tokens (group g) are staged once per block into LDS as fp32
// ([K][N] each).  KM >= K bounds the per-token registers (x and dt of every token).
// RING: the state comes from slot meta[2 b] of the row's ring [R][H][P][N] and the
// states after tokens 1 .. a go to the next a slots (mod R); state_out and states_all
// are unused.  dt_bias (nullable): the step is softplus(dt + dt_bias[h]).
template <typename IO, int N, int KM, bool RING>
__global__ __launch_bounds__(256) void k_verify(
    const float *state_in, const IO *__restrict__ x, const float *__restrict__ dt,
    const float *__restrict__ A, const IO *__restrict__ B, const IO *__restrict__ C,
    const float *__restrict__ D, const int32_t *__restrict__ accept_len, IO *__restrict__ y,
    float *state_out, float *__restrict__ states_all, int32_t *err_flag, int K, int H, int P,
    int G, float *ring, const int32_t *__restrict__ meta, int R,
    const float *__restrict__ dt_bias) {
    using S = VerifyShape<N>;
    extern __shared__ __align__(16) float sbc[];   // [K][N] B, then [K][N] C
    float *sB = sbc, *sC = sbc + K * N;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane % S::LR, rw = lane / S::LR;
    const int p = blockIdx.x * S::RB + wave * S::RW + rw;
    const int h = blockIdx.y, bi = blockIdx.z;
    const int g = h / (H / G);
    const bool valid = p < P;
    const size_t bh = size_t(bi) * H + h;
    const size_t row = (bh * P + (valid ? p : 0)) * N;
    // ring mode: the head slot of this row (reduced into [0, R) whatever meta holds,
    // so no access leaves the ring; an out-of-range head is reported), and the ring
    // of this (b) at head h
    int head = 0;
    if constexpr (RING) {
        const int raw = meta[2 * bi];
        head = ((raw % R) + R) % R;
        if (head != raw && err_flag && blockIdx.x == 0 && h == 0 && threadIdx.x == 0) *err_flag = 1;
    }
    const size_t slot_stride = size_t(H) * P * N;
    float *ring_bh = RING ? ring + size_t(bi) * R * slot_stride + size_t(h) * P * N : nullptr;
    const float *src = RING ? ring_bh + size_t(head) * slot_stride : state_in + bh * P * N;

    // All global loads are issued up front, without branches around them (range-
    // checked buffer views read 0 past their end), in the order they are needed: B
    // and C of the K tokens (staged into LDS before the barrier), x and dt, then the
    // state, so that the staging waits only for B and C.
    constexpr int kMaxK = KM;
    // the first 1024 elements of B and C ([K][N]; every K <= 1024 / N), one group of 4
    // per thread, held raw until the LDS stores
    using Raw = std::conditional_t<std::is_same_v<IO, float>, f32x4, u32x2>;
    const int i0 = 4 * int(threadIdx.x);   // element k * N + n of [K][N]
    Raw bq, cq;
    {
        const uint32_t bc_bytes = (uint32_t(K - 1) * uint32_t(G) * N + N) * uint32_t(sizeof(IO));
        const __amdgpu_buffer_rsrc_t bres = buffer_rsrc(B + (size_t(bi) * K * G + g) * N, bc_bytes);
        const __amdgpu_buffer_rsrc_t cres = buffer_rsrc(C + (size_t(bi) * K * G + g) * N, bc_bytes);
        const uint32_t off = i0 < K * N ? (uint32_t(i0 / N) * uint32_t(G) * N + uint32_t(i0 % N)) * uint32_t(sizeof(IO))
                                        : kBufOutOfRange;
        if constexpr (std::is_same_v<IO, float>) {
            bq = __builtin_amdgcn_raw_buffer_load_b128(bres, int(off), 0, 0);
            cq = __builtin_amdgcn_raw_buffer_load_b128(cres, int(off), 0, 0);
        } else {
            bq = __builtin_amdgcn_raw_buffer_load_b64(bres, int(off), 0, 0);
            cq = __builtin_amdgcn_raw_buffer_load_b64(cres, int(off), 0, 0);
        }
    }
    // x and y of this (b, h): token k, row p at [k * H * P + p] from these bases
    const size_t xy0 = (size_t(bi) * K * H + h) * P;
    const uint32_t tok_stride = uint32_t(H) * uint32_t(P);
    // x of every token for this row and dt of every token for this head, all loads in
    // flight at once: range-checked buffer views (K tokens; positions past K and rows
    // past P read 0), so that no load sits behind a branch and waits on the last
    float xr[kMaxK], dtr[kMaxK];
    {
        const __amdgpu_buffer_rsrc_t xres =
            buffer_rsrc(x + xy0, (uint32_t(K - 1) * tok_stride + uint32_t(P)) * uint32_t(sizeof(IO)));
        const __amdgpu_buffer_rsrc_t dres =
            buffer_rsrc(dt + size_t(bi) * K * H + h, (uint32_t(K - 1) * uint32_t(H) + 1u) * 4u);
#pragma unroll
        for (int k = 0; k < kMaxK; ++k) {
            const uint32_t off = valid ? (uint32_t(k) * tok_stride + uint32_t(p)) * uint32_t(sizeof(IO))
                                       : kBufOutOfRange;
            if constexpr (std::is_same_v<IO, float>)
                xr[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xres, int(off), 0, 0));
            else
                xr[k] = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(xres, int(off), 0, 0));
            dtr[k] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(dres, int(uint32_t(k) * uint32_t(H) * 4u), 0, 0));
        }
    }
    // the state streams through once: non-temporal loads and stores
    float4 s[S::J];
    {
        const __amdgpu_buffer_rsrc_t sres = buffer_rsrc(src, uint32_t(P) * N * 4u);
#pragma unroll
        for (int j = 0; j < S::J; ++j) {
            const int n = j * 4 * S::LR + lr * 4;
            const uint32_t off = valid ? (uint32_t(p) * N + uint32_t(n)) * 4u : kBufOutOfRange;
            const f32x4 t4 = __builtin_amdgcn_raw_buffer_load_b128(sres, int(off), 0, kBufNonTemporal);
            s[j] = make_float4(t4.x, t4.y, t4.z, t4.w);
        }
    }
    if (i0 < K * N) {
        if constexpr (std::is_same_v<IO, float>) {
            *reinterpret_cast<float4 *>(sB + i0) = make_float4(bq.x, bq.y, bq.z, bq.w);
            *reinterpret_cast<float4 *>(sC + i0) = make_float4(cq.x, cq.y, cq.z, cq.w);
        } else {
            *reinterpret_cast<float4 *>(sB + i0) = make_float4(bf16_lo(bq.x), bf16_hi(bq.x), bf16_lo(bq.y), bf16_hi(bq.y));
            *reinterpret_cast<float4 *>(sC + i0) = make_float4(bf16_lo(cq.x), bf16_hi(cq.x), bf16_lo(cq.y), bf16_hi(cq.y));
        }
    }
    for (int i = i0 + 1024; i < K * N; i += 1024) {   // K * N > 1024: the rest
        const int k = i / N, n = i % N;
        const size_t src = ((size_t(bi) * K + k) * G + g) * N + n;
        *reinterpret_cast<float4 *>(sB + i) = load4<IO>(B + src);
        *reinterpret_cast<float4 *>(sC + i) = load4<IO>(C + src);
    }

    int a = accept_len[bi];
    if (a < 0 || a > K) {
        if (err_flag && blockIdx.x == 0 && h == 0 && threadIdx.x == 0) *err_flag = 1;
        a = a < 0 ? 0 : K;
    }
    if (dt_bias) {
        const float bias = dt_bias[h];
#pragma unroll
        for (int k = 0; k < kMaxK; ++k) dtr[k] = softplus(dtr[k] + bias);
    }
    if (!RING && a == 0 && valid) {
#pragma unroll
        for (int j = 0; j < S::J; ++j)
            __builtin_nontemporal_store(f32x4{s[j].x, s[j].y, s[j].z, s[j].w},
                                            reinterpret_cast<f32x4 *>(state_out + row + j * 4 * S::LR + lr * 4));
    }
    __syncthreads();

    const float Ah = A[h], Dh = D[h];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        if (k >= K) break;
        const size_t tk = size_t(bi) * K + k;
        const float d = dtr[k];
        const float decay = expf(d * Ah);
        const float xk = xr[k];
        const float u = d * xk;
        float part = 0.f;
#pragma unroll
        for (int j = 0; j < S::J; ++j) {
            const int n = j * 4 * S::LR + lr * 4;
            const float4 bb = *reinterpret_cast<const float4 *>(sB + k * N + n);
            const float4 cc = *reinterpret_cast<const float4 *>(sC + k * N + n);
            s[j].x = decay * s[j].x + u * bb.x;
            s[j].y = decay * s[j].y + u * bb.y;
            s[j].z = decay * s[j].z + u * bb.z;
            s[j].w = decay * s[j].w + u * bb.w;
            part += cc.x * s[j].x + cc.y * s[j].y + cc.z * s[j].z + cc.w * s[j].w;
        }
        part = row_sum<S::LR>(part);
        if (valid && lr == 0)
            y[xy0 + (uint32_t(k) * tok_stride + uint32_t(p))] = from_f32<IO>(part + Dh * xk);
        if (RING && valid && k < a) {
            int slot = head + k + 1;
            slot = slot >= R ? slot - R : slot;
            float *dst = ring_bh + size_t(slot) * slot_stride + size_t(p) * N;
#pragma unroll
            for (int j = 0; j < S::J; ++j)
                __builtin_nontemporal_store(f32x4{s[j].x, s[j].y, s[j].z, s[j].w},
                                            reinterpret_cast<f32x4 *>(dst + j * 4 * S::LR + lr * 4));
        }
        if (!RING && valid) {
            if (states_all) {
                float *dst = states_all + ((tk * H + h) * P + p) * N;
#pragma unroll
                for (int j = 0; j < S::J; ++j)
                    __builtin_nontemporal_store(f32x4{s[j].x, s[j].y, s[j].z, s[j].w},
                                                reinterpret_cast<f32x4 *>(dst + j * 4 * S::LR + lr * 4));
            }
            if (k + 1 == a) {
#pragma unroll
                for (int j = 0; j < S::J; ++j)
                    __builtin_nontemporal_store(f32x4{s[j].x, s[j].y, s[j].z, s[j].w},
                                            reinterpret_cast<f32x4 *>(state_out + row + j * 4 * S::LR + lr * 4));
            }
        }
    }
}

template <typename IO, int N, int KM>
static hipError_t launch_verify_nk(const VerifyArgs &a, hipStream_t stream) {
    using S = VerifyShape<N>;
    dim3 grid((a.P + S::RB - 1) / S::RB, a.H, a.b);
    const size_t lds = size_t(2) * a.K * N * sizeof(float);
    if (a.ring)
        hipLaunchKernelGGL((k_verify<IO, N, KM, true>), grid, dim3(256), lds, stream, a.state_in,
                           static_cast<const IO *>(a.x), a.dt, a.A, static_cast<const IO *>(a.B),
                           static_cast<const IO *>(a.C), a.D, a.accept_len, static_cast<IO *>(a.y),
                           a.state_out, a.states_all, a.err_flag, a.K, a.H, a.P, a.G, a.ring,
                           a.meta, a.R, a.dt_bias);
    else
        hipLaunchKernelGGL((k_verify<IO, N, KM, false>), grid, dim3(256), lds, stream, a.state_in,
                           static_cast<const IO *>(a.x), a.dt, a.A, static_cast<const IO *>(a.B),
                           static_cast<const IO *>(a.C), a.D, a.accept_len, static_cast<IO *>(a.y),
                           a.state_out, a.states_all, a.err_flag, a.K, a.H, a.P, a.G, nullptr,
                           nullptr, 0, a.dt_bias);
    return hipGetLastError();
}

// the smallest register bound KM in {4, 8, 16} that holds K tokens
template <typename IO, int N>
static hipError_t launch_verify_n(const VerifyArgs &a, hipStream_t stream) {
    if (a.K <= 4) return launch_verify_nk<IO, N, 4>(a, stream);
    if (a.K <= 8) return launch_verify_nk<IO, N, 8>(a, stream);
    return launch_verify_nk<IO, N, 16>(a, stream);
}

template <typename IO>
static hipError_t launch_verify_io(const VerifyArgs &a, hipStream_t stream) {
    switch (a.N) {
        case 16: return launch_verify_n<IO, 16>(a, stream);
        case 32: return launch_verify_n<IO, 32>(a, stream);
        case 64: return launch_verify_n<IO, 64>(a, stream);
        case 128: return launch_verify_n<IO, 128>(a, stream);
        case 256: return launch_verify_n<IO, 256>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------- state ring
// Slot 0 of every row <- init_state (or zeros); head and depth <- 0.
__global__ __launch_bounds__(256) void k_ring_init(float *__restrict__ ring, int32_t *__restrict__ meta,
                                                   const float *__restrict__ init, int R,
                                                   size_t slot) {
    const int bi = blockIdx.y;
    for (size_t e = size_t(blockIdx.x) * 256 + threadIdx.x; e < slot; e += size_t(gridDim.x) * 256)
        ring[size_t(bi) * R * slot + e] = init ? init[size_t(bi) * slot + e] : 0.f;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        meta[2 * bi] = 0;
        meta[2 * bi + 1] = 0;
    }
}

// After a round: head <- (head + a) mod R, depth <- min(depth + a, R - 1), with a the
// accepted count clamped into [0, K] as the verify kernel clamped it.
__global__ __launch_bounds__(256) void k_ring_advance(int32_t *__restrict__ meta,
                                                      const int32_t *__restrict__ accept_len,
                                                      int b, int K, int R) {
    const int bi = blockIdx.x * 256 + threadIdx.x;
    if (bi >= b) return;
    int a = accept_len[bi];
    a = a < 0 ? 0 : (a > K ? K : a);
    const int head = ((meta[2 * bi] % R) + R) % R;
    const int depth = min(max(meta[2 * bi + 1], 0), R - 1);
    meta[2 * bi] = (head + a) % R;
    meta[2 * bi + 1] = min(depth + a, R - 1);
}

// head <- head - n (mod R), depth <- depth - n; n outside [0, depth] is clamped into
// it and reported through err_flag.
__global__ __launch_bounds__(256) void k_ring_rollback(int32_t *__restrict__ meta,
                                                       const int32_t *__restrict__ steps,
                                                       int32_t *err_flag, int b, int R) {
    const int bi = blockIdx.x * 256 + threadIdx.x;
    if (bi >= b) return;
    const int head = ((meta[2 * bi] % R) + R) % R;
    const int depth = min(max(meta[2 * bi + 1], 0), R - 1);
    int n = steps[bi];
    if (n < 0 || n > depth) {
        if (err_flag) *err_flag = 1;
        n = n < 0 ? 0 : depth;
    }
    meta[2 * bi] = ((head - n) % R + R) % R;
    meta[2 * bi + 1] = depth - n;
}

hipError_t launch_ring_init(float *ring, int32_t *meta, const float *init, int b, int R,
                            size_t slot, hipStream_t stream) {
    const unsigned gx = unsigned(std::min<size_t>((slot + 255) / 256, 1024));
    hipLaunchKernelGGL(k_ring_init, dim3(gx, b), dim3(256), 0, stream, ring, meta, init, R, slot);
    return hipGetLastError();
}

hipError_t launch_ring_advance(int32_t *meta, const int32_t *accept_len, int b, int K, int R,
                               hipStream_t stream) {
    hipLaunchKernelGGL(k_ring_advance, dim3((b + 255) / 256), dim3(256), 0, stream, meta,
                       accept_len, b, K, R);
    return hipGetLastError();
}

hipError_t launch_ring_rollback(int32_t *meta, const int32_t *steps, int32_t *err_flag, int b,
                                int R, hipStream_t stream) {
    hipLaunchKernelGGL(k_ring_rollback, dim3((b + 255) / 256), dim3(256), 0, stream, meta, steps,
                       err_flag, b, R);
    return hipGetLastError();
}

bool verify_supported_n(int N) {
    return N == 16 || N == 32 || N == 64 || N == 128 || N == 256;
}

hipError_t launch_verify(const VerifyArgs &a, hipStream_t stream) {
    if (a.bf16) return launch_verify_io<bf16_bits>(a, stream);
    return launch_verify_io<float>(a, stream);
}

}  // namespace ssd
