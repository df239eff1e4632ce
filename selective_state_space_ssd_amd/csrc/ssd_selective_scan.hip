// ssd_selective_scan.hip -- selective scan with one channel per head and a diagonal
// state matrix, on gfx950: the recurrence the SSD layer replaces, kept as a
// comparison kernel on the same data.
//
// Per (batch b, channel d) and state index n, with group g = d / (Dch/G):
//   h[n] <- exp(dt[b,t,d] A[d][n]) h[n] + dt[b,t,d] x[b,t,d] B[b,t,g,n]
//   y[b,t,d] = sum_n C[b,t,g,n] h[n] + D[d] x[b,t,d]
// B, C and the step dt depend on the token, A is fixed ("另辟蹊径--Mamba介绍",
// «Selectively Retain Information»); the state is carried by a scan («The Scan
// Operation»); compared with SSD, the head dimension is 1 and A is a full diagonal
// instead of a scalar times the identity (Bi-Mamba page, «Preliminary: Mamba
// Series»).  Discretisation, scan and the product with C run in one kernel and the
// per-token states never leave registers («Hardware-aware Algorithm»).
//
// Layout of the work: 8 lanes share a channel, each holding SL = N / 8 consecutive
// states, so a 256-thread block covers DC = 32 channels of one batch row.  The block
// walks the sequence in tiles of T tokens: x, dt, B and C of a tile are staged in LDS
// once for all DC channels, in fp32 (loaded into registers while the previous tile is
// computed, converted once at staging), the T steps run from LDS (each step: SL exponentials, the state
// update, the partial C . h, a sum over the NL lanes), and the tile's y is written back
// from LDS with coalesced stores.  Time runs sequentially inside a lane; the SL states
// of a lane are independent chains, and the parallelism is over (batch, channel,
// state).
#include <type_traits>

#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

namespace {

constexpr int kSelThreads = 256;

template <typename IO, int N>
struct SelShape {
    static constexpr int NL = 8;                      // lanes per channel
    static constexpr int SL = N / NL;                 // states per lane
    static constexpr int CW = 64 / NL;                // channels per wave
    static constexpr int DC = 4 * CW;                 // channels per block
    static constexpr int T = N <= 64 ? 64 : 32;       // tokens per tile (a multiple of 8)
    static_assert(N % 16 == 0 && N >= 16 && N <= 256, "N must be 16, 32, 64, 128 or 256");
    static constexpr int VW = 16 / int(sizeof(IO));   // elements per 16-byte piece
    static constexpr size_t kLds = size_t(T) * DC * 4 * 3 + size_t(T) * N * 4 * 2;
};

// Sum over groups of NL consecutive lanes (NL 4 or 8); every lane of a group ends
// with the group's sum.
template <int NL>
__device__ __forceinline__ float group_sum(float v) {
    constexpr int kQuadSwap1 = 0xB1, kQuadSwap2 = 0x4E, kRowHalfMirror = 0x141;
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kQuadSwap1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kQuadSwap2, 0xF, 0xF, false));
    if constexpr (NL >= 8)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kRowHalfMirror, 0xF, 0xF, false));
    static_assert(NL == 4 || NL == 8, "groups of 4 or 8 lanes");
    return v;
}

// SL consecutive fp32 values of one staged row (16-byte LDS reads where SL allows)
template <int SL>
__device__ __forceinline__ void lds_row(const float *src, float (&out)[SL]) {
    if constexpr (SL % 4 == 0) {
#pragma unroll
        for (int j = 0; j < SL; j += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(src + j);
            out[j] = v.x;
            out[j + 1] = v.y;
            out[j + 2] = v.z;
            out[j + 3] = v.w;
        }
    } else {
        static_assert(SL == 2, "2 or a multiple of 4 states per lane");
        const float2 v = *reinterpret_cast<const float2 *>(src);
        out[0] = v.x;
        out[1] = v.y;
    }
}

template <typename IO, int N>
__global__ __launch_bounds__(kSelThreads) void k_selective_scan(
    const IO *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const IO *__restrict__ B, const IO *__restrict__ C, const float *__restrict__ D,
    const float *__restrict__ init_state, IO *__restrict__ y, float *__restrict__ final_state,
    int L, int Dch, int G) {
    using S = SelShape<IO, N>;
    constexpr int T = S::T, DC = S::DC, NL = S::NL, SL = S::SL, VW = S::VW;
    static_assert(NL == 8, "group_sum and the channel layout assume 8 lanes per channel");
    extern __shared__ __align__(16) float sm[];
    float *xs = sm;                                  // [T][DC] x
    float *ds = xs + T * DC;                         // [T][DC] dt
    float *ys = ds + T * DC;                         // [T][DC] y
    float *bs = ys + T * DC;                         // [T][N] B
    float *cs = bs + T * N;                          // [T][N] C

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bi = blockIdx.y, d0 = blockIdx.x * DC;
    const int g = d0 / (Dch / G);    // the block's channels share one group
    const int dl = wave * S::CW + lane / NL;   // channel of this lane within the block
    const int n0 = (lane % NL) * SL;           // its SL states
    const int d = d0 + dl;

    // decays in the log2 domain, D, and the entering state
    float a2[SL], h[SL];
#pragma unroll
    for (int j = 0; j < SL; ++j) {
        a2[j] = A[size_t(d) * N + n0 + j] * kLog2e;
        h[j] = init_state ? init_state[(size_t(bi) * Dch + d) * N + n0 + j] : 0.f;
    }
    const float Dd = D[d];
    const bool writer = (lane % NL) == 0;

    // tile loads through buffer views of the tile's rows (rows past the sequence read
    // 0), held in registers until the LDS is free: x and dt one element per slot (row
    // t holds channels d0 .. d0+DC-1, contiguous in memory), B and C 16 bytes per slot
    constexpr int NX = T * DC / kSelThreads;
    constexpr int NV = (T * N / VW + kSelThreads - 1) / kSelThreads;
    static_assert(T * DC % kSelThreads == 0, "whole x / dt slots per thread");
    IO xr[NX];
    float dr[NX];
    uint4 br[NV], cr[NV];
    auto load_tile = [&](int t0) {
        const int tl = min(T, L - t0);
        const size_t row0 = size_t(bi) * L + t0;
        const __amdgpu_buffer_rsrc_t xv = buffer_rsrc(x + row0 * Dch + d0, uint32_t(tl) * uint32_t(Dch) * sizeof(IO));
        const __amdgpu_buffer_rsrc_t dv = buffer_rsrc(dt + row0 * Dch + d0, uint32_t(tl) * uint32_t(Dch) * 4u);
        const __amdgpu_buffer_rsrc_t bv = buffer_rsrc(B + row0 * G * N + size_t(g) * N,
                                                      uint32_t(tl) * uint32_t(G * N) * sizeof(IO));
        const __amdgpu_buffer_rsrc_t cv = buffer_rsrc(C + row0 * G * N + size_t(g) * N,
                                                      uint32_t(tl) * uint32_t(G * N) * sizeof(IO));
#pragma unroll
        for (int k = 0; k < NX; ++k) {
            const int i = tid + k * kSelThreads, t = i / DC, c = i % DC;
            const int off = t * Dch + c;
            if constexpr (std::is_same_v<IO, float>)
                xr[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xv, off * 4, 0, 0));
            else
                xr[k] = IO(__builtin_amdgcn_raw_buffer_load_b16(xv, off * 2, 0, 0));
            dr[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(dv, off * 4, 0, 0));
        }
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int i = min((tid + k * kSelThreads) * VW, T * N - VW), t = i / N, n = i % N;
            const int off = (t * G * N + n) * int(sizeof(IO));
            br[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(bv, off, 0, 0));
            cr[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(cv, off, 0, 0));
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int k = 0; k < NX; ++k) {
            const int i = tid + k * kSelThreads;
            xs[i] = to_f32<IO>(xr[k]);
            ds[i] = dr[k];
        }
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int i = (tid + k * kSelThreads) * VW;
            if (i < T * N) {
                if constexpr (std::is_same_v<IO, float>) {
                    *reinterpret_cast<uint4 *>(bs + i) = br[k];
                    *reinterpret_cast<uint4 *>(cs + i) = cr[k];
                } else {
                    const uint32_t *bw = &br[k].x, *cw = &cr[k].x;
#pragma unroll
                    for (int q = 0; q < 4; q += 2) {
                        *reinterpret_cast<float4 *>(bs + i + 2 * q) =
                            make_float4(bf16_lo(bw[q]), bf16_hi(bw[q]), bf16_lo(bw[q + 1]), bf16_hi(bw[q + 1]));
                        *reinterpret_cast<float4 *>(cs + i + 2 * q) =
                            make_float4(bf16_lo(cw[q]), bf16_hi(cw[q]), bf16_lo(cw[q + 1]), bf16_hi(cw[q + 1]));
                    }
                }
            }
        }
    };

    load_tile(0);
    for (int t0 = 0; t0 < L; t0 += T) {
        const int tl = min(T, L - t0);
        store_tile();
        __syncthreads();
        if (t0 + T < L) load_tile(t0 + T);   // in flight during this tile's steps
        // ---- the tile's steps (rows past the sequence hold x = dt = 0 and are not
        // written back), in groups of U: the y values of a group go to LDS together
        // after its steps, so that no step's LDS reads are ordered behind the previous
        // step's y store
        constexpr int U = SL <= 4 ? 8 : 32 / SL;   // the group's inputs fit the registers
        for (int t = 0; t < tl; t += U) {
            float yv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int tu = t + u;   // tu < T: the tile's rows past tl read zeros
                const float xv = xs[tu * DC + dl], dv = ds[tu * DC + dl];
                float bv[SL], cv[SL];
                lds_row<SL>(bs + tu * N + n0, bv);
                lds_row<SL>(cs + tu * N + n0, cv);
                const float uu = dv * xv;
                // the partial C . h in up to four independent sums (shorter chains)
                constexpr int NP = SL < 4 ? SL : 4;
                float pp[NP];
#pragma unroll
                for (int j = 0; j < NP; ++j) pp[j] = 0.f;
#pragma unroll
                for (int j = 0; j < SL; ++j) {
                    h[j] = __builtin_amdgcn_exp2f(dv * a2[j]) * h[j] + uu * bv[j];
                    pp[j % NP] += cv[j] * h[j];
                }
                float part = pp[0];
#pragma unroll
                for (int j = 1; j < NP; ++j) part += pp[j];
                yv[u] = group_sum<NL>(part) + Dd * xv;
            }
            if (writer) {
#pragma unroll
                for (int u = 0; u < U; ++u) ys[(t + u) * DC + dl] = yv[u];
            }
        }
        __syncthreads();
        // ---- write the tile's y (the next tile's staging touches only xs, ds, bs, cs)
        for (int i = tid; i < tl * DC; i += kSelThreads) {
            const int t = i / DC, c = i % DC;
            y[(size_t(bi) * L + t0 + t) * Dch + d0 + c] = from_f32<IO>(ys[i]);
        }
    }
    if (final_state) {
#pragma unroll
        for (int j = 0; j < SL; ++j) final_state[(size_t(bi) * Dch + d) * N + n0 + j] = h[j];
    }
}

template <typename IO, int N>
hipError_t launch_sel_n(const SelectiveArgs &a, hipStream_t stream) {
    using S = SelShape<IO, N>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_selective_scan<IO, N>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(S::kLds));
    if (e != hipSuccess) return e;
    const dim3 grid(a.Dch / S::DC, a.b);
    hipLaunchKernelGGL((k_selective_scan<IO, N>), grid, dim3(kSelThreads), S::kLds, stream,
                       static_cast<const IO *>(a.x), a.dt, a.A, static_cast<const IO *>(a.B),
                       static_cast<const IO *>(a.C), a.D, a.init_state, static_cast<IO *>(a.y),
                       a.final_state, a.L, a.Dch, a.G);
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_sel_io(const SelectiveArgs &a, hipStream_t stream) {
    switch (a.N) {
        case 16: return launch_sel_n<IO, 16>(a, stream);
        case 32: return launch_sel_n<IO, 32>(a, stream);
        case 64: return launch_sel_n<IO, 64>(a, stream);
        case 128: return launch_sel_n<IO, 128>(a, stream);
        case 256: return launch_sel_n<IO, 256>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int selective_channels_per_block(int N) {
    switch (N) {   // the same for both I/O types
        case 16: return SelShape<float, 16>::DC;
        case 32: return SelShape<float, 32>::DC;
        case 64: return SelShape<float, 64>::DC;
        case 128: return SelShape<float, 128>::DC;
        case 256: return SelShape<float, 256>::DC;
        default: return 0;
    }
}

hipError_t launch_selective_scan(const SelectiveArgs &a, hipStream_t stream) {
    if (a.bf16) return launch_sel_io<bf16_bits>(a, stream);
    return launch_sel_io<float>(a, stream);
}

}  // namespace ssd
