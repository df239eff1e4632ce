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
// Layout of the work: every lane holds SL consecutive states of one channel (2 for
// N <= 32, else 4), so NL = N/SL lanes share a channel and a 256-thread block
// covers DC = 256 SL/N channels of one batch.  The block walks the sequence in
// tiles of T tokens: x, dt, B and C of a tile are staged in LDS (loaded into
// registers while the previous tile is computed), the T steps run from LDS (each
// step: SL exponentials, the state update, the partial C . h, a sum over the NL
// lanes), and the tile's y is written back from LDS with coalesced stores.  Time
// runs sequentially inside a lane; the parallelism is over (batch, channel, state).
#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

namespace {

constexpr int kSelThreads = 256;

template <int N>
struct SelShape {
    static constexpr int SL = N <= 32 ? 2 : 4;        // states per lane
    static constexpr int NL = N / SL;                 // lanes per channel
    static constexpr int CW = 64 / NL;                // channels per wave
    static constexpr int DC = 4 * CW;                 // channels per block
    static constexpr int T = N >= 256 ? 32 : 64;      // tokens per tile
    static_assert(N % 16 == 0 && N >= 16 && N <= 256, "N must be 16, 32, 64, 128 or 256");
    static constexpr size_t kLds = size_t(T) * DC * 4 * 3 + size_t(T) * N * 4 * 2;
};

// Sum over groups of NL consecutive lanes (NL a power of two, 4 .. 64); every lane
// of a group ends with the group's sum.
template <int NL>
__device__ __forceinline__ float group_sum(float v) {
    constexpr int kQuadSwap1 = 0xB1, kQuadSwap2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140;
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kQuadSwap1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kQuadSwap2, 0xF, 0xF, false));
    if constexpr (NL >= 8)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kRowHalfMirror, 0xF, 0xF, false));
    if constexpr (NL >= 16)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kRowMirror, 0xF, 0xF, false));
    if constexpr (NL >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (NL >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

template <typename IO, int N>
__global__ __launch_bounds__(kSelThreads) void k_selective_scan(
    const IO *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const IO *__restrict__ B, const IO *__restrict__ C, const float *__restrict__ D,
    const float *__restrict__ init_state, IO *__restrict__ y, float *__restrict__ final_state,
    int L, int Dch, int G) {
    using S = SelShape<N>;
    constexpr int T = S::T, DC = S::DC, NL = S::NL;
    extern __shared__ __align__(16) float sm[];
    float *xs = sm;                  // [T][DC] x
    float *ds = xs + T * DC;         // [T][DC] dt
    float *ys = ds + T * DC;         // [T][DC] y
    float *bs = ys + T * DC;         // [T][N] B
    float *cs = bs + T * N;          // [T][N] C

    constexpr int SL = S::SL;
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

    // tile loads, held in registers until the LDS is free: x and dt one element per
    // slot (row t of the tile holds channels d0 .. d0+DC-1, contiguous in memory), B
    // and C 16 bytes per slot (rows of N contiguous elements)
    constexpr int NX = (T * DC + kSelThreads - 1) / kSelThreads;
    constexpr int VW = 16 / int(sizeof(IO));
    constexpr int NV = (T * N / VW + kSelThreads - 1) / kSelThreads;
    IO xr[NX];
    float dr[NX];
    uint4 br[NV], cr[NV];
    auto load_tile = [&](int t0) {
        const int tl = min(T, L - t0);
#pragma unroll
        for (int k = 0; k < NX; ++k) {
            const int i = tid + k * kSelThreads, t = i / DC, c = i % DC;
            const bool ok = i < T * DC && t < tl;
            const size_t src = (size_t(bi) * L + t0 + (ok ? t : 0)) * Dch + d0 + c;
            xr[k] = ok ? x[src] : IO(0);
            dr[k] = ok ? dt[src] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int i = (tid + k * kSelThreads) * VW, t = i / N, n = i % N;
            const bool ok = i < T * N && t < tl;
            const size_t src = ((size_t(bi) * L + t0 + (ok ? t : 0)) * G + g) * N + n;
            br[k] = ok ? *reinterpret_cast<const uint4 *>(B + src) : make_uint4(0, 0, 0, 0);
            cr[k] = ok ? *reinterpret_cast<const uint4 *>(C + src) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int k = 0; k < NX; ++k) {
            const int i = tid + k * kSelThreads;
            if (i < T * DC) {
                xs[i] = to_f32<IO>(xr[k]);
                ds[i] = dr[k];
            }
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
                    for (int q = 0; q < 4; ++q) {
                        bs[i + 2 * q] = bf16_lo(bw[q]);
                        bs[i + 2 * q + 1] = bf16_hi(bw[q]);
                        cs[i + 2 * q] = bf16_lo(cw[q]);
                        cs[i + 2 * q + 1] = bf16_hi(cw[q]);
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
        // ---- the tile's steps, in groups of U: the inputs of a group are read from
        // LDS together (the y stores to LDS would otherwise order every step's reads
        // after the previous step's store), then the steps run, then the y values go
        // out together
        constexpr int U = SL == 2 ? 8 : 4;
        int t = 0;
        for (; t + U <= tl; t += U) {
            float xv[U], dv[U], bv[U][SL], cv[U][SL], yv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                xv[u] = xs[(t + u) * DC + dl];
                dv[u] = ds[(t + u) * DC + dl];
#pragma unroll
                for (int j = 0; j < SL; ++j) {
                    bv[u][j] = bs[(t + u) * N + n0 + j];
                    cv[u][j] = cs[(t + u) * N + n0 + j];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float uu = dv[u] * xv[u];
                float part = 0.f;
#pragma unroll
                for (int j = 0; j < SL; ++j) {
                    h[j] = __builtin_amdgcn_exp2f(dv[u] * a2[j]) * h[j] + uu * bv[u][j];
                    part += cv[u][j] * h[j];
                }
                yv[u] = group_sum<NL>(part) + Dd * xv[u];
            }
            if (writer) {
#pragma unroll
                for (int u = 0; u < U; ++u) ys[(t + u) * DC + dl] = yv[u];
            }
        }
        for (; t < tl; ++t) {   // the last partial group
            const float xv = xs[t * DC + dl], dv = ds[t * DC + dl];
            const float uu = dv * xv;
            float part = 0.f;
#pragma unroll
            for (int j = 0; j < SL; ++j) {
                h[j] = __builtin_amdgcn_exp2f(dv * a2[j]) * h[j] + uu * bs[t * N + n0 + j];
                part += cs[t * N + n0 + j] * h[j];
            }
            part = group_sum<NL>(part);
            if (writer) ys[t * DC + dl] = part + Dd * xv;
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
    using S = SelShape<N>;
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
    switch (N) {
        case 16: return SelShape<16>::DC;
        case 32: return SelShape<32>::DC;
        case 64: return SelShape<64>::DC;
        case 128: return SelShape<128>::DC;
        case 256: return SelShape<256>::DC;
        default: return 0;
    }
}

hipError_t launch_selective_scan(const SelectiveArgs &a, hipStream_t stream) {
    if (a.bf16) return launch_sel_io<bf16_bits>(a, stream);
    return launch_sel_io<float>(a, stream);
}

}  // namespace ssd
