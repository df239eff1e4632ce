// ssd_chunk_scan.hip -- SSD chunked scan on gfx950 (CDNA4), three kernels.
//
// The sequence map of a selective SSM with a scalar decay per head is one
// lower-triangular semiseparable matrix; cutting it into Q x Q blocks gives
// quadratic diagonal blocks and low-rank off-diagonal blocks, which is the
// four-step chunked algorithm (Mamba-2 article (msbhsh.com), «SSD 算法：分块矩阵
// 分解» and «SSD 算法：分块和形态传递»).  With a_t = dt_t A_h and Acum the
// inclusive sum of a inside a chunk (kept in the log2 domain here):
//
//   step 1  Y_diag[t] = sum_{s<=t} (C_t . B_s) exp(Acum_t - Acum_s) dt_s x_s
//   step 2  S_c       = sum_s exp(Acum_end - Acum_s) dt_s x_s (outer) B_s
//   step 3  H_c       = exp(Acum_end) H_{c-1} + S_c          (H_{-1} = initial state)
//   step 4  Y_off[t]  = exp(Acum_t) C_t . H_{c-1}
//   y = Y_diag + Y_off + D x
//
// Kernels (one workgroup of 256 threads = 4 waves per (chunk, head, batch)):
//   k_chunk_state  discretisation + in-chunk decay scan, step 2 on MFMA
//   k_state_pass   step 3, a short sequential scan over chunks per state element
//   k_chunk_out    steps 1 and 4 on MFMA plus the D skip term
//
// MFMA operands that contract over tokens need the token index contiguous, so x
// and B are staged in LDS transposed ([channel][token]); operands that contract
// over the state dimension use the natural [token][n] layout.  Step 1 computes
// the transposed score tile (B C^T, rows s, cols t) whose accumulator layout is
// directly the B operand of the next MFMA, so the masked scores never leave
// registers.
#include <type_traits>

#include "ssd_device.h"
#include "ssd_kernels.h"
#include "ssd_stage.h"

namespace ssd {

namespace {

// ---------------------------------------------------------------- step 2 kernel
template <typename IO, int P>
__global__ __launch_bounds__(kThreads) void k_chunk_state(
    const IO *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const IO *__restrict__ B, float *__restrict__ S, float *__restrict__ alpha, int L, int H,
    int N, int G, int Q, int nc) {
    constexpr bool kBF = !std::is_same_v<IO, float>;
    const int c = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
    const int g = h / (H / G);
    const int t0 = c * Q, qlen = min(Q, L - t0);
    const int QS = lds_stride<IO>(Q);
    extern __shared__ __align__(16) unsigned char smem[];
    float *acum = reinterpret_cast<float *>(smem);
    float *wsc = acum + kThreads;
    float *tmp = wsc + kThreads;
    IO *XwT = reinterpret_cast<IO *>(smem + kScalarLds);   // [P][QS]  w_t x_t, transposed
    IO *BT = XwT + P * QS;                                  // [N][QS]  B_t, transposed
    const int tid = threadIdx.x;
    const size_t bh = size_t(bi) * H + h;

    const float d = chunk_cumsum(dt, A[h], bi, L, H, h, t0, qlen, acum, tmp);
    __syncthreads();
    const float aend = acum[qlen - 1];
    // weight of token t in the chunk state: decay from t to the chunk end, times dt_t
    wsc[tid] = tid < qlen ? exp2f(aend - acum[tid]) * d : 0.f;
    if (tid == 0) alpha[bh * nc + c] = exp2f(aend);
    __syncthreads();

    stage_transposed<IO, true>(x + ((size_t(bi) * L + t0) * H + h) * P, size_t(H) * P, P, Q,
                               qlen, XwT, QS, wsc);
    stage_transposed<IO, false>(B + ((size_t(bi) * L + t0) * G + g) * N, size_t(G) * N, N, Q,
                                qlen, BT, QS, nullptr);
    __syncthreads();

    // S[p][n] = sum_t XwT[p][t] BT[n][t]: 16x16 output tiles spread over the waves
    const int lane = tid & 63, wave = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
    const int ntn = N / 16, ntiles = (P / 16) * ntn;
    float *Sout = S + (bh * nc + c) * size_t(P) * N;
    for (int ti = wave; ti < ntiles; ti += 4) {
        const int pt = ti / ntn, nt = ti % ntn;
        const IO *arow = XwT + (pt * 16 + r16) * QS;
        const IO *brow = BT + (nt * 16 + r16) * QS;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (kBF) {
            for (int k0 = 0; k0 < Q; k0 += 32)
                acc = mfma_bf16(as_bf16x8(*reinterpret_cast<const uint4 *>(arow + k0 + 8 * g4)),
                                as_bf16x8(*reinterpret_cast<const uint4 *>(brow + k0 + 8 * g4)),
                                acc);
        } else {
            for (int k0 = 0; k0 < Q; k0 += 4) acc = mfma_f32(arow[k0 + g4], brow[k0 + g4], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) Sout[(pt * 16 + 4 * g4 + i) * N + nt * 16 + r16] = acc[i];
    }
}

// ---------------------------------------------------------------- step 3 kernel
// The scan over the chunk states, four state elements per thread: H_{-1} = init_state
// (zeros if null), hprev[c] = H_{c-1} (not written when hprev is null), H_c = alpha_c
// H_{c-1} + S_c, final_state = H_{nc-1} (when not null), and alpha_total = the product
// of the chunk decays (when not null).  The states and decays of 8 chunks are loaded
// ahead of the dependent chain.
template <typename IO>
__global__ __launch_bounds__(kThreads) void k_state_pass(
    const float *__restrict__ S, const float *__restrict__ alpha,
    const float *init_state, IO *__restrict__ hprev, float *final_state, float *alpha_total,
    int H, int PN, int nc) {
    constexpr int kBatch = 8;
    const size_t bh = size_t(blockIdx.z) * H + blockIdx.y;
    const int e = (blockIdx.x * kThreads + threadIdx.x) * 4;
    if (e >= PN) return;
    float4 hc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (init_state) hc = *reinterpret_cast<const float4 *>(init_state + bh * PN + e);
    float at = 1.f;
    for (int c0 = 0; c0 < nc; c0 += kBatch) {
        float4 sv[kBatch];
        float al[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int c = min(c0 + k, nc - 1);
            sv[k] = *reinterpret_cast<const float4 *>(S + (bh * nc + c) * size_t(PN) + e);
            al[k] = alpha[bh * nc + c];
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (c0 + k >= nc) break;
            if (hprev) {
                const size_t off = (bh * nc + c0 + k) * size_t(PN) + e;
                if constexpr (std::is_same_v<IO, float>) {
                    *reinterpret_cast<float4 *>(hprev + off) = hc;
                } else {
                    *reinterpret_cast<uint2 *>(hprev + off) =
                        make_uint2(pack_bf16x2(hc.x, hc.y), pack_bf16x2(hc.z, hc.w));
                }
            }
            hc.x = al[k] * hc.x + sv[k].x;
            hc.y = al[k] * hc.y + sv[k].y;
            hc.z = al[k] * hc.z + sv[k].z;
            hc.w = al[k] * hc.w + sv[k].w;
            at *= al[k];
        }
    }
    if (final_state) *reinterpret_cast<float4 *>(final_state + bh * PN + e) = hc;
    if (alpha_total && e == 0) alpha_total[bh] = at;
}

// ------------------------------------------------------------- steps 1 + 4 kernel
template <typename IO, int P>
__global__ __launch_bounds__(kThreads) void k_chunk_out(
    const IO *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const IO *__restrict__ B, const IO *__restrict__ C, const float *__restrict__ D,
    const IO *__restrict__ hprev, IO *__restrict__ y, int L, int H, int N, int G, int Q,
    int nc) {
    constexpr bool kBF = !std::is_same_v<IO, float>;
    constexpr int NPT = P / 16;
    const int c = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
    const int g = h / (H / G);
    const int t0 = c * Q, qlen = min(Q, L - t0);
    const int QS = lds_stride<IO>(Q), NS = lds_stride<IO>(N);
    extern __shared__ __align__(16) unsigned char smem[];
    float *acum = reinterpret_cast<float *>(smem);
    float *dts = acum + kThreads;
    float *tmp = dts + kThreads;
    IO *Bs = reinterpret_cast<IO *>(smem + kScalarLds);   // [Q][NS]  B_s natural
    IO *XT = Bs + Q * NS;                                  // [P][QS]  x transposed
    IO *Hb = XT + P * QS;                                  // [P][NS]  state entering chunk
    const int tid = threadIdx.x;
    const size_t bh = size_t(bi) * H + h;

    const float d = chunk_cumsum(dt, A[h], bi, L, H, h, t0, qlen, acum, tmp);
    dts[tid] = d;
    stage_rows<IO>(B + ((size_t(bi) * L + t0) * G + g) * N, size_t(G) * N, Q, qlen, N, Bs, NS);
    stage_transposed<IO, false>(x + ((size_t(bi) * L + t0) * H + h) * P, size_t(H) * P, P, Q,
                                qlen, XT, QS, nullptr);
    stage_rows<IO>(hprev + (bh * nc + c) * size_t(P) * N, N, P, P, N, Hb, NS);
    __syncthreads();

    const int lane = tid & 63, wave = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
    const float Dh = D[h];
    const int ntt = Q / 16;
    const int nk32 = round_up(N, 32) / 32;
    // 16-token output tiles, dealt to the waves in a snake order so that the
    // causal (triangular) work is balanced.
    for (int m = 0; m < ntt / 4; ++m) {
        const int T = 4 * m + ((m & 1) ? 3 - wave : wave);
        const int tl0 = T * 16;
        if (tl0 >= qlen) continue;
        const int t = tl0 + r16;   // this lane's output token (MFMA column)
        const bool tv = t < qlen;
        const IO *Crow = C + ((size_t(bi) * L + t0 + (tv ? t : 0)) * G + g) * N;

        f32x4 acc[NPT];
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};

        // C operand of this tile (B-operand layout: column t, k = n), bf16 only
        uint4 creg[8];
        if constexpr (kBF) {
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                creg[kk] = make_uint4(0, 0, 0, 0);
                const int n0 = kk * 32 + 8 * g4;
                if (kk < nk32 && tv && n0 < N)
                    creg[kk] = *reinterpret_cast<const uint4 *>(Crow + n0);
            }
        }

        // step 4: Y_off^T[p][t] = sum_n H[p][n] C[t][n], then scale column t by exp(Acum_t)
        if constexpr (kBF) {
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                if (kk >= nk32) break;
                const bf16x8 bop = as_bf16x8(creg[kk]);
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt)
                    acc[pt] = mfma_bf16(
                        as_bf16x8(*reinterpret_cast<const uint4 *>(
                            Hb + (pt * 16 + r16) * NS + kk * 32 + 8 * g4)),
                        bop, acc[pt]);
            }
        } else {
            for (int k0 = 0; k0 < N; k0 += 4) {
                const float bop = tv ? Crow[k0 + g4] : 0.f;
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt)
                    acc[pt] = mfma_f32(Hb[(pt * 16 + r16) * NS + k0 + g4], bop, acc[pt]);
            }
        }
        const float acum_t = acum[tv ? t : 0];
        const float et = tv ? exp2f(acum_t) : 0.f;
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) acc[pt] *= et;

        // step 1: masked scores M^T[s][t] = (B_s . C_t) exp(Acum_t - Acum_s) dt_s for s <= t,
        // contracted with x over s.
        if constexpr (kBF) {
            for (int s0 = 0; s0 <= tl0 + 15 && s0 < qlen; s0 += 32) {
                float gv[2][4];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int sb = s0 + 16 * half;
                    f32x4 gt = {0.f, 0.f, 0.f, 0.f};
                    if (sb <= tl0 + 15 && sb < qlen) {
                        const IO *brow = Bs + (sb + r16) * NS + 8 * g4;
#pragma unroll
                        for (int kk = 0; kk < 8; ++kk) {
                            if (kk >= nk32) break;
                            gt = mfma_bf16(
                                as_bf16x8(*reinterpret_cast<const uint4 *>(brow + kk * 32)),
                                as_bf16x8(creg[kk]), gt);
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int s = sb + 4 * g4 + i;
                        const bool ok = tv && s <= t && s < qlen;
                        gv[half][i] = ok ? gt[i] * exp2f(fminf(acum_t - acum[s], 0.f)) * dts[s] : 0.f;
                    }
                }
                const bf16x8 bop = as_bf16x8(make_uint4(
                    pack_bf16x2(gv[0][0], gv[0][1]), pack_bf16x2(gv[0][2], gv[0][3]),
                    pack_bf16x2(gv[1][0], gv[1][1]), pack_bf16x2(gv[1][2], gv[1][3])));
#pragma unroll
                for (int pt = 0; pt < NPT; ++pt) {
                    const IO *xr = XT + (pt * 16 + r16) * QS + s0 + 4 * g4;
                    acc[pt] = mfma_bf16(as_bf16x8(*reinterpret_cast<const uint2 *>(xr),
                                                  *reinterpret_cast<const uint2 *>(xr + 16)),
                                        bop, acc[pt]);
                }
            }
        } else {
            for (int sb = 0; sb <= tl0 + 15 && sb < qlen; sb += 16) {
                f32x4 gt = {0.f, 0.f, 0.f, 0.f};
                for (int k0 = 0; k0 < N; k0 += 4) {
                    const float bop = tv ? Crow[k0 + g4] : 0.f;
                    gt = mfma_f32(Bs[(sb + r16) * NS + k0 + g4], bop, gt);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = sb + 4 * g4 + i;
                    const bool ok = tv && s <= t && s < qlen;
                    const float gvi = ok ? gt[i] * exp2f(fminf(acum_t - acum[s], 0.f)) * dts[s] : 0.f;
#pragma unroll
                    for (int pt = 0; pt < NPT; ++pt)
                        acc[pt] = mfma_f32(XT[(pt * 16 + r16) * QS + sb + 4 * g4 + i], gvi,
                                           acc[pt]);
                }
            }
        }

        // epilogue: + D x, round, store y[t][p .. p+3]
        if (tv) {
            IO *yrow = y + ((size_t(bi) * L + t0 + t) * H + h) * P;
#pragma unroll
            for (int pt = 0; pt < NPT; ++pt) {
                const int p0 = pt * 16 + 4 * g4;
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    o[i] = acc[pt][i] + Dh * to_f32<IO>(XT[(p0 + i) * QS + t]);
                if constexpr (kBF) {
                    *reinterpret_cast<uint2 *>(yrow + p0) =
                        make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
                } else {
                    *reinterpret_cast<float4 *>(yrow + p0) = make_float4(o[0], o[1], o[2], o[3]);
                }
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_copy_state(const float *init, float *out,
                                                          size_t count) {
    const size_t i = size_t(blockIdx.x) * kThreads + threadIdx.x;
    if (i < count) out[i] = init ? init[i] : 0.f;
}

template <typename IO>
size_t lds_state_bytes(int P, int N, int Q) {
    return kScalarLds + size_t(P + N) * lds_stride<IO>(Q) * sizeof(IO);
}

template <typename IO>
size_t lds_out_bytes(int P, int N, int Q) {
    return kScalarLds +
           (size_t(Q) * lds_stride<IO>(N) + size_t(P) * lds_stride<IO>(Q) +
            size_t(P) * lds_stride<IO>(N)) *
               sizeof(IO);
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

template <typename IO, int P>
hipError_t launch_p(const ChunkScanArgs &a, const ChunkScanPlan &pl, hipStream_t stream) {
    char *ws = static_cast<char *>(a.workspace);
    float *S = reinterpret_cast<float *>(ws + pl.off_states);
    float *alpha = reinterpret_cast<float *>(ws + pl.off_alpha);
    IO *hprev = reinterpret_cast<IO *>(ws + pl.off_hprev);
    const IO *x = static_cast<const IO *>(a.x);
    const IO *B = static_cast<const IO *>(a.B);
    const IO *C = static_cast<const IO *>(a.C);
    IO *y = static_cast<IO *>(a.y);
    hipError_t e;

    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_chunk_state<IO, P>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(pl.lds_state));
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_chunk_out<IO, P>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(pl.lds_out));
    if (e != hipSuccess) return e;

    const dim3 grid(pl.nc, a.H, a.b);
    hipLaunchKernelGGL((k_chunk_state<IO, P>), grid, dim3(kThreads), pl.lds_state, stream, x,
                       a.dt, a.A, B, S, alpha, a.L, a.H, a.N, a.G, a.Q, pl.nc);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    const int PN = P * a.N;
    const dim3 gpass((PN / 4 + kThreads - 1) / kThreads, a.H, a.b);
    hipLaunchKernelGGL((k_state_pass<IO>), gpass, dim3(kThreads), 0, stream, S, alpha,
                       a.init_state, hprev, a.final_state, nullptr, a.H, PN, pl.nc);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    hipLaunchKernelGGL((k_chunk_out<IO, P>), grid, dim3(kThreads), pl.lds_out, stream, x, a.dt,
                       a.A, B, C, a.D, hprev, y, a.L, a.H, a.N, a.G, a.Q, pl.nc);
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_io(const ChunkScanArgs &a, const ChunkScanPlan &pl, hipStream_t stream) {
    switch (a.P) {
        case 16: return launch_p<IO, 16>(a, pl, stream);
        case 32: return launch_p<IO, 32>(a, pl, stream);
        case 64: return launch_p<IO, 64>(a, pl, stream);
        case 128: return launch_p<IO, 128>(a, pl, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

ChunkScanPlan plan_chunk_scan(int b, int L, int H, int P, int N, int G, int Q, bool bf16) {
    ChunkScanPlan pl;
    if (b <= 0 || L <= 0 || Q <= 0) return pl;
    pl.nc = (L + Q - 1) / Q;
    const size_t io = bf16 ? 2 : 4;
    const size_t units = size_t(b) * H * pl.nc;
    // the first kWsHeaderBytes hold the header of the single-pass kernel (ticket and
    // call number, error word, preparation marker): a workspace prepared once keeps
    // it whichever kernel a later call runs
    pl.off_states = kWsHeaderBytes;
    pl.off_alpha = pl.off_states + align256(units * size_t(P) * N * 4);
    pl.off_hprev = pl.off_alpha + align256(units * 4);
    pl.total = pl.off_hprev + align256(units * size_t(P) * N * io);
    if (bf16) {
        pl.lds_state = lds_state_bytes<bf16_bits>(P, N, Q);
        pl.lds_out = lds_out_bytes<bf16_bits>(P, N, Q);
    } else {
        pl.lds_state = lds_state_bytes<float>(P, N, Q);
        pl.lds_out = lds_out_bytes<float>(P, N, Q);
    }
    const bool shape_ok = (Q == 64 || Q == 128 || Q == 256) &&
                          (P == 16 || P == 32 || P == 64 || P == 128) && N % 16 == 0 &&
                          N >= 16 && N <= 256 && H <= 65535 && b <= 65535 && G > 0 && H % G == 0;
    pl.supported = shape_ok && pl.lds_state <= kMaxLds && pl.lds_out <= kMaxLds;
    return pl;
}

hipError_t launch_chunk_scan(const ChunkScanArgs &a, const ChunkScanPlan &pl,
                             hipStream_t stream) {
    if (a.bf16) return launch_io<bf16_bits>(a, pl, stream);
    return launch_io<float>(a, pl, stream);
}

size_t chunk_states_lds(int P, int N, int Q, bool bf16) {
    return bf16 ? lds_state_bytes<bf16_bits>(P, N, Q) : lds_state_bytes<float>(P, N, Q);
}

hipError_t launch_chunk_states(const void *x, const float *dt, const float *A, const void *B,
                               float *S, float *alpha, int b, int L, int H, int P, int N, int G,
                               int Q, bool bf16, hipStream_t stream) {
    const int nc = (L + Q - 1) / Q;
    if (nc == 0 || b == 0) return hipSuccess;
    const size_t lds = chunk_states_lds(P, N, Q, bf16);
    const dim3 grid(nc, H, b);
    hipError_t e = hipErrorInvalidValue;
    auto go = [&](auto io_tag, auto p_tag) {
        using IO = decltype(io_tag);
        constexpr int PP = decltype(p_tag)::value;
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_chunk_state<IO, PP>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return;
        hipLaunchKernelGGL((k_chunk_state<IO, PP>), grid, dim3(kThreads), lds, stream,
                           static_cast<const IO *>(x), dt, A, static_cast<const IO *>(B), S,
                           alpha, L, H, N, G, Q, nc);
        e = hipGetLastError();
    };
    auto by_p = [&](auto io_tag) {
        switch (P) {
            case 16: go(io_tag, std::integral_constant<int, 16>{}); break;
            case 32: go(io_tag, std::integral_constant<int, 32>{}); break;
            case 64: go(io_tag, std::integral_constant<int, 64>{}); break;
            case 128: go(io_tag, std::integral_constant<int, 128>{}); break;
            default: break;
        }
    };
    if (bf16) by_p(bf16_bits{}); else by_p(float{});
    return e;
}

hipError_t launch_state_fold(const float *S, const float *alpha, float *state, float *alpha_total,
                             int b, int H, int PN, int n, hipStream_t stream) {
    if (b == 0) return hipSuccess;
    const dim3 gpass((PN / 4 + kThreads - 1) / kThreads, H, b);
    hipLaunchKernelGGL((k_state_pass<float>), gpass, dim3(kThreads), 0, stream, S, alpha, nullptr,
                       static_cast<float *>(nullptr), state, alpha_total, H, PN, n);
    return hipGetLastError();
}

hipError_t launch_copy_state(const float *init_state, float *final_state, size_t count,
                             hipStream_t stream) {
    if (count == 0) return hipSuccess;
    const size_t blocks = (count + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(k_copy_state, dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                       init_state, final_state, count);
    return hipGetLastError();
}

}  // namespace ssd
