// ssd_slice_state.hip -- the state a slice of the sequence leaves from a zero start,
// and the slice's total decay, without forming any output.
//
// In the sequence-parallel layout (Mamba-2 article (msbhsh.com), «序列并行») every
// device contributes the pair (total decay, final state) of its slice.  Computed
// first, the pair lets the devices exchange and combine states before any output
// exists, after which each device scans its slice once from its entering state.  The
// pair is steps 2 and 3 of the chunked algorithm («SSD 算法：分块和形态传递») with
// the outputs of steps 1 and 4 left out:
//
//   state = sum over chunks c of (decay from the end of c to the end of the slice)
//           * sum_{t in c} dt_t (decay from t to the end of c) x_t (outer) B_t
//
// k_slice_state_bf (bf16 I/O, P = 64, N in {64, 128, 256}): one workgroup of 8 waves
// per (run of 128-token segments, head, batch).  The run's P x N state stays in MFMA
// accumulators: at each segment it decays by the segment's total decay and takes the
// segment's contribution, one bf16 MFMA contraction over the segment's tokens of
// (dt_t times the decay to the segment end) x_t against B_t (fp32 accumulation).  The
// next segment's x, B and dt are loaded while the current one is multiplied.  Each run
// writes its state and total decay; the step 3 scan (k_state_pass) folds the runs in
// order.  Runs are sized so that about two workgroups per CU are launched.
#include <algorithm>
#include <type_traits>

#include "ssd_device.h"
#include "ssd_kernels.h"

namespace ssd {

namespace {

constexpr int kSS = 128;        // tokens per segment
constexpr int kSSP = kSS + 16;  // LDS row stride (bf16) of the transposed tiles: 72
                                // dwords, free of bank conflicts for the 16-byte MFMA
                                // operand reads and for the staging stores below
constexpr int kSlots = 512;     // workgroups the launch aims at (two per CU of gfx950)

template <int N>
struct SliceFz {
    static constexpr int P = 64;
    static constexpr int NTN = N / 16;             // state column tiles
    static constexpr int NTW = NTN / 4;            // column tiles per wave
    static constexpr int kXItems = (kSS / 8) * (P / 8);   // 8 x 8 staging blocks of x
    static constexpr int kBItems = (kSS / 8) * (N / 8);   // ... and of B
    static constexpr int IPT = (kXItems + kBItems + 511) / 512;   // blocks per thread
    static constexpr size_t kLds = size_t(P + N) * kSSP * 2 + kSS * 4;
    static constexpr int kWgPerCu = kLds <= 80 * 1024 ? 2 : 1;
    static_assert(N % 64 == 0 && N <= 256, "N must be 64, 128 or 256");
};

// Staging block `it` of a [16 token blocks][CB channel blocks] grid: 64 consecutive
// blocks form an 8 x 8 square taken along diagonals (lane l: token block l % 8,
// channel block (l % 8 + l / 8) % 8), so that each of the 8 row loads of a wave reads
// 8 whole 128-byte row pieces and 8 consecutive lanes store to distinct LDS banks.
template <int CB>
__device__ __forceinline__ void staging_block(int it, int &tb, int &cb) {
    const int blk = it >> 6, l = it & 63;
    tb = 8 * (blk % 2) + (l & 7);
    cb = 8 * (blk / 2) + (((l & 7) + (l >> 3)) & 7);
    static_assert(CB % 8 == 0, "whole 8 x 8 squares");
}

template <int N>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2 * SliceFz<N>::kWgPerCu)))
void k_slice_state_bf(const bf16_bits *__restrict__ x, const float *__restrict__ dt,
                      const float *__restrict__ A, const bf16_bits *__restrict__ B,
                      float *__restrict__ S, float *__restrict__ alpha, int L, int H, int G,
                      int segs_per_part, int parts) {
    using F = SliceFz<N>;
    constexpr int P = F::P;
    extern __shared__ __align__(16) unsigned char smem[];
    bf16_bits *XT = reinterpret_cast<bf16_bits *>(smem);   // [P][kSSP] decay-weighted x
    bf16_bits *BT = XT + P * kSSP;                          // [N][kSSP] B, transposed
    float *wts = reinterpret_cast<float *>(BT + N * kSSP);  // [kSS] token weights
    const int part = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
    const size_t bh = size_t(bi) * H + h;
    const float Al2 = A[h] * kLog2e;
    const int nseg = (L + kSS - 1) / kSS;
    const int s_begin = part * segs_per_part, s_end = min(s_begin + segs_per_part, nseg);

    // range-checked views of the batch row: tokens at or past L read 0
    const __amdgpu_buffer_rsrc_t xres =
        buffer_rsrc(x + size_t(bi) * L * H * P, uint32_t(L) * uint32_t(H * P) * 2u);
    const __amdgpu_buffer_rsrc_t bres =
        buffer_rsrc(B + size_t(bi) * L * G * N, uint32_t(L) * uint32_t(G * N) * 2u);
    const __amdgpu_buffer_rsrc_t dtres =
        buffer_rsrc(dt + size_t(bi) * L * H, uint32_t(L) * uint32_t(H) * 4u);

    // the staging blocks of this thread: blocks below kXItems are x's, the rest B's
    uint4 raw[F::IPT][8];
    float dq[2];   // dt of tokens 2 lane, 2 lane + 1 of the segment (the decay layout)
    auto load = [&](int s) {
        const int t0 = s * kSS;
#pragma unroll
        for (int k = 0; k < F::IPT; ++k) {
            const int it = tid + 512 * k;
            if (it >= F::kXItems + F::kBItems) continue;
            int tb, cb;
            if (it < F::kXItems) {
                staging_block<P / 8>(it, tb, cb);
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    raw[k][r] = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                   xres, int(((t0 + 8 * tb + r) * H + h) * P * 2 + 16 * cb), 0,
                                   kBufNonTemporal));
            } else {
                staging_block<N / 8>(it - F::kXItems, tb, cb);
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    raw[k][r] = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                   bres, int(((t0 + 8 * tb + r) * G + g) * N * 2 + 16 * cb), 0, 0));
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
            dq[i] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(dtres, int(((t0 + 2 * lane + i) * H + h) * 4), 0, 0));
    };

    // state tiles of this wave: row tiles 2 (w / 4) + {0, 1}, column tiles (w % 4) NTW + j
    const int pt0 = 2 * (w / 4), nt0 = (w % 4) * F::NTW;
    f32x4 acc[2][F::NTW];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int j = 0; j < F::NTW; ++j) acc[k][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;   // log2 of the run's decay so far

    if (s_begin < s_end) load(s_begin);
    for (int s = s_begin; s < s_end; ++s) {
        // decay inside the segment (log2 domain), computed by every wave for all of its
        // tokens: tokens 2 lane and 2 lane + 1, then a wave scan
        const float a0 = dq[0] * Al2, a01 = a0 + dq[1] * Al2;
        const float run = wave_inclusive_scan(a01);
        const float aend = lane_value(run, 63);
        if (w == 0) {
            // weight of token t: dt_t times the decay from t to the segment end (<= dt_t)
            const float c0 = run - a01 + a0;
            *reinterpret_cast<float2 *>(wts + 2 * lane) =
                make_float2(dq[0] * __builtin_amdgcn_exp2f(fminf(aend - c0, 0.f)),
                            dq[1] * __builtin_amdgcn_exp2f(fminf(aend - run, 0.f)));
        }
        __syncthreads();   // weights visible; the previous segment's products are done

        // stage: x rows scaled by their weights, then both tiles transposed (8 x 8 blocks
        // in registers, 16-byte LDS stores)
#pragma unroll
        for (int k = 0; k < F::IPT; ++k) {
            const int it = tid + 512 * k;
            if (it >= F::kXItems + F::kBItems) continue;
            int tb, cb;
            bf16_bits *dst;
            if (it < F::kXItems) {
                staging_block<P / 8>(it, tb, cb);
                const float4 w0 = *reinterpret_cast<const float4 *>(wts + 8 * tb);
                const float4 w1 = *reinterpret_cast<const float4 *>(wts + 8 * tb + 4);
                const float wr[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    uint4 &v = raw[k][r];
                    const float f = wr[r];
                    v = make_uint4(pack_bf16x2(bf16_lo(v.x) * f, bf16_hi(v.x) * f),
                                   pack_bf16x2(bf16_lo(v.y) * f, bf16_hi(v.y) * f),
                                   pack_bf16x2(bf16_lo(v.z) * f, bf16_hi(v.z) * f),
                                   pack_bf16x2(bf16_lo(v.w) * f, bf16_hi(v.w) * f));
                }
                dst = XT;
            } else {
                staging_block<N / 8>(it - F::kXItems, tb, cb);
                dst = BT;
            }
            uint4 cols[8];
            transpose8x8_b16(raw[k], cols);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<uint4 *>(dst + (8 * cb + j) * kSSP + 8 * tb) = cols[j];
        }
        if (s + 1 < s_end) load(s + 1);   // in flight during this segment's products
        __syncthreads();

        // the run's state decays through the segment, then takes its contribution
        const float al = __builtin_amdgcn_exp2f(fminf(aend, 0.f));
        lsum += aend;
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int j = 0; j < F::NTW; ++j) acc[k][j] *= al;
#pragma unroll
        for (int kk = 0; kk < kSS / 32; ++kk) {
            uint4 af[2], bfr[F::NTW];
#pragma unroll
            for (int k = 0; k < 2; ++k)
                af[k] = *reinterpret_cast<const uint4 *>(XT + ((pt0 + k) * 16 + r16) * kSSP +
                                                         32 * kk + 8 * g4);
#pragma unroll
            for (int j = 0; j < F::NTW; ++j)
                bfr[j] = *reinterpret_cast<const uint4 *>(BT + ((nt0 + j) * 16 + r16) * kSSP +
                                                          32 * kk + 8 * g4);
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int j = 0; j < F::NTW; ++j)
                    acc[k][j] = mfma_bf16(as_bf16x8(af[k]), as_bf16x8(bfr[j]), acc[k][j]);
        }
    }

    // the run's state, [P][N] fp32 (element (row 4 g4 + i, column r16) of each tile),
    // and its total decay
    float *Sout = S + (bh * parts + part) * size_t(P) * N;
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int j = 0; j < F::NTW; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                Sout[((pt0 + k) * 16 + 4 * g4 + i) * N + (nt0 + j) * 16 + r16] = acc[k][j][i];
    if (tid == 0) alpha[bh * parts + part] = __builtin_amdgcn_exp2f(fminf(lsum, 0.f));
}

template <int N>
hipError_t launch_fast(const bf16_bits *x, const float *dt, const float *A, const bf16_bits *B,
                       float *S, float *alpha, int b, int L, int H, int G,
                       const SliceStatePlan &pl, hipStream_t stream) {
    using F = SliceFz<N>;
    if constexpr (F::kLds > 64 * 1024) {
        const hipError_t e =
            hipFuncSetAttribute(reinterpret_cast<const void *>(&k_slice_state_bf<N>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(F::kLds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_slice_state_bf<N>), dim3(pl.parts, H, b), dim3(512), F::kLds, stream, x,
                       dt, A, B, S, alpha, L, H, G, pl.segs_per_part, pl.parts);
    return hipGetLastError();
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

SliceStatePlan plan_slice_state(int b, int L, int H, int P, int N, int G, bool bf16) {
    SliceStatePlan pl;
    const bool shape_ok = (P == 16 || P == 32 || P == 64 || P == 128) && N % 16 == 0 &&
                          N >= 16 && N <= 256 && H <= 65535 && b <= 65535 && G > 0 &&
                          H % G == 0 && b >= 0 && L >= 0;
    if (!shape_ok) return pl;
    // the dedicated kernel addresses a batch row through 32-bit buffer offsets
    const size_t rows = size_t(L) + kSS;
    const bool small = rows * H * P * 2 < (size_t(1) << 31) && rows * G * N * 2 < (size_t(1) << 31) &&
                       rows * H * 4 < (size_t(1) << 31);
    pl.fast = bf16 && P == 64 && (N == 64 || N == 128 || N == 256) && small;
    if (pl.fast) {
        // runs of whole segments, about kSlots workgroups in all
        const int nseg = (L + kSS - 1) / kSS;
        const long heads = long(b) * H;
        const int target = int(std::max(1L, std::min(long(nseg), (kSlots + heads - 1) / std::max(heads, 1L))));
        pl.segs_per_part = nseg ? (nseg + target - 1) / target : 1;
        pl.parts = nseg ? (nseg + pl.segs_per_part - 1) / pl.segs_per_part : 0;
    } else {
        for (const int Q : {256, 128, 64}) {   // the longest chunk whose tiles fit in LDS
            if (chunk_states_lds(P, N, Q, bf16) <= kMaxLds) {
                pl.Q = Q;
                break;
            }
        }
        if (pl.Q == 0) return pl;
        pl.parts = (L + pl.Q - 1) / pl.Q;
    }
    pl.supported = true;
    const size_t units = size_t(b) * H * pl.parts;
    pl.off_alpha = align256(units * size_t(P) * N * 4);
    pl.total = units ? pl.off_alpha + align256(units * 4) : 0;
    return pl;
}

hipError_t launch_slice_state(const void *x, const float *dt, const float *A, const void *B,
                              float *state, float *alpha_total, void *workspace, int b, int L,
                              int H, int P, int N, int G, bool bf16, const SliceStatePlan &pl,
                              hipStream_t stream) {
    if (b == 0) return hipSuccess;
    float *S = static_cast<float *>(workspace);
    float *alpha = reinterpret_cast<float *>(static_cast<char *>(workspace) + pl.off_alpha);
    if (pl.parts > 0) {
        hipError_t e;
        if (pl.fast) {
            const auto *xb = static_cast<const bf16_bits *>(x);
            const auto *Bb = static_cast<const bf16_bits *>(B);
            e = N == 64    ? launch_fast<64>(xb, dt, A, Bb, S, alpha, b, L, H, G, pl, stream)
                : N == 128 ? launch_fast<128>(xb, dt, A, Bb, S, alpha, b, L, H, G, pl, stream)
                           : launch_fast<256>(xb, dt, A, Bb, S, alpha, b, L, H, G, pl, stream);
        } else {
            e = launch_chunk_states(x, dt, A, B, S, alpha, b, L, H, P, N, G, pl.Q, bf16, stream);
        }
        if (e != hipSuccess) return e;
    }
    return launch_state_fold(S, alpha, state, alpha_total, b, H, P * N, pl.parts, stream);
}

}  // namespace ssd
