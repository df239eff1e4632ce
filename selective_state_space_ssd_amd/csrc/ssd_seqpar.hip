// ssd_seqpar.hip -- per-device pieces of the sequence-parallel (context-parallel) scan.
//
// A long sequence is split over devices (Mamba-2 article (msbhsh.com), «序列并行»):
// each device scans its slice from a zero state (ssd_chunk_scan_fwd), the devices
// exchange the pair (total decay of the slice, final state), every device folds its
// predecessors' pairs into the state entering its slice, and corrects its outputs
// by that state's contribution.  The pairs compose associatively because the state
// passing is linear (Mamba-2 article, «SSD 算法：分块和形态传递», step 3, here over
// slices instead of chunks).  With a_t = dt_t A_h and cum_t the sum of a over the
// slice up to and including t:
//   k_seq_decay   alpha = exp(cum_last) per (b, h)
//   k_seq_combine h_in[0] = init, h_in[j+1] = alpha_j h_in[j] + S_j
//   k_seq_apply   y_t += exp(cum_t) C_t . h_in   and   final += exp(cum_last) h_in
// The exchange itself (an all-gather of b H (P N + 1) floats per device) is a
// collective outside this library.
#include <algorithm>

#include "ssd_device.h"
#include "ssd_kernels.h"
#include "ssd_stage.h"

namespace ssd {

namespace {

constexpr int kSeg = 256;   // tokens per workgroup of the correction

// alpha[b, h] = exp(sum_t dt[b, t, h] A[h]): one wave per (head, batch), lanes over
// tokens, summed in a fixed order.
__global__ __launch_bounds__(64) void k_seq_decay(const float *__restrict__ dt,
                                                  const float *__restrict__ A,
                                                  float *__restrict__ alpha, int L, int H) {
    const int h = blockIdx.x, bi = blockIdx.y, lane = threadIdx.x;
    float s = 0.f;
    for (int base = lane; base < L; base += 8 * 64) {   // 8 loads in flight per lane
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int t = base + 64 * k;
            const float x = dt[(size_t(bi) * L + min(t, L - 1)) * H + h];
            v[k] = t < L ? x : 0.f;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) s += v[k];
    }
    s = wave_sum(s);
    if (lane == 0) alpha[size_t(bi) * H + h] = exp2f(s * A[h] * kLog2e);
}

// h_in[j] for the n slices, four state elements per thread.  The slices' states and
// decays are loaded 8 at a time ahead of the dependent chain.
__global__ __launch_bounds__(256) void k_seq_combine(const float *__restrict__ alpha,
                                                     const float *__restrict__ S,
                                                     const float *__restrict__ init,
                                                     float *__restrict__ h_in, int n, int bH,
                                                     int PN) {
    constexpr int kBatch = 8;
    const size_t bh = size_t(blockIdx.z) * gridDim.y + blockIdx.y;
    const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= PN) return;
    float4 h = make_float4(0.f, 0.f, 0.f, 0.f);
    if (init) h = *reinterpret_cast<const float4 *>(init + bh * PN + e);
    for (int j0 = 0; j0 < n; j0 += kBatch) {
        float4 sv[kBatch];
        float al[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int j = min(j0 + k, n - 1);
            sv[k] = *reinterpret_cast<const float4 *>(S + (size_t(j) * bH + bh) * PN + e);
            al[k] = alpha[size_t(j) * bH + bh];
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (j0 + k >= n) break;
            *reinterpret_cast<float4 *>(h_in + (size_t(j0 + k) * bH + bh) * PN + e) = h;
            h.x = al[k] * h.x + sv[k].x;
            h.y = al[k] * h.y + sv[k].y;
            h.z = al[k] * h.z + sv[k].z;
            h.w = al[k] * h.w + sv[k].w;
        }
    }
}

// One workgroup (4 waves) per (256-token segment, head, batch).  The products are
// Y^T[p][t] = sum_n h_in[p][n] C_t[n]: tiles with rows p and columns t, so each lane
// updates 4 consecutive p of one token.
// bf16 I/O: h_in rounded to bf16 as the MFMA operand (v_mfma_f32_16x16x32_bf16);
// fp32 I/O: fp32 operands (v_mfma_f32_16x16x4f32).  kMaxKq = ceil(N / 32) (bf16).
template <typename IO, int kMaxKq>
__global__ __launch_bounds__(256) void k_seq_apply(
    IO *__restrict__ y, float *__restrict__ final_state, const float *__restrict__ dt,
    const float *__restrict__ A, const IO *__restrict__ C, const float *__restrict__ h_in, int L,
    int H, int P, int N, int G) {
    constexpr bool kBF = !std::is_same_v<IO, float>;
    const int seg = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
    const int g = h / (H / G);
    const int t0 = seg * kSeg, slen = min(kSeg, L - t0);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
    const size_t bh = size_t(bi) * H + h;
    const float Al = A[h] * kLog2e;
    __shared__ float ecum[kSeg];
    __shared__ float tmp[8];

    // sum of a over the tokens before the segment (log2 domain), fixed order; the
    // loads of each batch of 8 are issued together
    float pre = 0.f;
    for (int base = 0; base < t0; base += 8 * 256) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int t = base + k * 256 + tid;
            const float x = dt[(size_t(bi) * L + min(t, t0 - 1)) * H + h];
            v[k] = t < t0 ? x : 0.f;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) pre += v[k];
    }
    pre = wave_sum(pre);
    if (lane == 0) tmp[w] = pre;
    __syncthreads();
    pre = ((tmp[0] + tmp[1]) + (tmp[2] + tmp[3])) * Al;
    const float d = tid < slen ? dt[(size_t(bi) * L + t0 + tid) * H + h] : 0.f;
    const float cs = pre + block_inclusive_scan_256(d * Al, tmp + 4);
    ecum[tid] = exp2f(cs);
    __syncthreads();

    const float *hin = h_in + bh * size_t(P) * N;
    const int ptiles = P / 16;
    const int ntb = (slen + 15) / 16;
    if constexpr (kBF) {
        // the segment's y rows are staged in LDS with whole-row 16-byte accesses; wave
        // w takes token tiles w, w + 4, ... and every p tile (4 per pass), so each C
        // row is read by one wave; h_in of the p tiles as MFMA A operands (bf16, k
        // steps of 32; n >= N read 0); results are added to the staged rows
        extern __shared__ __align__(16) unsigned char ysm[];
        bf16_bits *ys = reinterpret_cast<bf16_bits *>(ysm);   // [kSeg][P + 8]
        const int YS = P + 8, vpr = P / 8;
        bf16_bits *yseg = y + (size_t(bi) * L + t0) * size_t(H) * P + size_t(h) * P;
        for (int base = 0; base < slen * vpr; base += 8 * 256) {   // 8 row pieces in flight
            uint4 v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = min(base + k * 256 + tid, slen * vpr - 1);
                const int t = i / vpr, c = i % vpr;
                v[k] = *reinterpret_cast<const uint4 *>(yseg + size_t(t) * H * P + 8 * c);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = base + k * 256 + tid;
                if (i < slen * vpr)
                    *reinterpret_cast<uint4 *>(ys + (i / vpr) * YS + 8 * (i % vpr)) = v[k];
            }
        }
        __syncthreads();
        for (int pb = 0; pb < ptiles; pb += 4) {
            const int npt = min(4, ptiles - pb);
            // loads without branches (clamped in-range addresses, values zeroed after),
            // so they are all in flight at once
            uint4 hq[4][kMaxKq];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int kq = 0; kq < kMaxKq; ++kq) {
                    const int n0 = 32 * kq + 8 * g4;
                    const bool ok = j < npt && n0 < N;
                    const float *hr = hin + (16 * (pb + min(j, npt - 1)) + r16) * N + min(n0, N - 8);
                    const float4 h0 = *reinterpret_cast<const float4 *>(hr);
                    const float4 h1 = *reinterpret_cast<const float4 *>(hr + 4);
                    const uint4 v = make_uint4(pack_bf16x2(h0.x, h0.y), pack_bf16x2(h0.z, h0.w),
                                               pack_bf16x2(h1.x, h1.y), pack_bf16x2(h1.z, h1.w));
                    hq[j][kq] = ok ? v : make_uint4(0, 0, 0, 0);
                }
            for (int tb = w; tb < ntb; tb += 4) {
                const int t = 16 * tb + r16;
                const bool tv = t < slen;
                const bf16_bits *crow = C + ((size_t(bi) * L + t0 + (tv ? t : 0)) * G + g) * N;
                uint4 cq[kMaxKq];
#pragma unroll
                for (int kq = 0; kq < kMaxKq; ++kq) {
                    const int n0 = 32 * kq + 8 * g4;
                    const uint4 v = *reinterpret_cast<const uint4 *>(crow + min(n0, N - 8));
                    cq[kq] = n0 < N ? v : make_uint4(0, 0, 0, 0);
                }
                const float e = ecum[t];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (j >= npt) break;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kq = 0; kq < kMaxKq; ++kq)
                        acc = mfma_bf16(as_bf16x8(hq[j][kq]), as_bf16x8(cq[kq]), acc);
                    if (tv) {   // 4 consecutive p of token t in the staged row
                        uint2 *yp = reinterpret_cast<uint2 *>(ys + t * YS + 16 * (pb + j) + 4 * g4);
                        uint2 v = *yp;
                        v.x = pack_bf16x2(bf16_lo(v.x) + e * acc[0], bf16_hi(v.x) + e * acc[1]);
                        v.y = pack_bf16x2(bf16_lo(v.y) + e * acc[2], bf16_hi(v.y) + e * acc[3]);
                        *yp = v;
                    }
                }
            }
        }
        __syncthreads();
        for (int i = tid; i < slen * vpr; i += 256) {
            const int t = i / vpr, c = i % vpr;
            *reinterpret_cast<uint4 *>(yseg + size_t(t) * H * P + 8 * c) =
                *reinterpret_cast<const uint4 *>(ys + t * YS + 8 * c);
        }
    } else {
        for (int pt = w; pt < ptiles; pt += 4) {
            const int p0 = 16 * pt + 4 * g4;
            for (int tb = 0; tb < ntb; ++tb) {
                const int t = 16 * tb + r16;
                const bool tv = t < slen;
                const IO *crow = C + ((size_t(bi) * L + t0 + (tv ? t : 0)) * G + g) * N;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int k0 = 0; k0 < N; k0 += 4)
                    acc = mfma_f32(hin[(16 * pt + r16) * N + k0 + g4], to_f32<IO>(crow[k0 + g4]), acc);
                if (tv) {   // 4 consecutive p of token t, one 16-byte access
                    const float e = ecum[t];
                    IO *yp = y + ((size_t(bi) * L + t0 + t) * H + h) * P + p0;
                    float4 v = *reinterpret_cast<const float4 *>(yp);
                    v.x += e * acc[0];
                    v.y += e * acc[1];
                    v.z += e * acc[2];
                    v.w += e * acc[3];
                    *reinterpret_cast<float4 *>(yp) = v;
                }
            }
        }
    }
    if (final_state && t0 + slen == L) {   // the segment holding the last token
        const float e = ecum[slen - 1];
        float *fs = final_state + bh * size_t(P) * N;
        for (int i = tid; i < P * N; i += 256) fs[i] += e * hin[i];
    }
}

// bf16 I/O with P <= 64 (one pass over the channel tiles): one workgroup (4 waves)
// per (256-token segment, head, batch) as above, with fewer memory round trips and
// less L2 traffic.  The entering state, the dt values of the decay and the C rows of
// each wave's first token tile are loaded together at the start.  The state is
// rounded to bf16 once per workgroup into LDS (instead of once per wave from L2),
// each wave takes its MFMA A operands from there, and the segment's y rows are then
// loaded and staged over the same LDS region.  (Loaded at the start, the y rows would
// have to stay in registers across the barriers, which the compiler places in scratch
// memory.)  The C rows of the next token tile are loaded during the current one's
// products.  For N <= 128 the registers are held to 128 per lane, so that four
// workgroups fit on a CU (their LDS, 37 KB each at P = 64, does too).
template <int kMaxKq>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kMaxKq <= 4 ? 4 : 1))) void k_seq_apply_bf(
    bf16_bits *__restrict__ y, float *__restrict__ final_state, const float *__restrict__ dt,
    const float *__restrict__ A, const bf16_bits *__restrict__ C, const float *__restrict__ h_in,
    int L, int H, int P, int N, int G) {
    constexpr int NPAD = 32 * kMaxKq, HSTR = NPAD + 16;   // bf16 row stride of the state copy
    constexpr int kB = 8;                                 // 16-byte pieces in flight per thread
    const int seg = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
    const int g = h / (H / G);
    const int t0 = seg * kSeg, slen = min(kSeg, L - t0);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
    const size_t bh = size_t(bi) * H + h;
    const float Al = A[h] * kLog2e;
    __shared__ float ecum[kSeg];
    __shared__ float tmp[8];
    extern __shared__ __align__(16) unsigned char sm[];
    bf16_bits *ys = reinterpret_cast<bf16_bits *>(sm);   // [kSeg][P + 8] staged y rows
    bf16_bits *hs = ys;                                   // [P][HSTR] state copy, before them
    const int YS = P + 8, vpr = P / 8, ptiles = P / 16;
    const int ntb = (slen + 15) / 16;
    const float *hin = h_in + bh * size_t(P) * N;
    bf16_bits *yseg = y + (size_t(bi) * L + t0) * size_t(H) * P + size_t(h) * P;
    const int hpieces = P * N / 4, ypieces = slen * vpr;

    // the state in batches of kB pieces per thread; the first batch is loaded with the
    // other loads of the first round trip
    auto load_h = [&](float4 (&v)[kB], int base) {
#pragma unroll
        for (int k = 0; k < kB; ++k)
            v[k] = *reinterpret_cast<const float4 *>(hin + 4 * min(base + k * 256 + tid, hpieces - 1));
    };
    // the stores use the loads' clamped indices: a piece past the end rewrites the
    // last piece with its own value, so no store sits behind a branch
    auto store_h = [&](const float4 (&v)[kB], int base) {   // rounded to bf16 into LDS
#pragma unroll
        for (int k = 0; k < kB; ++k) {
            const int e = 4 * min(base + k * 256 + tid, hpieces - 1), pr = e / N, n = e % N;
            *reinterpret_cast<uint2 *>(hs + pr * HSTR + n) =
                make_uint2(pack_bf16x2(v[k].x, v[k].y), pack_bf16x2(v[k].z, v[k].w));
        }
    };
    float4 hv[kB];
    // C row of token 16 tb + r16, k = n (B operand) of the wave's current tile
    uint4 cq[kMaxKq];
    auto load_c = [&](int tb) {
        const int t = 16 * tb + r16;
        const bf16_bits *crow = C + ((size_t(bi) * L + t0 + (t < slen ? t : 0)) * G + g) * N;
#pragma unroll
        for (int kq = 0; kq < kMaxKq; ++kq) {
            const int n0 = 32 * kq + 8 * g4;
            const uint4 v = *reinterpret_cast<const uint4 *>(crow + min(n0, N - 8));
            cq[kq] = n0 < N ? v : make_uint4(0, 0, 0, 0);
        }
    };
    load_h(hv, 0);
    load_c(w);   // rows past the segment read row 0
    const float d = dt[(size_t(bi) * L + t0 + min(tid, slen - 1)) * H + h];
    // sum of a over the tokens before the segment (log2 domain), fixed order; the
    // loads of each batch of 8 are issued together
    float pre = 0.f;
    for (int base = 0; base < t0; base += 8 * 256) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int t = base + k * 256 + tid;
            const float x = dt[(size_t(bi) * L + min(t, t0 - 1)) * H + h];
            v[k] = t < t0 ? x : 0.f;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) pre += v[k];
    }
    pre = wave_sum(pre);
    if (lane == 0) tmp[w] = pre;
    // the state, rounded to bf16, into LDS (columns N .. NPAD-1 zero)
    store_h(hv, 0);
    for (int base = kB * 256; base < hpieces; base += kB * 256) {
        float4 v[kB];
        load_h(v, base);
        store_h(v, base);
    }
    if (NPAD > N) {
        const int pad = NPAD - N;
        for (int i = tid; i < P * pad; i += 256) hs[(i / pad) * HSTR + N + i % pad] = 0;
    }
    __syncthreads();
    pre = ((tmp[0] + tmp[1]) + (tmp[2] + tmp[3])) * Al;
    const float cs = pre + block_inclusive_scan_256(tid < slen ? d * Al : 0.f, tmp + 4);
    ecum[tid] = exp2f(cs);
    // the MFMA A operands of every channel tile (k steps of 32 over n)
    uint4 hq[4][kMaxKq];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int kq = 0; kq < kMaxKq; ++kq)
            hq[j][kq] = *reinterpret_cast<const uint4 *>(
                hs + (16 * min(j, ptiles - 1) + r16) * HSTR + 32 * kq + 8 * g4);
    __syncthreads();   // operands taken, ecum complete: the y rows go over the state copy
    {
        // at most kSeg * 64 / 8 = kB * 256 pieces of 16 bytes: one batch; a piece past
        // the end is a clamped copy of the last one
        uint4 yv[kB];
#pragma unroll
        for (int k = 0; k < kB; ++k) {
            const int i = min(k * 256 + tid, ypieces - 1);
            yv[k] = *reinterpret_cast<const uint4 *>(yseg + size_t(i / vpr) * H * P + 8 * (i % vpr));
        }
#pragma unroll
        for (int k = 0; k < kB; ++k) {
            const int i = min(k * 256 + tid, ypieces - 1);
            *reinterpret_cast<uint4 *>(ys + (i / vpr) * YS + 8 * (i % vpr)) = yv[k];
        }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < kSeg / 64; ++m) {
        const int tb = w + 4 * m;
        if (tb >= ntb) break;
        uint4 cur[kMaxKq];
#pragma unroll
        for (int kq = 0; kq < kMaxKq; ++kq) cur[kq] = cq[kq];
        if (tb + 4 < ntb) load_c(tb + 4);   // in flight during these products
        const int t = 16 * tb + r16;
        const float e = ecum[t];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j >= ptiles) break;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kq = 0; kq < kMaxKq; ++kq)
                acc = mfma_bf16(as_bf16x8(hq[j][kq]), as_bf16x8(cur[kq]), acc);
            if (t < slen) {   // 4 consecutive p of token t in the staged row
                uint2 *yp = reinterpret_cast<uint2 *>(ys + t * YS + 16 * j + 4 * g4);
                uint2 v = *yp;
                v.x = pack_bf16x2(bf16_lo(v.x) + e * acc[0], bf16_hi(v.x) + e * acc[1]);
                v.y = pack_bf16x2(bf16_lo(v.y) + e * acc[2], bf16_hi(v.y) + e * acc[3]);
                *yp = v;
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < ypieces; i += 256)
        *reinterpret_cast<uint4 *>(yseg + size_t(i / vpr) * H * P + 8 * (i % vpr)) =
            *reinterpret_cast<const uint4 *>(ys + (i / vpr) * YS + 8 * (i % vpr));
    if (final_state && t0 + slen == L) {   // the segment holding the last token
        const float ef = ecum[slen - 1];
        float *fs = final_state + bh * size_t(P) * N;
        const int PN = P * N;
        for (int base = 0; base < PN; base += 16 * 256) {   // 16 elements in flight per thread
            float fv[16], hvv[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int i = min(base + k * 256 + tid, PN - 1);
                fv[k] = fs[i];
                hvv[k] = hin[i];
            }
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int i = base + k * 256 + tid;
                if (i < PN) fs[i] = fv[k] + ef * hvv[k];
            }
        }
    }
}

// final += h_in (a slice with no tokens: its decay is 1)
__global__ __launch_bounds__(256) void k_seq_add(float *__restrict__ final_state,
                                                 const float *__restrict__ h_in, size_t count) {
    const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
    if (i < count) final_state[i] += h_in[i];
}

}  // namespace

hipError_t launch_seq_decay(const float *dt, const float *A, float *alpha, int b, int L, int H,
                            hipStream_t stream) {
    hipLaunchKernelGGL(k_seq_decay, dim3(H, b), dim3(64), 0, stream, dt, A, alpha, L, H);
    return hipGetLastError();
}

hipError_t launch_seq_combine(const float *alpha, const float *S, const float *init, float *h_in,
                              int n, int b, int H, int PN, hipStream_t stream) {
    hipLaunchKernelGGL(k_seq_combine, dim3((PN / 4 + 255) / 256, H, b), dim3(256), 0, stream,
                       alpha, S, init, h_in, n, b * H, PN);
    return hipGetLastError();
}

hipError_t launch_seq_apply(void *y, float *final_state, const float *dt, const float *A,
                            const void *C, const float *h_in, int b, int L, int H, int P, int N,
                            int G, bool bf16, hipStream_t stream) {
    if (L == 0) {
        if (!final_state) return hipSuccess;
        const size_t count = size_t(b) * H * P * N;
        hipLaunchKernelGGL(k_seq_add, dim3(unsigned((count + 255) / 256)), dim3(256), 0, stream,
                           final_state, h_in, count);
        return hipGetLastError();
    }
    const dim3 grid((L + kSeg - 1) / kSeg, H, b);
    if (!bf16) {
        hipLaunchKernelGGL((k_seq_apply<float, 1>), grid, dim3(256), 0, stream,
                           static_cast<float *>(y), final_state, dt, A,
                           static_cast<const float *>(C), h_in, L, H, P, N, G);
        return hipGetLastError();
    }
    if (P <= 64) {   // one pass over the channel tiles
        const size_t lds = std::max(size_t(kSeg) * (P + 8), size_t(P) * (32 * ((N + 31) / 32) + 16)) * 2;
        auto go1 = [&](auto kq) {
            hipLaunchKernelGGL((k_seq_apply_bf<decltype(kq)::value>), grid, dim3(256), lds, stream,
                               static_cast<bf16_bits *>(y), final_state, dt, A,
                               static_cast<const bf16_bits *>(C), h_in, L, H, P, N, G);
            return hipGetLastError();
        };
        switch ((N + 31) / 32) {
            case 1: return go1(std::integral_constant<int, 1>{});
            case 2: return go1(std::integral_constant<int, 2>{});
            case 3: return go1(std::integral_constant<int, 3>{});
            case 4: return go1(std::integral_constant<int, 4>{});
            case 5: return go1(std::integral_constant<int, 5>{});
            case 6: return go1(std::integral_constant<int, 6>{});
            case 7: return go1(std::integral_constant<int, 7>{});
            case 8: return go1(std::integral_constant<int, 8>{});
            default: return hipErrorInvalidValue;
        }
    }
    const size_t lds = size_t(kSeg) * (P + 8) * 2;   // staged y rows of one segment
    auto go = [&](auto kq) {
        if (lds > 64 * 1024) {   // above the default dynamic LDS limit
            const hipError_t e = hipFuncSetAttribute(
                reinterpret_cast<const void *>(&k_seq_apply<bf16_bits, decltype(kq)::value>),
                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL((k_seq_apply<bf16_bits, decltype(kq)::value>), grid, dim3(256), lds,
                           stream, static_cast<bf16_bits *>(y), final_state, dt, A,
                           static_cast<const bf16_bits *>(C), h_in, L, H, P, N, G);
        return hipGetLastError();
    };
    switch ((N + 31) / 32) {
        case 1: return go(std::integral_constant<int, 1>{});
        case 2: return go(std::integral_constant<int, 2>{});
        case 3: return go(std::integral_constant<int, 3>{});
        case 4: return go(std::integral_constant<int, 4>{});
        case 5: return go(std::integral_constant<int, 5>{});
        case 6: return go(std::integral_constant<int, 6>{});
        case 7: return go(std::integral_constant<int, 7>{});
        case 8: return go(std::integral_constant<int, 8>{});
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
