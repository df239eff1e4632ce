// ssd_chunk_bwd.hip -- gradients of the SSD chunked scan on gfx950.
//
// The forward map, per (b, h) with a_t = dt_t A_h and cum the in-chunk inclusive sum
// of a (Mamba-2 article (msbhsh.com), «SSD 算法：分块矩阵分解» and «SSD 算法：分块和
// 形态传递»):
//   y_t   = sum_{s<=t} (C_t . B_s) e^{cum_t - cum_s} dt_s x_s + e^{cum_t} C_t . Hin + D x_t
//   Hout  = e^{cum_end} Hin + sum_s e^{cum_end - cum_s} dt_s x_s (outer) B_s
// For upstream gradients dy and dH_final the backward pass runs
//   1. k_bwd_states: per chunk, the forward chunk state S_c (weights w_s =
//      e^{cum_end - cum_s} dt_s on x (outer) B) and the adjoint source
//      E_c = sum_t e^{cum_t} dy_t (outer) C_t, plus the chunk decay alpha_c = e^{cum_end};
//   2. k_bwd_state_pass: the state entering every chunk, Hin_{c+1} = alpha_c Hin_c + S_c,
//      and the gradient of the state leaving it, Gh_{c-1} = alpha_c Gh_c + E_c with
//      Gh_{nc-1} = dH_final; d init_state = Gh_{-1};
//   3. k_bwd_chunk: every in-chunk gradient from Hin_c and Gh_c;
//   4. k_bwd_reduce_bc / k_bwd_reduce_h: dB and dC summed over the heads of a group,
//      dA and dD over batch and chunks, in a fixed order (no atomics).
// Chunks are 64 tokens (the gradient does not depend on the chunking).  Products run
// on v_mfma_f32_16x16x4f32 with fp32 operands staged in LDS: each lane supplies one
// element of each operand, so a transposed operand is only a different address, and
// every gradient stays fp32 until dx, dB and dC are rounded to the I/O type.
//
// Gradient formulas (natural-log units; G = C B^T, W = dy x^T, Lm[t][s] =
// e^{cum_t - cum_s} for s <= t, dS = W Lm dt_s, M = G Lm dt_s, R = dS G):
//   dx_s  = sum_t M[t][s] dy_t + w_s (Gh B_s) + D dy_s
//   dB_s  = sum_t dS[t][s] C_t + w_s (x_s^T Gh)
//   dC_t  = sum_s dS[t][s] B_s + e^{cum_t} (dy_t^T Hin)
//   d dt_s (direct) = sum_t (G Lm W)[t][s] + e^{cum_end - cum_s} v_s,  v_s = x_s . (Gh B_s)
//   d cum_t = sum_s R[t][s] - sum_s R[s][t] + e^{cum_t} C_t . (dy_t^T Hin) - w_t v_t
//             (+ e^{cum_end} <Gh, Hin> + sum_s w_s v_s at the last token)
//   d a_t = sum_{tau >= t} d cum_tau;  d dt_t += A d a_t;  dA = sum dt_t d a_t;
//   dD = sum x . dy.
#include <cmath>

#include "ssd_device.h"
#include "ssd_kernels.h"
#include "ssd_stage.h"

namespace ssd {

namespace {

constexpr int QB = 64;     // tokens per backward chunk
constexpr int kPad = 4;    // fp32 LDS row padding (floats)
constexpr double kBwdCus = 256.0;   // CUs of gfx950, for the heads-per-workgroup plan

// Sum of one value per thread over the 256-thread block, in a fixed order; every
// thread returns the total.  `red` is LDS scratch of 4 floats.  Starts with a barrier.
__device__ __forceinline__ float block_sum(float v, float *red) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// Stage rows [0, QB) of a [token][W] slice (token t at src + t * tok_stride) into LDS
// as fp32, dst[t * stride + w] = scale_t * src, zero for t >= qlen.
template <typename IO>
__device__ __forceinline__ void stage_f32(const IO *__restrict__ src, size_t tok_stride, int W,
                                          int qlen, float *dst, int stride, const float *scale) {
    for (int i = threadIdx.x; i < QB * W; i += kThreads) {
        const int t = i / W, w = i % W;
        float v = 0.f;
        if (t < qlen) v = to_f32<IO>(src[size_t(t) * tok_stride + w]);
        if (scale) v *= scale[t];
        dst[t * stride + w] = v;
    }
}

__host__ __device__ constexpr size_t states_lds_bytes(int P, int N) {
    return size_t(4 * 256) * 4 + size_t(QB) * ((P + kPad) + (N + kPad)) * 4;
}

__host__ __device__ constexpr size_t chunk_lds_bytes(int P, int N) {
    return size_t(5 * 256 + 11 * QB + 8) * 4 +
           size_t(QB) * (2 * (P + kPad) + 2 * (N + kPad) + 2 * (QB + kPad)) * 4;
}

// ------------------------------------------------------------ step 1
// S[p][n] = sum_t w_t x_t[p] B_t[n] (w_t = e^{cum_end - cum_t} dt_t) and
// E[p][n] = sum_t e^{cum_t} dy_t[p] C_t[n] for one (chunk, head, batch).
template <typename IO, int P>
__global__ __launch_bounds__(kThreads) void k_bwd_states(
    const IO *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const IO *__restrict__ B, const IO *__restrict__ C, const IO *__restrict__ dy,
    float *__restrict__ S, float *__restrict__ E, float *__restrict__ alpha, int L, int H, int N,
    int G, int nc) {
    constexpr int XS = P + kPad;
    const int NS = N + kPad;
    const int c = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
    const int g = h / (H / G);
    const int t0 = c * QB, qlen = min(QB, L - t0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
    const size_t bhc = (size_t(bi) * H + h) * nc + c;

    extern __shared__ __align__(16) float sm[];
    float *acum = sm, *tmp = sm + 256, *wfw = sm + 512, *wadj = sm + 768;
    float *Xw = sm + 1024;            // [QB][XS]
    float *Bs = Xw + QB * XS;         // [QB][NS]

    const float d = chunk_cumsum(dt, A[h], bi, L, H, h, t0, qlen, acum, tmp);
    __syncthreads();
    const float aend = acum[qlen - 1];
    wfw[tid] = tid < qlen ? exp2f(aend - acum[tid]) * d : 0.f;
    wadj[tid] = tid < qlen ? exp2f(acum[tid]) : 0.f;
    if (tid == 0) alpha[bhc] = exp2f(aend);
    __syncthreads();

    const int ntn = N / 16, ntiles = (P / 16) * ntn;
    for (int pass = 0; pass < 2; ++pass) {
        const IO *u = pass == 0 ? x : dy;
        const IO *v = pass == 0 ? B : C;
        stage_f32<IO>(u + ((size_t(bi) * L + t0) * H + h) * P, size_t(H) * P, P, qlen, Xw, XS,
                      pass == 0 ? wfw : wadj);
        stage_f32<IO>(v + ((size_t(bi) * L + t0) * G + g) * N, size_t(G) * N, N, qlen, Bs, NS,
                      nullptr);
        __syncthreads();
        float *out = (pass == 0 ? S : E) + bhc * size_t(P) * N;
        for (int ti = wave; ti < ntiles; ti += 4) {
            const int pt = ti / ntn, nt = ti % ntn;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < QB; k0 += 4)
                acc = mfma_f32(Xw[(k0 + g4) * XS + 16 * pt + r16], Bs[(k0 + g4) * NS + 16 * nt + r16], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) out[(16 * pt + 4 * g4 + i) * N + 16 * nt + r16] = acc[i];
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ step 2
// In place: S becomes Hin (state entering each chunk), E becomes Gh (gradient of the
// state leaving each chunk).  Four state elements per thread.
__global__ __launch_bounds__(kThreads) void k_bwd_state_pass(
    float *__restrict__ S, float *__restrict__ E, const float *__restrict__ alpha,
    const float *__restrict__ init_state, const float *__restrict__ d_final,
    float *__restrict__ d_init, int H, int PN, int nc) {
    const size_t bh = size_t(blockIdx.z) * H + blockIdx.y;
    const int e = (blockIdx.x * kThreads + threadIdx.x) * 4;
    if (e >= PN) return;
    float4 hc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (init_state) hc = *reinterpret_cast<const float4 *>(init_state + bh * PN + e);
    for (int c = 0; c < nc; ++c) {
        float4 *p = reinterpret_cast<float4 *>(S + (bh * nc + c) * size_t(PN) + e);
        const float4 s = *p;
        *p = hc;
        const float al = alpha[bh * nc + c];
        hc.x = al * hc.x + s.x;
        hc.y = al * hc.y + s.y;
        hc.z = al * hc.z + s.z;
        hc.w = al * hc.w + s.w;
    }
    float4 gc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (d_final) gc = *reinterpret_cast<const float4 *>(d_final + bh * PN + e);
    for (int c = nc - 1; c >= 0; --c) {
        float4 *p = reinterpret_cast<float4 *>(E + (bh * nc + c) * size_t(PN) + e);
        const float4 v = *p;
        *p = gc;
        const float al = alpha[bh * nc + c];
        gc.x = al * gc.x + v.x;
        gc.y = al * gc.y + v.y;
        gc.z = al * gc.z + v.z;
        gc.w = al * gc.w + v.w;
    }
    if (d_init) *reinterpret_cast<float4 *>(d_init + bh * PN + e) = gc;
}

// ------------------------------------------------------------ step 3
// One workgroup (4 waves) per (chunk, head, batch).  Wave w owns tokens
// [16w, 16w + 16) as the output rows of every product.
template <typename IO, int P>
__global__ __launch_bounds__(kThreads) void k_bwd_chunk(
    const IO *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const IO *__restrict__ B, const IO *__restrict__ C, const float *__restrict__ D,
    const IO *__restrict__ dy, const float *__restrict__ hin, const float *__restrict__ gh,
    IO *__restrict__ dx, float *__restrict__ ddt, float *__restrict__ dBp, float *__restrict__ dCp,
    float *__restrict__ dAp, float *__restrict__ dDp, int L, int H, int N, int G, int nc) {
    constexpr int XS = P + kPad, QS = QB + kPad;
    const int NS = N + kPad;
    const int c = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
    const int g = h / (H / G);
    const int t0 = c * QB, qlen = min(QB, L - t0);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
    const size_t bhc = (size_t(bi) * H + h) * nc + c;
    const float *Hin = hin + bhc * size_t(P) * N;
    const float *Gh = gh + bhc * size_t(P) * N;

    extern __shared__ __align__(16) float sm[];
    float *acum = sm;                 // [256] log2-domain in-chunk cumsum of dt A
    float *dts = acum + 256;          // [256] dt
    float *tmp = dts + 256;           // [256] scan scratch, then d dt
    float *wsv = tmp + 256;           // [256] w_s = e^{cum_end - cum_s} dt_s
    float *eac = wsv + 256;           // [256] e^{cum_t}
    float *rowR = eac + 256;          // [QB]    sum over s of R[t][s]
    float *colR = rowR + QB;          // [4][QB] per-wave sums over t of R[t][s]
    float *colGLW = colR + 4 * QB;    // [4][QB] per-wave sums over t of (G Lm W)[t][s]
    float *vs = colGLW + 4 * QB;      // [QB]    v_s
    float *yoc = vs + QB;             // [QB]    C_t . (dy_t^T Hin)
    float *red = yoc + QB;            // [8]
    float *Xn = red + 8;              // [QB][XS] x
    float *DYn = Xn + QB * XS;        // [QB][XS] dy
    float *Bn = DYn + QB * XS;        // [QB][NS] B
    float *Cn = Bn + QB * NS;         // [QB][NS] C
    float *Mt = Cn + QB * NS;         // [QB][QS] M[t][s]
    float *St = Mt + QB * QS;         // [QB][QS] dS[t][s]

    const float Ah = A[h];
    const float d = chunk_cumsum(dt, Ah, bi, L, H, h, t0, qlen, acum, tmp);
    dts[tid] = d;
    stage_f32<IO>(x + ((size_t(bi) * L + t0) * H + h) * P, size_t(H) * P, P, qlen, Xn, XS, nullptr);
    stage_f32<IO>(dy + ((size_t(bi) * L + t0) * H + h) * P, size_t(H) * P, P, qlen, DYn, XS, nullptr);
    stage_f32<IO>(B + ((size_t(bi) * L + t0) * G + g) * N, size_t(G) * N, N, qlen, Bn, NS, nullptr);
    stage_f32<IO>(C + ((size_t(bi) * L + t0) * G + g) * N, size_t(G) * N, N, qlen, Cn, NS, nullptr);
    __syncthreads();
    const float aend = acum[qlen - 1];
    wsv[tid] = tid < qlen ? exp2f(aend - acum[tid]) * d : 0.f;
    eac[tid] = tid < qlen ? exp2f(acum[tid]) : 0.f;

    // ---- G[t][s] = C_t . B_s and W[t][s] = dy_t . x_s for this wave's rows t; then
    // M, dS and the row / column sums that feed d cum and d dt
    {
        float rsum[4] = {0.f, 0.f, 0.f, 0.f};
        for (int sb = 0; sb < QB / 16; ++sb) {
            f32x4 Gt = {0.f, 0.f, 0.f, 0.f}, Wt = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < N; k0 += 4)
                Gt = mfma_f32(Cn[(16 * w + r16) * NS + k0 + g4], Bn[(16 * sb + r16) * NS + k0 + g4], Gt);
            for (int k0 = 0; k0 < P; k0 += 4)
                Wt = mfma_f32(DYn[(16 * w + r16) * XS + k0 + g4], Xn[(16 * sb + r16) * XS + k0 + g4], Wt);
            const int s = 16 * sb + r16;
            const float ds = dts[s];
            float cr = 0.f, cglw = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * w + 4 * g4 + i;
                const float lm = (s <= t && t < qlen) ? exp2f(acum[t] - acum[s]) : 0.f;
                const float gl = Gt[i] * lm;
                const float dsv = Wt[i] * lm * ds;
                Mt[t * QS + s] = gl * ds;
                St[t * QS + s] = dsv;
                const float r = dsv * Gt[i];
                rsum[i] += r;
                cr += r;
                cglw += gl * Wt[i];
            }
            cr = group4_sum(cr);
            cglw = group4_sum(cglw);
            if (g4 == 0) {
                colR[w * QB + s] = cr;
                colGLW[w * QB + s] = cglw;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = row16_sum(rsum[i]);
            if (r16 == 0) rowR[16 * w + 4 * g4 + i] = v;
        }
    }
    __syncthreads();

    // ---- dx rows s of this wave, and v_s = x_s . U_s with U[s][p] = B_s . Gh[p]
    {
        const float Dh = D[h];
        float vpart[4] = {0.f, 0.f, 0.f, 0.f};
        for (int pb = 0; pb < P / 16; ++pb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f}, U = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < QB; k0 += 4)
                acc = mfma_f32(Mt[(k0 + g4) * QS + 16 * w + r16], DYn[(k0 + g4) * XS + 16 * pb + r16], acc);
            for (int k0 = 0; k0 < N; k0 += 4)
                U = mfma_f32(Bn[(16 * w + r16) * NS + k0 + g4], Gh[(16 * pb + r16) * N + k0 + g4], U);
            const int p = 16 * pb + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = 16 * w + 4 * g4 + i;
                vpart[i] += Xn[s * XS + p] * U[i];
                const float v = acc[i] + wsv[s] * U[i] + Dh * DYn[s * XS + p];
                if (s < qlen) dx[((size_t(bi) * L + t0 + s) * H + h) * P + p] = from_f32<IO>(v);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = row16_sum(vpart[i]);
            if (r16 == 0) vs[16 * w + 4 * g4 + i] = v;
        }
    }

    // ---- dC rows t and dB rows s of this wave (per-head partials)
    {
        float ypart[4] = {0.f, 0.f, 0.f, 0.f};
        for (int nb = 0; nb < N / 16; ++nb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f}, V = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < QB; k0 += 4)
                acc = mfma_f32(St[(16 * w + r16) * QS + k0 + g4], Bn[(k0 + g4) * NS + 16 * nb + r16], acc);
            for (int k0 = 0; k0 < P; k0 += 4)
                V = mfma_f32(DYn[(16 * w + r16) * XS + k0 + g4], Hin[(k0 + g4) * N + 16 * nb + r16], V);
            const int n = 16 * nb + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * w + 4 * g4 + i;
                ypart[i] += Cn[t * NS + n] * V[i];
                if (t < qlen) dCp[((size_t(bi) * L + t0 + t) * H + h) * N + n] = acc[i] + eac[t] * V[i];
            }
        }
        for (int nb = 0; nb < N / 16; ++nb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f}, X2 = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < QB; k0 += 4)
                acc = mfma_f32(St[(k0 + g4) * QS + 16 * w + r16], Cn[(k0 + g4) * NS + 16 * nb + r16], acc);
            for (int k0 = 0; k0 < P; k0 += 4)
                X2 = mfma_f32(Xn[(16 * w + r16) * XS + k0 + g4], Gh[(k0 + g4) * N + 16 * nb + r16], X2);
            const int n = 16 * nb + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = 16 * w + 4 * g4 + i;
                if (s < qlen) dBp[((size_t(bi) * L + t0 + s) * H + h) * N + n] = acc[i] + wsv[s] * X2[i];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = row16_sum(ypart[i]);
            if (r16 == 0) yoc[16 * w + 4 * g4 + i] = v;
        }
    }

    // ---- scalars: <Gh, Hin>, sum x . dy; then d cum -> d a -> d dt, dA
    float ghin = 0.f, xdy = 0.f;
    for (int i = tid; i < P * N; i += kThreads) ghin += Gh[i] * Hin[i];
    for (int i = tid; i < QB * P; i += kThreads) {
        const int o = (i / P) * XS + i % P;
        xdy += Xn[o] * DYn[o];
    }
    ghin = block_sum(ghin, red);   // its first barrier also publishes vs and yoc
    xdy = block_sum(xdy, red + 4);
    if (tid == 0) {
        float dend = exp2f(aend) * ghin;
        for (int s = 0; s < qlen; ++s) dend += wsv[s] * vs[s];
        float run = 0.f, dA = 0.f;
        for (int t = qlen - 1; t >= 0; --t) {
            const float cr = (colR[t] + colR[QB + t]) + (colR[2 * QB + t] + colR[3 * QB + t]);
            float dc = rowR[t] - cr + eac[t] * yoc[t] - wsv[t] * vs[t];
            if (t == qlen - 1) dc += dend;
            run += dc;
            const float glw = (colGLW[t] + colGLW[QB + t]) + (colGLW[2 * QB + t] + colGLW[3 * QB + t]);
            tmp[t] = glw + exp2f(aend - acum[t]) * vs[t] + Ah * run;
            dA += dts[t] * run;
        }
        dAp[bhc] = dA;
        dDp[bhc] = xdy;
    }
    __syncthreads();
    if (tid < qlen) ddt[(size_t(bi) * L + t0 + tid) * H + h] = tmp[tid];
}

// ------------------------------------------------------------ step 4
// dB[row, g, n] = sum over the nparts / G parts of group g of dBp[row, part, n] (parts
// are heads, or blocks of heads); dC alike.
template <typename IO>
__global__ __launch_bounds__(kThreads) void k_bwd_reduce_bc(
    const float *__restrict__ dBp, const float *__restrict__ dCp, IO *__restrict__ dB,
    IO *__restrict__ dC, size_t rows, int nparts, int G, int N) {
    const size_t i = size_t(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= rows * G * N) return;
    const int n = int(i % N);
    const int g = int((i / N) % G);
    const size_t row = i / (size_t(G) * N);
    const int ppg = nparts / G;
    float sb = 0.f, sc = 0.f;
    for (int k = 0; k < ppg; ++k) {
        const size_t src = (row * nparts + g * ppg + k) * N + n;
        sb += dBp[src];
        sc += dCp[src];
    }
    dB[i] = from_f32<IO>(sb);
    dC[i] = from_f32<IO>(sc);
}

// dA[h] = sum over (b, c) of dAp[b, h, c]; dD alike.
__global__ __launch_bounds__(kThreads) void k_bwd_reduce_h(
    const float *__restrict__ dAp, const float *__restrict__ dDp, float *__restrict__ dA,
    float *__restrict__ dD, int b, int H, int nc) {
    const int h = blockIdx.x;
    float sa = 0.f, sd = 0.f;
    for (int i = threadIdx.x; i < b * nc; i += kThreads) {
        const size_t src = (size_t(i / nc) * H + h) * nc + i % nc;
        sa += dAp[src];
        sd += dDp[src];
    }
    __shared__ float red[8];
    sa = block_sum(sa, red);
    sd = block_sum(sd, red + 4);
    if (threadIdx.x == 0) {
        dA[h] = sa;
        dD[h] = sd;
    }
}

template <typename IO, int P>
hipError_t launch_bwd_p(const ChunkScanBwdArgs &a, const ChunkScanBwdPlan &pl, hipStream_t stream) {
    char *ws = static_cast<char *>(a.workspace);
    float *S = reinterpret_cast<float *>(ws + pl.off_hin);
    float *E = reinterpret_cast<float *>(ws + pl.off_gh);
    float *alpha = reinterpret_cast<float *>(ws + pl.off_alpha);
    float *dBp = reinterpret_cast<float *>(ws + pl.off_dbp);
    float *dCp = reinterpret_cast<float *>(ws + pl.off_dcp);
    float *dAp = reinterpret_cast<float *>(ws + pl.off_dap);
    float *dDp = reinterpret_cast<float *>(ws + pl.off_ddp);
    const IO *x = static_cast<const IO *>(a.x), *B = static_cast<const IO *>(a.B);
    const IO *C = static_cast<const IO *>(a.C), *dy = static_cast<const IO *>(a.dy);
    const dim3 grid(pl.nc, a.H, a.b);
    hipError_t e;

    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_bwd_states<IO, P>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(pl.lds_states));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_bwd_states<IO, P>), grid, dim3(kThreads), pl.lds_states, stream, x, a.dt,
                       a.A, B, C, dy, S, E, alpha, a.L, a.H, a.N, a.G, pl.nc);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    const int PN = P * a.N;
    hipLaunchKernelGGL(k_bwd_state_pass, dim3((PN / 4 + kThreads - 1) / kThreads, a.H, a.b),
                       dim3(kThreads), 0, stream, S, E, alpha, a.init_state, a.d_final, a.d_init,
                       a.H, PN, pl.nc);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_bwd_chunk<IO, P>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(pl.lds_chunk));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_bwd_chunk<IO, P>), grid, dim3(kThreads), pl.lds_chunk, stream, x, a.dt,
                       a.A, B, C, a.D, dy, S, E, static_cast<IO *>(a.dx), a.ddt, dBp, dCp, dAp,
                       dDp, a.L, a.H, a.N, a.G, pl.nc);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    return launch_bwd_reduce(a, pl, stream);
}

template <typename IO>
hipError_t launch_bwd_io(const ChunkScanBwdArgs &a, const ChunkScanBwdPlan &pl, hipStream_t stream) {
    switch (a.P) {
        case 32: return launch_bwd_p<IO, 32>(a, pl, stream);
        case 64: return launch_bwd_p<IO, 64>(a, pl, stream);
        default: return hipErrorInvalidValue;
    }
}

size_t align256b(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

ChunkScanBwdPlan plan_chunk_scan_bwd(int b, int L, int H, int P, int N, int G, bool bf16) {
    ChunkScanBwdPlan pl;
    if (b <= 0 || L <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G) return pl;
    pl.nc = (L + QB - 1) / QB;
    const size_t units = size_t(b) * H * pl.nc;
    pl.bf16_path = bf16 && P == 64 && chunk_bwd_bf16_lds(N) != 0;
    if (pl.bf16_path) {
        // heads per workgroup (a divisor of the group size): the chunk kernel runs one
        // workgroup per CU, and a workgroup costs about hb + 0.75 head times (staging B
        // and C and the C B^T tiles, shared by its heads, take 0.75), so the launch
        // takes ceil(workgroups / CUs) (hb + 0.75) head times; the CU count is that of
        // gfx950 (256), so that the plan depends on the shape only.  Ties go to the
        // larger block (fewer dB / dC partials).  Measured at the L = 2048 layer (b 4,
        // H 80): 8 heads 460 us per call, 10: 452, 16: 471, 20: 433, 40: 424.
        const int hpg = H / G;
        double best = 0.0;
        for (int d = 1; d <= hpg; ++d) {
            if (hpg % d != 0) continue;
            const double wgs = double(pl.nc) * double(H / d) * double(b);
            const double t = std::ceil(wgs / kBwdCus) * (d + 0.75);
            if (d == 1 || t <= best) {
                best = t;
                pl.hb = d;
            }
        }
        pl.nparts = H / pl.hb;
        const size_t st = units * size_t(P) * N * 2;
        const size_t part = size_t(b) * L * pl.nparts * N * 4;
        pl.off_hin = 0;
        pl.off_gh = align256b(st);
        pl.off_dbp = pl.off_gh + align256b(st);
        pl.off_dcp = pl.off_dbp + align256b(part);
        pl.off_dap = pl.off_dcp + align256b(part);
        pl.off_ddp = pl.off_dap + align256b(units * 4);
        pl.total = pl.off_ddp + align256b(units * 4);
        pl.lds_chunk = chunk_bwd_bf16_lds(N);
        pl.supported = H <= 65535 && b <= 65535 && pl.lds_chunk <= kMaxLds;
        return pl;
    }
    pl.nparts = H;
    const size_t st = units * size_t(P) * N * 4;
    const size_t part = size_t(b) * L * H * N * 4;
    pl.off_hin = 0;
    pl.off_gh = align256b(st);
    pl.off_alpha = pl.off_gh + align256b(st);
    pl.off_dbp = pl.off_alpha + align256b(units * 4);
    pl.off_dcp = pl.off_dbp + align256b(part);
    pl.off_dap = pl.off_dcp + align256b(part);
    pl.off_ddp = pl.off_dap + align256b(units * 4);
    pl.total = pl.off_ddp + align256b(units * 4);
    pl.lds_states = states_lds_bytes(P, N);
    pl.lds_chunk = chunk_lds_bytes(P, N);
    pl.supported = (P == 32 || P == 64) && N % 16 == 0 && N >= 16 && H <= 65535 &&
                   b <= 65535 && pl.lds_chunk <= kMaxLds && pl.lds_states <= kMaxLds;
    return pl;
}

hipError_t launch_bwd_reduce(const ChunkScanBwdArgs &a, const ChunkScanBwdPlan &pl,
                             hipStream_t stream) {
    char *ws = static_cast<char *>(a.workspace);
    const float *dBp = reinterpret_cast<const float *>(ws + pl.off_dbp);
    const float *dCp = reinterpret_cast<const float *>(ws + pl.off_dcp);
    const float *dAp = reinterpret_cast<const float *>(ws + pl.off_dap);
    const float *dDp = reinterpret_cast<const float *>(ws + pl.off_ddp);
    const size_t rows = size_t(a.b) * a.L;
    const size_t cnt = rows * a.G * a.N;
    const dim3 grid(unsigned((cnt + kThreads - 1) / kThreads));
    if (a.bf16)
        hipLaunchKernelGGL((k_bwd_reduce_bc<bf16_bits>), grid, dim3(kThreads), 0, stream, dBp, dCp,
                           static_cast<bf16_bits *>(a.dB), static_cast<bf16_bits *>(a.dC), rows,
                           pl.nparts, a.G, a.N);
    else
        hipLaunchKernelGGL((k_bwd_reduce_bc<float>), grid, dim3(kThreads), 0, stream, dBp, dCp,
                           static_cast<float *>(a.dB), static_cast<float *>(a.dC), rows,
                           pl.nparts, a.G, a.N);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_bwd_reduce_h, dim3(a.H), dim3(kThreads), 0, stream, dAp, dDp, a.dA, a.dD,
                       a.b, a.H, pl.nc);
    return hipGetLastError();
}

hipError_t launch_chunk_scan_bwd(const ChunkScanBwdArgs &a, const ChunkScanBwdPlan &pl,
                                 hipStream_t stream) {
    if (pl.bf16_path) {
        const hipError_t e = launch_chunk_scan_bwd_bf16(a, pl, stream);
        if (e != hipSuccess) return e;
        return launch_bwd_reduce(a, pl, stream);
    }
    if (a.bf16) return launch_bwd_io<bf16_bits>(a, pl, stream);
    return launch_bwd_io<float>(a, pl, stream);
}

}  // namespace ssd
