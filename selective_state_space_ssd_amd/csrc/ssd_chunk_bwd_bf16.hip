// ssd_chunk_bwd_bf16.hip -- gradients of the SSD chunked scan, bf16 I/O, head
// dimension 64, state size 64 or 128: the bf16 matrix-core path.
//
// Same mathematics as ssd_chunk_bwd.hip (the chunked decomposition of the Mamba-2
// article (msbhsh.com), «SSD 算法：分块矩阵分解» and «SSD 算法：分块和形态传递», run in
// reverse; intermediate states recomputed rather than stored, "另辟蹊径--Mamba介绍",
// «Hardware-aware Algorithm»), organised for fewer HBM bytes:
//
//   k_bwd_chain    one workgroup per (direction, head, batch) walks the 64-token chunks
//                  in order (forward) or in reverse, keeping the P x N state in MFMA
//                  accumulators: the forward walk writes the state entering each chunk,
//                  Hin_c; the reverse walk writes the gradient of the state leaving it,
//                  Gh_c, and finally d init_state.  Each chunk's contribution
//                  (sum_t w_t x_t (outer) B_t, or sum_t e^{cum_t} dy_t (outer) C_t) is
//                  one bf16 MFMA product added onto the decayed state, so no per-chunk
//                  state ever goes to HBM in fp32.  The states are stored in bf16, in
//                  the layouts the next kernel reads as MFMA operands.
//   k_bwd_chunk_bf one workgroup per (chunk, block of up to 8 heads of one group,
//                  batch): C B^T once per block, then per head the score tiles, dx,
//                  and the head's dB / dC contributions, which stay in registers across
//                  the block so only one fp32 partial per block reaches HBM.
//
// bf16 rounding happens where an MFMA operand is not an input: the decay-weighted x
// and dy of the chain, the masked score matrices M and dS, and the states Hin, Gh.
// Every sum runs in fp32; the row and column sums that feed d dt use the fp32 scores.
#include "ssd_device.h"
#include "ssd_kernels.h"
#include "ssd_stage.h"

namespace ssd {

namespace {

constexpr int QB = 64;     // tokens per chunk
constexpr int HP = 64;     // head dimension P of this path
constexpr int RS = 80;     // LDS row stride (bf16) of rows of 64 elements

__device__ __forceinline__ bf16x8 lds16(const bf16_bits *p) {
    return as_bf16x8(*reinterpret_cast<const uint4 *>(p));
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0, 0, 0, 0); }

// ------------------------------------------------------------ state chains
// dir 0: Hin_c for c = 0 .. nc-1 (HinT, [n][p] per chunk).
// dir 1: Gh_c for c = nc-1 .. 0 (GhT [n][p] and Gh [p][n]), then d_init.
// The state is held twice in the reverse walk, as tiles with rows p (written as GhT)
// and with rows n (written as Gh), so every store writes 4 consecutive values.
template <int N>
__global__ __launch_bounds__(kThreads) void k_bwd_chain(
    const bf16_bits *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const bf16_bits *__restrict__ B, const bf16_bits *__restrict__ C,
    const bf16_bits *__restrict__ dy, const float *__restrict__ init_state,
    const float *__restrict__ d_final, bf16_bits *__restrict__ hinT, bf16_bits *__restrict__ ghT,
    bf16_bits *__restrict__ ghN, float *__restrict__ d_init, int L, int H, int G, int nc) {
    constexpr int NT = N / 16, NTW = NT / 4, NG = N / 8, PN = HP * N;
    const int dir = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
    const int g = h / (H / G);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
    const size_t bh = size_t(bi) * H + h;
    const float Ah = A[h];

    __shared__ __align__(16) bf16_bits AT[HP * RS];    // [p][t] weighted x or dy
    __shared__ __align__(16) bf16_bits VT[N * RS];     // [n][t] B or C
    __shared__ float wts[QB];
    __shared__ float al_sh;

    const bf16_bits *u = dir == 0 ? x : dy;
    const bf16_bits *v = dir == 0 ? B : C;

    // state tiles: rows p (tile nt: p = 16w + 4g4 + i, n = 16nt + r16)
    f32x4 accP[NT];
    // reverse walk only: rows n (tile j, pt: n = 16(NTW w + j) + 4g4 + i, p = 16pt + r16)
    f32x4 accN[NTW][4];
    {
        const float *s0 = dir == 0 ? init_state : d_final;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                accP[nt][i] = s0 ? s0[bh * PN + (16 * w + 4 * g4 + i) * N + 16 * nt + r16] : 0.f;
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
                if (dir == 1 && d_final)
                    q = *reinterpret_cast<const float4 *>(
                        d_final + bh * PN + (16 * pt + r16) * N + 16 * (NTW * w + j) + 4 * g4);
                accN[j][pt] = {q.x, q.y, q.z, q.w};
            }
    }

    // prefetch registers: u rows (token pair tpu, p group pgu), v rows (2 items)
    const int tpu = tid >> 3, pgu = tid & 7;
    uint4 ua, ub, va[2], vb[2];
    float dreg = 0.f;
    auto load = [&](int c) {
        const int t0 = c * QB, qlen = min(QB, L - t0);
        const int ta = 2 * tpu, tb = ta + 1;
        ua = ta < qlen ? *reinterpret_cast<const uint4 *>(u + ((size_t(bi) * L + t0 + ta) * H + h) * HP + 8 * pgu) : zero4();
        ub = tb < qlen ? *reinterpret_cast<const uint4 *>(u + ((size_t(bi) * L + t0 + tb) * H + h) * HP + 8 * pgu) : zero4();
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int item = tid + k * kThreads;
            const int tp = item / NG, ng = item % NG;
            const int t = 2 * tp;
            va[k] = (item < 32 * NG && t < qlen)
                        ? *reinterpret_cast<const uint4 *>(v + ((size_t(bi) * L + t0 + t) * G + g) * N + 8 * ng)
                        : zero4();
            vb[k] = (item < 32 * NG && t + 1 < qlen)
                        ? *reinterpret_cast<const uint4 *>(v + ((size_t(bi) * L + t0 + t + 1) * G + g) * N + 8 * ng)
                        : zero4();
        }
        dreg = lane < qlen ? dt[(size_t(bi) * L + t0 + lane) * H + h] : 0.f;
    };

    load(dir == 0 ? 0 : nc - 1);
    for (int step = 0; step < nc; ++step) {
        const int c = dir == 0 ? step : nc - 1 - step;
        const int qlen = min(QB, L - c * QB);
        if (w == 0) {
            const float cs = wave_inclusive_scan(lane < qlen ? dreg * Ah * kLog2e : 0.f);
            const float aend = __shfl(cs, qlen - 1, 64);
            wts[lane] = lane < qlen ? (dir == 0 ? exp2f(aend - cs) * dreg : exp2f(cs)) : 0.f;
            if (lane == 0) al_sh = exp2f(aend);
        }
        __syncthreads();
        const float al = al_sh;
        {   // stage the weighted u transposed and v transposed, token pairs
            const float wa = wts[2 * tpu], wb = wts[2 * tpu + 1];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t ea = (&ua.x)[j >> 1], eb = (&ub.x)[j >> 1];
                const float fa = (j & 1) ? bf16_hi(ea) : bf16_lo(ea);
                const float fb = (j & 1) ? bf16_hi(eb) : bf16_lo(eb);
                *reinterpret_cast<uint32_t *>(AT + (8 * pgu + j) * RS + 2 * tpu) = pack_bf16x2(fa * wa, fb * wb);
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int item = tid + k * kThreads;
                if (item < 32 * NG) {
                    const int tp = item / NG, ng = item % NG;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const uint32_t ea = (&va[k].x)[j >> 1], eb = (&vb[k].x)[j >> 1];
                        const uint32_t lo = (j & 1) ? (ea >> 16) : (ea & 0xffffu);
                        const uint32_t hi = (j & 1) ? (eb & 0xffff0000u) : (eb << 16);
                        *reinterpret_cast<uint32_t *>(VT + (8 * ng + j) * RS + 2 * tp) = lo | hi;
                    }
                }
            }
        }
        if (step + 1 < nc) load(dir == 0 ? c + 1 : c - 1);
        __syncthreads();

        // store the state (entering chunk c forward, leaving chunk c in reverse)
        const size_t so = (bh * nc + c) * size_t(PN);
        bf16_bits *dstT = dir == 0 ? hinT : ghT;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            *reinterpret_cast<uint2 *>(dstT + so + (16 * nt + r16) * HP + 16 * w + 4 * g4) =
                make_uint2(pack_bf16x2(accP[nt][0], accP[nt][1]), pack_bf16x2(accP[nt][2], accP[nt][3]));
        if (dir == 1) {
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int pt = 0; pt < 4; ++pt)
                    *reinterpret_cast<uint2 *>(ghN + so + (16 * pt + r16) * N + 16 * (NTW * w + j) + 4 * g4) =
                        make_uint2(pack_bf16x2(accN[j][pt][0], accN[j][pt][1]),
                                   pack_bf16x2(accN[j][pt][2], accN[j][pt][3]));
        }

        // state <- al * state + (this chunk's contribution)
        bf16x8 a0 = lds16(AT + (16 * w + r16) * RS + 8 * g4);
        bf16x8 a1 = lds16(AT + (16 * w + r16) * RS + 32 + 8 * g4);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 s = accP[nt] * al;
            s = mfma_bf16(a0, lds16(VT + (16 * nt + r16) * RS + 8 * g4), s);
            accP[nt] = mfma_bf16(a1, lds16(VT + (16 * nt + r16) * RS + 32 + 8 * g4), s);
        }
        if (dir == 1) {
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int nt = NTW * w + j;
                const bf16x8 c0 = lds16(VT + (16 * nt + r16) * RS + 8 * g4);
                const bf16x8 c1 = lds16(VT + (16 * nt + r16) * RS + 32 + 8 * g4);
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    f32x4 s = accN[j][pt] * al;
                    s = mfma_bf16(c0, lds16(AT + (16 * pt + r16) * RS + 8 * g4), s);
                    accN[j][pt] = mfma_bf16(c1, lds16(AT + (16 * pt + r16) * RS + 32 + 8 * g4), s);
                }
            }
        }
    }
    if (dir == 1 && d_init) {
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
                *reinterpret_cast<float4 *>(d_init + bh * PN + (16 * pt + r16) * N + 16 * (NTW * w + j) + 4 * g4) =
                    make_float4(accN[j][pt][0], accN[j][pt][1], accN[j][pt][2], accN[j][pt][3]);
    }
}

// ------------------------------------------------------------ in-chunk gradients
template <int N>
struct ChunkLds {
    static constexpr int NS = N + 16;                      // row stride of [t][n]
    static constexpr int kScalars = 4 * QB + QB + 4 * 4 * QB + 8;
    static constexpr size_t off_Bn = size_t(kScalars) * 4;
    static constexpr size_t off_Cn = off_Bn + size_t(QB) * NS * 2;
    static constexpr size_t off_BT = off_Cn + size_t(QB) * NS * 2;
    static constexpr size_t off_CT = off_BT + size_t(N) * RS * 2;
    static constexpr size_t off_X = off_CT + size_t(N) * RS * 2;
    static constexpr size_t off_DY = off_X + size_t(QB) * RS * 2;
    static constexpr size_t off_DYT = off_DY + size_t(QB) * RS * 2;
    static constexpr size_t off_MT = off_DYT + size_t(HP) * RS * 2;
    static constexpr size_t off_DS = off_MT + size_t(QB) * RS * 2;
    static constexpr size_t off_DST = off_DS + size_t(QB) * RS * 2;
    static constexpr size_t bytes = off_DST + size_t(QB) * RS * 2;
};

template <int N>
__global__ __launch_bounds__(kThreads) void k_bwd_chunk_bf(
    const bf16_bits *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const bf16_bits *__restrict__ B, const bf16_bits *__restrict__ C, const float *__restrict__ D,
    const bf16_bits *__restrict__ dy, const bf16_bits *__restrict__ hinT,
    const bf16_bits *__restrict__ ghT, const bf16_bits *__restrict__ ghN,
    bf16_bits *__restrict__ dx, float *__restrict__ ddt, float *__restrict__ dBp,
    float *__restrict__ dCp, float *__restrict__ dAp, float *__restrict__ dDp, int L, int H,
    int G, int nc, int HB) {
    using Lay = ChunkLds<N>;
    constexpr int NS = Lay::NS, NT = N / 16, NTW = NT / 4, KN = N / 32, NG = N / 8, PN = HP * N;
    const int c = blockIdx.x, hbk = blockIdx.y, bi = blockIdx.z;
    const int nblk = gridDim.y;
    const int h0 = hbk * HB;
    const int g = h0 / (H / G);
    const int t0 = c * QB, qlen = min(QB, L - t0);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r16 = lane & 15, g4 = lane >> 4;

    extern __shared__ __align__(16) unsigned char smem[];
    float *acum = reinterpret_cast<float *>(smem);   // [QB]
    float *dts = acum + QB;                          // [QB]
    float *wsv = dts + QB;                           // [QB] e^{cum_end - cum_s} dt_s
    float *eac = wsv + QB;                           // [QB] e^{cum_t}
    float *rowR = eac + QB;                          // [QB]
    float *colR = rowR + QB;                         // [4][QB]
    float *colGLW = colR + 4 * QB;                   // [4][QB]
    float *vsp = colGLW + 4 * QB;                    // [4][QB] per-wave parts of v_s
    float *yocp = vsp + 4 * QB;                      // [4][QB] per-wave parts of C_t . V_t
    float *red = yocp + 4 * QB;                      // [8]
    bf16_bits *Bn = reinterpret_cast<bf16_bits *>(smem + Lay::off_Bn);     // [s][n]
    bf16_bits *Cn = reinterpret_cast<bf16_bits *>(smem + Lay::off_Cn);     // [t][n]
    bf16_bits *BT = reinterpret_cast<bf16_bits *>(smem + Lay::off_BT);     // [n][s]
    bf16_bits *CT = reinterpret_cast<bf16_bits *>(smem + Lay::off_CT);     // [n][t]
    bf16_bits *Xn = reinterpret_cast<bf16_bits *>(smem + Lay::off_X);      // [s][p]
    bf16_bits *DYn = reinterpret_cast<bf16_bits *>(smem + Lay::off_DY);    // [t][p]
    bf16_bits *DYT = reinterpret_cast<bf16_bits *>(smem + Lay::off_DYT);   // [p][t]
    bf16_bits *MT = reinterpret_cast<bf16_bits *>(smem + Lay::off_MT);     // [s][t]
    bf16_bits *DS = reinterpret_cast<bf16_bits *>(smem + Lay::off_DS);     // [t][s]
    bf16_bits *DST = reinterpret_cast<bf16_bits *>(smem + Lay::off_DST);   // [s][t]

    // x / dy of one head: token pair tpu, p group pgu
    const int tpu = tid >> 3, pgu = tid & 7;
    uint4 xa, xb, ya, yb;
    auto load_xy = [&](int h) {
        const int ta = 2 * tpu, tb = ta + 1;
        const size_t ra = ((size_t(bi) * L + t0 + ta) * H + h) * HP + 8 * pgu;
        const size_t rb = ra + size_t(H) * HP;
        xa = ta < qlen ? *reinterpret_cast<const uint4 *>(x + ra) : zero4();
        xb = tb < qlen ? *reinterpret_cast<const uint4 *>(x + rb) : zero4();
        ya = ta < qlen ? *reinterpret_cast<const uint4 *>(dy + ra) : zero4();
        yb = tb < qlen ? *reinterpret_cast<const uint4 *>(dy + rb) : zero4();
    };
    load_xy(h0);

    // B and C of the group, natural and transposed
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int item = tid + k * kThreads;
        if (item < 32 * NG) {
            const int tp = item / NG, ng = item % NG, t = 2 * tp;
            const size_t r0 = ((size_t(bi) * L + t0 + t) * G + g) * N + 8 * ng;
            const size_t r1 = r0 + size_t(G) * N;
            const uint4 b0 = t < qlen ? *reinterpret_cast<const uint4 *>(B + r0) : zero4();
            const uint4 b1 = t + 1 < qlen ? *reinterpret_cast<const uint4 *>(B + r1) : zero4();
            const uint4 c0 = t < qlen ? *reinterpret_cast<const uint4 *>(C + r0) : zero4();
            const uint4 c1 = t + 1 < qlen ? *reinterpret_cast<const uint4 *>(C + r1) : zero4();
            *reinterpret_cast<uint4 *>(Bn + t * NS + 8 * ng) = b0;
            *reinterpret_cast<uint4 *>(Bn + (t + 1) * NS + 8 * ng) = b1;
            *reinterpret_cast<uint4 *>(Cn + t * NS + 8 * ng) = c0;
            *reinterpret_cast<uint4 *>(Cn + (t + 1) * NS + 8 * ng) = c1;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int sh = 16 * (j & 1);
                const uint32_t bl = ((&b0.x)[j >> 1] >> sh) & 0xffffu, bh = ((&b1.x)[j >> 1] >> sh) & 0xffffu;
                const uint32_t cl = ((&c0.x)[j >> 1] >> sh) & 0xffffu, ch = ((&c1.x)[j >> 1] >> sh) & 0xffffu;
                *reinterpret_cast<uint32_t *>(BT + (8 * ng + j) * RS + t) = bl | (bh << 16);
                *reinterpret_cast<uint32_t *>(CT + (8 * ng + j) * RS + t) = cl | (ch << 16);
            }
        }
    }
    __syncthreads();

    // G[t][s] = C_t . B_s for this wave's rows t, all s (shared by the heads)
    f32x4 Gt[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kq = 0; kq < KN; ++kq)
            acc = mfma_bf16(lds16(Cn + (16 * w + r16) * NS + 32 * kq + 8 * g4),
                            lds16(Bn + (16 * sb + r16) * NS + 32 * kq + 8 * g4), acc);
        Gt[sb] = acc;
    }

    f32x4 accB[NTW][4], accC[NTW][4];
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            accB[j][k] = {0.f, 0.f, 0.f, 0.f};
            accC[j][k] = {0.f, 0.f, 0.f, 0.f};
        }

    for (int hh = 0; hh < HB; ++hh) {
        const int h = h0 + hh;
        const size_t bhc = (size_t(bi) * H + h) * nc + c;
        const size_t so = bhc * size_t(PN);
        // states of this head as MFMA A operands (rows owned by this wave)
        uint4 ghp[KN], ght[NTW][2], hnt[NTW][2];
#pragma unroll
        for (int kq = 0; kq < KN; ++kq)
            ghp[kq] = *reinterpret_cast<const uint4 *>(ghN + so + (16 * w + r16) * N + 32 * kq + 8 * g4);
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int kp = 0; kp < 2; ++kp) {
                const size_t o = so + (16 * (NTW * w + j) + r16) * HP + 32 * kp + 8 * g4;
                ght[j][kp] = *reinterpret_cast<const uint4 *>(ghT + o);
                hnt[j][kp] = *reinterpret_cast<const uint4 *>(hinT + o);
            }
        const float dreg = lane < qlen ? dt[(size_t(bi) * L + t0 + lane) * H + h] : 0.f;
        const float Ah = A[h];
        const float cs = wave_inclusive_scan(lane < qlen ? dreg * Ah * kLog2e : 0.f);
        const float aend = __shfl(cs, qlen - 1, 64);
        if (w == 0) {
            const bool valid = lane < qlen;
            acum[lane] = valid ? cs : 0.f;
            dts[lane] = dreg;
            wsv[lane] = valid ? exp2f(aend - cs) * dreg : 0.f;
            eac[lane] = valid ? exp2f(cs) : 0.f;
        }
        // stage x, dy (natural) and dy transposed
        *reinterpret_cast<uint4 *>(Xn + (2 * tpu) * RS + 8 * pgu) = xa;
        *reinterpret_cast<uint4 *>(Xn + (2 * tpu + 1) * RS + 8 * pgu) = xb;
        *reinterpret_cast<uint4 *>(DYn + (2 * tpu) * RS + 8 * pgu) = ya;
        *reinterpret_cast<uint4 *>(DYn + (2 * tpu + 1) * RS + 8 * pgu) = yb;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int sh = 16 * (j & 1);
            const uint32_t lo = ((&ya.x)[j >> 1] >> sh) & 0xffffu, hi = ((&yb.x)[j >> 1] >> sh) & 0xffffu;
            *reinterpret_cast<uint32_t *>(DYT + (8 * pgu + j) * RS + 2 * tpu) = lo | (hi << 16);
        }
        if (hh + 1 < HB) load_xy(h + 1);
        __syncthreads();

        // ---- scores of this wave's rows t: W = dy x^T, then M, dS and the sums
        {
            float rsum[4] = {0.f, 0.f, 0.f, 0.f};
            const bf16x8 d0 = lds16(DYn + (16 * w + r16) * RS + 8 * g4);
            const bf16x8 d1 = lds16(DYn + (16 * w + r16) * RS + 32 + 8 * g4);
            float at[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) at[i] = acum[16 * w + 4 * g4 + i];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                f32x4 Wt = {0.f, 0.f, 0.f, 0.f};
                Wt = mfma_bf16(d0, lds16(Xn + (16 * sb + r16) * RS + 8 * g4), Wt);
                Wt = mfma_bf16(d1, lds16(Xn + (16 * sb + r16) * RS + 32 + 8 * g4), Wt);
                const int s = 16 * sb + r16;
                const float ds = dts[s], as = acum[s];
                float mv[4], sv[4], cr = 0.f, cglw = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * w + 4 * g4 + i;
                    const float lm = (s <= t && t < qlen) ? exp2f(at[i] - as) : 0.f;
                    const float gl = Gt[sb][i] * lm;
                    mv[i] = gl * ds;
                    sv[i] = Wt[i] * lm * ds;
                    const float r = sv[i] * Gt[sb][i];
                    rsum[i] += r;
                    cr += r;
                    cglw += gl * Wt[i];
                    DS[t * RS + s] = f32_to_bf16(sv[i]);
                }
                *reinterpret_cast<uint2 *>(MT + s * RS + 16 * w + 4 * g4) =
                    make_uint2(pack_bf16x2(mv[0], mv[1]), pack_bf16x2(mv[2], mv[3]));
                *reinterpret_cast<uint2 *>(DST + s * RS + 16 * w + 4 * g4) =
                    make_uint2(pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3]));
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

        // ---- dx^T[p][s] (rows p of this wave) and U^T[p][s] = Gh[p] . B_s
        {
            const float Dh = D[h];
            const bf16x8 e0 = lds16(DYT + (16 * w + r16) * RS + 8 * g4);
            const bf16x8 e1 = lds16(DYT + (16 * w + r16) * RS + 32 + 8 * g4);
            const int p0 = 16 * w + 4 * g4;
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                const int s = 16 * sb + r16;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f}, U = {0.f, 0.f, 0.f, 0.f};
                acc = mfma_bf16(e0, lds16(MT + s * RS + 8 * g4), acc);
                acc = mfma_bf16(e1, lds16(MT + s * RS + 32 + 8 * g4), acc);
#pragma unroll
                for (int kq = 0; kq < KN; ++kq)
                    U = mfma_bf16(as_bf16x8(ghp[kq]), lds16(Bn + s * NS + 32 * kq + 8 * g4), U);
                const uint2 d4 = *reinterpret_cast<const uint2 *>(DYn + s * RS + p0);
                const uint2 x4 = *reinterpret_cast<const uint2 *>(Xn + s * RS + p0);
                const float dyv[4] = {bf16_lo(d4.x), bf16_hi(d4.x), bf16_lo(d4.y), bf16_hi(d4.y)};
                const float xv[4] = {bf16_lo(x4.x), bf16_hi(x4.x), bf16_lo(x4.y), bf16_hi(x4.y)};
                const float ws = wsv[s];
                float o[4], vp = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    o[i] = acc[i] + ws * U[i] + Dh * dyv[i];
                    vp += xv[i] * U[i];
                }
                if (s < qlen)
                    *reinterpret_cast<uint2 *>(dx + ((size_t(bi) * L + t0 + s) * H + h) * HP + p0) =
                        make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
                vp = group4_sum(vp);
                if (g4 == 0) vsp[w * QB + s] = vp;
            }
        }

        // ---- dC^T[n][t] += BT dS^T + e^{cum_t} V^T,  V^T[n][t] = Hin^T[n] . dy_t
        {
            float yp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int nt = NTW * w + j;
                const bf16x8 b0 = lds16(BT + (16 * nt + r16) * RS + 8 * g4);
                const bf16x8 b1 = lds16(BT + (16 * nt + r16) * RS + 32 + 8 * g4);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const int t = 16 * tb + r16;
                    f32x4 V = {0.f, 0.f, 0.f, 0.f}, dc = {0.f, 0.f, 0.f, 0.f};
                    V = mfma_bf16(as_bf16x8(hnt[j][0]), lds16(DYn + t * RS + 8 * g4), V);
                    V = mfma_bf16(as_bf16x8(hnt[j][1]), lds16(DYn + t * RS + 32 + 8 * g4), V);
                    dc = mfma_bf16(b0, lds16(DS + t * RS + 8 * g4), dc);
                    dc = mfma_bf16(b1, lds16(DS + t * RS + 32 + 8 * g4), dc);
                    const float e = eac[t];
                    const uint2 c4 = *reinterpret_cast<const uint2 *>(Cn + t * NS + 16 * nt + 4 * g4);
                    const float cv[4] = {bf16_lo(c4.x), bf16_hi(c4.x), bf16_lo(c4.y), bf16_hi(c4.y)};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        accC[j][tb][i] += dc[i] + e * V[i];
                        yp[tb] += cv[i] * V[i];
                    }
                }
            }
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const float v = group4_sum(yp[tb]);
                if (g4 == 0) yocp[w * QB + 16 * tb + r16] = v;
            }
        }

        // ---- dB^T[n][s] += CT dS + w_s X2^T,  X2^T[n][s] = Gh^T[n] . x_s
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int nt = NTW * w + j;
            const bf16x8 c0 = lds16(CT + (16 * nt + r16) * RS + 8 * g4);
            const bf16x8 c1 = lds16(CT + (16 * nt + r16) * RS + 32 + 8 * g4);
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                const int s = 16 * sb + r16;
                f32x4 X2 = {0.f, 0.f, 0.f, 0.f}, db = {0.f, 0.f, 0.f, 0.f};
                X2 = mfma_bf16(as_bf16x8(ght[j][0]), lds16(Xn + s * RS + 8 * g4), X2);
                X2 = mfma_bf16(as_bf16x8(ght[j][1]), lds16(Xn + s * RS + 32 + 8 * g4), X2);
                db = mfma_bf16(c0, lds16(DST + s * RS + 8 * g4), db);
                db = mfma_bf16(c1, lds16(DST + s * RS + 32 + 8 * g4), db);
                const float ws = wsv[s];
#pragma unroll
                for (int i = 0; i < 4; ++i) accB[j][sb][i] += db[i] + ws * X2[i];
            }
        }

        // ---- <Gh, Hin> and sum x . dy of this head
        {
            float gp = 0.f, xp = 0.f;
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int kp = 0; kp < 2; ++kp)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t a = (&ght[j][kp].x)[q], b = (&hnt[j][kp].x)[q];
                        gp += bf16_lo(a) * bf16_lo(b) + bf16_hi(a) * bf16_hi(b);
                    }
            {   // x . dy from LDS (the registers already hold the next head): token
                // tid / 4, 16 values
                const int t = tid >> 2, p0 = 16 * (tid & 3);
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const uint4 xv = *reinterpret_cast<const uint4 *>(Xn + t * RS + p0 + 8 * k);
                    const uint4 yv = *reinterpret_cast<const uint4 *>(DYn + t * RS + p0 + 8 * k);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t a = (&xv.x)[q], b = (&yv.x)[q];
                        xp += bf16_lo(a) * bf16_lo(b) + bf16_hi(a) * bf16_hi(b);
                    }
                }
            }
            gp = wave_sum(gp);
            xp = wave_sum(xp);
            if (lane == 0) {
                red[w] = gp;
                red[4 + w] = xp;
            }
        }
        __syncthreads();

        // ---- d cum -> d a -> d dt and dA, dD partials (wave 0, lane = token)
        if (w == 0) {
            const int t = lane;
            const bool valid = t < qlen;
            const float v = (vsp[t] + vsp[QB + t]) + (vsp[2 * QB + t] + vsp[3 * QB + t]);
            const float y = (yocp[t] + yocp[QB + t]) + (yocp[2 * QB + t] + yocp[3 * QB + t]);
            const float cr = (colR[t] + colR[QB + t]) + (colR[2 * QB + t] + colR[3 * QB + t]);
            const float glw = (colGLW[t] + colGLW[QB + t]) + (colGLW[2 * QB + t] + colGLW[3 * QB + t]);
            const float ghin = (red[0] + red[1]) + (red[2] + red[3]);
            const float xdy = (red[4] + red[5]) + (red[6] + red[7]);
            const float wt = wsv[t];
            const float dend = exp2f(aend) * ghin + wave_sum(wt * v);
            float dc = valid ? rowR[t] - cr + eac[t] * y - wt * v : 0.f;
            if (t == qlen - 1) dc += dend;
            const float inc = wave_inclusive_scan(dc);
            const float da = __shfl(inc, 63, 64) - inc + dc;     // sum over tau >= t
            if (valid)
                ddt[(size_t(bi) * L + t0 + t) * H + h] = glw + exp2f(aend - cs) * v + Ah * da;
            const float dA = wave_sum(valid ? dreg * da : 0.f);
            if (lane == 0) {
                dAp[bhc] = dA;
                dDp[bhc] = xdy;
            }
        }
    }

    // per-block partials of dB and dC: tiles with rows n, columns s (or t)
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const int n0 = 16 * (NTW * w + j) + 4 * g4;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int s = 16 * k + r16;
            if (s < qlen) {
                const size_t o = ((size_t(bi) * L + t0 + s) * nblk + hbk) * N + n0;
                *reinterpret_cast<float4 *>(dBp + o) =
                    make_float4(accB[j][k][0], accB[j][k][1], accB[j][k][2], accB[j][k][3]);
                *reinterpret_cast<float4 *>(dCp + o) =
                    make_float4(accC[j][k][0], accC[j][k][1], accC[j][k][2], accC[j][k][3]);
            }
        }
    }
}

template <int N>
hipError_t launch_n(const ChunkScanBwdArgs &a, const ChunkScanBwdPlan &pl, hipStream_t stream) {
    char *ws = static_cast<char *>(a.workspace);
    bf16_bits *hinT = reinterpret_cast<bf16_bits *>(ws + pl.off_hin);
    bf16_bits *ghT = reinterpret_cast<bf16_bits *>(ws + pl.off_gh);
    bf16_bits *ghN = reinterpret_cast<bf16_bits *>(ws + pl.off_ghn);
    float *dBp = reinterpret_cast<float *>(ws + pl.off_dbp);
    float *dCp = reinterpret_cast<float *>(ws + pl.off_dcp);
    float *dAp = reinterpret_cast<float *>(ws + pl.off_dap);
    float *dDp = reinterpret_cast<float *>(ws + pl.off_ddp);
    const bf16_bits *x = static_cast<const bf16_bits *>(a.x), *B = static_cast<const bf16_bits *>(a.B);
    const bf16_bits *C = static_cast<const bf16_bits *>(a.C), *dy = static_cast<const bf16_bits *>(a.dy);
    hipError_t e;
    hipLaunchKernelGGL((k_bwd_chain<N>), dim3(2, a.H, a.b), dim3(kThreads), 0, stream, x, a.dt, a.A,
                       B, C, dy, a.init_state, a.d_final, hinT, ghT, ghN, a.d_init, a.L, a.H, a.G,
                       pl.nc);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t lds = ChunkLds<N>::bytes;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_bwd_chunk_bf<N>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_bwd_chunk_bf<N>), dim3(pl.nc, a.H / pl.hb, a.b), dim3(kThreads), lds,
                       stream, x, a.dt, a.A, B, C, a.D, dy, hinT, ghT, ghN,
                       static_cast<bf16_bits *>(a.dx), a.ddt, dBp, dCp, dAp, dDp, a.L, a.H, a.G,
                       pl.nc, pl.hb);
    return hipGetLastError();
}

}  // namespace

size_t chunk_bwd_bf16_lds(int N) {
    if (N == 64) return ChunkLds<64>::bytes;
    if (N == 128) return ChunkLds<128>::bytes;
    return 0;
}

hipError_t launch_chunk_scan_bwd_bf16(const ChunkScanBwdArgs &a, const ChunkScanBwdPlan &pl,
                                      hipStream_t stream) {
    if (a.N == 64) return launch_n<64>(a, pl, stream);
    if (a.N == 128) return launch_n<128>(a, pl, stream);
    return hipErrorInvalidValue;
}

}  // namespace ssd
