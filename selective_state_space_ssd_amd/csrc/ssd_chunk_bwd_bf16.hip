// ssd_chunk_bwd_bf16.hip -- gradients of the SSD chunked scan, bf16 I/O, head
// dimension 64, state size 64 or 128: the bf16 matrix-core path.
//
// Same mathematics as ssd_chunk_bwd.hip (the chunked decomposition of the Mamba-2
// article (msbhsh.com), «SSD 算法：分块矩阵分解» and «SSD 算法：分块和形态传递», run in
// reverse; intermediate states recomputed rather than stored, "另辟蹊径--Mamba介绍",
// «Hardware-aware Algorithm»), organised for fewer HBM bytes:
//
//   k_bwd_chain    one workgroup walks the 64-token chunks of one batch row in order
//                  (forward, two heads of a group when the group has an even number
//                  of heads) or in reverse (one head), keeping the P x N state in MFMA
//                  accumulators: the forward walk writes the state entering each chunk,
//                  Hin_c; the reverse walk writes the gradient of the state leaving it,
//                  Gh_c, and finally d init_state.  Each chunk's contribution
//                  (sum_t w_t x_t (outer) B_t, or sum_t e^{cum_t} dy_t (outer) C_t) is
//                  one bf16 MFMA product added onto the decayed state, so no per-chunk
//                  state ever goes to HBM in fp32.  The states are stored in bf16, in
//                  MFMA accumulator tile order (contiguous stores; the next kernel
//                  assembles its operands from two 8-byte pieces).
//   k_bwd_chunk_bf one workgroup of 8 waves per (chunk, block of heads of one group,
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
constexpr int RSA = 72;    // the same for the chain walk's weighted-u rows (keeps two
                           // two-head walk workgroups within one CU's LDS)

__device__ __forceinline__ bf16x8 lds16(const bf16_bits *p) {
    return as_bf16x8(*reinterpret_cast<const uint4 *>(p));
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0, 0, 0, 0); }

// ------------------------------------------------------------ state chains
__device__ __forceinline__ uint4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0));
}

constexpr int kChainThreads = 512;   // 4 loader waves + 4 state waves

// Stored states keep the MFMA accumulator order: 16 x 16 tiles of 256 values, lane l
// of the producing wave holding 4 consecutive bf16 at 4 l (tile element (4 (l / 16) +
// i, l % 16) at 4 l + i), so every store writes 512 contiguous bytes.
//   Hin^T, Gh^T: tile nt * 4 + pt holds rows p 16 pt .. (i), columns n 16 nt .. (l % 16)
// (the chunk kernel reads Gh^T in both operand layouts from an LDS copy)
__device__ __forceinline__ int tile_off(int tile, int l) { return tile * 256 + 4 * l; }

// The 8 consecutive values (along the tile rows) that lane (r16, g4) of a consumer
// supplies as an MFMA operand at k step kk (32 values): rows 32 kk + 8 g4 .. + 7 of
// column r16, taken from tiles t_base + (2 kk + g4 / 2) * t_stride as two 8-byte
// pieces of lanes r16 + 32 (g4 & 1) and r16 + 32 (g4 & 1) + 16.
__device__ __forceinline__ uint4 tile_operand(__amdgpu_buffer_rsrc_t st, int t_base, int t_stride,
                                              int kk, int r16, int g4) {
    const int tile = t_base + (2 * kk + (g4 >> 1)) * t_stride;
    const int l = r16 + 32 * (g4 & 1);
    const u32x2 lo = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(st, tile_off(tile, l) * 2, 0, 0));
    const u32x2 hi = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(st, tile_off(tile, l + 16) * 2, 0, 0));
    return make_uint4(lo[0], lo[1], hi[0], hi[1]);
}

// Inputs of one chunk step held by a loader thread: the token pair (2 tpu, 2 tpu + 1)
// of u (x or dy) at p group pgu for each of the FH walked heads, two token-pair items
// of v (B or C, shared by the heads of a group), and dt of each head.
template <int FH>
struct ChainPf {
    uint4 ua[FH], ub[FH], va[2], vb[2];
    float d[FH];
};

// One chain walk per workgroup of 8 waves with split roles, so that no wave waits on
// another kind of memory traffic (the vector-memory counter is per wave and in order):
//   loader waves 0-3  load chunk inputs two steps ahead through buffer resources
//                     sized to the chunk's valid tokens (tokens past the end read as
//                     zero), scan the chunk's decays, and stage the weighted u and v
//                     transposed into one of two LDS buffers;
//   state waves 4-7   hold the P x N state in MFMA accumulators, store it, and add the
//                     staged chunk's contribution: state <- alpha state + U^T V.
// One barrier per step hands a staged buffer from the loaders to the state waves.
// DIR 0: Hin_c for c = 0 .. nc-1 (as Hin^T tiles), starting from init_state, for FH
//        heads of one group at once (they share B, so one staged V serves both).
// DIR 1: Gh_c for c = nc-1 .. 0 (as Gh^T tiles) from d_final, then d_init; it walks
// one head.
// With FH = 2 the LDS of a workgroup (72 KiB) stays under half of the CU's 160 KiB, so
// two fit; the per-buffer decay factors live in the unused padding of the first AT row.
template <int N, int FH>
struct ChainLds {
    bf16_bits AT[2][FH][HP * RSA];  // [p][t] weighted u of each walked head, two buffers
    bf16_bits VT[2][N * RSA];       // [n][t] v, two buffers
};

// Transposed staging rows (64 tokens: eight 16-byte chunks of 8 tokens) hold chunk c
// of row r at chunk position c ^ swz8(r).  A 4-byte LDS store of a wave is served in
// two passes of 32 lanes over 32 banks (measured with the bank-conflict counter); the
// 32 lanes of a pass store one token pair of 4 consecutive pairs (one chunk) in each
// of 8 rows that lie a multiple of 32 dwords apart, so without the swizzle they meet
// on 4 banks (8-way conflicts), and with it on 32.  An MFMA operand read is one
// whole chunk per lane, found at its row's position (tests/test_chain_staging_layout.py
// replays the stores and reads on the host: placement and bank spread).
__device__ __forceinline__ int swz8(int r) { return (r >> 3) & 7; }

template <int N, int DIR, int FH>
__device__ __forceinline__ void chain_walk(
    const bf16_bits *__restrict__ u, const float *__restrict__ dt, const float *__restrict__ A,
    const bf16_bits *__restrict__ v, const float *__restrict__ s0, bf16_bits *__restrict__ dstT,
    float *__restrict__ d_init, int L, int H, int G, int nc, ChainLds<N, FH> &sm, int h,
    int bi) {
    constexpr int NT = N / 16, NG = N / 8, PN = HP * N;
    constexpr int kVItems = (32 * NG + kThreads - 1) / kThreads;
    constexpr int WH = DIR == 0 ? FH : 1;   // heads this walk carries
    static_assert(HP + 2 * (2 * FH) <= RSA, "decay factors must fit in the row padding");
    auto &AT = sm.AT;
    auto &VT = sm.VT;
    float *al_sh = reinterpret_cast<float *>(&sm.AT[0][0][HP]);   // [buf * FH + head]
    const int g = h / (H / G);
    float Ah[WH];
#pragma unroll
    for (int k = 0; k < WH; ++k) Ah[k] = A[h + k];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
    const size_t bh = size_t(bi) * H + h;
    auto chunk_of = [&](int step) { return DIR == 0 ? step : nc - 1 - step; };

    if (w < 4) {
        // ------------------------------------------------ loader waves
        const int tpu = tid >> 3, pgu = tid & 7;
        auto load = [&](ChainPf<WH> &f, int step) {
            const bool live = step < nc;
            const int t0 = live ? chunk_of(step) * QB : 0;
            const int qlen = live ? min(QB, L - t0) : 0;
            const size_t tok0 = size_t(bi) * L + t0;
            const auto ur = buffer_rsrc(u + tok0 * H * HP, uint32_t(qlen) * uint32_t(H * HP) * 2u);
            const auto vr = buffer_rsrc(v + tok0 * G * N, uint32_t(qlen) * uint32_t(G * N) * 2u);
            const auto dr = buffer_rsrc(dt + tok0 * H, uint32_t(qlen) * uint32_t(H) * 4u);
#pragma unroll
            for (int k = 0; k < WH; ++k) {
                const uint32_t uo = (uint32_t(2 * tpu) * H + h + k) * HP + 8 * pgu;
                f.ua[k] = ld128(ur, uo * 2u);
                f.ub[k] = ld128(ur, (uo + H * HP) * 2u);
            }
#pragma unroll
            for (int k = 0; k < kVItems; ++k) {
                const int item = min(tid + k * kThreads, 32 * NG - 1);
                const int tp = (item >> 3) & 31, ng = (item & 7) | ((item >> 8) << 3);
                const uint32_t vo = (uint32_t(2 * tp) * G + g) * N + 8 * ng;
                f.va[k] = ld128(vr, vo * 2u);
                f.vb[k] = ld128(vr, (vo + G * N) * 2u);
            }
#pragma unroll
            for (int k = 0; k < WH; ++k)
                f.d[k] = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(dr, int((lane * H + h + k) * 4), 0, 0));
        };
        auto stage = [&](const ChainPf<WH> &f, int step) {
            const bool live = step < nc;
            const int qlen = live ? min(QB, L - chunk_of(step) * QB) : 1;
            const int buf = step & 1;
#pragma unroll
            for (int k = 0; k < WH; ++k) {
                const float cs = wave_inclusive_scan(f.d[k] * Ah[k] * kLog2e);
                const float aend = lane_value(cs, qlen - 1);
                const float wv = lane < qlen ? (DIR == 0 ? exp2f(aend - cs) * f.d[k] : exp2f(cs)) : 0.f;
                if (tid == 0) al_sh[buf * FH + k] = exp2f(aend);
                const float wa = __shfl(wv, 2 * tpu, 64), wb = __shfl(wv, 2 * tpu + 1, 64);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t ea = (&f.ua[k].x)[j >> 1], eb = (&f.ub[k].x)[j >> 1];
                    const float fa = (j & 1) ? bf16_hi(ea) : bf16_lo(ea);
                    const float fb = (j & 1) ? bf16_hi(eb) : bf16_lo(eb);
                    const int p = 8 * pgu + j;
                    *reinterpret_cast<uint32_t *>(
                        &AT[buf][k][p * RSA + 8 * ((tpu >> 2) ^ swz8(p)) + 2 * (tpu & 3)]) =
                        pack_bf16x2(fa * wa, fb * wb);
                }
            }
#pragma unroll
            for (int k = 0; k < kVItems; ++k) {
                const int item = tid + k * kThreads;
                if (item < 32 * NG) {
                    // lanes of a store pass: 4 token pairs (one chunk) x 8 channel groups
                    const int tp = (item >> 3) & 31, ng = (item & 7) | ((item >> 8) << 3);
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const uint32_t ea = (&f.va[k].x)[j >> 1], eb = (&f.vb[k].x)[j >> 1];
                        const uint32_t lo = (j & 1) ? (ea >> 16) : (ea & 0xffffu);
                        const uint32_t hi = (j & 1) ? (eb & 0xffff0000u) : (eb << 16);
                        const int n = 8 * ng + j;
                        *reinterpret_cast<uint32_t *>(
                            &VT[buf][n * RSA + 8 * ((tp >> 2) ^ swz8(n)) + 2 * (tp & 3)]) = lo | hi;
                    }
                }
            }
        };
        ChainPf<WH> f0, f1;
        load(f0, 0);
        load(f1, 1);
        stage(f0, 0);
        load(f0, 2);
        __syncthreads();
        // iteration s stages step s + 1 (set (s + 1) & 1) and refills that set with s + 3
        int s = 0;
        for (; s + 1 < nc; s += 2) {
            stage(f1, s + 1);
            load(f1, s + 3);
            __syncthreads();
            stage(f0, s + 2);
            load(f0, s + 4);
            __syncthreads();
        }
        if (s < nc) __syncthreads();
        return;
    }

    // ---------------------------------------------------- state waves
    const int sw = w - 4;
    f32x4 accP[WH][NT];
#pragma unroll
    for (int k = 0; k < WH; ++k)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                accP[k][nt][i] =
                    s0 ? s0[(bh + k) * PN + (16 * sw + 4 * g4 + i) * N + 16 * nt + r16] : 0.f;
    __syncthreads();
    for (int step = 0; step < nc; ++step) {
        const int c = chunk_of(step);
        const int buf = step & 1;
        // the lane's row and lane group, re-derived each step from an opaque copy of the
        // lane index: otherwise the per-tile LDS addresses are hoisted out of the loop and
        // spill, and each scratch reload waits (one in-order counter) for this step's
        // state stores to complete
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int r16 = ln & 15, g4 = ln >> 4;
        // store the state (entering chunk c forward, leaving chunk c in reverse)
        const size_t so = (bh * nc + c) * size_t(PN);
#pragma unroll
        for (int k = 0; k < WH; ++k)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                *reinterpret_cast<uint2 *>(dstT + so + size_t(k) * nc * PN + tile_off(nt * 4 + sw, lane)) =
                    make_uint2(pack_bf16x2(accP[k][nt][0], accP[k][nt][1]),
                               pack_bf16x2(accP[k][nt][2], accP[k][nt][3]));
        // the stores above are issued before the update starts: otherwise the packed
        // values stay live next to the update's operands and spill
        __builtin_amdgcn_sched_barrier(0);
        // state <- al * state + (this chunk's contribution)
        const bf16_bits *vt = VT[buf];
#pragma unroll
        for (int k = 0; k < WH; ++k) {
            const float al = al_sh[buf * FH + k];
            const bf16_bits *at = AT[buf][k] + (16 * sw + r16) * RSA;
            const int fa = swz8(16 * sw + r16);
            const bf16x8 a0 = lds16(at + 8 * (g4 ^ fa));
            const bf16x8 a1 = lds16(at + 8 * ((4 + g4) ^ fa));
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16_bits *vr = vt + (16 * nt + r16) * RSA;
                const int fv = swz8(16 * nt + r16);
                f32x4 t = accP[k][nt] * al;
                t = mfma_bf16(a0, lds16(vr + 8 * (g4 ^ fv)), t);
                accP[k][nt] = mfma_bf16(a1, lds16(vr + 8 * ((4 + g4) ^ fv)), t);
            }
        }
        __syncthreads();
    }
    if constexpr (DIR == 1) {
        if (d_init) {
            // addresses computed here, from an opaque copy of the lane index, rather
            // than kept (and spilled) through the walk
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const int r16 = ln & 15, g4 = ln >> 4;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    d_init[bh * PN + (16 * sw + 4 * g4 + i) * N + 16 * nt + r16] = accP[0][nt][i];
        }
    }
}

// Both walks in one launch, so that the independent chains of every (head, batch) run
// at the same time: workgroups 0 .. nfwd-1 walk forward over FH heads of one group
// each (batch row, then head pair), the following b H workgroups walk one head each in
// reverse.  With FH = 2 and 72 KiB of LDS per workgroup, all b H (1 + 1/FH) workgroups
// of the L=2048 layer (480) are resident at once on 256 CUs (two per CU), where one
// head per forward walk (640) needed a second round.
template <int N, int FH>
__global__ __launch_bounds__(kChainThreads, 4) void k_bwd_chain(
    const bf16_bits *__restrict__ x, const bf16_bits *__restrict__ dy,
    const float *__restrict__ dt, const float *__restrict__ A, const bf16_bits *__restrict__ B,
    const bf16_bits *__restrict__ C, const float *__restrict__ init_state,
    const float *__restrict__ d_final, bf16_bits *__restrict__ hinT, bf16_bits *__restrict__ ghT,
    float *__restrict__ d_init, int L, int H, int G, int nc, int nfwd) {
    __shared__ __align__(16) ChainLds<N, FH> sm;
    const int wg = blockIdx.x;
    if (wg < nfwd) {
        const int hp = H / FH;
        chain_walk<N, 0, FH>(x, dt, A, B, init_state, hinT, nullptr, L, H, G, nc, sm,
                             FH * (wg % hp), wg / hp);
    } else {
        const int r = wg - nfwd;
        chain_walk<N, 1, FH>(dy, dt, A, C, d_final, ghT, d_init, L, H, G, nc, sm, r % H,
                             r / H);
    }
}

// ------------------------------------------------------------ in-chunk gradients
// 8 waves (two per SIMD: the 143 KiB of LDS allow one workgroup per CU).  Tile
// ownership, with hw = w / 4 and q = w % 4:
//   scores W, M, dS       rows t of block q, s tiles 2 hw, 2 hw + 1
//   dx^T, U^T             rows p of block q, s tiles 2 hw, 2 hw + 1
//   V^T, dC^T, X2^T, dB^T rows n of tile w % NT, t (or s) tiles TW (w / NT) .. + TW - 1
constexpr int kChunkThreads = 512;

template <int N>
struct ChunkLds {
    static constexpr int NT = N / 16;
    static constexpr int NS = N + 16;                      // row stride of [t][n]
    // acum, dts, wsv, eac, rowR parts [2], colR [4], colGLW [4], vsp [4], yocp [NT], red
    static constexpr int kScalars = (4 + 2 + 4 + 4 + 4 + NT) * QB + 16;
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
    static constexpr size_t off_GH = off_DST + size_t(QB) * RS * 2;   // Gh^T tiles of a head
    static constexpr size_t bytes = off_GH + size_t(HP) * N * 2;
};

template <int N>
__global__ __launch_bounds__(kChunkThreads) void k_bwd_chunk_bf(
    const bf16_bits *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const bf16_bits *__restrict__ B, const bf16_bits *__restrict__ C, const float *__restrict__ D,
    const bf16_bits *__restrict__ dy, const bf16_bits *__restrict__ hinT,
    const bf16_bits *__restrict__ ghT, bf16_bits *__restrict__ dx, float *__restrict__ ddt, float *__restrict__ dBp,
    float *__restrict__ dCp, float *__restrict__ dAp, float *__restrict__ dDp, int L, int H,
    int G, int nc, int HB) {
    using Lay = ChunkLds<N>;
    constexpr int NS = Lay::NS, NT = N / 16, KN = N / 32, NG = N / 8, PN = HP * N;
    constexpr int TW = NT / 2;                 // t (s) tiles per wave in the n phases
    const int c = blockIdx.x, hbk = blockIdx.y, bi = blockIdx.z;
    const int nblk = gridDim.y;
    const int h0 = hbk * HB;
    const int g = h0 / (H / G);
    const int t0 = c * QB, qlen = min(QB, L - t0);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r16 = lane & 15, g4 = lane >> 4;
    const int q = w & 3, hw = w >> 2;          // row block and column half (scores, dx)
    const int ntw = w % NT, tb0 = (w / NT) * TW;   // n tile and first t tile (n phases)

    extern __shared__ __align__(16) unsigned char smem[];
    float *acum = reinterpret_cast<float *>(smem);   // [QB]
    float *dts = acum + QB;                          // [QB]
    float *wsv = dts + QB;                           // [QB] e^{cum_end - cum_s} dt_s
    float *eac = wsv + QB;                           // [QB] e^{cum_t}
    float *rowR = eac + QB;                          // [2][QB] parts of sum_s R[t][s]
    float *colR = rowR + 2 * QB;                     // [4][QB] parts of sum_t R[t][s]
    float *colGLW = colR + 4 * QB;                   // [4][QB] parts of sum_t (G Lm W)[t][s]
    float *vsp = colGLW + 4 * QB;                    // [4][QB] parts of v_s
    float *yocp = vsp + 4 * QB;                      // [NT][QB] parts of C_t . V_t
    float *red = yocp + NT * QB;                     // [16]
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
    bf16_bits *GH = reinterpret_cast<bf16_bits *>(smem + Lay::off_GH);     // Gh^T tiles

    // one head's x (threads 0-255) or dy (threads 256-511): token pair tpu, p group pgu
    const bool is_dy = tid >= kThreads;
    const int tpu = (tid & 255) >> 3, pgu = tid & 7;
    // x, dy, dt, dx and ddt through buffer views of the chunk's qlen rows (32-bit
    // offsets; rows past them read 0 and their stores are dropped)
    const size_t tok0 = size_t(bi) * L + t0;
    const __amdgpu_buffer_rsrc_t xyres =
        buffer_rsrc((is_dy ? dy : x) + tok0 * H * HP, uint32_t(qlen) * uint32_t(H * HP) * 2u);
    const __amdgpu_buffer_rsrc_t dtres = buffer_rsrc(dt + tok0 * H, uint32_t(qlen) * uint32_t(H) * 4u);
    const __amdgpu_buffer_rsrc_t dxres = buffer_rsrc(dx + tok0 * H * HP, uint32_t(qlen) * uint32_t(H * HP) * 2u);
    const __amdgpu_buffer_rsrc_t ddtres = buffer_rsrc(ddt + tok0 * H, uint32_t(qlen) * uint32_t(H) * 4u);
    uint4 ra, rb;
    float dnext;
    auto load_head = [&](int h) {
        const int ta = 2 * tpu;
        const int o = ((ta * H + h) * HP + 8 * pgu) * 2;
        ra = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xyres, o, 0, 0));
        rb = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xyres, o + H * HP * 2, 0, 0));
        dnext = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(dtres, (lane * H + h) * 4, 0, 0));
    };
    load_head(h0);

    // B and C of the group, natural and transposed (one token-pair item of each)
    for (int item = tid; item < 32 * NG; item += kChunkThreads) {
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
    __syncthreads();

    // G[t][s] = C_t . B_s on this wave's score tiles (shared by the heads)
    f32x4 Gt[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int sb = 2 * hw + k;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kq = 0; kq < KN; ++kq)
            acc = mfma_bf16(lds16(Cn + (16 * q + r16) * NS + 32 * kq + 8 * g4),
                            lds16(Bn + (16 * sb + r16) * NS + 32 * kq + 8 * g4), acc);
        Gt[k] = acc;
    }

    f32x4 accB[TW], accC[TW];
#pragma unroll
    for (int k = 0; k < TW; ++k) {
        accB[k] = {0.f, 0.f, 0.f, 0.f};
        accC[k] = {0.f, 0.f, 0.f, 0.f};
    }

    // a head's states as MFMA A operands (rows owned by this wave)
    // (Gh: rows p of block q, k = n; Gh^T and Hin^T: rows n of tile ntw, k = p).  Gh is
    // stored once, as Gh^T tiles: a head's tiles are loaded one head ahead into
    // registers (issued once the previous head's operands are built), copied to LDS at
    // the top of the head, and both operand layouts are read from that copy.  Hin^T is
    // read at the top of its head.
    uint4 ghp[KN], ght[2], hnt[2];
    constexpr int GPT = HP * N * 2 / 16 / kChunkThreads;   // 16-byte pieces per thread
    static_assert(GPT >= 1 && HP * N * 2 % (16 * kChunkThreads) == 0, "whole pieces");
    uint4 ghq[GPT];
    auto state_view = [&](const bf16_bits *base, int hs) {
        const size_t so = ((size_t(bi) * H + h0 + hs) * nc + c) * size_t(PN);
        return buffer_rsrc(base + so, uint32_t(PN) * 2u);
    };
    auto load_gh = [&](int hs) {
        const __amdgpu_buffer_rsrc_t gt = state_view(ghT, hs);
#pragma unroll
        for (int k = 0; k < GPT; ++k)
            ghq[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   gt, (tid + k * kChunkThreads) * 16, 0, 0));
    };
    load_gh(0);
    // The LDS copy keeps element e of the tiles at gh_swz(e): within each tile the
    // 16-byte groups of the 64-element row group m = (e / 64) mod 4 (lanes 16 m ..
    // 16 m + 15 of the stored accumulator layout) are permuted by m.  The row reads
    // below take one element per lane from the row groups of 4 lanes each, which
    // without it meet on one bank per group (6 conflict cycles per read, measured with
    // the bank-conflict counter) and with it spread over the banks; 8- and 16-byte
    // pieces stay whole.
    auto gh_swz = [](int e) { return e ^ (((e >> 6) & 3) << 3); };
    // 8 consecutive bf16 of the LDS copy at element stride 4: Gh[p][n0 .. n0+7] for the
    // lane's row p = 16 q + r16, n0 = 32 kq + 8 g4 (tile (n0 / 16) * 4 + q, lane
    // 16 (r16 / 4) + n0 % 16 + j, element r16 % 4); the row group is m = r16 / 4, so
    // element base + 8 j sits at base + 8 (j ^ m).  The addresses come from an opaque
    // copy of the lane index, so they are formed at each use rather than held.
    auto gh_rows_p = [&](int kq) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int rr = ln & 15, gg = ln >> 4, m = rr >> 2;
        const int base = ((2 * kq + (gg >> 1)) * 4 + q) * 256 + 4 * (16 * m + 8 * (gg & 1)) + (rr & 3);
        uint32_t wv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = base + 8 * (j ^ m);
            wv[j] = uint32_t(GH[e]) | (uint32_t(GH[e + 4]) << 16);
        }
        return make_uint4(wv[0], wv[1], wv[2], wv[3]);
    };
    // Gh^T operand (rows n of tile ntw, k = p) from the LDS copy: the same two 8-byte
    // pieces as tile_operand reads from memory
    auto gh_rows_n = [&](int kp) {
        const int tile = ntw * 4 + 2 * kp + (g4 >> 1);
        const int l = r16 + 32 * (g4 & 1);
        const uint2 lo = *reinterpret_cast<const uint2 *>(GH + gh_swz(tile_off(tile, l)));
        const uint2 hi = *reinterpret_cast<const uint2 *>(GH + gh_swz(tile_off(tile, l + 16)));
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
    };

    for (int hh = 0; hh < HB; ++hh) {
        const int h = h0 + hh;
        const size_t bhc = (size_t(bi) * H + h) * nc + c;
        {
            const __amdgpu_buffer_rsrc_t ht = state_view(hinT, hh);
#pragma unroll
            for (int kp = 0; kp < 2; ++kp) hnt[kp] = tile_operand(ht, ntw * 4, 1, kp, r16, g4);
        }
        // this head's Gh^T tiles to LDS (the previous head's reads of the copy ended
        // before its last barrier)
#pragma unroll
        for (int k = 0; k < GPT; ++k)
            *reinterpret_cast<uint4 *>(GH + gh_swz((tid + k * kChunkThreads) * 8)) = ghq[k];
        const float dreg = dnext;
        const float Ah = A[h];
        const float cs = wave_inclusive_scan(dreg * Ah * kLog2e);
        const float aend = lane_value(cs, qlen - 1);
        if (w == 0) {   // wave 0 reads the previous head's scalars until here
            const bool valid = lane < qlen;
            acum[lane] = valid ? cs : 0.f;
            dts[lane] = dreg;
            wsv[lane] = valid ? exp2f(aend - cs) * dreg : 0.f;
            eac[lane] = valid ? exp2f(cs) : 0.f;
        }
        // stage x (natural) or dy (natural and transposed)
        {
            bf16_bits *dstn = is_dy ? DYn : Xn;
            *reinterpret_cast<uint4 *>(dstn + (2 * tpu) * RS + 8 * pgu) = ra;
            *reinterpret_cast<uint4 *>(dstn + (2 * tpu + 1) * RS + 8 * pgu) = rb;
            if (is_dy) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int sh = 16 * (j & 1);
                    const uint32_t lo = ((&ra.x)[j >> 1] >> sh) & 0xffffu, hi = ((&rb.x)[j >> 1] >> sh) & 0xffffu;
                    const int p = 8 * pgu + j;   // chunk swizzle as in the state walks' staging
                    *reinterpret_cast<uint32_t *>(DYT + p * RS + 8 * ((tpu >> 2) ^ swz8(p)) + 2 * (tpu & 3)) =
                        lo | (hi << 16);
                }
            }
        }
        if (hh + 1 < HB) load_head(h + 1);
        __syncthreads();
        // both layouts of Gh from the LDS copy; then the next head's tiles can load
#pragma unroll
        for (int kq = 0; kq < KN; ++kq) ghp[kq] = gh_rows_p(kq);
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) ght[kp] = gh_rows_n(kp);
        if (hh + 1 < HB) load_gh(hh + 1);

        // ---- scores on this wave's tiles: W = dy x^T, then M, dS and the sums
        {
            float rsum[4] = {0.f, 0.f, 0.f, 0.f};
            const bf16x8 d0 = lds16(DYn + (16 * q + r16) * RS + 8 * g4);
            const bf16x8 d1 = lds16(DYn + (16 * q + r16) * RS + 32 + 8 * g4);
            float at[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) at[i] = acum[16 * q + 4 * g4 + i];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int sb = 2 * hw + k;
                f32x4 Wt = {0.f, 0.f, 0.f, 0.f};
                Wt = mfma_bf16(d0, lds16(Xn + (16 * sb + r16) * RS + 8 * g4), Wt);
                Wt = mfma_bf16(d1, lds16(Xn + (16 * sb + r16) * RS + 32 + 8 * g4), Wt);
                const int s = 16 * sb + r16;
                const float ds = dts[s], as = acum[s];
                float mv[4], sv[4], cr = 0.f, cglw = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * q + 4 * g4 + i;
                    const float lm = (s <= t && t < qlen) ? exp2f(at[i] - as) : 0.f;
                    const float gl = Gt[k][i] * lm;
                    mv[i] = gl * ds;
                    sv[i] = Wt[i] * lm * ds;
                    const float r = sv[i] * Gt[k][i];
                    rsum[i] += r;
                    cr += r;
                    cglw += gl * Wt[i];
                    DS[t * RS + s] = f32_to_bf16(sv[i]);
                }
                *reinterpret_cast<uint2 *>(MT + s * RS + 16 * q + 4 * g4) =
                    make_uint2(pack_bf16x2(mv[0], mv[1]), pack_bf16x2(mv[2], mv[3]));
                *reinterpret_cast<uint2 *>(DST + s * RS + 16 * q + 4 * g4) =
                    make_uint2(pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3]));
                cr = group4_sum(cr);
                cglw = group4_sum(cglw);
                if (g4 == 0) {
                    colR[q * QB + s] = cr;
                    colGLW[q * QB + s] = cglw;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = row16_sum(rsum[i]);
                if (r16 == 0) rowR[hw * QB + 16 * q + 4 * g4 + i] = v;
            }
        }
        __syncthreads();

        // ---- dx^T[p][s] (rows p of block q) and U^T[p][s] = Gh[p] . B_s
        {
            const float Dh = D[h];
            const int fd = swz8(16 * q + r16);
            const bf16x8 e0 = lds16(DYT + (16 * q + r16) * RS + 8 * (g4 ^ fd));
            const bf16x8 e1 = lds16(DYT + (16 * q + r16) * RS + 8 * ((4 + g4) ^ fd));
            const int p0 = 16 * q + 4 * g4;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int s = 16 * (2 * hw + k) + r16;
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
                const u32x2 ov = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
                __builtin_amdgcn_raw_buffer_store_b64(ov, dxres, ((s * H + h) * HP + p0) * 2, 0, 0);
                vp = group4_sum(vp);
                if (g4 == 0) vsp[q * QB + s] = vp;
            }
        }

        // ---- dC^T[n][t] += BT dS^T + e^{cum_t} V^T,  V^T[n][t] = Hin^T[n] . dy_t
        {
            const bf16x8 b0 = lds16(BT + (16 * ntw + r16) * RS + 8 * g4);
            const bf16x8 b1 = lds16(BT + (16 * ntw + r16) * RS + 32 + 8 * g4);
#pragma unroll
            for (int k = 0; k < TW; ++k) {
                const int t = 16 * (tb0 + k) + r16;
                f32x4 V = {0.f, 0.f, 0.f, 0.f}, dc = {0.f, 0.f, 0.f, 0.f};
                V = mfma_bf16(as_bf16x8(hnt[0]), lds16(DYn + t * RS + 8 * g4), V);
                V = mfma_bf16(as_bf16x8(hnt[1]), lds16(DYn + t * RS + 32 + 8 * g4), V);
                dc = mfma_bf16(b0, lds16(DS + t * RS + 8 * g4), dc);
                dc = mfma_bf16(b1, lds16(DS + t * RS + 32 + 8 * g4), dc);
                const float e = eac[t];
                const uint2 c4 = *reinterpret_cast<const uint2 *>(Cn + t * NS + 16 * ntw + 4 * g4);
                const float cv[4] = {bf16_lo(c4.x), bf16_hi(c4.x), bf16_lo(c4.y), bf16_hi(c4.y)};
                float yp = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    accC[k][i] += dc[i] + e * V[i];
                    yp += cv[i] * V[i];
                }
                yp = group4_sum(yp);
                if (g4 == 0) yocp[ntw * QB + t] = yp;
            }
        }

        // ---- dB^T[n][s] += CT dS + w_s X2^T,  X2^T[n][s] = Gh^T[n] . x_s
        {
            const bf16x8 c0 = lds16(CT + (16 * ntw + r16) * RS + 8 * g4);
            const bf16x8 c1 = lds16(CT + (16 * ntw + r16) * RS + 32 + 8 * g4);
#pragma unroll
            for (int k = 0; k < TW; ++k) {
                const int s = 16 * (tb0 + k) + r16;
                f32x4 X2 = {0.f, 0.f, 0.f, 0.f}, db = {0.f, 0.f, 0.f, 0.f};
                X2 = mfma_bf16(as_bf16x8(ght[0]), lds16(Xn + s * RS + 8 * g4), X2);
                X2 = mfma_bf16(as_bf16x8(ght[1]), lds16(Xn + s * RS + 32 + 8 * g4), X2);
                db = mfma_bf16(c0, lds16(DST + s * RS + 8 * g4), db);
                db = mfma_bf16(c1, lds16(DST + s * RS + 32 + 8 * g4), db);
                const float ws = wsv[s];
#pragma unroll
                for (int i = 0; i < 4; ++i) accB[k][i] += db[i] + ws * X2[i];
            }
        }

        // ---- <Gh, Hin> (waves 0 .. NT-1 hold each n row once) and sum x . dy
        {
            float gp = 0.f, xp = 0.f;
            if (w < NT) {
#pragma unroll
                for (int kp = 0; kp < 2; ++kp)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t a = (&ght[kp].x)[j], b = (&hnt[kp].x)[j];
                        gp += bf16_lo(a) * bf16_lo(b) + bf16_hi(a) * bf16_hi(b);
                    }
            }
            {   // token tid / 8, 8 values at 8 (tid % 8)
                const int t = tid >> 3, p0 = 8 * (tid & 7);
                const uint4 xv = *reinterpret_cast<const uint4 *>(Xn + t * RS + p0);
                const uint4 yv = *reinterpret_cast<const uint4 *>(DYn + t * RS + p0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t a = (&xv.x)[j], b = (&yv.x)[j];
                    xp += bf16_lo(a) * bf16_lo(b) + bf16_hi(a) * bf16_hi(b);
                }
            }
            gp = wave_sum(gp);
            xp = wave_sum(xp);
            if (lane == 0) {
                red[w] = gp;
                red[8 + w] = xp;
            }
        }
        __syncthreads();

        // ---- d cum -> d a -> d dt and dA, dD partials (wave 0, lane = token)
        if (w == 0) {
            const int t = lane;
            const bool valid = t < qlen;
            float v = 0.f, y = 0.f, cr = 0.f, glw = 0.f, ghin = 0.f, xdy = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v += vsp[k * QB + t];
                cr += colR[k * QB + t];
                glw += colGLW[k * QB + t];
            }
#pragma unroll
            for (int k = 0; k < NT; ++k) y += yocp[k * QB + t];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                ghin += red[k];
                xdy += red[8 + k];
            }
            const float rr = rowR[t] + rowR[QB + t];
            const float wt = wsv[t];
            const float dend = exp2f(aend) * ghin + wave_sum(wt * v);
            float dc = valid ? rr - cr + eac[t] * y - wt * v : 0.f;
            if (t == qlen - 1) dc += dend;
            const float inc = wave_inclusive_scan(dc);
            const float da = lane_value(inc, 63) - inc + dc;     // sum over tau >= t
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(glw + exp2f(aend - cs) * v + Ah * da),
                                                  ddtres, (t * H + h) * 4, 0, 0);
            const float dA = wave_sum(valid ? dreg * da : 0.f);
            if (lane == 0) {
                dAp[bhc] = dA;
                dDp[bhc] = xdy;
            }
        }
    }

    // per-block partials of dB and dC: tiles with rows n, columns s (or t)
    const int n0 = 16 * ntw + 4 * g4;
#pragma unroll
    for (int k = 0; k < TW; ++k) {
        const int s = 16 * (tb0 + k) + r16;
        if (s < qlen) {
            const size_t o = ((size_t(bi) * L + t0 + s) * nblk + hbk) * N + n0;
            *reinterpret_cast<float4 *>(dBp + o) = make_float4(accB[k][0], accB[k][1], accB[k][2], accB[k][3]);
            *reinterpret_cast<float4 *>(dCp + o) = make_float4(accC[k][0], accC[k][1], accC[k][2], accC[k][3]);
        }
    }
}

template <int N>
hipError_t launch_n(const ChunkScanBwdArgs &a, const ChunkScanBwdPlan &pl, hipStream_t stream) {
    char *ws = static_cast<char *>(a.workspace);
    bf16_bits *hinT = reinterpret_cast<bf16_bits *>(ws + pl.off_hin);
    bf16_bits *ghT = reinterpret_cast<bf16_bits *>(ws + pl.off_gh);
    float *dBp = reinterpret_cast<float *>(ws + pl.off_dbp);
    float *dCp = reinterpret_cast<float *>(ws + pl.off_dcp);
    float *dAp = reinterpret_cast<float *>(ws + pl.off_dap);
    float *dDp = reinterpret_cast<float *>(ws + pl.off_ddp);
    const bf16_bits *x = static_cast<const bf16_bits *>(a.x), *B = static_cast<const bf16_bits *>(a.B);
    const bf16_bits *C = static_cast<const bf16_bits *>(a.C), *dy = static_cast<const bf16_bits *>(a.dy);
    hipError_t e;
    // two heads per forward walk whenever a group has an even number of heads
    if ((a.H / a.G) % 2 == 0) {
        const int nfwd = a.b * a.H / 2;
        hipLaunchKernelGGL((k_bwd_chain<N, 2>), dim3(nfwd + a.b * a.H), dim3(kChainThreads), 0,
                           stream, x, dy, a.dt, a.A, B, C, a.init_state, a.d_final, hinT, ghT,
                           a.d_init, a.L, a.H, a.G, pl.nc, nfwd);
    } else {
        const int nfwd = a.b * a.H;
        hipLaunchKernelGGL((k_bwd_chain<N, 1>), dim3(nfwd + a.b * a.H), dim3(kChainThreads), 0,
                           stream, x, dy, a.dt, a.A, B, C, a.init_state, a.d_final, hinT, ghT,
                           a.d_init, a.L, a.H, a.G, pl.nc, nfwd);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t lds = ChunkLds<N>::bytes;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_bwd_chunk_bf<N>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_bwd_chunk_bf<N>), dim3(pl.nc, a.H / pl.hb, a.b), dim3(kChunkThreads), lds,
                       stream, x, a.dt, a.A, B, C, a.D, dy, hinT, ghT,
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
