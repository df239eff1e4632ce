// ssd_chunk_fused.hip -- single-pass SSD chunked scan for gfx950 (bf16 I/O, P = 64).
//
// Same four steps as the chunked algorithm of the Mamba-2 article (msbhsh.com),
// «SSD 算法：分块矩阵分解» / «SSD 算法：分块和形态传递», fused into one kernel so that
// x is read once, y is written once and no per-chunk state makes a round trip
// through HBM:
//
//   * one workgroup (8 waves, two per SIMD) per (batch, chunk, block of HB heads of
//     one group);
//   * C B^T of the chunk is computed once per workgroup and kept in registers as
//     MFMA operands (it is shared by every head of the group);
//   * decay: every token of x is pre-scaled by dt times its decay to the chunk end
//     (a factor <= 1), which makes step 2 a plain contraction.  When the total
//     decay of a head over the chunk is moderate (-log2 decay <= kFastSpan, always
//     true for step sizes and decay rates in the usual ranges) step 1 uses the same
//     scaled x, causally masked, and rescales each output column once by the decay
//     from its token to the chunk end (a factor >= 1, at most 2^kFastSpan).
//     Otherwise the head takes an exact fallback for step 1 that only exponentiates
//     non-positive numbers: each score is multiplied by its pairwise decay and dt
//     and contracted with x as given;
//   * step 3 (state passing) is a chain between workgroups: the workgroup of
//     chunk c waits until chunk c-1 of the same head has published its state,
//     publishes H_c = exp(Acum_end) H_{c-1} + S_c, and only then needs H_{c-1} for
//     its own outputs.  Every chunk of a chain (batch row, block of heads) runs on
//     one XCD: work items come from one queue per XCD, a workgroup takes its ticket
//     from the queue of the XCD it runs on (read from the hardware), and a queue
//     holds a run of chains, chunk-major.  The hand-off then stays in that XCD's L2:
//     the state and its ready flag are stored write-back (a store completes at the
//     L2) and read with coherent loads, which the L2 serves; the writer waits for
//     its state stores to complete before it raises the flag, and no cache-wide
//     fence is needed.  Within a queue every item a workgroup waits for has an
//     earlier ticket, held by a workgroup that is already running: the chain cannot
//     deadlock.  The wait is bounded; on time-out the state is poisoned with NaN and
//     an error word in the workspace is set, so a failure is loud and never a hang.
//
// Step 1, 2 and 4 contractions use v_mfma_f32_16x16x32_bf16 with fp32 accumulation;
// the in-chunk decay cumsum is a wavefront scan.
#include <algorithm>
#include <atomic>
#include <cmath>

#include "ssd_device.h"
#include "ssd_kernels.h"
#include "ssd_stage.h"

namespace ssd {

namespace {

constexpr int kFT = 512;                    // threads per workgroup
constexpr int kFW = kFT / 64;               // waves per workgroup
constexpr uint32_t kSpinLimit = 1u << 20;   // about a second of polling before giving up
// Largest -log2(decay over one chunk) handled by the single-reference form: scaled
// x stays >= 2^-100 * |dt x| (normal fp32 / bf16 range) and the output rescale stays
// <= 2^100.
constexpr float kFastSpan = 100.f;

template <int Q, int N>
struct Fz {
    static constexpr int P = 64;
    static constexpr int PT = P / 16;              // 16-row channel tiles
    static constexpr int NT = Q / 16;              // 16-token output tiles
    static constexpr int NSB = Q / 32;             // 32-token blocks
    static constexpr int TPW = (NT + kFW - 1) / kFW;   // output tiles per wave
    static constexpr int NK = (N + 31) / 32;       // 32-wide k-steps over N
    static constexpr int NPAD = NK * 32;
    // LDS row strides of the token-contiguous tiles and of the state tile.  The pads
    // of 16 elements make the 16-byte MFMA operand reads (16 rows x 4 lane groups)
    // conflict-free on gfx950; a pad of 8 gives 2-way bank conflicts (measured with
    // the LDS bank-conflict counter).
    static constexpr int QS = Q + 16;
    static constexpr int HS = NPAD + 16;
    static constexpr int XS = P;                   // LDS row stride of x in token-major order
    static constexpr int NTN = N / 16;             // state column tiles
    // state tiles of a wave (PTW row tiles x NTW column tiles; each operand fragment
    // read from LDS feeds NTW or PTW products): with 8 column tiles the waves form a
    // 2 x 4 grid of 2 x 2 blocks; with more, each wave owns whole columns; with fewer,
    // the waves of one column split its channel tiles
    static constexpr bool kGrid22 = NTN == 8 && kFW == 8 && PT == 4;
    static constexpr int NTW = kGrid22 ? 2 : NTN >= kFW ? NTN / kFW : 1;
    static constexpr int WPN = NTN >= kFW ? 1 : kFW / NTN;     // waves per column tile
    static constexpr int PTW = kGrid22 ? 2 : NTN >= kFW ? PT : (PT >= WPN ? PT / WPN : 1);
    static constexpr size_t kScalars = 3104;       // acum, dts, dtn [256], misc
    static constexpr size_t kLds = kScalars + size_t(N) * QS * 2 + size_t(P) * QS * 2 +
                                   size_t(Q) * XS * 2 + size_t(P) * HS * 2;
    // B in natural layout is staged, before the head loop, over the x / state regions
    static constexpr bool kBnatFits =
        size_t(Q) * HS <= size_t(P) * QS + size_t(Q) * XS + size_t(P) * HS;
    static_assert(Q % 64 == 0 && Q <= 256, "Q must be 64, 128 or 256");
    static_assert(N % 16 == 0, "N must be a multiple of 16");
    // workgroups per CU the LDS allows (at most two); with two, every wave must fit
    // in a quarter of the register file
    static constexpr int kWgPerCu = kLds <= 80 * 1024 ? 2 : 1;
    // LDS operand reads run this many k-steps ahead of the matrix products (deeper
    // pipelining needs registers that two workgroups per CU do not have)
    static constexpr int kDepth = kWgPerCu == 1 ? 2 : 1;
};

// t-tile handled by wave w in its m-th slot: a snake order so that the waves get
// similar amounts of causal work.
__device__ __forceinline__ int tile_of(int m, int w) {
    return kFW * m + ((m & 1) ? kFW - 1 - w : w);
}

__device__ __forceinline__ uint4 ld_bf16x8_global(const bf16_bits *p, bool ok) {
    return ok ? *reinterpret_cast<const uint4 *>(p) : make_uint4(0, 0, 0, 0);
}

// 16 bytes at a 32-bit byte offset from a workgroup-uniform base (scalar base
// register + one offset register per lane)
__device__ __forceinline__ uint4 ld_b128_off(const void *base, uint32_t byte_off, bool ok) {
    return ok ? *reinterpret_cast<const uint4 *>(static_cast<const char *>(base) + byte_off)
              : make_uint4(0, 0, 0, 0);
}


// A decay factor 2^x, x <= 0, with the hardware transcendental (results below the
// normal range flush to zero, which is what a decay factor that small means).  The
// argument is clamped at 0 so that a value computed for a masked-out (s > t) pair can
// never be inf and turn a discarded 0 * inf into NaN.
__device__ __forceinline__ float exp2_dec(float x) { return __builtin_amdgcn_exp2f(fminf(x, 0.f)); }

// Token order of the k dimension in the token-contiguous LDS tiles (x decayed, B
// transposed).  Inside each 32-token block the 4-token groups are interleaved: token
// 4g + i (g < 4) sits at 8g + i and token 16 + 4g + i at 8g + 4 + i.  The eight k
// values a lane of lane group g4 supplies to a 16x16x32 product are then the tokens
// 4g4 .. 4g4+3 and 16+4g4 .. 16+4g4+3 -- the rows of its score fragment, which comes
// from an accumulator -- and they are one contiguous 16-byte read.  Both operands of
// the chunk-state contraction use the same order, so it does not change that sum.
__device__ __forceinline__ int tok_pos32(int u) {   // u = token within its 32-block
    return ((u & 12) << 1) | ((u & 16) >> 2) | (u & 3);
}

// Element offset of x[t][c] in the token-major LDS copy (64 channels per row, no
// padding): the eight 8-channel blocks of row t are XOR-swizzled by
// ((t / 4) ^ 2 (t % 4)) % 8.  With it both the 16-byte staging stores (8 lanes on 8
// consecutive token groups) and the 8-byte reads of the D x epilogue (16 lanes on 16
// consecutive tokens) are free of bank conflicts (measured on gfx950).
__device__ __forceinline__ int xn_off(int t, int c) {
    return t * 64 + 8 * ((c >> 3) ^ (((t >> 2) ^ ((t & 3) << 1)) & 7)) + (c & 7);
}

// Stage the chunk's B rows ([Q tokens][N channels] bf16, token t at
// src + t * tok_stride) into LDS twice from one read: transposed, bt[n * bt_stride + k]
// (k = token position, order above; for the chunk-state contraction), and in natural
// order, bn[t * bn_stride + n] for n < NPAD (zero padded; for the score tiles).  Work
// items are 8 tokens (the ones at 8 consecutive positions) x 8 channels: eight 16-byte
// row loads, all issued before any LDS store, a register transpose, 16-byte LDS
// stores.  With at least 8 channel blocks, the 64 items of a wave form an 8 x 8 block
// of (token block, channel block) taken along diagonals: lane l has token block l % 8
// and channel block (l % 8 + l / 8) % 8, so that each load instruction reads 8 rows
// 128 contiguous bytes each, and every 8 consecutive lanes store to distinct banks in
// both layouts.
template <int kThreads, int Q, int N, int NPAD>
__device__ __forceinline__ void stage_B(const bf16_bits *__restrict__ src, size_t tok_stride,
                                        int qlen, bf16_bits *bt, int bt_stride, bf16_bits *bn,
                                        int bn_stride) {
    constexpr int TG = Q / 8, CG = NPAD / 8, items = TG * CG;
    constexpr bool kDiag = CG % 8 == 0 && TG % 8 == 0;
#pragma unroll
    for (int it0 = 0; it0 < items; it0 += kThreads) {
        const int it = it0 + int(threadIdx.x);
        if (items % kThreads != 0 && it >= items) break;
        int tb, cb;
        if constexpr (kDiag) {
            const int blk = it >> 6, l = it & 63;
            tb = 8 * (blk % (TG / 8)) + (l & 7);
            cb = 8 * (blk / (TG / 8)) + (((l & 7) + (l >> 3)) & 7);
        } else {
            tb = it % TG;
            cb = it / TG;
        }
        const int w0 = 8 * cb;
        int tok[8];   // the tokens at positions 8 tb .. 8 tb + 7
#pragma unroll
        for (int i = 0; i < 8; ++i) tok[i] = 32 * (tb >> 2) + (i < 4 ? 4 * (tb & 3) + i : 16 + 4 * (tb & 3) + i - 4);
        uint4 rows[8], cols[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            rows[i] = (tok[i] < qlen && w0 < N)
                          ? *reinterpret_cast<const uint4 *>(src + size_t(tok[i]) * tok_stride + w0)
                          : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<uint4 *>(bn + tok[i] * bn_stride + w0) = rows[i];
        if (w0 < N) {
            transpose8x8_b16(rows, cols);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<uint4 *>(bt + (w0 + j) * bt_stride + 8 * tb) = cols[j];
        }
    }
}

// The chunk-to-chunk state hand-off is read by another workgroup on the same XCD: it
// is stored write-back (default policy; the store completes at the XCD's L2) and read
// with the coherent policy (sc1), which the L2 serves for a line this XCD wrote (a
// load with sc0 alone can be served stale by the CU's own cache; measured).  In the
// ring the state is kept in the accumulator layout: 16x16 tile (pt, nt) at float
// offset (pt * N/16 + nt) * 256, lane l's four values (rows 4(l/16) + i, column
// l % 16) at l * 4 + i, so that each lane moves 16 bytes per access.
constexpr int kBufL2 = 16;   // cache-policy bits of a buffer load: sc1 (coherent; served by
                             // the XCD's L2 when the line was written on this XCD)
// Wait until this wave's outstanding memory operations have completed.
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// A 32-bit word read coherently (from the XCD's L2 when this XCD wrote it; the asm
// statement keeps a polling read inside its loop), and a word written to the XCD's L2
// (write-back: the store completes at the L2, not at memory).
__device__ __forceinline__ uint32_t ld_l2(const uint32_t *p) {
    asm volatile("" ::: "memory");
    return __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(p, 4u), 0, 0, kBufL2);
}
__device__ __forceinline__ void st_l2(uint32_t *p, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b32(v, buffer_rsrc(p, 4u), 0, 0, 0);
}

template <int Q, int N>
__global__ __launch_bounds__(kFT) __attribute__((amdgpu_waves_per_eu(2 * Fz<Q, N>::kWgPerCu)))
void k_ssd_fused(
    const bf16_bits *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const bf16_bits *__restrict__ B, const bf16_bits *__restrict__ C,
    const float *__restrict__ D, const float *__restrict__ init_state,
    bf16_bits *__restrict__ y, float *__restrict__ final_state, float *hbuf, uint32_t *flags,
    uint32_t *hdr, int L, int H, int G, int HB, int nchains, int nc, int nq) {
    using F = Fz<Q, N>;
    constexpr int P = F::P;
    extern __shared__ __align__(16) unsigned char smem[];
    float *acum = reinterpret_cast<float *>(smem);     // [256] log2-domain decay cumsum
    float *dts = acum + 256;                            // [256] dt of the current head
    float *dtn = dts + 256;                             // [256] dt of the next head
    int *misc = reinterpret_cast<int *>(dtn + 256);     // [8]
    bf16_bits *BT = reinterpret_cast<bf16_bits *>(smem + F::kScalars);   // [N][QS]
    bf16_bits *XwT = BT + N * F::QS;                    // [P][QS] block-decayed dt x
    bf16_bits *XN = XwT + P * F::QS;                    // [Q][XS] x as given, token-major (xn_off)
    bf16_bits *Hs = XN + Q * F::XS;                     // [P][HS] entering state, bf16

    const int tid = threadIdx.x, lane = tid & 63;
    // wave index; held in a scalar register except in the Q = 256 kernels, whose scalar
    // registers are short (they spill some into vector-register lanes, never to
    // scratch; a scalar copy of the wave index adds to those spills)
    const int w = Q == 256 ? tid >> 6 : __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g4 = lane >> 4;

    if (tid == 0) {
        // A prepared workspace carries the magic word.  Work items are handed out by one
        // queue per XCD: each queue takes a run of consecutive chains (batch row, block
        // of heads), so that chains sharing a batch row's B and C share an L2 where they
        // can, and a queue's items are its chains' chunks in chunk-major order,
        // so every chunk of a chain runs on one XCD and the chain's hand-off stays in
        // that XCD's L2.  A workgroup reads the XCD it runs on from the hardware and
        // takes a ticket from that XCD's queue.  The hardware places workgroup i on XCD
        // i mod nq, and the launch gives every XCD W = gridDim / nq workgroups, as many
        // as the longest queue has items.  A queue is one 64-bit word: the tickets taken
        // (low half) and the call number ("epoch", high half), so one atomic add gives
        // a workgroup both; the workgroup that takes a queue's W-th ticket wraps the
        // count back to 0 and advances that queue's epoch.  Every call advances every
        // queue once, so all queues carry the same call number.  Ready flags carry
        // epoch + 1, so flags left by earlier calls (or other shapes' data in the flag
        // region) never read as ready.  A ticket beyond W (more workgroups on an XCD
        // than the launch placed there) sets the error word.  Without a prepared
        // workspace every item runs at its own index and never waits (its handed-over
        // states are NaN).
        const uint32_t magic =
            __hip_atomic_load(&hdr[kWsMagicWord], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool prepared = magic == kWsMagic;
        int it = -1;
        uint32_t epoch = 0;
        if (prepared) {
            uint32_t xcc;
            asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
            const int x = int(xcc & 15u) % nq;
            unsigned long long *q = reinterpret_cast<unsigned long long *>(hdr + kWsQueueWord + 2 * x);
            const uint64_t old = atomicAdd(q, 1ull);
            const uint32_t t = uint32_t(old), W = gridDim.x / unsigned(nq);
            epoch = uint32_t(old >> 32);
            if (t == W - 1u) atomicAdd(q, (1ull << 32) - W);
            if (t >= W)
                __hip_atomic_store(&hdr[kWsErrorWord], 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int per = (nchains + nq - 1) / nq;            // chains per queue
            const int nchx = max(0, min(per, nchains - x * per));   // the last may hold fewer
            if (t < uint32_t(nchx * nc)) it = int(t) / nchx * nchains + x * per + int(t) % nchx;
        } else if (blockIdx.x < unsigned(nchains * nc)) {
            it = int(blockIdx.x);
        }
        misc[0] = it;
        misc[2] = prepared;
        misc[3] = int(epoch + 1u);
    }
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(misc[0]);   // uniform: keep it scalar
    const bool ws_ok = __builtin_amdgcn_readfirstlane(misc[2]) != 0;
    const uint32_t ready = uint32_t(__builtin_amdgcn_readfirstlane(misc[3]));   // flag value
    if (item < 0) return;   // more workgroups on this XCD than its queue has items
    const int c = item / nchains, chain = item % nchains;
    const int hblocks = H / HB;
    const int bi = chain / hblocks, h0 = (chain % hblocks) * HB;
    const int g = h0 / (H / G);
    const int t0 = c * Q, qlen = min(Q, L - t0);
    const size_t tok0 = size_t(bi) * L + t0;
    const bool last = (c == nc - 1);
    const __amdgpu_buffer_rsrc_t yres =
        buffer_rsrc(y + tok0 * H * P, uint32_t(qlen) * uint32_t(H * P) * 2u);

    // ---- global loads of the prologue, all issued before the first LDS store:
    // C rows of this wave's output tiles (B-operand layout: column t, k = n), kept for
    // the whole workgroup; B of the chunk
    uint4 cf[F::TPW][F::NK];
#pragma unroll
    for (int m = 0; m < F::TPW; ++m) {
        const int T = tile_of(m, w);
        const int t = 16 * T + r16;
#pragma unroll
        for (int kk = 0; kk < F::NK; ++kk) {
            const int n0 = kk * 32 + 8 * g4;
            cf[m][kk] = ld_bf16x8_global(C + ((tok0 + t) * G + g) * N + n0,
                                         T < F::NT && t < qlen && n0 < N);
        }
    }
    // x and dt are read through range-checked buffer views of the chunk's qlen rows:
    // rows past them read 0, and no load sits behind a branch, so the compiler can
    // count the memory operations in flight and wait only for the ones it needs.
    // Thread tid < Q holds dt of token tid.  x is staged in blocks of 4 tokens x 8
    // channels: lane l of wave w holds tokens xt0 .. xt0+3, xt0 = 32w + 4(l % 8), and
    // channels xc0 .. xc0+7, xc0 = 8(l / 8), so that 8 lanes read one whole 128-byte
    // row of x per load (8 rows per instruction).  The decay cumsum uses another
    // layout (lane l: tokens 4l .. 4l+3, computed by every wave for the whole chunk);
    // lane xsl of that layout holds the staging lane's tokens.  In the decayed copy
    // they sit at position xp0 (token order of the contraction tiles).
    const __amdgpu_buffer_rsrc_t xres =
        buffer_rsrc(x + tok0 * H * P, uint32_t(qlen) * uint32_t(H * P) * 2u);
    const __amdgpu_buffer_rsrc_t dtres = buffer_rsrc(dt + tok0 * H, uint32_t(qlen) * uint32_t(H) * 4u);
    const int tq0 = 4 * lane;
    const int xsl = 8 * w + (lane & 7), xt0 = 4 * xsl, xc0 = 8 * (lane >> 3);
    const int xp0 = 32 * w + tok_pos32(4 * (lane & 7));
    auto load_x = [&](uint4 (&xq)[4], int hx) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            xq[k] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(
                           xres, int((((xt0 + k) * H + hx) * P + xc0) * 2), 0, kBufNonTemporal));
    };
    auto load_dt = [&](int hx) {   // 0 past qlen; a head past the block reads unused data
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(dtres, int((tid * H + hx) * 4), 0, 0));
    };
    // With one workgroup per CU nothing else covers load latency: x is loaded one
    // head ahead and dt two heads ahead (the value for head h + 1 is loaded while
    // head h - 1 is processed; one strided 4-byte read per token).  With two, the
    // other workgroup covers it and the registers are worth more: x and dt are
    // loaded at the start of the head before the one they serve.  The first head's
    // loads are issued before B's, whose wait retires them.
    constexpr bool kPrefetchX = F::kWgPerCu == 1;
    // A and D of the block's heads, lane j holding head h0 + j (HB <= 16), read per
    // head with v_readlane: a scalar load per head would share its wait counter with
    // the LDS reads and put a memory round trip in front of the first LDS wait of the
    // cumsum and of the epilogue
    const float a_lanes = lane < HB ? A[h0 + lane] : 0.f;
    const float d_lanes = lane < HB ? D[h0 + lane] : 0.f;
    const float dt_first = load_dt(h0);
    float dt_pipe = kPrefetchX ? load_dt(h0 + 1) : 0.f;
    uint4 xq[4];       // x of the lane's 4 staging tokens, channels xc0 .. xc0+7
    if constexpr (kPrefetchX) load_x(xq, h0);
    // B of the chunk: transposed for the chunk-state contraction (step 2), and in
    // natural layout (over the x / state regions, free until the head loop) for the
    // score tiles
    bf16_bits *Bnat = XwT;   // [Q][HS]
    stage_B<kFT, Q, N, F::NPAD>(B + (tok0 * G + g) * N, size_t(G) * N, qlen, BT, F::QS, Bnat,
                                F::HS);
    if (tid < Q) dtn[tid] = dt_first;
    __syncthreads();

    // ---- G^T = B C^T tiles of this wave's output tiles, kept as MFMA B operands:
    // gfrag[m][S] is 32-token block S of tile slot m in bf16, for S = 0 .. T / 2; the
    // last of them is the diagonal block, causally masked (head independent)
    constexpr int kSlots = (kFW / 2) * F::TPW;     // max blocks of a slot
    uint4 gfrag[F::TPW][kSlots];
#pragma unroll
    for (int m = 0; m < F::TPW; ++m) {
        const int T = tile_of(m, w);
        if (T >= F::NT) continue;
        const int nsb = T / 2, t = 16 * T + r16;
#pragma unroll
        for (int S = 0; S <= (kFW / 2) * (m + 1) - 1 && S < F::NSB; ++S) {
            if (S > nsb) break;
            f32x4 gt[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                gt[half] = f32x4{0.f, 0.f, 0.f, 0.f};
                const bf16_bits *brow = Bnat + (32 * S + 16 * half + r16) * F::HS + 8 * g4;
#pragma unroll
                for (int kk = 0; kk < F::NK; ++kk)
                    gt[half] = mfma_bf16(as_bf16x8(*reinterpret_cast<const uint4 *>(brow + 32 * kk)),
                                         as_bf16x8(cf[m][kk]), gt[half]);
            }
            if (S == nsb) {   // keep s <= t only
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (32 * S + 16 * half + 4 * g4 + i > t) gt[half][i] = 0.f;
            }
            gfrag[m][S] = make_uint4(pack_bf16x2(gt[0][0], gt[0][1]),
                                     pack_bf16x2(gt[0][2], gt[0][3]),
                                     pack_bf16x2(gt[1][0], gt[1][1]),
                                     pack_bf16x2(gt[1][2], gt[1][3]));
        }
    }
    __syncthreads();   // Bnat is overwritten by the first head's x

    // state tiles of this wave (step 2 accumulators and the hand-off)
    const int nt_base = F::kGrid22 ? 2 * (w % 4) : F::NTN >= kFW ? w : (w % F::NTN);
    const int pt_base = F::kGrid22 ? 2 * (w / 4) : F::NTN >= kFW ? 0 : (w / F::NTN);
    constexpr int NT_STEP = F::kGrid22 ? 1 : kFW;
    constexpr int PT_STEP = F::kGrid22 || F::NTN >= kFW ? 1 : F::WPN;
    const bool s_active = pt_base < F::PT;

    // zero the padding columns of the entering-state tile once
    if constexpr (F::NPAD > N) {
        for (int it = tid; it < P * (F::NPAD - N); it += kFT)
            Hs[(it / (F::NPAD - N)) * F::HS + N + it % (F::NPAD - N)] = 0;
    }

    for (int hh = 0; hh < HB; ++hh) {
        const int h = h0 + hh;
        const size_t bh = size_t(bi) * H + h;
        // ---- discretisation and in-chunk decay cumsum (inclusive, log2 domain),
        // computed by every wave for all tokens: 4 tokens per lane + a wave scan
        if constexpr (!kPrefetchX) load_x(xq, h);
        const float Al2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a_lanes), hh)) * kLog2e;
        float dq[4], aq[4];
        {
            const float4 d4 = *reinterpret_cast<const float4 *>(dtn + tq0);
            dq[0] = d4.x; dq[1] = d4.y; dq[2] = d4.z; dq[3] = d4.w;
        }
        // dt of the next head (thread tid < Q holds token tid), stored to dtn once
        // every wave has read this head's values (after the staging barrier)
        const float dt_next = kPrefetchX ? dt_pipe : load_dt(h + 1);
        aq[0] = dq[0] * Al2;
        aq[1] = aq[0] + dq[1] * Al2;
        aq[2] = aq[1] + dq[2] * Al2;
        aq[3] = aq[2] + dq[3] * Al2;
        const float run = wave_inclusive_scan(aq[3]);
        const float excl = run - aq[3];
#pragma unroll
        for (int k = 0; k < 4; ++k) aq[k] += excl;   // constant past qlen (dt = 0 there)
        const float aend = __shfl(aq[(Q - 1) & 3], (Q - 1) >> 2, 64);
        const bool fast = -aend <= kFastSpan;   // uniform over the workgroup
        if (w == 0) {
            *reinterpret_cast<float4 *>(acum + tq0) = make_float4(aq[0], aq[1], aq[2], aq[3]);
            *reinterpret_cast<float4 *>(dts + tq0) = make_float4(dq[0], dq[1], dq[2], dq[3]);
        }
        // ---- x of this head: x as given, token-major (for the D x term), and x
        // decayed to the chunk end (times dt), transposed to [channel][token]; 4 tokens
        // x 8 channels per lane.  The factors are computed in the cumsum layout and
        // fetched from lane xsl.
        float xf[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) xf[k] = __shfl(exp2_dec(aend - aq[k]) * dq[k], xsl, 64);
        if (xt0 < Q) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                *reinterpret_cast<uint4 *>(XN + xn_off(xt0 + k, xc0)) = xq[k];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float f = xf[k];
                uint4 &r = xq[k];
                r = make_uint4(pack_bf16x2(bf16_lo(r.x) * f, bf16_hi(r.x) * f),
                               pack_bf16x2(bf16_lo(r.y) * f, bf16_hi(r.y) * f),
                               pack_bf16x2(bf16_lo(r.z) * f, bf16_hi(r.z) * f),
                               pack_bf16x2(bf16_lo(r.w) * f, bf16_hi(r.w) * f));
            }
            uint2 cols[8];
            transpose4x8_b16(xq, cols);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<uint2 *>(XwT + (xc0 + j) * F::QS + xp0) = cols[j];
        }
        // ---- step 3, first half: wait for the previous chunk of this head to publish
        // its state.  Thread 0 polls while the other waves finish staging, and the
        // staging barrier hands the outcome to the workgroup; the state loads are then
        // issued before the step 2 products, which cover their latency.
        if (c > 0 && tid == 0) {
            uint32_t *flag = flags + bh * nc + (c - 1);
            uint32_t it = 0;
            int ok = ws_ok;
            while (ok && ld_l2(flag) != ready) {
                __builtin_amdgcn_s_sleep(2);
                if (++it > kSpinLimit) {
                    ok = 0;
                    __hip_atomic_store(&hdr[kWsErrorWord], 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
            misc[1] = ok;
        }
        __syncthreads();

        if (tid < Q) dtn[tid] = dt_next;
        const float *hsrc = nullptr;   // state entering this chunk, fp32 [P][N]; null = zeros
        bool coherent = false, poisoned = false;
        if (c > 0) {
            poisoned = __builtin_amdgcn_readfirstlane(misc[1]) == 0;
            coherent = true;
            hsrc = hbuf + (bh * 2 + ((c - 1) & 1)) * size_t(P) * N;
        } else if (init_state) {
            hsrc = init_state + bh * size_t(P) * N;
        }
        // one read of the entering state, in the accumulator layout: it feeds the
        // update and the bf16 copy in LDS
        float hp[F::PTW][F::NTW][4];
        // offset of element (k, j, i) of the wave's tiles in a [P][N] state
        auto off = [&](int k, int j, int i) {
            return ((pt_base + PT_STEP * k) * 16 + 4 * g4 + i) * N + (nt_base + NT_STEP * j) * 16 + r16;
        };
        // off(k, j, 0) - off(0, 0, 0), a constant (passed as the scalar offset of a
        // buffer access)
        auto tile_offset = [&](int k, int j) { return PT_STEP * k * 16 * N + NT_STEP * j * 16; };
        // off(0, 0, 0) recomputed from an opaque copy of the thread index
        auto lane_offset = [&]() {
            int t = tid;
            asm volatile("" : "+v"(t));
            const int l = t & 63, ww = t >> 6;
            const int ntb = F::kGrid22 ? 2 * (ww % 4) : F::NTN >= kFW ? ww : (ww % F::NTN);
            const int ptb = F::kGrid22 ? 2 * (ww / 4) : F::NTN >= kFW ? 0 : (ww / F::NTN);
            return (ptb * 16 + 4 * (l >> 4)) * N + ntb * 16 + (l & 15);
        };
#pragma unroll
        for (int k = 0; k < F::PTW; ++k)
#pragma unroll
            for (int j = 0; j < F::NTW; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) hp[k][j][i] = 0.f;
        if (s_active) {
            if (coherent) {
                const __amdgpu_buffer_rsrc_t ring = buffer_rsrc(hsrc, uint32_t(P * N * 4));
#pragma unroll
                for (int k = 0; k < F::PTW; ++k)
#pragma unroll
                    for (int j = 0; j < F::NTW; ++j) {
                        const int tile = (pt_base + PT_STEP * k) * F::NTN + nt_base + NT_STEP * j;
                        const f32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
                            ring, (tile * 64 + lane) * 16, 0, kBufL2);
#pragma unroll
                        for (int i = 0; i < 4; ++i) hp[k][j][i] = v[i];
                    }
            } else if (hsrc) {
                // the initial state (first chunk only): offsets from an opaque copy of the
                // thread index, so that they are computed here and not kept live (in 64-bit
                // registers) through the whole head loop for this one-off read
                const __amdgpu_buffer_rsrc_t src = buffer_rsrc(hsrc, uint32_t(P * N * 4));
                const int lo = lane_offset();
#pragma unroll
                for (int k = 0; k < F::PTW; ++k)
#pragma unroll
                    for (int j = 0; j < F::NTW; ++j)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            hp[k][j][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                src, (lo + i * N) * 4, tile_offset(k, j) * 4, 0));
            }
        }
        // ---- step 2: S_c = XwT^T B (x already carries dt and the decay to the chunk end)
        f32x4 accS[F::PTW][F::NTW];
#pragma unroll
        for (int k = 0; k < F::PTW; ++k)
#pragma unroll
            for (int j = 0; j < F::NTW; ++j) accS[k][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (s_active) {
            // software pipelined: the LDS operands of block S + kDepth - 1 are read
            // while block S is multiplied
            constexpr int DP = F::kDepth;
            uint4 af[DP][F::PTW], bfr[DP][F::NTW];
#pragma unroll
            for (int L = 0; L < DP - 1; ++L) {
#pragma unroll
                for (int k = 0; k < F::PTW; ++k)
                    af[L][k] = *reinterpret_cast<const uint4 *>(
                        XwT + ((pt_base + PT_STEP * k) * 16 + r16) * F::QS + 32 * L + 8 * g4);
#pragma unroll
                for (int j = 0; j < F::NTW; ++j)
                    bfr[L][j] = *reinterpret_cast<const uint4 *>(
                        BT + ((nt_base + NT_STEP * j) * 16 + r16) * F::QS + 32 * L + 8 * g4);
            }
#pragma unroll
            for (int S = 0; S < F::NSB; ++S) {
                const int L = S + DP - 1;   // block whose operands are read now
                if (L < F::NSB) {
#pragma unroll
                    for (int k = 0; k < F::PTW; ++k)
                        af[L % DP][k] = *reinterpret_cast<const uint4 *>(
                            XwT + ((pt_base + PT_STEP * k) * 16 + r16) * F::QS + 32 * L + 8 * g4);
#pragma unroll
                    for (int j = 0; j < F::NTW; ++j)
                        bfr[L % DP][j] = *reinterpret_cast<const uint4 *>(
                            BT + ((nt_base + NT_STEP * j) * 16 + r16) * F::QS + 32 * L + 8 * g4);
                }
                if (DP > 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int k = 0; k < F::PTW; ++k)
#pragma unroll
                    for (int j = 0; j < F::NTW; ++j)
                        accS[k][j] = mfma_bf16(as_bf16x8(af[S % DP][k]),
                                               as_bf16x8(bfr[S % DP][j]), accS[k][j]);
            }
        }

        // ---- step 3, second half: H_c = exp(Acum_end) H_{c-1} + S_c
        const float alpha = exp2_dec(aend);
        const float nanv = __int_as_float(0x7fc00000);
        if (s_active) {
            if (poisoned) {
#pragma unroll
                for (int k = 0; k < F::PTW; ++k)
#pragma unroll
                    for (int j = 0; j < F::NTW; ++j)
#pragma unroll
                        for (int i = 0; i < 4; ++i) hp[k][j][i] = nanv;
            }
            // fast form: the entering state reaches token t with decay
            // 2^(acum_t - aend) * 2^aend; the second factor is folded into the copy
            const float sc = fast ? alpha : 1.f;
#pragma unroll
            for (int k = 0; k < F::PTW; ++k)
#pragma unroll
                for (int j = 0; j < F::NTW; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int p = (pt_base + PT_STEP * k) * 16 + 4 * g4 + i;
                        const int n = (nt_base + NT_STEP * j) * 16 + r16;
                        Hs[p * F::HS + n] = f32_to_bf16(hp[k][j][i] * sc);
                        hp[k][j][i] = alpha * hp[k][j][i] + accS[k][j][i];
                    }
            if (!last) {
                const __amdgpu_buffer_rsrc_t ring =
                    buffer_rsrc(hbuf + (bh * 2 + (c & 1)) * size_t(P) * N, uint32_t(P * N * 4));
#pragma unroll
                for (int k = 0; k < F::PTW; ++k)
#pragma unroll
                    for (int j = 0; j < F::NTW; ++j) {
                        const int tile = (pt_base + PT_STEP * k) * F::NTN + nt_base + NT_STEP * j;
                        const f32x4 v = {hp[k][j][0], hp[k][j][1], hp[k][j][2], hp[k][j][3]};
                        __builtin_amdgcn_raw_buffer_store_b128(v, ring, (tile * 64 + lane) * 16, 0, 0);
                    }
            } else if (final_state) {
                // the final state (last chunk only), offsets as for the initial state
                const __amdgpu_buffer_rsrc_t dst =
                    buffer_rsrc(final_state + bh * size_t(P) * N, uint32_t(P * N * 4));
                const int lo = lane_offset();
#pragma unroll
                for (int k = 0; k < F::PTW; ++k)
#pragma unroll
                    for (int j = 0; j < F::NTW; ++j)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(hp[k][j][i]), dst,
                                                                  (lo + i * N) * 4, tile_offset(k, j) * 4, 0);
            }
        }
        if (!last) wait_vm();   // this wave's state stores are complete and visible
        __syncthreads();
        if (!last && tid == 0) st_l2(flags + bh * nc + c, ready);
        if constexpr (kPrefetchX) {
            // loads for the heads ahead, issued after the hand-off so that its wait for
            // the state stores does not wait for them too: x of the next head, in
            // flight during this head's outputs, and dt of the head after it
            if (hh + 1 < HB) load_x(xq, h + 1);
            dt_pipe = load_dt(h + 2);
        }

        // ---- steps 1 and 4 for this wave's output tiles
        const float Dh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d_lanes), hh));
        // step 4 (entering state through C, referenced to the chunk start) for all
        // of the wave's tile slots at once: each state fragment read from LDS feeds
        // every slot; the reads of k-step kk are in flight during the products of
        // k-step kk - 1
        f32x4 acc[F::TPW][F::PT];
        bool slot_ok[F::TPW];
#pragma unroll
        for (int m = 0; m < F::TPW; ++m) {
            const int T = tile_of(m, w);
            slot_ok[m] = T < F::NT && 16 * T < qlen;   // uniform over the wave
#pragma unroll
            for (int pt = 0; pt < F::PT; ++pt) acc[m][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        {
            constexpr int DP = F::kDepth;
            uint4 hf[DP][F::PT];
#pragma unroll
            for (int L = 0; L < DP - 1; ++L)
#pragma unroll
                for (int pt = 0; pt < F::PT; ++pt)
                    hf[L][pt] = *reinterpret_cast<const uint4 *>(
                        Hs + (pt * 16 + r16) * F::HS + L * 32 + 8 * g4);
#pragma unroll
            for (int kk = 0; kk < F::NK; ++kk) {
                const int L = kk + DP - 1;
                if (L < F::NK) {
#pragma unroll
                    for (int pt = 0; pt < F::PT; ++pt)
                        hf[L % DP][pt] = *reinterpret_cast<const uint4 *>(
                            Hs + (pt * 16 + r16) * F::HS + L * 32 + 8 * g4);
                }
                if (DP > 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int m = 0; m < F::TPW; ++m)
                    if (slot_ok[m]) {
#pragma unroll
                        for (int pt = 0; pt < F::PT; ++pt)
                            acc[m][pt] = mfma_bf16(as_bf16x8(hf[kk % DP][pt]),
                                                   as_bf16x8(cf[m][kk]), acc[m][pt]);
                    }
            }
        }
        // y of the wave's tiles, rounded and regrouped, stored together after the last
        // tile: a store that cannot issue (the memory pipeline full of the next head's
        // x loads) would otherwise hold up the products of the tiles after it
        // step 1 in the usual case, for all tile slots at once: x decayed to the chunk
        // end against the score tiles of every block up to the diagonal one, then each
        // output column rescaled to its own token.  A slot's blocks are 0 .. T / 2, so
        // the slots of a wave share their first blocks: each x fragment read from LDS
        // feeds every slot that reaches its block.  The fragments of block S + kDepth - 1
        // are read while block S is multiplied.
        if (fast) {
            int nsbm[F::TPW];
            int nmax = -1;   // uniform over the wave
#pragma unroll
            for (int m = 0; m < F::TPW; ++m) {
                nsbm[m] = slot_ok[m] ? tile_of(m, w) / 2 : -1;
                nmax = max(nmax, nsbm[m]);
            }
            constexpr int DP = F::kDepth;
            uint4 xf8[DP][F::PT];   // tokens 32S + 4g4 + 0..3 and 32S + 16 + 4g4 + 0..3
#pragma unroll
            for (int L = 0; L < DP - 1; ++L)
#pragma unroll
                for (int pt = 0; pt < F::PT; ++pt)
                    xf8[L][pt] = *reinterpret_cast<const uint4 *>(
                        XwT + (pt * 16 + r16) * F::QS + 32 * L + 8 * g4);
#pragma unroll
            for (int S = 0; S < F::NSB; ++S) {
                if (S > nmax) break;
                const int L = S + DP - 1;
                if (L <= nmax) {
#pragma unroll
                    for (int pt = 0; pt < F::PT; ++pt)
                        xf8[L % DP][pt] = *reinterpret_cast<const uint4 *>(
                            XwT + (pt * 16 + r16) * F::QS + 32 * L + 8 * g4);
                }
                if (DP > 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int m = 0; m < F::TPW; ++m) {
                    if (S > (kFW / 2) * (m + 1) - 1) continue;   // past any tile of slot m
                    if (S <= nsbm[m]) {
                        const uint4 gop = gfrag[m][S];
#pragma unroll
                        for (int pt = 0; pt < F::PT; ++pt)
                            acc[m][pt] = mfma_bf16(as_bf16x8(xf8[S % DP][pt]), as_bf16x8(gop),
                                                   acc[m][pt]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < F::TPW; ++m) {
                const int t = 16 * tile_of(m, w) + r16;
                const float u = slot_ok[m] && t < qlen ? __builtin_amdgcn_exp2f(acum[t] - aend) : 0.f;
#pragma unroll
                for (int pt = 0; pt < F::PT; ++pt) acc[m][pt] *= u;
            }
        }
        // y of the wave's tiles, rounded and regrouped, stored together after the last
        // tile: a store that cannot issue (the memory pipeline full of the next head's
        // x loads) would otherwise hold up the products of the tiles after it
        u32x4 yq[F::TPW][F::PT / 2];
        uint32_t yoff[F::TPW];
#pragma unroll
        for (int m = 0; m < F::TPW; ++m) {
            const int T = tile_of(m, w);
            const int tl0 = 16 * T;
            const int t = tl0 + r16;
            const bool tv = t < qlen;
            const int nsb = T / 2;
            // a slot without rows computes nothing; the epilogue still runs (its stores
            // fall outside the chunk's rows and are dropped) so that every wave issues
            // the same stores on every path
            if (slot_ok[m] && !fast) {
                // exact fallback: entering state decays by 2^acum_t; every score tile
                // (off-diagonal and the masked diagonal one) is multiplied element by
                // element by dt_s 2^(acum_t - acum_s) and contracted with x as given
                const float at = acum[t];
                const float e0 = tv ? exp2_dec(at) : 0.f;
#pragma unroll
                for (int pt = 0; pt < F::PT; ++pt) acc[m][pt] *= e0;
                // a rolled loop (rare path, kept small): the score fragment of block S
                // is picked from the register array with a static select chain
#pragma unroll 1
                for (int S = 0; S <= nsb; ++S) {
                    uint4 gsrc = gfrag[m][0];
#pragma unroll
                    for (int k = 1; k < kSlots && k < F::NSB; ++k)
                        if (k == S) gsrc = gfrag[m][k];
                    float mv[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int s = 32 * S + (j < 4 ? 4 * g4 + j : 16 + 4 * g4 + j - 4);
                        const uint32_t wd = (&gsrc.x)[j >> 1];
                        const float gv = (j & 1) ? bf16_hi(wd) : bf16_lo(wd);
                        mv[j] = (tv && s <= t) ? gv * exp2_dec(at - acum[s]) * dts[s] : 0.f;
                    }
                    const bf16x8 mop = as_bf16x8(make_uint4(pack_bf16x2(mv[0], mv[1]),
                                                            pack_bf16x2(mv[2], mv[3]),
                                                            pack_bf16x2(mv[4], mv[5]),
                                                            pack_bf16x2(mv[6], mv[7])));
#pragma unroll
                    for (int pt = 0; pt < F::PT; ++pt) {
                        // x as given, channel pt * 16 + r16, the fragment's eight tokens
                        const int c = pt * 16 + r16, s0 = 32 * S + 4 * g4;
                        uint32_t xw[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int s = s0 + (q < 2 ? 2 * q : 16 + 2 * (q - 2));
                            xw[q] = uint32_t(XN[xn_off(s, c)]) | (uint32_t(XN[xn_off(s + 1, c)]) << 16);
                        }
                        acc[m][pt] = mfma_bf16(as_bf16x8(make_uint4(xw[0], xw[1], xw[2], xw[3])),
                                               mop, acc[m][pt]);
                    }
                }
            }
            // epilogue: + D x, round to bf16 (stored after the loop).  The stores go
            // through a buffer resource that covers the chunk's qlen rows: rows past
            // them are dropped by the range check, so no lane or wave branches around a
            // store (and the compiler can count the stores in flight when it waits for
            // the next head's x).  Streaming (non-temporal): y is not read again here.
            {
                uint2 xd[F::PT];   // x[t][p0 .. p0+3]
                const int tx = min(t, Q - 1);
#pragma unroll
                for (int pt = 0; pt < F::PT; ++pt)
                    xd[pt] = *reinterpret_cast<const uint2 *>(XN + xn_off(tx, pt * 16 + 4 * g4));
                const uint32_t row_off = uint32_t((t * H + h) * P) * 2u;
                uint32_t v[F::PT][2];   // bf16 pairs of channels pt*16 + 4*g4 + 0..3
#pragma unroll
                for (int pt = 0; pt < F::PT; ++pt) {
                    float o[4];
                    o[0] = acc[m][pt][0] + Dh * bf16_lo(xd[pt].x);
                    o[1] = acc[m][pt][1] + Dh * bf16_hi(xd[pt].x);
                    o[2] = acc[m][pt][2] + Dh * bf16_lo(xd[pt].y);
                    o[3] = acc[m][pt][3] + Dh * bf16_hi(xd[pt].y);
                    v[pt][0] = pack_bf16x2(o[0], o[1]);
                    v[pt][1] = pack_bf16x2(o[2], o[3]);
                }
                // regroup channel tiles pt, pt+1 between lane rows (v_permlane16_swap:
                // odd rows of the first operand trade places with even rows of the
                // second) so that each lane holds 8 consecutive channels: row g4 gets
                // channels (pt + (g4 & 1)) * 16 + (g4 >> 1) * 8 + 0..7, and the four
                // lanes of a token write 64 contiguous bytes per store
#pragma unroll
                for (int pt = 0; pt < F::PT; pt += 2) {
                    const auto s0 = __builtin_amdgcn_permlane16_swap(v[pt][0], v[pt + 1][0], false, false);
                    const auto s1 = __builtin_amdgcn_permlane16_swap(v[pt][1], v[pt + 1][1], false, false);
                    yq[m][pt / 2] = u32x4{s0[0], s1[0], s0[1], s1[1]};
                }
                yoff[m] = row_off;
            }
        }
#pragma unroll
        for (int m = 0; m < F::TPW; ++m)
#pragma unroll
            for (int pt = 0; pt < F::PT; pt += 2) {
                const int c0 = (pt + (g4 & 1)) * 16 + (g4 >> 1) * 8;
                __builtin_amdgcn_raw_buffer_store_b128(yq[m][pt / 2], yres, int(yoff[m] + 2u * c0), 0,
                                                       kBufNonTemporal);
            }
        __syncthreads();
    }
}

// Heads per workgroup.  A workgroup computes the chunk's score tiles once and then runs
// its HB heads one after another, so a larger HB amortises the item prologue (ticket,
// B and C loads, score tiles) but makes fewer, longer work items.  Items run from nq
// queues (one per XCD), each with slots / nq resident workgroups and at most
// ceil(chains / nq) chains; the estimate in head-times is
//   ceil(items of a queue / its slots) * (prologue + HB)
//     + (chunks of one chain in flight - 1) * link,
// the second term being the fill of the chunk-to-chunk hand-off chain.  A partial last
// round costs a whole one (measured: at L2k, 8 heads per workgroup leave 40 items for
// the 32 CUs of an XCD and take 118 us against 89 us with 10).  With one workgroup per
// CU nothing covers the prologue: timestamps put it at about 1.15 head times and a
// chain link at about 0.2.  With two per CU the other workgroup covers part of the
// prologue and of the link, and 1.0 and 0.1 fit the measurements.  HB ranges over the
// divisors of H / G up to 16 (a block never straddles two groups); ties go to the
// smaller HB.
int heads_per_workgroup(int b, int H, int G, int nc, int slots, int wg_per_cu, int nq) {
    const double prologue = wg_per_cu == 1 ? 1.15 : 1.0;
    const double link = wg_per_cu == 1 ? 0.2 : 0.1;
    const int hpg = H / G;
    const double qslots = std::max(1.0, double(slots) / nq);
    int best = 1;
    double best_t = 0.0;
    for (int hb = 1; hb <= 16 && hb <= hpg; ++hb) {
        if (hpg % hb) continue;
        const double qchains = std::ceil(double(b) * (H / hb) / nq);
        const double rounds = std::ceil(qchains * nc / qslots);
        const double inflight = std::min(double(nc), std::ceil(qslots / qchains));
        const double t = rounds * (prologue + hb) + (inflight - 1.0) * link;
        if (hb == 1 || t < best_t - 1e-9) {
            best = hb;
            best_t = t;
        }
    }
    return best;
}

// Per-device values the launch needs, read from the runtime once per device and then
// kept: the CU count, and whether the kernel's LDS limit has been raised.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

hipError_t device_cu_count(int dev, int *cus) {
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = g_cu_count[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cus = c;
            return hipSuccess;
        }
    }
    const hipError_t e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess && dev >= 0 && dev < kMaxDevices && *cus > 0)
        g_cu_count[dev].store(*cus, std::memory_order_relaxed);
    return e;
}

// The number of XCDs of the device (the work queues of the single-pass kernel): 1, 2, 4
// or 8, as the runtime reports it; anything else counts as 1.
std::atomic<int> g_xcc_count[kMaxDevices];

hipError_t device_xcc_count(int dev, int *nq) {
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = g_xcc_count[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *nq = c;
            return hipSuccess;
        }
    }
    int n = 1;
    const hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev);
    if (e != hipSuccess) return e;
    *nq = (n == 1 || n == 2 || n == 4 || n == 8) ? n : 1;
    if (dev >= 0 && dev < kMaxDevices) g_xcc_count[dev].store(*nq, std::memory_order_relaxed);
    return hipSuccess;
}

template <int Q, int N>
hipError_t launch_fused_qn(const ChunkScanArgs &a, const FusedPlan &fp, hipStream_t stream) {
    using F = Fz<Q, N>;
    static std::atomic<bool> lds_set[kMaxDevices];
    char *ws = static_cast<char *>(a.workspace);
    uint32_t *hdr = reinterpret_cast<uint32_t *>(ws + fp.off_hdr);
    uint32_t *flags = reinterpret_cast<uint32_t *>(ws + fp.off_flags);
    float *hbuf = reinterpret_cast<float *>(ws + fp.off_hbuf);
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < kMaxDevices;
    if (!cached || !lds_set[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_ssd_fused<Q, N>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(F::kLds));
        if (e != hipSuccess) return e;
        if (cached) lds_set[dev].store(true, std::memory_order_release);
    }
    e = device_cu_count(dev, &cus);
    if (e != hipSuccess) return e;
    int nq = 1;
    e = device_xcc_count(dev, &nq);
    if (e != hipSuccess) return e;
    const int HB = heads_per_workgroup(a.b, a.H, a.G, fp.nc, std::max(1, cus) * F::kWgPerCu,
                                       F::kWgPerCu, nq);
    const int nchains = a.b * (a.H / HB);
    // every XCD gets as many workgroups as the longest queue has items
    const unsigned items = unsigned(nq) * unsigned((nchains + nq - 1) / nq) * unsigned(fp.nc);
    hipLaunchKernelGGL((k_ssd_fused<Q, N>), dim3(items), dim3(kFT), F::kLds, stream,
                       static_cast<const bf16_bits *>(a.x), a.dt, a.A,
                       static_cast<const bf16_bits *>(a.B), static_cast<const bf16_bits *>(a.C),
                       a.D, a.init_state, static_cast<bf16_bits *>(a.y), a.final_state, hbuf,
                       flags, hdr, a.L, a.H, a.G, HB, nchains, fp.nc, nq);
    return hipGetLastError();
}

template <int Q>
hipError_t launch_fused_q(const ChunkScanArgs &a, const FusedPlan &fp, hipStream_t stream) {
    switch (a.N) {
        case 16: return launch_fused_qn<Q, 16>(a, fp, stream);
        case 32: return launch_fused_qn<Q, 32>(a, fp, stream);
        case 64: return launch_fused_qn<Q, 64>(a, fp, stream);
        case 128: return launch_fused_qn<Q, 128>(a, fp, stream);
        case 256:
            if constexpr (Fz<Q, 256>::kLds <= kMaxLds && Fz<Q, 256>::kBnatFits)
                return launch_fused_qn<Q, 256>(a, fp, stream);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

template <int Q, int N>
size_t fused_lds() { return Fz<Q, N>::kBnatFits ? Fz<Q, N>::kLds : size_t(-1); }

size_t fused_lds_bytes(int Q, int N) {
#define SSD_LDS_CASE(q)                                  \
    if (Q == q) {                                        \
        switch (N) {                                     \
            case 16: return fused_lds<q, 16>();          \
            case 32: return fused_lds<q, 32>();          \
            case 64: return fused_lds<q, 64>();          \
            case 128: return fused_lds<q, 128>();        \
            case 256: return fused_lds<q, 256>();        \
        }                                                \
    }
    SSD_LDS_CASE(64)
    SSD_LDS_CASE(128)
    SSD_LDS_CASE(256)
#undef SSD_LDS_CASE
    return size_t(-1);
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

namespace {
__global__ void k_workspace_init(uint32_t *ws, size_t words) {
    const size_t stride = size_t(gridDim.x) * blockDim.x;
    for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < words; i += stride)
        ws[i] = i == size_t(kWsMagicWord) ? kWsMagic : 0u;
}
}  // namespace

namespace {
// One lane copies the header's time-out error word to the caller's word and, when
// asked, clears it (device-scope accesses, as the scan's own writer uses).
__global__ void k_workspace_error(uint32_t *hdr, int32_t *err_out, int clear) {
    if (threadIdx.x != 0) return;
    const uint32_t v =
        __hip_atomic_load(&hdr[kWsErrorWord], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    err_out[0] = int32_t(v);
    if (clear) __hip_atomic_store(&hdr[kWsErrorWord], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
}  // namespace

hipError_t launch_workspace_error(void *workspace, int32_t *err_out, bool clear,
                                  hipStream_t stream) {
    hipLaunchKernelGGL(k_workspace_error, dim3(1), dim3(64), 0, stream,
                       static_cast<uint32_t *>(workspace), err_out, clear ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_workspace_init(void *workspace, size_t bytes, hipStream_t stream) {
    const size_t words = bytes / 4;
    if (words == 0) return hipSuccess;
    const size_t blocks = std::min<size_t>((words + 255) / 256, 4096);
    hipLaunchKernelGGL(k_workspace_init, dim3(unsigned(blocks)), dim3(256), 0, stream,
                       static_cast<uint32_t *>(workspace), words);
    return hipGetLastError();
}

FusedPlan plan_fused(int b, int L, int H, int P, int N, int G, int Q, bool bf16) {
    FusedPlan fp;
    if (!bf16 || P != 64 || b <= 0 || L <= 0) return fp;
    if (Q != 64 && Q != 128 && Q != 256) return fp;
    if (N != 16 && N != 32 && N != 64 && N != 128 && N != 256) return fp;
    if (G <= 0 || H % G != 0) return fp;
    const size_t lds = fused_lds_bytes(Q, N);
    if (lds > kMaxLds) return fp;
    fp.HB = 1;   // the launch picks the heads per workgroup for the device it runs on
    fp.nc = (L + Q - 1) / Q;
    const size_t items = size_t(b) * H * fp.nc;   // upper bound (one head per workgroup)
    if (items > 0x7fffffffu) return fp;
    fp.off_hdr = 0;
    fp.off_flags = kWsHeaderBytes;
    fp.off_hbuf = fp.off_flags + align256(size_t(b) * H * fp.nc * 4);
    fp.total = fp.off_hbuf + align256(size_t(b) * H * 2 * size_t(P) * N * 4);
    fp.lds = lds;
    fp.supported = true;
    return fp;
}

hipError_t launch_fused(const ChunkScanArgs &a, const FusedPlan &fp, hipStream_t stream) {
    switch (a.Q) {
        case 64: return launch_fused_q<64>(a, fp, stream);
        case 128: return launch_fused_q<128>(a, fp, stream);
        case 256: return launch_fused_q<256>(a, fp, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
