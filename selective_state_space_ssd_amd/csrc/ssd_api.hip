// ssd_api.hip -- the C ABI declared in include/ssd_mi355x.h: host-side argument
// checks, workspace planning and dispatch to the gfx950 kernels.  Every check runs
// before anything is enqueued; a failed check enqueues nothing.
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "ssd_kernels.h"
#include "ssd_mi355x.h"

namespace {

// Workspace of ssd_chunk_scan_fwd_noalloc: a file-scope device array, one copy per GPU,
// placed in device memory when the code object is loaded (nothing is allocated at run
// time).  Host code uses the device address hipGetSymbolAddress returns for the
// current device, never the array's name.
constexpr size_t kNoallocBytes = SSD_NOALLOC_WORKSPACE_BYTES;
__device__ __align__(256) unsigned char scratch[kNoallocBytes];
constexpr int kNoallocDevices = 64;
std::mutex g_noalloc_mu;
std::atomic<void *> g_noalloc_ptr[kNoallocDevices];

// The current device's copy of `scratch`.  The first call on a device looks up its
// address and prepares it (fill kernel on `stream`: zeroes, marker word); a stream
// being captured cannot take that first preparation.
ssd_status_t noalloc_workspace(hipStream_t stream, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SSD_ERR_HIP;
    if (dev < 0 || dev >= kNoallocDevices) return SSD_ERR_UNSUPPORTED;
    void *p = g_noalloc_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_noalloc_mu);
        p = g_noalloc_ptr[dev].load(std::memory_order_acquire);
        if (!p) {
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return SSD_ERR_HIP;
            if (cs != hipStreamCaptureStatusNone) return SSD_ERR_UNSUPPORTED;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return SSD_ERR_HIP;
            if (ssd::launch_workspace_init(p, kNoallocBytes, stream) != hipSuccess)
                return SSD_ERR_HIP;
            g_noalloc_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return SSD_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    uintptr_t lo = 0, hi = 0;   // [lo, hi); empty when lo == hi
    Range() = default;
    Range(const void *p, size_t bytes)
        : lo(reinterpret_cast<uintptr_t>(p)), hi(reinterpret_cast<uintptr_t>(p) + (p ? bytes : 0)) {}
    bool overlaps(const Range &o) const { return lo < o.hi && o.lo < hi; }
    bool same(const Range &o) const { return lo == o.lo && hi == o.hi; }
};

}  // namespace

extern "C" {

const char *ssd_status_string(ssd_status_t s) {
    switch (s) {
        case SSD_OK: return "SSD_OK";
        case SSD_ERR_NULL_ARG: return "SSD_ERR_NULL_ARG: a required pointer is NULL";
        case SSD_ERR_BAD_DIM: return "SSD_ERR_BAD_DIM: invalid dimension";
        case SSD_ERR_GROUPS: return "SSD_ERR_GROUPS: H is not a multiple of G";
        case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED: shape, chunk size or dtype not supported";
        case SSD_ERR_ALIGN: return "SSD_ERR_ALIGN: pointer not suitably aligned";
        case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace missing or too small";
        case SSD_ERR_ALIAS: return "SSD_ERR_ALIAS: output overlaps an input";
        case SSD_ERR_HIP: return "SSD_ERR_HIP: HIP runtime error";
    }
    return "unknown ssd_status_t";
}

const char *ssd_version(void) { return "ssd_mi355x 0.1.0 gfx950"; }

size_t ssd_chunk_scan_workspace_bytes(int b, int L, int H, int P, int N, int G, int Q,
                                      ssd_dtype_t io) {
    if (b < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || Q <= 0) return size_t(-1);
    if (io != SSD_DTYPE_F32 && io != SSD_DTYPE_BF16) return size_t(-1);
    if (b == 0 || L == 0) return 0;
    const bool bf16 = io == SSD_DTYPE_BF16;
    const ssd::FusedPlan fp = ssd::plan_fused(b, L, H, P, N, G, Q, bf16);
    if (fp.supported) return fp.total;
    return ssd::plan_chunk_scan(b, L, H, P, N, G, Q, bf16).total;
}

ssd_status_t ssd_chunk_scan_workspace_init(void *workspace, size_t workspace_bytes,
                                           void *hip_stream) {
    if (workspace_bytes == 0) return SSD_OK;
    if (!workspace) return SSD_ERR_NULL_ARG;
    if (!aligned(workspace, 16)) return SSD_ERR_ALIGN;
    const hipError_t e = ssd::launch_workspace_init(workspace, workspace_bytes,
                                                    static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

ssd_status_t ssd_chunk_scan_workspace_error(void *workspace, size_t workspace_bytes,
                                            int32_t *err_out, int clear, void *hip_stream) {
    if (!workspace || !err_out) return SSD_ERR_NULL_ARG;
    if (!aligned(workspace, 16) || !aligned(err_out, 4)) return SSD_ERR_ALIGN;
    if (workspace_bytes < ssd::kWsHeaderBytes) return SSD_ERR_WORKSPACE;
    if (Range(workspace, ssd::kWsHeaderBytes).overlaps(Range(err_out, 4))) return SSD_ERR_ALIAS;
    const hipError_t e = ssd::launch_workspace_error(workspace, err_out, clear != 0,
                                                     static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // extern "C"

namespace {

// Argument checks of a chunk-scan call, everything but the workspace; on SSD_OK the
// plan of the path the call takes and the workspace it needs (0 for an empty problem).
struct ScanPlan {
    ssd::FusedPlan fplan;
    ssd::ChunkScanPlan plan;
    size_t ws_need = 0;
    bool empty = false;
};

ssd_status_t check_scan(const void *x, const float *dt, const float *A, const void *B,
                        const void *C, const float *D, const float *init_state, const void *y,
                        const float *final_state, int b, int L, int H, int P, int N, int G,
                        int Q, ssd_dtype_t io, ScanPlan *sp) {
    if (io != SSD_DTYPE_F32 && io != SSD_DTYPE_BF16) return SSD_ERR_UNSUPPORTED;
    if (b < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || Q <= 0) return SSD_ERR_BAD_DIM;
    if (H % G != 0) return SSD_ERR_GROUPS;
    const size_t state_bytes = size_t(b) * H * P * N * sizeof(float);
    if (b == 0 || L == 0) {   // empty sequence: final state is the initial state
        sp->empty = true;
        if (final_state && b > 0) {
            if (!aligned(final_state, 16) || (init_state && !aligned(init_state, 16)))
                return SSD_ERR_ALIGN;
            if (init_state && Range(init_state, state_bytes).overlaps(Range(final_state, state_bytes)) &&
                !Range(init_state, state_bytes).same(Range(final_state, state_bytes)))
                return SSD_ERR_ALIAS;
        }
        return SSD_OK;
    }
    if (!x || !dt || !A || !B || !C || !D || !y) return SSD_ERR_NULL_ARG;
    const bool bf16 = io == SSD_DTYPE_BF16;
    sp->fplan = ssd::plan_fused(b, L, H, P, N, G, Q, bf16);
    sp->plan = ssd::plan_chunk_scan(b, L, H, P, N, G, Q, bf16);
    if (!sp->fplan.supported && !sp->plan.supported) return SSD_ERR_UNSUPPORTED;
    sp->ws_need = sp->fplan.supported ? sp->fplan.total : sp->plan.total;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(y, 16) ||
        !aligned(init_state, 16) || !aligned(final_state, 16) || !aligned(dt, 4) ||
        !aligned(A, 4) || !aligned(D, 4))
        return SSD_ERR_ALIGN;
    const size_t esz = bf16 ? 2 : 4;
    const Range rx(x, size_t(b) * L * H * P * esz), ry(y, size_t(b) * L * H * P * esz);
    const Range rB(B, size_t(b) * L * G * N * esz), rC(C, size_t(b) * L * G * N * esz);
    const Range rdt(dt, size_t(b) * L * H * 4), rA(A, size_t(H) * 4), rD(D, size_t(H) * 4);
    const Range rinit(init_state, state_bytes), rfin(final_state, state_bytes);
    const Range inputs[] = {rx, rB, rC, rdt, rA, rD, rinit};
    for (const Range &in : inputs) {
        if (ry.overlaps(in)) return SSD_ERR_ALIAS;
        // final_state may replace init_state in place, but may not clobber other inputs
        if (&in != &inputs[6] && rfin.overlaps(in)) return SSD_ERR_ALIAS;
    }
    if (rfin.overlaps(rinit) && !rfin.same(rinit)) return SSD_ERR_ALIAS;
    if (ry.overlaps(rfin)) return SSD_ERR_ALIAS;
    return SSD_OK;
}

// Enqueue a checked call on `workspace` (checked by the caller too).
ssd_status_t run_scan(const void *x, const float *dt, const float *A, const void *B,
                      const void *C, const float *D, const float *init_state, void *y,
                      float *final_state, int b, int L, int H, int P, int N, int G, int Q,
                      ssd_dtype_t io, const ScanPlan &sp, void *workspace, hipStream_t stream) {
    if (sp.empty) {
        if (final_state && b > 0 &&
            ssd::launch_copy_state(init_state, final_state, size_t(b) * H * P * N, stream) !=
                hipSuccess)
            return SSD_ERR_HIP;
        return SSD_OK;
    }
    ssd::ChunkScanArgs a;
    a.x = x; a.dt = dt; a.A = A; a.B = B; a.C = C; a.D = D;
    a.init_state = init_state; a.y = y; a.final_state = final_state;
    a.b = b; a.L = L; a.H = H; a.P = P; a.N = N; a.G = G; a.Q = Q;
    a.bf16 = io == SSD_DTYPE_BF16;
    a.workspace = workspace;
    const hipError_t e = sp.fplan.supported ? ssd::launch_fused(a, sp.fplan, stream)
                                            : ssd::launch_chunk_scan(a, sp.plan, stream);
    return e == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

}  // namespace

extern "C" {

ssd_status_t ssd_chunk_scan_fwd(const void *x, const float *dt, const float *A, const void *B,
                                const void *C, const float *D, const float *init_state, void *y,
                                float *final_state, int b, int L, int H, int P, int N, int G,
                                int Q, ssd_dtype_t io, void *workspace, size_t workspace_bytes,
                                void *hip_stream) {
    ScanPlan sp;
    ssd_status_t st = check_scan(x, dt, A, B, C, D, init_state, y, final_state, b, L, H, P, N,
                                 G, Q, io, &sp);
    if (st != SSD_OK) return st;
    if (!sp.empty) {
        if (!aligned(workspace, 16)) return SSD_ERR_ALIGN;
        if (!workspace || workspace_bytes < sp.ws_need) return SSD_ERR_WORKSPACE;
        const size_t esz = io == SSD_DTYPE_BF16 ? 2 : 4;
        const size_t state_bytes = size_t(b) * H * P * N * sizeof(float);
        const Range rws(workspace, sp.ws_need);
        const Range others[] = {
            Range(x, size_t(b) * L * H * P * esz), Range(y, size_t(b) * L * H * P * esz),
            Range(B, size_t(b) * L * G * N * esz), Range(C, size_t(b) * L * G * N * esz),
            Range(dt, size_t(b) * L * H * 4), Range(A, size_t(H) * 4), Range(D, size_t(H) * 4),
            Range(init_state, state_bytes), Range(final_state, state_bytes)};
        for (const Range &o : others)
            if (rws.overlaps(o)) return SSD_ERR_ALIAS;
    }
    return run_scan(x, dt, A, B, C, D, init_state, y, final_state, b, L, H, P, N, G, Q, io, sp,
                    workspace, static_cast<hipStream_t>(hip_stream));
}

ssd_status_t ssd_chunk_scan_fwd_noalloc(const void *x, const float *dt, const float *A,
                                        const void *B, const void *C, const float *D,
                                        const float *init_state, void *y, float *final_state,
                                        int b, int L, int H, int P, int N, int G, int Q,
                                        ssd_dtype_t io, void *hip_stream) {
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    ScanPlan sp;
    ssd_status_t st = check_scan(x, dt, A, B, C, D, init_state, y, final_state, b, L, H, P, N,
                                 G, Q, io, &sp);
    if (st != SSD_OK) return st;
    void *ws = nullptr;
    if (!sp.empty) {
        if (sp.ws_need > kNoallocBytes) return SSD_ERR_WORKSPACE;
        st = noalloc_workspace(stream, &ws);
        if (st != SSD_OK) return st;
    }
    return run_scan(x, dt, A, B, C, D, init_state, y, final_state, b, L, H, P, N, G, Q, io, sp,
                    ws, stream);
}

ssd_status_t ssd_verify_step(const float *state_in, const void *x, const float *dt,
                             const float *A, const void *B, const void *C, const float *D,
                             const int32_t *accept_len, void *y, float *state_out,
                             float *states_all, int32_t *err_flag, int b, int K, int H, int P,
                             int N, int G, ssd_dtype_t io, void *hip_stream) {
    if (io != SSD_DTYPE_F32 && io != SSD_DTYPE_BF16) return SSD_ERR_UNSUPPORTED;
    if (b < 0 || K <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0) return SSD_ERR_BAD_DIM;
    if (H % G != 0) return SSD_ERR_GROUPS;
    if (K > 16 || !ssd::verify_supported_n(N) || H > 65535 || b > 65535)
        return SSD_ERR_UNSUPPORTED;
    if (b == 0) return SSD_OK;
    if (!state_in || !x || !dt || !A || !B || !C || !D || !accept_len || !y || !state_out)
        return SSD_ERR_NULL_ARG;
    const bool bf16 = io == SSD_DTYPE_BF16;
    const size_t esz = bf16 ? 2 : 4;
    if (!aligned(state_in, 16) || !aligned(state_out, 16) || !aligned(states_all, 16) ||
        !aligned(B, 16) || !aligned(C, 16) || !aligned(x, esz) || !aligned(y, esz) ||
        !aligned(dt, 4) || !aligned(A, 4) || !aligned(D, 4) || !aligned(accept_len, 4) ||
        !aligned(err_flag, 4))
        return SSD_ERR_ALIGN;

    const size_t state_bytes = size_t(b) * H * P * N * 4;
    const Range rin(state_in, state_bytes), rout(state_out, state_bytes);
    const Range rall(states_all, state_bytes * K);
    const Range rx(x, size_t(b) * K * H * P * esz), ry(y, size_t(b) * K * H * P * esz);
    const Range rB(B, size_t(b) * K * G * N * esz), rC(C, size_t(b) * K * G * N * esz);
    const Range rdt(dt, size_t(b) * K * H * 4), rA(A, size_t(H) * 4), rD(D, size_t(H) * 4);
    const Range racc(accept_len, size_t(b) * 4), rerr(err_flag, 4);
    if (rout.overlaps(rin) && !rout.same(rin)) return SSD_ERR_ALIAS;
    const Range others[] = {rx, rB, rC, rdt, rA, rD, racc};
    const Range outs[] = {rout, rall, ry, rerr};
    for (const Range &o : outs)
        for (const Range &i : others)
            if (o.overlaps(i)) return SSD_ERR_ALIAS;
    if (rall.overlaps(rin) || rall.overlaps(rout) || ry.overlaps(rin) || ry.overlaps(rout) ||
        ry.overlaps(rall) || rerr.overlaps(rin) || rerr.overlaps(rout) || rerr.overlaps(rall) ||
        rerr.overlaps(ry))
        return SSD_ERR_ALIAS;

    ssd::VerifyArgs a;
    a.state_in = state_in; a.x = x; a.dt = dt; a.A = A; a.B = B; a.C = C; a.D = D;
    a.accept_len = accept_len; a.y = y; a.state_out = state_out; a.states_all = states_all;
    a.err_flag = err_flag;
    a.b = b; a.K = K; a.H = H; a.P = P; a.N = N; a.G = G;
    a.bf16 = bf16;
    if (ssd::launch_verify(a, static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return SSD_ERR_HIP;
    return SSD_OK;
}

ssd_status_t ssd_verify_ring_init(float *ring, int32_t *meta, const float *init_state, int b,
                                  int R, int H, int P, int N, void *hip_stream) {
    if (b < 0 || R < 2 || H <= 0 || P <= 0 || N <= 0) return SSD_ERR_BAD_DIM;
    if (b > 65535) return SSD_ERR_UNSUPPORTED;
    if (b == 0) return SSD_OK;
    if (!ring || !meta) return SSD_ERR_NULL_ARG;
    if (!aligned(ring, 16) || !aligned(init_state, 4) || !aligned(meta, 4)) return SSD_ERR_ALIGN;
    const size_t slot = size_t(H) * P * N;
    const Range rr(ring, size_t(b) * R * slot * 4), ri(init_state, size_t(b) * slot * 4);
    const Range rm(meta, size_t(b) * 8);
    if (rr.overlaps(ri) || rr.overlaps(rm) || rm.overlaps(ri)) return SSD_ERR_ALIAS;
    if (ssd::launch_ring_init(ring, meta, init_state, b, R, slot,
                              static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return SSD_ERR_HIP;
    return SSD_OK;
}

ssd_status_t ssd_verify_ring(float *ring, int32_t *meta, const void *x, const float *dt,
                             const float *dt_bias, const float *A, const void *B, const void *C,
                             const float *D, const int32_t *accept_len, void *y,
                             int32_t *err_flag, int b, int K, int R, int H, int P, int N, int G,
                             ssd_dtype_t io, void *hip_stream) {
    if (io != SSD_DTYPE_F32 && io != SSD_DTYPE_BF16) return SSD_ERR_UNSUPPORTED;
    if (b < 0 || K <= 0 || R <= K || H <= 0 || P <= 0 || N <= 0 || G <= 0) return SSD_ERR_BAD_DIM;
    if (H % G != 0) return SSD_ERR_GROUPS;
    if (K > 16 || !ssd::verify_supported_n(N) || H > 65535 || b > 65535)
        return SSD_ERR_UNSUPPORTED;
    if (b == 0) return SSD_OK;
    if (!ring || !meta || !x || !dt || !A || !B || !C || !D || !accept_len || !y)
        return SSD_ERR_NULL_ARG;
    const bool bf16 = io == SSD_DTYPE_BF16;
    const size_t esz = bf16 ? 2 : 4;
    if (!aligned(ring, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(x, esz) ||
        !aligned(y, esz) || !aligned(dt, 4) || !aligned(dt_bias, 4) || !aligned(A, 4) ||
        !aligned(D, 4) || !aligned(accept_len, 4) || !aligned(err_flag, 4) || !aligned(meta, 4))
        return SSD_ERR_ALIGN;
    const Range rring(ring, size_t(b) * R * H * P * N * 4), rmeta(meta, size_t(b) * 8);
    const Range rx(x, size_t(b) * K * H * P * esz), ry(y, size_t(b) * K * H * P * esz);
    const Range rB(B, size_t(b) * K * G * N * esz), rC(C, size_t(b) * K * G * N * esz);
    const Range rdt(dt, size_t(b) * K * H * 4), rbias(dt_bias, size_t(H) * 4);
    const Range rA(A, size_t(H) * 4), rD(D, size_t(H) * 4);
    const Range racc(accept_len, size_t(b) * 4), rerr(err_flag, 4);
    const Range ins[] = {rx, rB, rC, rdt, rbias, rA, rD, racc};
    const Range outs[] = {rring, rmeta, ry, rerr};
    for (int i = 0; i < 4; ++i) {
        for (const Range &in : ins)
            if (outs[i].overlaps(in)) return SSD_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (outs[i].overlaps(outs[j])) return SSD_ERR_ALIAS;
    }
    ssd::VerifyArgs a;
    a.state_in = nullptr; a.x = x; a.dt = dt; a.A = A; a.B = B; a.C = C; a.D = D;
    a.accept_len = accept_len; a.y = y; a.state_out = nullptr; a.states_all = nullptr;
    a.err_flag = err_flag;
    a.b = b; a.K = K; a.H = H; a.P = P; a.N = N; a.G = G;
    a.bf16 = bf16;
    a.ring = ring; a.meta = meta; a.R = R; a.dt_bias = dt_bias;
    const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (ssd::launch_verify(a, stream) != hipSuccess) return SSD_ERR_HIP;
    if (ssd::launch_ring_advance(meta, accept_len, b, K, R, stream) != hipSuccess)
        return SSD_ERR_HIP;
    return SSD_OK;
}

ssd_status_t ssd_verify_ring_rollback(int32_t *meta, const int32_t *steps, int32_t *err_flag,
                                      int b, int R, void *hip_stream) {
    if (b < 0 || R < 2) return SSD_ERR_BAD_DIM;
    if (b == 0) return SSD_OK;
    if (!meta || !steps) return SSD_ERR_NULL_ARG;
    if (!aligned(meta, 4) || !aligned(steps, 4) || !aligned(err_flag, 4)) return SSD_ERR_ALIGN;
    const Range rm(meta, size_t(b) * 8), rs(steps, size_t(b) * 4), re(err_flag, 4);
    if (rm.overlaps(rs) || rm.overlaps(re) || rs.overlaps(re)) return SSD_ERR_ALIAS;
    if (ssd::launch_ring_rollback(meta, steps, err_flag, b, R,
                                  static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return SSD_ERR_HIP;
    return SSD_OK;
}

ssd_status_t ssd_seq_total_decay(const float *dt, const float *A, float *alpha, int b, int L,
                                 int H, void *hip_stream) {
    if (b < 0 || L < 0 || H <= 0) return SSD_ERR_BAD_DIM;
    if (b > 65535) return SSD_ERR_UNSUPPORTED;
    if (b == 0) return SSD_OK;
    if (!A || !alpha || (L > 0 && !dt)) return SSD_ERR_NULL_ARG;
    if (!aligned(dt, 4) || !aligned(A, 4) || !aligned(alpha, 4)) return SSD_ERR_ALIGN;
    const Range ra(alpha, size_t(b) * H * 4);
    if (ra.overlaps(Range(dt, size_t(b) * L * H * 4)) || ra.overlaps(Range(A, size_t(H) * 4)))
        return SSD_ERR_ALIAS;
    if (ssd::launch_seq_decay(dt, A, alpha, b, L, H, static_cast<hipStream_t>(hip_stream)) !=
        hipSuccess)
        return SSD_ERR_HIP;
    return SSD_OK;
}

size_t ssd_seq_slice_state_workspace_bytes(int b, int L, int H, int P, int N, int G,
                                           ssd_dtype_t io) {
    if (io != SSD_DTYPE_F32 && io != SSD_DTYPE_BF16) return size_t(-1);
    if (b < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return size_t(-1);
    const ssd::SliceStatePlan pl = ssd::plan_slice_state(b, L, H, P, N, G, io == SSD_DTYPE_BF16);
    return pl.supported ? pl.total : size_t(-1);
}

ssd_status_t ssd_seq_slice_state(const void *x, const float *dt, const float *A, const void *B,
                                 float *state, float *alpha, int b, int L, int H, int P, int N,
                                 int G, ssd_dtype_t io, void *workspace, size_t workspace_bytes,
                                 void *hip_stream) {
    if (io != SSD_DTYPE_F32 && io != SSD_DTYPE_BF16) return SSD_ERR_UNSUPPORTED;
    if (b < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0) return SSD_ERR_BAD_DIM;
    if (H % G != 0) return SSD_ERR_GROUPS;
    const bool bf16 = io == SSD_DTYPE_BF16;
    const ssd::SliceStatePlan pl = ssd::plan_slice_state(b, L, H, P, N, G, bf16);
    if (!pl.supported) return SSD_ERR_UNSUPPORTED;
    if (b == 0) return SSD_OK;
    if (!A || !state || !alpha || (L > 0 && (!x || !dt || !B))) return SSD_ERR_NULL_ARG;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(state, 16) || !aligned(dt, 4) ||
        !aligned(A, 4) || !aligned(alpha, 4) || !aligned(workspace, 16))
        return SSD_ERR_ALIGN;
    if (pl.total > 0 && (!workspace || workspace_bytes < pl.total)) return SSD_ERR_WORKSPACE;
    const size_t esz = bf16 ? 2 : 4;
    const Range rs(state, size_t(b) * H * P * N * 4), ra(alpha, size_t(b) * H * 4),
        rw(workspace, pl.total);
    const Range ins[] = {Range(x, size_t(b) * L * H * P * esz), Range(dt, size_t(b) * L * H * 4),
                         Range(A, size_t(H) * 4), Range(B, size_t(b) * L * G * N * esz)};
    for (const Range &in : ins)
        if (rs.overlaps(in) || ra.overlaps(in) || rw.overlaps(in)) return SSD_ERR_ALIAS;
    if (rs.overlaps(ra) || rs.overlaps(rw) || ra.overlaps(rw)) return SSD_ERR_ALIAS;
    if (ssd::launch_slice_state(x, dt, A, B, state, alpha, workspace, b, L, H, P, N, G, bf16, pl,
                                static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return SSD_ERR_HIP;
    return SSD_OK;
}

ssd_status_t ssd_seq_combine(const float *alpha, const float *S, const float *init_state,
                             float *h_in, int n, int b, int H, int P, int N, void *hip_stream) {
    if (n < 0 || b < 0 || H <= 0 || P <= 0 || N <= 0) return SSD_ERR_BAD_DIM;
    if ((size_t(P) * N) % 4 != 0 || H > 65535 || b > 65535) return SSD_ERR_UNSUPPORTED;
    if (n == 0 || b == 0) return SSD_OK;
    if (!alpha || !S || !h_in) return SSD_ERR_NULL_ARG;
    if (!aligned(alpha, 4) || !aligned(S, 16) || !aligned(init_state, 16) || !aligned(h_in, 16))
        return SSD_ERR_ALIGN;
    const size_t st = size_t(b) * H * P * N * 4;
    const Range rh(h_in, st * n);
    if (rh.overlaps(Range(alpha, size_t(n) * b * H * 4)) || rh.overlaps(Range(S, st * n)) ||
        rh.overlaps(Range(init_state, st)))
        return SSD_ERR_ALIAS;
    if (ssd::launch_seq_combine(alpha, S, init_state, h_in, n, b, H, P * N,
                                static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return SSD_ERR_HIP;
    return SSD_OK;
}

ssd_status_t ssd_seq_apply_state(void *y, float *final_state, const float *dt, const float *A,
                                 const void *C, const float *h_in, int b, int L, int H, int P,
                                 int N, int G, ssd_dtype_t io, void *hip_stream) {
    if (io != SSD_DTYPE_F32 && io != SSD_DTYPE_BF16) return SSD_ERR_UNSUPPORTED;
    if (b < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0) return SSD_ERR_BAD_DIM;
    if (H % G != 0) return SSD_ERR_GROUPS;
    if (P % 16 != 0 || P > 256 || N % 16 != 0 || N > 256 || H > 65535 || b > 65535)
        return SSD_ERR_UNSUPPORTED;
    if (b == 0) return SSD_OK;
    if (!A || !h_in || (L > 0 && (!y || !dt || !C))) return SSD_ERR_NULL_ARG;
    const bool bf16 = io == SSD_DTYPE_BF16;
    const size_t esz = bf16 ? 2 : 4;
    if (!aligned(y, 16) || !aligned(final_state, 4) || !aligned(dt, 4) || !aligned(A, 4) ||
        !aligned(C, 16) || !aligned(h_in, 16))
        return SSD_ERR_ALIGN;
    const size_t st = size_t(b) * H * P * N * 4;
    const Range ry(y, size_t(b) * L * H * P * esz), rf(final_state, st);
    const Range ins[] = {Range(dt, size_t(b) * L * H * 4), Range(A, size_t(H) * 4),
                         Range(C, size_t(b) * L * G * N * esz), Range(h_in, st)};
    for (const Range &in : ins)
        if (ry.overlaps(in) || rf.overlaps(in)) return SSD_ERR_ALIAS;
    if (ry.overlaps(rf)) return SSD_ERR_ALIAS;
    if (ssd::launch_seq_apply(y, final_state, dt, A, C, h_in, b, L, H, P, N, G, bf16,
                              static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return SSD_ERR_HIP;
    return SSD_OK;
}

ssd_status_t ssd_selective_scan_fwd(const void *x, const float *dt, const float *A, const void *B,
                                    const void *C, const float *D, const float *init_state,
                                    void *y, float *final_state, int b, int L, int Dch, int N,
                                    int G, ssd_dtype_t io, void *hip_stream) {
    if (io != SSD_DTYPE_F32 && io != SSD_DTYPE_BF16) return SSD_ERR_UNSUPPORTED;
    if (b < 0 || L < 0 || Dch <= 0 || N <= 0 || G <= 0) return SSD_ERR_BAD_DIM;
    if (Dch % G != 0) return SSD_ERR_GROUPS;
    const int dc = ssd::selective_channels_per_block(N);
    if (dc == 0 || (Dch / G) % dc != 0 || b > 65535) return SSD_ERR_UNSUPPORTED;
    const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    const size_t state_bytes = size_t(b) * Dch * N * 4;
    if (b == 0 || L == 0) {   // empty sequence: the final state is the initial one
        if (final_state && b > 0) {
            if (!aligned(final_state, 16) || !aligned(init_state, 16)) return SSD_ERR_ALIGN;
            const Range ri(init_state, state_bytes), rf(final_state, state_bytes);
            if (ri.overlaps(rf) && !ri.same(rf)) return SSD_ERR_ALIAS;
            if (ssd::launch_copy_state(init_state, final_state, state_bytes / 4, stream) != hipSuccess)
                return SSD_ERR_HIP;
        }
        return SSD_OK;
    }
    if (!x || !dt || !A || !B || !C || !D || !y) return SSD_ERR_NULL_ARG;
    const bool bf16 = io == SSD_DTYPE_BF16;
    const size_t esz = bf16 ? 2 : 4;
    if (!aligned(x, esz) || !aligned(y, esz) || !aligned(B, esz) || !aligned(C, esz) ||
        !aligned(dt, 4) || !aligned(D, 4) || !aligned(A, 16) || !aligned(init_state, 16) ||
        !aligned(final_state, 16))
        return SSD_ERR_ALIGN;
    const Range rx(x, size_t(b) * L * Dch * esz), ry(y, size_t(b) * L * Dch * esz);
    const Range rdt(dt, size_t(b) * L * Dch * 4), rA(A, size_t(Dch) * N * 4);
    const Range rB(B, size_t(b) * L * G * N * esz), rC(C, size_t(b) * L * G * N * esz);
    const Range rD(D, size_t(Dch) * 4), rinit(init_state, state_bytes), rfin(final_state, state_bytes);
    const Range inputs[] = {rx, rdt, rA, rB, rC, rD, rinit};
    for (const Range &in : inputs)
        if (ry.overlaps(in) || rfin.overlaps(in)) return SSD_ERR_ALIAS;
    if (ry.overlaps(rfin)) return SSD_ERR_ALIAS;
    ssd::SelectiveArgs a;
    a.x = x; a.dt = dt; a.A = A; a.B = B; a.C = C; a.D = D; a.init_state = init_state;
    a.y = y; a.final_state = final_state;
    a.b = b; a.L = L; a.Dch = Dch; a.N = N; a.G = G;
    a.bf16 = bf16;
    if (ssd::launch_selective_scan(a, stream) != hipSuccess) return SSD_ERR_HIP;
    return SSD_OK;
}

size_t ssd_chunk_scan_bwd_workspace_bytes(int b, int L, int H, int P, int N, int G,
                                          ssd_dtype_t io) {
    if (b < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0) return size_t(-1);
    if (io != SSD_DTYPE_F32 && io != SSD_DTYPE_BF16) return size_t(-1);
    if (b == 0 || L == 0) return 0;
    return ssd::plan_chunk_scan_bwd(b, L, H, P, N, G, io == SSD_DTYPE_BF16).total;
}

ssd_status_t ssd_chunk_scan_bwd(const void *x, const float *dt, const float *A, const void *B,
                                const void *C, const float *D, const float *init_state,
                                const void *dy, const float *d_final, void *dx, float *ddt,
                                float *dA, void *dB, void *dC, float *dD, float *d_init, int b,
                                int L, int H, int P, int N, int G, ssd_dtype_t io,
                                void *workspace, size_t workspace_bytes, void *hip_stream) {
    if (io != SSD_DTYPE_F32 && io != SSD_DTYPE_BF16) return SSD_ERR_UNSUPPORTED;
    if (b < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0) return SSD_ERR_BAD_DIM;
    if (H % G != 0) return SSD_ERR_GROUPS;
    if (!dA || !dD) return SSD_ERR_NULL_ARG;
    if (!aligned(dA, 4) || !aligned(dD, 4)) return SSD_ERR_ALIGN;
    const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    const size_t state_bytes = size_t(b) * H * P * N * 4;
    const Range rdA(dA, size_t(H) * 4), rdD(dD, size_t(H) * 4);
    if (rdA.overlaps(rdD)) return SSD_ERR_ALIAS;

    if (b == 0 || L == 0) {   // empty sequence: d_init = d_final, no parameter gradient
        const Range rdf(d_final, state_bytes), rdi(d_init, state_bytes);
        if (!aligned(d_final, 16) || !aligned(d_init, 16)) return SSD_ERR_ALIGN;
        if (rdi.overlaps(rdf) && !rdi.same(rdf)) return SSD_ERR_ALIAS;
        if (rdi.overlaps(rdA) || rdi.overlaps(rdD)) return SSD_ERR_ALIAS;
        if (ssd::launch_copy_state(nullptr, dA, size_t(H), stream) != hipSuccess ||
            ssd::launch_copy_state(nullptr, dD, size_t(H), stream) != hipSuccess)
            return SSD_ERR_HIP;
        if (d_init && b > 0 &&
            ssd::launch_copy_state(d_final, d_init, state_bytes / 4, stream) != hipSuccess)
            return SSD_ERR_HIP;
        return SSD_OK;
    }
    if (!x || !dt || !A || !B || !C || !D || !dy || !dx || !ddt || !dB || !dC)
        return SSD_ERR_NULL_ARG;
    const ssd::ChunkScanBwdPlan plan = ssd::plan_chunk_scan_bwd(b, L, H, P, N, G, io == SSD_DTYPE_BF16);
    if (!plan.supported) return SSD_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(dy, 16) ||
        !aligned(dx, 16) || !aligned(dB, 16) || !aligned(dC, 16) || !aligned(init_state, 16) ||
        !aligned(d_final, 16) || !aligned(d_init, 16) || !aligned(workspace, 16) ||
        !aligned(dt, 4) || !aligned(A, 4) || !aligned(D, 4) || !aligned(ddt, 4))
        return SSD_ERR_ALIGN;
    if (!workspace || workspace_bytes < plan.total) return SSD_ERR_WORKSPACE;

    const bool bf16 = io == SSD_DTYPE_BF16;
    const size_t esz = bf16 ? 2 : 4;
    const size_t xb = size_t(b) * L * H * P * esz, bcb = size_t(b) * L * G * N * esz;
    const Range inputs[] = {Range(x, xb), Range(dt, size_t(b) * L * H * 4), Range(A, size_t(H) * 4),
                            Range(B, bcb), Range(C, bcb), Range(D, size_t(H) * 4),
                            Range(init_state, state_bytes), Range(dy, xb),
                            Range(d_final, state_bytes)};
    const Range outputs[] = {Range(dx, xb), Range(ddt, size_t(b) * L * H * 4), rdA, Range(dB, bcb),
                             Range(dC, bcb), rdD, Range(d_init, state_bytes),
                             Range(workspace, plan.total)};
    const int n_out = sizeof(outputs) / sizeof(outputs[0]);
    for (int i = 0; i < n_out; ++i) {
        for (const Range &in : inputs)
            if (outputs[i].overlaps(in)) return SSD_ERR_ALIAS;
        for (int j = i + 1; j < n_out; ++j)
            if (outputs[i].overlaps(outputs[j])) return SSD_ERR_ALIAS;
    }

    ssd::ChunkScanBwdArgs a;
    a.x = x; a.dt = dt; a.A = A; a.B = B; a.C = C; a.D = D; a.init_state = init_state;
    a.dy = dy; a.d_final = d_final;
    a.dx = dx; a.ddt = ddt; a.dA = dA; a.dB = dB; a.dC = dC; a.dD = dD; a.d_init = d_init;
    a.b = b; a.L = L; a.H = H; a.P = P; a.N = N; a.G = G;
    a.bf16 = bf16;
    a.workspace = workspace;
    if (ssd::launch_chunk_scan_bwd(a, plan, stream) != hipSuccess) return SSD_ERR_HIP;
    return SSD_OK;
}

}  // extern "C"
