// ssd_kernels.h -- host-side launch interface between the C ABI (ssd_api.hip) and
// the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssd {

constexpr size_t kMaxLds = 160 * 1024;   // LDS per CU on gfx950

struct VerifyArgs {
    const float *state_in;
    const void *x;
    const float *dt;
    const float *A;
    const void *B;
    const void *C;
    const float *D;
    const int32_t *accept_len;
    void *y;
    float *state_out;
    float *states_all;
    int32_t *err_flag;
    int b, K, H, P, N, G;
    bool bf16;
    // multi-round mode: ring [b, R, H, P, N] fp32 and meta [b][2] = (head, depth);
    // state_in / state_out / states_all unused when ring is set
    float *ring = nullptr;
    const int32_t *meta = nullptr;
    int R = 0;
    const float *dt_bias = nullptr;   // nullable: step = softplus(dt + dt_bias[h])
};

bool verify_supported_n(int N);
hipError_t launch_verify(const VerifyArgs &a, hipStream_t stream);
hipError_t launch_ring_init(float *ring, int32_t *meta, const float *init, int b, int R,
                            size_t slot, hipStream_t stream);
hipError_t launch_ring_advance(int32_t *meta, const int32_t *accept_len, int b, int K, int R,
                               hipStream_t stream);
hipError_t launch_ring_rollback(int32_t *meta, const int32_t *steps, int32_t *err_flag, int b,
                                int R, hipStream_t stream);

// selective scan, one channel per head, diagonal A (ssd_selective_scan.hip)
struct SelectiveArgs {
    const void *x;
    const float *dt;
    const float *A;
    const void *B;
    const void *C;
    const float *D;
    const float *init_state;
    void *y;
    float *final_state;
    int b, L, Dch, N, G;
    bool bf16;
};

// channels one workgroup covers for this N (0: N not supported); the channels of a
// group must be a multiple of it
int selective_channels_per_block(int N);
hipError_t launch_selective_scan(const SelectiveArgs &a, hipStream_t stream);

struct ChunkScanArgs {
    const void *x;
    const float *dt;
    const float *A;
    const void *B;
    const void *C;
    const float *D;
    const float *init_state;
    void *y;
    float *final_state;
    int b, L, H, P, N, G, Q;
    bool bf16;
    void *workspace;
};

// Sizes and workspace layout of one chunked-scan call.
struct ChunkScanPlan {
    int nc = 0;                 // number of chunks, ceil(L / Q)
    size_t off_states = 0;      // fp32 [b, H, nc, P, N]: chunk states, step 2 output
    size_t off_alpha = 0;       // fp32 [b, H, nc]: total decay of each chunk
    size_t off_hprev = 0;       // io   [b, H, nc, P, N]: state entering each chunk
    size_t total = 0;           // workspace bytes
    size_t lds_state = 0;       // dynamic LDS of the chunk-state kernel
    size_t lds_out = 0;         // dynamic LDS of the chunk-output kernel
    bool supported = false;     // this build runs the shape
};

ChunkScanPlan plan_chunk_scan(int b, int L, int H, int P, int N, int G, int Q, bool bf16);

// Workspace of the single-pass kernel: a 256-byte header, one ready flag per (batch,
// head, chunk) and a two-slot fp32 state ring per (batch, head) for the chunk-to-chunk
// hand-off.  Header words: 2 = error word (1: a hand-off timed out; 2: more workgroups
// ran on an XCD than the launch placed there), 32 = magic word, and at word 48 + 2 x
// the 64-bit queue of XCD x (x < 8): tickets taken (low half) and call number (high
// half).  ssd_chunk_scan_workspace_init zeroes it and writes the magic word; every
// completed call leaves each queue's count at zero and advances its call number (all
// queues together), and its ready flags hold that call's tag (call number + 1), which
// no later call waits for.  The three-kernel path keeps its buffers after the header,
// so a prepared workspace stays prepared whichever path a call takes.
constexpr uint32_t kWsMagic = 0x55d5ca11u;
constexpr size_t kWsHeaderBytes = 256;   // reserved by both chunk-scan layouts
constexpr int kWsErrorWord = 2;
constexpr int kWsMagicWord = 32;
constexpr int kWsQueueWord = 48;  // XCD x's queue: 64-bit word at word 48 + 2 x, x < 8
struct FusedPlan {
    int nc = 0;
    int HB = 1;                 // heads per workgroup (the launch picks it per device)
    size_t off_hdr = 0;         // uint32 [64]: error word, magic, per-XCD queues
    size_t off_flags = 0;       // uint32 [b, H, nc]
    size_t off_hbuf = 0;        // fp32   [b, H, 2, P, N]
    size_t total = 0;
    size_t lds = 0;
    bool supported = false;
};

FusedPlan plan_fused(int b, int L, int H, int P, int N, int G, int Q, bool bf16);
hipError_t launch_fused(const ChunkScanArgs &a, const FusedPlan &plan, hipStream_t stream);
hipError_t launch_chunk_scan(const ChunkScanArgs &a, const ChunkScanPlan &plan,
                             hipStream_t stream);
// gradients of the chunked scan (ssd_chunk_bwd.hip)
struct ChunkScanBwdArgs {
    const void *x;
    const float *dt;
    const float *A;
    const void *B;
    const void *C;
    const float *D;
    const float *init_state;    // may be null (zero initial state)
    const void *dy;
    const float *d_final;       // may be null (no final-state gradient)
    void *dx;
    float *ddt;
    float *dA;
    void *dB;
    void *dC;
    float *dD;
    float *d_init;              // may be null (not wanted)
    int b, L, H, P, N, G;
    bool bf16;
    void *workspace;
};

// Two implementations: the bf16 matrix-core path (bf16 I/O, P = 64, N in {64, 128};
// states in bf16, dB / dC partials per block of heads) and the fp32 path (everything
// else; fp32 states, partials per head).
struct ChunkScanBwdPlan {
    int nc = 0;                 // 64-token chunks
    bool bf16_path = false;
    int hb = 1;                 // heads per workgroup (bf16 path)
    int nparts = 0;             // dB / dC partials per token: H (fp32 path) or H / hb
    size_t off_hin = 0;         // fp32 [b,H,nc,P,N] chunk states then Hin | bf16 Hin^T
    size_t off_gh = 0;          // fp32 [b,H,nc,P,N] adjoint sources then Gh | bf16 Gh^T
    size_t off_alpha = 0;       // fp32 path: fp32 [b,H,nc]
    size_t off_dbp = 0;         // fp32 [b, L, nparts, N]
    size_t off_dcp = 0;         // fp32 [b, L, nparts, N]
    size_t off_dap = 0;         // fp32 [b, H, nc]
    size_t off_ddp = 0;         // fp32 [b, H, nc]
    size_t total = 0;
    size_t lds_states = 0;
    size_t lds_chunk = 0;
    bool supported = false;
};

ChunkScanBwdPlan plan_chunk_scan_bwd(int b, int L, int H, int P, int N, int G, bool bf16);
hipError_t launch_chunk_scan_bwd(const ChunkScanBwdArgs &a, const ChunkScanBwdPlan &plan,
                                 hipStream_t stream);
// bf16 path (ssd_chunk_bwd_bf16.hip): LDS bytes of its chunk kernel (0: N unsupported)
size_t chunk_bwd_bf16_lds(int N);
hipError_t launch_chunk_scan_bwd_bf16(const ChunkScanBwdArgs &a, const ChunkScanBwdPlan &plan,
                                      hipStream_t stream);
// dB, dC = sums of the fp32 partials over the parts of each group
hipError_t launch_bwd_reduce(const ChunkScanBwdArgs &a, const ChunkScanBwdPlan &plan,
                             hipStream_t stream);

// sequence-parallel pieces (ssd_seqpar.hip)
hipError_t launch_seq_decay(const float *dt, const float *A, float *alpha, int b, int L, int H,
                            hipStream_t stream);
hipError_t launch_seq_combine(const float *alpha, const float *S, const float *init, float *h_in,
                              int n, int b, int H, int PN, hipStream_t stream);
hipError_t launch_seq_apply(void *y, float *final_state, const float *dt, const float *A,
                            const void *C, const float *h_in, int b, int L, int H, int P, int N,
                            int G, bool bf16, hipStream_t stream);

// Step 2 alone over chunks of Q tokens (ssd_chunk_scan.hip): S fp32 [b, H, nc, P, N]
// and the chunk decays alpha fp32 [b, H, nc]; LDS the kernel needs for a shape.
size_t chunk_states_lds(int P, int N, int Q, bool bf16);
hipError_t launch_chunk_states(const void *x, const float *dt, const float *A, const void *B,
                               float *S, float *alpha, int b, int L, int H, int P, int N, int G,
                               int Q, bool bf16, hipStream_t stream);
// Step 3 over n pieces from a zero state, final state only: state = the fold of
// S [b, H, n, P * N] by alpha [b, H, n]; alpha_total [b, H] = the product of alpha.
hipError_t launch_state_fold(const float *S, const float *alpha, float *state, float *alpha_total,
                             int b, int H, int PN, int n, hipStream_t stream);

// The state a slice of the sequence leaves from a zero start, and its total decay
// (the pair one device contributes to the sequence-parallel scan; ssd_slice_state.hip).
// The slice is cut into `parts` runs of tokens; each run's state (from zero) and decay
// go to the workspace, fp32 [b, H, parts, P, N] then fp32 [b, H, parts], and the scan
// of step 3 folds them.  bf16 I/O with P = 64 and N in {64, 128, 256} has a kernel of
// its own (runs of 128-token segments, the state kept in registers along a run); other
// shapes take the chunk-state kernel of the three-kernel path, one run per chunk.
struct SliceStatePlan {
    bool fast = false;          // the dedicated kernel
    int Q = 0;                  // generic path: chunk length (the longest that fits in LDS)
    int segs_per_part = 0;      // dedicated kernel: 128-token segments per run
    int parts = 0;              // runs folded by step 3
    size_t off_alpha = 0;
    size_t total = 0;           // workspace bytes (0 for an empty problem)
    bool supported = false;
};
SliceStatePlan plan_slice_state(int b, int L, int H, int P, int N, int G, bool bf16);
hipError_t launch_slice_state(const void *x, const float *dt, const float *A, const void *B,
                              float *state, float *alpha_total, void *workspace, int b, int L,
                              int H, int P, int N, int G, bool bf16, const SliceStatePlan &plan,
                              hipStream_t stream);

// final_state = init_state (or zeros) for an empty sequence.
hipError_t launch_copy_state(const float *init_state, float *final_state, size_t count,
                             hipStream_t stream);
// Zero the workspace and write the magic word.
hipError_t launch_workspace_init(void *workspace, size_t bytes, hipStream_t stream);
// err_out[0] = the header's time-out error word; cleared afterwards when asked.
hipError_t launch_workspace_error(void *workspace, int32_t *err_out, bool clear,
                                  hipStream_t stream);

}  // namespace ssd
