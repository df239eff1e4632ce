/*
 * ssd_mi355x.h -- C ABI of the MI355X (gfx950) SSD hot-path library.
 *
 * Two operations of a Mamba-2 SSD (state space duality) layer:
 *
 *   ssd_chunk_scan_fwd  the selective scan of a whole sequence, computed with the
 *                       chunked block decomposition of the semiseparable sequence
 *                       map (Mamba-2 article (msbhsh.com), «SSD 算法：分块矩阵分解»
 *                       and «SSD 算法：分块和形态传递»);
 *   ssd_verify_step     the recurrent update over K draft tokens that a target model
 *                       runs when it verifies speculative-decoding drafts, handing
 *                       back the state at the accepted position ("如何将 Llama 变成
 *                       Mamba？研究人员推出新工作并提高推理速度", «推测解码»).
 *
 * and, built on them: ssd_chunk_scan_bwd (the gradients of the chunked scan),
 * ssd_verify_ring (verify rounds on a device-resident ring of recent states, with
 * rollback), the per-device pieces of the sequence-parallel scan (ssd_seq_*) and, as a comparison kernel on the same data, ssd_selective_scan_fwd
 * (the selective scan with one channel per head and a diagonal A that SSD replaces).
 *
 * Both compute, per batch row b and head h (group g = h / (H/G)):
 *
 *   h_t = exp(dt_t * A_h) * h_{t-1} + dt_t * x_t (outer) B_t      state [P x N]
 *   y_t = C_t . h_t + D_h * x_t                                    (sum over N)
 *
 * ("另辟蹊径--Mamba介绍", «The Recurrent Representation»: the output reads the
 * updated state; «What is a State Space Model?»: D is a skip term; Bi-Mamba page,
 * «Preliminary: Mamba Series»: in SSD, A is one scalar per head.)  dt is taken as
 * given: no softplus, bias or clamp is applied inside the library, except that
 * ssd_verify_ring can apply softplus(dt + bias) when a bias vector is passed.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array pointer is a DEVICE pointer to row-major contiguous memory, owned
 *   by the caller.  The library never allocates or frees device memory and keeps
 *   no global state; calls are re-entrant and thread-safe, except that calls sharing
 *   one chunk-scan workspace must not overlap in time.
 * - x, B, C and y have the I/O element type `io` (fp32 or bf16 bit patterns);
 *   dt, A, D and every state are fp32; accept_len is int32.
 * - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the null stream) and
 *   the call returns without waiting.  Kernel faults surface on a later
 *   synchronisation, as for any HIP launch.
 * - Arguments are checked on the host before anything is enqueued; a failed
 *   check returns its status and enqueues nothing.  SSD_ERR_HIP reports a launch
 *   error returned by the HIP runtime.  No C++ exception crosses the ABI.
 * - NaN or Inf in the inputs propagate to the outputs; they are not checked.
 * - The recurrence is taken to be a decay: dt >= 0 and A <= 0, so that every factor
 *   exp(dt * A) is at most 1 (what the discretisation produces: A_h = -exp(.) and a
 *   softplus step).  Kernels clamp decay exponents at 0 where a masked product could
 *   otherwise overflow; inputs outside this domain give unspecified results and are
 *   not checked.
 */
#ifndef SSD_MI355X_H
#define SSD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL_ARG = 1,     /* a required pointer is NULL                          */
    SSD_ERR_BAD_DIM = 2,      /* a dimension is negative / zero where it must not be */
    SSD_ERR_GROUPS = 3,       /* H is not a multiple of G                            */
    SSD_ERR_UNSUPPORTED = 4,  /* shape / chunk size / dtype this build does not run  */
    SSD_ERR_ALIGN = 5,        /* a pointer is not 16-byte aligned                    */
    SSD_ERR_WORKSPACE = 6,    /* workspace missing or smaller than required          */
    SSD_ERR_ALIAS = 7,        /* outputs overlap inputs in a way that is not allowed */
    SSD_ERR_HIP = 8           /* the HIP runtime reported an error                   */
} ssd_status_t;

typedef enum {
    SSD_DTYPE_F32 = 0,        /* x, B, C, y are float                                */
    SSD_DTYPE_BF16 = 1        /* x, B, C, y are bfloat16 (uint16 bit patterns); the
                                 MFMA operands are bf16 with fp32 accumulation       */
} ssd_dtype_t;

/*
 * Workspace size in bytes that ssd_chunk_scan_fwd needs for these dimensions
 * (0 for an empty problem).  Returns (size_t)-1 when the dimensions are invalid.
 */
size_t ssd_chunk_scan_workspace_bytes(int b, int L, int H, int P, int N, int G, int Q,
                                      ssd_dtype_t io);

/*
 * ssd_chunk_scan_workspace_init -- prepare a workspace once, before its first use
 * by ssd_chunk_scan_fwd (enqueued on hip_stream; workspace_bytes as allocated, at
 * least what the calls need, 16-byte aligned).  This call is required: without it
 * the chunk-to-chunk hand-off of the bf16 single-pass kernel never reads as ready.
 *
 * Step 3 of the chunked scan (the state passed from chunk to chunk, Mamba-2 article,
 * «SSD 算法：分块和形态传递») runs as a hand-off between workgroups through the
 * workspace: a 256-byte header (a work queue per XCD with its call number, an error
 * word, a preparation marker) and one ready flag per (batch, head, chunk).  This call
 * zeroes the workspace and writes the marker.  Each ssd_chunk_scan_fwd call takes a
 * new call number, tags the flags it raises with it, and leaves the queues at zero
 * when it completes; flags of earlier calls therefore never read as ready, and one prepared
 * workspace serves any number of later calls of any shape and I/O type that fits
 * (the fp32 / other-P path keeps its buffers after the header).  Calls that share a
 * workspace must run one at a time (same stream, or ordered by events): calls that
 * overlap on one workspace race.  A call that finds the workspace not prepared does
 * not wait: the outputs of every chunk after the first then hold NaN.  A call that
 * timed out waiting for a neighbouring chunk (the device broke its forward-progress
 * guarantee) completes with NaN in the affected outputs and sets the workspace's
 * error word (read it with ssd_chunk_scan_workspace_error); the workspace stays
 * usable.  After a call that was aborted mid-way, prepare the workspace again.
 * Returns SSD_ERR_NULL_ARG for a NULL workspace with workspace_bytes > 0,
 * SSD_ERR_ALIGN, or SSD_ERR_HIP.
 */
ssd_status_t ssd_chunk_scan_workspace_init(void *workspace, size_t workspace_bytes,
                                           void *hip_stream);

/*
 * ssd_chunk_scan_workspace_error -- copy the time-out error word of a prepared
 * chunk-scan workspace to err_out, and optionally clear it.
 *
 * The word is 0 while no chunk of any ssd_chunk_scan_fwd call on this workspace (since
 * it was prepared or last cleared) gave up waiting for the state of the chunk before
 * it; 1 once one did (its state and outputs were written as NaN); 2 if more
 * workgroups of a call ran on one XCD than the launch placed there (the launch relies
 * on the hardware placing workgroup i on XCD i mod the XCD count; outputs of that
 * call may be incomplete).  A healthy device never sets it.
 *   workspace, workspace_bytes  the workspace (device, 16-byte aligned, at least the
 *                               256-byte header)
 *   err_out   device int32, written
 *   clear     nonzero: reset the word to 0 after copying it
 * Enqueued on hip_stream, ordered after the calls it should observe; allocates
 * nothing.  Returns SSD_ERR_NULL_ARG, SSD_ERR_ALIGN (workspace 16 B, err_out 4 B),
 * SSD_ERR_WORKSPACE (fewer than 256 bytes), SSD_ERR_ALIAS (err_out inside the header)
 * or SSD_ERR_HIP.
 */
ssd_status_t ssd_chunk_scan_workspace_error(void *workspace, size_t workspace_bytes,
                                            int32_t *err_out, int clear, void *hip_stream);

/*
 * ssd_chunk_scan_fwd -- SSD chunked scan over a whole sequence.
 *
 * Method (Mamba-2 article, «SSD 算法：分块和形态传递»): the sequence is cut into
 * chunks of Q tokens; (1) inside each chunk the outputs are the quadratic,
 * attention-like masked form (C B^T o L)(dt o x); (2) each chunk's own state
 * contribution sum_s exp(sum of a after s) dt_s x_s (outer) B_s; (3) a short scan
 * over chunks passes the state on, H_c = exp(sum of a over chunk c) H_{c-1} + S_c;
 * (4) the state entering a chunk reaches its outputs through C.  Steps 1, 2 and 4
 * run on the matrix cores, step 3 is the only sequential part.  The result equals
 * the token-by-token recurrence above for every Q (up to rounding).
 *
 * Arguments (all device pointers):
 *   x          [b, L, H, P]  io       input per token and head
 *   dt         [b, L, H]     fp32     step size per token and head (> 0 expected)
 *   A          [H]           fp32     scalar state decay rate per head (< 0 expected)
 *   B, C       [b, L, G, N]  io       input / output projections, shared by the H/G
 *                                     heads of each group (head h reads group h/(H/G))
 *   D          [H]           fp32     skip term per head
 *   init_state [b, H, P, N]  fp32     state before token 0; NULL means zeros
 *   y          [b, L, H, P]  io       output (written)
 *   final_state[b, H, P, N]  fp32     state after token L-1 (written); NULL = skip
 *   Q                                 chunk length: 64, 128 or 256 (the last chunk
 *                                     may be shorter: L need not be a multiple of Q)
 *   workspace, workspace_bytes        at least ssd_chunk_scan_workspace_bytes(...)
 *                                     bytes, 16-byte aligned, prepared once by
 *                                     ssd_chunk_scan_workspace_init and left to the
 *                                     library between calls
 * Supported on this build: P in {16, 32, 64, 128}, N a multiple of 16 in [16, 256],
 * and the chunk tiles must fit the 160 KiB LDS of one CU (else
 * SSD_ERR_UNSUPPORTED).  b == 0 or L == 0 is a valid empty problem (final_state
 * then equals init_state, or zeros).  Every pointer must be 16-byte aligned except
 * dt, A, D (4-byte).  y must not overlap any input.
 */
ssd_status_t ssd_chunk_scan_fwd(const void *x, const float *dt, const float *A, const void *B,
                                const void *C, const float *D, const float *init_state, void *y,
                                float *final_state, int b, int L, int H, int P, int N, int G,
                                int Q, ssd_dtype_t io, void *workspace, size_t workspace_bytes,
                                void *hip_stream);

/*
 * Bytes of the buffer ssd_chunk_scan_fwd_noalloc takes its workspace from (64 MiB, one
 * per GPU).
 */
#define SSD_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)

/*
 * ssd_chunk_scan_fwd_noalloc -- ssd_chunk_scan_fwd for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * Same arguments (less the workspace), computation, results (bit for bit) and errors
 * as ssd_chunk_scan_fwd.  The workspace is a buffer of SSD_NOALLOC_WORKSPACE_BYTES in
 * the library's own device memory, one per GPU, which that GPU holds until the process
 * ends.  The call allocates and frees nothing and calls no allocating routine.
 * - A problem whose workspace (ssd_chunk_scan_workspace_bytes) exceeds that size is
 *   refused with SSD_ERR_WORKSPACE before anything is enqueued.  For scale: the
 *   2.7B-shaped layer (b 4, L 2048, H 80, P 64, N 128, bf16) needs 21 MB, and
 *   b 8, L 4096, H 32, P 64, N 256, Q 128 (bf16) needs 34 MB.
 * - The first call on a device prepares that device's buffer: it looks up the buffer's
 *   address and enqueues a fill kernel on hip_stream ahead of the scan.  That first
 *   call must not be made while hip_stream is being captured into a graph
 *   (SSD_ERR_UNSUPPORTED, nothing enqueued); later calls may be captured.
 * - Every call on a GPU shares that GPU's buffer, which keeps the last call's contents
 *   (the hand-off protocol of ssd_chunk_scan_workspace_init leaves it ready for the
 *   next call).  Calls on one GPU must therefore not overlap in time: issue them on one
 *   stream, or order them with events.  Calls that overlap race.
 * - A hand-off time-out (see ssd_chunk_scan_workspace_init) shows only as NaN outputs:
 *   the buffer's error word is not exposed.
 */
ssd_status_t ssd_chunk_scan_fwd_noalloc(const void *x, const float *dt, const float *A,
                                        const void *B, const void *C, const float *D,
                                        const float *init_state, void *y, float *final_state,
                                        int b, int L, int H, int P, int N, int G, int Q,
                                        ssd_dtype_t io, void *hip_stream);

/*
 * ssd_verify_step -- K draft tokens applied to an existing state.
 *
 * Mamba keeps only its current state, so a verifier that may reject part of the
 * draft must keep the state at the accepted position for rollback ("如何将 Llama
 * 变成 Mamba？...", «推测解码»).  For every (b, h), starting from state_in, the
 * recurrence above runs over k = 1..K; y is written for all K positions.
 *
 * Arguments (all device pointers):
 *   state_in   [b, H, P, N]     fp32   state before the first draft token
 *   x          [b, K, H, P]     io
 *   dt         [b, K, H]        fp32
 *   A          [H]              fp32
 *   B, C       [b, K, G, N]     io
 *   D          [H]              fp32
 *   accept_len [b]              int32  accepted draft tokens a_b in [0, K]
 *   y          [b, K, H, P]     io     outputs for all K positions (written)
 *   state_out  [b, H, P, N]     fp32   state after a_b tokens (written); a_b = 0
 *                                      copies state_in bit for bit.  May equal
 *                                      state_in exactly (in-place update).
 *   states_all [b, K, H, P, N]  fp32   NULL, or the state after each of the K tokens
 *   err_flag   int32            NULL, or a device word set to 1 when some
 *                                      accept_len lies outside [0, K] (that value is
 *                                      clamped into range); never cleared here
 * Supported: K in [1, 16], N in {16, 32, 64, 128, 256}, any P >= 1.  state_in,
 * state_out and states_all must be 16-byte aligned; state_out must not partially
 * overlap state_in, and states_all must not overlap either.
 */
ssd_status_t ssd_verify_step(const float *state_in, const void *x, const float *dt,
                             const float *A, const void *B, const void *C, const float *D,
                             const int32_t *accept_len, void *y, float *state_out,
                             float *states_all, int32_t *err_flag, int b, int K, int H, int P,
                             int N, int G, ssd_dtype_t io, void *hip_stream);

/*
 * ssd_selective_scan_fwd -- selective scan with one channel per head and a diagonal
 * state matrix (the recurrence SSD replaces), for comparisons on the same data.
 *
 * B, C and the step dt depend on the token while A is fixed ("另辟蹊径--Mamba介绍",
 * «Selectively Retain Information»); the state is carried by a scan («The Scan
 * Operation»).  Against SSD the head dimension is 1 and A is a full diagonal of N
 * values per channel instead of one scalar per head (Bi-Mamba page, «Preliminary:
 * Mamba Series»).  Per (b, channel d), group g = d / (Dch/G), state index n:
 *
 *   h[n] <- exp(dt[b,t,d] * A[d][n]) * h[n] + dt[b,t,d] * x[b,t,d] * B[b,t,g,n]
 *   y[b,t,d] = sum_n C[b,t,g,n] * h[n] + D[d] * x[b,t,d]
 *
 * Arguments (all device pointers):
 *   x           [b, L, Dch]  io
 *   dt          [b, L, Dch]  fp32   step per token and channel, taken as given
 *   A           [Dch, N]     fp32   decay rate per channel and state (16-byte aligned)
 *   B, C        [b, L, G, N] io
 *   D           [Dch]        fp32
 *   init_state  [b, Dch, N]  fp32   NULL means zeros (16-byte aligned)
 *   y           [b, L, Dch]  io     written
 *   final_state [b, Dch, N]  fp32   NULL, or the state after the last token (written;
 *                                   with L = 0 it is init_state, or zeros)
 * Supported: N in {16, 32, 64, 128, 256}; the channels of one group (Dch / G) must be
 * a multiple of 32 (one workgroup's channels).  Outputs must not overlap
 * inputs or each other.  Errors as for the other entry points; nothing is enqueued
 * when a check fails.
 */
ssd_status_t ssd_selective_scan_fwd(const void *x, const float *dt, const float *A, const void *B,
                                    const void *C, const float *D, const float *init_state,
                                    void *y, float *final_state, int b, int L, int Dch, int N,
                                    int G, ssd_dtype_t io, void *hip_stream);

/*
 * Multi-round verify on a ring of states.
 *
 * A verifier that runs round after round keeps a ring buffer of the most recent
 * states and, when a draft is rejected, restores the state of the last accepted
 * position ("Llama 3与Mamba混合架构：加速推理的蒸馏技术解析", «状态管理机制»;
 * "如何将 Llama 变成 Mamba？...", «推测解码»).  Here the ring lives in device memory:
 *
 *   ring  [b, R, H, P, N] fp32   R states per batch row
 *   meta  [b][2]          int32  (head, depth): slot head holds the current state,
 *                                and the depth slots behind it (head - 1, ... mod R)
 *                                the states of the depth positions before it
 *
 * so a whole decode loop (rounds and rollbacks) runs without reading anything back to
 * the host between calls.
 *
 * ssd_verify_ring_init: slot 0 of every row <- init_state (NULL = zeros), head and
 * depth <- 0.  ring 16-byte aligned; R >= 2.
 *
 * ssd_verify_ring: one round of K draft tokens from the head state of every row, by
 * the recurrence at the top of this file (y for all K positions).  With a =
 * accept_len[b], the states after tokens 1 .. a are stored in slots head + 1 ..
 * head + a (mod R); then head <- (head + a) mod R and depth <- min(depth + a, R - 1).
 * R must exceed K (the head slot is never overwritten in a round).  dt_bias [H] fp32,
 * or NULL: when given, the step used is softplus(dt + dt_bias[h]) = ln(1 + e^(dt +
 * dt_bias[h])), the discretisation step computed inside the kernel ("另辟蹊径--Mamba
 * 介绍", «Hardware-aware Algorithm»); when NULL, dt is taken as given.  x, dt, B, C, D,
 * A, y as for ssd_verify_step.  accept_len outside [0, K] is clamped and reported
 * through err_flag (NULL allowed) as in ssd_verify_step.  Supported: K in [1, 16], N
 * in {16, 32, 64, 128, 256}.  The round is two launches on hip_stream.
 *
 * ssd_verify_ring_rollback: head <- head - steps[b] (mod R), depth <- depth -
 * steps[b]; steps [b] int32 in [0, depth] (values outside are clamped and reported
 * through err_flag).  The states ahead of the new head stay in the ring but are no
 * longer reachable.
 *
 * All pointers are device pointers; outputs (ring, meta, y, err_flag) must not overlap
 * the inputs or each other.  Errors as for the other entry points.
 */
ssd_status_t ssd_verify_ring_init(float *ring, int32_t *meta, const float *init_state, int b,
                                  int R, int H, int P, int N, void *hip_stream);
ssd_status_t ssd_verify_ring(float *ring, int32_t *meta, const void *x, const float *dt,
                             const float *dt_bias, const float *A, const void *B, const void *C,
                             const float *D, const int32_t *accept_len, void *y,
                             int32_t *err_flag, int b, int K, int R, int H, int P, int N, int G,
                             ssd_dtype_t io, void *hip_stream);
ssd_status_t ssd_verify_ring_rollback(int32_t *meta, const int32_t *steps, int32_t *err_flag,
                                      int b, int R, void *hip_stream);

/*
 * Sequence (context) parallelism: the per-device pieces.
 *
 * A long sequence is split into n slices, one per device (Mamba-2 article, «序列并行»).
 * The devices exchange (alpha, S) = (total decay of the slice, the state it leaves from
 * a zero start), and each device folds its predecessors' pairs into the state h_in
 * entering its slice.  The pairs compose associatively because the state passing is
 * linear (the scan over chunks of «SSD 算法：分块和形态传递», step 3, run over slices).
 * Two orders of work give the same outputs:
 *   states first: ssd_seq_slice_state gives the pair without computing any output;
 *     after the exchange, ssd_seq_combine gives h_in and ssd_chunk_scan_fwd with
 *     init_state = h_in gives the slice's y and final state in one pass;
 *   outputs first: ssd_chunk_scan_fwd from a zero state gives y and S,
 *     ssd_seq_total_decay gives alpha, and after the exchange and ssd_seq_combine,
 *     ssd_seq_apply_state adds h_in's contribution to y and the final state.
 * The exchange is a collective outside this library; on one device these calls and
 * the per-slice scans reproduce the scan of the whole sequence.
 *
 * ssd_seq_slice_state: state[b, h] = the final state of the recurrence at the top of
 *   this file run over the slice from a zero state (what ssd_chunk_scan_fwd returns as
 *   final_state with init_state NULL), alpha[b, h] = the total decay of the slice
 *   (the product of the decays of its chunks, exp(sum_t dt A) up to rounding).  It
 *   computes the chunk states of step 2 and folds them with the scan of step 3; no
 *   output y is formed.  x [b, L, H, P] and B [b, L, G, N] io, 16-byte aligned; dt
 *   [b, L, H], A [H]; state [b, H, P, N] (16-byte aligned) and alpha [b, H] fp32.  The
 *   caller passes a workspace of ssd_seq_slice_state_workspace_bytes (16-byte
 *   aligned; 0 bytes when L = 0; (size_t)-1 means dimensions this build does not
 *   run), which holds the chunk states between the two
 *   launches and may be reused once the call has completed.  Supported: P in {16, 32,
 *   64, 128}, N a multiple of 16 up to 256.  L = 0 gives a zero state and alpha = 1.
 *
 * ssd_seq_total_decay: alpha[b, h] = exp(sum_t dt[b, t, h] * A[h]) over the slice;
 *   dt [b, L, H], A [H], alpha [b, H], all fp32 (L = 0 gives 1).
 * ssd_seq_combine: h_in[0] = init_state (NULL = zeros), h_in[j + 1] = alpha[j] h_in[j]
 *   + S[j] for j < n; alpha [n, b, H], S and h_in [n, b, H, P, N], init_state
 *   [b, H, P, N], fp32, states 16-byte aligned.
 * ssd_seq_apply_state: with cum_t the sum of dt * A over the slice through token t,
 *   y[b, t, h, :] += exp(cum_t) * sum_n C[b, t, g, n] h_in[b, h, :, n] in place, and
 *   final_state (NULL = skip; the slice's zero-state final state on entry) +=
 *   exp(cum_last) h_in.  y [b, L, H, P] and C [b, L, G, N] io; dt [b, L, H]; h_in
 *   [b, H, P, N] fp32 (y, C and h_in 16-byte aligned).  bf16 I/O rounds h_in to
 *   bf16 as the matrix-core operand; fp32 I/O keeps fp32.  Supported: P and N
 *   multiples of 16, at most 256.  L = 0 leaves y alone and adds h_in to final_state.
 * Outputs must not overlap inputs.  Errors as for the other entry points.
 */
size_t ssd_seq_slice_state_workspace_bytes(int b, int L, int H, int P, int N, int G,
                                           ssd_dtype_t io);
ssd_status_t ssd_seq_slice_state(const void *x, const float *dt, const float *A, const void *B,
                                 float *state, float *alpha, int b, int L, int H, int P, int N,
                                 int G, ssd_dtype_t io, void *workspace, size_t workspace_bytes,
                                 void *hip_stream);
ssd_status_t ssd_seq_total_decay(const float *dt, const float *A, float *alpha, int b, int L,
                                 int H, void *hip_stream);
ssd_status_t ssd_seq_combine(const float *alpha, const float *S, const float *init_state,
                             float *h_in, int n, int b, int H, int P, int N, void *hip_stream);
ssd_status_t ssd_seq_apply_state(void *y, float *final_state, const float *dt, const float *A,
                                 const void *C, const float *h_in, int b, int L, int H, int P,
                                 int N, int G, ssd_dtype_t io, void *hip_stream);

/*
 * Workspace size in bytes that ssd_chunk_scan_bwd needs for these dimensions (0 for
 * an empty problem).  Returns (size_t)-1 when the dimensions are invalid.
 */
size_t ssd_chunk_scan_bwd_workspace_bytes(int b, int L, int H, int P, int N, int G,
                                          ssd_dtype_t io);

/*
 * ssd_chunk_scan_bwd -- gradients of ssd_chunk_scan_fwd.
 *
 * For upstream gradients dy (of y) and d_final (of final_state), the gradients of
 * sum(dy * y) + sum(d_final * final_state) with respect to every input of the
 * recurrence at the top of this file.  The intermediate states are not kept by the
 * forward pass; they are recomputed here ("另辟蹊径--Mamba介绍", «Hardware-aware
 * Algorithm»: recomputation in the backward pass).  The computation runs the
 * chunked decomposition of the forward pass (Mamba-2 article, «SSD 算法：分块和形态
 * 传递») in reverse: the states entering every 64-token chunk, the adjoint state
 * recurrence from d_final back to d_init, then every in-chunk gradient on the
 * matrix cores.  Sums over heads (dB, dC), batch and chunks (dA, dD) run in a fixed
 * order, so the results are deterministic.  Every gradient is accumulated in fp32;
 * dx, dB and dC are rounded to the I/O type once at the end.
 *
 * Arguments (all device pointers; shapes as for ssd_chunk_scan_fwd):
 *   x, dt, A, B, C, D, init_state   the forward inputs (init_state NULL = zeros)
 *   dy         [b, L, H, P]  io     gradient of y
 *   d_final    [b, H, P, N]  fp32   gradient of final_state; NULL = zero
 *   dx         [b, L, H, P]  io     written
 *   ddt        [b, L, H]     fp32   written
 *   dA, dD     [H]           fp32   written (summed over batch and tokens)
 *   dB, dC     [b, L, G, N]  io     written (summed over the heads of each group)
 *   d_init     [b, H, P, N]  fp32   gradient of init_state (written); NULL = skip
 *   workspace, workspace_bytes      at least ssd_chunk_scan_bwd_workspace_bytes(...)
 *                                   bytes, 16-byte aligned; scratch, no preparation
 * Supported on this build: P in {32, 64}, N a multiple of 16 with the chunk tiles in
 * the 160 KiB LDS of one CU (N <= 128 at P = 64), else SSD_ERR_UNSUPPORTED.  b == 0
 * or L == 0 is a valid empty problem: dA and dD are zero and d_init equals d_final
 * (or zeros).  Pointers to io arrays, states and the workspace must be 16-byte
 * aligned, dt, A, D, ddt, dA, dD 4-byte.  Outputs must not overlap inputs, each
 * other or the workspace.
 */
ssd_status_t ssd_chunk_scan_bwd(const void *x, const float *dt, const float *A, const void *B,
                                const void *C, const float *D, const float *init_state,
                                const void *dy, const float *d_final, void *dx, float *ddt,
                                float *dA, void *dB, void *dC, float *dD, float *d_init, int b,
                                int L, int H, int P, int N, int G, ssd_dtype_t io,
                                void *workspace, size_t workspace_bytes, void *hip_stream);

/* Static, human-readable name of a status code. */
const char *ssd_status_string(ssd_status_t status);

/* Static version string of the library, e.g. "ssd_mi355x 0.1.0 gfx950". */
const char *ssd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_MI355X_H */
