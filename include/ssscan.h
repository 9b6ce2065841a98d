/*
 * ssscan.h — C ABI of the MI355X (gfx950) selective state-space (S6) scan library.
 *
 * What the library computes.  For every batch row b and channel d, with an
 * N-wide fp32 state h (N = dstate):
 *
 *     Delta_t = softplus(dt[b,d,t] + dt_bias[d])
 *     Abar_tn = exp(Delta_t * A[d,n])
 *     h_tn    = Abar_tn * h_(t-1)n + Delta_t * B[b,n,t] * x[b,d,t]
 *     y[b,d,t] = (sum_n C[b,n,t] * h_tn + Dskip[d] * x[b,d,t]) * silu(z[b,d,t])
 *
 * Sources: the reader's notes on the Mamba paper (kurisu.si), section "What they
 * did", item "Selective SSM (S6)" — Delta, B, C are computed from the input,
 * Delta through a softplus of a parameter plus a projection, A is a fixed
 * parameter entering as Abar = exp(Delta A), and the time-varying system is
 * evaluated as a recurrent scan whose expanded state never leaves on-chip
 * memory; same notes, "Architecture" — the state holds D x N numbers per
 * sequence; the tellworld.net summary, section "Architecture" — training runs the
 * recurrence over the whole sequence, generation needs one state update per
 * token.  The input term uses the first-order discretisation Bbar = Delta * B
 * (the pages give only Abar); the skip term Dskip and the silu gate (the gated
 * branch of the Mamba block, "Architecture" in the notes) multiply the whole sum.
 * silu(z) = z / (1 + exp(-z)).
 *
 * Layouts (row-major, last index fastest, all tensors contiguous):
 *     x, dt, z, y     (batch, dim, seqlen)    io dtype         decode: (batch, dim)
 *     B, C            (batch, dstate, seqlen) io dtype         decode: (batch, dstate)
 *     A               (dim, dstate)           fp32
 *     Dskip, dt_bias  (dim)                   fp32, NULL means all zeros
 *     h0, h_final     (batch, dim, dstate)    fp32, NULL h0 means a zero state
 *     state (decode)  (batch, dim, dstate)    fp32, updated in place
 * io dtype is SS_F32 (IEEE binary32) or SS_BF16 (bfloat16; y is rounded to
 * nearest-even).  The state and all internal arithmetic are fp32.
 *
 * Ownership and memory.  Every pointer is a device pointer owned by the caller
 * (e.g. a PyTorch tensor's data_ptr()); tensor base addresses must be 16-byte
 * aligned.  The library never allocates device memory: the scan's scratch space
 * is the caller's `workspace`, of at least ss_scan_fwd_workspace_bytes() bytes,
 * 256-byte aligned.  y must not overlap any input.  Inputs are read-only.
 *
 * Streams and synchronisation.  All work is enqueued on `stream` (a hipStream_t;
 * NULL = the default stream) and the calls return without waiting.  Calls that
 * share a workspace, y, state or h_final must be ordered on one stream.  The
 * library keeps no state between calls apart from the opt-in timing record
 * (ss_timing_*), and is safe to call from several host threads.
 *
 * Errors.  Every entry point returns an ss_status.  Arguments are validated on
 * the host before anything is launched; on a non-OK return nothing was enqueued
 * (except SS_ERR_HIP, reported when a launch itself fails, after which earlier
 * launches of the same call may have been enqueued).  ss_last_error() returns a
 * per-thread message describing the last non-OK status.  A fault inside a
 * kernel surfaces at the caller's next synchronisation, as for any HIP kernel.
 * No C++ exception crosses this interface and nothing aborts.
 */
#ifndef SSSCAN_H
#define SSSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SS_ABI_VERSION 1

typedef enum { SS_F32 = 0, SS_BF16 = 1 } ss_dtype;

typedef enum {
  SS_OK = 0,
  SS_ERR_INVALID_ARG = 1,   /* NULL required pointer, negative/zero size, misalignment, overlap */
  SS_ERR_UNSUPPORTED = 2,   /* dstate not in {1, 2, 4, 8, 16}, or an unknown dtype / plan */
  SS_ERR_WORKSPACE = 3,     /* workspace missing, misaligned or smaller than required */
  SS_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} ss_status;

/* Plan of one scan call: how the work is laid onto the GPU.
 *   state_groups:      waves per workgroup (1, 2 or 4); the state components are
 *                      split over the waves.
 *   lanes_per_channel: 1, 2 or 4 (0 means 1; 4 only with 4 state groups).  With
 *                      K > 1, K adjacent lanes share a channel and split that
 *                      wave's components again, so a workgroup covers 64/K
 *                      channels.  state_groups * lanes_per_channel must divide
 *                      into dstate.
 *   chunk_len:         tokens per sequence chunk; chunk_len >= seqlen means one
 *                      chunk.  Chunks are scanned in parallel and joined by an
 *                      exclusive scan of their (decay, end state) pairs, then
 *                      rescanned from their true initial states.  A multiple of
 *                      the tile length, state_groups * (8 for bf16, 4 for fp32). */
typedef struct {
  int32_t state_groups;
  int32_t lanes_per_channel;
  int64_t chunk_len;
} ss_scan_plan;

/* The plan ss_scan_fwd chooses for this shape on the current device. */
ss_status ss_scan_fwd_plan(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io,
                           ss_scan_plan* plan_out);

/* Bytes of workspace the scan needs for this shape under `plan` (NULL = the
 * automatic plan).  Returns 0 when the arguments are invalid. */
size_t ss_scan_fwd_workspace_bytes(int64_t batch, int64_t dim, int dstate, int64_t seqlen,
                                   ss_dtype io, const ss_scan_plan* plan);

/* Full-sequence selective scan.  Writes y (batch, dim, seqlen) and, when
 * h_final is non-NULL, the state after the last token (batch, dim, dstate).
 * z == NULL means no gate.  plan == NULL uses ss_scan_fwd_plan()'s choice. */
ss_status ss_scan_fwd(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io,
                      const void* x, const void* dt, const void* z,
                      const void* B, const void* C, const float* A,
                      const float* Dskip, const float* dt_bias, const float* h0,
                      void* y, float* h_final,
                      void* workspace, size_t workspace_bytes,
                      const ss_scan_plan* plan, void* stream);

/* One autoregressive decode step: for each (b, d), advance `state` by one token
 * with the same update as the scan and write y (batch, dim).  z == NULL means no
 * gate.  Needs no workspace.  batch * dim above 2^34 channels (a state of 1 TB
 * at dstate 16) returns SS_ERR_UNSUPPORTED. */
ss_status ss_state_update(int64_t batch, int64_t dim, int dstate, ss_dtype io, float* state,
                          const void* x, const void* dt, const void* z,
                          const void* B, const void* C, const float* A,
                          const float* Dskip, const float* dt_bias,
                          void* y, void* stream);

/* The same two operations with the zero-order-hold discretisation of the input
 * term: Bbar x = (exp(Delta A) - 1)/A * B * x (Delta * B * x where A = 0), the
 * discretisation under which selection is exactly gating (Theorem 1 in the
 * reader's notes on the Mamba paper, kurisu.si, "Main results (verified)").
 * Arguments, layouts, ownership, streams and errors are those of ss_scan_fwd and
 * ss_state_update. */
ss_status ss_scan_fwd_zoh(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io,
                          const void* x, const void* dt, const void* z,
                          const void* B, const void* C, const float* A,
                          const float* Dskip, const float* dt_bias, const float* h0,
                          void* y, float* h_final,
                          void* workspace, size_t workspace_bytes,
                          const ss_scan_plan* plan, void* stream);
ss_status ss_state_update_zoh(int64_t batch, int64_t dim, int dstate, ss_dtype io, float* state,
                              const void* x, const void* dt, const void* z,
                              const void* B, const void* C, const float* A,
                              const float* Dskip, const float* dt_bias,
                              void* y, void* stream);

/* The same two operations with options, as a bitwise OR of ss_flags:
 *  SS_FLAG_ZOH         the zero-order-hold input term (as the _zoh entry points);
 *  SS_FLAG_DT_PER_ROW  dt holds one value per (batch row, token), shared by the
 *                      row's channels: (batch, seqlen) for the scan, (batch) for
 *                      the decode step.  Delta = softplus(dt[b, t] + dt_bias[d]):
 *                      the selective SSM's Delta is the softplus of a parameter
 *                      plus a projection of the input broadcast over channels
 *                      (reader's notes, kurisu.si, "What they did", Selective SSM
 *                      item); dt is that projection, dt_bias the parameter.  It
 *                      is the general form with dt[b, d, t] equal across d, and
 *                      reads batch * seqlen values of dt instead of batch * dim
 *                      * seqlen.
 * Unknown bits return SS_ERR_UNSUPPORTED.  Everything else is as for ss_scan_fwd
 * and ss_state_update. */
typedef enum { SS_FLAG_ZOH = 1u, SS_FLAG_DT_PER_ROW = 2u } ss_flags;
/* ckpt (nullable, fp32, 16-byte aligned, ss_scan_ckpt_bytes long, no overlap
 * with anything else) receives the state entering every chunk of the backward
 * pass (16 tokens at dstate >= 8), laid out (batch, chunks, dim, dstate): a
 * training step's forward hands them to ss_scan_bwd_ex (with the same flags),
 * which then skips its own checkpoint sweep. */
ss_status ss_scan_fwd_ex(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io, uint32_t flags,
                         const void* x, const void* dt, const void* z,
                         const void* B, const void* C, const float* A,
                         const float* Dskip, const float* dt_bias, const float* h0,
                         void* y, float* h_final, float* ckpt,
                         void* workspace, size_t workspace_bytes,
                         const ss_scan_plan* plan, void* stream);
size_t ss_scan_ckpt_bytes(int64_t batch, int64_t dim, int dstate, int64_t seqlen);
ss_status ss_state_update_ex(int64_t batch, int64_t dim, int dstate, ss_dtype io, uint32_t flags, float* state,
                             const void* x, const void* dt, const void* z,
                             const void* B, const void* C, const float* A,
                             const float* Dskip, const float* dt_bias,
                             void* y, void* stream);

/* Context (sequence) parallelism.  A sequence cut into shards, one per GPU,
 * needs a single exchange: the recurrence is linear in the state, so a shard
 * run from a zero state ends in h_end, and from a state h it ends in
 * exp(A dsum) h + h_end, where dsum is the shard's sum of Delta (per component,
 * exp(A[d,n] dsum[b,d])).  The pages evaluate the recurrence with a parallel
 * algorithm in recurrent mode (Mamba abstract, on the "Mamba models" page, and
 * the tellworld.net summary, "Architecture"); this is its two-level form.
 *  1. Each shard: ss_scan_shard_state -> (dsum, h_end).
 *  2. Exchange the (dsum, h_end) pairs (an all-gather), then ss_scan_shard_combine
 *     -> the state entering each shard.
 *  3. Each shard: ss_scan_fwd with h0 = its entering state.
 *
 * ss_scan_shard_state: inputs as for ss_scan_fwd (z, C, Dskip are not needed);
 * outputs dsum (batch, dim) fp32 (4-byte aligned) and h_end (batch, dim, dstate)
 * fp32 (16-byte aligned).  The workspace is that of ss_scan_fwd with the
 * automatic plan (ss_scan_fwd_workspace_bytes(..., NULL)).  seqlen == 0 gives
 * zeros.  The _zoh form uses the zero-order-hold input term. */
ss_status ss_scan_shard_state(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io,
                              const void* x, const void* dt, const void* B, const float* A,
                              const float* dt_bias, float* dsum, float* h_end,
                              void* workspace, size_t workspace_bytes, void* stream);
ss_status ss_scan_shard_state_zoh(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io,
                                  const void* x, const void* dt, const void* B, const float* A,
                                  const float* dt_bias, float* dsum, float* h_end,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ss_scan_shard_combine: the exclusive scan over nshards shards in order.
 * dsum (nshards, batch, dim) and h_end (nshards, batch, dim, dstate) are the
 * shards' results stacked shard-major (as an all-gather leaves them); h0
 * (batch, dim, dstate) is the sequence's initial state (NULL = zero).  Writes
 * h_in (nshards, batch, dim, dstate), the state entering each shard, and
 * h_final (batch, dim, dstate), the state after the last shard; either may be
 * NULL.  All fp32, 4-byte aligned; outputs may not overlap inputs. */
ss_status ss_scan_shard_combine(int64_t batch, int64_t dim, int dstate, int64_t nshards,
                                const float* A, const float* dsum, const float* h_end,
                                const float* h0, float* h_in, float* h_final, void* stream);

/* Backward pass of ss_scan_fwd (first-order input term; ss_scan_bwd_ex with
 * SS_FLAG_ZOH is that of ss_scan_fwd_zoh): the gradients of a
 * loss with respect to every input of the scan, given dy = dLoss/dy and
 * dh_final = dLoss/dh_final.  Training differentiates the scan, and the state
 * is recomputed in the backward pass instead of being stored (reader's notes on
 * the Mamba paper, kurisu.si, "What they did", Selective SSM item): the call
 * takes the forward's inputs, not its outputs.
 *
 * Inputs: x, dt, z, B, C, A, Dskip, dt_bias, h0 exactly as given to ss_scan_fwd
 * (z, Dskip, dt_bias, h0 nullable); dy (batch, dim, seqlen) in the I/O dtype;
 * dh_final (batch, dim, dstate) fp32, NULL = zero.
 * Outputs, all written (never accumulated into):
 *   dx, ddt (batch, dim, seqlen) and dB, dC (batch, dstate, seqlen) in the I/O
 *     dtype, required when seqlen > 0;
 *   dz (batch, dim, seqlen) in the I/O dtype, given exactly when z is;
 *   dA (dim, dstate), dDskip (dim), ddt_bias (dim), dh0 (batch, dim, dstate)
 *     fp32, each nullable (not computed when NULL).  They are the gradients
 *     with respect to Dskip, dt_bias and h0 also when those inputs are NULL
 *     (read as zero).
 * Alignment, aliasing (no output may overlap an input, another output or the
 * workspace) and stream rules are those of ss_scan_fwd.  The workspace (size
 * from ss_scan_bwd_workspace_bytes, 256-byte aligned, caller-owned, contents
 * need not be preserved between calls) holds the state checkpoints and the
 * partial sums.  seqlen == 0 needs no workspace: dh0 = dh_final (or zero) and
 * dA, dDskip, ddt_bias are zeroed.  Results are deterministic: every sum runs
 * in a fixed order. */
size_t ss_scan_bwd_workspace_bytes(int64_t batch, int64_t dim, int dstate, int64_t seqlen,
                                   ss_dtype io);
ss_status ss_scan_bwd(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io,
                      const void* x, const void* dt, const void* z,
                      const void* B, const void* C, const float* A,
                      const float* Dskip, const float* dt_bias, const float* h0,
                      const void* dy, const float* dh_final,
                      void* dx, void* ddt, void* dz, void* dB, void* dC,
                      float* dA, float* dDskip, float* ddt_bias, float* dh0,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ss_scan_bwd with options, the backward of ss_scan_fwd_ex with the same flags:
 *  SS_FLAG_ZOH         the zero-order-hold input term c = (e^(Delta A) - 1)/A
 *                      (Delta when A = 0) in place of Delta, whose derivatives
 *                      are dc/dDelta = e^(Delta A) and dc/dA = Delta^2 psi(Delta A),
 *                      psi(u) = (u e^u - e^u + 1)/u^2 (c is formed as in the
 *                      forward: (e^(Delta A) - 1)/A where |Delta A| >= 1/20, a
 *                      Taylor polynomial of Delta phi(Delta A) below);
 *  SS_FLAG_DT_PER_ROW  dt is (batch, seqlen), and ddt, also (batch, seqlen) in the
 *                      I/O dtype, is the gradient of that shared dt, the sum over
 *                      channels of the per-channel gradient (in a fixed order).
 * Unknown bits return SS_ERR_UNSUPPORTED.  ckpt (nullable) holds the
 * checkpoints a ss_scan_fwd_ex call stored for the same inputs (same x, dt, B,
 * A, dt_bias, h0 and flags), and the backward then reads them instead of
 * recomputing them.  Everything else is as for ss_scan_bwd; with flags 0,
 * results are identical to ss_scan_bwd's. */
ss_status ss_scan_bwd_ex(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io, uint32_t flags,
                         const void* x, const void* dt, const void* z,
                         const void* B, const void* C, const float* A,
                         const float* Dskip, const float* dt_bias, const float* h0,
                         const void* dy, const float* dh_final, const float* ckpt,
                         void* dx, void* ddt, void* dz, void* dB, void* dC,
                         float* dA, float* dDskip, float* ddt_bias, float* dh0,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Splitting a long sequence in the backward pass.  The backward takes each
 * (batch row, channel block) through all of its tokens in one workgroup, so a
 * long sequence with few rows and channels would leave most of the GPU idle.
 * It is then cut into segments run by separate workgroups, the backward
 * counterpart of the forward's chunks (the pages evaluate the recurrence with a
 * parallel scan; reader's notes on the Mamba paper, kurisu.si, "What they did").
 * Each segment starts from the state entering it (every segment's end state
 * from a zero start, chained by the forward's combine; or the checkpoints in
 * ckpt) and from the adjoint carried in from the tokens after it.  That adjoint follows from the
 * same linearity run backwards: a segment passes on exp(A sum Delta) times what
 * enters it plus its own aggregate sum_t (prod of Abar up to t) dr_t C_t, with
 * dr = dy silu(z), which needs no state; a combine from dh_final chains them.
 * One reverse pass over each segment gives both aggregates.
 * The gradients equal the unsplit ones up to rounding (across a segment the
 * decay is applied as one exponential rather than a product of per-token
 * factors).
 *   ss_scan_bwd_segment_len: the segment length ss_scan_bwd and ss_scan_bwd_ex
 *     use for this shape on the current device: seqlen when they run the
 *     sequence whole (sequences shorter than 8192 tokens, or with at least two
 *     workgroups per CU, a workgroup taking 32 channels of a batch row at
 *     dstate >= 8 and 64 below; 0 when seqlen is 0), and 0 for invalid
 *     arguments.
 *   ss_scan_bwd_seg: ss_scan_bwd_ex with an explicit segment_len: 0 for the
 *     automatic choice, else a positive multiple of 64 (SS_ERR_INVALID_ARG
 *     otherwise, or beyond 2^20 segments); a length of at least seqlen runs the
 *     sequence whole.  Its workspace size is ss_scan_bwd_seg_workspace_bytes
 *     with the same segment_len (0 for invalid arguments). */
int64_t ss_scan_bwd_segment_len(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io);
size_t ss_scan_bwd_seg_workspace_bytes(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io,
                                       int64_t segment_len);
ss_status ss_scan_bwd_seg(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io, uint32_t flags,
                          int64_t segment_len,
                          const void* x, const void* dt, const void* z,
                          const void* B, const void* C, const float* A,
                          const float* Dskip, const float* dt_bias, const float* h0,
                          const void* dy, const float* dh_final, const float* ckpt,
                          void* dx, void* ddt, void* dz, void* dB, void* dC,
                          float* dA, float* dDskip, float* ddt_bias, float* dh0,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Size of the static device scratch array behind ss_scan_fwd_noalloc (32 MiB per GPU). */
#define SS_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* ss_scan_fwd_noalloc — for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * operation, arguments, layouts and errors are those of ss_scan_fwd_ex without
 * the workspace; nothing is allocated.  The scratch space (on chunked plans, the
 * chunk aggregates and entering states; one-chunk plans need none) is a static
 * device array of SS_NOALLOC_SCRATCH_BYTES that every GPU the library runs on
 * holds until the process ends; its device address is looked up on the first
 * call on each device.  A call whose ss_scan_fwd_workspace_bytes() exceeds that
 * size (e.g. the million-token plan's 69 MB of chunk aggregates) returns
 * SS_ERR_WORKSPACE before any device work.  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (other streams, other host
 * threads) race, and the caller must order them.  The array keeps the last
 * call's contents; a call reads no scratch byte it has not written itself. */
size_t ss_scan_fwd_noalloc_max_bytes(void);
ss_status ss_scan_fwd_noalloc(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io, uint32_t flags,
                              const void* x, const void* dt, const void* z,
                              const void* B, const void* C, const float* A,
                              const float* Dskip, const float* dt_bias, const float* h0,
                              void* y, float* h_final, float* ckpt,
                              const ss_scan_plan* plan, void* stream);

/* Opt-in timing of the main scan kernels (for benchmarks).  While enabled, each
 * ss_scan_fwd call records HIP events around its scan kernel launches on its
 * stream, and each ss_scan_bwd call around its backward kernels.  ss_timing_read synchronises on the recorded events and returns the
 * summed kernel time in milliseconds and the number of calls recorded since the
 * last ss_timing_reset. */
ss_status ss_timing_enable(int enable);
ss_status ss_timing_reset(void);
ss_status ss_timing_read(double* total_ms, int64_t* calls);

const char* ss_status_string(ss_status status);
const char* ss_last_error(void);
int ss_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSSCAN_H */
