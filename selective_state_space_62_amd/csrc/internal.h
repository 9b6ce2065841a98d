// Internal interface between the C-ABI layer (api.cpp) and the HIP kernels.
// Not installed; the public interface is include/ssscan.h.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "ssscan.h"

namespace ssscan {

// Records the per-thread message that ss_last_error() returns and passes the
// status through (printf-style message).
ss_status record_error(ss_status st, const char* fmt, ...);
ss_status record_hip_error(hipError_t e, const char* what);

enum IoType : int32_t { kIoF32 = 0, kIoBf16 = 1 };

// Shape and plan of one scan launch.
struct ScanDims {
  int64_t batch;
  int64_t dim;
  int64_t seqlen;
  int64_t chunk_len;    // tokens per chunk (a multiple of the tile length)
  int32_t num_chunks;   // ceil(seqlen / chunk_len)
  int32_t dstate;       // N
  int32_t groups;       // waves per workgroup
  int32_t io;           // IoType
  int32_t vec;          // 1: every lane's span of a row is aligned for one vector access
  int32_t lanes;        // lanes per channel (1, 2 or 4); each lane owns dstate/(groups*lanes) states
  int32_t dt_row;       // 1: dt is (batch, seqlen), one value per token shared by a row's channels
  int64_t ck_count;     // with ScanPtrs::ckpt: checkpoints per channel, ceil(seqlen / bwd_chunk_tokens(dstate))
  int32_t buf;          // 1: whole aligned tiles go through buffer resources (every offset fits 31 bits)
};

struct ScanPtrs {
  const void* x;
  const void* dt;
  const void* z;        // nullable
  const void* B;        // (batch, dstate, seqlen), io dtype
  const void* C;        // (batch, dstate, seqlen), io dtype (not read by the aggregate pass)
  const float* A;
  const float* Dskip;   // nullable
  const float* dt_bias; // nullable
  const float* h0;      // nullable
  const float* h_in;    // chunked: (batch, dim, num_chunks, dstate) initial state of each chunk
  void* y;
  float* h_final;       // nullable
  float* agg_h;         // chunk end states from zero (batch, dim, num_chunks, dstate)
  float* agg_s;         // chunk sums of Delta (batch, dim, num_chunks)
  float* ckpt;          // nullable: (batch, ck_count, dim, dstate) state entering every backward chunk
};

// Shape of one backward launch.
struct BwdDims {
  int64_t batch;
  int64_t dim;
  int64_t seqlen;
  int64_t cblocks;      // channel blocks per batch row (64 / lanes-per-channel channels each)
  int32_t dstate;
  int32_t io;
  int32_t vec;          // 1: every lane's 2-token span of a row is aligned for one vector access
  int32_t have_ckpt;    // 1: BwdPtrs::ckpt already holds the checkpoints (stored by the forward)
  int32_t dt_row;       // 1: dt (and ddt) hold one value per (batch row, token), shared by the channels
  int32_t zoh;          // 1: zero-order-hold input term
  int32_t nseg;         // sequence segments run by separate workgroups (1: the whole sequence)
  int64_t seg_len;      // tokens per segment (a multiple of the chunk length; >= seqlen when nseg == 1)
};

// dB/dC partials per (batch row, channel block): 2 N outputs plus one for the
// per-row dt gradient, for every token of whole backward chunks
constexpr int bwd_part_outputs(int dstate) { return 2 * dstate + 1; }

struct BwdPtrs {
  const void* x;
  const void* dt;
  const void* z;          // nullable
  const float* bc;        // workspace: (batch, seqlen, dstate, 2) fp32, B and C interleaved
  const float* A;
  const float* Dskip;     // nullable
  const float* dt_bias;   // nullable
  const float* h0;        // nullable
  const void* dy;
  const float* dh_final;  // nullable
  void* dx;
  void* ddt;
  void* dz;               // non-null exactly when z is
  void* dB;
  void* dC;
  float* dA;              // nullable
  float* dDskip;          // nullable
  float* ddt_bias;        // nullable
  float* dh0;             // nullable
  float* ckpt;            // workspace: (batch, chunks, dim, dstate) state at every chunk start
  float* part;            // workspace: (batch, cblocks, chunk, bwd_part_outputs, chunk token) partial sums
  float* dA_p;            // workspace: (nseg, batch, dim, dstate) per-(segment, row) sums
  float* dD_p;            // workspace: (nseg, batch, dim)
  float* dbias_p;         // workspace: (nseg, batch, dim)
  // split sequences (nseg > 1), each (batch, dim, nseg, dstate) or (batch, dim, nseg):
  const float* h_seg;     // the state entering each segment (unless ckpt holds the checkpoints)
  const float* lam_seg;   // the adjoint carried into each segment from the tokens after it
  float* adj_m;           // workspace: each segment's adjoint aggregate from a zero start
  float* adj_s;           // workspace: each segment's sum of Delta
  float* agg_h;           // workspace: each segment's end state from a zero start (no ckpt)
};

// Backward plan: lanes per channel and chunk length (tokens) for a state size.
// The chunk length is also the interval of the forward's stored checkpoints.
constexpr int bwd_chunk_tokens(int dstate) {
  return 2 * (dstate >= 4 ? 4 : dstate) * (dstate >= 8 ? 2 : 1);
}
int bwd_lanes_per_channel(int dstate);
int bwd_chunk_len(int dstate);

// Tokens of every input row a wave loads and owns per tile: 16 bytes, except
// 32 bytes (8 fp32 tokens) for the four-lanes-per-channel plan, whose lanes
// would otherwise own a single token each.
constexpr int wave_tokens(int lanes, int io) { return io == kIoBf16 ? 8 : (lanes == 4 ? 8 : 4); }
// Tokens per tile.
inline int tile_len(int groups, int lanes, int io) { return groups * wave_tokens(lanes, io); }
// Tokens of a row each lane loads per tile (its span).
inline int span_len(int lanes, int io) { return wave_tokens(lanes, io) / lanes; }

hipError_t launch_prep_bc(const ScanDims& dm, const void* B, const void* C, float* bc, hipStream_t s);
hipError_t launch_scan(const ScanDims& dm, const ScanPtrs& p, bool aggregate, bool zoh, hipStream_t s);
hipError_t launch_scan_bf16_euler(const ScanDims& dm, const ScanPtrs& p, bool aggregate, hipStream_t s);
hipError_t launch_scan_bf16_zoh(const ScanDims& dm, const ScanPtrs& p, bool aggregate, hipStream_t s);
hipError_t launch_scan_f32_euler(const ScanDims& dm, const ScanPtrs& p, bool aggregate, hipStream_t s);
hipError_t launch_scan_f32_zoh(const ScanDims& dm, const ScanPtrs& p, bool aggregate, hipStream_t s);
hipError_t launch_combine(const ScanDims& dm, const float* A, const float* agg_h, const float* agg_s,
                          const float* h0, float* h_in, hipStream_t s);
hipError_t launch_copy_state(int64_t count, const float* src, float* dst, hipStream_t s);
hipError_t launch_shard_reduce(const ScanDims& dm, const float* A, const float* agg_h, const float* agg_s,
                               float* h_end, float* dsum, hipStream_t s);
hipError_t launch_shard_combine(int64_t batch, int64_t dim, int dstate, int64_t nshards, const float* A,
                                const float* dsum, const float* h_end, const float* h0, float* h_in, float* h_final,
                                hipStream_t s);
hipError_t launch_scan_bwd(const BwdDims& dm, const BwdPtrs& p, hipStream_t s);
// split sequences: the segments' aggregates in one pass (adj_m for segments
// 1 .. nseg-1, adj_s, and with states also agg_h for every segment), then the
// adjoint carried into every segment (lam_seg) from dh_final
hipError_t launch_bwd_segment_agg(const BwdDims& dm, const BwdPtrs& p, bool states, hipStream_t s);
hipError_t launch_bwd_adjoint_combine(const BwdDims& dm, const float* A, const float* dh_final, const float* adj_m,
                                      const float* adj_s, float* lam_seg, hipStream_t s);
// the main backward kernel alone, zero-order-hold form (scan_bwd_zoh.hip)
hipError_t launch_scan_bwd_zoh_main(const BwdDims& dm, const BwdPtrs& p, hipStream_t s);
hipError_t launch_fill_zero(float* dst, int64_t n, hipStream_t s);
hipError_t launch_state_update(int64_t batch, int64_t dim, int dstate, int io, bool zoh, bool dt_row, float* state,
                               const void* x, const void* dt, const void* z, const void* B, const void* C,
                               const float* A, const float* Dskip, const float* dt_bias, void* y,
                               hipStream_t s);

}  // namespace ssscan
