// The scan kernel template and its launch dispatch, shared by the translation
// units that instantiate it (one per I/O dtype and discretisation, compiled in
// parallel).  See scan_fwd.hip for the design.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace ssscan {
namespace scan_detail {

using namespace dev;

// Workgroup index -> logical block, so that consecutive logical blocks (the
// channel blocks of one batch row, which share that row's B and C) land on the
// same XCD; workgroups are dealt to the 8 XCDs round-robin.
__device__ __forceinline__ int64_t xcd_logical_block(int64_t wg, int64_t nwg) {
  if ((nwg & 7) != 0) return wg;
  return (wg & 7) * (nwg >> 3) + (wg >> 3);
}

// A wave-uniform 64-bit value moved to scalar registers, so that the values
// derived from it (loop bounds, offsets) are computed by the scalar unit.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// At most 96 VGPRs (5 waves per SIMD) for the plans with two or four lanes per
// channel and up to 2 state components per lane: with 4 waves per workgroup and
// 28 KB of LDS, five workgroups fit on a CU at once, which the two-lanes-per-
// channel plan needs to keep every CU's share resident.  One-lane plans (each
// lane owns 8 or 4 tokens of the per-token work) and plans with more components
// per lane get no occupancy target.
// CKPT_K (full pass only): also store the state entering every backward-pass
// chunk, for a training step's backward.  It is a separate instantiation so
// that the plain scan keeps its registers.
// ROWS: rows of at least 1 MB (see ROWOWN below).
template <int N, int G, int K, typename IO, bool AGG, bool ZOH, bool CKPT_K, bool ROWS = false>
__global__ __launch_bounds__(64 * G) __attribute__((amdgpu_waves_per_eu(K >= 2 && N / (G * K) <= 2 ? 5 : 1, 10))) void scan_kernel(
    const ScanDims dm, const typename IO::T* __restrict__ x, const typename IO::T* __restrict__ dt,
    const typename IO::T* __restrict__ z, const typename IO::T* __restrict__ Bm,
    const typename IO::T* __restrict__ Cm, const float* __restrict__ A,
    const float* __restrict__ Dskip, const float* __restrict__ dt_bias, const float* __restrict__ h0,
    const float* __restrict__ h_in, typename IO::T* __restrict__ y, float* __restrict__ h_final,
    float* __restrict__ agg_h, float* __restrict__ agg_s, float* __restrict__ ckpt) {
  constexpr int CPB = 64 / K;            // channels per workgroup (K adjacent lanes per channel)
  constexpr int SG = G * K;              // state groups (one per lane of a channel per wave)
  constexpr int NS = N / SG;             // state components per lane
  // tokens owned per wave per tile (16 bytes of a row; 32 for fp32 with four lanes per channel)
  constexpr int TPW = wave_tokens(K, IO::kPerSpan == 8 ? kIoBf16 : kIoF32);
  constexpr int SPAN = TPW / K;          // of which each lane of a channel owns SPAN
  constexpr int T = TPW * G;             // tile length
  constexpr int THREADS = 64 * G;
  constexpr int SW = SpanT<IO, SPAN>::kWords;
  // The tile's B/C: 2N rows (B_n, then C_n) of T tokens each, read straight
  // from the (batch, N, L) inputs in runs of 4 tokens, one run per thread:
  // thread q takes row q % 2N and tokens 4 (q / 2N) .. + 3, so that the lanes
  // of a wave write different LDS banks.
  constexpr int BC_RUNS = 2 * N * T / 4;
  static_assert(BC_RUNS <= THREADS && T % 4 == 0, "one 4-token run of a B/C row per thread");
  constexpr int BW = SpanT<IO, 4>::kWords;
  static_assert(NS >= 1 && N % SG == 0, "G * K must divide N");
  static_assert(K == 1 || K == 2 || K == 4, "one, two or four lanes per channel");
  constexpr bool SHARE_DD = (G * K) > 1;   // Delta is computed once and shared through LDS

  // (Delta, Delta*x) per token and channel, and partial readouts per token, wave
  // and channel.  The rows are padded by one channel: the K lanes of a channel
  // own tokens SPAN apart, which without the pad fall in the same LDS bank.
  __shared__ float2 s_dd[SHARE_DD ? T : 1][CPB + 1];
  __shared__ float s_part[(SHARE_DD && !AGG) ? T : 1][G][CPB + 1];
  __shared__ __attribute__((aligned(16))) float s_bc[T * 2 * N];   // the tile's B_n, C_n (token, n, {B, C})
  // A whole tile's y goes through LDS: the owners write their spans in phase C,
  // and after the next tile's first barrier every thread stores 8 bytes, the
  // lanes of a row covering its whole segment of the tile in one instruction.
  // Stored straight from the owners, each wave put 16 bytes on each of the
  // block's rows per tile: four times the write requests.  Used when the block's
  // tile of y is exactly 8 bytes per thread and a row's segment of the tile is
  // at most half a cache line (64 bytes: the bf16 plans).  The fp32 four-lane
  // plan's waves already fill a 128-byte line per row and tile, and staging
  // only cost it time (0.148 -> 0.151 ms at the 130M shape).
  constexpr int EBY = (int)sizeof(typename IO::T);
  // Owners of the per-token work (phases A and C).  With ROWOWN (rows of at
  // least 1 MB; bf16, four waves of 32 channels, 32-token tiles) lane l of wave
  // w owns tokens SPAN (l % 8) .. + SPAN - 1 of row 8 w + l / 8: the 8 lanes of
  // a row take its 64-byte segment of the tile, so each wave's load or store
  // covers that segment of 8 rows in one instruction, and y needs no staging.
  // Owning a span of its own channel, each wave reads 16 bytes of all 32 rows:
  // when the rows share their offset within the memory pages (2^20-token rows
  // lie 2 MB apart) the vector L1 loses the line between the waves' requests,
  // and every piece goes to L2 (million-token forward 17.0 -> 14.1 ms).  At
  // shorter rows that costs nothing, while the owners' reads of the readout
  // partials meet two-way bank conflicts (2.8B-shaped layer 5% slower), so
  // there a lane owns SPAN tokens of its own channel.
  constexpr bool ROWOWN = ROWS;
  static_assert(!ROWS || (SHARE_DD && K == 2 && G == 4 && CPB == 8 * G && T * EBY == 64 && SPAN * 8 == T),
                "row segments: bf16, four waves of 32 channels, 32-token tiles");
  constexpr bool STAGE_Y = !ROWOWN && !AGG && SHARE_DD && CPB * T * EBY == 8 * THREADS && T * EBY <= 64;
  constexpr int YROW = (T * EBY + 8) / 4;   // words per staged row (padded against bank conflicts)
  __shared__ __attribute__((aligned(16))) uint32_t s_y[STAGE_Y ? CPB : 1][STAGE_Y ? YROW : 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int c = lane / K;                 // channel within the block
  const int hk = lane % K;                // lane of the channel
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sg = w * K + hk;              // state group of this lane
  const int oc = ROWOWN ? w * 8 + (lane >> 3) : c;                  // owner: channel within the block
  const int otok = ROWOWN ? (lane & 7) * SPAN : w * TPW + hk * SPAN;   // owner: first token in a tile

  // logical block -> (chunk, batch row, channel block), channel block fastest
  const int64_t cblocks = (dm.dim + CPB - 1) / CPB;
  const int64_t nwg = cblocks * dm.batch * dm.num_chunks;
  int64_t lb = xcd_logical_block(blockIdx.x, nwg);
  const int64_t cb = uniform64(lb % cblocks);
  lb /= cblocks;
  const int64_t b = uniform64(lb % dm.batch);
  const int64_t chunk = uniform64(lb / dm.batch);

  const int64_t d = cb * CPB + c;
  const bool act = d < dm.dim;
  const int64_t dc = act ? d : dm.dim - 1;   // clamped: inactive lanes compute on a valid row
  const int64_t L = dm.seqlen;
  const int64_t t0 = chunk * dm.chunk_len;
  const int64_t t1 = (t0 + dm.chunk_len < L) ? t0 + dm.chunk_len : L;
  const int64_t ch = b * dm.dim + dc;
  const int64_t row = ch * L;
  const int64_t dt_row = dm.dt_row ? b * L : row;   // dt per (row, token) is shared by the row's channels
  // the owner's channel (the same as the lane's own unless ROWOWN)
  const int64_t od = cb * CPB + oc;
  const bool oact = od < dm.dim;
  const int64_t odc = oact ? od : dm.dim - 1;
  const int64_t orow = (b * dm.dim + odc) * L;
  const int64_t odt_row = dm.dt_row ? b * L : orow;
  const bool vec = dm.vec != 0;
  const bool has_z = z != nullptr;

  float A2[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) A2[s] = A[dc * N + sg * NS + s] * kLog2e;
  // Zero-order hold: the input term c B x with c = (e^(Delta A) - 1)/A from
  // zoh_coef: (E - 1)/A from the E = e^(Delta A) already at hand where
  // |Delta A| >= 1/20, a Taylor polynomial of Delta phi(Delta A) below (A = 0
  // included), with no reciprocal per element.
  float inv_a[ZOH ? NS : 1];
  if constexpr (ZOH) {
#pragma unroll
    for (int s = 0; s < NS; ++s) inv_a[s] = 1.0f / A[dc * N + sg * NS + s];
  }
  // the owner's (phases A and C)
  const float bias2 = dt_bias ? dt_bias[odc] * kLog2e : 0.0f;
  const float skip = Dskip ? Dskip[odc] : 0.0f;

  float h[NS];
  {
    const float* hi = nullptr;
    if constexpr (!AGG) {
      if (h_in) hi = h_in + (ch * dm.num_chunks + chunk) * N + sg * NS;
      else if (h0) hi = h0 + ch * N + sg * NS;
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) h[s] = hi ? hi[s] : 0.0f;
  }
  float dsum = 0.0f;   // AGG: sum of Delta over the chunk
  // checkpoints for the backward pass: the state entering every ck_len-token chunk
  float* __restrict__ ck_row = nullptr;
  if constexpr (CKPT_K) {
    if (ckpt && act) ck_row = ckpt + (b * dm.ck_count * dm.dim + dc) * N + sg * NS;   // (batch, chunk, dim, N)
  }
  constexpr int CKL = bwd_chunk_tokens(N);   // checkpoint interval (a power of 2)
  if constexpr (CKPT_K) {
    if (ck_row && (t0 % CKL) == 0) {
#pragma unroll
      for (int s = 0; s < NS; ++s) ck_row[(t0 / CKL) * dm.dim * N + s] = h[s];
    }
  }

  // this thread's B/C run: row bc_r (B_n for bc_r < N, else C_(bc_r - N)), tokens
  // 4 bc_g .. 4 bc_g + 3 of the tile (the aggregate pass loads C too and never
  // reads it).  With a run for every thread (N = 16) the loads are
  // unconditional: a load under an exec mask leaves the compiler unsure how many
  // memory operations are in flight, and it then waits for all of them,
  // including the previous tile's y store, before using the next run.
  const bool bc_act = BC_RUNS >= THREADS || tid < BC_RUNS;
  const int bc_r = tid % (2 * N);
  const int bc_g = tid / (2 * N);
  const int bc_n = bc_r < N ? bc_r : bc_r - N;
  const typename IO::T* __restrict__ bc_src = (bc_r < N ? Bm : Cm) + (b * N + bc_n) * L;
  const bool vec4 = (L % 4) == 0;
  // A tile's raw inputs held in registers: this lane's spans of x, dt and z and
  // this thread's run of B/C.  The next tile's are loaded while the current one
  // computes; whole tiles alternate between two of these.
  struct Spans {
    uint32_t x[SW], dt[SW], z[SW], bc[BW];
  };
  auto load_bc_tile = [&](int64_t ts, Spans& S) {
    const int64_t first = ts + 4 * bc_g;
    const int64_t v = t1 - first;
    const int valid = bc_act ? (int)(v < 0 ? 0 : (v < 4 ? v : 4)) : 0;
    load_span<IO, 4>(bc_src, first, valid, vec4, S.bc);
  };
  // Buffer resources of whole aligned tiles (dm.buf): the workgroup's rows of x,
  // z and y, the dt rows (the workgroup's, or the batch row's shared one), and
  // the batch row's B/C re-layout; per-lane offsets are fixed, the tile's token
  // offset goes in a scalar register.  Without z the z loads read x (unused).
  const bool use_buf = dm.buf != 0;
  constexpr int EB = (int)sizeof(typename IO::T);
  const int64_t row0 = b * dm.dim + cb * CPB;                  // the workgroup's first row
  const int64_t nrows = (dm.dim - cb * CPB < CPB) ? dm.dim - cb * CPB : CPB;
  const __amdgpu_buffer_rsrc_t rs_x = make_rsrc(x + row0 * L, nrows * L * EB);
  const __amdgpu_buffer_rsrc_t rs_z = has_z ? make_rsrc(z + row0 * L, nrows * L * EB) : rs_x;
  const __amdgpu_buffer_rsrc_t rs_dt =
      dm.dt_row ? make_rsrc(dt + b * L, L * EB) : make_rsrc(dt + row0 * L, nrows * L * EB);
  const uint32_t vo_row = (uint32_t)(((odc - cb * CPB) * L + otok) * EB);
  const uint32_t vo_dt = dm.dt_row ? (uint32_t)(otok * EB) : vo_row;

  // first token of the span this lane owns in the tile starting at ts
  auto own_first = [&](int64_t ts) { return ts + otok; };
  auto own_valid = [&](int64_t first) {
    const int64_t v = t1 - first;
    return (int)(v < 0 ? 0 : (v < SPAN ? v : SPAN));
  };

  // the next whole tile (starting at ts) through the buffer resources
  auto load_buf_tile = [&](int64_t ts, Spans& S) {
    const uint32_t so = (uint32_t)(ts * EB);
    buf_load_span<IO, SPAN>(rs_x, vo_row, so, S.x);
    buf_load_span<IO, SPAN>(rs_dt, vo_dt, so, S.dt);
    if constexpr (!AGG) buf_load_span<IO, SPAN>(rs_z, vo_row, so, S.z);   // the aggregate pass has no gate
    // (B or C differs between lanes, so the run comes through a plain vector load)
    if (bc_act) load_span<IO, 4>(bc_src, ts + 4 * bc_g, 4, true, S.bc);
  };

  Spans S0, S1;
#pragma unroll
  for (int k = 0; k < SW; ++k) S0.z[k] = S1.z[k] = 0u;   // z is read only with a gate
#pragma unroll
  for (int k = 0; k < BW; ++k) S0.bc[k] = S1.bc[k] = 0u;
  {
    const int64_t tf = own_first(t0);
    const int valid = own_valid(tf);
    load_span<IO, SPAN>(x, orow + tf, valid, vec, S0.x);
    load_span<IO, SPAN>(dt, odt_row + tf, valid, vec, S0.dt);
    if (!AGG && has_z) load_span<IO, SPAN>(z, orow + tf, valid, vec, S0.z);
    load_bc_tile(t0, S0);
  }

  // One tile from the spans `cur`, loading the next tile's into `nxt`.  FULL (a
  // compile-time tag) means all T tokens lie inside the chunk: no per-token
  // masks, no guards in the inner loop.  NEXT_BUF (compile-time): the next tile
  // is whole and goes through the buffer resources.
  // The staged tile of y (token y_pend_ts onward; -1: none) to HBM: thread q
  // stores bytes 8 (q % PPR) .. + 7 of row q / PPR of the tile.  With nothing
  // staged, or for rows past dim, the offset lies beyond the buffer and the
  // hardware drops the store, so every tile issues the same stores.
  int64_t y_pend_ts = -1;
  auto flush_y = [&]() {
    if constexpr (STAGE_Y) {
      constexpr int PPR = T * EBY / 8;   // 8-byte pieces per row
      const int r = tid / PPR, q = tid % PPR;
      const uint2 v = *reinterpret_cast<const uint2*>(&s_y[r][2 * q]);
      const bool ok = y_pend_ts >= 0 && r < nrows;
      const uint32_t vo = ok ? (uint32_t)(r * L * EB + q * 8) : 0x80000000u;
      const uint32_t so = (uint32_t)((y_pend_ts < 0 ? 0 : y_pend_ts) * EB);
      typedef unsigned int u2 __attribute__((ext_vector_type(2)));
      const u2 d = {v.x, v.y};
      __builtin_amdgcn_raw_buffer_store_b64(d, make_rsrc(y + row0 * L, nrows * L * EB), vo, so, 0);
      y_pend_ts = -1;
    }
  };
  auto tile = [&](auto full_tag, auto ck_tag, auto nbuf_tag, int64_t ts, const Spans& cur, Spans& nxt) {
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr bool CKPT = decltype(ck_tag)::value && CKPT_K;
    constexpr bool NEXT_BUF = decltype(nbuf_tag)::value;
    const int64_t tf = own_first(ts);
    const int valid = FULL ? SPAN : own_valid(tf);
    const uint32_t(&cx)[SW] = cur.x;
    const uint32_t(&cdt)[SW] = cur.dt;
    const uint32_t(&cz)[SW] = cur.z;

    // phase A: Delta and Delta*x for the owned tokens; stage the B/C tile
    float xv[SPAN], zv[SPAN], dl[SPAN], dx[SPAN];
#pragma unroll
    for (int i = 0; i < SPAN; ++i) {
      xv[i] = span_elem<IO>(cx, i);
      zv[i] = span_elem<IO>(cz, i);
      const float delta = softplus_dt(span_elem<IO>(cdt, i), bias2);
      if constexpr (FULL) dl[i] = delta;
      else dl[i] = (i < valid) ? delta : 0.0f;            // padding tokens leave the state alone
      dx[i] = ZOH ? xv[i] : dl[i] * xv[i];   // zero-order hold shares x itself
    }
    if (bc_act) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s_bc[(4 * bc_g + i) * (2 * N) + 2 * bc_n + (bc_r < N ? 0 : 1)] = span_elem<IO>(cur.bc, i);
    }
    // prefetch the next tile: plain vector loads when it is whole and aligned
    // (every tile but the last), masked loads otherwise
    if constexpr (NEXT_BUF) {
      load_buf_tile(ts + T, nxt);
    } else if (use_buf && ts + 2 * T <= t1) {
      load_buf_tile(ts + T, nxt);
    } else if (vec && ts + 2 * T <= t1) {
      const int64_t tn = tf + T;
      load_span<IO, SPAN>(x, orow + tn, SPAN, true, nxt.x);
      load_span<IO, SPAN>(dt, odt_row + tn, SPAN, true, nxt.dt);
      if (!AGG && has_z) load_span<IO, SPAN>(z, orow + tn, SPAN, true, nxt.z);
      load_bc_tile(ts + T, nxt);
    } else if (ts + T < t1) {
      const int64_t tn = tf + T;
      const int validn = own_valid(tn);
      load_span<IO, SPAN>(x, orow + tn, validn, vec, nxt.x);
      load_span<IO, SPAN>(dt, odt_row + tn, validn, vec, nxt.dt);
      if (!AGG && has_z) load_span<IO, SPAN>(z, orow + tn, validn, vec, nxt.z);
      load_bc_tile(ts + T, nxt);
    }
    if constexpr (SHARE_DD) {
#pragma unroll
      for (int i = 0; i < SPAN; ++i) s_dd[otok + i][oc] = make_float2(dl[i], dx[i]);
    }
    __syncthreads();
    if constexpr (STAGE_Y) {
      if (use_buf) flush_y();
    }
    // Phase B runs at a raised wave priority and phases C and A at the
    // default, so a SIMD's issue favours the waves sweeping the state over
    // those of other workgroups in their short owner phases (5-6% faster at
    // the 2.8B shape than one priority throughout).
    __builtin_amdgcn_s_setprio(2);

    // phase B: this lane's state components through every token of the tile.
    // The LDS operands of token j + PD are read before token j is computed (PD
    // tokens ahead: with one component per lane a token's work is too short to
    // cover an LDS read's latency).
    float yp[SHARE_DD ? 1 : T];
    struct Ops {
      float d, dx, bcv[2 * NS];
    };
    auto fetch = [&](int j, Ops& o) {
      if constexpr (SHARE_DD) {
        const float2 v = s_dd[j][c];
        o.d = v.x;
        o.dx = v.y;
      } else {
        o.d = dl[j];
        o.dx = dx[j];
      }
      const float* src = s_bc + j * (2 * N) + 2 * sg * NS;
      if constexpr (NS == 1) {
        const float2 v = *reinterpret_cast<const float2*>(src);
        o.bcv[0] = v.x;
        o.bcv[1] = v.y;
      } else {
#pragma unroll
        for (int q = 0; q < 2 * NS; q += 4) {
          const float4 v = *reinterpret_cast<const float4*>(src + q);
          o.bcv[q] = v.x;
          o.bcv[q + 1] = v.y;
          o.bcv[q + 2] = v.z;
          o.bcv[q + 3] = v.w;
        }
      }
    };
    // o.dx is Delta x (first order) or x (zero-order hold)
    auto compute = [&](int j, const Ops& o) {
      float acc = 0.0f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const float u2 = o.d * A2[s];
        const float E = __builtin_amdgcn_exp2f(u2);
        float in;
        if constexpr (!ZOH) {
          in = o.dx * o.bcv[2 * s];                       // first order: Bbar x = Delta B x
        } else {
          in = zoh_coef(u2, E, o.d, inv_a[s]) * (o.dx * o.bcv[2 * s]);   // c x B (o.dx is x)
        }
        h[s] = fmaf(E, h[s], in);
        if constexpr (!AGG) acc = (s == 0) ? o.bcv[1] * h[0] : fmaf(o.bcv[2 * s + 1], h[s], acc);
      }
      if constexpr (AGG) {
        dsum += o.d;
      } else {
        // both lanes of a channel end with the channel's sum over this wave's components
        // the K lanes of a channel (adjacent in a quad) end with the channel's sum
        // (the empty asm stops the compiler from refolding the readout product into
        // the first DPP add, which costs a move and a second multiply)
        if constexpr (K >= 2) asm volatile("" : "+v"(acc));
        if constexpr (K >= 2) acc += __builtin_amdgcn_update_dpp(0.0f, acc, 0xB1, 0xf, 0xf, true);   // [1,0,3,2]
        if constexpr (K == 4) acc += __builtin_amdgcn_update_dpp(0.0f, acc, 0x4E, 0xf, 0xf, true);   // [2,3,0,1]
        // one lane of the channel stores the sum (the others hold the same value);
        // the empty asm keeps the DPP add (fused into one instruction) ahead of
        // the masked store instead of sunk into it
        if constexpr (SHARE_DD) {
          if constexpr (K >= 2) asm volatile("" : "+v"(acc));
          if (K == 1 || hk == 0) s_part[j][w][c] = acc;
        } else {
          yp[j] = acc;
        }
      }
    };
    const int nj = FULL ? T : (int)(t1 - ts);
    constexpr int NMID = (T > CKL) ? T / CKL - 1 : 1;   // checkpoint positions inside the tile
    float hmid[NMID][NS];
    constexpr int PD = NS == 1 ? 3 : (ZOH ? 1 : 2);   // tokens of LDS operands in flight ahead
    auto sweep = [&]() {
      Ops ring[PD + 1];
#pragma unroll
      for (int q = 0; q < PD; ++q)
        if (q < T && (FULL || q < nj)) fetch(q, ring[q]);
#pragma unroll
      for (int j = 0; j < T; ++j) {
        if (FULL || j < nj) {
          if (j + PD < T && (FULL || j + PD < nj)) fetch(j + PD, ring[(j + PD) % (PD + 1)]);
          compute(j, ring[j % (PD + 1)]);
          if constexpr (CKPT && T > CKL) {
            // the state after token ts + j enters checkpoint chunk (ts + j + 1) / CKL;
            // tiles start at multiples of T, so inside a tile the positions are
            // fixed: keep a copy (no branch here), stored after the tile
            if ((j + 1) % CKL == 0 && j + 1 < T) {
#pragma unroll
              for (int s = 0; s < NS; ++s) hmid[(j + 1) / CKL - 1][s] = h[s];
            }
          }
        }
      }
    };
    sweep();
    if constexpr (AGG) {
      // The aggregate pass stores nothing per token: left free, the compiler
      // sinks its sweep below the barrier that ends the tile, keeping every LDS
      // operand of the tile live across it (up to 256 VGPRs, one or two waves
      // per SIMD instead of five).  Consuming the results here pins the sweep.
#pragma unroll
      for (int s = 0; s < NS; ++s) asm volatile("" : "+v"(h[s]));
      asm volatile("" : "+v"(dsum));
    }

    if constexpr (CKPT) {
      if (ck_row) {
        if constexpr (T > CKL) {
#pragma unroll
          for (int m = 0; m < NMID; ++m) {
            const int64_t tn = ts + (m + 1) * CKL;
            if ((FULL || (m + 1) * CKL <= nj) && tn < L) {
#pragma unroll
              for (int s = 0; s < NS; ++s) ck_row[(tn / CKL) * dm.dim * N + s] = hmid[m][s];
            }
          }
        }
        // the state after the tile's last token; at a chunk's end (te == t1 < L)
        // the next chunk stores that slot from its entering state, so each slot
        // has exactly one writer and the checkpoints are reproducible
        const int64_t te = ts + nj;
        if (te % CKL == 0 && te < t1) {
#pragma unroll
          for (int s = 0; s < NS; ++s) ck_row[(te / CKL) * dm.dim * N + s] = h[s];
        }
      }
    }

    // phase C: the owner of each token sums the partial readouts, adds the skip
    // term, applies the gate and stores y
    if constexpr (SHARE_DD) __syncthreads();
    __builtin_amdgcn_s_setprio(0);
    if constexpr (!AGG) {
      float yv[SPAN];
#pragma unroll
      for (int i = 0; i < SPAN; ++i) {
        float acc;
        if constexpr (SHARE_DD) {
          const int j = otok + i;
          acc = s_part[j][0][oc];
#pragma unroll
          for (int g = 1; g < G; ++g) acc += s_part[j][g][oc];
        } else {
          acc = yp[i];
        }
        yv[i] = fmaf(skip, xv[i], acc);
      }
      if (has_z) {
#pragma unroll
        for (int i = 0; i < SPAN; ++i) yv[i] *= silu(zv[i]);
      }
      if (STAGE_Y && FULL && use_buf) {
        // into the staged tile, stored after the next tile's first barrier
        uint32_t o[SpanT<IO, SPAN>::kWords];
        if constexpr (IO::kPerSpan == 4) {
#pragma unroll
          for (int i = 0; i < SPAN; ++i) o[i] = __float_as_uint(yv[i]);
        } else {
#pragma unroll
          for (int i = 0; i < SPAN; i += 2) o[i >> 1] = pack_bf16x2(yv[i], yv[i + 1]);
        }
        const int w0 = otok * EBY / 4;   // first word of this lane's span
#pragma unroll
        for (int q = 0; q < SpanT<IO, SPAN>::kWords; ++q) s_y[STAGE_Y ? oc : 0][w0 + q] = o[q];
        y_pend_ts = ts;
      } else if (FULL && use_buf) {
        // unconditional for the same reason as the B/C loads: lanes of channels
        // past dim store beyond the buffer's range, which the hardware drops
        const uint32_t vo_y = oact ? vo_row : 0x80000000u;
        buf_store_span<IO, SPAN>(make_rsrc(y + row0 * L, nrows * L * EB), vo_y, (uint32_t)(ts * EB), yv);
      } else if (oact && (FULL || valid > 0)) {
        store_span<IO, SPAN>(y, orow + tf, valid, vec, yv);
      }
    }
  };

  using CkTag = std::integral_constant<bool, CKPT_K>;
  int64_t ts = t0;
  if (use_buf) {
    // pairs of whole tiles whose next tiles are whole: the two span sets
    // alternate, so nothing is copied between tiles
    for (; ts + 3 * T <= t1; ts += 2 * T) {
      tile(std::true_type{}, CkTag{}, std::true_type{}, ts, S0, S1);
      tile(std::true_type{}, CkTag{}, std::true_type{}, ts + T, S1, S0);
    }
  }
  for (; ts < t1; ts += T) {
    if (ts + T <= t1) tile(std::true_type{}, CkTag{}, std::false_type{}, ts, S0, S1);
    else tile(std::false_type{}, CkTag{}, std::false_type{}, ts, S0, S1);
    S0 = S1;
  }
  if constexpr (STAGE_Y) {
    if (use_buf && y_pend_ts >= 0) {   // the chunk's last staged tile
      __syncthreads();
      flush_y();
    }
  }

  if (act) {
    if constexpr (AGG) {
      float* o = agg_h + (ch * dm.num_chunks + chunk) * N + sg * NS;
#pragma unroll
      for (int s = 0; s < NS; ++s) o[s] = h[s];
      if (sg == 0) agg_s[ch * dm.num_chunks + chunk] = dsum;
    } else if (h_final && chunk == dm.num_chunks - 1) {
#pragma unroll
      for (int s = 0; s < NS; ++s) h_final[ch * N + sg * NS + s] = h[s];
    }
  }
}

template <int N, int G, int K, typename IO, bool AGG, bool ZOH, bool CKPT, bool ROWS>
hipError_t launch_scan_one(const ScanDims& dm, const ScanPtrs& p, hipStream_t s, int64_t nwg) {
  using E = typename IO::T;
  hipLaunchKernelGGL((scan_kernel<N, G, K, IO, AGG, ZOH, CKPT, ROWS>), dim3((unsigned)nwg), dim3(64 * G), 0, s,
                     dm, (const E*)p.x, (const E*)p.dt, (const E*)p.z, (const E*)p.B, (const E*)p.C, p.A, p.Dskip,
                     p.dt_bias, p.h0, p.h_in,
                     (E*)p.y, p.h_final, p.agg_h, p.agg_s, CKPT ? p.ckpt : nullptr);
  return hipGetLastError();
}

// rows of at least 1 MB take the row-segment owners (bf16, two lanes per
// channel, four waves)
template <int N, int G, int K, typename IO, bool AGG, bool ZOH, bool CKPT>
hipError_t launch_scan_r(const ScanDims& dm, const ScanPtrs& p, hipStream_t s, int64_t nwg) {
  if constexpr (K == 2 && G == 4 && sizeof(typename IO::T) == 2) {
    if (dm.seqlen * 2 >= (int64_t(1) << 20)) return launch_scan_one<N, G, K, IO, AGG, ZOH, CKPT, true>(dm, p, s, nwg);
  }
  return launch_scan_one<N, G, K, IO, AGG, ZOH, CKPT, false>(dm, p, s, nwg);
}

template <int N, int G, int K, typename IO, bool AGG, bool ZOH>
hipError_t launch_scan_t(const ScanDims& dm, const ScanPtrs& p, hipStream_t s) {
  const int64_t cblocks = (dm.dim + 64 / K - 1) / (64 / K);
  const int64_t nwg = cblocks * dm.batch * dm.num_chunks;
  if constexpr (!AGG) {
    if (p.ckpt) return launch_scan_r<N, G, K, IO, false, ZOH, true>(dm, p, s, nwg);
  }
  return launch_scan_r<N, G, K, IO, AGG, ZOH, false>(dm, p, s, nwg);
}

template <int N, int G, typename IO, bool AGG, bool ZOH>
hipError_t launch_scan_k(const ScanDims& dm, const ScanPtrs& p, hipStream_t s) {
  if (dm.lanes == 1) return launch_scan_t<N, G, 1, IO, AGG, ZOH>(dm, p, s);
  if constexpr (N >= 2 * G) {
    if (dm.lanes == 2) return launch_scan_t<N, G, 2, IO, AGG, ZOH>(dm, p, s);
  }
  if constexpr (N >= 4 * G && G == 4) {
    if (dm.lanes == 4) return launch_scan_t<N, G, 4, IO, AGG, ZOH>(dm, p, s);
  }
  return hipErrorInvalidValue;
}

template <int N, typename IO, bool AGG, bool ZOH>
hipError_t launch_scan_g(const ScanDims& dm, const ScanPtrs& p, hipStream_t s) {
  switch (dm.groups) {
    case 1: return launch_scan_k<N, 1, IO, AGG, ZOH>(dm, p, s);
    case 2: if constexpr (N >= 2) return launch_scan_k<N, 2, IO, AGG, ZOH>(dm, p, s); else break;
    case 4: if constexpr (N >= 4) return launch_scan_k<N, 4, IO, AGG, ZOH>(dm, p, s); else break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <typename IO, bool AGG, bool ZOH>
hipError_t launch_scan_n(const ScanDims& dm, const ScanPtrs& p, hipStream_t s) {
  switch (dm.dstate) {
    case 1: return launch_scan_g<1, IO, AGG, ZOH>(dm, p, s);
    case 2: return launch_scan_g<2, IO, AGG, ZOH>(dm, p, s);
    case 4: return launch_scan_g<4, IO, AGG, ZOH>(dm, p, s);
    case 8: return launch_scan_g<8, IO, AGG, ZOH>(dm, p, s);
    case 16: return launch_scan_g<16, IO, AGG, ZOH>(dm, p, s);
    default: return hipErrorInvalidValue;
  }
}

// Entry used by the instantiating translation units.
template <typename IO, bool ZOH>
hipError_t launch_scan_impl(const ScanDims& dm, const ScanPtrs& p, bool aggregate, hipStream_t s) {
  return aggregate ? launch_scan_n<IO, true, ZOH>(dm, p, s) : launch_scan_n<IO, false, ZOH>(dm, p, s);
}

}  // namespace scan_detail
}  // namespace ssscan
