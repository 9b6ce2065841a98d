// C ABI of the selective-scan library: argument validation, planning, launches,
// error reporting and the opt-in kernel timing record.  See include/ssscan.h.
#include "ssscan.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace {

thread_local std::string g_last_error;

ss_status fail(ss_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ss_status hip_fail(hipError_t e, const char* what) {
  return fail(SS_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

}  // namespace

namespace ssscan {

ss_status record_error(ss_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ss_status record_hip_error(hipError_t e, const char* what) { return hip_fail(e, what); }

}  // namespace ssscan

namespace {

bool valid_dstate(int n) { return n == 1 || n == 2 || n == 4 || n == 8 || n == 16; }

int elem_bytes(ss_dtype io) { return io == SS_BF16 ? 2 : 4; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
  const char* name;
  uintptr_t lo, hi;   // [lo, hi)
};

Range rng(const char* name, const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{name, lo, p ? lo + (uintptr_t)bytes : lo};
}

bool overlap(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// Device properties are queried once per device.
int device_cus() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

constexpr int64_t kMaxDim = int64_t(1) << 40;

ss_status check_sizes(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io) {
  if (io != SS_F32 && io != SS_BF16) return fail(SS_ERR_UNSUPPORTED, "io dtype %d is not SS_F32 or SS_BF16", (int)io);
  if (!valid_dstate(dstate)) return fail(SS_ERR_UNSUPPORTED, "dstate %d is not one of 1, 2, 4, 8, 16", dstate);
  if (batch < 1 || dim < 1 || seqlen < 0)
    return fail(SS_ERR_INVALID_ARG, "sizes must be batch >= 1, dim >= 1, seqlen >= 0 (got %lld, %lld, %lld)",
                (long long)batch, (long long)dim, (long long)seqlen);
  if (batch > kMaxDim || dim > kMaxDim || seqlen > kMaxDim)
    return fail(SS_ERR_INVALID_ARG, "a size exceeds 2^40");
  const __int128 elems = (__int128)batch * dim * (seqlen > 0 ? seqlen : 1) * 16;
  if (elems > ((__int128)1 << 62)) return fail(SS_ERR_INVALID_ARG, "tensor sizes overflow 64-bit byte offsets");
  return SS_OK;
}

struct Plan {
  int groups;
  int lanes;
  int64_t chunk_len;
  int num_chunks;
  int tile;
};

int io_code(ss_dtype io) { return io == SS_BF16 ? ssscan::kIoBf16 : ssscan::kIoF32; }

// Automatic plan.  Four waves per workgroup split the state components, and for
// N >= 8 two lanes per channel split them further, so a workgroup covers 32
// channels: twice as many equal workgroups for the same work, which evens out
// the per-CU load when the workgroup count is not a multiple of the CU count.
// Chunking doubles the VALU work of all but the first chunk, so it is used only
// when the unchunked launch would leave most SIMDs idle; then chunks are sized
// for ~64 workgroups per CU, at least 2048 tokens each (the long-context
// workload: 16 chunks 19.6 ms, 64 chunks 17.0 ms, 256 chunks 16.2 ms).
Plan auto_plan(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io) {
  Plan p;
  p.groups = dstate >= 4 ? 4 : dstate;
  p.lanes = dstate >= 8 ? 2 : 1;
  p.tile = ssscan::tile_len(p.groups, p.lanes, io_code(io));
  const int64_t cpb = 64 / p.lanes;
  const int64_t wgs = ((dim + cpb - 1) / cpb) * batch;
  const int64_t waves = wgs * p.groups;
  const int64_t simds = (int64_t)device_cus() * 4;
  int64_t chunks = 1;
  if (waves * 2 < simds && seqlen >= 8192) {
    // ~64 workgroups per CU: small chunks balance best over the CUs, while the
    // combine over chunks stays negligible
    const int64_t cus = simds / 4;
    chunks = (64 * cus + wgs - 1) / wgs;
    const int64_t max_chunks = seqlen / 2048;
    if (chunks > max_chunks) chunks = max_chunks;
    if (chunks < 1) chunks = 1;
  }
  // Unchunked launches with fewer than two workgroups per CU (one wave per SIMD
  // each) leave SIMDs idle; four lanes per channel (one state component each)
  // halve the channels per workgroup and double the workgroups, for a little more
  // VALU work per channel (130M-shaped layer: 384 -> 768 workgroups).
  if (chunks == 1 && dstate >= 16 && wgs < 2 * (simds / 4)) {
    p.lanes = 4;
    p.tile = ssscan::tile_len(p.groups, p.lanes, io_code(io));
  }
  int64_t cl = (seqlen + chunks - 1) / chunks;
  cl = ((cl + p.tile - 1) / p.tile) * p.tile;
  if (cl < p.tile) cl = p.tile;
  p.chunk_len = cl;
  p.num_chunks = seqlen > 0 ? (int)((seqlen + cl - 1) / cl) : 1;
  return p;
}

ss_status make_plan(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io, const ss_scan_plan* in,
                    Plan* out) {
  if (!in) {
    *out = auto_plan(batch, dim, dstate, seqlen, io);
    return SS_OK;
  }
  Plan p;
  p.groups = in->state_groups;
  p.lanes = in->lanes_per_channel == 0 ? 1 : in->lanes_per_channel;
  if (!(p.groups == 1 || p.groups == 2 || p.groups == 4) || p.groups > dstate)
    return fail(SS_ERR_UNSUPPORTED, "plan.state_groups %d must be 1, 2 or 4 and at most dstate (%d)", p.groups,
                dstate);
  if (!(p.lanes == 1 || p.lanes == 2 || (p.lanes == 4 && p.groups == 4)) || p.groups * p.lanes > dstate)
    return fail(SS_ERR_UNSUPPORTED,
                "plan.lanes_per_channel %d must be 1, 2 or 4 (4 with 4 state groups), with state_groups * "
                "lanes_per_channel <= dstate (%d)",
                in->lanes_per_channel, dstate);
  p.tile = ssscan::tile_len(p.groups, p.lanes, io_code(io));
  int64_t cl = in->chunk_len;
  if (cl <= 0) return fail(SS_ERR_INVALID_ARG, "plan.chunk_len must be positive (got %lld)", (long long)cl);
  if (cl >= seqlen) {
    cl = ((seqlen + p.tile - 1) / p.tile) * p.tile;
    if (cl < p.tile) cl = p.tile;
  }
  if (cl % p.tile != 0)
    return fail(SS_ERR_INVALID_ARG, "plan.chunk_len %lld is not a multiple of the tile length %d", (long long)cl,
                p.tile);
  const int64_t nc = seqlen > 0 ? (seqlen + cl - 1) / cl : 1;
  if (nc > (1 << 20)) return fail(SS_ERR_INVALID_ARG, "plan gives %lld chunks (limit 2^20)", (long long)nc);
  p.chunk_len = cl;
  p.num_chunks = (int)nc;
  *out = p;
  return SS_OK;
}

struct WsLayout {
  size_t agg_h, agg_s, h_in, total;
};

size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

// The forward's scratch: on chunked plans only, each chunk's end state from a
// zero start and sum of Delta, and each chunk's entering state.
WsLayout ws_layout(int64_t batch, int64_t dim, int dstate, int64_t seqlen, const Plan& p) {
  (void)seqlen;
  WsLayout w{};
  size_t off = 0;
  if (p.num_chunks > 1) {
    const size_t st = (size_t)batch * dim * p.num_chunks * dstate * sizeof(float);
    w.agg_h = off;
    off += round256(st);
    w.agg_s = off;
    off += round256((size_t)batch * dim * p.num_chunks * sizeof(float));
    w.h_in = off;
    off += round256(st);
  }
  w.total = off;
  return w;
}

// ---- timing record ----
struct Timing {
  std::mutex mu;
  bool enabled = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
  double total_ms = 0.0;
  int64_t calls = 0;
};
Timing g_timing;

bool timing_on() {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  return g_timing.enabled;
}

ss_status timing_pair(hipEvent_t* a, hipEvent_t* b) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (!g_timing.pool.empty()) {
    *a = g_timing.pool.back().first;
    *b = g_timing.pool.back().second;
    g_timing.pool.pop_back();
    return SS_OK;
  }
  hipError_t e = hipEventCreate(a);
  if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  e = hipEventCreate(b);
  if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  return SS_OK;
}

}  // namespace

extern "C" {

int ss_abi_version(void) { return SS_ABI_VERSION; }

const char* ss_status_string(ss_status s) {
  switch (s) {
    case SS_OK: return "SS_OK";
    case SS_ERR_INVALID_ARG: return "SS_ERR_INVALID_ARG";
    case SS_ERR_UNSUPPORTED: return "SS_ERR_UNSUPPORTED";
    case SS_ERR_WORKSPACE: return "SS_ERR_WORKSPACE";
    case SS_ERR_HIP: return "SS_ERR_HIP";
    default: return "SS_ERR_UNKNOWN";
  }
}

const char* ss_last_error(void) { return g_last_error.c_str(); }

ss_status ss_scan_fwd_plan(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io,
                           ss_scan_plan* plan_out) {
  ss_status st = check_sizes(batch, dim, dstate, seqlen, io);
  if (st != SS_OK) return st;
  if (!plan_out) return fail(SS_ERR_INVALID_ARG, "plan_out is NULL");
  const Plan p = auto_plan(batch, dim, dstate, seqlen, io);
  plan_out->state_groups = p.groups;
  plan_out->lanes_per_channel = p.lanes;
  plan_out->chunk_len = p.chunk_len;
  return SS_OK;
}

size_t ss_scan_fwd_workspace_bytes(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io,
                                   const ss_scan_plan* plan) {
  if (check_sizes(batch, dim, dstate, seqlen, io) != SS_OK) return 0;
  Plan p;
  if (make_plan(batch, dim, dstate, seqlen, io, plan, &p) != SS_OK) return 0;
  const WsLayout w = ws_layout(batch, dim, dstate, seqlen, p);
  return w.total > 0 ? w.total : 256;
}

}  // extern "C"

namespace {

ss_status scan_fwd_impl(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io, const void* x,
                        const void* dt, const void* z, const void* B, const void* C, const float* A,
                        const float* Dskip, const float* dt_bias, const float* h0, void* y, float* h_final,
                        void* workspace, size_t workspace_bytes, const ss_scan_plan* plan, void* stream, bool zoh,
                        bool dt_row = false, float* ckpt = nullptr) {
  ss_status st = check_sizes(batch, dim, dstate, seqlen, io);
  if (st != SS_OK) return st;
  Plan p;
  st = make_plan(batch, dim, dstate, seqlen, io, plan, &p);
  if (st != SS_OK) return st;

  const int64_t eb = elem_bytes(io);
  const int64_t seq_bytes = batch * dim * seqlen * eb;
  const int64_t bc_bytes = batch * dstate * seqlen * eb;
  const int64_t st_bytes = batch * dim * dstate * 4;
  if (seqlen > 0) {
    if (!x) return fail(SS_ERR_INVALID_ARG, "x is NULL");
    if (!dt) return fail(SS_ERR_INVALID_ARG, "dt is NULL");
    if (!B) return fail(SS_ERR_INVALID_ARG, "B is NULL");
    if (!C) return fail(SS_ERR_INVALID_ARG, "C is NULL");
    if (!y) return fail(SS_ERR_INVALID_ARG, "y is NULL");
  }
  if (!A) return fail(SS_ERR_INVALID_ARG, "A is NULL");
  const void* a16[] = {x, dt, z, B, C, A, h0, y, h_final};
  const char* n16[] = {"x", "dt", "z", "B", "C", "A", "h0", "y", "h_final"};
  for (int i = 0; i < 9; ++i)
    if (a16[i] && !aligned(a16[i], 16)) return fail(SS_ERR_INVALID_ARG, "%s is not 16-byte aligned", n16[i]);
  if (Dskip && !aligned(Dskip, 4)) return fail(SS_ERR_INVALID_ARG, "Dskip is not 4-byte aligned");
  if (dt_bias && !aligned(dt_bias, 4)) return fail(SS_ERR_INVALID_ARG, "dt_bias is not 4-byte aligned");

  const WsLayout wl = ws_layout(batch, dim, dstate, seqlen, p);
  if (seqlen > 0) {
    if (!workspace) return fail(SS_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", wl.total);
    if (!aligned(workspace, 256)) return fail(SS_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < wl.total)
      return fail(SS_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, wl.total);
  }

  // outputs must not overlap inputs, each other, or the workspace
  const int64_t dt_bytes = dt_row ? batch * seqlen * eb : seq_bytes;
  const Range ins[] = {rng("x", x, seq_bytes), rng("dt", dt, dt_bytes), rng("z", z, seq_bytes),
                       rng("B", B, bc_bytes), rng("C", C, bc_bytes), rng("A", A, dim * dstate * 4),
                       rng("Dskip", Dskip, dim * 4), rng("dt_bias", dt_bias, dim * 4), rng("h0", h0, st_bytes)};
  if (ckpt && !aligned(ckpt, 16)) return fail(SS_ERR_INVALID_ARG, "ckpt is not 16-byte aligned");
  const int64_t ck_len = ssscan::bwd_chunk_len(dstate);
  const int64_t ck_count = (seqlen + ck_len - 1) / ck_len;
  const Range outs[] = {rng("y", y, seq_bytes), rng("h_final", h_final, st_bytes),
                        rng("workspace", workspace, seqlen > 0 ? (int64_t)wl.total : 0),
                        rng("ckpt", ckpt, batch * dim * ck_count * dstate * 4)};
  for (const Range& o : outs) {
    for (const Range& i : ins)
      if (overlap(o, i)) return fail(SS_ERR_INVALID_ARG, "%s overlaps input %s", o.name, i.name);
  }
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return fail(SS_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, outs[j].name);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (seqlen == 0) {
    if (h_final) {
      hipError_t e = ssscan::launch_copy_state(batch * dim * dstate, h0, h_final, s);
      if (e != hipSuccess) return hip_fail(e, "copy_state launch");
    }
    return SS_OK;
  }

  ssscan::ScanDims dm{};
  dm.batch = batch;
  dm.dim = dim;
  dm.seqlen = seqlen;
  dm.chunk_len = p.chunk_len;
  dm.num_chunks = p.num_chunks;
  dm.dstate = dstate;
  dm.groups = p.groups;
  dm.lanes = p.lanes;
  dm.io = io_code(io);
  dm.vec = (seqlen % ssscan::span_len(p.lanes, dm.io)) == 0 ? 1 : 0;
  // buffer resources address a workgroup's rows with 32-bit offsets
  dm.buf = (dm.vec && seqlen % 4 == 0 && (64 / p.lanes) * seqlen * elem_bytes(io) < (int64_t(1) << 31) &&
            dstate * seqlen * elem_bytes(io) < (int64_t(1) << 31)) ? 1 : 0;
  dm.dt_row = dt_row ? 1 : 0;
  dm.ck_count = ck_count;

  const int64_t cpb = 64 / p.lanes;
  const int64_t nwg = ((dim + cpb - 1) / cpb) * batch * p.num_chunks;
  if (nwg > 0x7fffffffLL) return fail(SS_ERR_INVALID_ARG, "launch needs %lld workgroups (limit 2^31-1)", (long long)nwg);

  char* ws = static_cast<char*>(workspace);
  ssscan::ScanPtrs sp{};
  sp.x = x;
  sp.dt = dt;
  sp.z = z;
  sp.B = B;
  sp.C = C;
  sp.A = A;
  sp.Dskip = Dskip;
  sp.dt_bias = dt_bias;
  sp.h0 = h0;
  sp.y = y;
  sp.h_final = h_final;
  sp.ckpt = ckpt;
  hipError_t e;
  const bool timed = timing_on();
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (timed) {
    st = timing_pair(&ev0, &ev1);
    if (st != SS_OK) return st;
    e = hipEventRecord(ev0, s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }

  if (p.num_chunks > 1) {
    sp.agg_h = reinterpret_cast<float*>(ws + wl.agg_h);
    sp.agg_s = reinterpret_cast<float*>(ws + wl.agg_s);
    float* h_in = reinterpret_cast<float*>(ws + wl.h_in);
    e = ssscan::launch_scan(dm, sp, /*aggregate=*/true, zoh, s);
    if (e != hipSuccess) return hip_fail(e, "scan (aggregate) launch");
    e = ssscan::launch_combine(dm, A, sp.agg_h, sp.agg_s, h0, h_in, s);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    sp.h_in = h_in;
  }
  e = ssscan::launch_scan(dm, sp, /*aggregate=*/false, zoh, s);
  if (e != hipSuccess) return hip_fail(e, "scan launch");

  if (timed) {
    e = hipEventRecord(ev1, s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    std::lock_guard<std::mutex> lk(g_timing.mu);
    g_timing.pending.emplace_back(ev0, ev1);
  }
  return SS_OK;
}

ss_status state_update_impl(int64_t batch, int64_t dim, int dstate, ss_dtype io, float* state, const void* x,
                            const void* dt, const void* z, const void* B, const void* C, const float* A,
                            const float* Dskip, const float* dt_bias, void* y, void* stream, bool zoh,
                            bool dt_row = false) {
  ss_status st = check_sizes(batch, dim, dstate, 1, io);
  if (st != SS_OK) return st;
  if ((__int128)batch * dim > ((__int128)1 << 34))
    return fail(SS_ERR_UNSUPPORTED, "batch * dim exceeds 2^34 channels (%lld x %lld)", (long long)batch,
                (long long)dim);
  const char* names[] = {"state", "x", "dt", "B", "C", "A", "y"};
  const void* req[] = {state, x, dt, B, C, A, y};
  for (int i = 0; i < 7; ++i)
    if (!req[i]) return fail(SS_ERR_INVALID_ARG, "%s is NULL", names[i]);
  const void* a16[] = {state, x, dt, z, B, C, A, y};
  const char* n16[] = {"state", "x", "dt", "z", "B", "C", "A", "y"};
  for (int i = 0; i < 8; ++i)
    if (a16[i] && !aligned(a16[i], 16)) return fail(SS_ERR_INVALID_ARG, "%s is not 16-byte aligned", n16[i]);
  if (Dskip && !aligned(Dskip, 4)) return fail(SS_ERR_INVALID_ARG, "Dskip is not 4-byte aligned");
  if (dt_bias && !aligned(dt_bias, 4)) return fail(SS_ERR_INVALID_ARG, "dt_bias is not 4-byte aligned");
  const int64_t eb = elem_bytes(io);
  const int64_t tok = batch * dim * eb;
  const Range ins[] = {rng("x", x, tok), rng("dt", dt, dt_row ? batch * eb : tok), rng("z", z, tok),
                       rng("B", B, batch * dstate * eb), rng("C", C, batch * dstate * eb),
                       rng("A", A, dim * dstate * 4), rng("Dskip", Dskip, dim * 4),
                       rng("dt_bias", dt_bias, dim * 4)};
  const Range outs[] = {rng("state", state, batch * dim * dstate * 4), rng("y", y, tok)};
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (overlap(o, i)) return fail(SS_ERR_INVALID_ARG, "%s overlaps input %s", o.name, i.name);
  if (overlap(outs[0], outs[1])) return fail(SS_ERR_INVALID_ARG, "state overlaps y");
  hipError_t e = ssscan::launch_state_update(batch, dim, dstate, io_code(io), zoh, dt_row, state, x, dt, z, B, C, A, Dskip,
                                             dt_bias, y, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "state_update launch");
  return SS_OK;
}

ss_status shard_state_impl(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io, const void* x,
                           const void* dt, const void* B, const float* A, const float* dt_bias, float* dsum,
                           float* h_end, void* workspace, size_t workspace_bytes, void* stream, bool zoh) {
  ss_status st = check_sizes(batch, dim, dstate, seqlen, io);
  if (st != SS_OK) return st;
  if (!A || !dsum || !h_end) return fail(SS_ERR_INVALID_ARG, "%s is NULL", !A ? "A" : (!dsum ? "dsum" : "h_end"));
  if (seqlen > 0 && (!x || !dt || !B)) return fail(SS_ERR_INVALID_ARG, "%s is NULL", !x ? "x" : (!dt ? "dt" : "B"));
  const void* a16[] = {x, dt, B, A, h_end};
  const char* n16[] = {"x", "dt", "B", "A", "h_end"};
  for (int i = 0; i < 5; ++i)
    if (a16[i] && !aligned(a16[i], 16)) return fail(SS_ERR_INVALID_ARG, "%s is not 16-byte aligned", n16[i]);
  if (dt_bias && !aligned(dt_bias, 4)) return fail(SS_ERR_INVALID_ARG, "dt_bias is not 4-byte aligned");
  if (!aligned(dsum, 4)) return fail(SS_ERR_INVALID_ARG, "dsum is not 4-byte aligned");
  const Plan p = auto_plan(batch, dim, dstate, seqlen, io);
  const WsLayout wl = ws_layout(batch, dim, dstate, seqlen, p);
  if (seqlen > 0) {
    if (!workspace) return fail(SS_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", wl.total);
    if (!aligned(workspace, 256)) return fail(SS_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < wl.total)
      return fail(SS_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, wl.total);
  }
  const int64_t eb = elem_bytes(io);
  const int64_t seq_bytes = batch * dim * seqlen * eb;
  const Range ins[] = {rng("x", x, seq_bytes), rng("dt", dt, seq_bytes), rng("B", B, batch * dstate * seqlen * eb),
                       rng("A", A, dim * dstate * 4), rng("dt_bias", dt_bias, dim * 4)};
  const Range outs[] = {rng("dsum", dsum, batch * dim * 4), rng("h_end", h_end, batch * dim * dstate * 4),
                        rng("workspace", workspace, seqlen > 0 ? (int64_t)wl.total : 0)};
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (overlap(o, i)) return fail(SS_ERR_INVALID_ARG, "%s overlaps input %s", o.name, i.name);
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return fail(SS_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, outs[j].name);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (seqlen == 0) {
    e = ssscan::launch_fill_zero(h_end, batch * dim * dstate, s);
    if (e == hipSuccess) e = ssscan::launch_fill_zero(dsum, batch * dim, s);
    return e == hipSuccess ? SS_OK : hip_fail(e, "zero-fill launch");
  }
  ssscan::ScanDims dm{};
  dm.batch = batch;
  dm.dim = dim;
  dm.seqlen = seqlen;
  dm.chunk_len = p.chunk_len;
  dm.num_chunks = p.num_chunks;
  dm.dstate = dstate;
  dm.groups = p.groups;
  dm.lanes = p.lanes;
  dm.io = io_code(io);
  dm.vec = (seqlen % ssscan::span_len(p.lanes, dm.io)) == 0 ? 1 : 0;
  // buffer resources address a workgroup's rows with 32-bit offsets
  dm.buf = (dm.vec && seqlen % 4 == 0 && (64 / p.lanes) * seqlen * elem_bytes(io) < (int64_t(1) << 31) &&
            dstate * seqlen * elem_bytes(io) < (int64_t(1) << 31)) ? 1 : 0;
  char* ws = static_cast<char*>(workspace);
  ssscan::ScanPtrs sp{};
  sp.x = x;
  sp.dt = dt;
  sp.B = B;
  sp.C = B;   // the aggregate pass reads no C
  sp.A = A;
  sp.dt_bias = dt_bias;
  if (p.num_chunks == 1) {
    sp.agg_h = h_end;   // (batch, dim, 1, N) and (batch, dim, 1)
    sp.agg_s = dsum;
    e = ssscan::launch_scan(dm, sp, /*aggregate=*/true, zoh, s);
    return e == hipSuccess ? SS_OK : hip_fail(e, "scan (aggregate) launch");
  }
  sp.agg_h = reinterpret_cast<float*>(ws + wl.agg_h);
  sp.agg_s = reinterpret_cast<float*>(ws + wl.agg_s);
  e = ssscan::launch_scan(dm, sp, /*aggregate=*/true, zoh, s);
  if (e != hipSuccess) return hip_fail(e, "scan (aggregate) launch");
  e = ssscan::launch_shard_reduce(dm, A, sp.agg_h, sp.agg_s, h_end, dsum, s);
  return e == hipSuccess ? SS_OK : hip_fail(e, "shard reduce launch");
}

// Segments of a split backward.  The backward takes a (batch row, channel
// block) through all its tokens in one workgroup, so a long sequence with few
// rows and channels would leave most CUs idle; it is then cut into segments run
// by separate workgroups, whose incoming state and adjoint come from aggregate
// passes and combines (about a third of the main pass's work again).
// Automatic, as the forward's chunks: sequences of at least 8192 tokens whose
// unsplit launch has fewer than two workgroups per CU get about 64 workgroups
// per CU, in segments of at least 2048 tokens (million-token workload: 7
// segments 132 ms, 24 segments 96.6 ms, 128 segments 83.2 ms, 512 segments
// 80.2 ms).  Segment lengths are multiples of 64 tokens: whole backward chunks
// and whole forward tiles.
constexpr int64_t kBwdSegAlign = 64;

struct BwdSeg {
  int64_t len;   // tokens per segment; when n == 1, the sequence padded to whole chunks
  int64_t n;     // segments
};

BwdSeg bwd_seg_of_len(int64_t seqlen, int dstate, int64_t len) {
  const int64_t ck = ssscan::bwd_chunk_len(dstate);
  if (len <= 0 || len >= seqlen) return BwdSeg{(seqlen + ck - 1) / ck * ck, 1};
  return BwdSeg{len, (seqlen + len - 1) / len};
}

BwdSeg bwd_auto_segments(int64_t batch, int64_t dim, int dstate, int64_t seqlen) {
  const int64_t cpb = 64 / ssscan::bwd_lanes_per_channel(dstate);
  const int64_t wgs = ((dim + cpb - 1) / cpb) * batch;
  const int64_t cus = device_cus();
  int64_t n = 1;
  if (seqlen >= 8192 && wgs < 2 * cus) {
    n = (64 * cus + wgs - 1) / wgs;
    const int64_t nmax = seqlen / 2048;
    if (n > nmax) n = nmax;
  }
  if (n <= 1) return bwd_seg_of_len(seqlen, dstate, 0);
  int64_t len = (seqlen + n - 1) / n;
  len = (len + kBwdSegAlign - 1) / kBwdSegAlign * kBwdSegAlign;
  return bwd_seg_of_len(seqlen, dstate, len);
}

// requested: 0 = automatic, else the segment length (a positive multiple of 64)
ss_status bwd_plan_segments(int64_t batch, int64_t dim, int dstate, int64_t seqlen, int64_t requested,
                            BwdSeg* out) {
  if (requested < 0 || requested % kBwdSegAlign != 0)
    return fail(SS_ERR_INVALID_ARG, "segment_len %lld must be 0 (automatic) or a positive multiple of %lld",
                (long long)requested, (long long)kBwdSegAlign);
  *out = requested == 0 ? bwd_auto_segments(batch, dim, dstate, seqlen) : bwd_seg_of_len(seqlen, dstate, requested);
  if (out->n > (1 << 20))
    return fail(SS_ERR_INVALID_ARG, "segment_len %lld gives %lld segments (limit 2^20)", (long long)requested,
                (long long)out->n);
  return SS_OK;
}

struct BwdLayout {
  size_t bc, ckpt, part, dA_p, dD_p, dbias_p, h_seg, agg_h, lam_seg, adj_m, adj_s, total;
  int64_t cblocks, chunks;
};

BwdLayout bwd_layout(int64_t batch, int64_t dim, int dstate, int64_t seqlen, const BwdSeg& sg) {
  BwdLayout w{};
  const int64_t cpb = 64 / ssscan::bwd_lanes_per_channel(dstate);
  const int64_t ck = ssscan::bwd_chunk_len(dstate);
  w.cblocks = (dim + cpb - 1) / cpb;
  w.chunks = (seqlen + ck - 1) / ck;
  size_t off = 0;
  w.bc = off;
  off += round256((size_t)batch * seqlen * dstate * 2 * sizeof(float));
  w.ckpt = off;
  off += round256((size_t)batch * dim * w.chunks * dstate * sizeof(float));
  w.part = off;   // partials (batch, channel block, chunk, output, chunk token)
  off += round256((size_t)batch * w.cblocks * ssscan::bwd_part_outputs(dstate) * (w.chunks * ck) * sizeof(float));
  w.dA_p = off;   // per-(segment, row) sums
  off += round256((size_t)sg.n * batch * dim * dstate * sizeof(float));
  w.dD_p = off;
  off += round256((size_t)sg.n * batch * dim * sizeof(float));
  w.dbias_p = off;
  off += round256((size_t)sg.n * batch * dim * sizeof(float));
  if (sg.n > 1) {
    const size_t st = (size_t)batch * dim * sg.n * dstate * sizeof(float);
    const size_t sc = (size_t)batch * dim * sg.n * sizeof(float);
    w.h_seg = off;   // state entering each segment
    off += round256(st);
    w.agg_h = off;   // each segment's end state from zero
    off += round256(st);
    w.lam_seg = off;   // adjoint entering each segment
    off += round256(st);
    w.adj_m = off;   // each segment's adjoint aggregate
    off += round256(st);
    w.adj_s = off;   // each segment's sum of Delta (the exponent of both decays)
    off += round256(sc);
  }
  w.total = off;
  return w;
}

ss_status scan_bwd_impl(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io, const void* x,
                        const void* dt, const void* z, const void* B, const void* C, const float* A,
                        const float* Dskip, const float* dt_bias, const float* h0, const void* dy,
                        const float* dh_final, void* dx, void* ddt, void* dz, void* dB, void* dC, float* dA,
                        float* dDskip, float* ddt_bias, float* dh0, void* workspace, size_t workspace_bytes,
                        void* stream, const float* ckpt = nullptr, bool dt_row = false, bool zoh = false,
                        int64_t seg_req = 0) {
  ss_status st = check_sizes(batch, dim, dstate, seqlen, io);
  if (st != SS_OK) return st;
  BwdSeg sgm;
  st = bwd_plan_segments(batch, dim, dstate, seqlen, seg_req, &sgm);
  if (st != SS_OK) return st;
  if (!A) return fail(SS_ERR_INVALID_ARG, "A is NULL");
  if (ckpt && !aligned(ckpt, 16)) return fail(SS_ERR_INVALID_ARG, "ckpt is not 16-byte aligned");
  if (seqlen > 0) {
    const char* names[] = {"x", "dt", "B", "C", "dy", "dx", "ddt", "dB", "dC"};
    const void* req[] = {x, dt, B, C, dy, dx, ddt, dB, dC};
    for (int i = 0; i < 9; ++i)
      if (!req[i]) return fail(SS_ERR_INVALID_ARG, "%s is NULL", names[i]);
  }
  if ((z == nullptr) != (dz == nullptr))
    return fail(SS_ERR_INVALID_ARG, "dz must be given exactly when z is (z %s, dz %s)", z ? "set" : "NULL",
                dz ? "set" : "NULL");
  const void* a16[] = {x, dt, z, B, C, A, h0, dy, dh_final, dx, ddt, dz, dB, dC, dA, dh0};
  const char* n16[] = {"x", "dt", "z", "B", "C", "A", "h0", "dy", "dh_final", "dx", "ddt", "dz", "dB", "dC",
                       "dA", "dh0"};
  for (int i = 0; i < 16; ++i)
    if (a16[i] && !aligned(a16[i], 16)) return fail(SS_ERR_INVALID_ARG, "%s is not 16-byte aligned", n16[i]);
  const void* a4[] = {Dskip, dt_bias, dDskip, ddt_bias};
  const char* n4[] = {"Dskip", "dt_bias", "dDskip", "ddt_bias"};
  for (int i = 0; i < 4; ++i)
    if (a4[i] && !aligned(a4[i], 4)) return fail(SS_ERR_INVALID_ARG, "%s is not 4-byte aligned", n4[i]);

  const BwdLayout wl = bwd_layout(batch, dim, dstate, seqlen, sgm);
  if (seqlen > 0) {
    if (!workspace) return fail(SS_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", wl.total);
    if (!aligned(workspace, 256)) return fail(SS_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < wl.total)
      return fail(SS_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, wl.total);
  }
  const int64_t eb = elem_bytes(io);
  const int64_t seq_bytes = batch * dim * seqlen * eb;
  const int64_t dt_bytes = dt_row ? batch * seqlen * eb : seq_bytes;   // dt and ddt
  const int64_t bc_bytes = batch * dstate * seqlen * eb;
  const int64_t st_bytes = batch * dim * dstate * 4;
  const Range ins[] = {rng("x", x, seq_bytes), rng("dt", dt, dt_bytes), rng("z", z, seq_bytes),
                       rng("B", B, bc_bytes), rng("C", C, bc_bytes), rng("A", A, dim * dstate * 4),
                       rng("Dskip", Dskip, dim * 4), rng("dt_bias", dt_bias, dim * 4), rng("h0", h0, st_bytes),
                       rng("dy", dy, seq_bytes), rng("dh_final", dh_final, st_bytes),
                       rng("ckpt", ckpt, batch * dim * wl.chunks * dstate * 4)};
  const Range outs[] = {rng("dx", dx, seq_bytes), rng("ddt", ddt, dt_bytes), rng("dz", dz, seq_bytes),
                        rng("dB", dB, bc_bytes), rng("dC", dC, bc_bytes), rng("dA", dA, dim * dstate * 4),
                        rng("dDskip", dDskip, dim * 4), rng("ddt_bias", ddt_bias, dim * 4),
                        rng("dh0", dh0, st_bytes), rng("workspace", workspace, seqlen > 0 ? (int64_t)wl.total : 0)};
  constexpr int kOuts = sizeof(outs) / sizeof(outs[0]);
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (overlap(o, i)) return fail(SS_ERR_INVALID_ARG, "%s overlaps input %s", o.name, i.name);
  for (int i = 0; i < kOuts; ++i)
    for (int j = i + 1; j < kOuts; ++j)
      if (overlap(outs[i], outs[j])) return fail(SS_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, outs[j].name);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (seqlen == 0) {
    // no tokens: the final state is h0, so dh0 = dh_final; every other gradient is zero
    if (dh0) {
      e = dh_final ? ssscan::launch_copy_state(batch * dim * dstate, dh_final, dh0, s)
                   : ssscan::launch_fill_zero(dh0, batch * dim * dstate, s);
      if (e != hipSuccess) return hip_fail(e, "dh0 launch");
    }
    float* zero[] = {dA, dDskip, ddt_bias};
    const int64_t count[] = {dim * dstate, dim, dim};
    for (int i = 0; i < 3; ++i) {
      e = ssscan::launch_fill_zero(zero[i], count[i], s);
      if (e != hipSuccess) return hip_fail(e, "zero-fill launch");
    }
    return SS_OK;
  }
  const int64_t nwg = wl.cblocks * batch * sgm.n;
  if (nwg > 0x7fffffffLL) return fail(SS_ERR_INVALID_ARG, "launch needs %lld workgroups (limit 2^31-1)", (long long)nwg);

  char* ws = static_cast<char*>(workspace);
  ssscan::ScanDims pd{};
  pd.batch = batch;
  pd.dim = dim;
  pd.seqlen = seqlen;
  pd.dstate = dstate;
  pd.io = io_code(io);
  float* bcw = reinterpret_cast<float*>(ws + wl.bc);
  e = ssscan::launch_prep_bc(pd, B, C, bcw, s);
  if (e != hipSuccess) return hip_fail(e, "prep_bc launch");

  ssscan::BwdDims dm{};
  dm.batch = batch;
  dm.dim = dim;
  dm.seqlen = seqlen;
  dm.cblocks = wl.cblocks;
  dm.dstate = dstate;
  dm.io = io_code(io);
  dm.vec = (seqlen % 2) == 0 ? 1 : 0;
  dm.have_ckpt = ckpt ? 1 : 0;
  dm.dt_row = dt_row ? 1 : 0;
  dm.zoh = zoh ? 1 : 0;
  dm.nseg = (int32_t)sgm.n;
  dm.seg_len = sgm.len;
  ssscan::BwdPtrs bp{};
  bp.x = x;
  bp.dt = dt;
  bp.z = z;
  bp.bc = bcw;
  bp.A = A;
  bp.Dskip = Dskip;
  bp.dt_bias = dt_bias;
  bp.h0 = h0;
  bp.dy = dy;
  bp.dh_final = dh_final;
  bp.dx = dx;
  bp.ddt = ddt;
  bp.dz = dz;
  bp.dB = dB;
  bp.dC = dC;
  bp.dA = dA;
  bp.dDskip = dDskip;
  bp.ddt_bias = ddt_bias;
  bp.dh0 = dh0;
  bp.ckpt = ckpt ? const_cast<float*>(ckpt) : reinterpret_cast<float*>(ws + wl.ckpt);
  bp.part = reinterpret_cast<float*>(ws + wl.part);
  bp.dA_p = reinterpret_cast<float*>(ws + wl.dA_p);
  bp.dD_p = reinterpret_cast<float*>(ws + wl.dD_p);
  bp.dbias_p = reinterpret_cast<float*>(ws + wl.dbias_p);
  if (sgm.n > 1) {
    bp.h_seg = reinterpret_cast<const float*>(ws + wl.h_seg);
    bp.lam_seg = reinterpret_cast<const float*>(ws + wl.lam_seg);
    bp.adj_m = reinterpret_cast<float*>(ws + wl.adj_m);
    bp.adj_s = reinterpret_cast<float*>(ws + wl.adj_s);
    bp.agg_h = reinterpret_cast<float*>(ws + wl.agg_h);
  }

  const bool timed = timing_on();
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (timed) {
    st = timing_pair(&ev0, &ev1);
    if (st != SS_OK) return st;
    e = hipEventRecord(ev0, s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  if (sgm.n > 1) {
    // the segments' aggregates in one pass (their states only when no checkpoints
    // give them), then the combines: the state entering every segment (from h0)
    // and the adjoint entering it from the tokens after it (from dh_final)
    e = ssscan::launch_bwd_segment_agg(dm, bp, /*states=*/!ckpt, s);
    if (e != hipSuccess) return hip_fail(e, "segment aggregate launch");
    if (!ckpt) {
      ssscan::ScanDims cd{};
      cd.batch = batch;
      cd.dim = dim;
      cd.dstate = dstate;
      cd.num_chunks = (int32_t)sgm.n;
      e = ssscan::launch_combine(cd, A, bp.agg_h, bp.adj_s, h0, reinterpret_cast<float*>(ws + wl.h_seg), s);
      if (e != hipSuccess) return hip_fail(e, "combine launch");
    }
    e = ssscan::launch_bwd_adjoint_combine(dm, A, dh_final, bp.adj_m, bp.adj_s, reinterpret_cast<float*>(ws + wl.lam_seg),
                                           s);
    if (e != hipSuccess) return hip_fail(e, "adjoint combine launch");
  }
  e = ssscan::launch_scan_bwd(dm, bp, s);
  if (e != hipSuccess) return hip_fail(e, "scan_bwd launch");
  if (timed) {
    e = hipEventRecord(ev1, s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    std::lock_guard<std::mutex> lk(g_timing.mu);
    g_timing.pending.emplace_back(ev0, ev1);
  }
  return SS_OK;
}

}  // namespace

extern "C" {

ss_status ss_scan_fwd(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io, const void* x,
                      const void* dt, const void* z, const void* B, const void* C, const float* A,
                      const float* Dskip, const float* dt_bias, const float* h0, void* y, float* h_final,
                      void* workspace, size_t workspace_bytes, const ss_scan_plan* plan, void* stream) {
  return scan_fwd_impl(batch, dim, dstate, seqlen, io, x, dt, z, B, C, A, Dskip, dt_bias, h0, y, h_final,
                       workspace, workspace_bytes, plan, stream, false);
}

ss_status ss_scan_fwd_zoh(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io, const void* x,
                          const void* dt, const void* z, const void* B, const void* C, const float* A,
                          const float* Dskip, const float* dt_bias, const float* h0, void* y, float* h_final,
                          void* workspace, size_t workspace_bytes, const ss_scan_plan* plan, void* stream) {
  return scan_fwd_impl(batch, dim, dstate, seqlen, io, x, dt, z, B, C, A, Dskip, dt_bias, h0, y, h_final,
                       workspace, workspace_bytes, plan, stream, true);
}

ss_status ss_state_update(int64_t batch, int64_t dim, int dstate, ss_dtype io, float* state, const void* x,
                          const void* dt, const void* z, const void* B, const void* C, const float* A,
                          const float* Dskip, const float* dt_bias, void* y, void* stream) {
  return state_update_impl(batch, dim, dstate, io, state, x, dt, z, B, C, A, Dskip, dt_bias, y, stream, false);
}

ss_status ss_state_update_zoh(int64_t batch, int64_t dim, int dstate, ss_dtype io, float* state, const void* x,
                              const void* dt, const void* z, const void* B, const void* C, const float* A,
                              const float* Dskip, const float* dt_bias, void* y, void* stream) {
  return state_update_impl(batch, dim, dstate, io, state, x, dt, z, B, C, A, Dskip, dt_bias, y, stream, true);
}

ss_status ss_scan_fwd_ex(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io, uint32_t flags,
                         const void* x, const void* dt, const void* z, const void* B, const void* C, const float* A,
                         const float* Dskip, const float* dt_bias, const float* h0, void* y, float* h_final,
                         float* ckpt, void* workspace, size_t workspace_bytes, const ss_scan_plan* plan,
                         void* stream) {
  if (flags & ~(uint32_t)(SS_FLAG_ZOH | SS_FLAG_DT_PER_ROW))
    return fail(SS_ERR_UNSUPPORTED, "unknown flags 0x%x", (unsigned)flags);
  return scan_fwd_impl(batch, dim, dstate, seqlen, io, x, dt, z, B, C, A, Dskip, dt_bias, h0, y, h_final,
                       workspace, workspace_bytes, plan, stream, (flags & SS_FLAG_ZOH) != 0,
                       (flags & SS_FLAG_DT_PER_ROW) != 0, ckpt);
}

size_t ss_scan_ckpt_bytes(int64_t batch, int64_t dim, int dstate, int64_t seqlen) {
  if (check_sizes(batch, dim, dstate, seqlen, SS_F32) != SS_OK) return 0;
  const int64_t ck = ssscan::bwd_chunk_len(dstate);
  return (size_t)batch * dim * ((seqlen + ck - 1) / ck) * dstate * sizeof(float);
}

ss_status ss_state_update_ex(int64_t batch, int64_t dim, int dstate, ss_dtype io, uint32_t flags, float* state,
                             const void* x, const void* dt, const void* z, const void* B, const void* C,
                             const float* A, const float* Dskip, const float* dt_bias, void* y, void* stream) {
  if (flags & ~(uint32_t)(SS_FLAG_ZOH | SS_FLAG_DT_PER_ROW))
    return fail(SS_ERR_UNSUPPORTED, "unknown flags 0x%x", (unsigned)flags);
  return state_update_impl(batch, dim, dstate, io, state, x, dt, z, B, C, A, Dskip, dt_bias, y, stream,
                           (flags & SS_FLAG_ZOH) != 0, (flags & SS_FLAG_DT_PER_ROW) != 0);
}

ss_status ss_scan_shard_state(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io, const void* x,
                              const void* dt, const void* B, const float* A, const float* dt_bias, float* dsum,
                              float* h_end, void* workspace, size_t workspace_bytes, void* stream) {
  return shard_state_impl(batch, dim, dstate, seqlen, io, x, dt, B, A, dt_bias, dsum, h_end, workspace,
                          workspace_bytes, stream, false);
}

ss_status ss_scan_shard_state_zoh(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io,
                                  const void* x, const void* dt, const void* B, const float* A, const float* dt_bias,
                                  float* dsum, float* h_end, void* workspace, size_t workspace_bytes, void* stream) {
  return shard_state_impl(batch, dim, dstate, seqlen, io, x, dt, B, A, dt_bias, dsum, h_end, workspace,
                          workspace_bytes, stream, true);
}

ss_status ss_scan_shard_combine(int64_t batch, int64_t dim, int dstate, int64_t nshards, const float* A,
                                const float* dsum, const float* h_end, const float* h0, float* h_in, float* h_final,
                                void* stream) {
  if (!valid_dstate(dstate)) return fail(SS_ERR_UNSUPPORTED, "dstate %d is not one of 1, 2, 4, 8, 16", dstate);
  if (batch < 1 || dim < 1 || nshards < 1)
    return fail(SS_ERR_INVALID_ARG, "sizes must be batch, dim, nshards >= 1 (got %lld, %lld, %lld)",
                (long long)batch, (long long)dim, (long long)nshards);
  if (batch > kMaxDim || dim > kMaxDim || nshards > kMaxDim) return fail(SS_ERR_INVALID_ARG, "a size exceeds 2^40");
  if ((__int128)nshards * batch * dim * dstate * 4 > ((__int128)1 << 62))
    return fail(SS_ERR_INVALID_ARG, "tensor sizes overflow 64-bit byte offsets");
  if (!A || !dsum || !h_end) return fail(SS_ERR_INVALID_ARG, "%s is NULL", !A ? "A" : (!dsum ? "dsum" : "h_end"));
  const void* a4[] = {A, dsum, h_end, h0, h_in, h_final};
  const char* n4[] = {"A", "dsum", "h_end", "h0", "h_in", "h_final"};
  for (int i = 0; i < 6; ++i)
    if (a4[i] && !aligned(a4[i], 4)) return fail(SS_ERR_INVALID_ARG, "%s is not 4-byte aligned", n4[i]);
  const int64_t st_bytes = batch * dim * dstate * 4;
  const Range ins[] = {rng("A", A, dim * dstate * 4), rng("dsum", dsum, nshards * batch * dim * 4),
                       rng("h_end", h_end, nshards * st_bytes), rng("h0", h0, st_bytes)};
  const Range outs[] = {rng("h_in", h_in, nshards * st_bytes), rng("h_final", h_final, st_bytes)};
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (overlap(o, i)) return fail(SS_ERR_INVALID_ARG, "%s overlaps input %s", o.name, i.name);
  if (overlap(outs[0], outs[1])) return fail(SS_ERR_INVALID_ARG, "h_in overlaps h_final");
  hipError_t e = ssscan::launch_shard_combine(batch, dim, dstate, nshards, A, dsum, h_end, h0, h_in, h_final,
                                              reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? SS_OK : hip_fail(e, "shard combine launch");
}

size_t ss_scan_bwd_workspace_bytes(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io) {
  return ss_scan_bwd_seg_workspace_bytes(batch, dim, dstate, seqlen, io, 0);
}

int64_t ss_scan_bwd_segment_len(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io) {
  if (check_sizes(batch, dim, dstate, seqlen, io) != SS_OK) return 0;
  const BwdSeg sg = bwd_auto_segments(batch, dim, dstate, seqlen);
  return sg.n > 1 ? sg.len : seqlen;
}

size_t ss_scan_bwd_seg_workspace_bytes(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io,
                                       int64_t segment_len) {
  if (check_sizes(batch, dim, dstate, seqlen, io) != SS_OK) return 0;
  if (seqlen == 0) return 0;
  BwdSeg sg;
  if (bwd_plan_segments(batch, dim, dstate, seqlen, segment_len, &sg) != SS_OK) return 0;
  return bwd_layout(batch, dim, dstate, seqlen, sg).total;
}

ss_status ss_scan_bwd(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io, const void* x,
                      const void* dt, const void* z, const void* B, const void* C, const float* A,
                      const float* Dskip, const float* dt_bias, const float* h0, const void* dy,
                      const float* dh_final, void* dx, void* ddt, void* dz, void* dB, void* dC, float* dA,
                      float* dDskip, float* ddt_bias, float* dh0, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return scan_bwd_impl(batch, dim, dstate, seqlen, io, x, dt, z, B, C, A, Dskip, dt_bias, h0, dy, dh_final, dx,
                       ddt, dz, dB, dC, dA, dDskip, ddt_bias, dh0, workspace, workspace_bytes, stream);
}

ss_status ss_scan_bwd_ex(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io, uint32_t flags,
                         const void* x, const void* dt, const void* z, const void* B, const void* C, const float* A,
                         const float* Dskip, const float* dt_bias, const float* h0, const void* dy,
                         const float* dh_final, const float* ckpt, void* dx, void* ddt, void* dz, void* dB, void* dC,
                         float* dA, float* dDskip, float* ddt_bias, float* dh0, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (flags & ~(uint32_t)(SS_FLAG_ZOH | SS_FLAG_DT_PER_ROW))
    return fail(SS_ERR_UNSUPPORTED, "unknown flags 0x%x", (unsigned)flags);
  return scan_bwd_impl(batch, dim, dstate, seqlen, io, x, dt, z, B, C, A, Dskip, dt_bias, h0, dy, dh_final, dx,
                       ddt, dz, dB, dC, dA, dDskip, ddt_bias, dh0, workspace, workspace_bytes, stream, ckpt,
                       (flags & SS_FLAG_DT_PER_ROW) != 0, (flags & SS_FLAG_ZOH) != 0);
}

ss_status ss_scan_bwd_seg(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io, uint32_t flags,
                          int64_t segment_len, const void* x, const void* dt, const void* z, const void* B,
                          const void* C, const float* A, const float* Dskip, const float* dt_bias, const float* h0,
                          const void* dy, const float* dh_final, const float* ckpt, void* dx, void* ddt, void* dz,
                          void* dB, void* dC, float* dA, float* dDskip, float* ddt_bias, float* dh0, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (flags & ~(uint32_t)(SS_FLAG_ZOH | SS_FLAG_DT_PER_ROW))
    return fail(SS_ERR_UNSUPPORTED, "unknown flags 0x%x", (unsigned)flags);
  return scan_bwd_impl(batch, dim, dstate, seqlen, io, x, dt, z, B, C, A, Dskip, dt_bias, h0, dy, dh_final, dx,
                       ddt, dz, dB, dC, dA, dDskip, ddt_bias, dh0, workspace, workspace_bytes, stream, ckpt,
                       (flags & SS_FLAG_DT_PER_ROW) != 0, (flags & SS_FLAG_ZOH) != 0, segment_len);
}

ss_status ss_timing_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.enabled = enable != 0;
  return SS_OK;
}

ss_status ss_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (auto& pr : g_timing.pending) {
    hipError_t e = hipEventSynchronize(pr.second);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    g_timing.pool.push_back(pr);
  }
  g_timing.pending.clear();
  g_timing.total_ms = 0.0;
  g_timing.calls = 0;
  return SS_OK;
}

ss_status ss_timing_read(double* total_ms, int64_t* calls) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (auto& pr : g_timing.pending) {
    hipError_t e = hipEventSynchronize(pr.second);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    g_timing.total_ms += ms;
    g_timing.calls += 1;
    g_timing.pool.push_back(pr);
  }
  g_timing.pending.clear();
  if (total_ms) *total_ms = g_timing.total_ms;
  if (calls) *calls = g_timing.calls;
  return SS_OK;
}

}  // extern "C"
