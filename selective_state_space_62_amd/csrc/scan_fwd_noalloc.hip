// ss_scan_fwd_noalloc: the forward scan (ss_scan_fwd_ex) for callers that cannot
// allocate device memory — code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc.  Its scratch space (on chunked plans, the
// chunk aggregates and entering states) is a static device array of this file
// instead of a caller-owned workspace.
//
// The array's name is a host-side stand-in in host code; its device address is
// looked up once per device with hipGetSymbolAddress (each GPU holds its own
// copy at its own address) and only that address is handed to the kernels.
// Nothing in the scratch needs to start at zero: every byte a call reads was
// written earlier in the same call.  Every call on one GPU shares that GPU's
// array, so calls that overlap in time on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"
#include "ssscan.h"

constexpr size_t kScratchBytes = SS_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up on the first call on that
// device (with that device current).
ss_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return ssscan::record_hip_error(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return ssscan::record_error(SS_ERR_UNSUPPORTED, "device %d is beyond the static scratch table (%d devices)", dev,
                                kMaxDevices);
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return ssscan::record_hip_error(e, "hipGetSymbolAddress(scratch)");
    if (!p) return ssscan::record_error(SS_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SS_OK;
}

}  // namespace

extern "C" {

size_t ss_scan_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

ss_status ss_scan_fwd_noalloc(int64_t batch, int64_t dim, int dstate, int64_t seqlen, ss_dtype io, uint32_t flags,
                              const void* x, const void* dt, const void* z, const void* B, const void* C,
                              const float* A, const float* Dskip, const float* dt_bias, const float* h0, void* y,
                              float* h_final, float* ckpt, const ss_scan_plan* plan, void* stream) {
  const size_t need = ss_scan_fwd_workspace_bytes(batch, dim, dstate, seqlen, io, plan);
  if (need == 0)   // invalid sizes or plan: the full call reports which, before any device work
    return ss_scan_fwd_ex(batch, dim, dstate, seqlen, io, flags, x, dt, z, B, C, A, Dskip, dt_bias, h0, y, h_final,
                          ckpt, nullptr, 0, plan, stream);
  if (need > kScratchBytes)
    return ssscan::record_error(SS_ERR_WORKSPACE,
                                "this call needs %zu bytes of scratch; the static array holds %zu "
                                "(use ss_scan_fwd_ex with a workspace)", need, kScratchBytes);
  void* ws = nullptr;
  const ss_status st = scratch_address(&ws);
  if (st != SS_OK) return st;
  return ss_scan_fwd_ex(batch, dim, dstate, seqlen, io, flags, x, dt, z, B, C, A, Dskip, dt_bias, h0, y, h_final,
                        ckpt, ws, kScratchBytes, plan, stream);
}

}  // extern "C"
