// The fused dispatch+combine for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the dispatch layout's workspace (error word and per-tile count
// table) lives in a file-scope device array of the library instead of a
// caller buffer.  The caller still passes every input and output.
//
// The array is a host-side stand-in in host code: its device address is
// looked up once per device with hipGetSymbolAddress (that device current)
// and only that address is ever handed to a kernel.  Each GPU holds its own
// copy until the process ends.  Every call on a GPU shares that GPU's copy,
// so calls that overlap on one GPU (concurrent streams, or threads) race.
#include <mutex>

#include "moe_internal.h"

static __device__ __align__(256) unsigned char scratch[MOE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
void *g_scratch[kMaxDevices];  // device address of `scratch`, per device
std::mutex g_scratch_mu;

int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return MOE_ELAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return MOE_ELAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_dispatch_combine_noalloc(
    const moe_cfg *cfg, const void *x, const float *logits,
    const float *expert_scale, int32_t *topk_idx, float *topk_w,
    const moe_layout *layout, void *send, void *out, hipStream_t stream) {
  int rc = moe::check_fused(cfg, x, logits, topk_idx, topk_w, layout, send,
                            out);
  if (rc != MOE_OK) return rc;
  if (moe::layout_geom(*cfg).ws_bytes > (size_t)MOE_SCRATCH_BYTES)
    return MOE_ESCRATCH;
  void *ws = nullptr;
  if ((rc = scratch_address(&ws)) != MOE_OK) return rc;
  // The error word starts at zero on every call (a fill kernel, which graph
  // capture records as a kernel node); the count table needs no clearing,
  // since the layout writes every entry it later reads.
  hipError_t e = moe::launch_fill_u32((uint32_t *)ws, 0u,
                                      moe::kWsHeader / 4, stream);
  if (e == hipSuccess)
    e = moe::launch_fused(*cfg, x, logits, expert_scale, topk_idx, topk_w,
                          *layout, send, out, ws, stream);
  return e == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}
