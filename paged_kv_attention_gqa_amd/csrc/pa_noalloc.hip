// pa_attention_fwd_noalloc: the paged GQA forward for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops and
// harnesses that forbid hipMalloc).  The split partials that
// pa_attention_fwd keeps in a caller workspace live here in one file-scope
// device array of fixed size, which each GPU the library runs on holds until
// the process ends.  The kernels are those of pa_attention_fwd.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "paged_attn.h"
#include "pa_host.h"

namespace {
constexpr size_t kScratchBytes = size_t(32) << 20;  // PA_NOALLOC_SCRATCH_BYTES
constexpr int kMaxDevices = 64;
}  // namespace
static_assert(kScratchBytes == PA_NOALLOC_SCRATCH_BYTES, "header and library agree on the scratch size");

// In host code this name is a host-side stand-in for the array, not its
// device address: only the address that hipGetSymbolAddress returns for the
// current device may reach a kernel or a copy.
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

// Device address of `scratch` on each device, looked up once per device with
// that device current.
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

hipError_t scratch_on(int dev, void** ptr) {
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = g_ptr[dev];
  return g_err[dev];
}

}  // namespace

extern "C" int pa_attention_fwd_noalloc(const pa_plan* plan, int32_t dtype, const void* q, const void* k_pool,
                                        const void* v_pool, void* out, float* lse, int32_t head_dim,
                                        int32_t v_head_dim, float scale, void* stream) {
  if (!plan) return pa::host_fail(PA_ERR_INVALID, "plan is NULL");
  size_t need = 0;
  int rc = pa_plan_workspace_bytes(plan, v_head_dim, &need);
  if (rc != PA_OK) return rc;
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "plan needs %zu bytes of split partials; the no-allocation forward holds %zu "
             "(pass a workspace to pa_attention_fwd, or plan fewer splits)",
             need, kScratchBytes);
    return pa::host_fail(PA_ERR_WORKSPACE, msg);
  }
  if (need == 0)  // no split row: no partials, nothing of the array is used
    return pa_attention_fwd(plan, dtype, q, k_pool, v_pool, out, lse, head_dim, v_head_dim, scale, nullptr, 0,
                            nullptr, stream);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pa::host_fail(PA_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return pa::host_fail(PA_ERR_DEVICE, "device index beyond this library's table");
  void* ws = nullptr;
  e = scratch_on(dev, &ws);
  if (e != hipSuccess || !ws) return pa::host_fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) failed");
  // every partial slot the plan's merge reads is written by exactly one
  // piece of the same call, so nothing needs clearing between calls
  return pa_attention_fwd(plan, dtype, q, k_pool, v_pool, out, lse, head_dim, v_head_dim, scale, ws,
                          kScratchBytes, nullptr, stream);
}
