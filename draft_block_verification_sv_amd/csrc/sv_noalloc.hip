// sv_verify_block_noalloc: sv_verify_block with the library's own fixed scratch buffer in place
// of a caller workspace, for callers that cannot allocate device memory around the call (code
// under stream capture, tight serving loops, harnesses that forbid allocation).
//
// The scratch is a file-scope device array of kScratchBytes; every GPU the library runs on
// holds its own copy until the process ends.  Its device address on the current device is
// looked up once per device (hipGetSymbolAddress, with that device current) and used for every
// later call there: the array's name is a host-side stand-in in host code and is never passed
// to a kernel.  The verification kernels write every scratch byte they read within the call,
// except the arrival flags of rows split over several workgroups, which count only when
// they hold that launch's own nonzero epoch and are cleared by the part that finishes the
// row, so nothing has to start at zero.  All calls on one GPU share that GPU's array: calls that
// overlap on one GPU (two streams, or two host threads) race on it and must be serialised by
// the caller.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/specverify.h"

namespace {

constexpr size_t kScratchBytes = SV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_lookup[kMaxDevices];

// The scratch array's address on the current device.
hipError_t scratch_on_current_device(void** out) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_lookup[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = (g_lookup[dev] == hipSuccess) ? p : nullptr;
  });
  if (g_lookup[dev] != hipSuccess) return g_lookup[dev];
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" sv_status sv_verify_block_noalloc(
    int32_t dtype, int32_t B, int32_t k_max, int64_t V, int64_t ld_target, int64_t ld_draft,
    int64_t n_draft_rows, const void* target_logits, const void* draft_logits, const int32_t* k,
    const int32_t* draft_tokens, const float* uniforms, const float* temperature, float delta,
    int32_t* accept_len, int32_t* out_tokens, float* rkl_out, float* p_at_draft,
    float* q_at_draft, int32_t* device_status, void* stream) {
  // The host checks first, with no workspace: every problem but the missing workspace is
  // reported exactly as sv_verify_block reports it, before any HIP call.
  const sv_status pre = sv_verify_block(dtype, B, k_max, V, ld_target, ld_draft, n_draft_rows,
                                        target_logits, draft_logits, k, draft_tokens, uniforms,
                                        temperature, delta, accept_len, out_tokens, rkl_out,
                                        p_at_draft, q_at_draft, device_status, nullptr, 0, stream);
  if (pre != SV_ERR_WORKSPACE) return pre;
  void* ws = nullptr;
  if (scratch_on_current_device(&ws) != hipSuccess || ws == nullptr) return SV_ERR_HIP;
  const sv_status s = sv_verify_block(dtype, B, k_max, V, ld_target, ld_draft, n_draft_rows,
                                      target_logits, draft_logits, k, draft_tokens, uniforms,
                                      temperature, delta, accept_len, out_tokens, rkl_out,
                                      p_at_draft, q_at_draft, device_status, ws, kScratchBytes,
                                      stream);
  // every other check passed and the layout still does not fit the fixed buffer
  return s == SV_ERR_WORKSPACE ? SV_ERR_SCRATCH : s;
}
