// sv_verify_window without a workspace argument, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The workspace lives in a file-scope
// device array of fixed size; each GPU the library runs on holds its own copy
// until the process ends.  Nothing here allocates.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sv.h"

// Workspace of every sv_verify_window_noalloc call on one GPU.  In host code
// the name stands for a host-side shadow, not a device address: only its
// address from hipGetSymbolAddress is passed on.
static __device__ __align__(256) unsigned char scratch[SV_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};  // device address of `scratch`, per device

// Device address of the current device's scratch array, looked up once per
// device (with that device current); nullptr if the lookup fails.
void *scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int sv_verify_window_noalloc(const void *target_logits, int64_t target_seq_stride,
                                        const void *draft_logits, int64_t draft_seq_stride, int dtype,
                                        const int32_t *draft_tokens, const int32_t *window_len,
                                        int32_t B, int32_t gamma, int32_t V,
                                        uint64_t seed, uint64_t tag, const uint64_t *seq_ids,
                                        const int64_t *base_pos,
                                        int32_t *n_accepted, int32_t *out_tokens,
                                        float *p_draft, float *q_draft, hipStream_t stream) {
  // Argument errors come first, whatever the state of the device: the
  // workspace call checks every argument before its workspace, so without one
  // it reports either an argument error or only the missing workspace, and
  // enqueues nothing either way.
  const int args = sv_verify_window(target_logits, target_seq_stride, draft_logits, draft_seq_stride, dtype,
                                    draft_tokens, window_len, B, gamma, V, seed, tag, seq_ids, base_pos, n_accepted,
                                    out_tokens, p_draft, q_draft, nullptr, 0, stream);
  if (args != SV_EWORKSPACE) return args;
  if (sv_workspace_size(SV_OP_WINDOW, B, gamma, V, dtype) > SV_SCRATCH_BYTES) return SV_ESCRATCH;
  void *ws = scratch_ptr();
  if (!ws) return SV_ELAUNCH;
  return sv_verify_window(target_logits, target_seq_stride, draft_logits, draft_seq_stride, dtype, draft_tokens,
                          window_len, B, gamma, V, seed, tag, seq_ids, base_pos, n_accepted, out_tokens, p_draft,
                          q_draft, ws, SV_SCRATCH_BYTES, stream);
}
