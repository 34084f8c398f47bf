// Host-side launch entry points of the kernels, called by the C ABI after it
// has validated every argument. Internal to libattn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tam {

struct AttnShape {
  int B, Hq, Hkv, S, D;
  bool causal;
  float scale;
};

hipError_t launch_fwd(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      uint16_t* o, float* lse, hipStream_t stream);

// Workspace layout of the backward pass (bytes, 256-aligned offsets).
size_t bwd_workspace_bytes(const AttnShape& sh);

hipError_t launch_bwd(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* o, const uint16_t* dout, const float* lse, uint16_t* dq,
                      uint16_t* dk, uint16_t* dv, void* workspace, hipStream_t stream,
                      hipEvent_t* events = nullptr);

}  // namespace tam
