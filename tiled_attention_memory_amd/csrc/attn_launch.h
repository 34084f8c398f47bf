// Host-side launch entry points of the kernels, called by the C ABI after it
// has validated every argument. Internal to libattn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tam {

// Sq query rows against Sk keys; under a causal mask key j is visible to
// query row i when j <= i + dlt (dlt = query position - key position of the
// first rows, clamped to [-Sq, Sk]). The whole-sequence calls use Sq = Sk and
// dlt = 0.
struct AttnShape {
  int B, Hq, Hkv, Sq, Sk, D;
  bool causal;
  int dlt;
  float scale;
  // dropout on the probabilities: byte threshold t (probability t / 256; 0 =
  // none) and the generator seed
  int drop_t = 0;
  unsigned long long seed = 0;
  // rotary embedding: (cos, sin) table [S][D/2] in device memory; the forward
  // kernel rotates Q with it at load, the backward kernels rotate dQ and dK back
  const float2* rope = nullptr;
};

// Query-stationary kernels give each unit `rows` query rows. A shorter
// sequence would leave most of a unit empty, so 2^p query heads of one group
// (which read the same K and V) share it, each in rows >> p of its rows; the
// packing p (0, 1 or 2) is the largest whose heads still fit.
inline int head_pack(const AttnShape& sh, int rows) {
  const int group = sh.Hq / sh.Hkv;
  if (sh.Sq <= rows / 4 && group % 4 == 0) return 2;
  if (sh.Sq <= rows / 2 && group % 2 == 0) return 1;
  return 0;
}

constexpr int kMaxMerge = 16;  // partial results one merge call combines

// Exactly one of o (bf16) and o32 (fp32) is set.
hipError_t launch_fwd(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      uint16_t* o, float* o32, float* lse, hipStream_t stream);

hipError_t launch_merge(const float* const* o_parts, const float* const* lse_parts, int n, uint16_t* o,
                        float* lse, long long rows, int D, hipStream_t stream);
// Part b at o_base + b * o_stride and lse_base + b * lse_stride (any n >= 1).
hipError_t launch_merge_strided(const float* o_base, const float* lse_base, int n, long long o_stride,
                                long long lse_stride, uint16_t* o, float* lse, long long rows, int D,
                                hipStream_t stream);

// Decode: Sq new tokens of every query head against Sk cached keys, split
// over the keys; dlt = Sk - Sq places the tokens at the end of the cache.
struct DecodePlan {
  int splits, chunk;
};
DecodePlan decode_plan(const AttnShape& sh);
size_t decode_workspace_bytes(const AttnShape& sh);
// Rotary embedding (whole sequences, positions 0 .. S-1).
struct RopeLayout {
  size_t table, k_rot, q_rot, bwd, total;
};
RopeLayout rope_layout(const AttnShape& sh);
hipError_t launch_fwd_rope(AttnShape sh, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           float* lse, void* workspace, double base, hipStream_t stream);
hipError_t launch_bwd_rope(AttnShape sh, const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                           const uint16_t* dout, const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                           void* workspace, double base, hipStream_t stream);

hipError_t launch_decode(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                         float* lse, void* workspace, hipStream_t stream);

// Workspace layout of the backward pass (bytes, 256-aligned offsets).
size_t bwd_workspace_bytes(const AttnShape& sh);

hipError_t launch_bwd(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* o, const uint16_t* dout, const float* lse, uint16_t* dq,
                      uint16_t* dk, uint16_t* dv, void* workspace, hipStream_t stream,
                      hipEvent_t* events = nullptr);

// Whole-sequence backward of at most 64 tokens (no dropout, no rotation): one
// kernel forms dQ, dK and dV; with several head subsets it leaves fp32 dK/dV
// partials ([nsplit][2][B*Hkv*S*D] at `part`) for the fixed-order reduce.
bool bwd_short_path(const AttnShape& sh);
int bwd_short_split(const AttnShape& sh);
size_t bwd_short_workspace_bytes(const AttnShape& sh);
hipError_t launch_bwd_short(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const uint16_t* dout, const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                            float* part, hipStream_t stream);
// Fixed-order sum of ns fp32 partials [ns][2][B*Hkv*Sk*D] into bf16 dK, dV.
hipError_t launch_bwd_reduce(const AttnShape& sh, const float* part, int ns, uint16_t* dk, uint16_t* dv,
                             hipStream_t stream);

// Fixed device scratch of attn_bwd_noalloc (one copy per GPU, held until the
// process ends): its size, and the current device's address of it (looked up
// on the first call on that device).
constexpr size_t kNoallocScratchBytes = (size_t)256 << 20;
hipError_t noalloc_scratch(void** out);

// Block protocol of the backward pass (one query block, key blocks in turn).
// The need of one block call with sh.Sk keys, and the size that covers every
// call with a key block of at most sh.Sk keys.
size_t bwd_block_workspace_bytes(const AttnShape& sh);
size_t bwd_block_workspace_bytes_upto(const AttnShape& sh);
hipError_t launch_bwd_block_begin(const AttnShape& sh, const uint16_t* o, const uint16_t* dout, const float* lse,
                                  void* workspace, hipStream_t stream);
hipError_t launch_bwd_block_dq(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const uint16_t* dout, void* workspace, hipStream_t stream);
hipError_t launch_bwd_block_dq_end(const AttnShape& sh, uint16_t* dq, void* workspace, hipStream_t stream);
hipError_t launch_bwd_block_dkdv(const AttnShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const uint16_t* dout, uint16_t* dk, uint16_t* dv, void* workspace,
                                 hipStream_t stream);

}  // namespace tam
