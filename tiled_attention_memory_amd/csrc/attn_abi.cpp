// C ABI of libattn.so: argument validation, then dispatch to the kernels.
// The contract (layout, ownership, error behaviour) is stated in include/attn.h.
#include "attn.h"

#include <math.h>
#include <stdint.h>

#include <new>

#include "attn_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Shapes shared by both passes. Element counts must fit comfortably in 64 bits
// and the per-launch unit counts in a 32-bit grid.
int check_shape(int B, int Hq, int Hkv, int S, int D) {
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || S > ATTN_MAX_SEQ) return ATTN_ERR_BAD_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_BAD_SHAPE;
  const long long bh = (long long)B * Hq;
  if (bh > (1LL << 24)) return ATTN_ERR_BAD_SHAPE;
  // the largest tile grid: 8 * ceil(B*Hq/8) units per 64-row tile; the
  // row-parallel grids need B*Hq*S / 8 blocks at most
  const long long tiles = (S + 63) / 64;
  if ((bh + 8) * tiles > 0x7fffffffLL) return ATTN_ERR_BAD_SHAPE;
  if (bh * S > (1LL << 33)) return ATTN_ERR_BAD_SHAPE;
  return ATTN_OK;
}

int check_common(int B, int Hq, int Hkv, int S, int D, int causal, float scale) {
  const int st = check_shape(B, Hq, Hkv, S, D);
  if (st != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_BAD_FLAG;
  if (!isfinite(scale)) return ATTN_ERR_BAD_SCALE;
  return ATTN_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

}  // namespace

extern "C" {

#define ATTN_EXPORT __attribute__((visibility("default")))

ATTN_EXPORT int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
             int S, int D, int causal, float scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL_POINTER;
  int st = check_common(B, Hq, Hkv, S, D, causal, scale);
  if (st != ATTN_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_MISALIGNED;
  const size_t qb = (size_t)B * Hq * S * D * 2, kb = (size_t)B * Hkv * S * D * 2;
  const size_t lb = (size_t)B * Hq * S * 4;
  const Range rq = range_of(q, qb), rk = range_of(k, kb), rv = range_of(v, kb);
  const Range ro = range_of(o, qb), rl = range_of(lse, lb);
  if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) || overlap(rl, rq) || overlap(rl, rk) ||
      overlap(rl, rv) || overlap(ro, rl))
    return ATTN_ERR_ALIAS;
  try {
    const tam::AttnShape sh{B, Hq, Hkv, S, D, causal != 0, scale};
    return from_hip(tam::launch_fwd(sh, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                    static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse,
                                    stream));
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_EXPORT int attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D, size_t* bytes) {
  if (!bytes) return ATTN_ERR_NULL_POINTER;
  const int st = check_shape(B, Hq, Hkv, S, D);
  if (st != ATTN_OK) return st;
  const tam::AttnShape sh{B, Hq, Hkv, S, D, true, 1.f};
  *bytes = tam::bwd_workspace_bytes(sh);
  return ATTN_OK;
}

ATTN_EXPORT int attn_bwd_timed(const void* q, const void* k, const void* v, const void* o, const void* dout,
                               const float* lse, void* dq, void* dk, void* dv, void* workspace,
                               size_t workspace_bytes, int B, int Hq, int Hkv, int S, int D, int causal,
                               float scale, hipStream_t stream, hipEvent_t* events) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_ERR_NULL_POINTER;
  int st = check_common(B, Hq, Hkv, S, D, causal, scale);
  if (st != ATTN_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return ATTN_ERR_MISALIGNED;
  const tam::AttnShape sh{B, Hq, Hkv, S, D, causal != 0, scale};
  const size_t need = tam::bwd_workspace_bytes(sh);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_MISALIGNED;
  const size_t qb = (size_t)B * Hq * S * D * 2, kb = (size_t)B * Hkv * S * D * 2;
  const size_t lb = (size_t)B * Hq * S * 4;
  const Range ins[] = {range_of(q, qb), range_of(k, kb), range_of(v, kb), range_of(o, qb),
                       range_of(dout, qb), range_of(lse, lb)};
  const Range outs[] = {range_of(dq, qb), range_of(dk, kb), range_of(dv, kb), range_of(workspace, need)};
  for (int i = 0; i < 4; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return ATTN_ERR_ALIAS;
  }
  try {
    return from_hip(tam::launch_bwd(sh, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                    static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(o),
                                    static_cast<const uint16_t*>(dout), lse, static_cast<uint16_t*>(dq),
                                    static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), workspace,
                                    stream, events));
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_EXPORT int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, int B, int Hq, int Hkv, int S, int D, int causal,
                         float scale, hipStream_t stream) {
  return attn_bwd_timed(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, S, D,
                        causal, scale, stream, nullptr);
}

ATTN_EXPORT const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL_POINTER: return "a required pointer is NULL";
    case ATTN_ERR_BAD_SHAPE: return "B, Hq, Hkv or S out of range, or Hq not a multiple of Hkv";
    case ATTN_ERR_UNSUPPORTED_HEAD_DIM: return "head dimension D must be 64 or 128";
    case ATTN_ERR_BAD_SCALE: return "softmax scale must be finite";
    case ATTN_ERR_MISALIGNED: return "pointers must be 16-byte aligned";
    case ATTN_ERR_WORKSPACE: return "workspace missing or smaller than attn_bwd_workspace_bytes()";
    case ATTN_ERR_HIP: return "the HIP runtime reported an error while launching";
    case ATTN_ERR_BAD_FLAG: return "causal must be 0 or 1";
    case ATTN_ERR_ALIAS: return "an output overlaps an input or another output";
    default: return "unknown status";
  }
}

ATTN_EXPORT int attn_version(void) { return ATTN_VERSION; }

}  // extern "C"
