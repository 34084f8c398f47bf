// C ABI of libattn.so: argument validation, then dispatch to the kernels.
// The contract (layout, ownership, error behaviour) is stated in include/attn.h
// include/attn_block.h, include/attn_decode.h, include/attn_dropout.h and
// include/attn_rope.h.
#include "attn.h"
#include "attn_block.h"
#include "attn_decode.h"
#include "attn_dropout.h"
#include "attn_rope.h"

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

// Shapes shared by every call. Element counts must fit comfortably in 64 bits
// and the per-launch unit counts in a 32-bit grid. Sq query rows, Sk keys.
int check_shape(int B, int Hq, int Hkv, int Sq, int Sk, int D) {
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED_HEAD_DIM;
  if (B < 1 || Hq < 1 || Hkv < 1) return ATTN_ERR_BAD_SHAPE;
  if (Sq < 1 || Sq > ATTN_MAX_SEQ || Sk < 1 || Sk > ATTN_MAX_SEQ) return ATTN_ERR_BAD_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_BAD_SHAPE;
  const long long bh = (long long)B * Hq;
  if (bh > (1LL << 24)) return ATTN_ERR_BAD_SHAPE;
  // the largest tile grid: 8 * ceil(B*Hq/8) units per 64-row tile; the
  // row-parallel grids need B*Hq*S / 8 blocks at most
  const long long s = Sq > Sk ? Sq : Sk;
  const long long tiles = (s + 63) / 64;
  if ((bh + 8) * tiles > 0x7fffffffLL) return ATTN_ERR_BAD_SHAPE;
  if (bh * s > (1LL << 33)) return ATTN_ERR_BAD_SHAPE;
  return ATTN_OK;
}

int check_common(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale) {
  const int st = check_shape(B, Hq, Hkv, Sq, Sk, D);
  if (st != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_BAD_FLAG;
  if (!isfinite(scale)) return ATTN_ERR_BAD_SCALE;
  return ATTN_OK;
}

// Block positions: any values up to 2^62 in magnitude; only their difference
// matters, and beyond [-Sq, Sk] every row sees all keys or none, so it is
// clamped to that range.
int check_positions(long long q_pos0, long long k_pos0) {
  const long long lim = 1LL << 62;
  if (q_pos0 > lim || q_pos0 < -lim || k_pos0 > lim || k_pos0 < -lim) return ATTN_ERR_BAD_SHAPE;
  return ATTN_OK;
}

tam::AttnShape block_shape(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, long long q_pos0,
                           long long k_pos0, float scale) {
  long long d = q_pos0 - k_pos0;
  if (d < -(long long)Sq) d = -(long long)Sq;
  if (d > (long long)Sk) d = Sk;
  return tam::AttnShape{B, Hq, Hkv, Sq, Sk, D, causal != 0, (int)d, scale};
}

tam::AttnShape square_shape(int B, int Hq, int Hkv, int S, int D, int causal, float scale) {
  return tam::AttnShape{B, Hq, Hkv, S, S, D, causal != 0, 0, scale};
}

int from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// decode against a key/value cache (attn_decode.h)
int check_decode(int B, int Hq, int Hkv, int Sq, int Sk, int D) {
  int st = check_shape(B, Hq, Hkv, Sq, Sk, D);
  if (st != ATTN_OK) return st;
  if (Sq > Sk || (long long)(Hq / Hkv) * Sq > 128) return ATTN_ERR_BAD_SHAPE;
  return ATTN_OK;
}
tam::AttnShape decode_shape(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale) {
  return tam::AttnShape{B, Hq, Hkv, Sq, Sk, D, causal != 0, Sk - Sq, scale};
}

}  // namespace

extern "C" {

#define ATTN_EXPORT __attribute__((visibility("default")))

namespace {
// Dropout threshold of probability p (see attn_dropout.h), or -1 when p is out of range.
int drop_threshold(float p) {
  if (!isfinite(p) || p < 0.f) return -1;
  const double t = floor(256.0 * (double)p + 0.5);
  return t > 255.0 ? -1 : (int)t;
}

int fwd_common(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int S, int D,
               int causal, float scale, int drop_t, unsigned long long seed, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL_POINTER;
  int st = check_common(B, Hq, Hkv, S, S, D, causal, scale);
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
    tam::AttnShape sh = square_shape(B, Hq, Hkv, S, D, causal, scale);
    sh.drop_t = drop_t;
    sh.seed = seed;
    return from_hip(tam::launch_fwd(sh, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                    static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), nullptr, lse,
                                    stream));
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}
}  // namespace

ATTN_EXPORT int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
             int S, int D, int causal, float scale, hipStream_t stream) {
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, S, D, causal, scale, 0, 0, stream);
}

ATTN_EXPORT int attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                                 int Hkv, int S, int D, int causal, float scale, float p, unsigned long long seed,
                                 hipStream_t stream) {
  const int t = drop_threshold(p);
  if (t < 0) return ATTN_ERR_BAD_SCALE;
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, S, D, causal, scale, t, seed, stream);
}

ATTN_EXPORT int attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D, size_t* bytes) {
  if (!bytes) return ATTN_ERR_NULL_POINTER;
  const int st = check_shape(B, Hq, Hkv, S, S, D);
  if (st != ATTN_OK) return st;
  *bytes = tam::bwd_workspace_bytes(square_shape(B, Hq, Hkv, S, D, 1, 1.f));
  return ATTN_OK;
}

namespace {
// noalloc: no caller workspace; the library's fixed scratch stands in for it
// (attn_bwd_noalloc), and sizes that need more are rejected.
int bwd_common(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq,
               void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int S, int D,
               int causal, float scale, int drop_t, unsigned long long seed, hipStream_t stream,
               hipEvent_t* events, bool noalloc = false) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_ERR_NULL_POINTER;
  int st = check_common(B, Hq, Hkv, S, S, D, causal, scale);
  if (st != ATTN_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return ATTN_ERR_MISALIGNED;
  tam::AttnShape sh = square_shape(B, Hq, Hkv, S, D, causal, scale);
  sh.drop_t = drop_t;
  sh.seed = seed;
  const size_t need = tam::bwd_workspace_bytes(sh);
  if (noalloc) {
    if (need > tam::kNoallocScratchBytes) return ATTN_ERR_SCRATCH_LIMIT;
  } else {
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_ERR_MISALIGNED;
  }
  const size_t qb = (size_t)B * Hq * S * D * 2, kb = (size_t)B * Hkv * S * D * 2;
  const size_t lb = (size_t)B * Hq * S * 4;
  const Range ins[] = {range_of(q, qb), range_of(k, kb), range_of(v, kb), range_of(o, qb),
                       range_of(dout, qb), range_of(lse, lb)};
  // the scratch is the library's own memory: no caller buffer can overlap it
  const int n_outs = noalloc ? 3 : 4;
  const Range outs[] = {range_of(dq, qb), range_of(dk, kb), range_of(dv, kb), range_of(workspace, need)};
  for (int i = 0; i < n_outs; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < n_outs; ++j)
      if (overlap(outs[i], outs[j])) return ATTN_ERR_ALIAS;
  }
  if (noalloc && tam::noalloc_scratch(&workspace) != hipSuccess) return ATTN_ERR_HIP;
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

}  // namespace

ATTN_EXPORT int attn_bwd_timed(const void* q, const void* k, const void* v, const void* o, const void* dout,
                               const float* lse, void* dq, void* dk, void* dv, void* workspace,
                               size_t workspace_bytes, int B, int Hq, int Hkv, int S, int D, int causal,
                               float scale, hipStream_t stream, hipEvent_t* events) {
  return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, S, D, causal, scale,
                    0, 0, stream, events);
}

ATTN_EXPORT int attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                 const float* lse, void* dq, void* dk, void* dv, void* workspace,
                                 size_t workspace_bytes, int B, int Hq, int Hkv, int S, int D, int causal,
                                 float scale, float p, unsigned long long seed, hipStream_t stream) {
  const int t = drop_threshold(p);
  if (t < 0) return ATTN_ERR_BAD_SCALE;
  return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, S, D, causal, scale,
                    t, seed, stream, nullptr);
}

ATTN_EXPORT int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, int B, int Hq, int Hkv, int S, int D, int causal,
                         float scale, hipStream_t stream) {
  return attn_bwd_timed(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, S, D,
                        causal, scale, stream, nullptr);
}

ATTN_EXPORT int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                 const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int S,
                                 int D, int causal, float scale, hipStream_t stream) {
  return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, nullptr, 0, B, Hq, Hkv, S, D, causal, scale, 0, 0, stream,
                    nullptr, true);
}

// ---------------------------------------------------------------------------
// context-parallel building block (attn_block.h)
// ---------------------------------------------------------------------------
ATTN_EXPORT int attn_fwd_block(const void* q, const void* k, const void* v, float* o_part, float* lse_part, int B,
                               int Hq, int Hkv, int Sq, int Sk, int D, int causal, long long q_pos0,
                               long long k_pos0, float scale, hipStream_t stream) {
  if (!q || !k || !v || !o_part || !lse_part) return ATTN_ERR_NULL_POINTER;
  int st = check_common(B, Hq, Hkv, Sq, Sk, D, causal, scale);
  if (st == ATTN_OK) st = check_positions(q_pos0, k_pos0);
  if (st != ATTN_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_part) || !aligned16(lse_part))
    return ATTN_ERR_MISALIGNED;
  const size_t qb = (size_t)B * Hq * Sq * D * 2, kb = (size_t)B * Hkv * Sk * D * 2;
  const size_t ob = (size_t)B * Hq * Sq * D * 4, lb = (size_t)B * Hq * Sq * 4;
  const Range ins[] = {range_of(q, qb), range_of(k, kb), range_of(v, kb)};
  const Range ro = range_of(o_part, ob), rl = range_of(lse_part, lb);
  for (const Range& r : ins)
    if (overlap(ro, r) || overlap(rl, r)) return ATTN_ERR_ALIAS;
  if (overlap(ro, rl)) return ATTN_ERR_ALIAS;
  try {
    const tam::AttnShape sh = block_shape(B, Hq, Hkv, Sq, Sk, D, causal, q_pos0, k_pos0, scale);
    return from_hip(tam::launch_fwd(sh, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                    static_cast<const uint16_t*>(v), nullptr, o_part, lse_part, stream));
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_EXPORT int attn_merge(const float* const* o_parts, const float* const* lse_parts, int n, void* o, float* lse,
                           int B, int Hq, int Sq, int D, hipStream_t stream) {
  if (!o_parts || !lse_parts || !o || !lse) return ATTN_ERR_NULL_POINTER;
  if (n < 1 || n > ATTN_MAX_MERGE) return ATTN_ERR_BAD_SHAPE;
  int st = check_shape(B, Hq, 1, Sq, Sq, D);
  if (st != ATTN_OK) return st;
  const long long rows = (long long)B * Hq * Sq;
  const Range ro = range_of(o, (size_t)rows * D * 2), rl = range_of(lse, (size_t)rows * 4);
  if (overlap(ro, rl)) return ATTN_ERR_ALIAS;
  if (!aligned16(o) || !aligned16(lse)) return ATTN_ERR_MISALIGNED;
  for (int i = 0; i < n; ++i) {
    if (!o_parts[i] || !lse_parts[i]) return ATTN_ERR_NULL_POINTER;
    if (!aligned16(o_parts[i]) || !aligned16(lse_parts[i])) return ATTN_ERR_MISALIGNED;
    const Range a = range_of(o_parts[i], (size_t)rows * D * 4), b = range_of(lse_parts[i], (size_t)rows * 4);
    if (overlap(ro, a) || overlap(ro, b) || overlap(rl, a) || overlap(rl, b)) return ATTN_ERR_ALIAS;
  }
  try {
    return from_hip(tam::launch_merge(o_parts, lse_parts, n, static_cast<uint16_t*>(o), lse, rows, D, stream));
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_EXPORT int attn_bwd_block_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D, size_t* bytes) {
  if (!bytes) return ATTN_ERR_NULL_POINTER;
  const int st = check_shape(B, Hq, Hkv, Sq, Sk, D);
  if (st != ATTN_OK) return st;
  *bytes = tam::bwd_block_workspace_bytes_upto(block_shape(B, Hq, Hkv, Sq, Sk, D, 1, 0, 0, 1.f));
  return ATTN_OK;
}

namespace {
// Workspace check shared by the block backward calls.
int check_block_ws(const tam::AttnShape& sh, const void* ws, size_t ws_bytes, size_t* need) {
  *need = tam::bwd_block_workspace_bytes(sh);
  if (!ws || ws_bytes < *need) return ATTN_ERR_WORKSPACE;
  if (!aligned16(ws)) return ATTN_ERR_MISALIGNED;
  return ATTN_OK;
}
}  // namespace

ATTN_EXPORT int attn_bwd_block_begin(const void* o, const void* dout, const float* lse, void* workspace,
                                     size_t workspace_bytes, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                     hipStream_t stream) {
  if (!o || !dout || !lse) return ATTN_ERR_NULL_POINTER;
  int st = check_shape(B, Hq, Hkv, Sq, Sk, D);
  if (st != ATTN_OK) return st;
  if (!aligned16(o) || !aligned16(dout) || !aligned16(lse)) return ATTN_ERR_MISALIGNED;
  const tam::AttnShape sh = block_shape(B, Hq, Hkv, Sq, Sk, D, 1, 0, 0, 1.f);
  size_t need;
  if ((st = check_block_ws(sh, workspace, workspace_bytes, &need)) != ATTN_OK) return st;
  const size_t qb = (size_t)B * Hq * Sq * D * 2, lb = (size_t)B * Hq * Sq * 4;
  const Range w = range_of(workspace, need);
  if (overlap(w, range_of(o, qb)) || overlap(w, range_of(dout, qb)) || overlap(w, range_of(lse, lb)))
    return ATTN_ERR_ALIAS;
  try {
    return from_hip(tam::launch_bwd_block_begin(sh, static_cast<const uint16_t*>(o),
                                                static_cast<const uint16_t*>(dout), lse, workspace, stream));
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_EXPORT int attn_bwd_block_dq(const void* q, const void* k, const void* v, const void* dout, void* workspace,
                                  size_t workspace_bytes, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                  int causal, long long q_pos0, long long k_pos0, float scale,
                                  hipStream_t stream) {
  if (!q || !k || !v || !dout) return ATTN_ERR_NULL_POINTER;
  int st = check_common(B, Hq, Hkv, Sq, Sk, D, causal, scale);
  if (st == ATTN_OK) st = check_positions(q_pos0, k_pos0);
  if (st != ATTN_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout)) return ATTN_ERR_MISALIGNED;
  const tam::AttnShape sh = block_shape(B, Hq, Hkv, Sq, Sk, D, causal, q_pos0, k_pos0, scale);
  size_t need;
  if ((st = check_block_ws(sh, workspace, workspace_bytes, &need)) != ATTN_OK) return st;
  const size_t qb = (size_t)B * Hq * Sq * D * 2, kb = (size_t)B * Hkv * Sk * D * 2;
  const Range w = range_of(workspace, need);
  if (overlap(w, range_of(q, qb)) || overlap(w, range_of(k, kb)) || overlap(w, range_of(v, kb)) ||
      overlap(w, range_of(dout, qb)))
    return ATTN_ERR_ALIAS;
  try {
    return from_hip(tam::launch_bwd_block_dq(sh, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                             static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout),
                                             workspace, stream));
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_EXPORT int attn_bwd_block_dq_end(void* dq, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                                      int Sq, int Sk, int D, float scale, hipStream_t stream) {
  if (!dq) return ATTN_ERR_NULL_POINTER;
  int st = check_common(B, Hq, Hkv, Sq, Sk, D, 1, scale);
  if (st != ATTN_OK) return st;
  if (!aligned16(dq)) return ATTN_ERR_MISALIGNED;
  const tam::AttnShape sh = block_shape(B, Hq, Hkv, Sq, Sk, D, 1, 0, 0, scale);
  size_t need;
  if ((st = check_block_ws(sh, workspace, workspace_bytes, &need)) != ATTN_OK) return st;
  if (overlap(range_of(workspace, need), range_of(dq, (size_t)B * Hq * Sq * D * 2))) return ATTN_ERR_ALIAS;
  try {
    return from_hip(tam::launch_bwd_block_dq_end(sh, static_cast<uint16_t*>(dq), workspace, stream));
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_EXPORT int attn_bwd_block_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk,
                                    void* dv, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                                    int Sq, int Sk, int D, int causal, long long q_pos0, long long k_pos0,
                                    float scale, hipStream_t stream) {
  if (!q || !k || !v || !dout || !dk || !dv) return ATTN_ERR_NULL_POINTER;
  int st = check_common(B, Hq, Hkv, Sq, Sk, D, causal, scale);
  if (st == ATTN_OK) st = check_positions(q_pos0, k_pos0);
  if (st != ATTN_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dk) || !aligned16(dv))
    return ATTN_ERR_MISALIGNED;
  const tam::AttnShape sh = block_shape(B, Hq, Hkv, Sq, Sk, D, causal, q_pos0, k_pos0, scale);
  size_t need;
  if ((st = check_block_ws(sh, workspace, workspace_bytes, &need)) != ATTN_OK) return st;
  const size_t qb = (size_t)B * Hq * Sq * D * 2, kb = (size_t)B * Hkv * Sk * D * 2;
  const Range ins[] = {range_of(q, qb), range_of(k, kb), range_of(v, kb), range_of(dout, qb)};
  const Range outs[] = {range_of(dk, kb), range_of(dv, kb), range_of(workspace, need)};
  for (int i = 0; i < 3; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return ATTN_ERR_ALIAS;
  }
  try {
    return from_hip(tam::launch_bwd_block_dkdv(sh, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                               static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout),
                                               static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), workspace,
                                               stream));
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

// ---------------------------------------------------------------------------
// decode against a key/value cache (attn_decode.h)
// ---------------------------------------------------------------------------

ATTN_EXPORT int attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D, size_t* bytes) {
  if (!bytes) return ATTN_ERR_NULL_POINTER;
  const int st = check_decode(B, Hq, Hkv, Sq, Sk, D);
  if (st != ATTN_OK) return st;
  *bytes = tam::decode_workspace_bytes(decode_shape(B, Hq, Hkv, Sq, Sk, D, 1, 1.f));
  return ATTN_OK;
}

ATTN_EXPORT int attn_decode(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                            size_t workspace_bytes, int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal,
                            float scale, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL_POINTER;
  int st = check_decode(B, Hq, Hkv, Sq, Sk, D);
  if (st != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_BAD_FLAG;
  if (!isfinite(scale)) return ATTN_ERR_BAD_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_MISALIGNED;
  const tam::AttnShape sh = decode_shape(B, Hq, Hkv, Sq, Sk, D, causal, scale);
  const size_t need = tam::decode_workspace_bytes(sh);
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_MISALIGNED;
  const size_t qb = (size_t)B * Hq * Sq * D * 2, kb = (size_t)B * Hkv * Sk * D * 2, lb = (size_t)B * Hq * Sq * 4;
  const Range ins[] = {range_of(q, qb), range_of(k, kb), range_of(v, kb)};
  const Range outs[] = {range_of(o, qb), range_of(lse, lb), range_of(workspace, need)};
  for (int i = 0; i < 3; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return ATTN_ERR_ALIAS;
  }
  try {
    return from_hip(tam::launch_decode(sh, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, workspace,
                                       stream));
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

// ---------------------------------------------------------------------------
// rotary position embedding (attn_rope.h)
// ---------------------------------------------------------------------------
ATTN_EXPORT int attn_rope_workspace_bytes(int B, int Hq, int Hkv, int S, int D, size_t* bytes) {
  if (!bytes) return ATTN_ERR_NULL_POINTER;
  const int st = check_shape(B, Hq, Hkv, S, S, D);
  if (st != ATTN_OK) return st;
  *bytes = tam::rope_layout(square_shape(B, Hq, Hkv, S, D, 1, 1.f)).total;
  return ATTN_OK;
}

ATTN_EXPORT int attn_fwd_rope(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                              size_t workspace_bytes, int B, int Hq, int Hkv, int S, int D, int causal, float scale,
                              float base, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL_POINTER;
  int st = check_common(B, Hq, Hkv, S, S, D, causal, scale);
  if (st != ATTN_OK) return st;
  if (!isfinite(base) || !(base > 0.f)) return ATTN_ERR_BAD_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_MISALIGNED;
  const tam::AttnShape sh = square_shape(B, Hq, Hkv, S, D, causal, scale);
  const size_t need = tam::rope_layout(sh).total;
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_MISALIGNED;
  const size_t qb = (size_t)B * Hq * S * D * 2, kb = (size_t)B * Hkv * S * D * 2, lb = (size_t)B * Hq * S * 4;
  const Range ins[] = {range_of(q, qb), range_of(k, kb), range_of(v, kb)};
  const Range outs[] = {range_of(o, qb), range_of(lse, lb), range_of(workspace, need)};
  for (int i = 0; i < 3; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return ATTN_ERR_ALIAS;
  }
  try {
    return from_hip(tam::launch_fwd_rope(sh, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                         static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, workspace,
                                         (double)base, stream));
  } catch (...) {
    return ATTN_ERR_HIP;
  }
}

ATTN_EXPORT int attn_bwd_rope(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                              int B, int Hq, int Hkv, int S, int D, int causal, float scale, float base,
                              hipStream_t stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_ERR_NULL_POINTER;
  int st = check_common(B, Hq, Hkv, S, S, D, causal, scale);
  if (st != ATTN_OK) return st;
  if (!isfinite(base) || !(base > 0.f)) return ATTN_ERR_BAD_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return ATTN_ERR_MISALIGNED;
  const tam::AttnShape sh = square_shape(B, Hq, Hkv, S, D, causal, scale);
  const size_t need = tam::rope_layout(sh).total;
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_MISALIGNED;
  const size_t qb = (size_t)B * Hq * S * D * 2, kb = (size_t)B * Hkv * S * D * 2, lb = (size_t)B * Hq * S * 4;
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
    return from_hip(tam::launch_bwd_rope(sh, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                         static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(o),
                                         static_cast<const uint16_t*>(dout), lse, static_cast<uint16_t*>(dq),
                                         static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), workspace,
                                         (double)base, stream));
  } catch (...) {
    return ATTN_ERR_HIP;
  }
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
    case ATTN_ERR_SCRATCH_LIMIT:
      return "these sizes need more backward workspace than the fixed scratch of attn_bwd_noalloc "
             "(ATTN_NOALLOC_SCRATCH_BYTES); use attn_bwd with a caller workspace";
    default: return "unknown status";
  }
}

ATTN_EXPORT int attn_version(void) { return ATTN_VERSION; }

}  // extern "C"
