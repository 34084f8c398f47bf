// Merge of partial attention results over disjoint key blocks, for gfx950.
//
// The page "使用 PyTorch FSDP 微調 Llama 2 70B" (agentlenshq.com), section
// "Flash Attention", combines score tiles with an online softmax; a sequence
// split across GPUs (context parallelism, run on the AMD MI300X pages at 32k
// and 128k tokens) combines whole key blocks the same way. Each block b gives a
// partial output O_b (normalised over its own keys) and its log-sum-exp LSE_b;
// the result over all blocks is
//   LSE = ln sum_b exp(LSE_b),   O = sum_b exp(LSE_b - LSE) O_b,
// with parts whose LSE is -inf (rows that saw no key of that block) weighing 0
// and a row that no block reaches left at O = 0, LSE = -inf.
//
// One pass over the parts, fp32 throughout, bf16 output: HBM-bound.
#include <math.h>

#include "attn_device.h"
#include "attn_launch.h"

namespace tam {
namespace {

constexpr int kThreads = 256;

struct MergeArgs {
  const float* o[kMaxMerge];     // part pointers, or
  const float* lse[kMaxMerge];
  const float* o_base;           // (when set) part b at o_base + b * o_stride
  const float* lse_base;
  long long o_stride, lse_stride;
  int n;
  uint16_t* out;
  float* lse_out;
  long long rows;
};

// Each row is handled by SG groups of D / 8 lanes, one wave or less: lane
// group q takes parts q, q + SG, ... and the groups' maxima and weighted sums
// are combined across lanes, so that rows with many parts (decode splits) do
// not walk them one after another.
constexpr int SG = 4;

template <int D>
__global__ __launch_bounds__(kThreads) void attn_merge_kernel(MergeArgs a) {
  constexpr int TPR = D / 8;         // lanes per group, 8 elements each
  constexpr int LPR = TPR * SG;      // lanes per row
  constexpr int RPB = kThreads / LPR;
  static_assert(LPR <= 64, "a row stays within one wave");
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % TPR;
  const int grp = (threadIdx.x / TPR) % SG;
  if (row >= a.rows) return;         // whole rows, so whole lane groups, leave together
  // One pass with a running max: each lane group folds its parts into
  // (m, tot, acc) relative to its largest LSE so far, loading four parts at a
  // time before folding any of them, so that their loads are in flight together.
  constexpr int U = 4;
  float m = -INFINITY, tot = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  auto fold = [&](auto lse_at, auto o_at) __attribute__((always_inline)) {
    for (int b0 = grp; b0 < a.n; b0 += U * SG) {
      float l[U];
      f32x4 o0[U], o1[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int b = b0 + u * SG;
        const int bl = b < a.n ? b : b0;  // past the last part: reload the first, weighed 0
        const f32x4* src = o_at(bl);
        l[u] = b < a.n ? lse_at(bl) : -INFINITY;
        o0[u] = src[0];
        o1[u] = src[1];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // a part with LSE = -inf weighs 0, whatever its output holds
        const bool use = l[u] != -INFINITY;
        const float mn = use ? fmaxf(m, l[u]) : m;
        const float r = use ? expf(m - mn) : 1.f;  // 0 while nothing has been folded in (m = -inf)
        const float w = use ? expf(l[u] - mn) : 0.f;
        tot = tot * r + w;
        acc0 = use ? acc0 * r + w * o0[u] : acc0;
        acc1 = use ? acc1 * r + w * o1[u] : acc1;
        m = mn;
      }
    }
  };
  if (a.o_base)
    fold([&](int b) { return a.lse_base[b * a.lse_stride + row]; },
         [&](int b) { return reinterpret_cast<const f32x4*>(a.o_base + b * a.o_stride + row * D + part * 8); });
  else
    fold([&](int b) { return a.lse[b][row]; },
         [&](int b) { return reinterpret_cast<const f32x4*>(a.o[b] + row * D + part * 8); });
  // combine the row's lane groups
#pragma unroll
  for (int x = TPR; x < LPR; x <<= 1) {
    const float mo = __shfl_xor(m, x), to = __shfl_xor(tot, x);
    f32x4 b0, b1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b0[i] = __shfl_xor(acc0[i], x);
      b1[i] = __shfl_xor(acc1[i], x);
    }
    const float mn = fmaxf(m, mo);
    const float r = m == -INFINITY ? 0.f : expf(m - mn);
    const float ro = mo == -INFINITY ? 0.f : expf(mo - mn);
    tot = tot * r + to * ro;
    acc0 = acc0 * r + b0 * ro;
    acc1 = acc1 * r + b1 * ro;
    m = mn;
  }
  if (grp != 0) return;
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  u32x4 w = {pack_bf16(acc0[0] * inv, acc0[1] * inv), pack_bf16(acc0[2] * inv, acc0[3] * inv),
             pack_bf16(acc1[0] * inv, acc1[1] * inv), pack_bf16(acc1[2] * inv, acc1[3] * inv)};
  *reinterpret_cast<u32x4*>(a.out + row * D + part * 8) = w;
  if (part == 0) a.lse_out[row] = tot > 0.f ? m + logf(tot) : -INFINITY;
}

hipError_t merge(MergeArgs& a, uint16_t* o, float* lse, long long rows, int D, hipStream_t stream) {
  a.out = o;
  a.lse_out = lse;
  a.rows = rows;
  const int rpb = kThreads / (D / 8 * SG);
  const long long grid = (rows + rpb - 1) / rpb;
  void* args[] = {&a};
  const void* k = D == 128 ? reinterpret_cast<const void*>(&attn_merge_kernel<128>)
                           : reinterpret_cast<const void*>(&attn_merge_kernel<64>);
  return hipLaunchKernel(k, dim3((unsigned)grid), dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_merge(const float* const* o_parts, const float* const* lse_parts, int n, uint16_t* o,
                        float* lse, long long rows, int D, hipStream_t stream) {
  MergeArgs a;
  for (int i = 0; i < kMaxMerge; ++i) {
    a.o[i] = i < n ? o_parts[i] : nullptr;
    a.lse[i] = i < n ? lse_parts[i] : nullptr;
  }
  a.o_base = a.lse_base = nullptr;
  a.o_stride = a.lse_stride = 0;
  a.n = n;
  return merge(a, o, lse, rows, D, stream);
}

hipError_t launch_merge_strided(const float* o_base, const float* lse_base, int n, long long o_stride,
                                long long lse_stride, uint16_t* o, float* lse, long long rows, int D,
                                hipStream_t stream) {
  MergeArgs a;
  for (int i = 0; i < kMaxMerge; ++i) a.o[i] = a.lse[i] = nullptr;
  a.o_base = o_base;
  a.lse_base = lse_base;
  a.o_stride = o_stride;
  a.lse_stride = lse_stride;
  a.n = n;
  return merge(a, o, lse, rows, D, stream);
}

}  // namespace tam
