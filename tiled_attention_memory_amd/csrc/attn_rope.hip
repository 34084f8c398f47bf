// Rotary position embedding for the attention kernels, gfx950.
//
// The AMD MI300X MoE training page trains with rotary embeddings of base
// 10^6; the rotation turns Q and K just before the product Q K^T that the page
// "使用 PyTorch FSDP 微調 Llama 2 70B" (agentlenshq.com), section "Flash
// Attention", fuses with the softmax. Rotate-half pairing: dimension d pairs
// with d + D/2 and turns by m * base^(-2d/D) at position m.
//
//   attn_rope_table_kernel: (cos, sin) per position and pair, from fp64
//       angles (so that long positions keep their accuracy), stored as fp32.
//   attn_rope_apply_kernel: a rotated bf16 copy of a [rows, D] tensor
//       (rows run over batch, head and position), with the same pair helper
//       the forward kernel uses on its Q rows, so both give identical bits.
// HBM-bound elementwise passes; the attention kernels take the table too.
#include <math.h>

#include "attn_device.h"
#include "attn_launch.h"

namespace tam {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void attn_rope_table_kernel(float2* tab, int S, int half_d, double base) {
  const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (long long)S * half_d) return;
  const int m = (int)(idx / half_d), d = (int)(idx % half_d);
  const double ang = (double)m * pow(base, -(double)d / (double)half_d);
  double sn, cs;
  sincos(ang, &sn, &cs);
  tab[idx] = make_float2((float)cs, (float)sn);
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_rope_apply_kernel(const uint16_t* x, uint16_t* out,
                                                                   const float2* tab, long long rows, int S) {
  constexpr int TPR = D / 16;  // threads per row: 8 pairs each
  const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= rows * TPR) return;
  const long long row = idx / TPR;
  const int d0 = 8 * (int)(idx % TPR);
  const int pos = (int)(row % S);
  const u32x4 lo = *reinterpret_cast<const u32x4*>(x + row * D + d0);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(x + row * D + D / 2 + d0);
  const float2* cs = tab + (size_t)pos * (D / 2) + d0;
  u32x4 ol, oh;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float l0, l1, h0, h1;
    rope_pair(bf16_lo(lo[j]), bf16_lo(hi[j]), cs[2 * j], false, &l0, &h0);
    rope_pair(bf16_hi(lo[j]), bf16_hi(hi[j]), cs[2 * j + 1], false, &l1, &h1);
    ol[j] = pack_bf16(l0, l1);
    oh[j] = pack_bf16(h0, h1);
  }
  *reinterpret_cast<u32x4*>(out + row * D + d0) = ol;
  *reinterpret_cast<u32x4*>(out + row * D + D / 2 + d0) = oh;
}

}  // namespace

hipError_t launch_rope_table(float2* tab, int S, int D, double base, hipStream_t stream) {
  const long long n = (long long)S * (D / 2);
  int half_d = D / 2;
  void* args[] = {(void*)&tab, (void*)&S, (void*)&half_d, (void*)&base};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_rope_table_kernel),
                         dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), args, 0, stream);
}

hipError_t launch_rope_apply(const uint16_t* x, uint16_t* out, const float2* tab, long long rows, int S, int D,
                             hipStream_t stream) {
  const long long n = rows * (D / 16);
  void* args[] = {(void*)&x, (void*)&out, (void*)&tab, (void*)&rows, (void*)&S};
  const void* k = D == 128 ? reinterpret_cast<const void*>(&attn_rope_apply_kernel<128>)
                           : reinterpret_cast<const void*>(&attn_rope_apply_kernel<64>);
  return hipLaunchKernel(k, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), args, 0, stream);
}

// Workspace of the RoPE passes: the table, rotated copies of K and Q, then
// the backward workspace of attn_bwd.
RopeLayout rope_layout(const AttnShape& sh) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  RopeLayout L;
  L.table = 0;
  L.k_rot = al((size_t)sh.Sq * (sh.D / 2) * sizeof(float2));
  L.q_rot = L.k_rot + al((size_t)sh.B * sh.Hkv * sh.Sk * sh.D * 2);
  L.bwd = L.q_rot + al((size_t)sh.B * sh.Hq * sh.Sq * sh.D * 2);
  L.total = L.bwd + bwd_workspace_bytes(sh);
  return L;
}

hipError_t launch_fwd_rope(AttnShape sh, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           float* lse, void* workspace, double base, hipStream_t stream) {
  const RopeLayout L = rope_layout(sh);
  char* ws = static_cast<char*>(workspace);
  float2* tab = reinterpret_cast<float2*>(ws + L.table);
  uint16_t* k_rot = reinterpret_cast<uint16_t*>(ws + L.k_rot);
  hipError_t e = launch_rope_table(tab, sh.Sq, sh.D, base, stream);
  if (e == hipSuccess) e = launch_rope_apply(k, k_rot, tab, (long long)sh.B * sh.Hkv * sh.Sk, sh.Sk, sh.D, stream);
  if (e != hipSuccess) return e;
  sh.rope = tab;  // Q is rotated inside the forward kernel
  return launch_fwd(sh, q, k_rot, v, o, nullptr, lse, stream);
}

hipError_t launch_bwd_rope(AttnShape sh, const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                           const uint16_t* dout, const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                           void* workspace, double base, hipStream_t stream) {
  const RopeLayout L = rope_layout(sh);
  char* ws = static_cast<char*>(workspace);
  float2* tab = reinterpret_cast<float2*>(ws + L.table);
  uint16_t* k_rot = reinterpret_cast<uint16_t*>(ws + L.k_rot);
  uint16_t* q_rot = reinterpret_cast<uint16_t*>(ws + L.q_rot);
  hipError_t e = launch_rope_table(tab, sh.Sq, sh.D, base, stream);
  if (e == hipSuccess) e = launch_rope_apply(k, k_rot, tab, (long long)sh.B * sh.Hkv * sh.Sk, sh.Sk, sh.D, stream);
  if (e == hipSuccess) e = launch_rope_apply(q, q_rot, tab, (long long)sh.B * sh.Hq * sh.Sq, sh.Sq, sh.D, stream);
  if (e != hipSuccess) return e;
  sh.rope = tab;  // the backward kernels rotate dQ and dK back in their epilogues
  return launch_bwd(sh, q_rot, k_rot, v, o, dout, lse, dq, dk, dv, ws + L.bwd, stream);
}

}  // namespace tam
