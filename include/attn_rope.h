/*
 * attn_rope.h - attention with rotary position embedding on Q and K
 * (libattn.so, gfx950).
 *
 * Rotary embedding turns each pair of dimensions of a query or key row by an
 * angle proportional to the row's position; the AMD MI300X MoE training page
 * trains with base 10^6. The rotation sits right before the product Q K^T
 * that the page "使用 PyTorch FSDP 微調 Llama 2 70B" (agentlenshq.com),
 * section "Flash Attention", fuses with the softmax. Pairing is rotate-half
 * (dimension d with d + D/2, the Llama and GPT-NeoX convention); row i of the
 * sequence is at position i:
 *
 *   a_d = i * base^(-2d/D),  d < D/2
 *   q'_d = q_d cos a_d - q_{d+D/2} sin a_d,  q'_{d+D/2} = q_{d+D/2} cos a_d + q_d sin a_d
 *   (likewise k'), then attention of attn.h on (q', k', v).
 *
 * The forward pass rotates Q inside the attention kernel as it loads each
 * query row, and K once into the workspace (it is shared by the group's query
 * heads); the backward pass rotates Q and K into the workspace and turns dQ
 * and dK back (the inverse rotation) inside the kernels that produce them,
 * before their bf16 rounding. Angles are formed in fp64. The rotated values
 * enter the bf16 products rounded to bf16, identically in both passes.
 *
 * Arguments, layout, outputs, errors and limits are those of attn_fwd and
 * attn_bwd in attn.h, plus base (finite and > 0, else ATTN_ERR_BAD_SCALE) and
 * a workspace of at least attn_rope_workspace_bytes(...) bytes for both calls
 * (the backward pass's own workspace included); o and lse passed to
 * attn_bwd_rope are those attn_fwd_rope wrote with the same base. dq and dk
 * are gradients with respect to the unrotated q and k.
 */
#ifndef TILED_ATTENTION_MEMORY_AMD_ATTN_ROPE_H
#define TILED_ATTENTION_MEMORY_AMD_ATTN_ROPE_H

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

int attn_rope_workspace_bytes(int B, int Hq, int Hkv, int S, int D, size_t* bytes);

int attn_fwd_rope(const void* q, const void* k, const void* v, void* o, float* lse,
                  void* workspace, size_t workspace_bytes,
                  int B, int Hq, int Hkv, int S, int D, int causal, float scale, float base,
                  hipStream_t stream);

int attn_bwd_rope(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv,
                  void* workspace, size_t workspace_bytes,
                  int B, int Hq, int Hkv, int S, int D, int causal, float scale, float base,
                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TILED_ATTENTION_MEMORY_AMD_ATTN_ROPE_H */
