/*
 * attn_decode.h - attention of a few new tokens against a key/value cache
 * (libattn.so, gfx950).
 *
 * The same exact attention as attn.h, for the shape of generation: Sq new
 * query tokens per head (sitting at positions Sk - Sq .. Sk - 1) against the
 * Sk cached keys and values, which already include the new tokens. With
 * causal = 1 token t sees keys 0 .. Sk - Sq + t. The page "使用 PyTorch FSDP
 * 微調 Llama 2 70B" (agentlenshq.com), section "Flash Attention", splits the
 * scores into tiles combined by an online softmax; here the key range of each
 * (batch, kv head) is split into chunks processed in parallel (as many as it
 * takes to occupy every CU; none when there are enough (batch, kv head)
 * pairs), each giving a partial output and log-sum-exp, and the chunks are
 * merged exactly by their log-sum-exps (the same combination as attn_merge in
 * attn_block.h). The query heads of a group share one pass over their cached
 * keys and values, which is what bounds this shape: every cached byte is read
 * once.
 *
 * Layout and rules as in attn.h: q, o bf16 [B, Hq, Sq, D]; k, v bf16
 * [B, Hkv, Sk, D]; lse f32 [B, Hq, Sq]; caller-owned, 16-byte aligned device
 * pointers; nothing allocated; work enqueued on `stream`; validation before
 * anything is enqueued. Limits: 1 <= Sq, (Hq / Hkv) * Sq <= 128, Sq <= Sk <=
 * ATTN_MAX_SEQ, D in {64, 128}.
 */
#ifndef TILED_ATTENTION_MEMORY_AMD_ATTN_DECODE_H
#define TILED_ATTENTION_MEMORY_AMD_ATTN_DECODE_H

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of device workspace attn_decode needs (fp32 partials of every chunk; a
 * small minimum when the keys are not split). */
int attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D, size_t* bytes);

/*
 * o   bf16 [B, Hq, Sq, D]  out
 * lse f32  [B, Hq, Sq]     out, natural log
 * workspace: at least attn_decode_workspace_bytes(...) bytes, contents ignored.
 * Returns an attn_status (ATTN_ERR_BAD_SHAPE when (Hq / Hkv) * Sq > 128 or Sq > Sk).
 */
int attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                void* workspace, size_t workspace_bytes,
                int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale,
                hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TILED_ATTENTION_MEMORY_AMD_ATTN_DECODE_H */
