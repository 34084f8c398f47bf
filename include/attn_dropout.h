/*
 * attn_dropout.h - attention with dropout on the probabilities (libattn.so, gfx950).
 *
 * The page "使用 PyTorch FSDP 微調 Llama 2 70B" (agentlenshq.com), section
 * "Flash Attention", names dropout, with masking and softmax, among the
 * elementwise steps whose HBM traffic the fused kernel removes. Here it is
 * fused into the same tiles: after the softmax, each probability P_ij is kept
 * with probability 1 - p and scaled by r = 1 / (1 - p), or dropped:
 *
 *   O = (P * M * r) V,   LSE as in attn.h (before dropout),
 *
 * and the backward pass regenerates M instead of storing it. M comes from a
 * counter-based generator, Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011): one call per 4 x 4
 * block of (query row i, key j) of query head h of batch b, with counter
 * (j / 4, i / 4, b * Hq + h, 0) and key (seed mod 2^32, seed / 2^32); the
 * pair's byte is byte j % 4 (low byte first) of word i % 4 of the output, and
 * the pair is kept when that byte is at least t = round(256 p). The dropout
 * probability is therefore t / 256 and r = 256 / (256 - t); p below 1/512
 * means no dropout. The same (seed, p) in the forward and backward calls
 * gives the same mask.
 *
 * Arguments, layout, workspace, errors and limits are those of attn_fwd and
 * attn_bwd in attn.h, plus p (finite, 0 <= p < 255.5 / 256, else
 * ATTN_ERR_BAD_SCALE) and seed. The backward pass takes the o and lse the
 * forward pass wrote with the same p and seed.
 */
#ifndef TILED_ATTENTION_MEMORY_AMD_ATTN_DROPOUT_H
#define TILED_ATTENTION_MEMORY_AMD_ATTN_DROPOUT_H

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

int attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int S, int D, int causal, float scale,
                     float p, unsigned long long seed, hipStream_t stream);

int attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes,
                     int B, int Hq, int Hkv, int S, int D, int causal, float scale,
                     float p, unsigned long long seed, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TILED_ATTENTION_MEMORY_AMD_ATTN_DROPOUT_H */
