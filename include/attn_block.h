/*
 * attn_block.h - context-parallel building block of libattn.so (gfx950).
 *
 * Attention between one query block and one key/value block of a longer
 * sequence, placed at global positions, plus the exact merge of the partial
 * results over key blocks and a backward pass that is exact over all blocks.
 * The page "使用 PyTorch FSDP 微調 Llama 2 70B" (agentlenshq.com), section
 * "Flash Attention", processes the scores in tiles combined by an online
 * softmax; a sequence split across GPUs (context parallelism, which the AMD
 * MI300X MoE training page runs at degree 2 for 32k and 8 for 128k tokens,
 * section 4.1) combines whole key blocks the same way. These calls are the
 * per-GPU work of such a split; moving blocks between GPUs is the caller's.
 *
 * Positions: query row i of the block sits at global position q_pos0 + i and
 * key j at k_pos0 + j. With causal = 1, key j is visible to row i when
 * k_pos0 + j <= q_pos0 + i. A row that sees no key of a block has no softmax
 * over it: its partial output is 0 and its partial log-sum-exp is -inf.
 *
 *   s_ij       = scale * <q_i, k_j>
 *   O_b,i      = sum_j softmax_j(s_i.) v_j        over the block's visible keys
 *   LSE_b,i    = ln sum_j exp(s_ij)
 *   merged:  LSE = ln sum_b exp(LSE_b),  O = sum_b exp(LSE_b - LSE) O_b
 *
 * Layout, ownership, threading, aliasing and error rules are those of attn.h:
 * contiguous row-major tensors, caller-owned device pointers (16-byte
 * aligned), nothing allocated, work enqueued on `stream` only, validation
 * before anything is enqueued. Q, dO, dQ are [B, Hq, Sq, D]; K, V, dK, dV are
 * [B, Hkv, Sk, D]; LSE is [B, Hq, Sq]. 1 <= Sq, Sk <= ATTN_MAX_SEQ;
 * |q_pos0|, |k_pos0| <= 2^62.
 */
#ifndef TILED_ATTENTION_MEMORY_AMD_ATTN_BLOCK_H
#define TILED_ATTENTION_MEMORY_AMD_ATTN_BLOCK_H

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_MAX_MERGE 16

/*
 * Forward pass of one block pair (the "Tiling" bullet of the section above,
 * applied to a block of keys at an offset).
 *   q        bf16 [B, Hq, Sq, D]   in
 *   k, v     bf16 [B, Hkv, Sk, D]  in
 *   o_part   f32  [B, Hq, Sq, D]   out: output normalised over this block's keys
 *   lse_part f32  [B, Hq, Sq]      out: natural-log log-sum-exp over them
 * Rows that see no key: o_part = 0, lse_part = -inf.
 * Returns an attn_status.
 */
int attn_fwd_block(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                   int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal,
                   long long q_pos0, long long k_pos0, float scale, hipStream_t stream);

/*
 * Merge n partial results (1 <= n <= ATTN_MAX_MERGE) of the same query block
 * over disjoint key blocks into the final output.
 *   o_parts[b]   f32 [B, Hq, Sq, D] in (device pointers, in a host array)
 *   lse_parts[b] f32 [B, Hq, Sq]    in
 *   o            bf16 [B, Hq, Sq, D] out, rounded to nearest even
 *   lse          f32  [B, Hq, Sq]    out (-inf where no part saw a key)
 * The outputs must not overlap any part. ATTN_ERR_BAD_SHAPE for n out of range.
 */
int attn_merge(const float* const* o_parts, const float* const* lse_parts, int n,
               void* o, float* lse, int B, int Hq, int Sq, int D, hipStream_t stream);

/*
 * Backward pass over the blocks (the "Recomputation" bullet), exact for the
 * whole row: the row term Delta_i = sum_j P_ij dP_ij needs every key block,
 * so dQ is gathered in one sweep over the key blocks and dK, dV in a second:
 *
 *   attn_bwd_block_begin     once: per-row terms from the merged o, lse and dO
 *   attn_bwd_block_dq        once per key block, in any order: accumulates that
 *                            block's part of dQ in the workspace
 *   attn_bwd_block_dq_end    once: writes dQ and the exact Delta
 *   attn_bwd_block_dkdv      once per key block: that block's dK, dV from this
 *                            query block (bf16, overwritten; summed over the
 *                            query heads of each group)
 *
 * o and lse are the merged results (attn_merge, or attn_fwd for one block).
 * The workspace belongs to one query block for the whole sequence of calls;
 * Sk in attn_bwd_block_workspace_bytes is the largest key block used, and the
 * size it returns serves every call whose key block holds at most Sk keys
 * (a shorter block may split the work more finely and need more partials
 * than the longest one; the size covers that). The calls of one sequence
 * must be ordered (one stream); each call is deterministic, so the results
 * are bitwise reproducible for a fixed order of key blocks. B, Hq, Hkv, Sq, D
 * (and scale) must be the same in every call.
 */
int attn_bwd_block_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D, size_t* bytes);

int attn_bwd_block_begin(const void* o, const void* dout, const float* lse,
                         void* workspace, size_t workspace_bytes,
                         int B, int Hq, int Hkv, int Sq, int Sk, int D, hipStream_t stream);

int attn_bwd_block_dq(const void* q, const void* k, const void* v, const void* dout,
                      void* workspace, size_t workspace_bytes,
                      int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal,
                      long long q_pos0, long long k_pos0, float scale, hipStream_t stream);

/* dq bf16 [B, Hq, Sq, D] out. Sk as given to attn_bwd_block_begin. */
int attn_bwd_block_dq_end(void* dq, void* workspace, size_t workspace_bytes,
                          int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                          hipStream_t stream);

/* dk, dv bf16 [B, Hkv, Sk, D] out. */
int attn_bwd_block_dkdv(const void* q, const void* k, const void* v, const void* dout,
                        void* dk, void* dv, void* workspace, size_t workspace_bytes,
                        int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal,
                        long long q_pos0, long long k_pos0, float scale, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TILED_ATTENTION_MEMORY_AMD_ATTN_BLOCK_H */
