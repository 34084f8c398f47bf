/*
 * attn.h - C ABI of the MI355X (gfx950) exact-attention library libattn.so.
 *
 * The operation is exact scaled-dot-product attention with an optional causal
 * mask and grouped-query heads, computed the way the page
 * "使用 PyTorch FSDP 微調 Llama 2 70B" (agentlenshq.com), section
 * "Flash Attention", describes: the score matrix is cut into tiles that stay
 * on chip, normalised with an online softmax, and fused with the products on
 * either side so that only the output and one log-sum-exp per row reach HBM
 * (bullets "Kernel Fusion" and "Tiling"); the backward pass recomputes the
 * probabilities from Q, K, V and that log-sum-exp instead of storing the
 * N x N matrix (bullet "Recomputation").
 *
 *   s_ij  = scale * <q_i, k_j>        (key j hidden from query i when causal and j > i)
 *   O_i   = sum_j softmax_j(s_i.) v_j
 *   LSE_i = ln sum_j exp(s_ij)        (natural log, over the visible keys)
 *
 * Query head h of batch b reads key/value head h / (Hq / Hkv) of batch b.
 *
 * Layout: every tensor is contiguous row-major; Q, O, dO, dQ are [B, Hq, S, D],
 * K, V, dK, dV are [B, Hkv, S, D], LSE is [B, Hq, S]. bf16 tensors hold raw
 * bfloat16 bit patterns (2 bytes per element); LSE is IEEE float32.
 *
 * Memory and ownership: every pointer is a device pointer owned by the caller.
 * The library allocates nothing, keeps no state between calls and may be
 * called from several host threads at once. Calls only enqueue work on the
 * given stream and never synchronise; results are ready when the stream
 * reaches that point. Outputs are overwritten, never accumulated into, and
 * must not overlap any input or each other.
 *
 * Errors: arguments are validated before anything is enqueued; on an error the
 * call returns a nonzero attn_status and enqueues nothing. A failure reported
 * by the HIP runtime when launching is returned as ATTN_ERR_HIP. No C++
 * exception crosses this interface.
 *
 * Limits: 1 <= B, Hq, Hkv; Hq % Hkv == 0; 1 <= S <= ATTN_MAX_SEQ; D in {64, 128};
 * causal in {0, 1}; scale finite (0 gives uniform weights over visible keys);
 * all pointers 16-byte aligned.
 */
#ifndef TILED_ATTENTION_MEMORY_AMD_ATTN_H
#define TILED_ATTENTION_MEMORY_AMD_ATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_VERSION 1
#define ATTN_MAX_SEQ (1 << 22)

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL_POINTER = 1,           /* a required pointer is NULL */
    ATTN_ERR_BAD_SHAPE = 2,              /* B, Hq, Hkv or S out of range, Hq % Hkv != 0, size overflow */
    ATTN_ERR_UNSUPPORTED_HEAD_DIM = 3,   /* D not in {64, 128} */
    ATTN_ERR_BAD_SCALE = 4,              /* scale is NaN or infinite */
    ATTN_ERR_MISALIGNED = 5,             /* a pointer is not 16-byte aligned */
    ATTN_ERR_WORKSPACE = 6,              /* workspace missing or smaller than required */
    ATTN_ERR_HIP = 7,                    /* the HIP runtime reported an error at launch */
    ATTN_ERR_BAD_FLAG = 8,               /* causal not 0 or 1 */
    ATTN_ERR_ALIAS = 9,                  /* an output overlaps an input or another output */
    ATTN_ERR_SCRATCH_LIMIT = 10          /* attn_bwd_noalloc: sizes need more than its fixed scratch */
} attn_status;

/*
 * Forward pass (bullets "Kernel Fusion" and "Tiling" of the section above).
 *   q   bf16 [B, Hq, S, D]    in
 *   k   bf16 [B, Hkv, S, D]   in
 *   v   bf16 [B, Hkv, S, D]   in
 *   o   bf16 [B, Hq, S, D]    out: the attention output, rounded to nearest even
 *   lse f32  [B, Hq, S]       out: natural-log log-sum-exp of each row's scaled,
 *                             masked scores (kept for the backward pass)
 * Returns an attn_status.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int S, int D, int causal, float scale,
             hipStream_t stream);

/*
 * Size in bytes of the device workspace attn_bwd needs for these sizes. Writes
 * it to *bytes. The workspace holds, per query row, the row term Delta and the
 * LSE in base 2 (fp32); fp16 copies of Q, dO and K scaled by powers of two,
 * with one exponent per 32-row block of Q and dO (and of Delta) and per
 * 64-key tile of K and V; and, when the query heads of a group are split into
 * subsets for load balance, fp32 dK/dV partials of each subset (the
 * one-kernel pass of S <= 64 uses only its partials). Examples: B=1, Hq=64,
 * Hkv=8, S=4096, D=128 needs 202 MiB; B=1, Hq=8, Hkv=1, S=81920, D=128 needs
 * 665 MiB.
 * Returns ATTN_OK, ATTN_ERR_NULL_POINTER (bytes NULL), ATTN_ERR_BAD_SHAPE or
 * ATTN_ERR_UNSUPPORTED_HEAD_DIM.
 */
int attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D, size_t* bytes);

/*
 * Backward pass (bullet "Recomputation" of the section above): gradients of
 * L = sum(O * dO) with respect to q, k and v, recomputing the probabilities
 * from q, k and lse.
 *   q, k, v, o, dout   bf16 as in attn_fwd (o and lse exactly as attn_fwd wrote them)
 *   lse                f32 [B, Hq, S] from attn_fwd
 *   dq   bf16 [B, Hq, S, D]   out
 *   dk   bf16 [B, Hkv, S, D]  out: summed over the Hq / Hkv query heads of each group
 *   dv   bf16 [B, Hkv, S, D]  out: summed likewise
 *   workspace, workspace_bytes: device scratch of at least
 *                      attn_bwd_workspace_bytes(...) bytes, 16-byte aligned,
 *                      owned by the caller; its contents on entry are ignored
 *                      and on return are unspecified.
 * dK and dV are accumulated without atomics; the results are bitwise
 * reproducible for the same inputs and sizes. The row term Delta is made
 * exact inside the pass (not taken from the rounded o alone). For S <= 64
 * every row's keys fit one tile and a single kernel forms dQ, dK and dV,
 * with Delta = sum_j P_ij dP_ij over the whole row (o is then not read).
 * Precision of the matrix products (every one accumulates in fp32; the
 * outputs are rounded to bf16 once, at the end):
 *   S >= 512: every product of the dK/dV kernel (S, dP, dV, dK) and the dQ
 *     kernel's products with K (S, P K and dQ) run on fp16 operands (11
 *     significant bits): Q, dO and K are copied to fp16 with one power-of-two
 *     scale per block of 32 rows or 64 keys, and P and dS enter with scales
 *     that keep them inside fp16's range. dP = dO V^T of the dQ kernel runs on
 *     the bf16 inputs.
 *     The gradients then carry an error of about 1e-4 to 3e-4 of their
 *     largest element beyond their bf16 rounding: inside 2e-2 for gradients of
 *     unit size, above it for gradients of 80 and more (a softmax scale several
 *     times 1/sqrt(D) on inputs of several units).
 *   S < 512 (and the one-kernel pass of S <= 64): bf16 products on the
 *     inputs, with P and dS entering as hi + lo pairs of bf16 values (about
 *     16 significant bits).
 * Returns an attn_status.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes,
             int B, int Hq, int Hkv, int S, int D, int causal, float scale,
             hipStream_t stream);

/*
 * attn_bwd for measurement tools: identical arguments, results and errors,
 * plus ATTN_BWD_EVENTS caller-created events (hipEventCreate) recorded on
 * `stream` around the backward kernels:
 *   events[0] first
 *   events[1] after the fp16 copy of K (S >= 512; else right after events[0]),
 *             before the dQ kernel; for S <= 64, after the one-kernel pass
 *   events[2] after the dQ kernel, before the dK/dV kernel (S <= 64: right
 *             after events[1])
 *   events[3] after the dK/dV kernel (S <= 64: right after events[2])
 *   events[4] after the fixed-order sum of per-head-subset dK/dV partials
 *             (recorded right after events[3] when no partials are used)
 * The events stay owned by the caller; pass NULL to behave exactly like attn_bwd.
 */
#define ATTN_BWD_EVENTS 5
int attn_bwd_timed(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes,
                   int B, int Hq, int Hkv, int S, int D, int causal, float scale,
                   hipStream_t stream, hipEvent_t* events);

/*
 * attn_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments as attn_bwd minus the workspace,
 * the same results (the same kernels, bitwise equal outputs) and errors.
 * The call itself allocates nothing. In place of a caller workspace it uses a
 * fixed device array inside the library, ATTN_NOALLOC_SCRATCH_BYTES (256 MiB)
 * on every GPU the library runs on, held from the first use of the library on
 * that GPU until the process ends. Sizes whose workspace
 * (attn_bwd_workspace_bytes) exceeds it return ATTN_ERR_SCRATCH_LIMIT and
 * enqueue nothing; B=1, Hq=64, Hkv=8, S=4096, D=128 needs 202 MiB and fits.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (different streams, or different host threads, without ordering
 * between them) race on it and give wrong results. Order them, e.g. on one
 * stream. The array's contents are not needed between calls (every call
 * writes what it reads). The current device must be the stream's device.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv,
                     int B, int Hq, int Hkv, int S, int D, int causal, float scale,
                     hipStream_t stream);

/* Static description of a status code (never NULL). */
const char* attn_status_string(int status);

/* ATTN_VERSION of the built library. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TILED_ATTENTION_MEMORY_AMD_ATTN_H */
