/*
 * fa2.h - C ABI of the MI355X (gfx950) FlashAttention-2 forward library, libfa2.so.
 *
 * The operation (pages "FlashAttention学习笔记(2)", sections "V2 的运作流程 /
 * forward" and "V2中的thread blocks排布"; "Flash Attention V2原理解读", FWD
 * pseudo-code commentary and the thread-block grid section;
 * "flash-attention123和ring-attention", 优化1-优化4):
 *
 *   for every batch b < B, head h < H and query row i < N:
 *     S[i][j] = scale * sum_k Q[b][h][i][k] * K[b][h][j][k]       (j < N)
 *     S[i][j] = -inf where causal != 0 and j > i                   (top-left aligned)
 *     O[b][h][i][:] = sum_j softmax_j(S[i][:]) * V[b][h][j][:]
 *     L[b][h][i]    = m_i + ln(l_i),  m_i = max_j S[i][j],  l_i = sum_j exp(S[i][j] - m_i)
 *
 * computed tile by tile: one workgroup per block of query rows (the outer
 * loop), K/V blocks streamed through LDS (the inner loop), an online running
 * row max and row sum, the division by l applied once after the loop, K/V
 * blocks that the causal mask covers entirely skipped, and only O and the
 * per-row logsumexp L written to memory.
 *
 * Conventions shared by every entry point:
 *   - Layout: Q, K, V and O are contiguous row-major [B][H][N][d] arrays of the
 *     element type given by `dtype`; L is a contiguous [B][H][N] float32 array.
 *     Queries and keys have the same length N.
 *   - Ownership: every array pointer is device memory of the current HIP device,
 *     allocated and owned by the caller.  The library allocates nothing, frees
 *     nothing and keeps no pointer after the call returns.  O and L must not
 *     overlap each other or Q, K, V.
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL means the
 *     default stream) and the call returns without synchronising.
 *   - Thread safety: calls may be made from any number of host threads.  The only
 *     mutable state is a thread-local error message.
 *   - Errors are returned as status codes and never thrown across the ABI.
 *     Argument errors are detected before any work is enqueued; a failed launch
 *     is reported as FA2_EHIP with the HIP error named in fa2_last_error().
 */
#ifndef FA2_H
#define FA2_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA2_OK = 0,
  FA2_EINVAL = -1,  /* an argument is invalid: null/misaligned/overlapping pointer, bad size, ... */
  FA2_ENOTSUP = -2, /* a valid request this build does not implement (head dim, dtype)           */
  FA2_EHIP = -3     /* the HIP runtime reported an error (no device, launch failure, ...)        */
} fa2_status_t;

typedef enum {
  FA2_BF16 = 0, /* bfloat16 Q/K/V/O; QK^T and PV on bf16 MFMA with float32 accumulation      */
  FA2_FP32 = 1  /* float32 Q/K/V/O; every step in float32 (exact mode, meant for small sizes) */
} fa2_dtype_t;

/*
 * fa2_fwd - the FlashAttention-2 forward pass.
 *
 *   Q, K, V  [B][H][N][d] inputs, device memory, 16-byte aligned.
 *   O        [B][H][N][d] output (same dtype), device memory, 16-byte aligned.
 *   L        [B][H][N] float32 output, the natural-log logsumexp of the scaled,
 *            masked logits of each row, device memory, 4-byte aligned.
 *   B, H, N  batch size, head count, sequence length; each >= 0.  A call with
 *            B*H*N == 0 does nothing and returns FA2_OK (pointers may be NULL).
 *   d        head dimension: 64, 128 or 256 (other values: FA2_ENOTSUP).
 *   causal   0: every key is visible; 1: key j is visible to row i iff j <= i.
 *   scale    softmax scale applied to Q K^T; any finite value (0 included).
 *   dtype    FA2_BF16 or FA2_FP32.
 *   stream   hipStream_t to enqueue on, or NULL for the default stream.
 *
 * Every element of O and L is written.  Results are deterministic: the same
 * inputs give the same bits on every call.
 */
fa2_status_t fa2_fwd(const void* Q, const void* K, const void* V, void* O, float* L,
                     int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                     fa2_dtype_t dtype, void* stream);

/*
 * fa2_launch_shape - the work decomposition fa2_fwd uses, as a host-only query.
 *
 * The work is one independent item per (query block, batch, head), with
 * num_m_block = ceil(N / kBlockM) query blocks per head: the pages' thread
 * blocks (page "FlashAttention学习笔记(2)", section "V2中的thread blocks排布";
 * "Flash Attention V2原理解读", the thread-block grid section).  Writes
 * kBlockM, num_m_block and the item count B*H*num_m_block through the
 * non-NULL out pointers.  The bf16 kernel runs the items on a persistent grid
 * of min(items, resident workgroups) workgroups; the fp32 kernel launches one
 * workgroup per item.  Makes no HIP call.  Returns FA2_EINVAL / FA2_ENOTSUP
 * for arguments fa2_fwd would reject on those grounds.
 */
fa2_status_t fa2_launch_shape(int64_t B, int64_t H, int64_t N, int64_t d, fa2_dtype_t dtype,
                              int64_t* kBlockM, int64_t* num_m_block, int64_t* items);

/* fa2_strerror - static description of a status code (never NULL). */
const char* fa2_strerror(fa2_status_t status);

/*
 * fa2_last_error - detail of the last failure on the calling thread: which
 * argument was rejected, or the HIP error name and text.  Empty string if the
 * thread's last call succeeded.  The pointer stays valid until the thread's
 * next call into the library.
 */
const char* fa2_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */
