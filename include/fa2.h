/*
 * fa2.h - C ABI of the MI355X (gfx950) FlashAttention-2 forward library, libfa2.so.
 *
 * The operation (pages "FlashAttention学习笔记(2)", sections "V2 的运作流程 /
 * forward" and "V2中的thread blocks排布"; "Flash Attention V2原理解读", FWD
 * pseudo-code commentary and the thread-block grid section;
 * "flash-attention123和ring-attention", 优化1-优化4):
 *
 *   for every batch b < B, head h < H and query row i < Nq:
 *     S[i][j] = scale * sum_k Q[b][h][i][k] * K[b][h][j][k]       (j < Nk)
 *     S[i][j] = -inf where causal != 0 and j > i + Nk - Nq        (bottom-right aligned)
 *     O[b][h][i][:] = sum_j softmax_j(S[i][:]) * V[b][h][j][:]
 *     L[b][h][i]    = m_i + ln(l_i),  m_i = max_j S[i][j],  l_i = sum_j exp(S[i][j] - m_i)
 *
 * computed tile by tile: one work item per block of query rows (the outer
 * loop), K/V blocks streamed through LDS (the inner loop), an online running
 * row max and row sum, the division by l applied once after the loop, K/V
 * blocks that the causal mask covers entirely skipped, and only O and the
 * per-row logsumexp L written to memory.
 *
 * With Nq == Nk == N (fa2_fwd) the mask is the usual j > i.  The grid follows
 * the query length alone (page "FlashAttention学习笔记(2)", section "V2中的thread
 * blocks排布"), so the key length may differ (fa2_fwd_cross).  A query that sees
 * no key (causal with Nq > Nk, its first Nq - Nk rows, or Nk == 0) has an empty
 * sum: L = -inf and O = 0.
 *
 * Conventions shared by every entry point:
 *   - Layout: Q and O are contiguous row-major [B][H][Nq][d] arrays and K, V
 *     [B][H][Nk][d] arrays of the element type given by `dtype`; L is a
 *     contiguous [B][H][Nq] float32 array.
 *   - Ownership: every array pointer is device memory of the current HIP device,
 *     allocated and owned by the caller.  The library allocates nothing, frees
 *     nothing and keeps no pointer after the call returns.  O and L (and a
 *     workspace, where one is taken) must not overlap each other or Q, K, V.
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

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA2_OK = 0,
  FA2_EINVAL = -1,  /* an argument is invalid: null/misaligned/overlapping pointer, bad size, ... */
  FA2_ENOTSUP = -2, /* a valid request this build does not implement (head dim, dtype)           */
  FA2_EHIP = -3,    /* the HIP runtime reported an error (no device, launch failure, ...)        */
  FA2_STATUS_MAX_ENUM = 0x7fffffff /* not a status: makes the type a full 32-bit int */
} fa2_status_t;

typedef enum {
  FA2_BF16 = 0, /* bfloat16 Q/K/V/O; QK^T and PV on bf16 MFMA with float32 accumulation      */
  FA2_FP32 = 1, /* float32 Q/K/V/O; every step in float32 (exact mode, meant for small sizes) */
  FA2_FP16 = 2, /* float16 Q/K/V/O; QK^T and PV on fp16 MFMA with float32 accumulation       */
  /* Not dtypes: the two widen the enum to every 32-bit signed value, so that a caller
   * passing any int (an unknown code included) hands over a valid value of the type,
   * which the entry points then reject with FA2_ENOTSUP. */
  FA2_DTYPE_INVALID = -1,
  FA2_DTYPE_MAX_ENUM = 0x7fffffff
} fa2_dtype_t;

/*
 * fa2_fwd - the FlashAttention-2 forward pass.
 *
 *   Q, K, V  [B][H][N][d] inputs, device memory, 16-byte aligned.
 *   O        [B][H][N][d] output (same dtype), device memory, 16-byte aligned.
 *   L        [B][H][N] float32 output, the natural-log logsumexp of the scaled,
 *            masked logits of each row, device memory, 4-byte aligned.
 *   B, H, N  batch size, head count, sequence length (queries = keys); each
 *            >= 0.  A call with B*H*N == 0 does nothing and returns FA2_OK
 *            (pointers may be NULL).
 *   d        head dimension: 32, 64, 96, 128 or 256 (other values: FA2_ENOTSUP).
 *   causal   0: every key is visible; 1: key j is visible to row i iff j <= i.
 *   scale    softmax scale applied to Q K^T; any finite value (0 included).
 *   dtype    FA2_BF16, FA2_FP16 or FA2_FP32.
 *   stream   hipStream_t to enqueue on, or NULL for the default stream.
 *
 * Every element of O and L is written.  Results are deterministic: the same
 * inputs give the same bits on every call.
 */
fa2_status_t fa2_fwd(const void* Q, const void* K, const void* V, void* O, float* L,
                     int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                     fa2_dtype_t dtype, void* stream);

/*
 * fa2_fwd_cross - the forward pass with Nq queries over Nk keys (cross
 * attention; with causal, a block of queries appended after Nk - Nq earlier
 * positions, as in decoding).
 *
 *   Q, O     [B][H][Nq][d]; K, V [B][H][Nk][d]; L [B][H][Nq]; alignment and
 *            memory as for fa2_fwd.
 *   Nq, Nk   query and key lengths, each >= 0.  B*H*Nq == 0 does nothing and
 *            returns FA2_OK.  Nk == 0 writes O = 0 and L = -inf (K and V are
 *            not read and may be NULL then).
 *   causal   1: key j is visible to query i iff j <= i + Nk - Nq (the last
 *            query sees every key); rows that see no key get O = 0, L = -inf.
 *   B, H, d, scale, dtype, stream: as for fa2_fwd.
 *
 * fa2_fwd(..., N, ...) is fa2_fwd_cross(..., N, N, ...).
 */
fa2_status_t fa2_fwd_cross(const void* Q, const void* K, const void* V, void* O, float* L,
                           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                           float scale, fa2_dtype_t dtype, void* stream);

/* Largest number of key/value splits fa2_fwd_splitkv accepts. */
#define FA2_MAX_SPLITS 128

/*
 * fa2_fwd_splitkv - the forward pass with the key/value sequence split across
 * work items, for problems whose query blocks alone cannot fill the GPU.
 *
 * The pages (page "Flash Attention V2原理解读", the thread-block grid section)
 * allow splitting the key/value sequence as well as the queries when the
 * (query block, batch, head) grid leaves the GPU partly idle, at the price of
 * one more combine step: each row of O then gets one part from every split.
 * It is the decoding shape's path: few queries (Nq) over a long key sequence
 * (Nk).  The K/V blocks a query block visits (all of them, or those up to the
 * diagonal when causal) are cut into num_splits contiguous parts of
 * ceil(blocks / num_splits) blocks.  Each (query block, batch, head, part) is a
 * work item that writes its partial result to the workspace: O_s, normalised
 * within its keys, and L_s = m_s + ln(l_s) (-inf for a row that sees none of
 * its keys).  A second kernel on the same stream merges them:
 *   L = ln sum_s exp(L_s),   O = sum_s exp(L_s - L) O_s
 * (a row that sees no key in any split: O = 0, L = -inf).  The result is the
 * operation fa2_fwd_cross computes, up to rounding.
 *
 *   Q, K, V, O, L, B, H, Nq, Nk, d, causal, scale, stream: as for fa2_fwd_cross.
 *   dtype            FA2_BF16 or FA2_FP16 (FA2_FP32 gives FA2_ENOTSUP).
 *   num_splits       1..FA2_MAX_SPLITS, or 0 for the value fa2_num_splits gives.
 *   workspace        device memory owned by the caller, 16-byte aligned, of at
 *                    least fa2_splitkv_workspace_size() bytes for the number of
 *                    splits used; it must not overlap Q, K, V, O or L.  Its
 *                    contents on entry do not matter; on return they are
 *                    unspecified.  Calls sharing a workspace must be ordered.
 *   workspace_bytes  the workspace's size; too small gives FA2_EINVAL.
 *
 * Every element of O and L is written; results are deterministic.
 */
fa2_status_t fa2_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* L,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                             float scale, fa2_dtype_t dtype, int num_splits, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Size in bytes of the device scratch fa2_fwd_splitkv_noalloc uses (32 MiB). */
#define FA2_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
/*
 * fa2_fwd_splitkv_noalloc - fa2_fwd_splitkv for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc) and so cannot provide a workspace either.
 *
 * The partial results go to a scratch array that the library itself holds in
 * device memory, FA2_NOALLOC_SCRATCH_BYTES per GPU, for the life of the
 * process; the call allocates nothing (no hipMalloc, no allocating library
 * routine).  The split kernel writes every partial entry the merge reads, so
 * nothing needs clearing between calls.
 *
 *   Q, K, V, O, L, B, H, Nq, Nk, d, causal, scale, dtype, num_splits, stream:
 *            as for fa2_fwd_splitkv, which computes the same result with the
 *            same kernels.
 * Limit: num_splits * B*H*Nq * (d + 1) * 4 (fa2_splitkv_workspace_size) must
 * not exceed FA2_NOALLOC_SCRATCH_BYTES; larger problems return FA2_EINVAL
 * before any HIP call (num_splits == 0 first takes fa2_num_splits's choice,
 * a device query).
 * Concurrency: every call on one GPU shares that GPU's scratch, so calls whose
 * execution overlaps on one GPU (from several host threads, or on several
 * streams without ordering) race and give wrong results; order them on one
 * stream, or use fa2_fwd_splitkv with a workspace each.
 */
fa2_status_t fa2_fwd_splitkv_noalloc(const void* Q, const void* K, const void* V, void* O,
                                     float* L, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                     int64_t d, int causal, float scale, fa2_dtype_t dtype,
                                     int num_splits, void* stream);
/*
 * fa2_splitkv_workspace_size - bytes of workspace fa2_fwd_splitkv needs with
 * num_splits splits: num_splits * B*H*Nq * (d + 1) * 4 (the float32 partial
 * O_s and L_s of every split).  Host-only: makes no HIP call.  Returns the
 * argument errors fa2_fwd_splitkv would (sizes, d, num_splits out of range).
 */
fa2_status_t fa2_splitkv_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                        int num_splits, size_t* bytes);

/*
 * fa2_num_splits - the number of splits the pages' rule chooses for this
 * problem on the current device (page "Flash Attention V2原理解读", the
 * thread-block grid section): for every candidate s in 1..min(K/V blocks of
 * the Nk keys, FA2_MAX_SPLITS), the utilisation of the GPU by items * s work
 * items, items = B*H*ceil(Nq / 128) (the split kernel's 128-row query
 * blocks), over the device's concurrently
 * resident workgroups (the busy fraction of the last round:
 * (n / slots) / ceil(n / slots)); then the smallest s whose utilisation is at
 * least 0.95 of the best.  Queries the current device's compute-unit count (a
 * HIP call; FA2_EHIP if that fails).
 */
fa2_status_t fa2_num_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                            int* num_splits);

/*
 * fa2_fwd_partial - attention of Q over one part of the key/value sequence,
 * kept as a partial result that fa2_merge can combine with the other parts.
 *
 * When the key/value sequence is split, each row of O gets one part from
 * every split, and the parts must be combined once more to reach the global
 * softmax result (page "Flash Attention V2原理解读", the thread-block grid
 * section).  This is the building block of that: with K and V one contiguous
 * shard of the keys (for example the shard another GPU holds, in a ring of
 * GPUs over a long sequence), it writes
 *   O_part[b][h][i][:] = sum_j softmax_j(S[i][:]) V[j][:]   over this shard only,
 *   L_part[b][h][i]    = ln sum_j exp(S[i][j])              (-inf: no visible key)
 * in float32, O_part = 0 for a row with no visible key.
 *
 *   Q        [B][H][Nq][d]; K, V [B][H][Nk][d] (the shard); dtype FA2_BF16 or
 *            FA2_FP16 (FA2_FP32: FA2_ENOTSUP); 16-byte aligned device memory.
 *   O_part   [B][H][Nq][d] float32 output, 16-byte aligned.
 *   L_part   [B][H][Nq] float32 output, 4-byte aligned.
 *   causal   as for fa2_fwd_cross (bottom-right: the shard that ends where the
 *            queries end); 0 for a shard entirely before the queries.
 *   B, H, Nq, Nk, d, scale, stream: as for fa2_fwd_cross.  Nk == 0 writes
 *            O_part = 0, L_part = -inf.
 */
fa2_status_t fa2_fwd_partial(const void* Q, const void* K, const void* V, float* O_part,
                             float* L_part, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                             int64_t d, int causal, float scale, fa2_dtype_t dtype, void* stream);

/*
 * fa2_merge - combine num_parts partial results over disjoint key sets into
 * the attention over all of them (page "Flash Attention V2原理解读", the
 * thread-block grid section: the extra combine step split keys need):
 *   L = ln sum_s exp(L_s),   O = sum_s exp(L_s - L) O_s
 * (a row whose every L_s is -inf: O = 0, L = -inf).
 *
 *   O_parts  [num_parts][rows][d] float32, 16-byte aligned (fa2_fwd_partial's
 *            outputs, one after another).
 *   L_parts  [num_parts][rows] float32, 4-byte aligned.
 *   O        [rows][d] output of type dtype (FA2_BF16, FA2_FP16 or FA2_FP32),
 *            16-byte aligned; L [rows] float32 output.  rows = B*H*Nq for
 *            the [B][H][Nq] layout.
 *   num_parts 1..FA2_MAX_SPLITS; d as for fa2_fwd.  rows == 0 does nothing.
 * The outputs must not overlap the parts.
 */
fa2_status_t fa2_merge(const float* O_parts, const float* L_parts, int num_parts, void* O,
                       float* L, int64_t rows, int64_t d, fa2_dtype_t dtype, void* stream);

/*
 * fa2_launch_shape - the work decomposition fa2_fwd uses, as a host-only query.
 *
 * The work is one independent item per (query block, batch, head), with
 * num_m_block = ceil(N / kBlockM) query blocks per head: the pages' thread
 * blocks (page "FlashAttention学习笔记(2)", section "V2中的thread blocks排布";
 * "Flash Attention V2原理解读", the thread-block grid section).  Writes
 * kBlockM, num_m_block and the item count B*H*num_m_block through the
 * non-NULL out pointers (N is the query length).  kBlockM is 128 for the
 * 16-bit kernel (four wavefronts of 32 rows), except for d = 128 when
 * B*H*ceil(N / 256) >= 256: 256 (eight wavefronts, one workgroup per compute
 * unit); 4 for fp32.  The 16-bit kernel runs the
 * items on a persistent grid of min(items, resident workgroups) workgroups;
 * the fp32 kernel launches one workgroup per item.  Makes no HIP call.  Returns FA2_EINVAL / FA2_ENOTSUP
 * for arguments fa2_fwd would reject on those grounds.
 */
fa2_status_t fa2_launch_shape(int64_t B, int64_t H, int64_t N, int64_t d, fa2_dtype_t dtype,
                              int64_t* kBlockM, int64_t* num_m_block, int64_t* items);

/*
 * Host-only views of the work schedules (they make no HIP call and run on any
 * host), computed by the same integer functions the kernels compile.
 *
 * fa2_schedule_map - the forward kernel's persistent grid: with `grid`
 * workgroups over `items` work items (page "FlashAttention学习笔记(2)", section
 * "V2中的thread blocks排布": one item per query block of one (batch, head), times
 * the key/value splits of fa2_fwd_splitkv), workgroup g walks its XCD's
 * contiguous range of items in snake-ordered rounds.  Writes, for each item i
 * < items: visits[i], the number of workgroups that process it (1 in a correct
 * schedule), and, where the pointers are not NULL, workgroup[i] and
 * position[i], the workgroup that processes it and its place in that
 * workgroup's sequence.  items and grid: 1..2^31-1 (FA2_EINVAL otherwise).
 */
fa2_status_t fa2_schedule_map(int64_t items, int64_t grid, int32_t* visits, int32_t* workgroup,
                              int32_t* position);
/*
 * fa2_schedule_blocks - the key/value blocks each workgroup of the 16-bit
 * forward kernel visits for a problem, summed over its items, when launched
 * with `grid` workgroups: blocks[g] for g < grid, and *items, the number of
 * work items.  B, H, Nq, Nk, d, dtype and causal are as for fa2_fwd_cross
 * (Nk >= 1, B*H*Nq >= 1); num_splits 0 gives the plain kernel (kBlockM as
 * fa2_launch_shape reports), 1..FA2_MAX_SPLITS the split-KV kernel.  The
 * grid fa2_fwd uses is min(items, workgroups resident on the device).
 * FA2_FP32 gives FA2_ENOTSUP (that kernel has one workgroup per item).
 */
fa2_status_t fa2_schedule_blocks(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                 fa2_dtype_t dtype, int causal, int num_splits, int64_t grid,
                                 int64_t* blocks, int64_t* items);
/*
 * fa2_bwd_block_map - the logical block (key block of the dK/dV kernel, query
 * block of the dQ kernel) that workgroup id takes in a backward grid of G
 * workgroups: logical[id] for id < G.  XCD x = id % 8 takes a contiguous range
 * of logical blocks, so the blocks of one head share an L2.  G: 1..2^31-1.
 */
fa2_status_t fa2_bwd_block_map(int64_t G, int32_t* logical);
/* fa2_strerror - static description of a status code (never NULL). */
const char* fa2_strerror(fa2_status_t status);

/*
 * fa2_bwd - the FlashAttention-2 backward pass: the gradients dQ, dK, dV of
 * O = fa2_fwd(Q, K, V) for an upstream gradient dO.
 *
 * The pages (page "FlashAttention学习笔记(2)", the forward section and the
 * forward/backward thread-block split; page "Flash Attention V2原理解读", the
 * backward discussion; page "flash-attention123和ring-attention", 优化1) fix the
 * structure: P is recomputed block by block as exp(scale * Q K^T - L) from the
 * forward's L alone, with K/V outer and Q inner (dK, dV accumulate along a K/V
 * block, dQ across K/V blocks).  The gradients are the chain rule of softmax
 * attention: D = rowsum(dO * O), dV = P^T dO, dS = P * (dO V^T - D),
 * dQ = scale * dS K, dK = scale * dS^T Q (with the causal mask, P = 0 above the
 * diagonal).  dQ is computed by a second, query-outer pass rather than with
 * atomics, so results are deterministic.
 *
 *   Q, K, V, O, dO   [B][H][N][d] inputs of type dtype, device memory, 16-byte
 *                    aligned; O is fa2_fwd's output for Q, K, V (only
 *                    rowsum(dO * O) is used).
 *   L                [B][H][N] float32, fa2_fwd's L, device memory, 4-byte aligned.
 *   dQ, dK, dV       [B][H][N][d] outputs of type dtype, device memory, 16-byte aligned.
 *   B, H, N, causal, scale, stream: as for fa2_fwd (the same values as the
 *                    forward call).  B*H*N == 0 does nothing and returns FA2_OK.
 *   d                32, 64, 96, 128 or 256 (others: FA2_ENOTSUP); d = 256 runs one
 *                    workgroup per CU (its dK and dV accumulators take 256 registers).
 *   dtype            FA2_BF16 or FA2_FP16 (FA2_FP32: FA2_ENOTSUP).
 *   workspace        device memory owned by the caller, 4-byte aligned, at least
 *                    fa2_bwd_workspace_size() bytes (it receives -D and L*log2(e));
 *                    contents on entry do not matter.  workspace_bytes is its size.
 * The outputs and the workspace must not overlap each other or any input.
 * Every element of dQ, dK and dV is written; results are deterministic.
 */
fa2_status_t fa2_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                     const float* L, void* dQ, void* dK, void* dV, int64_t B, int64_t H,
                     int64_t N, int64_t d, int causal, float scale, fa2_dtype_t dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa2_bwd_cross - the backward pass of fa2_fwd_cross: Q, O, dO, L and dQ have
 * Nq rows ([B][H][Nq][d], L [B][H][Nq]), K, V, dK and dV Nk rows; the causal
 * mask is aligned bottom-right as in the forward (key j visible to query i iff
 * j <= i + Nk - Nq).  A query that sees no key adds nothing (its dQ row is 0),
 * and a key no query sees gets dK = dV = 0.  Arrays of zero size may be NULL.
 * Everything else as for fa2_bwd; the workspace holds one float32 per query
 * row, padded (fa2_bwd_workspace_size with N = Nq).
 */
fa2_status_t fa2_bwd_cross(const void* Q, const void* K, const void* V, const void* O,
                           const void* dO, const float* L, void* dQ, void* dK, void* dV,
                           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                           float scale, fa2_dtype_t dtype, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * fa2_bwd_workspace_size - bytes of workspace fa2_bwd needs: B*H*N32 * 8 with
 * N32 = N rounded up to a multiple of 32 (two float32 arrays, -D = -rowsum(dO*O)
 * and L*log2(e), with each head's rows padded to N32; N = Nq for
 * fa2_bwd_cross).  Host-only: makes no HIP
 * call.  Returns the size and head dimension errors fa2_bwd would.
 */
fa2_status_t fa2_bwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, size_t* bytes);

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
