/*
 * jfa.h -- C ABI of the MI355X (gfx950) Jagged Flash Attention library (libjfa.so).
 *
 * Jagged Flash Attention is exact softmax attention applied directly to packed,
 * unpadded sequences addressed through an offsets tensor ("Meta's TLX attention
 * kernel outpaces FlashAttention-4 on B200", section "GEM's sequences do not fit
 * a fixed grid"; "Optimizing Jagged Flash Attention with TLX" reading note,
 * section "Why variable lengths change the problem").  Two modes:
 *
 *   broadcast-Q  one dense query sequence Q [Lq, H, D] attends to the K/V of every
 *                sequence b; output rows b*Lq + i.  In the backward pass every
 *                sequence adds into the same dQ (same sections of both pages).
 *   self         Q, K and V are all packed with the same offsets; optional causal
 *                mask inside each sequence (key j visible to query i iff j <= i,
 *                both counted from the sequence start).  Block-diagonal attention
 *                ("Meta's TLX Block Attention Beats Flash Attention v2 by 2.3x on
 *                Blackwell GPUs", section "The Pattern That Changes Everything") is
 *                the case where every sequence has 64 tokens.
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers to contiguous row-major memory, 16-byte
 *     aligned.  bf16 means IEEE bfloat16 stored as 2 bytes.
 *   - q      bf16 [Lq, H, D] (broadcast) or [T, H, D] (self).
 *   - k, v   bf16 [T, H, D], T = total_kv = offsets[batch].
 *   - offsets int32 or int64 [batch + 1] (offsets_is_int64 selects), device memory.
 *     Preconditions (not checked on the device): offsets[0] = 0, non-decreasing,
 *     offsets[batch] = total_kv.
 *   - o, d_o bf16 [rows, H, D] with rows = batch*Lq (broadcast) or T (self).
 *   - lse    fp32 [H, rows]: natural-log log-sum-exp of the scaled scores
 *            c * q_i . k_j over the visible keys; -inf for a row with no key.
 *   - dq like q, dk and dv like k; all bf16.  Accumulation is fp32 throughout.
 *   - head_dim must be 64 or 128 ("Meta's TLX Block Attention Beats Flash Attention
 *     v2 by 2.3x on Blackwell GPUs", section "Who Should Use This", names these two
 *     head sizes); heads >= 1.
 *   - Work is enqueued on `stream` without any host synchronisation; the caller
 *     keeps every buffer alive until that work completes.  Outputs are
 *     overwritten, never accumulated into.
 *   - The library allocates no device memory: scratch space comes from the
 *     caller's `workspace` (size from the matching *_workspace_size call, 256-byte
 *     aligned).  Its only state is a per-device cache of the compute-unit count
 *     and the schedule selector below.
 *   - Errors are returned as jfa_status_t; nothing aborts or throws across the
 *     ABI.  jfa_last_error() gives a thread-local message for the last non-OK
 *     status.  batch == 0 or rows == 0 is an OK no-op (outputs untouched except
 *     that dk/dv rows, which then do not exist).
 */
#ifndef JFA_H_
#define JFA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  JFA_OK = 0,
  JFA_ERR_INVALID_ARGUMENT = 1,   /* null/misaligned pointer, negative size, bad scale, bad flag */
  JFA_ERR_UNSUPPORTED = 2,        /* head_dim not in {64,128}, broadcast_q together with causal */
  JFA_ERR_WORKSPACE_TOO_SMALL = 3,
  JFA_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} jfa_status_t;

/* Tile schedule used by the forward and backward kernels (process-wide).
 *   JFA_SCHED_SORTED_ZIGZAG  forward tiles sorted by KV work (descending) and dealt
 *                            boustrophedon across persistent workgroups; backward
 *                            valid (b, h, KV-block) tiles dealt round-robin ("Meta's
 *                            TLX attention kernel outpaces FlashAttention-4 on B200",
 *                            section "Five changes unlocked the gains", item 1).
 *   JFA_SCHED_IDENTITY       tiles in natural (b, block, h) order, dealt round-robin.
 *   JFA_SCHED_DYNAMIC        sorted tiles claimed through a device atomic counter by
 *                            whichever workgroup is free (the same section, item 2).
 *                            Default: on MI355X it was the fastest of the three on
 *                            every measured workload.
 * Results are independent of the schedule: O, LSE, dK and dV bit for bit, dQ up to
 * the order of its fp32 additions. */
typedef enum {
  JFA_SCHED_SORTED_ZIGZAG = 0,
  JFA_SCHED_IDENTITY = 1,
  JFA_SCHED_DYNAMIC = 2
} jfa_schedule_t;

/* Selects the schedule for subsequent calls from any thread.  Returns
 * JFA_ERR_INVALID_ARGUMENT for an unknown value. */
jfa_status_t jfa_set_schedule(int schedule);
int jfa_get_schedule(void);

/* Bytes of workspace jfa_fwd and jfa_fwd_mxfp8 need for these sizes (0 if the sizes
 * are invalid). */
size_t jfa_fwd_workspace_size(int64_t batch, int64_t num_heads, int64_t head_dim,
                              int64_t q_len, int64_t total_kv, int broadcast_q, int causal);

/* Bytes of workspace jfa_bwd needs for these sizes (0 if the sizes are invalid).
 * It holds the fp32 dQ accumulator (8 stripes of [Lq, H, D] in broadcast mode,
 * [T, H, D] in self mode), the row sums delta [H, rows] and the tile plan. */
size_t jfa_bwd_workspace_size(int64_t batch, int64_t num_heads, int64_t head_dim,
                              int64_t q_len, int64_t total_kv, int broadcast_q, int causal);

/* Forward pass: O = softmax(c Q K^T) V per sequence and head, and its LSE.
 * q_len is Lq (> 0) in broadcast mode and must be 0 in self mode.  softmax_scale
 * c must be finite and > 0. */
jfa_status_t jfa_fwd(const void* q, const void* k, const void* v,
                     const void* offsets, int offsets_is_int64,
                     int64_t batch, int64_t num_heads, int64_t head_dim,
                     int64_t q_len, int64_t total_kv,
                     int broadcast_q, int causal, float softmax_scale,
                     void* o, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Forward pass that allocates nothing, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Arguments, results and errors are those of jfa_fwd without the
 * workspace: the tile plan lives in a device array of JFA_FWD_NOALLOC_SCRATCH_BYTES
 * (2 MiB) inside the library, one copy per GPU, held until the process ends; its
 * address is looked up on the first call on each device.  A problem whose
 * jfa_fwd_workspace_size exceeds that size gives JFA_ERR_WORKSPACE_TOO_SMALL (2 MiB
 * hold about 131,000 plan items of 16 bytes: one per sequence in broadcast mode, one
 * per 128- or 256-row query tile of each sequence in self mode, plus one per
 * sequence).  Every call on a GPU uses that GPU's one copy and leaves its plan there:
 * calls that overlap on one GPU (on other streams or threads) race, so the caller
 * serialises them.  Each call's plan kernel rewrites every plan word it uses, the
 * work counter included, before the attention kernel reads them.  The call is not
 * timed by jfa_profile_enable (it creates no events). */
#define JFA_FWD_NOALLOC_SCRATCH_BYTES (2u << 20)
jfa_status_t jfa_fwd_noalloc(const void* q, const void* k, const void* v,
                             const void* offsets, int offsets_is_int64,
                             int64_t batch, int64_t num_heads, int64_t head_dim,
                             int64_t q_len, int64_t total_kv,
                             int broadcast_q, int causal, float softmax_scale,
                             void* o, float* lse, void* stream);

/* Backward pass: gradients of sum(O * dO) with respect to q, k and v, given the
 * o and lse that jfa_fwd returned for the same inputs.  In broadcast mode dq is
 * the sum over all sequences ("Meta's TLX attention kernel outpaces FlashAttention-4
 * on B200", section "GEM's sequences do not fit a fixed grid").  In self mode with
 * short sequences (block-diagonal attention in 64-token blocks, for instance), the
 * row sums dO . O of a sequence that fits one backward tile are formed from the
 * tile's own probabilities and its rows of o are not read ("Meta's TLX Block
 * Attention Beats Flash Attention v2 by 2.3x on Blackwell GPUs", section "One
 * Constraint, Five Eliminations"); o must still be a valid pointer to the whole
 * tensor.  Same size rules as jfa_fwd. */
jfa_status_t jfa_bwd(const void* q, const void* k, const void* v,
                     const void* offsets, int offsets_is_int64,
                     int64_t batch, int64_t num_heads, int64_t head_dim,
                     int64_t q_len, int64_t total_kv,
                     int broadcast_q, int causal, float softmax_scale,
                     const void* o, const float* lse, const void* d_o,
                     void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Backward pass with the rotary-embedding conjugate fused into its epilogues
 * ("Meta's TLX Block Attention Beats Flash Attention v2 by 2.3x on Blackwell GPUs",
 * section "The Rotary Fusion Bonus").  q and k are the rotated vectors the forward
 * attended with, q = R(pos_q) q0 and k = R(pos_k) k0, where R(p) rotates each pair
 * of elements (d, d + D/2), d < D/2, by the angle whose cosine and sine are
 * rope_cos[p * D/2 + d] and rope_sin[p * D/2 + d]:
 *   x'[d] = x[d] cos - x[d + D/2] sin,  x'[d + D/2] = x[d + D/2] cos + x[d] sin.
 * dq and dk receive the gradients with respect to q0 and k0: the conjugate
 * rotation R(p)^T applied in fp32 to the attention gradients before their bf16
 * rounding (dq after the batch sum in broadcast mode).  dv is as in jfa_bwd.
 *   rope_cos, rope_sin: fp32 device arrays [max_pos][D/2], 16-byte aligned;
 *   pos_q: int32 device array, one position per query row ([Lq] in broadcast mode,
 *          [T] in self mode); pos_k: int32 device array [T], one per key row;
 *   positions outside [0, max_pos) are clamped into it.
 * dq is rotated either in the fp32 dQ finalize or, for the sequences that take the
 * single-tile path of jfa_bwd (self mode, D = 128, 64-key tiles, sequences within
 * one tile), by the tiles before they store it.  Same workspace
 * (jfa_bwd_workspace_size), ownership and error rules as jfa_bwd; null tables or
 * positions, max_pos outside [1, 2^24] or misaligned tables give
 * JFA_ERR_INVALID_ARGUMENT. */
jfa_status_t jfa_bwd_rope(const void* q, const void* k, const void* v,
                          const void* offsets, int offsets_is_int64,
                          int64_t batch, int64_t num_heads, int64_t head_dim,
                          int64_t q_len, int64_t total_kv,
                          int broadcast_q, int causal, float softmax_scale,
                          const void* o, const float* lse, const void* d_o,
                          const float* rope_cos, const float* rope_sin,
                          const int32_t* pos_q, const int32_t* pos_k, int64_t max_pos,
                          void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Block sizes of the block-sparse top-k forward.  They are constants of the method
 * as this library defines it (the pages name query blocks and key/value blocks but
 * give no sizes); the kernels are built to them, not the other way round.
 *   JFA_SPARSE_KEY_BLOCK              keys per key/value block
 *   JFA_SPARSE_QUERY_BLOCK_BROADCAST  rows of the broadcast query per query block
 *   JFA_SPARSE_QUERY_BLOCK_SELF       rows of a sequence per query block (self mode) */
#define JFA_SPARSE_KEY_BLOCK 64
#define JFA_SPARSE_QUERY_BLOCK_BROADCAST 256
#define JFA_SPARSE_QUERY_BLOCK_SELF 128

/* Block-sparse top-k forward ("Meta's TLX attention kernel outpaces FlashAttention-4
 * on B200" and "Optimizing Jagged Flash Attention with TLX" name a
 * block-sparse fork of the kernel: a scoring step picks the top k key/value blocks
 * for each query block, and attention runs only over those blocks).  Non-causal
 * modes only (causal gives JFA_ERR_UNSUPPORTED).
 *   Key blocks: JFA_SPARSE_KEY_BLOCK (64) consecutive keys of a sequence (the last
 *     may be partial).
 *   Query blocks: JFA_SPARSE_QUERY_BLOCK_BROADCAST (256) consecutive rows of the
 *     broadcast query sequence, or JFA_SPARSE_QUERY_BLOCK_SELF (128) consecutive
 *     rows of the sequence itself in self mode (the last may be partial).
 *   Score of (query block, key block), per head: softmax_scale * (mean query row) .
 *     (mean key row), computed in fp32.
 *   Selection: the topk highest scores (ties to the lower block index); a sequence
 *     with topk or fewer key blocks keeps all of them.  topk must be in [1, 64].
 *     Key blocks past the 4096th of a sequence (262144 keys) are not candidates.
 *   o, lse: as jfa_fwd, with attention restricted to the keys of the selected blocks.
 *   blocks: optional (may be null) int32 output [num_heads][Q][topk] listing each
 *     query block's selection in ascending order, -1 padded, where
 *     Q = jfa_fwd_sparse_query_blocks(batch, q_len, total_kv, broadcast_q) and the
 *     query block of sequence b, block m is b * ceil(q_len / 256) + m (broadcast) or
 *     sum over b' < b of ceil(n_b' / 128), plus m (self mode), with the block sizes
 *     above.
 * Workspace: jfa_fwd_sparse_workspace_size(...) bytes (0 for invalid sizes or topk).
 * Other rules as jfa_fwd. */
size_t jfa_fwd_sparse_workspace_size(int64_t batch, int64_t num_heads, int64_t head_dim, int64_t q_len,
                                     int64_t total_kv, int broadcast_q, int topk);
int64_t jfa_fwd_sparse_query_blocks(int64_t batch, int64_t q_len, int64_t total_kv, int broadcast_q);
jfa_status_t jfa_fwd_sparse(const void* q, const void* k, const void* v,
                            const void* offsets, int offsets_is_int64,
                            int64_t batch, int64_t num_heads, int64_t head_dim,
                            int64_t q_len, int64_t total_kv, int broadcast_q,
                            float softmax_scale, int topk,
                            void* o, float* lse, int32_t* blocks,
                            void* workspace, size_t workspace_bytes, void* stream);

/* MXFP8 forward ("Meta's TLX attention kernel outpaces FlashAttention-4 on B200",
 * section on the kernel's variants: E4M3 values with one E8M0 scale per block).
 *
 * E4M3: OCP 8-bit float (bias 7, subnormals, largest 448, no infinities).  E8M0:
 * code c stands for 2^(c - 127).  A block is 32 elements along a product's
 * contraction axis; its scale is the smallest 2^e with max|x| <= 448 * 2^e (nothing
 * saturates), and each element is x / 2^e rounded to the nearest E4M3, ties to even.
 *
 * jfa_mxfp8_quantize_rows: Q or K rows.  x: bf16 [rows][num_heads][head_dim]
 *   (head_dim 64 or 128); values: uint8 E4M3, same shape; scales: uint8 E8M0
 *   [rows][num_heads][head_dim / 32], block c covering columns 32 c .. 32 c + 31.
 *   x and values 16-byte aligned.  Inputs must be finite (no NaN or infinity).
 *
 * jfa_mxfp8_v_blocks(batch, total_kv) = batch + ceil(total_kv / 32): the number of
 *   V blocks G that values and scales of jfa_mxfp8_quantize_v must hold.
 * jfa_mxfp8_quantize_v: V by key blocks.  v: bf16 [total_kv][num_heads][head_dim];
 *   offsets as jfa_fwd.  Block j of sequence b (keys 32 j .. 32 j + 31 of the
 *   sequence; the last block's missing keys are stored as zeros) has index
 *   g = b + floor(offsets[b] / 32) + j.  values: uint8 E4M3 [G][num_heads][head_dim][32],
 *   the 32 bytes of (g, h, d) holding key k of the block at byte
 *   16 * ((k >> 2) & 1) + 4 * (k >> 3) + (k & 3) (the matrix-core operand order);
 *   scales: uint8 E8M0 [G][num_heads][head_dim].  Entries at indices no block uses
 *   are left unwritten and never read.
 *
 * jfa_fwd_mxfp8: the forward on these operands (q8/q_scales from Q rows in the
 *   layout jfa_fwd takes Q: [q_len] or [total_kv] rows; k8/k_scales from K rows;
 *   v8/v_scales from jfa_mxfp8_quantize_v with the same offsets).  Both products
 *   run on the block-scaled matrix cores with fp32 accumulation.  Softmax in base 2
 *   with x = fp32(S) * fp32(softmax_scale * log2 e), the row maximum rounded up to
 *   an integer m, p = 2^(x - m) in fp32 and l = sum of p; P is quantized in blocks
 *   of 32 keys (aligned to the sequence start) by the same rule before the product
 *   with V, so O = (deq P)(deq V) / l in bf16 [rows][num_heads][head_dim], and
 *   LSE = ln 2 * (m + log2 l) in fp32 [num_heads][rows] (-inf for a row with no
 *   keys, whose O is zero).  q8, k8, v8, v_scales, o and workspace
 *   must be 16-byte aligned, k_scales aligned to head_dim / 32 bytes.  Modes,
 *   offsets, sizes, workspace (jfa_fwd_workspace_size with the same sizes) and errors
 *   as jfa_fwd.
 * Profile names: "mx_quantize_rows", "mx_quantize_v", "plan_fwd", "fwd_mxfp8". */
int64_t jfa_mxfp8_v_blocks(int64_t batch, int64_t total_kv);
jfa_status_t jfa_mxfp8_quantize_rows(const void* x, int64_t rows, int64_t num_heads, int64_t head_dim,
                                     void* values, void* scales, void* stream);
jfa_status_t jfa_mxfp8_quantize_v(const void* v, const void* offsets, int offsets_is_int64,
                                  int64_t batch, int64_t num_heads, int64_t head_dim, int64_t total_kv,
                                  void* values, void* scales, void* stream);
jfa_status_t jfa_fwd_mxfp8(const void* q8, const void* q_scales, const void* k8, const void* k_scales,
                           const void* v8, const void* v_scales,
                           const void* offsets, int offsets_is_int64,
                           int64_t batch, int64_t num_heads, int64_t head_dim,
                           int64_t q_len, int64_t total_kv, int broadcast_q, int causal,
                           float softmax_scale, void* o, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Measurement support.  While enabled on a thread, every kernel this library
 * launches from that thread is bracketed by two HIP events recorded on the
 * launch stream (events are created on first use and reused).  Kernel names:
 * "plan_fwd", "fwd", "bwd_pre", "plan_bwd", "bwd", "dq_finalize", and for the
 * block-sparse forward "plan_sparse", "sparse_select", "fwd_sparse". */
jfa_status_t jfa_profile_enable(int enable);

/* Waits for the recorded launches of this thread, then writes per-kernel totals:
 * for entry i < max_entries, names[i * name_len ...] (NUL-terminated, truncated),
 * total_ms[i] (sum of event-measured durations) and launches[i].  *count receives
 * the number of distinct kernels seen.  The record is cleared.  Returns
 * JFA_ERR_HIP if an event query fails. */
jfa_status_t jfa_profile_read(char* names, int name_len, double* total_ms, int64_t* launches,
                              int max_entries, int* count);

/* Thread-local, NUL-terminated description of the last non-OK status returned
 * on this thread ("" if none).  Owned by the library; valid until the next call. */
const char* jfa_last_error(void);

/* Library version string, e.g. "jfa 0.1 gfx950". */
const char* jfa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* JFA_H_ */
