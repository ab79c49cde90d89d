/*
 * verify_attn.h - C ABI of the MI355X (gfx950) MLA tree-verify attention library.
 *
 * The operation (sources by page title and section):
 *   Multi-head latent attention for verifying a speculative draft tree. Every draft-tree
 *   query token, for every head, attends over a paged latent KV cache reached through slot
 *   indices, under a mask made of a prefix length plus a tree visibility matrix, and returns
 *   a 512-wide latent output row.
 *   - absorbed q [num_tok, H, 576] and paged KV [num_slots, 576] = 512 latent + 64 rope:
 *     "The Glue That Binds: Wiring a Custom CUDA Kernel into Production via C-ABI",
 *     section "The Broader Engineering Effort";
 *   - the latent kv_c is one 512-d vector per token shared by every head:
 *     "The Glue That Connects: Wiring a Custom Flash Attention Kernel into the C-ABI Layer",
 *     section "The Context: Building a Blackwell-Specific Verify Attention Kernel";
 *   - prefix-length-plus-visibility mask, split-K flash decode, paged reads by slot:
 *     "The Glue That Makes Kernels Run: A Study in Architectural Discipline",
 *     section "The Context: A Custom Kernel in Flight";
 *   - the mask indexed by the global key position, masked scores -inf:
 *     "The Glue That Connects", section "Design Decisions and Trade-Offs";
 *   - buffer dtypes (int64 kv_indices / qo_indptr / mask_indptr / out_cache_loc, int32
 *     kv_indptr, uint8 custom_mask), scalars bs, q_len, H, Dl, Dr, scale and a fixed split
 *     count, a caller workspace, no host synchronisation or allocation inside the call:
 *     "The Final Solder Joint: Updating the C-ABI Layer for CUDA Graph Capture-Safety",
 *     sections "The Investigation", "The Three-Edits Sequence", "Why the C-ABI Edit Matters"
 *     and "Assumptions and Design Decisions".
 *
 * Per request r with T_r = qo_indptr[r+1]-qo_indptr[r] tree tokens, tree token i, head h.
 * The key slots come in one of two layouts:
 *   - out_cache_loc == NULL: L_r = kv_indptr[r+1]-kv_indptr[r] keys, P_r = L_r - T_r, key j
 *     (0 <= j < L_r) in slot kv_indices[kv_indptr[r] + j]; the last T_r keys are the tree
 *     tokens in query order;
 *   - out_cache_loc != NULL: kv_indices[kv_indptr[r] ..] holds the P_r = kv_indptr[r+1]-
 *     kv_indptr[r] prefix slots only and tree key P_r + k is in slot
 *     out_cache_loc[qo_indptr[r] + k]; L_r = P_r + T_r. (Prefix slots from kv_indices, new
 *     tokens' slots from out_cache_loc, told apart by the kv_indptr offsets: "The Final
 *     Solder Joint", section "The Three-Edits Sequence".)
 *   key j is visible iff j < P_r or
 *   custom_mask[mask_indptr[r] + i*L_r + j] != 0 (prefix columns are ignored: a kernel may
 *   read them but never uses their value);
 *   s_j = sm_scale * <q[t,h,0:576], kv[slot_j,0:576]>,  t = qo_indptr[r] + i;
 *   out[t,h,0:512] = sum_j softmax(s)_j * kv[slot_j, 0:512] over the visible keys;
 *   out_lse[t,h] = natural-log sum-exp of the visible s_j;
 *   out_argmax[t,h] = the smallest visible key position j with the largest s_j.
 *   A row with no visible key gets out = 0, lse = -inf, argmax = -1.
 *
 * Arithmetic: fp32 inputs run in fp32 throughout (the simple kernel). bf16 inputs run on
 *   the matrix cores: scores from bf16 products accumulated in fp32; P rounded to fp16
 *   (nearest even) and the value dims converted from bf16 to fp16 with round-toward-zero for
 *   the P.V products, accumulated in fp32, with the denominator summed from the rounded P;
 *   each key split's normalised partial stored as 16-bit codes with one scale per 128 dims
 *   (one code step is 1/32767 of that group's largest value). The output error is thus
 *   relative to the magnitude of the value rows: a small multiple of 2^-11 of the largest
 *   visible value at worst, far less where the rounding errors average out.
 *   Value range (bf16 inputs): the fp16 conversion is exact for 2^-14 <= |v| <= 65280 (every
 *   bf16 value in fp16's normal range); below 2^-14 it truncates to an fp16 subnormal
 *   (absolute error under 2^-24); |v| >= 65536 saturates to +-65504. PRECONDITION: the
 *   latent dims (0..511) of every visible key row satisfy |v| <= 65280; larger values are
 *   not detected, they saturate. The score dims (all 576) have no such limit.
 *
 * Conventions
 *   Ownership: every tensor argument is caller-owned device memory. The library owns the
 *     context and, only when the config brings no workspace, a workspace it allocates in
 *     verify_attn_create (outside any stream capture) and frees in verify_attn_destroy.
 *   Errors: functions return va_status; no exception or abort crosses the ABI. The message
 *     of the last failure on the calling thread is verify_attn_last_error(). (The C-ABI
 *     layer's job of type marshalling and error codes between the kernels and their
 *     callers: "The Glue That Makes Kernels Run: A Study in Architectural Discipline",
 *     section "The Subject Message: Why It Was Written"; "The Glue That Connects", section
 *     "What the Edit Actually Does".)
 *   Bad device data (a slot outside [0, num_slots), L_r < T_r, T_r above max_q_per_req,
 *     offsets outside the buffers) never leads to an out-of-bounds access: the offending
 *     key is treated as invisible or the request's rows are written as empty rows, and a
 *     sticky bit is set in a status word read by verify_attn_read_device_status.
 *   Capture: verify_attn_run only enqueues kernels on `stream`; it allocates nothing,
 *     copies nothing and never synchronises, so it may be recorded into a hipGraph. The
 *     grid depends only on bs and the context's fixed configuration.
 *   Concurrency: calls on one context must not overlap in time (the workspace is shared);
 *     use one context per concurrently used stream.
 *   Streams are passed as `void*` holding a hipStream_t (NULL = the default stream).
 */
#ifndef VERIFY_ATTN_H
#define VERIFY_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct verify_attn_ctx verify_attn_ctx;

typedef enum {
  VA_OK = 0,
  VA_ERR_NULL = 1,        /* a required pointer is NULL                                   */
  VA_ERR_INVALID = 2,     /* a scalar is out of range or inconsistent with the config      */
  VA_ERR_UNSUPPORTED = 3, /* a valid request the library does not implement              */
  VA_ERR_WORKSPACE = 4,   /* the caller's workspace is too small or misaligned            */
  VA_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed                   */
} va_status;

/* element types of q and kv_buffer (in_dtype) and of out (out_dtype) */
enum { VA_BF16 = 0, VA_FP32 = 1 };

/* kernel family: AUTO picks MFMA for bf16 inputs and the simple fp32 kernel otherwise */
enum { VA_KERNEL_AUTO = 0, VA_KERNEL_SIMPLE = 1, VA_KERNEL_MFMA = 2 };

/* sticky device status bits (verify_attn_read_device_status) */
enum {
  VA_DEV_SLOT_RANGE = 1u,  /* a kv_indices entry outside [0, num_slots): key ignored        */
  VA_DEV_SEGMENT = 2u,     /* L_r < T_r, offsets outside kv_indices / mask / q, or a request
                              whose mask segment T_r*L_r reaches 2^31 bytes: rows empty */
  VA_DEV_Q_PER_REQ = 4u,   /* T_r > max_q_per_req: the request's rows written empty         */
  VA_DEV_TOKENS = 8u,      /* qo_indptr[bs] != num_tokens: uncovered rows written empty     */
  VA_DEV_TREE = 16u        /* a tree parent index that does not precede its child (-1: root)
                              (verify_attn_build_mask, verify_attn_accept)                  */
};

typedef struct {
  int32_t num_heads;      /* H >= 1                                                        */
  int32_t latent_dim;     /* Dl: must be 512                                               */
  int32_t rope_dim;       /* Dr: must be 64                                                */
  int32_t in_dtype;       /* VA_BF16 or VA_FP32 (q and kv_buffer)                          */
  int32_t out_dtype;      /* VA_FP32 or VA_BF16 (out)                                      */
  int32_t max_batch;      /* upper bound on bs                                             */
  int32_t max_q_per_req;  /* upper bound on T_r                                            */
  int64_t max_q_tokens;   /* upper bound on num_tokens                                     */
  int32_t num_splits;     /* key splits per request (1..256): each request's keys are cut
                             into that many splits (fewer if it has fewer 32-key tiles);
                             0 = MFMA kernel: chosen on the device at every call, one common
                             split length for the whole batch so that it has at most one work
                             item per compute unit (one per row tile when the batch has more
                             row tiles than that); simple kernel: chosen from the bounds     */
  int32_t kernel;         /* VA_KERNEL_*                                                   */
  void *workspace;        /* device memory, 256-byte aligned, or NULL: allocated at create.
                             Owned by the context until verify_attn_destroy: the caller must
                             not write it (its first bytes are set once, at create) */
  size_t workspace_bytes; /* size of `workspace` when it is not NULL                        */
} verify_attn_config;

typedef struct {
  int32_t kernel;         /* the kernel family actually used                              */
  int32_t num_splits;     /* the split count fixed for the context's life; 0 when the MFMA
                             kernel balances the splits on the device at every call         */
  int32_t rows_per_block; /* (token, head) rows handled by one partial workgroup           */
  int32_t row_tiles_per_req; /* row tiles a request can have (ceil(max_q_per_req*H / rows)) */
  size_t workspace_bytes; /* bytes of workspace in use                                     */
  int32_t partial_waves;  /* wavefronts per partial workgroup: 8 (two per SIMD: four hold the
                             query rows and compute scores and softmax, four hold most of the
                             output accumulators and stage the key tiles) for the MFMA kernel
                             when num_heads is a multiple of 64 (no work item then has 32
                             rows or fewer), else 4                                         */
} verify_attn_info;

/* Workspace bytes a config needs (0 if the config is invalid): per partial row about 1052
 * bytes for the MFMA kernel (512 16-bit codes, 4 group scales, 3 scalars) and about 2076 for
 * the fp32 kernel (512 floats, the same 7 words), with (128 * CUs + max_q_tokens * H) partial
 * rows for the MFMA kernel with num_splits = 0 (CUs = the current device's compute units
 * rounded up to a multiple of 8 and capped at 256; 256 when no device answers) and
 * num_splits * max_q_tokens * H otherwise, plus 16 bytes per output row. */
size_t verify_attn_workspace_bytes(const verify_attn_config *cfg);

/* Validates `cfg`, binds or allocates the workspace, clears its status words and a row of
 * zeros the kernels read in place of unusable key rows (synchronously, on the null stream).
 * Returns VA_OK and sets *out, or an error and leaves *out NULL. */
va_status verify_attn_create(const verify_attn_config *cfg, verify_attn_ctx **out);

/*
 * Enqueues one verify step on `stream`.
 *   q            [num_tokens, H, 576] in_dtype, contiguous.
 *   kv_buffer    [num_slots, 576] in_dtype, contiguous rows (the paged latent cache).
 *   kv_indices   int64 [num_kv_indices]: per request its L_r slots (prefix, then the tree
 *                tokens), or only its P_r prefix slots when out_cache_loc is given.
 *   kv_indptr    int32 [bs+1], non-decreasing, kv_indptr[bs] <= num_kv_indices.
 *   qo_indptr    int64 [bs+1], non-decreasing, qo_indptr[bs] == num_tokens.
 *   custom_mask  uint8 [mask_len]: request r's [T_r, L_r] row-major matrix at mask_indptr[r].
 *   mask_indptr  int64 [bs+1] element offsets into custom_mask.
 *   out_cache_loc NULL, or int64 [num_tokens]: the slot of every tree token (see above).
 *   out          [num_tokens, H, 512] out_dtype.
 *   out_lse      nullable float [num_tokens, H].
 *   out_argmax   nullable int32 [num_tokens, H].
 * Host-checked: pointers, 0 <= bs <= max_batch, 0 <= num_tokens <= max_q_tokens,
 * 0 < sm_scale < inf, num_slots >= 1. Returns VA_ERR_HIP if a launch fails.
 */
va_status verify_attn_run(verify_attn_ctx *ctx, const void *q, const void *kv_buffer,
                          int64_t num_slots, const int64_t *kv_indices, int64_t num_kv_indices,
                          const int32_t *kv_indptr, const int64_t *qo_indptr,
                          const uint8_t *custom_mask, int64_t mask_len,
                          const int64_t *mask_indptr, const int64_t *out_cache_loc, int32_t bs,
                          int64_t num_tokens, float sm_scale, void *out, float *out_lse,
                          int32_t *out_argmax, void *stream);

/*
 * Allocation-free variant of verify_attn_run, for callers that cannot allocate device memory:
 * code under stream capture, tight serving loops, harnesses that forbid allocation. It takes
 * the configuration instead of a context and, as its workspace, a static device scratch array
 * of the library: 64 MiB on each GPU it runs on, part of the code object, held until the
 * process ends. It calls no allocation routine. The tensor arguments, outputs, host checks and
 * semantics are those of verify_attn_run; cfg->workspace must be NULL (else VA_ERR_INVALID).
 * Limit: verify_attn_workspace_bytes(cfg) must be at most 64 MiB, else VA_ERR_WORKSPACE before
 * any device work (with num_splits = 0 on a 256-CU GPU: max_q_tokens up to 477 at H=64, up
 * to 3819 at H=8). The first call on a device looks the array's address up and clears its header
 * with a kernel on `stream` (capturable). Every call on one GPU shares that GPU's array and
 * leaves its contents behind, so calls that overlap in time on one GPU race: serialise them
 * (one stream) or use contexts. Bad index data is handled as verify_attn_run handles it (keys
 * ignored, rows emptied), but this path has no status read.
 */
va_status verify_attn_run_static(const verify_attn_config *cfg, const void *q,
                                 const void *kv_buffer, int64_t num_slots,
                                 const int64_t *kv_indices, int64_t num_kv_indices,
                                 const int32_t *kv_indptr, const int64_t *qo_indptr,
                                 const uint8_t *custom_mask, int64_t mask_len,
                                 const int64_t *mask_indptr, const int64_t *out_cache_loc,
                                 int32_t bs, int64_t num_tokens, float sm_scale, void *out,
                                 float *out_lse, int32_t *out_argmax, void *stream);

/* Synchronises `stream`, returns the sticky VA_DEV_* bits in *flags and clears them.
 * Never call it inside a stream capture. The hot path itself never synchronises or copies to
 * the host ("The Final Solder Joint", sections "The Capture-Safety Constraint" and "Why the
 * C-ABI Edit Matters"), so bad index data is reported through this separate, synchronising
 * call rather than by verify_attn_run. Errors: VA_ERR_NULL, VA_ERR_HIP. */
va_status verify_attn_read_device_status(verify_attn_ctx *ctx, void *stream, uint32_t *flags);

/* Profiling: when set (non-NULL hipEvent_t handles passed as void*), every later
 * verify_attn_run records `before` ahead of the partial kernel, `between` after it and
 * `after` after the combine kernel, on the run's stream. `after` may be NULL with the other
 * two set: a caller timing back-to-back runs then takes the next run's `before` (or an event
 * of its own after the last run) as the end of this one, one event fewer per run. Pass NULLs
 * to stop. Any other combination fails with VA_ERR_INVALID. Not for use while the stream is
 * being captured. */
va_status verify_attn_set_profiling_events(verify_attn_ctx *ctx, void *before, void *between,
                                           void *after);

/* Reports the fixed launch configuration of a context. */
va_status verify_attn_get_info(const verify_attn_ctx *ctx, verify_attn_info *info);

/*
 * Builds the verify mask from the draft trees on `stream` (capture-safe: kernels only). The
 * mask is rebuilt from the tree structure ("The Glue That Binds", section "The Thinking
 * Process"), in the layout verify_attn_run reads.
 *   parents      int64 [num_tokens]: for tree token t of request r (node i = t - qo_indptr[r]),
 *                the node index of its parent within the request, -1 for a root. A parent must
 *                precede its child; one that does not sets VA_DEV_TREE and ends that node's
 *                ancestor chain there.
 *   qo_indptr    int64 [bs+1]; kv_indptr int32 [bs+1]: as for verify_attn_run, with
 *                split_layout != 0 meaning kv_indptr counts prefix keys only (tree slots in
 *                out_cache_loc), so that L_r = P_r + T_r.
 *   custom_mask  uint8 [mask_len]: request r's [T_r, L_r] row-major matrix at mask_indptr[r];
 *                row i gets 1 in every prefix column j < P_r and, in column P_r + k, 1 iff
 *                node k is node i or one of its ancestors. Rows whose segment does not fit
 *                mask_len (or whose request is malformed) are left unwritten and set
 *                VA_DEV_SEGMENT.
 *   mask_indptr  int64 [bs+1]: read, or first written as the running sum of T_r * L_r from 0
 *                when write_mask_indptr != 0.
 * Host-checked: ctx, 0 <= bs <= max_batch, 0 <= num_tokens <= max_q_tokens, the context's
 * max_q_per_req <= 2048 (else VA_ERR_UNSUPPORTED), pointers when bs > 0.
 */
va_status verify_attn_build_mask(verify_attn_ctx *ctx, const int64_t *parents,
                                 const int64_t *qo_indptr, const int32_t *kv_indptr,
                                 int32_t split_layout, int32_t bs, int64_t num_tokens,
                                 uint8_t *custom_mask, int64_t mask_len, int64_t *mask_indptr,
                                 int32_t write_mask_indptr, void *stream);

/*
 * Greedy acceptance of the verified trees on `stream` (capture-safe). The library exposes tree
 * acceptance next to verify attention ("The Glue That Connects", section "What the Edit
 * Actually Does"); no algorithm is given there, so this is the plain greedy rule: node 0 of each
 * request is the root (the last accepted token); from it, the walk moves to the lowest-indexed
 * child whose draft token equals the target's token at the current node, until none matches.
 *   parents        int64 [num_tokens], as for verify_attn_build_mask.
 *   draft_tokens   int64 [num_tokens]: the token each tree node proposes.
 *   target_tokens  int64 [num_tokens]: the target model's token at each tree node (its argmax
 *                  after the model head).
 *   accept_len     int32 [bs]: accepted draft nodes (the path without the root).
 *   accept_path    int64 [bs, max_path]: the path's node indices, root first, -1 after it
 *                  (truncated to max_path).
 *   next_token     int64 [bs]: the target's token at the last node of the path.
 * A request without tree tokens gets 0, an all -1 path and -1; a malformed request sets
 * VA_DEV_SEGMENT and gets the same. A parent that does not precede its child sets VA_DEV_TREE;
 * that request's output is then unspecified (but every write stays in its rows).
 * Host-checked: ctx, 0 <= bs <= max_batch, 0 <= num_tokens <= max_q_tokens, max_path >= 1,
 * max_q_per_req <= 2048, pointers when bs > 0.
 */
va_status verify_attn_accept(verify_attn_ctx *ctx, const int64_t *parents,
                             const int64_t *draft_tokens, const int64_t *target_tokens,
                             const int64_t *qo_indptr, int32_t bs, int64_t num_tokens,
                             int32_t *accept_len, int64_t *accept_path, int32_t max_path,
                             int64_t *next_token, void *stream);

/* Frees the context and any workspace it allocated. NULL is a no-op. */
void verify_attn_destroy(verify_attn_ctx *ctx);

/* Message of the last failed call on this thread ("" if none; cleared by a successful call).
 * Thread-local, owned by the library, valid until the thread's next call. The error-code
 * convention it completes is cited under "Errors" above. */
const char *verify_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VERIFY_ATTN_H */
