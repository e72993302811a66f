/*
 * psb.h — packed-sequence block-diagonal attention for MI355X (gfx950).
 *
 * C ABI of the library libpsb.so.  Plain pointers and sizes only.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Device pointers point to memory the CALLER allocated (any HIP allocation on
 *   the current device); the library never allocates, frees or keeps device
 *   memory between calls.  Host pointers are read during the call only.
 * - `stream` is a hipStream_t (NULL = the legacy default stream).  Every call
 *   enqueues its kernels on that stream and returns without synchronizing; the
 *   outputs are valid once the stream reaches that point.  Calls are reentrant.
 * - The return value is a psb_status.  Argument errors are detected on the host
 *   before anything is enqueued (nothing is launched, no device memory is
 *   touched).  Errors that depend on device data are reported through the
 *   optional device word `status_word` (bits OR-ed in by the kernels; the caller
 *   zeroes it beforehand and reads it after synchronizing).
 * - Document ids are int32.  The padding id is -1000 (PSB_PAD_DOC_ID).
 *
 * Sources: the "nemo_automodel.components.models.glm5_next.cp" page (API
 * entries doc_ids_from_cu_seqlens and segment_cu_seqlens) and the
 * "nemo_automodel.components.distributed.blockdiag_cp" page (package overview;
 * cp_blockdiag_sdpa; BlockdiagCpModelState.packed_cu_seqlens).
 */
#ifndef PSB_H_
#define PSB_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t psb_status;

#define PSB_OK 0
#define PSB_ERR_INVALID_ARG (-1) /* null pointer, negative size, bad scale, ... */
#define PSB_ERR_SHAPE (-2)       /* inconsistent shapes / strides / shard range */
#define PSB_ERR_UNSUPPORTED (-3) /* head dim other than 64 or 128 */
#define PSB_ERR_CAPACITY (-4)    /* output or workspace buffer too small */
#define PSB_ERR_HIP (-5)         /* a HIP runtime call failed (e.g. launch) */
#define PSB_ERR_SCRATCH_LIMIT (-6) /* no-allocation call: plan tables exceed its static buffer */

#define PSB_PAD_DOC_ID (-1000)

/* Bits OR-ed into `status_word` by the kernels. */
#define PSB_DATA_CU_NOT_MONOTONE 1   /* cu_seqlens decreases somewhere */
#define PSB_DATA_CU_OUT_OF_RANGE 2   /* cu_seqlens[0] < 0 or cu_seqlens[N] > seq_len */
#define PSB_DATA_DOC_NOT_CONTIGUOUS 4 /* a non-padding id occurs in two separate runs of a row */
#define PSB_DATA_LENS_EXCEED_SEQ 8    /* document lengths of a row add up past seq_len */
#define PSB_DATA_BAD_POSITIONS 16     /* logical positions break the document rule */
#define PSB_DATA_BAD_LENGTHS 32       /* a real document length is negative or above its padded length */
#define PSB_DATA_KV_WINDOW 64         /* a query needs a key before the delivered key window */

/* Human-readable message for a status code (static storage, never NULL). */
const char* psb_status_string(psb_status status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t psb_version(void);

/*
 * Document ids from cumulative document boundaries (glm5_next.cp page,
 * doc_ids_from_cu_seqlens: boundaries -> ids [1, sequence]).
 *
 *   cu_seqlens   device, int32 [n_docs + 1]: document i covers
 *                positions [cu_seqlens[i], cu_seqlens[i+1]).
 *   n_docs       number of documents (>= 0).
 *   seq_len      row length S (>= 0).
 *   doc_ids_out  device, int32 [seq_len]: one row of the [1, S] result.
 *                Position p gets i + 1 for the document i covering it, and -1000
 *                when no document covers it.
 *   status_word  device int32 or NULL: PSB_DATA_CU_NOT_MONOTONE /
 *                PSB_DATA_CU_OUT_OF_RANGE are OR-ed in when cu_seqlens is not
 *                non-decreasing within [0, seq_len]; doc_ids_out is then
 *                unspecified.
 */
psb_status psb_doc_ids_from_cu_seqlens(const int32_t* cu_seqlens, int64_t n_docs, int64_t seq_len,
                                       int32_t* doc_ids_out, int32_t* status_word, void* stream);

/*
 * Document ids from per-document lengths (glm5_next.cp page,
 * doc_ids_from_seq_lens: lengths [batch, documents] -> ids [batch, sequence];
 * the inkling2 context_parallel page's unpack_row_layout pads such length tables
 * with -1000).
 *
 *   seq_lens       device int32 [B, n_docs], contiguous.  In each row the lengths
 *                  up to the first negative entry are documents (0 allowed: the
 *                  document takes an id and covers nothing).
 *   seq_len        row length S of the output.
 *   padding_value  id of positions no document covers (the page's default: -1000).
 *   doc_ids_out    device int32 [B, seq_len], contiguous: the j-th document of a row
 *                  covers the next seq_lens[b, j] positions with id j + 1.
 *   status_word    device int32 or NULL: PSB_DATA_LENS_EXCEED_SEQ is OR-ed in when a
 *                  row's lengths add up past seq_len (the output is then unspecified).
 * n_docs > 4096 returns PSB_ERR_UNSUPPORTED; B > 65535 PSB_ERR_SHAPE.
 */
psb_status psb_doc_ids_from_seq_lens(const int32_t* seq_lens, int64_t B, int64_t n_docs, int64_t seq_len,
                                     int32_t padding_value, int32_t* doc_ids_out, int32_t* status_word,
                                     void* stream);

/*
 * Padding mask and document positions of packed rows from their length tables
 * (inkling2 context_parallel page, unpack_row_layout: the packer's real and padded
 * lengths [batch, documents], padded with -1000, decide padding; token ids never do).
 *
 *   seq_lens, seq_lens_padded  device int32 [B, n_docs], contiguous.  A row's
 *                    documents are the entries before its first negative padded
 *                    length; document j takes the next seq_lens_padded[b, j]
 *                    positions, of which the first seq_lens[b, j] are real tokens.
 *   padding_mask_out device uint8 [B, seq_len], contiguous: 0 for a real token, 1 for
 *                    padding (inside a document's padded block or past the last one).
 *   position_ids_out device int32 [B, seq_len], contiguous: a real token's offset in
 *                    its document (0, 1, ...); 0 at padding.
 *   status_word      device int32 or NULL: PSB_DATA_BAD_LENGTHS is OR-ed in when some
 *                    0 <= seq_lens[b, j] <= seq_lens_padded[b, j] fails,
 *                    PSB_DATA_LENS_EXCEED_SEQ when a row's padded lengths add up past
 *                    seq_len (the outputs are then unspecified).
 * The caller owns every buffer.  n_docs > 4096 returns PSB_ERR_UNSUPPORTED; B > 65535
 * PSB_ERR_SHAPE; B == 0 or seq_len == 0 enqueues nothing.
 */
psb_status psb_unpack_row_layout(const int32_t* seq_lens, const int32_t* seq_lens_padded, int64_t B, int64_t n_docs,
                                 int64_t seq_len, uint8_t* padding_mask_out, int32_t* position_ids_out,
                                 int32_t* status_word, void* stream);

/*
 * Checks logical positions against the document rule (inkling2 context_parallel
 * page, validate_document_positions): inside a document positions grow by one, a
 * new document starts at 0, a gap never resumes an earlier document, and the first
 * kept token of a row may carry any non-negative offset (a shard can start inside a
 * document).  For the kept tokens of each row in order: the first >= 0; one right
 * after a kept token equals the previous + 1 or 0; one after dropped tokens equals 0.
 *
 *   keep         device uint8 [B, S] (0 = dropped), contiguous.
 *   positions    device int32 [B, S], contiguous.
 *   status_word  device int32, required: PSB_DATA_BAD_POSITIONS is OR-ed in when a
 *                row breaks the rule.  Diagnostic, not on the hot path.
 */
psb_status psb_validate_document_positions(const uint8_t* keep, const int32_t* positions, int64_t B, int64_t S,
                                           int32_t* status_word, void* stream);

/*
 * Boundaries of the maximal runs of equal document ids of one row, padding runs
 * included (glm5_next.cp page, segment_cu_seqlens: run boundaries covering the
 * full row).
 *
 *   doc_ids_row     device, int32 [seq_len].
 *   cu_out          device, int32 [cu_capacity]; receives [0, run starts..., seq_len]
 *                   (R + 1 entries for R runs; just [0] when seq_len == 0).
 *   cu_capacity     must be >= seq_len + 1 (the worst case), else PSB_ERR_CAPACITY.
 *   n_segments_out  device int32 scalar; receives R.
 */
psb_status psb_segment_cu_seqlens(const int32_t* doc_ids_row, int64_t seq_len, int32_t* cu_out,
                                  int64_t cu_capacity, int32_t* n_segments_out, void* stream);

/*
 * Checks the precondition blockdiag_attn_fwd relies on: in every row of
 * doc_ids [B, S] (row stride `row_stride` elements), each non-padding id forms
 * one contiguous run (inkling2 context_parallel page, validate_document_positions:
 * a gap never resumes an earlier document).  ORs PSB_DATA_DOC_NOT_CONTIGUOUS
 * into status_word (required here) when violated.  Diagnostic, not on the hot path.
 */
psb_status psb_validate_doc_ids(const int32_t* doc_ids, int64_t B, int64_t S, int64_t row_stride,
                                int32_t* status_word, void* stream);

/* Bytes of device workspace psb_blockdiag_attn_fwd needs for this problem. */
size_t psb_blockdiag_attn_fwd_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                                             int64_t D);

/*
 * Block-diagonal (per-document causal) attention forward (blockdiag_cp page:
 * package overview — a packed row needs a causal mask per document; and
 * cp_blockdiag_sdpa — the local queries run against the delivered keys with a
 * per-document causal mask rebuilt from the document ids; scale defaults to
 * D**-0.5; enable_gqa as in PyTorch sdpa; output [B, Hq, L, D] for the local rows).
 *
 * The query at local row i of batch b is global position qpos = seq_start + i.
 * It attends to key k iff doc_ids[b,k] == doc_ids[b,qpos], doc_ids[b,qpos] != -1000
 * and k <= qpos.  A query with no allowed key (a padding query) outputs 0.
 *
 *   q            device bf16 [B, Hq, L, D]   (strides q_strides, elements; D contiguous)
 *   k, v         device bf16 [B, Hkv, S, D]  (strides kv_strides, shared by k and v)
 *   doc_ids      device int32 [B, S], contiguous.  Precondition: each non-padding
 *                id forms one contiguous run per row (psb_validate_doc_ids checks it).
 *   q_strides    host int64[3] = strides of (B, H, seq) in elements, or NULL for
 *                contiguous [B, Hq, L, D]; kv_strides likewise for k and v.
 *   seq_start    global position of local row 0; 0 <= seq_start, seq_start + L <= S.
 *   scale        softmax scale (finite, any sign; callers pass D**-0.5 for the default).
 *                0 and -0 weigh every allowed key equally (each row is the mean of v
 *                over its document prefix).
 *   enable_gqa   non-zero: query head h reads kv head h / (Hq / Hkv) (Hq % Hkv == 0).
 *                Zero: requires Hq == Hkv, else PSB_ERR_SHAPE.
 *   out          device bf16 [B, Hq, L, D], contiguous; must not alias q, k or v.
 *   workspace    device, >= psb_blockdiag_attn_fwd_workspace_size(...) bytes,
 *                16-byte aligned (scheduler tables; contents need no initialisation).
 *   status_word  device int32 or NULL.  When non-NULL the call also enqueues the check of
 *                the doc_ids precondition (one extra launch after the attention kernel)
 *                and ORs PSB_DATA_DOC_NOT_CONTIGUOUS into the word when a non-padding id
 *                occurs in two separate runs of a row; the output is then unspecified.
 *                NULL skips the check.
 *
 * D must be 64 or 128 (else PSB_ERR_UNSUPPORTED).  Empty problems (B, Hq, L == 0)
 * enqueue nothing and return PSB_OK.
 */
psb_status psb_blockdiag_attn_fwd(const void* q, const void* k, const void* v,
                                  const int32_t* doc_ids, int64_t B, int64_t Hq, int64_t Hkv,
                                  int64_t L, int64_t S, int64_t D, const int64_t* q_strides,
                                  const int64_t* kv_strides, int64_t seq_start, float scale,
                                  int32_t enable_gqa, void* out, void* workspace,
                                  size_t workspace_bytes, int32_t* status_word, void* stream);

/*
 * psb_blockdiag_attn_fwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the scheduler tables live in a static device array of the library, one per
 * GPU, of psb_blockdiag_attn_fwd_noalloc_max_workspace() bytes (4 MiB), held until the
 * process ends.  The call allocates and frees nothing.
 *
 * Arguments, outputs, status_word and errors as in psb_blockdiag_attn_fwd (the stream must
 * belong to the current device), plus PSB_ERR_SCRATCH_LIMIT, returned before anything is
 * enqueued, when the problem's tables need more than the static array holds, i.e. when
 * psb_blockdiag_attn_fwd_workspace_size(B, Hq, Hkv, L, D) exceeds it (about
 * 4 MiB / 72 bytes = 58000 32-row query blocks over all rows; B * L up to 1.8M rows).
 * Every call on one GPU uses that GPU's array: calls that overlap in time on one GPU
 * (on different streams or from different threads without ordering) race and give
 * wrong outputs.  The array needs no clearing: each call's plan rewrites every entry the
 * attention kernel reads.
 */
size_t psb_blockdiag_attn_fwd_noalloc_max_workspace(void);
psb_status psb_blockdiag_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                          const int32_t* doc_ids, int64_t B, int64_t Hq, int64_t Hkv,
                                          int64_t L, int64_t S, int64_t D, const int64_t* q_strides,
                                          const int64_t* kv_strides, int64_t seq_start, float scale,
                                          int32_t enable_gqa, void* out, int32_t* status_word, void* stream);

/*
 * The two halves of psb_blockdiag_attn_fwd, for callers that run many
 * attention calls over one document layout (every layer of a model step shares
 * doc_ids): plan once, then run per layer.  The package overview of the
 * blockdiag_cp page lists "varlen metadata precompute" as the internal step this
 * corresponds to.
 *
 * psb_blockdiag_attn_plan writes the tile schedule for (doc_ids, B, Hq, Hkv, L,
 * S, seq_start, enable_gqa) into `workspace` (size from
 * psb_blockdiag_attn_fwd_workspace_size).  The row tiles are ordered longest key
 * range first, or kept in row order when even the longest is short next to the share
 * of all tiles each concurrent attention workgroup gets; that count comes from the
 * current device's compute units and D (which is otherwise checked only for
 * support).  The order affects speed only, never results.
 *
 * psb_blockdiag_attn_fwd_planned launches the attention kernel alone; it reads
 * the schedule from `workspace`, which must hold a plan made with the same
 * doc_ids contents and the same shape arguments, enqueued earlier on the same
 * stream (or otherwise ordered before this call).  A workspace that holds no such
 * plan gives wrong outputs but no out-of-bounds access.  Arguments and errors are
 * otherwise those of psb_blockdiag_attn_fwd.
 */
psb_status psb_blockdiag_attn_plan(const int32_t* doc_ids, int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                                   int64_t S, int64_t D, int64_t seq_start, int32_t enable_gqa,
                                   void* workspace, size_t workspace_bytes, void* stream);

psb_status psb_blockdiag_attn_fwd_planned(const void* q, const void* k, const void* v,
                                          const int32_t* doc_ids, int64_t B, int64_t Hq, int64_t Hkv,
                                          int64_t L, int64_t S, int64_t D, const int64_t* q_strides,
                                          const int64_t* kv_strides, int64_t seq_start, float scale,
                                          int32_t enable_gqa, void* out, const void* workspace,
                                          size_t workspace_bytes, int32_t* status_word, void* stream);

/*
 * The whole preparation of a step in one launch (two when B * ceil(L / 32) > 2048):
 * document ids, run boundaries and the attention plan for B rows at once from their
 * boundaries (glm5_next.cp page,
 * doc_ids_from_cu_seqlens and segment_cu_seqlens; blockdiag_cp package overview,
 * "varlen metadata precompute").  Outputs equal those of psb_doc_ids_from_cu_seqlens and
 * psb_segment_cu_seqlens run on each row, and of psb_blockdiag_attn_plan on the ids.
 *
 *   cu_seqlens     device int32 [B][cu_row_stride]: row b's boundaries in its first
 *                  n_docs + 1 entries.  Rows with fewer documents repeat their last
 *                  boundary (zero-length documents take an id and cover nothing).
 *   doc_ids_out    device int32 [B, S], contiguous (document i of a row gets id i + 1).
 *   seg_cu_out     device int32 [B, S + 1], contiguous: row b's run boundaries
 *                  [0, run starts..., S] in its first seg_n_out[b] + 1 entries.
 *   seg_n_out      device int32 [B]: number of runs per row.
 *   workspace      as for psb_blockdiag_attn_plan (may be NULL when L == 0 or Hq == 0).
 *   status_word    device int32 or NULL: the bits of psb_doc_ids_from_cu_seqlens.
 * Shape arguments and errors as in psb_blockdiag_attn_plan; B > 65535 returns
 * PSB_ERR_SHAPE.
 */
psb_status psb_blockdiag_prepare(const int32_t* cu_seqlens, int64_t cu_row_stride, int64_t n_docs, int64_t B,
                                 int64_t Hq, int64_t Hkv, int64_t L, int64_t S, int64_t D, int64_t seq_start,
                                 int32_t enable_gqa, int32_t* doc_ids_out, int32_t* seg_cu_out, int32_t* seg_n_out,
                                 void* workspace, size_t workspace_bytes, int32_t* status_word, void* stream);

/*
 * psb_blockdiag_attn_fwd_planned for training: also writes, per query row, the
 * log-sum-exp the backward needs (the blockdiag_cp page keeps this path active
 * while backward recomputes checkpointed forwards).
 *
 *   lse   device fp32 [B, Hq, L], contiguous, 4-byte aligned, required:
 *         lse = log(sum over the row's allowed keys of exp(scale * q.k)), natural
 *         log, computed from the same bf16-rounded probabilities the output uses
 *         (relative error of the sum <= 2^-8, so |error| of lse <= 2^-8 + fp32
 *         rounding); -inf for a row without keys.
 *
 * Everything else is as in psb_blockdiag_attn_fwd_planned.
 */
psb_status psb_blockdiag_attn_fwd_lse_planned(const void* q, const void* k, const void* v,
                                              const int32_t* doc_ids, int64_t B, int64_t Hq, int64_t Hkv,
                                              int64_t L, int64_t S, int64_t D, const int64_t* q_strides,
                                              const int64_t* kv_strides, int64_t seq_start, float scale,
                                              int32_t enable_gqa, void* out, float* lse,
                                              const void* workspace, size_t workspace_bytes,
                                              int32_t* status_word, void* stream);

/*
 * Backward of the block-diagonal attention (the blockdiag_cp page keeps this path
 * active while backward recomputes checkpointed forwards; the glm5_next.cp page
 * routes K/V gradients back to the rank that owns each shard, so for a query shard
 * dk / dv hold the contributions of that shard's rows only, to be summed across
 * ranks).  With s = scale * q.k on the allowed pairs, P = exp(s - lse):
 *   dv = P^T dout,  dP = dout v^T,  dS = P * (dP - rowsum(dout * out)),
 *   dq = scale dS k,  dk = scale dS^T q   (dk, dv summed over a kv head's query heads).
 *
 * psb_blockdiag_attn_bwd_workspace_size gives the bytes of a workspace that holds
 * the tile plan, the backward's per-row table and its key-side tile order; use it
 * for psb_blockdiag_attn_plan and psb_blockdiag_attn_fwd_lse_planned too.
 *
 * psb_blockdiag_attn_bwd_planned:
 *   q, k, v, doc_ids, shapes, seq_start, scale, enable_gqa  as in the forward call
 *                that produced out and lse; q, k, v contiguous.
 *   out, dout    device bf16 [B, Hq, L, D], contiguous: forward output and its gradient.
 *   lse          device fp32 [B, Hq, L] from psb_blockdiag_attn_fwd_lse_planned.
 *   dq           device bf16 [B, Hq, L, D], contiguous (written).
 *   dk, dv       device bf16 [B, Hkv, S, D], contiguous (written; 0 for keys no row
 *                of this call attends to).
 *   workspace    holds the plan for these arguments (psb_blockdiag_attn_plan enqueued
 *                earlier on this stream), >= psb_blockdiag_attn_bwd_workspace_size bytes,
 *                16-byte aligned.  The plan occupies the first
 *                psb_blockdiag_attn_fwd_workspace_size(B, Hq, Hkv, L, D) bytes and is only
 *                read; the call writes its per-row table and key-side tile order after it.
 *   status_word  device int32 or NULL: as in psb_blockdiag_attn_fwd (the doc_ids
 *                precondition check, PSB_DATA_DOC_NOT_CONTIGUOUS).
 * Errors as in the forward; every bf16 pointer must be 16-byte aligned and lse
 * 4-byte aligned (PSB_ERR_INVALID_ARG).  Outputs are fp32-accumulated, rounded once
 * to bf16; P and dS are rounded to bf16 before the products that consume them.
 */
size_t psb_blockdiag_attn_bwd_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t S,
                                             int64_t D);
psb_status psb_blockdiag_attn_bwd_planned(const void* q, const void* k, const void* v, const void* out,
                                          const void* dout, const float* lse, const int32_t* doc_ids,
                                          int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t S,
                                          int64_t D, int64_t seq_start, float scale, int32_t enable_gqa,
                                          void* dq, void* dk, void* dv, void* workspace,
                                          size_t workspace_bytes, int32_t* status_word, void* stream);

/*
 * Attention of a query shard against a delivered key WINDOW instead of the whole
 * row (blockdiag_cp page, package overview: the exchange layer may deliver only the
 * needed keys through a left halo, rather than all-gathering them; cp_blockdiag_sdpa:
 * the local rows run against the delivered keys).  A shard's rows need the keys
 * [w, seq_start + L), where w is the start of the document of its first non-padding
 * row (psb_shard_kv_window_start); keys after seq_start + L are never needed.
 *
 *   k, v         device bf16 [B, Hkv, kv_len, D] (kv_strides as in the forward; NULL =
 *                contiguous with this shape): the keys at global positions
 *                [kv_start, kv_start + kv_len).  Requires 0 <= kv_start <= seq_start and
 *                seq_start + L <= kv_start + kv_len <= S (else PSB_ERR_SHAPE).
 *   doc_ids      device int32 [B, S]: the whole rows' ids, as in the forward.
 *   lse          device fp32 [B, Hq, L] or NULL (as in psb_blockdiag_attn_fwd_lse_planned).
 *   status_word  device int32 or NULL: PSB_DATA_KV_WINDOW is OR-ed in when some row
 *                needs a key before kv_start; such rows then attend only to the keys
 *                inside the window.  PSB_DATA_DOC_NOT_CONTIGUOUS as in
 *                psb_blockdiag_attn_fwd.
 * The workspace holds a plan from psb_blockdiag_attn_plan for the same doc_ids and shape
 * arguments (the plan does not depend on the window).  Everything else is as in
 * psb_blockdiag_attn_fwd_planned; with kv_start = 0 and kv_len = S the results equal it.
 */
psb_status psb_blockdiag_attn_fwd_window_planned(const void* q, const void* k, const void* v,
                                                 const int32_t* doc_ids, int64_t B, int64_t Hq, int64_t Hkv,
                                                 int64_t L, int64_t S, int64_t D, const int64_t* q_strides,
                                                 const int64_t* kv_strides, int64_t seq_start, int64_t kv_start,
                                                 int64_t kv_len, float scale, int32_t enable_gqa, void* out,
                                                 float* lse, const void* workspace, size_t workspace_bytes,
                                                 int32_t* status_word, void* stream);

/*
 * The backward for a key window: k, v, dk, dv are device bf16 [B, Hkv, kv_len, D],
 * contiguous, for the keys [kv_start, kv_start + kv_len); dk / dv are the gradients of
 * those keys (the part the glm5_next.cp page's gathers route back to the ranks that own
 * them).  Window rules and status_word as in psb_blockdiag_attn_fwd_window_planned;
 * everything else as in psb_blockdiag_attn_bwd_planned (workspace size included).
 */
psb_status psb_blockdiag_attn_bwd_window_planned(const void* q, const void* k, const void* v, const void* out,
                                                 const void* dout, const float* lse, const int32_t* doc_ids,
                                                 int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t S,
                                                 int64_t D, int64_t seq_start, int64_t kv_start, int64_t kv_len,
                                                 float scale, int32_t enable_gqa, void* dq, void* dk, void* dv,
                                                 void* workspace, size_t workspace_bytes, int32_t* status_word,
                                                 void* stream);

/*
 * Start of the key window a query shard needs, per row (blockdiag_cp page, package
 * overview: needed-only key delivery through a left halo).  kv_start_out[b] =
 * min(seq_start, first position of the document of the shard's first non-padding row);
 * seq_start when the shard has no such row.  The halo a rank receives from earlier
 * ranks is [kv_start_out[b], seq_start).
 *
 *   doc_ids       device int32 [B, S], contiguous; each non-padding id one run per row.
 *   kv_start_out  device int32 [B] (written).
 * 0 <= seq_start, seq_start + L <= S (else PSB_ERR_SHAPE).  B == 0 enqueues nothing.
 */
psb_status psb_shard_kv_window_start(const int32_t* doc_ids, int64_t B, int64_t S, int64_t seq_start, int64_t L,
                                     int32_t* kv_start_out, void* stream);

/*
 * The dense-mask path (blockdiag_cp page, package overview: the kernels layer has a
 * dense-mask kernel next to the varlen ones).
 *
 * psb_blockdiag_dense_mask materialises the per-document causal mask of a query shard:
 *   mask_out[b][i][k] = 1 iff doc_ids[b,k] == doc_ids[b,q], doc_ids[b,q] != -1000 and
 *   k <= q, for q = seq_start + i; else 0 (also for the padding bytes S..row_stride-1).
 *   doc_ids     device int32 [B, S], contiguous.
 *   mask_out    device uint8 [B, L, row_stride], contiguous, 4-byte aligned;
 *               row_stride >= S and a multiple of 4 (else PSB_ERR_SHAPE).
 *
 * psb_masked_attn_fwd is attention under an explicit mask, the same for all heads:
 *   out[b,h,i] = softmax over the keys k with mask[b][i][k] != 0 of scale * q.k, times v;
 *   a row without such a key outputs 0 (and lse -inf).
 *   q            device bf16 [B, Hq, L, D] (q_strides, elements, or NULL = contiguous).
 *   k, v         device bf16 [B, Hkv, S, D] (kv_strides likewise).  L and S independent.
 *   mask         device uint8, row i of batch b at mask + b * mask_batch_stride +
 *                i * mask_row_stride (bytes; batch stride 0 shares one mask); 4-byte
 *                aligned, both strides multiples of 4, and every row readable up to S
 *                rounded up to 4 bytes (bytes past S are ignored).
 *   lse          device fp32 [B, Hq, L] or NULL (as in psb_blockdiag_attn_fwd_lse_planned).
 *   scale, enable_gqa, out  as in psb_blockdiag_attn_fwd.
 * Every key tile of every row is visited: the cost is that of unmasked attention.  No
 * workspace.  D must be 64 or 128.
 */
psb_status psb_blockdiag_dense_mask(const int32_t* doc_ids, int64_t B, int64_t S, int64_t seq_start, int64_t L,
                                    uint8_t* mask_out, int64_t row_stride, void* stream);
psb_status psb_masked_attn_fwd(const void* q, const void* k, const void* v, const uint8_t* mask,
                               int64_t mask_batch_stride, int64_t mask_row_stride, int64_t B, int64_t Hq,
                               int64_t Hkv, int64_t L, int64_t S, int64_t D, const int64_t* q_strides,
                               const int64_t* kv_strides, float scale, int32_t enable_gqa, void* out, float* lse,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PSB_H_ */
