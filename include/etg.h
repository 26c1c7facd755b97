/*
 * etg.h -- static embedding / tied lm_head service on AMD Instinct MI355X (gfx950).
 *
 * Two operations, after the embed server of "ADR-0008 -- Remote Embeddings and
 * lm_head Service":
 *
 *   etg_embed_gather   token ids -> f32 residual_0 rows        ("POST /v1/embed")
 *   etg_logits_topk    residuals -> top-k (id, logit) per row  ("POST /v1/logits")
 *
 * with the rest of that endpoint's response (etg_logits_topk_probs: probabilities
 * at a temperature; etg_logits_raw: the raw logits mode) and the residual wire
 * formats of "ADR-0009 -- Wire Format Evolution" (etg_embed_gather_wire,
 * etg_logits_topk_wire).
 *
 * The table is row-major and row-addressed: row i occupies bytes
 * [i * row_bytes, (i + 1) * row_bytes) of the table (HELIX Columnar Embedding
 * proposal, section 3, "Wire format" and "Index").  The lm_head is tied: the
 * same table serves both operations (ADR-0008, "Open Questions" item 1; HELIX
 * proposal section 5(a)); an untied lm_head is simply a second table handle.
 *
 * Conventions for every function below:
 *  - Pointers named d_* are DEVICE pointers (HBM of the current HIP device); the
 *    caller owns all of them.  The library keeps no device allocations and no
 *    hidden state (the one exception is the scratch array behind
 *    etg_logits_topk_noalloc): a table handle is immutable host metadata and may
 *    be shared by threads.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work
 *    is enqueued on it and the call returns without waiting.
 *  - Every function returns an etg_status; 0 is success.  A negative status
 *    means nothing was enqueued; etg_last_error() then holds a message for the
 *    calling thread (the analog of the pages' {"error": "message"} envelope,
 *    ADR-0008 "Error contract").  No function aborts or throws.
 */
#ifndef ETG_H
#define ETG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage dtype of the table rows. */
typedef enum {
  ETG_F32 = 0,  /* little-endian IEEE binary32; row_bytes = 4 * hidden             */
  ETG_BF16 = 1, /* bfloat16 (upper half of a binary32); row_bytes = 2 * hidden       */
  ETG_Q8_0 = 2, /* blocks of 32 values: little-endian binary16 scale, then 32 int8;
                   value = int8 * scale; row_bytes = 34 * hidden / 32.  (The
                   embeddinggemma.c port specification, "Tensor inventory": the Q8_0
                   token_embd is used by row-gather + dequant only.) */
  ETG_F16 = 3   /* little-endian IEEE binary16; row_bytes = 2 * hidden.  (ADR-0008
                   "Vindex Slice: embed": embeddings.bin is vocab x hidden f16, and
                   "Memory footprint": decoded to f32 per lookup.) */
} etg_dtype;

typedef enum {
  ETG_OK = 0,
  ETG_EINVAL = -1,     /* null pointer or handle                                       */
  ETG_EDTYPE = -2,     /* unknown dtype                                                */
  ETG_ESHAPE = -3,     /* hidden not a multiple of 4 (f32) / 8 (bf16, f16) / 32 (Q8_0), or
                          outside [1, 65536]; vocab outside [1, 2^31 - 1]; seq_len or
                          batch outside the supported range                            */
  ETG_EALIGN = -4,     /* a device pointer lacks the alignment its argument states     */
  ETG_ERANGE = -5,     /* k outside [1, min(vocab, 64)], an unknown path, a path that
                          cannot serve the call (dtype, hidden, probabilities or raw
                          logits on ETG_PATH_RANK), or a temperature out of range      */
  ETG_EWORKSPACE = -6, /* workspace smaller than etg_logits_topk_workspace() bytes     */
  ETG_EHIP = -8        /* a HIP runtime call failed (the message names it)             */
} etg_status;

typedef struct etg_table etg_table;

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t etg_version(void);

/* Bytes of one stored row (HELIX proposal, section 3: row_bytes = hidden * itemsize;
 * Q8_0: 34 bytes per 32 values).  Returns -1 for an unknown dtype or a hidden size
 * the dtype cannot store. */
int64_t etg_row_bytes(int32_t dtype, int64_t hidden);

/* The float32 nearest to sqrt(hidden), computed on the host: the embedding scale of
 * the embeddinggemma.c port specification, "Forward graph" (x = token_embd[ids] *
 * sqrt(768)).  Returns 0 for hidden < 1. */
float etg_sqrt_d(int64_t hidden);

/* Describe a table that already lives in device memory.
 *   d_rows  device pointer to vocab * etg_row_bytes(dtype, hidden) bytes, 16-byte
 *           aligned; BORROWED: the caller keeps it alive and unchanged while the
 *           handle is used.
 *   out     receives a new handle (host memory only; no device allocation).
 * Errors: EINVAL (null), EDTYPE, ESHAPE, EALIGN. */
int32_t etg_table_create(const void* d_rows, int32_t dtype, int64_t vocab, int64_t hidden,
                         etg_table** out);

/* Free a handle (not the rows).  NULL is accepted. */
int32_t etg_table_destroy(etg_table* table);

/*
 * Row gather (ADR-0008 "POST /v1/embed": one residual row of hidden f32 values per
 * token id; "Open Questions" item 2: a prefill of N ids is N independent lookups).
 *
 *   out[n][c] = deq(row ids[n])[c]                  when scale == 1.0f
 *   out[n][c] = round_f32(deq(row ids[n])[c] * scale) otherwise
 *
 * deq is exact: f32 rows are copied, bf16 and f16 rows widened, Q8_0 values are int8 * the
 * block's binary16 scale (exact in f32).  The optional scale is applied after the
 * dequant with one round-to-nearest-even f32 multiply; pass etg_sqrt_d(hidden) for
 * the x * sqrt(d) of the embeddinggemma.c "Forward graph".
 *
 *   d_ids        int32 [seq_len], 4-byte aligned; read as uint32 (ADR-0008 "GET
 *                /v1/embed/{token_id}": a 32-bit key).  An id >= vocab (as uint32;
 *                so every negative int32) is a bad token id.
 *   seq_len      0 <= seq_len <= 2^31 - 1; 0 enqueues nothing and returns ETG_OK.
 *   d_out        f32 [seq_len][hidden] row-major, 16-byte aligned, caller-owned.
 *   d_bad_count  NULLABLE int32 on the device.  For each bad id the kernel writes an
 *                all-zero row and atomically adds 1 here; the caller zeroes it before
 *                the call and reads it after the stream is synchronized.
 * Results are bit-identical to the definition above.
 */
int32_t etg_embed_gather(const etg_table* table, const int32_t* d_ids, int64_t seq_len,
                         float scale, float* d_out, int32_t* d_bad_count, void* stream);

/*
 * Residual wire formats (ADR-0009 "Wire Layout": residuals travel as f32, f16 or
 * per-position symmetric i8).  A row of `hidden` values is encoded as
 *   ETG_WIRE_F32  hidden little-endian binary32 (4 * hidden bytes)
 *   ETG_WIRE_F16  hidden little-endian binary16 (2 * hidden bytes): round to nearest
 *                 even, clamped to +-65504 (the page's clamp-to-max overflow)
 *   ETG_WIRE_I8   [scale f32][zero_point f32 = 0][hidden int8] (hidden + 8 bytes):
 *                 scale = max|x| / 127, q = round-half-even(x / scale), both in f32,
 *                 clamped to [-127, 127]; decoded as q * scale.  A row with scale 0
 *                 is all zeros.
 * Rows are contiguous.
 */
typedef enum { ETG_WIRE_F32 = 0, ETG_WIRE_F16 = 1, ETG_WIRE_I8 = 2 } etg_wire;

/* Bytes of one encoded row; -1 for an unknown format or hidden outside [1, 65536]. */
int64_t etg_wire_row_bytes(int32_t wire, int64_t hidden);

/* etg_embed_gather with the output rows encoded in `wire` (the embed response on the
 * wire, ADR-0009).  The encoded values are those etg_embed_gather writes (dequant,
 * then the optional scale); encoding is bit-exact to the definition above.
 *   d_out   seq_len * etg_wire_row_bytes(wire, hidden) bytes, 4-byte aligned
 *           (16-byte aligned for ETG_WIRE_F32, which is etg_embed_gather itself).
 * A bad id gives an all-zero record and is counted as in etg_embed_gather.
 * Errors: as etg_embed_gather; ETG_ERANGE for an unknown format. */
int32_t etg_embed_gather_wire(const etg_table* table, const int32_t* d_ids, int64_t seq_len,
                              float scale, int32_t wire, void* d_out, int32_t* d_bad_count,
                              void* stream);

/* Kernel path for etg_logits_topk_ex (ETG_PATH_AUTO is what etg_logits_topk uses). */
typedef enum {
  ETG_PATH_AUTO = 0,   /* f32 and f16 tables: ROW; Q8_0 tables: Q8 (both VALU past their
                          row limits); bf16 tables: STREAM up to 8 rows, WIDE up to 16,
                          RANK beyond (WIDE up to 64, then GEMM, when probabilities or
                          raw logits are asked for, or hidden > 16384)                    */
  ETG_PATH_VALU = 1,   /* any dtype: f32 vector FMAs, one table pass per 8 residuals     */
  ETG_PATH_STREAM = 2, /* bf16 tables: one HBM pass per 8 residuals, bf16 MFMA dot engine;
                          batches of <= 4 use a hi+lo bf16 split of the residual          */
  ETG_PATH_GEMM = 3,   /* bf16 tables: tiled bf16 MFMA contraction for large batches     */
  ETG_PATH_WIDE = 4,   /* bf16 tables: one HBM pass per 64 residuals, bf16 MFMA dot engine,
                          hi+lo bf16 split of the residual                                */
  ETG_PATH_Q8 = 5,     /* Q8_0 tables.  Two or more residuals and hidden a multiple of
                          256: one HBM pass per 8 residuals, one bf16 MFMA per 32-value
                          block (int8 values are exact in bf16; residual as a hi+lo bf16
                          split), the block's scale applied to the f32 result.  Otherwise
                          hidden <= 8192: one HBM pass per 2 residuals, lanes split each
                          row's blocks, f32 FMAs                                          */
  ETG_PATH_ROW = 6,    /* f32 / bf16 / f16 tables with rows <= 16 KiB: one HBM pass per
                          2 residuals, a wave per row, f32 FMAs (no bf16 rounding of the
                          residual)                                                       */
  ETG_PATH_RANK = 7    /* bf16 tables with hidden <= 16384, top-k only: the WIDE kernel
                          (one pass of up to 256 rows) or the GEMM tiles rank with the residual
                          rounded once to bf16, then every row that a rigorous error
                          bound cannot rule out is rescored with f32 FMAs from the f32
                          residual (half the MFMA work of the hi + lo split)               */
} etg_path;

/* Device workspace bytes etg_logits_topk(_ex) needs for this table, batch and k
 * (and path; ETG_PATH_AUTO for etg_logits_topk).  Depends only on these arguments.
 * Returns a negative etg_status for invalid arguments. */
int64_t etg_logits_topk_workspace(const etg_table* lm_head, int64_t batch, int32_t k);
int64_t etg_logits_topk_workspace_ex(const etg_table* lm_head, int64_t batch, int32_t k,
                                     int32_t path);

/*
 * Tied lm_head projection fused with top-k (ADR-0008 "POST /v1/logits":
 * logits = residual @ lm_head.T over every vocabulary row, then the top_k tokens in
 * descending order).  The V-wide logits are never written to memory.
 *
 *   L[b][v] = sum_i residual[b][i] * deq(row v)[i]   (f32 accumulation)
 *
 *   d_residual     f32 [batch][hidden] row-major, contiguous, 4-byte aligned.
 *   batch          1 <= batch <= 65536.
 *   k              1 <= k <= min(vocab, 64).
 *   d_topk_ids     int32 [batch][k]: ids ordered by logit descending; equal logits
 *                  (including -0 and +0) are ordered by ascending id.
 *   d_topk_scores  f32 [batch][k]: the logits of those ids.
 *   d_workspace    at least etg_logits_topk_workspace() bytes, 256-byte aligned.
 * Accuracy: |score - exact logit| <= 2e-3 * sum_i |r_i e_i| for bf16 and Q8_0
 * tables and <= 1e-5 * sum_i |r_i e_i| for f32 and f16 tables; ids can differ from the
 * exact order only among logits that tie within that bound.  Results are
 * deterministic (bitwise repeatable) for a given path.
 */
int32_t etg_logits_topk(const etg_table* lm_head, const float* d_residual, int64_t batch,
                        int32_t k, int32_t* d_topk_ids, float* d_topk_scores,
                        void* d_workspace, size_t workspace_bytes, void* stream);

/* As etg_logits_topk, with an explicit kernel path (ETG_ERANGE if the path does
 * not support the table's dtype). */
int32_t etg_logits_topk_ex(const etg_table* lm_head, const float* d_residual, int64_t batch,
                           int32_t k, int32_t* d_topk_ids, float* d_topk_scores,
                           void* d_workspace, size_t workspace_bytes, int32_t path,
                           void* stream);

/* As etg_logits_topk_ex, then the answer is also copied to host memory without a
 * synchronisation, the pinned-buffer, copy and event pattern of the Perplexity blog
 * "Fast embeddings on GPUs" (its serving runtime's lazy result tensors): after the
 * kernels, d_topk_ids / d_topk_scores are copied asynchronously on `stream` into
 * h_topk_ids / h_topk_scores (host memory of batch * k entries each, owned by the
 * caller; page-locked memory from hipHostMalloc keeps the copy asynchronous,
 * pageable memory works but the copy then blocks the calling thread), and `event`
 * (a hipEvent_t the caller created, passed as void*) is recorded after the copy.
 * The host buffers hold the answer once the event has completed
 * (hipEventSynchronize / hipEventQuery); the caller meanwhile prepares its next
 * step.  ETG_EINVAL if a host pointer, the scores or the event is NULL; the other
 * errors as etg_logits_topk_ex (nothing is copied or recorded then); ETG_EHIP if
 * the copy or the record fails to enqueue. */
int32_t etg_logits_topk_to_host(const etg_table* lm_head, const float* d_residual, int64_t batch,
                                int32_t k, int32_t* d_topk_ids, float* d_topk_scores,
                                void* d_workspace, size_t workspace_bytes, int32_t path,
                                int32_t* h_topk_ids, float* h_topk_scores, void* event,
                                void* stream);

/* As etg_logits_topk_ex, and records two caller-created hipEvent_t (passed as void*,
 * either may be NULL) on `stream` immediately before and after the kernel that
 * streams the table, so a caller can time that kernel alone with
 * hipEventElapsedTime.  For measurement; results are identical to etg_logits_topk_ex. */
int32_t etg_logits_topk_profiled(const etg_table* lm_head, const float* d_residual, int64_t batch,
                                 int32_t k, int32_t* d_topk_ids, float* d_topk_scores,
                                 void* d_workspace, size_t workspace_bytes, int32_t path,
                                 void* event_before, void* event_after, void* stream);

/*
 * Top-k with probabilities (ADR-0008 "POST /v1/logits": every listed token carries
 * its probability at the request's temperature).  As etg_logits_topk_ex, and
 *
 *   d_topk_probs[b][j] = exp(L[b][id_j] / T - lse_b),  lse_b = ln sum_v exp(L[b][v] / T)
 *
 * the softmax of L / T over the WHOLE vocabulary (so the k listed values need not
 * sum to 1).  The normaliser is fused into the same table pass: every block
 * summarises its slice of logits as (max, sum of exp) and the merge combines the
 * summaries, so no V-wide vector is written.
 *   temperature    T > 0, finite, with log2(e) / T a finite float (ETG_ERANGE
 *                  otherwise); it changes the probabilities, never the ids.
 *   d_topk_probs   f32 [batch][k], 4-byte aligned.
 * Accuracy: with every logit within its bound above (tol_v), the log of each
 * probability is within (tol_{id_j} + max_v tol_v) / T of the exact value, plus
 * about 1e-5 for the f32 exp2 / log2 and sums.  Workspace: as etg_logits_topk_ex.
 * ETG_PATH_RANK is rejected (ETG_ERANGE); ETG_PATH_AUTO takes GEMM where top-k
 * alone would take RANK.
 */
int32_t etg_logits_topk_probs(const etg_table* lm_head, const float* d_residual, int64_t batch,
                              int32_t k, float temperature, int32_t* d_topk_ids,
                              float* d_topk_scores, float* d_topk_probs, void* d_workspace,
                              size_t workspace_bytes, int32_t path, void* stream);

/*
 * Raw logits mode (ADR-0008 "POST /v1/logits": the full vector of vocab_size f32
 * logits, for beam search and sampling).
 *   d_logits   f32 [batch][vocab] row-major, 4-byte aligned, caller-owned:
 *              L[b][v] as defined for etg_logits_topk, with the same accuracy; on
 *              a given path these are bitwise the values its top-k ranks.
 *   d_workspace  at least etg_logits_raw_workspace() bytes, 256-byte aligned.
 * Writes batch * vocab * 4 bytes of HBM besides reading the table once per pass.
 * ETG_PATH_RANK is rejected (ETG_ERANGE), as for etg_logits_topk_probs.
 */
int64_t etg_logits_raw_workspace(const etg_table* lm_head, int64_t batch, int32_t path);
int32_t etg_logits_raw(const etg_table* lm_head, const float* d_residual, int64_t batch,
                       float* d_logits, void* d_workspace, size_t workspace_bytes, int32_t path,
                       void* stream);

/* etg_logits_topk_ex with the residual rows in a wire format (the logits request on
 * the wire, ADR-0009): each value is decoded (f16 widened, i8 as q * scale) where
 * the kernels read the residual, so the result is bitwise that of etg_logits_topk_ex
 * on the decoded f32 rows.
 *   d_residual  batch * etg_wire_row_bytes(wire, hidden) bytes; 2-byte aligned for
 *               ETG_WIRE_F16, 4-byte aligned otherwise.
 * Workspace: as etg_logits_topk_ex.  ETG_ERANGE for an unknown format. */
int32_t etg_logits_topk_wire(const etg_table* lm_head, const void* d_residual, int32_t wire,
                             int64_t batch, int32_t k, int32_t* d_topk_ids, float* d_topk_scores,
                             void* d_workspace, size_t workspace_bytes, int32_t path, void* stream);

/*
 * Measurement: a plain read stream of a device buffer (16-byte non-temporal loads,
 * one contiguous range per wave read 8 KiB at a time, 16 waves per compute unit),
 * the measured HBM
 * read bandwidth the table-streaming kernels are compared with beside the nominal
 * peak.  Reads `bytes` at d_src; writes d_sink[0] only if the XOR of all 32-bit
 * words of the buffer equals 0x9e3779b9 (so that the loads are not removed).
 *   d_src    device pointer, 16-byte aligned (ETG_EALIGN otherwise)
 *   bytes    a positive multiple of 16 (ETG_ESHAPE otherwise)
 *   d_sink   4 bytes of device memory, 4-byte aligned
 */
int32_t etg_hbm_read_probe(const void* d_src, int64_t bytes, uint32_t* d_sink, void* stream);

/*
 * Graph-cached endpoint calls for small, repeated shapes (the serving pattern of
 * the Perplexity blog "Fast embeddings on GPUs", section "Tulip": one GPU graph per
 * shape configuration, token counts padded to buckets that are multiples of 64 or
 * 256, captured lazily -- the first hit of a configuration runs eagerly, the
 * second is captured and replayed, later hits replay -- and the answer tracked as
 * a page-locked host buffer behind an event, its lazy result tensors).
 *
 * A step cache binds one table to caller-owned buffers at fixed addresses, which
 * the captured graphs read and write:
 *   d_ids         int32 [etg_step_cache_ids_capacity(max_ids)], device
 *   d_rows        f32 [ids capacity][hidden], device, 16-byte aligned: gathered rows
 *   d_residual    f32 [max_batch][hidden], device: the residual rows the caller
 *                 writes before etg_step_logits (rows 0 .. batch - 1 are read)
 *   d_topk_ids, d_topk_scores  [max_batch][k], device
 *   d_workspace   etg_step_cache_workspace(table, max_batch, k) bytes, 256-aligned
 *   h_ids         int32 [ETG_STEP_ID_SLOTS][ids capacity], page-locked host memory
 *                 (hipHostMalloc): a ring of id staging slots, one per call in turn;
 *                 a slot is rewritten only after the gather that last read it has
 *                 run (the call waits on the host for that if needed)
 *   h_topk_ids, h_topk_scores  [max_batch][k], page-locked host memory: the answer
 * All are borrowed and must outlive the cache, as must the table rows (the cache
 * copies the table handle's metadata).  Page-locked buffers mapped into the
 * device's address space (hipHostGetDevicePointer succeeds, as for hipHostMalloc
 * memory on this platform) are read and written by the kernels directly, so a call
 * is kernels only; otherwise the ids and the answer are copied with async memcpys
 * (d_ids, d_topk_ids, d_topk_scores are those copies' device ends).
 * use_graphs = 0 runs every call eagerly (the same work, for comparison).  A cache is not thread-safe across streams:
 * its calls are serialised by a lock, and calls in flight on different streams
 * share its buffers.  Work is enqueued on `stream`; a NULL stream cannot be
 * captured, so every call on it runs eagerly.
 *
 * Bucketing: n token ids take a graph of round_up(n, 64) rows for n <= 1024, else
 * round_up(n, 256); the padding ids are 0 and their rows (past row n of d_rows)
 * are not part of the answer.  Logits graphs are keyed by the exact batch.
 */
typedef struct etg_step_cache etg_step_cache;
#define ETG_STEP_ID_SLOTS 4

/* Padded id capacity for max_ids ids (the bucket of max_ids); -1 if max_ids < 1. */
int64_t etg_step_cache_ids_capacity(int64_t max_ids);
/* Workspace bytes for every batch up to max_batch at this k (negative status on error). */
int64_t etg_step_cache_workspace(const etg_table* table, int64_t max_batch, int32_t k);
/* Errors: EINVAL (null), ESHAPE (max_ids, max_batch), ERANGE (k), EALIGN, EWORKSPACE. */
int32_t etg_step_cache_create(const etg_table* table, int64_t max_ids, int64_t max_batch, int32_t k,
                              int32_t use_graphs, int32_t* d_ids, float* d_rows, const float* d_residual, int32_t* d_topk_ids,
                              float* d_topk_scores, void* d_workspace, size_t workspace_bytes, int32_t* h_ids,
                              int32_t* h_topk_ids, float* h_topk_scores, etg_step_cache** out);
/* Destroys the captured graphs and the handle (not the buffers).  NULL is accepted. */
int32_t etg_step_cache_destroy(etg_step_cache* cache);
/* Graphs captured so far and graph launches made (for tests and measurement). */
int32_t etg_step_cache_stats(etg_step_cache* cache, int64_t* graphs, int64_t* replays);
/* ADR-0008 "POST /v1/embed" on host ids: copies ids[0 .. n) into h_ids (padding
 * ids 0 up to the bucket) in the next slot of h_ids, then, in the captured
 * sequence, the gather of the bucket's rows into d_rows (scale as
 * etg_embed_gather).  Bad token ids (>= vocab as uint32) are refused on the host
 * with ETG_ERANGE, nothing enqueued.  1 <= n <= max_ids (ETG_ESHAPE). */
int32_t etg_step_gather(etg_step_cache* cache, const int32_t* h_ids, int64_t n, float scale, void* stream);
/* ADR-0008 "POST /v1/logits" on d_residual rows 0 .. batch - 1: top-k (as
 * etg_logits_topk, ETG_PATH_AUTO) into h_topk_ids / h_topk_scores; `event` (a
 * hipEvent_t the caller created, passed as void*, nullable) is recorded after it:
 * the host buffers hold the answer once the event has completed, until the next
 * etg_step_logits call.  1 <= batch <= max_batch. */
int32_t etg_step_logits(etg_step_cache* cache, int64_t batch, void* event, void* stream);

/*
 * Measurement: a plain write stream of a device buffer (16-byte non-temporal
 * stores, one contiguous range per wave written 8 KiB at a time, 16 waves per
 * compute unit), the measured HBM write bandwidth that the gathers (whose HBM
 * traffic is mostly their output rows) are compared with beside the nominal
 * peak.  Sets every 32-bit word of the `bytes` at d_dst to `value`.
 *   d_dst    device pointer, 16-byte aligned (ETG_EALIGN otherwise)
 *   bytes    a positive multiple of 16 (ETG_ESHAPE otherwise)
 */
int32_t etg_hbm_write_probe(void* d_dst, int64_t bytes, uint32_t value, void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  As etg_logits_topk
 * (ETG_PATH_AUTO), with the workspace taken from a library-owned device array of
 * ETG_NOALLOC_SCRATCH_BYTES bytes instead of a caller's buffer.  The call
 * allocates nothing; the array is a file-scope device variable, one copy per GPU
 * the library runs on, held until the process ends (its address is looked up
 * once per device, on the first call with that device current).
 *   Limit: shapes whose etg_logits_topk_workspace() exceeds
 *   ETG_NOALLOC_SCRATCH_BYTES are rejected with ETG_EWORKSPACE before any device
 *   work (32 MiB covers batches up to 1,024 rows at k = 40 on a 262,144-row
 *   table; the 31B-shaped decode step needs 22 KiB).
 *   Sharing: every call on a GPU uses that GPU's one array and overwrites it
 *   (the kernels write everything they read, so nothing depends on earlier
 *   calls).  Calls whose kernels can overlap on one GPU -- on different
 *   streams, or from threads enqueueing at the same time -- race on the array
 *   and give wrong answers; such callers pass their own workspaces to
 *   etg_logits_topk instead.  `stream` must belong to the current device.
 * Errors: those of etg_logits_topk; ETG_EWORKSPACE beyond the limit; ETG_EHIP if
 * the array's device address cannot be looked up.
 */
#define ETG_NOALLOC_SCRATCH_BYTES (32ll << 20)
int32_t etg_logits_topk_noalloc(const etg_table* lm_head, const float* d_residual, int64_t batch,
                                int32_t k, int32_t* d_topk_ids, float* d_topk_scores, void* stream);

/* Message of the calling thread's last failed call ("" if none). */
const char* etg_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ETG_H */
