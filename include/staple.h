/*
 * staple.h -- C ABI of libstaple, the MI355X (gfx950) hot path of the STAPLE
 * embedding-augmented gated FFN.
 *
 * One augmented layer computes, for positions i = 0..N-1 with token IDs t_i:
 *
 *     g_i = W_gate x_i,  a_i = W_up x_i,  u_i = a_i + E[t_i],
 *     h_i = silu(g_i) * u_i,  y_i = W_down h_i
 *
 * The pretrained up-projection is kept and the token-indexed table row is added
 * to it as a residual path (STAPLE abstract; news synopsis "Pretrained models
 * gain sparse capacity without retraining", Synopsis).  Only the rows of the
 * tokens present in a batch are touched: the batch is deduplicated once and
 * one inverse map serves every layer (STAPLE retrieval-path table, Prefill
 * row); the active rows form a compact U x d_ff block whose gradient is the
 * table-row gradient (AI Radio episode on STAPLE, paper summary).  The most
 * frequent rows live in an HBM cache and misses come from pinned host memory
 * (STAPLE Table 4 caption; retrieval-path table, Prefill and Decode rows).
 *
 * The forward and backward calls also run the STEM layer, the replacement
 * design STAPLE is compared against (STAPLE abstract; Table 1 and Table 4,
 * STEM rows): it has no up-projection and the table row takes its place,
 *
 *     u_i = E[t_i],  h_i = silu(W_gate x_i) * u_i,  y_i = W_down h_i,
 *
 * selected by passing w_up = NULL (row-major weights) or up_proj = 0 (packed).
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers owned by the caller unless marked "host".
 *     The library never frees or retains them.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and returns a staple_status_t.  A non-OK status from argument
 *     validation means nothing was enqueued and no output was written.
 *   - No call allocates device memory.  Scratch comes from a caller-provided
 *     workspace `ws` of `ws_bytes` bytes (256-byte aligned), sized by the
 *     matching *_workspace_bytes query.
 *   - Matrices are row-major.  Weights use the (out_features x in_features)
 *     layout: w_gate, w_up are [d_ff x d_model], w_down is [d_model x d_ff].
 *     Tables are token-major: row t is the d_ff-wide row of token t.
 *   - Counts whose value is only known on the device (n_unique, n_miss) are
 *     int32 device scalars; arrays they size are allocated by the caller for
 *     the worst case.
 *   - A token ID or row index outside its valid range found by a kernel is
 *     not read; the kernel records it in a per-device error word instead and
 *     the affected output is unspecified.  staple_get_device_error() reports
 *     and clears that word.
 */
#ifndef STAPLE_H
#define STAPLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t staple_status_t;

#define STAPLE_OK 0
#define STAPLE_ERR_INVALID_ARGUMENT (-1)  /* null pointer, bad size, misalignment */
#define STAPLE_ERR_UNSUPPORTED (-2)       /* dtype or shape the kernels do not handle */
#define STAPLE_ERR_WORKSPACE (-3)         /* workspace smaller than the query returned */
#define STAPLE_ERR_HIP (-4)               /* a HIP runtime call failed */
#define STAPLE_ERR_INDEX_RANGE (-5)       /* a kernel met an out-of-range ID or index */
#define STAPLE_ERR_HOST (-6)              /* host-side failure (thread pool, host ID check) */
#define STAPLE_ERR_SCRATCH_LIMIT (-7)     /* larger than the allocation-free call's fixed scratch */

/* Element types.  STAPLE_BF16: bfloat16 storage, fp32 accumulation.
 * STAPLE_F32: fp32 storage and accumulation. */
#define STAPLE_F32 0
#define STAPLE_BF16 1

/* Human-readable text of a status code (static storage). */
const char* staple_status_string(staple_status_t status);

/* Library version string (static storage). */
const char* staple_version(void);

/* Waits for `stream`, then reads and clears the calling device's error word.
 * Returns STAPLE_OK, or STAPLE_ERR_INDEX_RANGE if any kernel since the last
 * call met an out-of-range ID or index. */
staple_status_t staple_get_device_error(void* stream);

/* ------------------------------------------------------------------------
 * Batch dedup.  The batch's token IDs are deduplicated once and the inverse
 * map is reused by every augmented layer (STAPLE retrieval-path table,
 * Prefill row).
 *
 * Inputs : ids[n_tokens] int32, each in [0, vocab).
 * Outputs: uniq[n_tokens]      distinct IDs in ascending order; first
 *                              *n_unique entries are defined.
 *          inv[n_tokens]       uniq[inv[i]] == ids[i].
 *          sorted_pos[n_tokens] positions ordered by (ids[i], i) ascending.
 *          seg_start[n_tokens+1] sorted_pos[seg_start[u] .. seg_start[u+1])
 *                              are the positions of uniq[u]; entry *n_unique
 *                              equals n_tokens.
 *          n_unique            int32 device scalar, U.
 * n_tokens may be 0 (then *n_unique = 0 and seg_start[0] = 0).
 * vocab must be in [1, 2^31-1].  Out-of-range IDs set the device error word.
 * The result is deterministic (no atomics decide any output).
 * ------------------------------------------------------------------------ */
size_t staple_dedup_workspace_bytes(int64_t n_tokens);
staple_status_t staple_dedup(const int32_t* ids, int64_t n_tokens, int64_t vocab,
                             int32_t* uniq, int32_t* inv, int32_t* sorted_pos,
                             int32_t* seg_start, int32_t* n_unique,
                             void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Frequency-aware row cache: a static cache of the most frequent rows,
 * about 5% of the vocabulary (AI Radio episode on STAPLE: 5-6% cached,
 * frequency-aware; STAPLE Table 4 caption: 1 GB GPU cache).  One id->slot map
 * serves every layer; each layer has its own [capacity x d_ff] slot rows.
 * ------------------------------------------------------------------------ */

/* Count pass: counts[ids[i]] += 1 for every i (counts int64[vocab], not
 * cleared by the call).  Out-of-range IDs set the device error word. */
staple_status_t staple_cache_count(const int32_t* ids, int64_t n_tokens, int64_t vocab,
                                   int64_t* counts, void* stream);

/* Ranks IDs by count (larger first, ties by smaller ID) and assigns slot s to
 * the ID of rank s for s < capacity.  When fewer IDs than `capacity` have a
 * non-zero count the ranking still fills every slot.
 * counts int64[vocab], each in [0, 2^31-1] (larger values set the error word).
 * Outputs: id_to_slot int32[vocab] (slot, or -1 when not cached),
 *          slot_to_id int32[capacity].
 * 0 <= capacity <= vocab. */
size_t staple_cache_build_workspace_bytes(int64_t vocab);
staple_status_t staple_cache_build(const int64_t* counts, int64_t vocab, int64_t capacity,
                                   int32_t* id_to_slot, int32_t* slot_to_id,
                                   void* ws, size_t ws_bytes, void* stream);

/* Copies the cached rows of one layer's table into its slot rows:
 * slot_rows[s] = table[slot_to_id[s]] for s < capacity.  `table` is
 * [vocab x d_ff] of `dtype`, in device memory or in pinned host memory that
 * the device can address (hipHostMalloc); pageable host memory for `table` or
 * `slot_rows` is rejected with STAPLE_ERR_INVALID_ARGUMENT before any launch. */
staple_status_t staple_cache_fill(const void* table, int64_t vocab, int64_t d_ff, int32_t dtype,
                                  const int32_t* slot_to_id, int64_t capacity,
                                  void* slot_rows, void* stream);

/* Probes the cache for each unique ID (STAPLE retrieval-path table: a GPU
 * lookup probes the LFU cache) and compacts the misses in ascending order of
 * unique index.
 * Inputs : uniq[max_unique], n_unique (device scalar, <= max_unique),
 *          id_to_slot int32[vocab].
 * Outputs: code[max_unique]   slot of uniq[u] on a hit, -1-m on a miss where
 *                             m is u's place in the miss list.
 *          miss_uidx[max_unique] unique indices of the misses (first *n_miss).
 *          miss_ids[max_unique]  their token IDs (first *n_miss); may be NULL.
 *          n_miss               int32 device scalar. */
staple_status_t staple_cache_lookup(const int32_t* uniq, const int32_t* n_unique, int64_t max_unique,
                                    const int32_t* id_to_slot, int64_t vocab,
                                    int32_t* code, int32_t* miss_uidx, int32_t* miss_ids,
                                    int32_t* n_miss, void* stream);

/* Splits the batch's token positions by cache outcome, for a gate/up that
 * runs the cached tokens while the miss rows are in flight.
 * Inputs : inv int32[n_tokens] (token -> unique index, from staple_dedup),
 *          code int32[max_unique] and n_unique (from staple_cache_lookup).
 * Outputs: hit_pos  int32[n_tokens]: positions of tokens whose row is cached,
 *                   ascending (first counts[0]);
 *          miss_pos int32[n_tokens]: positions of the other tokens, ascending
 *                   (first counts[1]);
 *          tok_row  int32[n_tokens]: each token's row in its source block,
 *                   the cache slot for a hit, the miss index for a miss;
 *          counts   int32[2] device: {hits, misses}.
 * A token whose inv entry is outside [0, n_unique) sets the device error
 * word and is listed with the hits with tok_row -1.  max_unique <= n_tokens. */
staple_status_t staple_split_tokens(const int32_t* inv, int64_t n_tokens, const int32_t* code,
                                   const int32_t* n_unique, int64_t max_unique, int32_t* hit_pos,
                                   int32_t* miss_pos, int32_t* tok_row, int32_t* counts,
                                   void* stream);

/* Miss staging (STAPLE retrieval-path table, Prefill row: only cache-miss rows
 * come from the CPU, packed into pinned host buffers and sent with bulk
 * asynchronous host-to-device copies).  Runs on the calling thread: packs
 * rows host_table[host_miss_ids[m]] into host_staging (pinned,
 * [n_miss x d_ff]) with a pool of host threads, then enqueues one
 * hipMemcpyAsync host_staging -> dev_miss_rows on `stream` (normally a side
 * stream; the caller records an event after it).  The caller must not reuse
 * host_staging until that copy has completed.
 * host_table: host [vocab x d_ff]; host_miss_ids: host int32[n_miss], each in
 * [0, vocab) (checked on the host: STAPLE_ERR_HOST names a bad ID and nothing
 * is copied). */
staple_status_t staple_stage_misses(const void* host_table, int64_t vocab, int64_t d_ff,
                                    int32_t dtype, const int32_t* host_miss_ids, int32_t n_miss,
                                    void* host_staging, void* dev_miss_rows, void* stream);

/* Miss staging of a stack of layers on the GPU's DMA engines (STAPLE
 * retrieval-path table, Prefill row: miss rows packed into pinned host
 * buffers and sent with bulk asynchronous host-to-device copies).  For each
 * layer l < n_layers the rows host_tables[l][host_miss_ids[m]], m < n_miss,
 * are packed by the library's host threads into the block
 * host_staging + l * n_miss * d_ff elements, and that block is copied to
 * dev_miss_rows[l] by a DMA engine of the current device, which uses no
 * compute unit (layer l + 1 is packed while layer l's block is copied).
 * Runs on the calling thread and returns when every copy has completed; the
 * caller then enqueues what reads dev_miss_rows (staple_assemble_rows), and
 * must have seen earlier readers of dev_miss_rows finish (an event
 * synchronised on the host) before the call.
 *   host_tables: host array of n_layers host pointers, each [vocab x d_ff]
 *     with rows table_stride elements apart (0: d_ff; larger for tables
 *     interleaved by staple_group_tables_host), read by the host only;
 *   host_miss_ids: host int32[n_miss], each in [0, vocab) (checked first:
 *     STAPLE_ERR_HOST and nothing copied);
 *   host_staging: pinned host memory (hipHostMalloc) of
 *     n_layers * n_miss * d_ff elements;
 *   dev_miss_rows: host array of n_layers pointers to device memory, each
 *     [>= n_miss x d_ff].
 * STAPLE_ERR_UNSUPPORTED when the device's DMA engines cannot be reached
 * through the HSA runtime (nothing is copied; staple_stage_misses does the
 * same work with a stream copy); STAPLE_ERR_HIP when an engine reports a
 * failed copy.  Calls on one device take turns. */
staple_status_t staple_stage_misses_dma(int64_t n_layers, const void* const* host_tables,
                                        int64_t table_stride, int64_t vocab, int64_t d_ff,
                                        int32_t dtype, const int32_t* host_miss_ids,
                                        int32_t n_miss, void* host_staging,
                                        void* const* dev_miss_rows);

/* Compact leaf block assembly (AI Radio episode: only the active U x d_ff rows
 * are materialised on the GPU).
 * rows[u] = code[u] >= 0 ? cache_rows[code[u]] : miss_rows[-1-code[u]]
 * for u < *n_unique.  cache_rows [capacity x d_ff], miss_rows [>= n_miss x d_ff]. */
staple_status_t staple_assemble_rows(const void* cache_rows, int64_t capacity,
                                     const void* miss_rows, int64_t max_miss,
                                     const int32_t* code, const int32_t* n_unique,
                                     int64_t max_unique, int64_t d_ff, int32_t dtype,
                                     void* rows, void* stream);

/* Compact block assembly with the misses read straight from the table:
 * rows[u] = code[u] >= 0 ? cache_rows[code[u]] : table[uniq[u]] for
 * u < *n_unique, one workgroup per row.  `table` [vocab x d_ff] is in device
 * memory or in pinned host memory that the device can address (hipHostMalloc):
 * with a host table the misses cross PCIe inside the kernel, with no host
 * round trip for the miss list (STAPLE retrieval-path table, decode: misses
 * read from host memory).  uniq, code, n_unique as from staple_dedup and
 * staple_cache_lookup; pageable host memory for `table` or `rows` is rejected
 * with STAPLE_ERR_INVALID_ARGUMENT before any launch. */
staple_status_t staple_assemble_rows_from_table(const void* cache_rows, int64_t capacity,
                                                const void* table, int64_t vocab,
                                                const int32_t* uniq, const int32_t* code,
                                                const int32_t* n_unique, int64_t max_unique,
                                                int64_t d_ff, int32_t dtype, void* rows,
                                                void* stream);

/* Row gather: dst[r] = src[index[r]] for r < n, where n = *n_rows when n_rows
 * is non-NULL (a device scalar, <= max_rows) and max_rows otherwise.
 * src [src_rows x d_ff] in device memory or in pinned host memory that the
 * device can address (hipHostMalloc), dst [max_rows x d_ff] (device memory
 * or pinned host memory); pageable host memory for either is rejected with
 * STAPLE_ERR_INVALID_ARGUMENT before any launch.  Builds the
 * compact block R = E[uniq] when the whole table is device-resident, and
 * reads miss rows straight from a pinned host table (one workgroup per row,
 * whole-row reads over PCIe, no host round trip for the miss list). */
staple_status_t staple_gather_rows(const void* src, int64_t src_rows, const int32_t* index,
                                   const int32_t* n_rows, int64_t max_rows, int64_t d_ff,
                                   int32_t dtype, void* dst, void* stream);

/* ------------------------------------------------------------------------
 * Forward of one augmented layer.
 *   x [n_tokens x d_model] (dtype), w_gate, w_up [d_ff x d_model],
 *   w_down [d_model x d_ff] (dtype); w_up NULL selects the STEM layer
 *   (u = rows[row_index], the gate GEMM alone);
 *   rows [n_rows x d_ff] (dtype): the compact block R with row_index = inv,
 *   or a whole device-resident table with row_index = the token IDs.
 *   row_index int32[n_tokens], each in [0, n_rows).
 * Outputs: y [n_tokens x d_model] of out_dtype (STAPLE_F32 or STAPLE_BF16).
 *   save_g, save_u, save_h [n_tokens x d_ff] (dtype), each nullable: the
 *   pre-activation g, the up branch u = W_up x + E[t] (STEM: u = E[t]) and h,
 *   for the backward.
 * Layout requirements: d_model and d_ff multiples of 64; 16-byte aligned
 * pointers.  n_tokens >= 0 (0 enqueues nothing).
 * In bf16, g, u and y accumulate in fp32; h is rounded to bf16 once (the
 * operand of the down-projection); saved g and u are rounded to bf16.
 * ------------------------------------------------------------------------ */
/* Workspace of staple_ffn_fwd: room for h (used when save_h is NULL) plus
 * staple_ffn_down's workspace. */
size_t staple_ffn_fwd_workspace_bytes(int64_t n_tokens, int64_t d_model, int64_t d_ff,
                                      int32_t dtype);
staple_status_t staple_ffn_fwd(int64_t n_tokens, int64_t d_model, int64_t d_ff,
                               int32_t dtype, int32_t out_dtype,
                               const void* x, const void* w_gate, const void* w_up,
                               const void* w_down, const void* rows, int64_t n_rows,
                               const int32_t* row_index, void* y,
                               void* save_g, void* save_u, void* save_h,
                               void* ws, size_t ws_bytes, void* stream);

/* The two halves of staple_ffn_fwd, for callers that schedule them apart.
 * staple_ffn_gate_up: h = silu(W_gate x) * (W_up x + rows[row_index]) into
 *   h [n_tokens x d_ff] (dtype), with optional saves of g and u; the table
 *   rows are gathered inside the GEMM's epilogue (STAPLE retrieval-path table:
 *   compact-row reconstruction fused with the FFN).
 * staple_ffn_down: y = W_down h, y of out_dtype; its workspace holds the
 *   fp32 partial sums of the split-K decode kernel (zero bytes when the
 *   batch does not take that path).
 * Same layout rules and error behaviour as staple_ffn_fwd.  Batches of at
 * most 64 tokens in bf16 take the decode kernels (weights streamed once,
 * split-K down-projection); larger batches and fp32 take the tiled GEMMs. */
staple_status_t staple_ffn_gate_up(int64_t n_tokens, int64_t d_model, int64_t d_ff, int32_t dtype,
                                   const void* x, const void* w_gate, const void* w_up,
                                   const void* rows, int64_t n_rows, const int32_t* row_index,
                                   void* h, void* save_g, void* save_u, void* stream);

/* Gate/up over a subset of the batch's tokens, so that the tokens whose
 * table rows are cached can run while the miss rows are still being copied
 * from host memory (STAPLE retrieval-path table: misses staged on a side
 * stream, overlapped with the FFN).  Computes the rows token_pos[0 .. n_sel)
 * of h (and g, u) exactly as staple_ffn_gate_up computes them for the whole
 * batch; x, h, g, u are [n_tokens x ...] and row_index is indexed by token
 * position, so the two halves of a split batch can read their table rows from
 * different blocks (cache slots, staged misses).
 * token_pos: device int32[n_sel]; an entry outside [0, n_tokens) sets the
 * device error word and that token is neither read nor written. */
staple_status_t staple_ffn_gate_up_tokens(int64_t n_sel, const int32_t* token_pos,
                                          int64_t n_tokens, int64_t d_model, int64_t d_ff,
                                          int32_t dtype, const void* x, const void* w_gate,
                                          const void* w_up, const void* rows, int64_t n_rows,
                                          const int32_t* row_index, void* h, void* save_g,
                                          void* save_u, void* stream);

size_t staple_ffn_down_workspace_bytes(int64_t n_tokens, int64_t d_model, int64_t d_ff,
                                       int32_t dtype);
staple_status_t staple_ffn_down(int64_t n_tokens, int64_t d_model, int64_t d_ff, int32_t dtype,
                                int32_t out_dtype, const void* h, const void* w_down, void* y,
                                void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decode with packed weights.  The forward of a serving step (at most 64
 * tokens) streams every weight byte once per step, so its speed is the HBM
 * read rate of the weight stream; the row-major matrices make each load
 * instruction read 64-byte pieces of 16 rows a row apart.  A packed copy,
 * made once when the weights are loaded, stores the bytes in the order the
 * decode kernels read them (STAPLE's layer, abstract: the same
 * y = W_down (silu(W_gate x) * (W_up x + E[t])) as staple_ffn_fwd).
 *
 * staple_decode_pack_weights: bf16 only.  Either output may be NULL (then
 *   its source may be NULL too).
 *   w_gate, w_up [d_ff x d_model], w_down [d_model x d_ff] row-major bf16;
 *   w_up NULL packs the STEM layer's gate-only operand.
 *   packed_gate_up: 2 * d_ff * d_model bf16 elements (the size of w_gate and
 *     w_up together; d_ff * d_model for the gate-only operand); packed_down:
 *     d_model * d_ff elements.  Both are owned by the caller, device memory,
 *     16-byte aligned, and must not overlap the sources.
 *   Format (a private layout: produce it only with this call): an operand of
 *   R rows x K columns is cut into K/64 steps of R/16 row blocks; bytes
 *   ((s * R/16 + b) * 2 + j) * 1024 + 16 * l .. +16 hold bytes
 *   128 s + 64 j + 16 (l / 16) .. +16 of row l % 16 of block b.  A gate/up
 *   block b holds rows 8b .. 8b+7 of w_gate (block rows 0-7) and of w_up
 *   (block rows 8-15); a gate-only block b rows 16b .. 16b+15 of w_gate; a
 *   down block b rows 16b .. 16b+15 of w_down.
 *   d_model and d_ff multiples of 64.
 * staple_ffn_fwd_packed: staple_ffn_fwd for 1 <= n_tokens <= 64 in bf16
 *   (n_tokens == 0 enqueues nothing) reading the packed weights; same
 *   arguments otherwise, same workspace (staple_ffn_fwd_workspace_bytes),
 *   same outputs bit for bit as staple_ffn_fwd on the unpacked weights.
 *   up_proj: nonzero when packed_gate_up was packed with w_up (the STAPLE
 *   layer), 0 when it is the gate-only operand (the STEM layer, as
 *   staple_ffn_fwd with w_up = NULL); a mismatch reads the wrong layout.
 *   Larger batches or fp32 return STAPLE_ERR_UNSUPPORTED.
 * staple_ffn_gate_up_packed, staple_ffn_down_packed: its two halves, as
 *   staple_ffn_gate_up and staple_ffn_down are those of staple_ffn_fwd (same
 *   arguments with the packed operand in place of the row-major ones, same
 *   workspace for the down half, same bits), with the same limits as
 *   staple_ffn_fwd_packed.
 * ------------------------------------------------------------------------ */
staple_status_t staple_decode_pack_weights(int64_t d_model, int64_t d_ff, int32_t dtype,
                                           const void* w_gate, const void* w_up,
                                           const void* w_down, void* packed_gate_up,
                                           void* packed_down, void* stream);
staple_status_t staple_ffn_gate_up_packed(int64_t n_tokens, int64_t d_model, int64_t d_ff,
                                          int32_t dtype, const void* x,
                                          const void* packed_gate_up, int32_t up_proj,
                                          const void* rows, int64_t n_rows,
                                          const int32_t* row_index, void* h,
                                          void* save_g, void* save_u, void* stream);
staple_status_t staple_ffn_down_packed(int64_t n_tokens, int64_t d_model, int64_t d_ff,
                                       int32_t dtype, int32_t out_dtype, const void* h,
                                       const void* packed_down, void* y, void* ws,
                                       size_t ws_bytes, void* stream);
staple_status_t staple_ffn_fwd_packed(int64_t n_tokens, int64_t d_model, int64_t d_ff,
                                      int32_t dtype, int32_t out_dtype, const void* x,
                                      const void* packed_gate_up, int32_t up_proj,
                                      const void* packed_down, const void* rows, int64_t n_rows,
                                      const int32_t* row_index, void* y, void* save_g,
                                      void* save_u, void* save_h, void* ws, size_t ws_bytes,
                                      void* stream);

/* staple_ffn_fwd_packed_noalloc: staple_ffn_fwd_packed for callers that
 * cannot allocate device memory or pass a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments without ws/ws_bytes, same kernels and the same bits.  Its scratch
 * (h when save_h is NULL, and the down-projection's partial sums) is a fixed
 * 16 MiB device array inside the library, one per GPU, held until the
 * process ends; the call allocates nothing.  A problem whose workspace
 * (staple_ffn_fwd_workspace_bytes(n_tokens, d_model, d_ff, STAPLE_BF16))
 * exceeds 16 MiB returns STAPLE_ERR_SCRATCH_LIMIT before any launch: 64
 * tokens at 2048 x 8192 need 5 MiB, at 4096 x 11008 9.4 MiB.  Every call on
 * one GPU shares that array: calls that overlap on one GPU (other streams,
 * other threads) race and give undefined results; calls in stream order are
 * safe (nothing in it needs to start at zero). */
staple_status_t staple_ffn_fwd_packed_noalloc(int64_t n_tokens, int64_t d_model, int64_t d_ff,
                                              int32_t dtype, int32_t out_dtype, const void* x,
                                              const void* packed_gate_up, int32_t up_proj,
                                              const void* packed_down, const void* rows,
                                              int64_t n_rows, const int32_t* row_index, void* y,
                                              void* save_g, void* save_u, void* save_h,
                                              void* stream);

/* ------------------------------------------------------------------------
 * One decode step over a stack of layers whose tables live in pinned host
 * memory with the most frequent rows cached in HBM (STAPLE retrieval-path
 * table, Decode row: one dedup and cache probe per step, then the layers;
 * Table 4 caption: the 1 GB cache of frequent rows).  Enqueues on `stream`:
 *   1. staple_dedup of ids (the batch's n tokens) and staple_cache_lookup
 *      against id_to_slot (one launch: a decode batch fits one wave);
 *   2. the compact rows R_l = layers[l].rows of every layer that has them
 *      (hits from layers[l].cache_rows, misses read straight from
 *      layers[l].table, as staple_assemble_rows_from_table), one launch for
 *      up to 32 layers, so the host reads of all those layers' misses are in
 *      flight together;
 *   3. each layer's decode forward (staple_ffn_fwd_packed with rows = R_l,
 *      row_index = inv).  A layer with rows = NULL instead reads each
 *      token's row in place inside its gate/up kernel: from cache_rows when
 *      the row is cached, else from the table (over PCIe when it is in
 *      pinned host memory), loaded into LDS by a wave of its own while the
 *      weights stream (STAPLE retrieval-path table, Decode row: misses read
 *      zero-copy from host memory).  Its y has the same bits; no R_l is
 *      written.  This saves the assembly launch and pays off for tables in
 *      HBM; for tables in pinned host memory every workgroup then reads
 *      small pieces of the same miss rows over PCIe, and the one-launch
 *      assembly of whole rows measured faster.
 * The whole step is one native call: issuing it costs one call per step
 * instead of several per layer.
 *
 * group (0 .. 4): how the compact rows of the layers reach the device.
 *   0: every layer's rows are assembled before the first layer (step 2).
 *   G > 0: the layers form groups of G consecutive layers (the pages keep
 *     every four adjacent tables together and synchronise a group's lookups
 *     only where the group is first used: STAPLE retrieval-path table, Decode
 *     row).  Group 0's rows are assembled before the first layer; the rows of
 *     group k + 1 are copied while group k runs, by a copy wave in each
 *     workgroup of group k's gate/up launches (launch j of the group carries
 *     part j of the next group's unique rows, for all of its layers), so the
 *     PCIe reads of the misses hide under those launches' weight streams.
 *     Stream order makes group k + 1's rows complete before its first layer.
 *     Every layer needs `rows`.  A group whose part would not fit one
 *     launch's copy waves is assembled before the first layer instead.
 *   Every choice gives the same bits.
 *
 *   layers: host array of n_layers descriptors:
 *     x [n x d_model] bf16; packed_gate_up, packed_down from
 *     staple_decode_pack_weights (up_proj as for staple_ffn_fwd_packed);
 *     cache_rows [capacity x d_ff] bf16 device (slot s = the row of the ID
 *     with slot s in id_to_slot, e.g. from staple_cache_fill); table
 *     [vocab x d_ff] bf16, pinned host (hipHostMalloc) or device, whose
 *     token rows lie table_stride elements apart (0: d_ff; more when several
 *     layers' tables are interleaved token-major, as staple_group_tables_host
 *     makes them: layer j of a group then has table = group base + j d_ff and
 *     table_stride = (tables in the group) d_ff, so one miss of the group is
 *     one contiguous read of all its layers' rows); rows
 *     [n x d_ff] bf16 device, one per layer (it holds R_l after the step),
 *     or NULL (rows read in place, above);
 *     y [n x d_model] of out_dtype.
 *   1 <= n <= 64, d_model and d_ff multiples of 64 (else UNSUPPORTED).
 *   uniq, inv, sorted_pos [n], seg_start [n + 1], n_unique [1]: staple_dedup's
 *     outputs; code, miss_uidx [n], n_miss [1]: staple_cache_lookup's.
 *   ws: staple_decode_step_workspace_bytes(n, d_model, d_ff) bytes.
 * Same outputs bit for bit as the separate calls.  Argument errors return
 * before anything is enqueued; the device error word reports IDs or slots
 * out of range.
 * ------------------------------------------------------------------------ */
typedef struct staple_decode_layer {
  const void* x;
  const void* packed_gate_up;
  const void* packed_down;
  const void* cache_rows;
  const void* table;
  void* rows;
  void* y;
  int64_t table_stride;
} staple_decode_layer_t;

size_t staple_decode_step_workspace_bytes(int64_t n_tokens, int64_t d_model, int64_t d_ff);
staple_status_t staple_decode_step_cached(
    int64_t n_layers, const staple_decode_layer_t* layers, int64_t n_tokens, int64_t d_model,
    int64_t d_ff, int32_t up_proj, int32_t out_dtype, const int32_t* ids, int64_t vocab,
    const int32_t* id_to_slot, int64_t capacity, int32_t group, int32_t* uniq, int32_t* inv,
    int32_t* sorted_pos, int32_t* seg_start, int32_t* n_unique, int32_t* code,
    int32_t* miss_uidx, int32_t* n_miss, void* ws, size_t ws_bytes, void* stream);

/* Host-side layout of offloaded tables: every n_tables adjacent layers' tables
 * stored token-major in one block (STAPLE retrieval-path table, Decode row:
 * every four adjacent tables in a token-major CPU layout), so that the rows of
 * one token for all of those layers are one contiguous read:
 *   grouped[t * n_tables * d_ff + j * d_ff + c] = tables[j][t * d_ff + c].
 * tables: host array of n_tables host pointers, each [vocab x d_ff] of dtype;
 * grouped: host memory of vocab * n_tables * d_ff elements (pinned
 * (hipHostMalloc) when kernels are to read it), not overlapping the sources.
 * Runs on the calling thread with the library's host threads; synchronous.
 * 1 <= n_tables <= 64. */
staple_status_t staple_group_tables_host(const void* const* tables, int64_t n_tables,
                                         int64_t vocab, int64_t d_ff, int32_t dtype,
                                         void* grouped);

/* ------------------------------------------------------------------------
 * Rows of one prefill chunk for a stack of layers with host-offloaded tables
 * (STAPLE retrieval-path table, Prefill row: the prompt's tokens are
 * deduplicated once, the HBM cache is probed, one inverse map serves every
 * layer, later layers' rows are fetched while earlier layers run and
 * successive chunks are pipelined).  One call per chunk:
 *   1. (lookup = 1) staple_dedup of ids[0 .. n) (outputs uniq, inv,
 *      sorted_pos, seg_start, n_unique, as staple_dedup);
 *   2. (lookup = 1) staple_cache_lookup of the unique IDs (outputs code,
 *      miss_uidx, n_miss, as staple_cache_lookup; no miss-ID list);
 *   3. every layer's compact rows: layers[l].rows[u] = cache_rows_l[code[u]]
 *      on a hit, the table's row uniq[u] on a miss, for u < *n_unique, in one
 *      launch for up to 32 layers (a longer stack in slices of 32).
 * lookup = 0 skips steps 1 and 2 and reads uniq, code and n_unique as an
 * earlier call on the same chunk left them (nothing else is read or
 * written): the rows of some layers can then be fetched first (the first
 * layer's, say) and the others while those layers run.
 * With a pinned host table the misses cross PCIe inside that launch.  It
 * runs on at most max_workgroups workgroups (0: up to 512, enough to fill
 * the GPU); a small count (16-64) lets the assembly of the next chunk, issued
 * on a second stream, run beside the current chunk's GEMMs while holding
 * only that many compute units.  The caller orders the streams with events:
 * the next chunk's FFNs after this call, and this call after the FFNs that
 * still read the `rows` it overwrites.
 *   layers: host array of n_layers descriptors; cache_rows [capacity x d_ff]
 *     device (may be NULL when capacity is 0); table [vocab x d_ff], pinned
 *     host (hipHostMalloc) or device, token rows table_stride elements apart
 *     (0: d_ff; larger for tables interleaved by staple_group_tables_host);
 *     rows [n x d_ff] device.  All 16-byte aligned.
 *   ids [n] device, 1 <= n < 2^31; id_to_slot [vocab] from staple_cache_build.
 *   uniq, inv, sorted_pos, code, miss_uidx [n], seg_start [n + 1], n_unique,
 *     n_miss [1]: device outputs.
 *   ws: staple_prefill_rows_workspace_bytes(n) bytes (0 up to 4096 tokens;
 *     then ws may be NULL).
 * The same bits as the three separate calls (and as
 * staple_assemble_rows_from_table per layer), whatever max_workgroups.
 * Argument errors return before anything is enqueued; IDs out of range are
 * reported through the device error word.
 * ------------------------------------------------------------------------ */
typedef struct staple_row_source {
  const void* cache_rows;
  const void* table;
  int64_t table_stride;
  void* rows;
} staple_row_source_t;

size_t staple_prefill_rows_workspace_bytes(int64_t n_tokens);
staple_status_t staple_prefill_rows_cached(
    int64_t n_layers, const staple_row_source_t* layers, int64_t n_tokens, int64_t d_ff,
    int32_t dtype, const int32_t* ids, int64_t vocab, const int32_t* id_to_slot,
    int64_t capacity, int32_t lookup, int32_t max_workgroups, int32_t* uniq, int32_t* inv,
    int32_t* sorted_pos, int32_t* seg_start, int32_t* n_unique, int32_t* code, int32_t* miss_uidx,
    int32_t* n_miss, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Low-rank tables.  The embedding dimension r is a capacity axis of STAPLE
 * next to the number of augmented layers, r = 512 being its low-rank variant
 * (STAPLE Table 2, row L=12, r=512; AI Radio episode, paper summary: rank
 * 512 makes the token-indexed table sixteen times smaller, d_ff / r at d_ff
 * 8192).  Reading taken: a layer keeps a table E_r [vocab x r] and a learned
 * projection P [d_ff x r], and the up branch adds Z = P E_r[t]:
 *
 *     u_i = W_up x_i + P E_r[t_i]
 *
 * Z depends on the token alone, so it is formed once per unique ID of the
 * batch and the layer runs as the full-width one with Z as its compact rows:
 *   forward : R_r = E_r[uniq] (staple_gather_rows), Z = staple_lowrank_expand,
 *             staple_ffn_fwd(rows = Z, row_index = inv);
 *   backward: staple_ffn_bwd_table_grad gives d_rows = dL/dZ, then
 *             staple_lowrank_bwd gives the table-row gradient
 *             dE_r[uniq[u]] = P^T d_rows[u] and dP = sum_u d_rows[u] R_r[u]^T.
 *
 * staple_lowrank_expand: z[u] = P rows_r[u] for u < *n_rows (device scalar,
 *   <= max_rows); rows_r [max_rows x r], proj [d_ff x r], z [max_rows x d_ff],
 *   all of `dtype` (bf16: fp32 accumulation, Z rounded to bf16 once).  Rows
 *   of z past *n_rows are not written.
 * staple_lowrank_bwd: d_rows [max_rows x d_ff] fp32 (rows < *n_rows read),
 *   rows_r as above, proj [d_ff x r] (dtype).  Outputs: d_rows_r
 *   [max_rows x r] fp32 (rows < *n_rows written), d_proj [d_ff x r] fp32
 *   (overwritten; zeros when *n_rows is 0).  bf16: d_rows is rounded to bf16
 *   as the operand of both contractions, which accumulate in fp32.
 *   ws: staple_lowrank_bwd_workspace_bytes(max_rows, d_ff, dtype) bytes (the
 *   rounded d_rows; none for fp32).
 * r and d_ff multiples of 64; 16-byte aligned pointers.
 * ------------------------------------------------------------------------ */
staple_status_t staple_lowrank_expand(const void* rows_r, const int32_t* n_rows, int64_t max_rows,
                                      int64_t r, int64_t d_ff, int32_t dtype, const void* proj,
                                      void* z, void* stream);
size_t staple_lowrank_bwd_workspace_bytes(int64_t max_rows, int64_t d_ff, int32_t dtype);
staple_status_t staple_lowrank_bwd(const float* d_rows, const void* rows_r, const int32_t* n_rows,
                                   int64_t max_rows, int64_t r, int64_t d_ff, int32_t dtype,
                                   const void* proj, float* d_rows_r, float* d_proj, void* ws,
                                   size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * AdamW step on the table rows a batch touched.  The tables are trained with
 * AdamW with fp32 moments beside the bf16 table (STAPLE Figure 4 caption:
 * bf16 tables and fp32 AdamW moments in host DRAM; Table 3: peak learning
 * rate and weight decay of the table group).  For each listed row r with
 * gradient g (one row of d_rows, e.g. staple_ffn_bwd_table_grad's output,
 * paired with staple_dedup's uniq), in fp32:
 *   p = p (1 - lr wd);  m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
 *   p = p - lr / (1 - b1^step) * m / (sqrt(v) / sqrt(1 - b2^step) + eps)
 * and p is stored in the table's dtype (bf16: round to nearest even).
 * Rows not listed keep their parameters and moments; `step` (>= 1) is the
 * global step count used for the bias corrections.  The pages give no betas
 * or epsilon; callers pass them (0.9, 0.999, 1e-8 are the usual defaults).
 *
 * staple_adamw_rows: device pointers.  table [vocab x d_ff] (dtype), m, v
 *   [vocab x d_ff] fp32, grad [max_rows x d_ff] fp32 (row k is the gradient
 *   of table row rows[k]); rows int32[max_rows], distinct; n_rows a device
 *   scalar (NULL: all max_rows).  d_ff a multiple of 8; 16-byte aligned
 *   pointers.  A row outside [0, vocab) sets the device error word and is
 *   skipped.  Asynchronous on `stream`.
 * staple_adamw_rows_host: the same update on host memory with host threads
 *   (n_threads <= 0: up to 16), synchronous; rows and grad are host arrays of
 *   n_rows entries; a row outside [0, vocab) returns STAPLE_ERR_HOST before
 *   anything is written.  The offloaded layout: the table and its moments in
 *   host memory, the gradient rows copied from the device first.
 * staple_cache_refresh: after an update of the host table, copies every
 *   updated row that is cached (code[u] >= 0, as from staple_cache_lookup)
 *   back into its cache slot: cache_rows[code[u]] = table[uniq[u]] for
 *   u < *n_unique.  table: device or pinned host memory; cache_rows
 *   [capacity x d_ff] device.  Out-of-range codes or IDs set the device error
 *   word.
 * ------------------------------------------------------------------------ */
staple_status_t staple_adamw_rows(void* table, float* m, float* v, int64_t vocab, int64_t d_ff,
                                  int32_t dtype, const int32_t* rows, const int32_t* n_rows,
                                  int64_t max_rows, const float* grad, float lr, float beta1,
                                  float beta2, float eps, float weight_decay, int64_t step,
                                  void* stream);
staple_status_t staple_adamw_rows_host(void* table, float* m, float* v, int64_t vocab, int64_t d_ff,
                                       int32_t dtype, const int32_t* rows, int64_t n_rows,
                                       const float* grad, float lr, float beta1, float beta2,
                                       float eps, float weight_decay, int64_t step,
                                       int32_t n_threads);
staple_status_t staple_cache_refresh(const void* table, int64_t vocab, int64_t d_ff, int32_t dtype,
                                     const int32_t* uniq, const int32_t* code,
                                     const int32_t* n_unique, int64_t max_unique, void* cache_rows,
                                     int64_t capacity, void* stream);

/* The host update overlapped with the GPU step (the pages' placement keeps
 * the tables and their AdamW moments in host DRAM and still trains within 3%
 * of dense: STAPLE Figure 4 caption; abstract).  A handle owns pinned staging
 * for the gradient rows, a "rows ready" event and a worker thread:
 *   staple_host_adamw_create: once, for up to max_rows rows of width d_ff
 *     (allocates pinned memory and events; not on a hot path).
 *   staple_host_adamw_event: the handle's rows-ready event (a hipEvent_t);
 *     pass it to staple_ffn_bwd_table_grad as rows_event, which records it
 *     right after d_rows is complete, before the weight-gradient GEMMs.
 *   staple_host_adamw_start: after that backward call, on the same thread;
 *     returns at once.  The worker waits for the event, copies *n_unique,
 *     uniq and then the gradient rows (in chunks) to the host on the GPU's
 *     DMA engines (no compute unit is used; copy_stream carries these
 *     copies instead when the DMA engines cannot be reached) and applies the
 *     update of staple_adamw_rows_host (same arguments; table, m, v host
 *     memory; n_threads <= 0: up to 14, leaving the caller's thread and the
 *     runtime a core) to each chunk as it lands, while the GPU goes on.  grad, uniq,
 *     n_unique: device memory (d_rows and staple_dedup's uniq, n_unique),
 *     unchanged until the update finishes; uniq holds at least max_rows
 *     entries (all max_rows are copied) and grad at least *n_unique rows of
 *     d_ff floats.  code, cache_rows, capacity: the batch's cache probe
 *     (staple_cache_lookup's code) and the HBM cache; when code is not NULL
 *     and capacity > 0 the worker also refreshes the cached copies of each
 *     updated chunk (staple_cache_refresh's operation, launched on
 *     copy_stream; the table must then be pinned).  copy_stream is made to
 *     wait for the rows-ready event first; give it a stream that does not
 *     carry the training step, so that the refreshes run beside the step
 *     (streams share a few hardware queues: two streams taken one after the
 *     other from a pool usually land on different ones).  A second start
 *     before finish returns STAPLE_ERR_INVALID_ARGUMENT.
 *   staple_host_adamw_finish: waits for the host update and returns its
 *     status (STAPLE_ERR_HOST for an ID outside the table,
 *     STAPLE_ERR_INDEX_RANGE for a row count past max_rows: nothing
 *     updated; for a failure part way, rows of earlier chunks may be
 *     updated); `stream` (NULL: the null stream) is made to wait for every
 *     refresh the update launched, whatever the status.  Read the host
 *     table, and the cache on another stream, only after it.
 *   staple_host_adamw_destroy: waits for a running update, then frees all.
 * The rows are updated by the same routine as staple_adamw_rows_host, each
 * once and independently: the same bits as the serial update. */
typedef struct staple_host_adamw staple_host_adamw_t;
staple_status_t staple_host_adamw_create(int64_t max_rows, int64_t d_ff, staple_host_adamw_t** out);
void* staple_host_adamw_event(staple_host_adamw_t* h);
staple_status_t staple_host_adamw_start(staple_host_adamw_t* h, void* table, float* m, float* v,
                                        int64_t vocab, int32_t dtype, const int32_t* uniq,
                                        const int32_t* n_unique, const float* grad, float lr,
                                        float beta1, float beta2, float eps, float weight_decay,
                                        int64_t step, int32_t n_threads, const int32_t* code,
                                        void* cache_rows, int64_t capacity, void* copy_stream);
staple_status_t staple_host_adamw_finish(staple_host_adamw_t* h, void* stream);
void staple_host_adamw_destroy(staple_host_adamw_t* h);

/* ------------------------------------------------------------------------
 * Backward of one augmented layer with the table-row gradient.
 *   dy [n_tokens x d_model] (dtype): upstream gradient of y.
 *   saved_g, saved_u: the forward's save_g/save_u (required).
 *   saved_h: the forward's save_h, or NULL: h is then recomputed from the
 *     saved g and u (h = silu(g) * u, rounded to dtype) into the workspace,
 *     so dw_down may differ from a call with the forward's h by the rounding
 *     of g and u; every other output is the same either way.
 *   sorted_pos, inv, seg_start, n_unique: staple_dedup's outputs for this batch;
 *     *n_unique <= max_unique (a larger value sets the device error word and
 *     d_rows is not written).
 * Outputs (each overwritten, not accumulated):
 *   d_rows [max_unique x d_ff] fp32: row u (< *n_unique) is the sum, over the
 *     positions holding token uniq[u], of dL/du at that position (a plain sum,
 *     no averaging).
 *   dx [n_tokens x d_model] of out_dtype.
 *   dw_gate, dw_up [d_ff x d_model] fp32; dw_down [d_model x d_ff] fp32.
 *   freeze_up != 0: the up-projection is frozen (STAPLE Table 3 caption:
 *     frozen during warmup); dw_up is neither computed nor written (may be
 *     NULL) while the gradient still flows through W_up into dx and d_rows.
 *   w_up NULL: the STEM layer (saved_u = E[t] from its forward); dx = dL/dg
 *     W_gate, d_rows as above, dw_up neither computed nor written.
 *   rows_event: a hipEvent_t or NULL; when given it is recorded on `stream`
 *     right after d_rows is complete (before the weight- and input-gradient
 *     GEMMs), e.g. staple_host_adamw_event's, so the rows can leave for the
 *     host while the rest of the backward runs.
 * In bf16 the backward reads bf16 g and u, forms dL/du and dL/dg in fp32 and
 * rounds them to bf16 once, as operands of the weight- and input-gradient
 * contractions; every contraction accumulates in fp32; d_rows sums the fp32
 * dL/du values before that rounding, in fp32 (a fixed order: the result is
 * deterministic).
 * Workspace (staple_ffn_bwd_workspace_bytes): [dg | du] of n_tokens x 2 d_ff
 * (dtype), an n_tokens x d_ff fp32 block (fp32 dL/du, then the recomputed
 * h), and the segment sum's partial rows.
 * ------------------------------------------------------------------------ */
size_t staple_ffn_bwd_workspace_bytes(int64_t n_tokens, int64_t d_model, int64_t d_ff,
                                      int32_t dtype);
staple_status_t staple_ffn_bwd_table_grad(int64_t n_tokens, int64_t d_model, int64_t d_ff,
                                          int32_t dtype, int32_t out_dtype,
                                          const void* dy, const void* x,
                                          const void* w_gate, const void* w_up, const void* w_down,
                                          const void* saved_g, const void* saved_u,
                                          const void* saved_h,
                                          const int32_t* sorted_pos, const int32_t* inv,
                                          const int32_t* seg_start,
                                          const int32_t* n_unique, int64_t max_unique,
                                          float* d_rows, void* dx,
                                          float* dw_gate, float* dw_up, float* dw_down,
                                          int32_t freeze_up, void* ws, size_t ws_bytes,
                                          void* rows_event, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* STAPLE_H */
