/*
 * infllm.h -- C ABI of libinfllm.so: InfLLM's context-memory attention step
 * on one AMD Instinct MI355X (gfx950).
 *
 * The method (InfLLM: Training-Free Long-Context Extrapolation for LLMs with
 * an Efficient Context Memory; summary page, "Approach"; InfLLM Guide blog,
 * "Core Innovation 1" and "Core Innovation 2"): the distant part of the KV
 * cache is cut into fixed-size memory units; each unit is represented by its
 * top-scoring representative keys (or by the mean of its keys); every query
 * chunk scores all units, keeps the best k_m per KV head, and attends over
 * the initial tokens, the retrieved units and a local sliding window.
 *
 * The four calls mirror that statement:
 *   infllm_build_units  -- representative-token selection per unit
 *                          (infllm_build_units_range: a range of units, as
 *                          they leave the window while streaming;
 *                          infllm_build_units_qsum: also the block query
 *                          sums, for infllm_score_units_qsum)
 *   infllm_score_units  -- chunk-query . unit-representation scores
 *                          (infllm_score_units_varlen: a position per sequence)
 *   infllm_topk_units   -- top-k_m units per (sequence, KV head, chunk)
 *                          (infllm_select_units: scores and top-k together)
 *   infllm_attend       -- exact softmax attention over the working context
 *                          (infllm_attend_varlen: a position per sequence)
 *
 * Conventions shared by every call
 * --------------------------------
 *  Layout.  Q is [batch, n_q_heads, q_cap, head_dim] and K, V are
 *    [batch, n_kv_heads, kv_cap, head_dim], dense row-major, element type
 *    cfg->dtype (fp32, or bf16 stored as its 16-bit pattern).  Row t of a
 *    K/V head is absolute position t.  Query head g reads KV head g / G with
 *    G = n_q_heads / n_kv_heads.
 *  Pointers.  Every tensor pointer is a device pointer, 16-byte aligned.
 *    The library never dereferences them on the host.
 *  Ownership.  The caller allocates every buffer, including the workspace
 *    (size from infllm_workspace_size).  The library allocates nothing,
 *    keeps no state between calls and is re-entrant.
 *  Asynchrony.  Each call validates its arguments on the host, then only
 *    enqueues kernels on `stream` (a hipStream_t; NULL = the null stream)
 *    and returns; it never synchronises.  Device faults surface at the
 *    caller's next synchronisation.
 *  Errors.  Invalid arguments return INFLLM_ERR_INVALID_ARG (or
 *    INFLLM_ERR_UNSUPPORTED / INFLLM_ERR_WORKSPACE) before any device
 *    work is enqueued; a failed launch returns INFLLM_ERR_HIP.  Nothing is
 *    thrown across the ABI.
 *  Workspaces.  A workspace that carries counters (score calls with long
 *    chunks, the selection, split attention, the decode step) starts with
 *    a 256-byte header -- its first int32 counts waits of the decode step
 *    that timed out (infllm_workspace_status), its second the rows of the
 *    one-launch step that an attention workgroup selected itself, its
 *    third the units of a TOKENS build that summed their window's query
 *    rows themselves because a block sum they could have used was not
 *    published in time (diagnostics; all only grow) -- followed by a counter
 *    region of at least 64 KiB, then the call's data (partial sums and
 *    rows).  It must be zero-filled before its first use; every call
 *    leaves its counters at zero again.  Since every call kind keeps its
 *    counters in that region, one zero-filled workspace may serve calls of
 *    other kinds and shapes (if large enough) as long as each call's
 *    counters fit the first 64 KiB of the region (infllm_workspace_layout
 *    reports a call's region; e.g. a decode step needs 16 bytes per
 *    (sequence, KV head, position)).  A call whose counters need more
 *    binds the workspace to its own shape: zero-fill it again before
 *    other calls use it.  Calls that share a workspace must not overlap
 *    in time.
 *  Tuning.  The environment variables INFLLM_PREFILL_SPLITS,
 *    INFLLM_ROWS_WGS and INFLLM_STEP_SPLITS override split counts of the
 *    chunk attention, the decode attention and the one-launch decode step
 *    (workgroups per row); INFLLM_STEP_PRESPIN (0 .. 2^20) the polls of
 *    the one-launch step's attention workgroups for the row's selection
 *    before they select it themselves (same result, more work);
 *    INFLLM_BUILD_SPIN (0 .. 2^20) the polls of a TOKENS build's unit for
 *    the block sums it uses before it sums the query rows itself (0: it
 *    always does; the same selection up to rounding, more work).  They are
 *    read once per process, at the first call that needs them; workspace
 *    sizes follow them.
 *  Units.  Unit u is absolute block j = u + floor(n_init / block); its keys
 *    are positions [max(j*block, n_init), (j+1)*block).  A context of n_ctx
 *    tokens holds floor(n_ctx/block) - floor(n_init/block) units (blocks
 *    aligned to multiples of the unit size, as in the guide's figure of a
 *    unit spanning tokens 1024..1151).
 *  Chunks.  The query-chunk calls take `n_chunks` consecutive chunks of
 *    `chunk_len` queries: chunk c holds rows q_off + c*chunk_len ... of the
 *    Q buffer, at absolute positions q_pos + c*chunk_len ....  Each chunk has
 *    its own unit selection (retrieval during pre-filling is done per block
 *    of queries: authors' rebuttal, "Comparison to Well-trained Long LLM").
 *    A decode step is one chunk of length 1.
 */
#ifndef INFLLM_H
#define INFLLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define INFLLM_ABI_VERSION 2

#if defined(__GNUC__) || defined(__clang__)
#define INFLLM_API __attribute__((visibility("default")))
#else
#define INFLLM_API
#endif

typedef enum {
  INFLLM_OK = 0,
  INFLLM_ERR_INVALID_ARG = -1, /* a pointer, size or config field is invalid */
  INFLLM_ERR_UNSUPPORTED = -2, /* valid, but outside what the kernels handle */
  INFLLM_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  INFLLM_ERR_HIP = -4          /* a HIP launch failed */
} infllm_status;

typedef enum { INFLLM_F32 = 0, INFLLM_BF16 = 1 } infllm_dtype;

/* Unit representation: top-r_k representative tokens (summed), or the mean
 * of the unit's keys (summary page, "Measured effects": representative
 * tokens versus mean key vectors). */
typedef enum { INFLLM_REP_TOKENS = 0, INFLLM_REP_MEAN = 1 } infllm_rep_mode;

typedef enum {
  INFLLM_CALL_BUILD = 0,
  INFLLM_CALL_SCORE = 1,
  INFLLM_CALL_TOPK = 2,
  INFLLM_CALL_ATTEND = 3,
  INFLLM_CALL_BUILD_RANGE = 4,
  INFLLM_CALL_SELECT = 5,
  INFLLM_CALL_BUILD_QSUM = 6,
  INFLLM_CALL_SELECT_ATTEND = 7
} infllm_call;

typedef struct {
  int32_t n_q_heads;  /* H_q >= 1, multiple of n_kv_heads                  */
  int32_t n_kv_heads; /* H_kv >= 1                                          */
  int32_t head_dim;   /* d: 64 or 128                                       */
  int32_t block;      /* unit size B: multiple of 64, 64..1024              */
  int32_t n_init;     /* initial (sink) tokens, >= 0                        */
  int32_t window;     /* local window W >= 1: query t sees t-W+1 .. t       */
  int32_t rep_k;      /* representative tokens per unit, 1..block (TOKENS)  */
  int32_t top_k;      /* units retrieved per chunk k_m, 0..256              */
  int32_t rep_mode;   /* infllm_rep_mode                                    */
  int32_t dtype;      /* infllm_dtype of Q, K, V and the attention output  */
  double rope_theta;  /* 0: attention takes q and k as they are.  > 0: RoPE
                       * base theta; q and k hold vectors rotated at their
                       * absolute positions (rotate-half pairs (c, c + d/2)
                       * turned by p * theta^(-2c/d)), and the attention
                       * calls re-position every token to its place in the
                       * working context (below).  Build and scoring calls
                       * take q and k as they are either way.              */
} infllm_config;

/* Positions inside the working context (rope_theta > 0; InfLLM Guide,
 * "Operational Checklist", RoPE item: the native base is kept and memory
 * units take local relative offsets).  For the chunk whose first query is
 * at t0, with lo = max(n_init, t0 - W + 1):
 *   initial token p < n_init              sits at p
 *   key p of the unit in sel slot m       sits at n_init + m*B + (p mod B)
 *   token p >= lo (window keys, queries)  sits at n_init + k_m*B + (p - lo)
 * A key in both a selected unit and [lo, t0 + chunk_len) takes the last
 * rule; a repeated id takes its first slot.  Each attended logit is that of
 * q and k turned from their absolute positions to these ones (fp64 angle
 * reduction, fp32 rotation; the bf16 MFMA path rounds the turned keys of
 * initial and unit tokens to bf16). */

/* Units held by a context of n_ctx tokens: floor(n_ctx/B) - floor(n_init/B),
 * or 0.  Returns -1 for an invalid config. */
INFLLM_API int32_t infllm_num_units(const infllm_config *cfg, int64_t n_ctx);

/* Units eligible for a chunk whose last query is at position t_last: those
 * whose first key lies at or before t_last - W (a unit key is attended only
 * while it is outside the local window).  They form the prefix
 * [0, result) of [0, n_units).  Returns -1 for an invalid config. */
INFLLM_API int32_t infllm_num_eligible(const infllm_config *cfg, int64_t t_last, int32_t n_units);

/* Workspace bytes `call` needs for the given sizes (0 if none).  For BUILD
 * pass n = n_ctx; for BUILD_RANGE n = u_end - u_begin; for SCORE/TOPK/ATTEND
 * pass the chunk geometry (n unused for TOPK, which takes n_units in `n`). */
INFLLM_API size_t infllm_workspace_size(const infllm_config *cfg, int32_t call, int32_t batch, int64_t n,
                             int32_t chunk_len, int32_t n_chunks);

/*
 * infllm_build_units -- unit representations for a context of n_ctx tokens.
 *
 * TOKENS (summary page, "Approach": each unit is represented by its top-
 * scoring tokens chosen with attention-based scores; authors' rebuttal,
 * "Representative Tokens": the model selects discrete tokens).  Key p of
 * KV head h scores
 *     s_p = sum_{g in group(h)} sum_{i = p+1}^{min(p+W, n_ctx-1)} q_i^(g) . k_p
 * (raw, unscaled; the queries that follow it inside one local window).
 * Per unit the r_k keys with the highest s_p are kept (ties: lower
 * position), listed in ascending position in rep_idx, and the unit is
 * represented by their sum.  Scores are accumulated in fp64.
 * MEAN: the representation is the mean of the unit's keys; rep_idx unused.
 *
 *   q          [batch, H_q, q_cap, d]  queries of positions 0 .. n_ctx-1
 *   k          [batch, H_kv, kv_cap, d]
 *   n_ctx      context tokens, 1 <= n_ctx <= min(q_cap, kv_cap)
 *   rep_idx    out [batch, H_kv, U, r_k] int32 absolute positions, -1 pads
 *              (TOKENS; may be NULL for MEAN)
 *   unit_repr  out [batch, H_kv, U, d] fp32, U = infllm_num_units(n_ctx)
 *   workspace  >= infllm_workspace_size(cfg, INFLLM_CALL_BUILD, batch, n_ctx, 0, 0),
 *              zero-filled before its first use (TOKENS: it carries flags of
 *              published block sums, which every call leaves at zero)
 * TOKENS runs as one launch that reads the queries about once: one
 * workgroup per block, from the last block back, publishes its block's
 * query sum; each unit's window sums take the published sums of the blocks
 * after it (or sum them itself when one is not published yet: nothing
 * waits).
 */
INFLLM_API infllm_status infllm_build_units(const infllm_config *cfg, int32_t batch, const void *q,
                                 int64_t q_cap, const void *k, int64_t kv_cap, int64_t n_ctx,
                                 int32_t *rep_idx, float *unit_repr, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * infllm_build_units_qsum -- infllm_build_units that also writes the block
 * query sums it forms on the way (TOKENS), or forms them (MEAN):
 *     block_qsum[b][h][j] = sum over rows jB .. min((j+1)B, n_ctx) - 1 and
 *                           the group's query heads of q       (fp64)
 * for every block j < ceil(n_ctx / B), including those of the initial
 * tokens.  A chunk made of whole blocks sums its blocks' entries to get
 * its query sum (infllm_score_units_qsum), so the encoding pass reads the
 * queries for its chunk scores once instead of twice.
 *
 *   q          required in both modes
 *   block_qsum out [batch, H_kv, ceil(n_ctx/B), d] fp64, 16-byte aligned
 *   workspace  >= infllm_workspace_size(cfg, INFLLM_CALL_BUILD_QSUM, batch,
 *              n_ctx, 0, 0), zero-filled before its first use (TOKENS), as
 *              for infllm_build_units
 * Other arguments, outputs and errors as infllm_build_units.
 */
INFLLM_API infllm_status infllm_build_units_qsum(const infllm_config *cfg, int32_t batch,
                                      const void *q, int64_t q_cap, const void *k,
                                      int64_t kv_cap, int64_t n_ctx, int32_t *rep_idx,
                                      float *unit_repr, double *block_qsum, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * infllm_build_units_range -- the same representations for units u_begin ..
 * u_end-1 only: the streaming form, where a unit is added to the memory
 * when its tokens leave the local window (summary page, "Approach":
 * distant tokens are stored into memory units).  Scores use the queries
 * of positions < n_ctx, i.e. the windows are truncated at the current
 * position; a unit whose last key is at or before n_ctx-1-W (all its keys
 * have left the window of position n_ctx-1) gets exactly what a build of
 * any longer context gives it.  Work and workspace
 * grow with the number of units (plus ceil(W/B)+1 blocks of queries), not
 * with n_ctx; one launch (the blocks past the range that its windows reach
 * get workgroups that only publish their sums).
 *
 *   q, k, n_ctx     as infllm_build_units
 *   u_begin, u_end  0 <= u_begin <= u_end <= infllm_num_units(n_ctx)
 *   pool_units      unit capacity (row count) of rep_idx / unit_repr, >= u_end
 *   rep_idx    out rows u_begin .. u_end-1 of [batch, H_kv, pool_units, r_k]
 *              (TOKENS; may be NULL for MEAN); other rows untouched
 *   unit_repr  out rows u_begin .. u_end-1 of [batch, H_kv, pool_units, d]
 *   workspace  >= infllm_workspace_size(cfg, INFLLM_CALL_BUILD_RANGE, batch,
 *              u_end - u_begin, 0, 0), zero-filled before its first use
 *              (TOKENS: flags that every call leaves at zero)
 */
INFLLM_API infllm_status infllm_build_units_range(const infllm_config *cfg, int32_t batch,
                                       const void *q, int64_t q_cap, const void *k,
                                       int64_t kv_cap, int64_t n_ctx, int32_t u_begin,
                                       int32_t u_end, int32_t pool_units, int32_t *rep_idx,
                                       float *unit_repr, void *workspace,
                                       size_t workspace_bytes, void *stream);

/*
 * infllm_score_units -- relevance of every unit to each query chunk.
 *
 * (InfLLM Guide, "Core Innovation 2", item 2: a dot product of the query
 * against every unit representation; authors' rebuttal, "Latency Across
 * Different Context Windows": the lookup takes the dot product with all unit
 * representations.)  For chunk c and KV head h:
 *     score[u] = (sum over the chunk's queries and the group's query heads
 *                 of q) . unit_repr[u]              for u < e_c,
 *     score[u] = -inf                               otherwise,
 * with e_c = infllm_num_eligible(position of the chunk's last query).  The
 * query sum and the dot product are accumulated in fp64.
 *
 *   q          [batch, H_q, q_cap, d]; rows q_off .. q_off + n_chunks*chunk_len - 1
 *   q_pos      absolute position of row q_off
 *   unit_repr  [batch, H_kv, n_units, d] fp32 (from infllm_build_units)
 *   scores     out [batch, H_kv, n_chunks, n_units] fp32
 *   workspace  >= infllm_workspace_size(cfg, INFLLM_CALL_SCORE, batch, 0,
 *              chunk_len, n_chunks): arrival counters and fp64 partial query
 *              sums (0 bytes for short chunks).  It must be zero-filled before
 *              its first use; every call leaves the counters at zero again,
 *              and calls that share a workspace must not overlap in time.
 */
INFLLM_API infllm_status infllm_score_units(const infllm_config *cfg, int32_t batch, const void *q,
                                 int64_t q_cap, int64_t q_off, int64_t q_pos, int32_t chunk_len,
                                 int32_t n_chunks, const float *unit_repr, int32_t n_units,
                                 float *scores, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * infllm_score_units_varlen -- infllm_score_units for a batch of sequences
 * at different positions (a serving batch: one decode step, or one chunk
 * of prefill, per sequence).  Same arguments, except:
 *
 *   pos        device [batch] int64, 8-byte aligned: absolute position of
 *              row q_off of sequence b (replaces q_pos).  Read on the
 *              device, so it can be updated there between calls.  A
 *              negative position leaves no unit eligible; e_c is capped at
 *              n_units, as in infllm_score_units.
 *
 * Row b equals row b of infllm_score_units called with q_pos = pos[b] on
 * the same batch (bit for bit).  Workspace: INFLLM_CALL_SCORE, same sizes.
 */
INFLLM_API infllm_status infllm_score_units_varlen(const infllm_config *cfg, int32_t batch,
                                        const void *q, int64_t q_cap, int64_t q_off,
                                        const int64_t *pos, int32_t chunk_len, int32_t n_chunks,
                                        const float *unit_repr, int32_t n_units, float *scores,
                                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * infllm_score_units_qsum -- infllm_score_units for chunks made of whole
 * blocks, with the chunk query sums taken from block query sums
 * (infllm_build_units_qsum) instead of the queries: chunk c's sum is the
 * sum of the entries of its chunk_len / B blocks, added in block order in
 * fp64.  The same scores as infllm_score_units up to the fp64 rounding of
 * the sums' order.
 *
 *   block_qsum  [batch, H_kv, n_blocks, d] fp64
 *   q_pos       position of the first chunk's first query, a multiple of B
 *   chunk_len   a multiple of B; (q_pos + n_chunks*chunk_len) / B <= n_blocks
 *   unit_repr, n_units, scores   as infllm_score_units
 * No workspace.
 */
INFLLM_API infllm_status infllm_score_units_qsum(const infllm_config *cfg, int32_t batch,
                                      const double *block_qsum, int64_t n_blocks, int64_t q_pos,
                                      int32_t chunk_len, int32_t n_chunks,
                                      const float *unit_repr, int32_t n_units, float *scores,
                                      void *stream);

/*
 * infllm_select_units -- infllm_score_units followed by infllm_topk_units,
 * in one launch where the chunks are short (decode: the last slice of units
 * of a (sequence, KV head, chunk) to finish scoring selects that row's
 * units), in two otherwise.  Results are identical to the two calls.
 *
 *   q, q_cap, q_off, chunk_len, n_chunks, unit_repr, n_units
 *              as infllm_score_units
 *   q_pos      absolute position of row q_off (used when pos is NULL)
 *   pos        NULL, or device [batch] int64, 8-byte aligned: a position
 *              per sequence, as infllm_score_units_varlen
 *   scores     out [batch, H_kv, n_chunks, n_units] fp32 (also the
 *              selection's input)
 *   sel        out [batch, H_kv, n_chunks, k_m] int32, as infllm_topk_units
 *   workspace  >= infllm_workspace_size(cfg, INFLLM_CALL_SELECT, batch, 0,
 *              chunk_len, n_chunks): arrival counters (and the scoring
 *              workspace).  Zero-filled before its first use; every call
 *              leaves the counters at zero; calls that share a workspace
 *              must not overlap in time.
 */
INFLLM_API infllm_status infllm_select_units(const infllm_config *cfg, int32_t batch, const void *q,
                                  int64_t q_cap, int64_t q_off, int64_t q_pos,
                                  const int64_t *pos, int32_t chunk_len, int32_t n_chunks,
                                  const float *unit_repr, int32_t n_units, float *scores,
                                  int32_t *sel, void *workspace, size_t workspace_bytes,
                                  void *stream);

/*
 * infllm_topk_units -- keep the k_m best units per (sequence, KV head,
 * chunk) (InfLLM Guide, "Core Innovation 2", item 2: the top-k highest-
 * scoring units are loaded for exact attention).
 *
 * Among the finite scores, min(k_m, #finite) units are kept by (score
 * descending, unit index ascending) and written in ascending index order;
 * remaining slots are -1.  -inf marks an ineligible unit and is never kept.
 *
 *   scores  [batch, H_kv, n_chunks, n_units] fp32, no NaN
 *   sel     out [batch, H_kv, n_chunks, k_m] int32
 */
INFLLM_API infllm_status infllm_topk_units(const infllm_config *cfg, int32_t batch, int32_t n_chunks,
                                const float *scores, int32_t n_units, int32_t *sel,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * infllm_attend -- exact attention over the working context (InfLLM Guide,
 * "Core Innovation 2", item 3, the Working Context equation: sinks, the
 * retrieved units and the local window; "Core Innovation 1", items 1-2).
 *
 * Query t (chunk c) of query head g attends the keys p <= t with
 *     p < n_init                                  (initial tokens), or
 *     t - W < p                                   (local window, t included), or
 *     n_init <= p <= t - W and unit(p) in sel_c   (retrieved units),
 * softmax(q.k_p / sqrt(d)) . V, fp32 online softmax (bf16 MFMA products for
 * bf16 inputs).  The output is rounded to the input dtype.
 *
 *   q        [batch, H_q, q_cap, d]; rows q_off .., positions q_pos ..
 *   k, v     [batch, H_kv, kv_cap, d]; must hold every attended position
 *            (q_pos + n_chunks*chunk_len <= kv_cap)
 *   sel      [batch, H_kv, n_chunks, k_m] int32 unit ids (-1 = empty slot),
 *            e.g. from infllm_topk_units; ids must be < the number of units
 *            the K/V context holds (not checked on the device).  A row is
 *            a set: an id repeated in it is attended once, like the
 *            working context's membership test above.
 *   out      out [batch, H_q, out_cap, d], rows out_off .. out_off +
 *            n_chunks*chunk_len - 1, cfg->dtype
 *   lse      optional out [batch, H_q, out_cap] fp32 natural-log
 *            sum-exp of the scaled logits, same rows; may be NULL
 *   workspace >= infllm_workspace_size(cfg, INFLLM_CALL_ATTEND, batch, 0,
 *            chunk_len, n_chunks).  It must be zero-filled before its first
 *            use: it holds split-K arrival counters, which every call leaves
 *            at zero again.  Calls that share a workspace must not overlap.
 */
INFLLM_API infllm_status infllm_attend(const infllm_config *cfg, int32_t batch, const void *q, int64_t q_cap,
                            int64_t q_off, int64_t q_pos, int32_t chunk_len, int32_t n_chunks,
                            const void *k, const void *v, int64_t kv_cap, const int32_t *sel,
                            void *out, float *lse, int64_t out_cap, int64_t out_off,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * infllm_attend_varlen -- infllm_attend for a batch of sequences at
 * different positions.  Same arguments, except:
 *
 *   pos      device [batch] int64, 8-byte aligned: absolute position of
 *            row q_off of sequence b (replaces q_pos); sequence b attends
 *            its own K/V rows up to pos[b] + n_chunks*chunk_len - 1.
 *   kv_cap   must be >= n_chunks*chunk_len.
 *
 * The positions are checked on the device: a sequence with pos[b] < 0,
 * pos[b] + n_chunks*chunk_len > kv_cap or beyond 2^31 - 128 reads nothing
 * and gets NaN output rows (and NaN lse); the other sequences are
 * unaffected and the workspace stays valid.  Row b equals row b of
 * infllm_attend called with q_pos = pos[b] on the same batch (bit for
 * bit).  Workspace: INFLLM_CALL_ATTEND, same sizes.
 */
INFLLM_API infllm_status infllm_attend_varlen(const infllm_config *cfg, int32_t batch,
                                   const void *q, int64_t q_cap, int64_t q_off,
                                   const int64_t *pos, int32_t chunk_len, int32_t n_chunks,
                                   const void *k, const void *v, int64_t kv_cap,
                                   const int32_t *sel, void *out, float *lse, int64_t out_cap,
                                   int64_t out_off, void *workspace, size_t workspace_bytes,
                                   void *stream);

/*
 * infllm_select_attend -- one decode step: for each of n_pos consecutive
 * query positions (each a chunk of one query), score every unit, keep the
 * top k_m per KV head and attend over the working context (the lookup and
 * the attention of InfLLM Guide, "Core Innovation 2", items 2-3; SUMMARY,
 * Approach: each step looks up the relevant units and attends them with
 * the local window).  The result is that of infllm_select_units (chunk_len
 * 1, n_chunks n_pos) followed by infllm_attend or infllm_attend_varlen on
 * its selection: scores and sel are identical; out and lse equal up to fp32
 * rounding (the attention is split over workgroups differently).
 *
 * Where the shapes allow (bf16, k_m >= 1, a row's scores few enough to be
 * searched at once: up to 2,048 units; with rope_theta > 0 also head_dim
 * 128 and at most 4 query heads per KV head) it is one launch: in each
 * (sequence, KV head, position) row some workgroups score a slice of units
 * each and publish the scores, a selector workgroup selects the row's units
 * from them and publishes the selection, and every attention workgroup
 * attends its share of the local keys (initial tokens and window), then of
 * the selected units' keys.  A workgroup waits for the row's scores only
 * after checking that every slice of its row has been started, scoring the
 * ones that have not itself, and for the selector only a bounded time
 * before selecting the row itself (the same units), so the waits end
 * whatever the dispatch order or residency.  Otherwise it runs the two calls.  With INFLLM_STEP_SPLITS
 * set, rows of up to 64 x 256 units also take the one launch: each slice
 * then publishes only its best k_m scores (the row's top k_m is among
 * them).  infllm_step_plan reports which form a call takes.
 *
 *   q, q_cap, q_off, q_pos, pos, unit_repr, n_units
 *              as infllm_select_units (pos: as infllm_attend_varlen)
 *   k, v, kv_cap, out, lse, out_cap, out_off
 *              as infllm_attend, for n_pos positions
 *   scores     out [batch, H_kv, n_pos, n_units] fp32
 *   sel        out [batch, H_kv, n_pos, k_m] int32
 *   workspace  >= infllm_workspace_size(cfg, INFLLM_CALL_SELECT_ATTEND,
 *              batch, n_units, 1, n_pos).  Zero-filled before its first
 *              use; every call leaves it ready for the next; calls that
 *              share a workspace must not overlap in time.
 * Errors: as the two calls, checked before anything is enqueued.
 */
INFLLM_API infllm_status infllm_select_attend(const infllm_config *cfg, int32_t batch,
                                   const void *q, int64_t q_cap, int64_t q_off, int64_t q_pos,
                                   const int64_t *pos, int32_t n_pos, const float *unit_repr,
                                   int32_t n_units, const void *k, const void *v,
                                   int64_t kv_cap, float *scores, int32_t *sel, void *out,
                                   float *lse, int64_t out_cap, int64_t out_off,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * infllm_select_attend_static -- infllm_select_attend without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  It
 * allocates nothing: the step's workspace is a scratch array of 16 MiB
 * inside the library, one per GPU (each GPU that runs it holds the array
 * until the process ends; the current device's copy is used, its address
 * taken once per device), zero-filled at load and left with its counters
 * at zero by every call.
 *
 * Arguments, results and errors as infllm_select_attend, except:
 * INFLLM_ERR_WORKSPACE when the step needs more than the 16 MiB
 * (infllm_workspace_size(cfg, INFLLM_CALL_SELECT_ATTEND, batch, n_units,
 * 1, n_pos)) or more than the 64 KiB counter region (16 bytes per
 * (sequence, KV head, position) in the separate-call form, 80 in the
 * one-launch form); INFLLM_ERR_HIP when the array's address cannot be
 * obtained.  Every call on a GPU shares that GPU's array: calls that
 * overlap in time on one GPU (other streams, other threads) race and give
 * wrong results.  The status word of infllm_workspace_status is not
 * readable for it.
 */
INFLLM_API infllm_status infllm_select_attend_static(
    const infllm_config *cfg, int32_t batch, const void *q, int64_t q_cap, int64_t q_off,
    int64_t q_pos, const int64_t *pos, int32_t n_pos, const float *unit_repr, int32_t n_units,
    const void *k, const void *v, int64_t kv_cap, float *scores, int32_t *sel, void *out,
    float *lse, int64_t out_cap, int64_t out_off, void *stream);

/*
 * infllm_workspace_layout -- where a call keeps its counters: bytes
 * [*counters_begin, *counters_end) of its workspace (both 0 if it has
 * none), and *total = infllm_workspace_size of the same arguments.  Host
 * only.  Returns INFLLM_OK, or INFLLM_ERR_INVALID_ARG (outputs zeroed).
 */
INFLLM_API int32_t infllm_workspace_layout(const infllm_config *cfg, int32_t call, int32_t batch,
                                           int64_t n, int32_t chunk_len, int32_t n_chunks,
                                           size_t *counters_begin, size_t *counters_end,
                                           size_t *total);

/*
 * infllm_step_plan -- how infllm_select_attend runs a step of the given
 * sizes (host only).  plan[0..6] = {one launch (1) or the two calls (0),
 * workgroups per row, scoring workgroups per row, units each scores,
 * candidates each publishes, local-key weight of a scoring workgroup, of a
 * unit workgroup}; all 0 for the two calls.  Returns INFLLM_OK or
 * INFLLM_ERR_INVALID_ARG.
 */
INFLLM_API int32_t infllm_step_plan(const infllm_config *cfg, int32_t batch, int32_t n_units,
                                    int32_t n_pos, int32_t *plan);

/*
 * infllm_workspace_status -- synchronises `stream`, then reads the header
 * word of a workspace used by infllm_select_attend: the number of waits for
 * a row's selection that hit their bound since the workspace was zero-
 * filled (rows concerned got NaN outputs).  Every wait ends on its own
 * (see infllm_select_attend), so a nonzero count means the workspace was
 * not zero-filled or was shared by calls that overlapped in time.  The
 * only call that synchronises.  Returns INFLLM_OK, INFLLM_ERR_INVALID_ARG
 * or INFLLM_ERR_HIP.
 */
INFLLM_API int32_t infllm_workspace_status(const void *workspace, size_t workspace_bytes,
                                           int32_t *timeouts, void *stream);

/*
 * Unit cache -- every unit's K/V in host memory, a pool of n_slots hot
 * units per (sequence, KV head) in GPU memory, for contexts whose K/V do
 * not fit the GPU (InfLLM Guide, "Core Innovation 3": a least-recently-used
 * GPU pool of hot units over host-resident units; the representatives stay
 * on the GPU for scoring).  A decode step is then infllm_select_units,
 * infllm_cache_fetch and infllm_attend_cached on one stream; fetch and
 * attention take the same sel.
 *
 * Cache state: a caller-owned device buffer of infllm_cache_state_size
 * bytes, zero-filled before first use (zero = empty cache): a 256-byte
 * header (int64 hits, int64 misses: totals since zero-filled), then per
 * (sequence, KV head) the slot of each unit, the unit of each slot and the
 * step that last used each slot.  Returns 0 for an invalid shape.
 * Limits: n_units <= 65,536, n_slots <= 1,024.
 */
INFLLM_API size_t infllm_cache_state_size(const infllm_config *cfg, int32_t batch,
                                          int32_t n_units, int32_t n_slots);

/*
 * infllm_cache_fetch -- makes every unit of sel resident, per (sequence,
 * KV head), without a host round trip: one workgroup per (sequence, KV
 * head) reads sel on the device, updates the tables, and copies each
 * missed unit's block (B rows of K and of V) from host memory into its
 * slot with the GPU's own loads over the host link.  Policy: the selected
 * units already cached are hits (last use = step); the others, ascending by
 * unit id, take the slots no selected unit holds, least recently used first
 * (empty slots first, lower slot first among equals), evicting their units.
 *
 *   sel       device [batch, H_kv, n_pos, k_m] int32 unit ids (-1 = empty;
 *             ids outside [0, n_units) and repeats are ignored); the union
 *             of a (sequence, KV head)'s n_pos rows must fit: n_pos * k_m
 *             <= n_slots (checked)
 *   step      >= 1, larger than every step passed before on this state (not
 *             checked; equal steps protect the earlier call's units too)
 *   k_host,   pinned host memory the GPU reads at the same address
 *   v_host    (hipHostMalloc; other memory: INFLLM_ERR_INVALID_ARG),
 *             [batch, H_kv, host_cap, d], row p = position p; must hold
 *             every unit's block: host_cap >= (n_units + n_init/B) * B
 *   cache_k,  device [batch, H_kv, n_slots, B, d], cfg->dtype: slot c holds
 *   cache_v   the block of unit_of[c] (rows below n_init of unit 0 unused)
 *   state     the cache state (above)
 * Calls on one state must not overlap in time.
 */
INFLLM_API infllm_status infllm_cache_fetch(const infllm_config *cfg, int32_t batch,
                                            int32_t n_pos, const int32_t *sel, int32_t n_units,
                                            int64_t step, const void *k_host, const void *v_host,
                                            int64_t host_cap, void *cache_k, void *cache_v,
                                            int32_t n_slots, void *state, void *stream);

/*
 * infllm_attend_cached -- infllm_attend of n_pos single positions (chunks
 * of one, as in decoding) whose units' keys come from the unit cache.  The
 * result is bit for bit that of infllm_attend (chunk_len 1, n_chunks n_pos)
 * over the full K/V.
 *
 *   q, q_cap, q_off, q_pos, pos, sel, out, lse, out_cap, out_off
 *             as infllm_attend / infllm_attend_varlen
 *   k_local,  device [batch, H_kv, local_cap, d]: the initial tokens at rows
 *   v_local   0 .. n_init-1, position p >= n_init at row n_init + (p -
 *             n_init) mod (local_cap - n_init); local_cap - n_init >= W +
 *             n_pos - 1, so that every window of the call is held
 *   ctx_cap   context capacity: positions are checked against it as
 *             infllm_attend checks them against kv_cap
 *   cache_k, cache_v, n_slots, state, n_units
 *             the unit cache after infllm_cache_fetch of the same sel; a
 *             selected unit with keys to attend that is not cached gives its
 *             row NaN outputs
 *   workspace as infllm_attend with chunk_len 1, n_chunks n_pos
 * rope_theta must be 0 (INFLLM_ERR_UNSUPPORTED otherwise).
 */
INFLLM_API infllm_status infllm_attend_cached(
    const infllm_config *cfg, int32_t batch, const void *q, int64_t q_cap, int64_t q_off,
    int64_t q_pos, const int64_t *pos, int32_t n_pos, const void *k_local, const void *v_local,
    int64_t local_cap, int64_t ctx_cap, const int32_t *sel, int32_t n_units,
    const void *cache_k, const void *cache_v, int32_t n_slots, const void *state, void *out,
    float *lse, int64_t out_cap, int64_t out_off, void *workspace, size_t workspace_bytes,
    void *stream);

/*
 * infllm_cache_stats -- synchronises `stream`, then reads the hit and miss
 * totals of a cache state.  Returns INFLLM_OK, INFLLM_ERR_INVALID_ARG or
 * INFLLM_ERR_HIP.
 */
INFLLM_API int32_t infllm_cache_stats(const void *state, int64_t *hits, int64_t *misses,
                                      void *stream);

INFLLM_API const char *infllm_status_string(int32_t status);
INFLLM_API int32_t infllm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* INFLLM_H */
