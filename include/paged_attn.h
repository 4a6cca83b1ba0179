/*
 * paged_attn.h - single-token decode attention over a paged KV cache, for
 * AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes only.
 *
 * What the library computes
 * -------------------------
 * For every sequence b and query head h of one decode step,
 *
 *     out[b,h,:] = softmax_t( scale * q[b,h,:] . K_b[t,g,:] ) V_b[t,g,:],
 *     lse[b,h]   = ln sum_t exp( scale * q[b,h,:] . K_b[t,g,:] ),
 *
 * over the tokens t = 0 .. context_lens[b]-1 of that sequence, where the key
 * and value rows are not contiguous but gathered through a block table, and
 * g = h / (Hq / Hkv) is the KV head shared by a group of query heads.  Decode
 * attention reads the whole accumulated KV of each sequence for one query, so
 * it is bound by HBM bandwidth ("Why prefill and decode are opposite
 * problems" and "How the backend reads the paged KV" on the page "The
 * signature-dish specialist: vLLM's attention backend"; §2.2 of the
 * KernelFlume paper, academ.us/article/2606.29207).
 *
 * Layouts (all row-major, the last index contiguous)
 * --------------------------------------------------
 *   q            fp16  [B, Hq, D]
 *   k_cache      fp16  [num_blocks, block_size, Hkv, D]   physical pool of K
 *   v_cache      fp16  [num_blocks, block_size, Hkv, D]   physical pool of V
 *   block_table  int32 [B, block_table_stride]; entry [b, i] is the physical
 *                block holding tokens i*block_size .. i*block_size+block_size-1
 *                of sequence b.  Only entries i < ceil(context_lens[b] /
 *                block_size) are read; the rest may hold anything.
 *   context_lens int32 [B]; number of cached tokens of each sequence, the token
 *                being decoded included (its K/V must already be in the cache).
 *   out          fp16  [B, Hq, D];  lse fp32 [B, Hq] (natural log).
 * One block of one pool holds block_size * Hkv * D fp16 values, the block
 * stride of "Physical Memory Block Layout" on the page "Disaggregated
 * Inference Architecture: Paged KV-Cache Tiering, Chunked Prefill, and
 * Asynchronous Overlap"; logical block i holds tokens 16i .. 16i+15 (figure
 * "Virtual Sequence Address Space" on that page).
 *
 * Supported shapes: D = 128, block_size = 16, Hq / Hkv in {1, 2, 4, 6, 8},
 * 1 <= Hkv <= 64.  This covers the head configurations the KernelFlume paper
 * evaluates (§6.3): GQA Q32:KV8, Q48:KV8, Q64:KV8 and MHA Q32:KV32, Q40:KV40,
 * Q48:KV48.  Other shapes return PDA_EUNSUPPORTED.
 *
 * Conventions
 * -----------
 * - Device pointers: q, k_cache, v_cache, block_table, context_lens, out,
 *   lse, workspace and every partial buffer are device memory of the current
 *   HIP device.  `stream` is a hipStream_t (NULL = the default stream).
 * - Ownership: the caller allocates and owns every buffer, the workspace
 *   included.  The library never allocates or frees memory on these calls,
 *   never synchronises, and only enqueues kernels on `stream`, so the calls
 *   may be captured into a HIP graph.  Inputs are read-only (the KV pools
 *   too, except in paged_kv_append and paged_decode_attn_append, which write
 *   one slot per sequence); outputs must not alias inputs.
 * - Errors: a non-zero pda_status is returned and pda_last_error() gives a
 *   message for the calling thread.  Argument errors are detected on the host
 *   before anything is enqueued.  Device-side contract violations (a block
 *   id outside [0, num_blocks), context_lens[b] > max_blocks_per_seq *
 *   block_size or negative) are undefined behaviour; setting the environment
 *   variable PDA_DEBUG_VALIDATE=1 makes each call copy context_lens and the
 *   block table to the host and check them first (this synchronises the
 *   stream; for tests only).
 * - Results are bitwise deterministic for a fixed partition length: no
 *   floating-point atomics are used.
 * - Thread safety: calls may be made from several threads; the only global
 *   state is a per-device property cache filled on first use.
 */
#ifndef PAGED_ATTN_H_
#define PAGED_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PDA_OK = 0,
  PDA_EINVAL = 1,       /* bad argument: null pointer, Hq % Hkv != 0, ...   */
  PDA_EUNSUPPORTED = 2, /* valid but not built: D != 128, block_size != 16  */
  PDA_EHIP = 3          /* a HIP runtime or launch error                    */
} pda_status;

/*
 * Bytes of device workspace paged_decode_attn and paged_decode_attn_partial
 * need for these sizes (*bytes; 0 when B == 0), enough for every decode entry
 * point: fp16, FP8 and the fused appends.  partition_tokens as in
 * paged_decode_attn.  The size
 * depends on the device (its CU count sets the number of work-groups), so
 * query it on the device that will run the call.
 */
int pda_workspace_size(int B, int Hq, int Hkv, int D, int block_size,
                       int max_blocks_per_seq, int partition_tokens,
                       size_t* bytes);

/*
 * The same bytes for a caller that does not yet know Hkv: the largest
 * pda_workspace_size over every KV-head count Hkv that divides Hq and is
 * supported, so one workspace of this size serves paged_decode_attn,
 * paged_decode_attn_partial and their FP8 and fused-append forms whatever
 * grouping of the Hq query heads the call uses.  This is the sizing call of
 * the decode boundary (a split-K workspace for the attention node's partial,
 * KernelFlume paper §3.2).  Returns the last error of pda_workspace_size if no
 * KV-head count is accepted.
 */
int paged_decode_attn_workspace_size(int B, int Hq, int D, int block_size,
                                     int max_blocks_per_seq, int partition_tokens,
                                     size_t* bytes);

/* Workspace layout of one call shape; see pda_workspace_layout. */
typedef struct {
  size_t header_offset; /* int32 [4 + B]: k, U, n_runs, unit_tokens,
                           then the number of units before sequence b     */
  size_t lse_offset;    /* fp32 [n_slots, Hq]: lse of each stored partial  */
  size_t o_offset;      /* fp32 [n_slots, Hq, D]: normalised partials      */
  size_t total_bytes;   /* == pda_workspace_size                           */
  int n_runs;           /* runs the unit stream is cut into                */
  int n_slots;          /* n_runs + B                                      */
  int unit_tokens;      /* P: tokens per unit of the schedule              */
} pda_layout;

/*
 * Where the split-K partials live inside the workspace after a call, for
 * tests and debugging (kv_fp8: 1 for the *_fp8 entry points, else 0; the
 * number of runs depends on it).  The schedule: each sequence's tokens are cut into
 * units of P = unit_tokens tokens (the last one shorter); the units of all
 * sequences in order form one stream of U units, and run w is units
 * [w*k, (w+1)*k), k = ceil(U / n_runs) (each run is computed by one
 * work-group per group of up to 4 KV heads).  The tokens of sequence b in
 * run w form one contiguous range; unless that range is the whole sequence
 * (then the final output is written directly), its partial (o, lse) for
 * query head h is stored in slot w + b at
 * lse_offset + 4 * ((w + b) * Hq + h) and o_offset + 4 * D * ((w + b) * Hq
 * + h).  The header records k, U and the units before each sequence.
 */
int pda_workspace_layout(int B, int Hq, int Hkv, int D, int block_size,
                         int max_blocks_per_seq, int partition_tokens,
                         int kv_fp8, pda_layout* layout);

/*
 * Decode attention over a paged KV cache (see the top of this file).
 *
 * Split-K: each sequence's tokens are cut into contiguous units of
 * partition_tokens tokens (a multiple of block_size; 0 means 16, one block,
 * the finest balance).  The unit stream of the whole batch is dealt to a
 * persistent grid sized to the device's CUs in equal contiguous runs, so
 * every work-group reads the same number of KV bytes whatever the mix of
 * context lengths.  Within a work-group, one wavefront per KV head computes
 * the partial of all Hq / Hkv query heads that share that head over each
 * token range of its run; a sequence split over several work-groups is then
 * merged by log-sum-exp in a second kernel.  Partials over contiguous token
 * ranges and their merge are the attention-node / weight-node split of §3.1
 * "Kernel-level Disaggregation" and §3.2 "Workflow of Elastic Decoding" in
 * the KernelFlume paper, whose merge equals attention over the full range
 * (§5.1 "Query-First Attention"; the (m, l, O) update equations of
 * "Mathematical Formulation of Chunked Attention" on the
 * disaggregated-inference page).
 *
 * out            fp16 [B, Hq, D], written.
 * lse_out        fp32 [B, Hq] or NULL; natural-log log-sum-exp of the scaled
 *                scores.  A sequence with context_lens[b] == 0 gets out = 0
 *                and lse = -inf.
 * scale          multiplies q . k before the softmax (typically 1/sqrt(D)).
 * num_blocks     rows of k_cache / v_cache (used by PDA_DEBUG_VALIDATE).
 * max_blocks_per_seq  largest ceil(context_lens[b] / block_size) the call may
 *                see; sizes the workspace and the launch.
 * block_table_stride  int32 elements between rows of block_table
 *                (>= max_blocks_per_seq), so a column slice of a wider table
 *                can be passed without a copy.
 * workspace      device memory of at least pda_workspace_size() bytes, 256-byte
 *                aligned; contents on entry are ignored.
 */
int paged_decode_attn(void* out, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_table,
                      int64_t block_table_stride, const int32_t* context_lens,
                      int B, int Hq, int Hkv, int D, int block_size,
                      int64_t num_blocks, int max_blocks_per_seq, float scale,
                      int partition_tokens, float* lse_out, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * paged_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The split-K workspace is instead a fixed
 * device array of PDA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 * held until the process ends; its device address is looked up (never
 * allocated) on the first call on each device.  No allocation of any kind is
 * made on the call.  Arguments, results and errors are those of
 * paged_decode_attn (the same kernels, bit for bit the same output); a call
 * whose split-K workspace (at most pda_workspace_size for its shape) exceeds
 * the scratch returns PDA_EUNSUPPORTED before anything is enqueued.  Every call on one GPU
 * shares that GPU's scratch, which keeps the last call's contents: calls that
 * may overlap on one GPU (several streams, several host threads) race and
 * must be ordered by the caller.  Nothing in the scratch needs clearing
 * between calls: each call writes what it reads.
 */
#define PDA_NOALLOC_SCRATCH_BYTES (32u << 20)

int paged_decode_attn_noalloc(void* out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_table,
                              int64_t block_table_stride, const int32_t* context_lens,
                              int B, int Hq, int Hkv, int D, int block_size,
                              int64_t num_blocks, int max_blocks_per_seq, float scale,
                              int partition_tokens, float* lse_out, void* stream);

/*
 * The partial of a token range: same inputs as paged_decode_attn, where the
 * block table and context_lens describe the range a caller owns (a column
 * slice of the full table via block_table_stride, and the range's length).
 * Writes the normalised output o fp32 [B, Hq, D] and lse fp32 [B, Hq] of
 * attention over that range: the (o_i, m_i, l_i) partial an attention node
 * returns in §3.2 of the KernelFlume paper, with o_i normalised and
 * lse = m_i + ln l_i.  An empty range gives o = 0, lse = -inf.
 */
int paged_decode_attn_partial(float* o, float* lse, const void* q,
                              const void* k_cache, const void* v_cache,
                              const int32_t* block_table,
                              int64_t block_table_stride,
                              const int32_t* context_lens, int B, int Hq,
                              int Hkv, int D, int block_size,
                              int64_t num_blocks, int max_blocks_per_seq,
                              float scale, int partition_tokens,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * FP8 KV cache: as paged_decode_attn / paged_decode_attn_partial, with
 * k_cache and v_cache holding one FP8 E4M3 code per element (1 byte; the OCP
 * 8-bit format: sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, S.1111.111 = NaN) in the same [num_blocks, block_size, Hkv, D]
 * layout, and per-tensor scales: a stored K code c stands for
 * k_scale * value(c), a V code for v_scale * value(c).  This is the quantised
 * KV cache of "4. Quantised KV cache" on the page "Optimising decode in vLLM:
 * squeezing every token out of small hardware" (kv_cache_dtype fp8 with
 * per-tensor scales); it halves the bytes read per token.  Codes are decoded
 * exactly; arithmetic is as in the fp16 entry points.  NaN codes in valid
 * tokens give undefined results.
 */
int paged_decode_attn_fp8(void* out, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* block_table,
                          int64_t block_table_stride,
                          const int32_t* context_lens, int B, int Hq, int Hkv,
                          int D, int block_size, int64_t num_blocks,
                          int max_blocks_per_seq, float scale, float k_scale,
                          float v_scale, int partition_tokens, float* lse_out,
                          void* workspace, size_t workspace_bytes, void* stream);

int paged_decode_attn_partial_fp8(float* o, float* lse, const void* q,
                                  const void* k_cache, const void* v_cache,
                                  const int32_t* block_table,
                                  int64_t block_table_stride,
                                  const int32_t* context_lens, int B, int Hq,
                                  int Hkv, int D, int block_size,
                                  int64_t num_blocks, int max_blocks_per_seq,
                                  float scale, float k_scale, float v_scale,
                                  int partition_tokens, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Merge R partials over disjoint token ranges into attention over their
 * union, by log-sum-exp: with L = max_r lse_r and w_r = exp(lse_r - L),
 * lse = L + ln sum_r w_r and out = sum_r w_r o_r / sum_r w_r (the merge a
 * weight node applies to attention-node partials, KernelFlume paper §3.2 and
 * §5.1; "Mathematical Formulation of Chunked Attention" on the
 * disaggregated-inference page).  Partials with lse = -inf carry no weight;
 * if all are -inf, out = 0 and lse = -inf.
 *
 * o_parts   fp32 [R, B, Hq, D]    lse_parts fp32 [R, B, Hq]
 * out       fp16 [B, Hq, D]       lse_out   fp32 [B, Hq] or NULL
 * D must be 128.  R >= 1.
 */
int merge_partials(void* out, float* lse_out, const float* o_parts,
                   const float* lse_parts, int R, int B, int Hq, int D,
                   void* stream);

/*
 * KV append: write the newest token's key and value of every sequence into
 * its paged cache, in place, before attending.  The tail node appends
 * (K_new, V_new) and then attends over the updated range (KernelFlume paper
 * §3.2 "Workflow of Elastic Decoding", §5.1 "Query-First Attention").
 *
 * k_new, v_new   fp16 [B, Hkv, D].
 * context_lens   counts the new token: sequence b writes token t = ctx_b - 1,
 *                i.e. row (frame = block_table[b, t / block_size],
 *                slot = t % block_size) of both pools, all Hkv heads.
 *                ctx_b <= 0 writes nothing; the block holding token t must
 *                already be in the table (allocating blocks is the caller's).
 * Sequences must own distinct tail slots (each sequence's own last block).
 * A block id outside [0, num_blocks) or ctx_b > max_blocks_per_seq *
 * block_size skips that sequence.  D must be 128 and block_size 16.
 */
int paged_kv_append(void* k_cache, void* v_cache, const void* k_new,
                    const void* v_new, const int32_t* block_table,
                    int64_t block_table_stride, const int32_t* context_lens,
                    int B, int Hkv, int D, int block_size, int64_t num_blocks,
                    int max_blocks_per_seq, void* stream);

/*
 * paged_kv_append into FP8 (E4M3) pools, one code per element in the layout
 * of paged_decode_attn_fp8: the new rows (fp16 [B, Hkv, D]) are quantised with
 * the tensors' scales, code = E4M3 value nearest to fp32(x) * fp32(1 / scale)
 * (ties to the even code, the sign of zero kept, magnitudes at or above 448
 * saturate to +-448, NaN stays NaN), so that scale * value(code) is the stored
 * approximation of x, as paged_decode_attn_fp8 reads it (the FP8 KV cache of
 * "4. Quantised KV cache" in "Optimising decode in vLLM: squeezing every
 * token out of small hardware").  Slots, skip rules and errors as
 * paged_kv_append; k_scale / v_scale not finite or 0 -> PDA_EINVAL.
 */
int paged_kv_append_fp8(void* k_cache, void* v_cache, const void* k_new,
                        const void* v_new, const int32_t* block_table,
                        int64_t block_table_stride, const int32_t* context_lens,
                        int B, int Hkv, int D, int block_size, int64_t num_blocks,
                        int max_blocks_per_seq, float k_scale, float v_scale,
                        void* stream);

/*
 * paged_kv_append and paged_decode_attn in one call, for fp16 caches (the
 * append before the attention of the same passages of the KernelFlume paper,
 * fused into the attention's launch): the newest token of every sequence
 * (position context_lens[b] - 1, which the context length already counts)
 * gets k_new[b] / v_new[b] (fp16 [B, Hkv, D]) in its cache slot, and the
 * attention uses those rows for that token.  Sequences must own distinct
 * tail slots, as for paged_kv_append.  The
 * cache is left as paged_kv_append leaves it and out / lse_out are bit for
 * bit those of paged_decode_attn after paged_kv_append; sequences whose
 * length is 0 or above max_blocks_per_seq * block_size, or whose frame lies
 * outside the pool, get no append (as in paged_kv_append).  One launch fewer
 * per decode step.  Other arguments, the workspace and the errors are those of
 * paged_decode_attn; k_new / v_new null with B > 0 -> PDA_EINVAL.  The caches
 * are written: they must not be read by other work on the GPU meanwhile.
 */
int paged_decode_attn_append(void* out, const void* q, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, const int32_t* block_table,
                             int64_t block_table_stride, const int32_t* context_lens, int B,
                             int Hq, int Hkv, int D, int block_size, int64_t num_blocks,
                             int max_blocks_per_seq, float scale, int partition_tokens,
                             float* lse_out, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * paged_kv_append_fp8 and paged_decode_attn_fp8 in one call: the newest
 * token's rows are quantised into the FP8 pools exactly as paged_kv_append_fp8
 * does and attended as paged_decode_attn_fp8 reads them; caches, out and
 * lse_out are bit for bit those of the two calls.  Arguments, skip rules and
 * errors as paged_decode_attn_append, with the scales of paged_decode_attn_fp8
 * (both must be non-zero).
 */
int paged_decode_attn_append_fp8(void* out, const void* q, const void* k_new,
                                 const void* v_new, void* k_cache, void* v_cache,
                                 const int32_t* block_table, int64_t block_table_stride,
                                 const int32_t* context_lens, int B, int Hq, int Hkv,
                                 int D, int block_size, int64_t num_blocks,
                                 int max_blocks_per_seq, float scale, float k_scale,
                                 float v_scale, int partition_tokens, float* lse_out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Multi-query attention: several query tokens of each sequence at once, the
 * last n_q tokens of the sequence, over its paged K/V.  Covers a prefill
 * chunk, whose queries see the earlier chunks unmasked and the current chunk
 * causally ("Mathematical Formulation of Chunked Attention" on the
 * disaggregated-inference page), the k tokens a draft model proposed, which
 * the verifier checks in one pass (speculative decoding in the post
 * "Optimising decode in vLLM: squeezing every token out of small hardware"),
 * and the shared-prefix pass of cascade attention, where the decode queries
 * of every request that shares a prefix attend to it at once without a mask
 * ("What FlashInfer brings: JIT and cascade attention" on the page "The
 * signature-dish specialist: vLLM's attention backend").
 *
 * q            fp16  [num_queries, Hq, D]; rows query_start[s] ..
 *              query_start[s+1]-1 are the queries of sequence s, in position
 *              order.
 * query_start  int32 [S + 1], non-decreasing, query_start[0] = 0 and
 *              query_start[S] = num_queries (values are clamped into
 *              [0, num_queries] on the device).
 * block_table  int32 [S, block_table_stride]; context_lens int32 [S]: cached
 *              tokens of sequence s, its n_q query tokens included.
 * causal != 0: query i (0-based) of sequence s, with n = context_lens[s] and
 *              n_q its query count, sits at position n - n_q + i and attends to
 *              tokens 0 .. n - n_q + i.  causal == 0: every query attends to all
 *              n tokens.  A query with nothing to attend to (n_q > n) gets
 *              out = 0 and lse = -inf.
 * out          fp16 [num_queries, Hq, D]; lse_out fp32 [num_queries, Hq] or
 *              NULL.  The _partial form writes fp32 o and a non-NULL lse
 *              instead (a partial for merge_partials).
 * partition_tokens: 0 = automatic, else the unit length in tokens (a
 *              multiple of 16) by which the work is balanced over the GPU.
 * workspace    device memory of at least pda_multi_query_workspace_size()
 *              bytes, 256-byte aligned; it holds the schedule and partials.
 * Shapes as for paged_decode_attn (D = 128, block_size = 16, Hq / Hkv in
 * {1, 2, 4, 6, 8}, Hkv <= 64), and S <= 4000.  pda_multi_query_workspace_size
 * covers both cache formats.
 *
 * Cascade attention for B decode requests in R groups that share a prefix
 * (requests group_start[r] .. group_start[r+1]-1 share prefix r): call
 * paged_multi_query_attn_partial with the R prefix rows as the sequences,
 * query_start = group_start and causal = 0; call paged_decode_attn_partial
 * with the B suffix rows; then merge_partials with R = 2 over the two
 * (o, lse) pairs.
 */
int pda_multi_query_workspace_size(int S, int num_queries, int Hq, int Hkv, int D,
                                   int block_size, int max_blocks_per_seq,
                                   int partition_tokens, size_t* bytes);

int paged_multi_query_attn(void* out, float* lse_out, const void* q,
                           const int32_t* query_start, int num_queries,
                           const void* k_cache, const void* v_cache,
                           const int32_t* block_table, int64_t block_table_stride,
                           const int32_t* context_lens, int S, int Hq, int Hkv,
                           int D, int block_size, int64_t num_blocks,
                           int max_blocks_per_seq, float scale, int causal,
                           int partition_tokens, void* workspace,
                           size_t workspace_bytes, void* stream);

int paged_multi_query_attn_partial(float* o, float* lse, const void* q,
                                   const int32_t* query_start, int num_queries,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_table,
                                   int64_t block_table_stride,
                                   const int32_t* context_lens, int S, int Hq,
                                   int Hkv, int D, int block_size,
                                   int64_t num_blocks, int max_blocks_per_seq,
                                   float scale, int causal, int partition_tokens,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * The same over an FP8 (E4M3) cache: k_cache / v_cache hold one E4M3 code per
 * element (uint8, same layout), decoded as k = k_scale * e4m3(code) and
 * v = v_scale * e4m3(code), as for paged_decode_attn_fp8.
 */
int paged_multi_query_attn_fp8(void* out, float* lse_out, const void* q,
                               const int32_t* query_start, int num_queries,
                               const void* k_cache, const void* v_cache,
                               const int32_t* block_table, int64_t block_table_stride,
                               const int32_t* context_lens, int S, int Hq, int Hkv,
                               int D, int block_size, int64_t num_blocks,
                               int max_blocks_per_seq, float scale, float k_scale,
                               float v_scale, int causal, int partition_tokens,
                               void* workspace, size_t workspace_bytes, void* stream);

int paged_multi_query_attn_partial_fp8(float* o, float* lse, const void* q,
                                       const int32_t* query_start, int num_queries,
                                       const void* k_cache, const void* v_cache,
                                       const int32_t* block_table,
                                       int64_t block_table_stride,
                                       const int32_t* context_lens, int S, int Hq,
                                       int Hkv, int D, int block_size,
                                       int64_t num_blocks, int max_blocks_per_seq,
                                       float scale, float k_scale, float v_scale,
                                       int causal, int partition_tokens, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Diagnostic, no part of the attention path: reads `bytes` (a multiple of 16)
 * of device memory at `src` (16-byte aligned) with 16-byte loads, ordinary or
 * (nontemporal != 0) non-temporal, the load forms of the attention kernels,
 * enqueued on `stream`.  Timed, it gives the read bandwidth a plain streaming
 * kernel reaches on the device: a measured ceiling to set the decode kernels'
 * KV-read rate against, beside the HBM peak.  `sink` (one unsigned of device
 * memory) is written only if the xor of a thread's words hits one fixed
 * value, which no ordinary buffer does; nothing else is written.  Returns
 * PDA_EINVAL for null pointers or a misaligned `src` or size.
 */
int pda_stream_read(const void* src, size_t bytes, unsigned* sink, int nontemporal,
                    void* stream);

/*
 * Diagnostic, no part of the attention path: times one LDS read form of the
 * multi-query kernels, form 0 = ds_read_b128, 1 = ds_read_b64, 2 =
 * ds_read_b64_tr_b16, 3 = ds_read_b32.  Launches `work_groups` work-groups of
 * 256 threads on `stream`; each fills a 64 KiB LDS stage with word i =
 * i * 2654435761 (mod 2^32), then each wave issues 16 conflict-free reads of
 * the form per pass, `iters` passes (read r covers bytes [r S, (r + 1) S) of
 * the stage, S = 64 lanes times the form's width, lane l at l times the
 * width), and thread t of work-group b writes the wrapping 32-bit sum of the
 * words it received to out[256 b + t] (out: device memory of 256 x
 * work_groups unsigned).  With a profiler's SQ_LDS_IDX_ACTIVE count it gives
 * that counter's cost per instruction of each form and the count per clock
 * of a kernel bound by nothing else.  Returns PDA_EINVAL for a form outside
 * 0..3, negative sizes or a null `out` when work_groups > 0.
 */
int pda_lds_probe(int form, unsigned* out, int work_groups, int iters, void* stream);

/* Message for the last non-OK return on the calling thread ("" if none). */
const char* pda_last_error(void);

/* Library version string. */
const char* pda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H_ */
