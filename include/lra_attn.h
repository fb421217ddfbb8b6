/*
 * lra_attn.h — C ABI of the Flash-LoRA-Attention library for AMD MI355X (gfx950).
 *
 * Multi-LoRA agents share one base KV cache (K_base, V_base) and one low-rank
 * (LR) cache (L_k = X A_k, L_v = X A_v under shared-A LoRA); each agent owns a
 * small up-projection B_k, B_v.  The library computes
 *
 *     O = softmax(Q (K_base + L_k B_k)^T * scale) (V_base + L_v B_v)
 *
 * without expanding L B to head dimension in memory: the score uses
 * Q K_base^T + (Q B_k^T) L_k^T and the value side P V_base + (P L_v) B_v, with
 * the rank-r intermediate kept through the streaming pass and B_v applied once
 * per query row at the end.
 *
 * Sources (LRAgent, arXiv 2602.01053v2, paperlayer.ai summary and the
 * gist.science explainers; PReCache, arXiv 2609.34054, ai.info abstract and the
 * rit.work blog):
 *   - cache decomposition Y = X W0 + X A B ............. LRAgent App. A.3
 *   - BaseShared / BaseLRShared (shared A => shared LR) LRAgent §3
 *   - reordering O = P V_base + (P V_lr) B, online softmax over streamed
 *     K/V blocks, one post-multiplication per query block  LRAgent §3, App. B
 *   - key-side adapter rebuilt before RoPE ............. LRAgent App. D.1
 *   - LR cache built for new context by X A ............ PReCache (PreLRShared)
 *
 * General conventions
 *   - Every buffer is owned by the caller; the library never allocates, frees
 *     or keeps a pointer after a call returns.  Device pointers must be 16-byte
 *     aligned.  Output buffers must not alias inputs.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = default
 *     stream).  They keep no global mutable state except the per-thread error
 *     text returned by lra_last_error().
 *   - Scalar arguments are validated before any HIP call; on failure nothing is
 *     launched and a nonzero lra_status is returned.  Launch failures return
 *     LRA_ERR_HIP.  Faults inside kernels surface at the caller's next
 *     synchronisation, as for any HIP kernel.
 *   - Element counts and layouts below are in elements of the storage type
 *     (dims->dtype): LRA_BF16 = bfloat16 bits, LRA_F32 = IEEE float.
 *     Accumulation is always fp32.  bf16 outputs are rounded to nearest even.
 *   - Environment switches (measurement and tests; results stay within the
 *     documented precision whatever they select): LRA_DECODE_CHUNK (256, 512,
 *     1024, 2048 or 4096 tokens per decode workgroup; default: planned from the
 *     longest context), LRA_DECODE_TARGET_WG (workgroups the chunk plan aims at,
 *     default 256), LRA_DECODE_PERSISTENT (0 or 1: one-shot or chunk-queue
 *     decode workgroups; default: chosen by grid size), LRA_LR_BUILD_PATH (split
 *     or single: the LR build's d_model-split or single-pass kernel instead of
 *     the LDS-staged one).
 *   - Supported: head_dim in {64, 128}, rank in {4, 8, 16, 32} (4: the rank of
 *     the query/key/value/output LoRA setting, LRAgent App. D.1),
 *     n_q_heads % n_kv_heads == 0, page_size == 16.  Query heads map to KV
 *     head hq / (n_q_heads / n_kv_heads) (contiguous groups).
 */
#ifndef LRA_ATTN_H
#define LRA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t lra_status;
#define LRA_OK 0
#define LRA_ERR_NULL_PTR 1            /* a required pointer is NULL */
#define LRA_ERR_BAD_SHAPE 2           /* inconsistent or out-of-range sizes */
#define LRA_ERR_UNSUPPORTED 3         /* valid but not implemented (dtype, d, r, page) */
#define LRA_ERR_MISALIGNED 4          /* a device pointer is not 16-byte aligned */
#define LRA_ERR_WORKSPACE_TOO_SMALL 5 /* workspace_bytes below the queried size */
#define LRA_ERR_HIP 6                 /* a HIP runtime call or launch failed */

#define LRA_F32 0
#define LRA_BF16 1

#define LRA_ABI_VERSION 6

typedef struct lra_dims {
    int32_t n_q_heads;   /* H_q */
    int32_t n_kv_heads;  /* H_kv; H_q % H_kv == 0 */
    int32_t head_dim;    /* d: 64 or 128 */
    int32_t rank;        /* r: 4, 8, 16 or 32 */
    int32_t dtype;       /* LRA_F32 or LRA_BF16, for every tensor of the call */
    float softmax_scale; /* <= 0 selects 1/sqrt(head_dim) */
    /* 0: one LR cache shared by every agent (BaseLRShared, shared A).  > 0: one
     * LR cache per agent (BaseShared, or PreLRShared with per-agent A; LRAgent
     * §3, PReCache): agent a's L_k / L_v start lr_agent_stride elements after
     * agent a-1's, in l_k / l_v of lra_attn_prefill and lk_pool / lv_pool of
     * lra_attn_decode (which then packs at most 4 requests per row group,
     * with or without RoPE), lra_attn_prefill_paged,
     * lra_cache_append and the naive baselines.  The staged paged prefill
     * takes 0 only. */
    int64_t lr_agent_stride;
} lra_dims;

/* ABI version of the loaded library (LRA_ABI_VERSION it was built with). */
int32_t lra_abi_version(void);

/* Static text for a status code (never NULL). */
const char* lra_status_str(lra_status status);

/* Detail of the last failing call on this host thread ("" if none). */
const char* lra_last_error(void);

/*
 * Paged decode: one new query token per request over its context's shared
 * caches (LRAgent §3 BaseLRShared decode; App. B kernel).  Requests are grouped
 * by context: the requests of context c are ctx_req_start[c] ..
 * ctx_req_start[c+1]-1, and every request of a context reads that context's
 * base and LR pages once per KV head (GQA and cross-agent sharing).
 *
 *   q              [n_req, H_q, d]                         device
 *   ctx_req_start  [n_ctx + 1] int32, non-decreasing,      device
 *                  ctx_req_start[0] == 0, [n_ctx] == n_req;
 *                  no context may hold more than max_req_per_ctx requests
 *   req_agent      [n_req] int32 in [0, n_agents)          device
 *   k_pool         [n_pages, H_kv, d/8, page_size, 8]      device
 *                  (key t of a page: its 8-element groups of dims are
 *                  page_size*8 elements apart)
 *   v_pool         [n_pages, H_kv, d, page_size]           device (dim-major)
 *   lk_pool        [n_pages, page_size, r]                 device
 *   lv_pool        [n_pages, r, page_size]                 device (rank-major)
 *                  With dims->lr_agent_stride > 0 these are n_agents pools
 *                  lr_agent_stride elements apart (stride >= n_pages *
 *                  page_size * r, else LRA_ERR_BAD_SHAPE), agent a's at
 *                  a * lr_agent_stride; request
 *                  i reads req_agent[i]'s pool through the same block table.
 *   block_table    [n_ctx, max_blocks] int32               device
 *                  logical token t of context c is in page
 *                  block_table[c][t / page_size], slot t % page_size; the base
 *                  and LR pools share page ids.  Ids outside [0, n_pages) are
 *                  clamped so reads stay in bounds (the result for that context
 *                  is then unspecified).
 *   ctx_len        [n_ctx] int32, 0 <= ctx_len[c] <= max_ctx_len,
 *                  max_ctx_len <= max_blocks * page_size   device
 *                  The newest token is part of the context; a context of
 *                  length 0 yields zero output rows.  A length above
 *                  max_ctx_len (device data the host cannot check) is cut to
 *                  max_ctx_len: the chunk count, the workspace and the RoPE
 *                  rows are sized for it, so the call stays in bounds and
 *                  leaves the workspace counters at zero.
 *   b_k, b_v       [n_agents, r, H_kv * d]; head h uses columns h*d .. h*d+d-1
 *   rope_cos,
 *   rope_sin       NULL (no rotation of the adapter key term) or both
 *                  [rope_rows, d/2] fp32 device tables of
 *                  cos/sin(pos * theta^(-2i/d)) (lra_rope_table_build); the
 *                  key at token index j of a context has position j.  The
 *                  bf16 kernel reads only some rows and derives the others
 *                  by angle addition (row p + 128 from row p and row 128), so
 *                  the tables must hold a plain rotation: row p =
 *                  cos/sin(p * w_i) for fixed frequencies w_i (no scaling
 *                  of cos and sin by a factor).
 *   rope_rows      rows of each table; with tables it must be at least
 *                  max(max_ctx_len, 1) (else LRA_ERR_BAD_SHAPE); ignored
 *                  without them.  K_base
 *                  is expected already rotated; the adapter key term
 *                  L_k B_k is rebuilt at head dimension for each request and
 *                  rotated (rotate-half pairing i, i+d/2) before it meets the
 *                  query (LRAgent App. D.1), never stored.
 *   out            [n_req, H_q, d]                          device
 *   workspace      device scratch of at least
 *                  lra_attn_decode_workspace_size(...) bytes (0 when every
 *                  context fits one workgroup's chunk of tokens; NULL is then
 *                  accepted).  It holds per-chunk partial rows
 *                  (m, l, O_base[d], O_lr[r]), one counter per work unit and
 *                  the two words of the chunk queue that persistent
 *                  workgroups (one per compute unit, chosen when the chunks
 *                  outnumber the GPU several times over) pull from; its size
 *                  grows with the number of chunks, never with
 *                  tokens x head_dim.  It must be zero-filled before its first
 *                  use; every completed call leaves the counters at zero again,
 *                  so later calls on the same stream can reuse it without
 *                  clearing.  Calls that share one workspace must not run
 *                  concurrently.
 */
size_t lra_attn_decode_workspace_size(const lra_dims* dims, int32_t n_req, int32_t n_ctx,
                                      int32_t max_req_per_ctx, int32_t max_ctx_len);

lra_status lra_attn_decode(const lra_dims* dims,
                           const void* q, int32_t n_req,
                           const int32_t* ctx_req_start, int32_t n_ctx, int32_t max_req_per_ctx,
                           const int32_t* req_agent,
                           const void* k_pool, const void* v_pool,
                           const void* lk_pool, const void* lv_pool,
                           int32_t n_pages, int32_t page_size,
                           const int32_t* block_table, int32_t max_blocks,
                           const int32_t* ctx_len, int32_t max_ctx_len,
                           const void* b_k, const void* b_v, int32_t n_agents,
                           const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                           void* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Decode that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, result and bits as lra_attn_decode
 * without the workspace (bf16 only: the fp32 path needs no scratch and returns
 * LRA_ERR_UNSUPPORTED here).  The split-K partials, merge counters and chunk
 * queue live in the library's own device array of
 * LRA_DECODE_NOALLOC_SCRATCH_BYTES per GPU (the first
 * LRA_DECODE_NOALLOC_COUNTER_BYTES of it hold the counters), held from the
 * first call on that GPU until the process ends.  The first call on a GPU
 * clears the counters with a small kernel on `stream`; every completed call
 * leaves them at zero again.  A call whose counters (n_units + 2 int32, where
 * n_units = n_ctx x row groups x H_kv) or partials do not fit returns
 * LRA_ERR_WORKSPACE_TOO_SMALL before any HIP call.  Every call on one GPU
 * shares that GPU's array, so calls that overlap on one GPU (several streams
 * or host threads) race: the caller must order them.
 */
#define LRA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
#define LRA_DECODE_NOALLOC_COUNTER_BYTES ((size_t)64 << 10)
lra_status lra_attn_decode_noalloc(const lra_dims* dims,
                                   const void* q, int32_t n_req,
                                   const int32_t* ctx_req_start, int32_t n_ctx, int32_t max_req_per_ctx,
                                   const int32_t* req_agent,
                                   const void* k_pool, const void* v_pool,
                                   const void* lk_pool, const void* lv_pool,
                                   int32_t n_pages, int32_t page_size,
                                   const int32_t* block_table, int32_t max_blocks,
                                   const int32_t* ctx_len, int32_t max_ctx_len,
                                   const void* b_k, const void* b_v, int32_t n_agents,
                                   const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                                   void* out, void* stream);

/*
 * Chunked prefill over one shared context (LRAgent §3: agents compute only the
 * newly appended context; App. B: accumulated length L = L_p + L_c; App. D.1:
 * key adapter rebuilt before RoPE).  The q_len new tokens are the last q_len
 * of the kv_len cached tokens (their base and LR rows are already written) and
 * attend causally: new token i sits at position kv_len - q_len + i and sees
 * keys 0 .. kv_len - q_len + i.
 *
 *   q          [n_req, q_len, H_q, d]          device
 *   req_agent  [n_req] int32 in [0, n_agents)  device
 *   k_base     [H_kv, kv_len, d]               device
 *   v_base     [H_kv, kv_len, d]               device
 *   l_k, l_v   [kv_len, r]                     device; with
 *              dims->lr_agent_stride > 0, one [kv_len, r] cache per agent,
 *              agent a's at a * lr_agent_stride elements (stride >=
 *              kv_len * r, else LRA_ERR_BAD_SHAPE)
 *   b_k, b_v   [n_agents, r, H_kv * d]         device
 *   rope_cos,
 *   rope_sin   NULL (no rotation of the adapter key term) or both
 *              [rope_rows, d/2] fp32 device tables of cos/sin(pos * theta^(-2i/d))
 *              (see lra_rope_table_build), rope_rows >= kv_len (else
 *              LRA_ERR_BAD_SHAPE; ignored without tables).  The bf16 kernel
 *              reads rows 0..63 and the first row of each 64-key tile and
 *              derives the others by angle addition, so the tables must hold
 *              a plain rotation: row p = cos/sin(p * w_i) for fixed
 *              frequencies w_i.  K_base is expected already rotated;
 *              the kernel rotates only L_k B_k (rotate-half pairing i, i+d/2)
 *              before adding it to K_base.
 *   out        [n_req, q_len, H_q, d]          device
 *   Requires 1 <= q_len <= kv_len.
 */
lra_status lra_attn_prefill(const lra_dims* dims,
                            const void* q, int32_t n_req, int32_t q_len,
                            const int32_t* req_agent,
                            const void* k_base, const void* v_base, int32_t kv_len,
                            const void* l_k, const void* l_v,
                            const void* b_k, const void* b_v, int32_t n_agents,
                            const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                            void* out, void* stream);

/*
 * Chunked prefill over one context held in the paged pools of lra_attn_decode
 * (LRAgent §3: agents process only the newly appended context; App. B: the
 * accumulated context L = L_p + L_c).  Same computation as lra_attn_prefill
 * with k_base/v_base/l_k/l_v taken from the pages: logical token t is in page
 * block_table[t / page_size], slot t % page_size (the q_len new tokens are the
 * last q_len of the kv_len tokens, already appended with lra_cache_append).
 * The pages are read in place (no staging, no workspace); the output equals
 * that of lra_attn_prefill over the same tokens laid out contiguously, bit
 * for bit.
 *   block_table  [max_blocks] int32, this context's row   device
 *                entries past ceil(kv_len / page_size) are not read; ids
 *                outside [0, n_pages) are clamped so reads stay in bounds
 *                (the result is then unspecified)
 *   lk_pool,
 *   lv_pool      with dims->lr_agent_stride > 0: n_agents pools
 *                lr_agent_stride >= n_pages * page_size * r elements apart
 *                (else LRA_ERR_BAD_SHAPE); request i reads req_agent[i]'s
 * Other arguments and layouts as in lra_attn_decode / lra_attn_prefill.
 * bf16 only.
 */
lra_status lra_attn_prefill_paged(const lra_dims* dims,
                                  const void* q, int32_t n_req, int32_t q_len,
                                  const int32_t* req_agent,
                                  const void* k_pool, const void* v_pool,
                                  const void* lk_pool, const void* lv_pool,
                                  int32_t n_pages, int32_t page_size,
                                  const int32_t* block_table, int32_t max_blocks,
                                  int32_t kv_len,
                                  const void* b_k, const void* b_v, int32_t n_agents,
                                  const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                                  void* out, void* stream);
/*
 * The same prefill through a contiguous copy: the context's keys, values and
 * LR rows are first gathered from the pages into the workspace, then attended
 * as in lra_attn_prefill.  Kept as a fallback and as a cross-check of the
 * direct path (identical output); costs an extra read and write of the
 * context and 2*H_kv*kv_len*d*2 + 2*kv_len*r*2 bytes of workspace.
 *   workspace    >= lra_attn_prefill_paged_staged_workspace_size(dims, kv_len)
 *                bytes, device, caller-owned; no state is kept between calls
 * Shared LR cache only (dims->lr_agent_stride == 0).  bf16 only.
 */
size_t lra_attn_prefill_paged_staged_workspace_size(const lra_dims* dims, int32_t kv_len);
lra_status lra_attn_prefill_paged_staged(const lra_dims* dims,
                                         const void* q, int32_t n_req, int32_t q_len,
                                         const int32_t* req_agent,
                                         const void* k_pool, const void* v_pool,
                                         const void* lk_pool, const void* lv_pool,
                                         int32_t n_pages, int32_t page_size,
                                         const int32_t* block_table, int32_t max_blocks,
                                         int32_t kv_len,
                                         const void* b_k, const void* b_v, int32_t n_agents,
                                         const float* rope_cos, const float* rope_sin,
                                         int32_t rope_rows, void* out, void* workspace,
                                         size_t workspace_bytes, void* stream);
/*
 * Append new tokens to the paged pools (the decode-time and prefill-time write
 * of the base K/V rows and the LR rows; LRAgent §3 BaseLRShared: one LR row
 * per token serves every agent; BaseShared: one per agent).  Token i goes to
 * slot slot_mapping[i] = page * page_size + offset; a negative slot skips the
 * token.
 *   slot_mapping   [n_tok] int64                    device
 *   k_new, v_new   [n_tok, H_kv, d] (K already rotated if the model uses RoPE)
 *   lk_new, lv_new [n_lr, n_tok, r]  (e.g. rows written by lra_lr_cache_build)
 *   n_lr           LR row sets: 1 with one shared LR pool
 *                  (dims->lr_agent_stride == 0); with per-agent pools
 *                  (lr_agent_stride >= n_pages * page_size * r) set a goes to
 *                  agent a's pools, for a < n_lr (the pools must hold n_lr)
 *   k_pool ...     the pools of lra_attn_decode, written in place
 * Slots at or past n_pages * page_size are skipped.  Two tokens with the same
 * slot leave either one.  bf16 only.
 */
lra_status lra_cache_append(const lra_dims* dims, int32_t n_tok, const int64_t* slot_mapping,
                            const void* k_new, const void* v_new,
                            const void* lk_new, const void* lv_new, int32_t n_lr,
                            void* k_pool, void* v_pool, void* lk_pool, void* lv_pool,
                            int32_t n_pages, int32_t page_size, void* stream);
/*
 * Low-rank cache rows for new tokens (PReCache PreLRShared; LRAgent §3
 * BaseLRShared with shared A):  L_k[row_offset + i] = x[i] A_k,
 * L_v[row_offset + i] = x[i] A_v  for i < n_tok, i.e. L = X A.  With n_lr > 1
 * (one A per agent: BaseShared, or PreLRShared with per-agent adapters) one
 * call builds every agent's cache, X [A_1 .. A_n]: agent a's rows go to
 * l_k + a * lr_agent_stride (the layout lra_dims.lr_agent_stride describes).
 *
 *   x          [n_tok, d_model]   device
 *   a_k, a_v   [n_lr, rank, d_model] device: the down-projections stored as
 *              out x in (row t is column t of A), the usual layout of a LoRA
 *              "A" weight
 *   n_lr       number of LR caches (1: shared A)
 *   l_k, l_v   n_lr blocks lr_agent_stride elements apart (ignored for
 *              n_lr = 1), each [>= row_offset + n_tok, rank]; rows written in
 *              place  device
 *   workspace  optional (may be NULL), device, caller-owned, 16-byte aligned,
 *              >= lra_lr_cache_build_workspace_size(...) bytes, zero-filled
 *              before its first use (each call leaves it ready for the next:
 *              its counters return to zero).  bf16 builds whose d_model is a
 *              multiple of 256 (512 for rank <= 8) stage X and A through LDS,
 *              one workgroup per 16 tokens over the whole of d_model, and use
 *              no workspace.  Otherwise, with a workspace, they split d_model
 *              over several workgroups per token block and add the fp32
 *              partials in a fixed order; without one a workgroup covers each
 *              token's whole d_model.  Every path is deterministic.
 *              Concurrent calls must not share a workspace.
 *   Requires d_model % 32 == 0.  bf16 results are rounded to nearest even
 *   once, after fp32 accumulation.
 *   Errors: LRA_ERR_WORKSPACE_TOO_SMALL, LRA_ERR_MISALIGNED for a workspace
 *   that is given but too small or misaligned.
 */
lra_status lra_lr_cache_build(int32_t dtype, const void* x, int32_t n_tok, int32_t d_model,
                              const void* a_k, const void* a_v, int32_t rank, int32_t n_lr,
                              void* l_k, void* l_v, int64_t row_offset,
                              int64_t lr_agent_stride, void* workspace, size_t workspace_bytes,
                              void* stream);
/* Workspace bytes lra_lr_cache_build uses for these sizes (0: none needed;
 * also 0 for fp32 and for arguments lra_lr_cache_build rejects). */
size_t lra_lr_cache_build_workspace_size(int32_t dtype, int32_t n_tok, int32_t d_model, int32_t rank,
                                         int32_t n_lr);

/*
 * RoPE tables for prefill and decode: cos/sin of pos * theta^(-2i/d), pos in
 * [0, n_pos), i in [0, head_dim/2), computed in fp64 and stored as fp32,
 * row-major [n_pos, head_dim/2].  (LRAgent App. D.1 names RoPE; the frequency
 * formula is the standard rotary one.)
 */
lra_status lra_rope_table_build(double theta, int32_t head_dim, int32_t n_pos,
                                float* cos_out, float* sin_out, void* stream);

/*
 * Measurement baseline, not part of the method: the naive reconstruction that
 * Flash-LoRA-Attention avoids (LRAgent §3 "Flash-LoRA-Attention" and App. B:
 * expanding the low-rank terms to head dimension before attention).  For every
 * request i (context c, agent a = req_agent[i]) and every block b of c
 * (b < min(ceil(ctx_len[c] / page_size), out_blocks)) it writes page
 * i * out_blocks + b of k_out / v_out:
 *     K = K_base + L_k B_k^(a),  V = V_base + L_v B_v^(a)   (every KV head)
 * in the layouts of k_pool / v_pool, bf16 rounded to nearest even.  Decode
 * attention over those pages (lra_attn_decode with one context per request,
 * block table i * out_blocks + b and B = 0) is then plain attention over
 * per-request materialised caches.  Arguments as in lra_attn_decode (L_k, L_v
 * from agent a's pools when dims->lr_agent_stride > 0);
 *   k_out, v_out   [n_req * out_blocks, H_kv, ...] device, caller-owned
 *   out_blocks     blocks reserved per request, 1 <= out_blocks <= max_blocks
 * bf16 only.  Blocks past a context's length are not written.
 */
lra_status lra_naive_expand_pages(const lra_dims* dims, int32_t n_req,
                                  const int32_t* ctx_req_start, int32_t n_ctx,
                                  const int32_t* req_agent,
                                  const void* k_pool, const void* v_pool,
                                  const void* lk_pool, const void* lv_pool,
                                  int32_t n_pages, int32_t page_size,
                                  const int32_t* block_table, int32_t max_blocks,
                                  const int32_t* ctx_len,
                                  const void* b_k, const void* b_v, int32_t n_agents,
                                  void* k_out, void* v_out, int32_t out_blocks,
                                  void* stream);

/*
 * Measurement baseline for prefill, not part of the method: the naive
 * reconstruction of LRAgent §3 / App. B for a chunked prefill.  For every
 * request i (agent a = req_agent[i]) it writes to the workspace
 *     K_i = K_base + rot(L_k B_k^(a)),  V_i = V_base + L_v B_v^(a)
 * ([n_req, H_kv, kv_len, d] each, bf16 rounded to nearest even; rot as in
 * lra_attn_prefill when RoPE tables are given), then runs plain causal
 * attention of each request's queries over its own K_i, V_i.  Arguments and
 * result as in lra_attn_prefill (with lr_agent_stride the agent's own LR rows
 * are expanded), plus
 *   workspace   device, caller-owned, >= lra_naive_prefill_workspace_size()
 *               bytes; holds the expanded caches (2 x n_req x H_kv x kv_len x
 *               d x 2 bytes), no state is kept between calls
 * bf16 only.
 */
size_t lra_naive_prefill_workspace_size(const lra_dims* dims, int32_t n_req, int32_t kv_len);
lra_status lra_naive_prefill(const lra_dims* dims,
                             const void* q, int32_t n_req, int32_t q_len,
                             const int32_t* req_agent,
                             const void* k_base, const void* v_base, int32_t kv_len,
                             const void* l_k, const void* l_v,
                             const void* b_k, const void* b_v, int32_t n_agents,
                             const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                             void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Device ceilings, not part of the method: two measurement kernels that give the
 * rates this device sustains, so that the attention kernels' rates can be set
 * against a rate reached on the same chip as well as against the published peaks.
 *
 * lra_ceiling_hbm_read streams n_bytes from buf (device, 16-byte aligned, n_bytes a
 * positive multiple of 16) with 16-byte loads, sixteen in flight per lane, and
 * keeps nothing.
 *   n_workgroups  256-lane workgroups in the grid; 0 chooses 16 per CU (4096),
 *                 fewer when the buffer is smaller
 *   flags         LRA_READ_NONTEMPORAL: non-temporal loads (else ordinary cached
 *                 loads); LRA_READ_CHUNKED: workgroup b reads the b-th contiguous
 *                 chunk of the buffer (else a grid-stride sweep, each wavefront
 *                 instruction covering 1 KB, the grid moving front to back)
 *   sink          device, 16-byte aligned, >= 4 bytes; written only when the XOR
 *                 fold of the 16-byte words one lane read equals 0x6a09e667 (a
 *                 guard against the loads being removed)
 * Algorithmic bytes per call: n_bytes.
 *
 * lra_ceiling_mfma_bf16 runs n_workgroups workgroups of four wavefronts; each
 * wavefront issues iters rounds of four independent v_mfma_f32_32x32x16_bf16
 * (fp32 accumulation).  lds_operands of every MFMA's two operands come from a
 * new 16-byte LDS read per lane (1 KB per wavefront per operand): 0 keeps both
 * in registers, 1 reads B, 2 reads A and B.  n_workgroups in [1, 65535], iters
 * in [1, 2^20].  sink as above (written only for an impossible sum).
 * Flops per call: n_workgroups * 4 * iters * 4 * (2 * 32 * 32 * 16)
 *               = n_workgroups * iters * 524288;
 * LDS bytes read per call: lds_operands * n_workgroups * 4 * iters * 4 * 1024.
 *
 * Both are asynchronous on stream and allocate nothing.  Errors: LRA_ERR_NULL_PTR,
 * LRA_ERR_MISALIGNED, LRA_ERR_BAD_SHAPE, LRA_ERR_HIP.
 */
#define LRA_READ_NONTEMPORAL 1
#define LRA_READ_CHUNKED 2
lra_status lra_ceiling_hbm_read(const void* buf, size_t n_bytes, int32_t n_workgroups, int32_t flags,
                                uint32_t* sink, void* stream);
lra_status lra_ceiling_mfma_bf16(int32_t lds_operands, int32_t n_workgroups, int32_t iters, uint32_t* sink,
                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LRA_ATTN_H */
