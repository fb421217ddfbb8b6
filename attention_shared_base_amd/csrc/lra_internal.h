// Host-side interfaces between the C-ABI layer (api.hip) and the kernel
// translation units.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lra_attn.h"

namespace lra {

void set_error(const char* fmt, ...);
lra_status check_launch(const char* what);

// ----------------------------------------------------------------- decode
// Work decomposition of one decode call.  A work unit is (context, row group,
// KV head); a row group holds up to 16 query rows = rpg requests x g heads.
// Each unit's keys are cut into chunks of `chunk` tokens (256 .. 2048); one
// workgroup handles one (unit, chunk), and the last workgroup of a unit with
// several chunks merges their partials.
struct DecodePlan {
    int g;          // query heads per KV head
    int rpg;        // requests per row group (16 / g)
    int n_rg;       // row groups per context
    int n_units;    // n_ctx * n_rg * H_kv
    int chunk;      // tokens per workgroup
    int n_split;    // chunks per unit at max_ctx_len
    int persistent; // 1: one workgroup per CU pulls items from a queue in the workspace
    int grid;       // workgroups launched (multiple of 8; non-persistent mode)
    size_t ws_counter_bytes;
    size_t ws_part_bytes;
    size_t ws_total;
};

bool decode_plan(const lra_dims& d, int n_req, int n_ctx, int max_req_per_ctx, int max_ctx_len,
                 DecodePlan* plan);

struct DecodeArgs {
    const void* q;
    const int32_t* ctx_req_start;
    const int32_t* req_agent;
    const void* k_pool;
    const void* v_pool;
    const void* lk_pool;
    const void* lv_pool;
    const int32_t* block_table;
    const int32_t* ctx_len;
    const void* b_k;
    const void* b_v;
    const float* rope_cos;  // NULL: no RoPE on the adapter key; else [rope_rows, d/2]
    const float* rope_sin;
    void* out;
    void* workspace;
    int32_t rope_rows;      // rows of the RoPE tables (>= max(max_ctx_len, 1) when given)
    int32_t n_req, n_ctx, n_pages, max_blocks, max_ctx_len, n_agents;
    int32_t h_q, h_kv, head_dim, rank;
    float scale;
    int64_t lr_stride;  // elements between agents' LR pools (0: one shared LR cache)
};

lra_status launch_decode_bf16(const DecodeArgs& a, const DecodePlan& p, hipStream_t s);

// ----------------------------------------------------------------- prefill
struct PrefillArgs {
    const void* q;
    const int32_t* req_agent;
    const void* k_base;
    const void* v_base;
    const void* l_k;
    const void* l_v;
    const void* b_k;
    const void* b_v;
    const float* rope_cos;  // NULL: no RoPE on the adapter key; else [rope_rows >= kv_len, d/2]
    const float* rope_sin;
    void* out;
    int32_t n_req, q_len, kv_len, n_agents;
    int32_t h_q, h_kv, head_dim, rank;
    float scale;
    int64_t lr_stride;  // elements between agents' LR caches (0: one shared LR cache)
    // measurement baseline only: plain attention (no low-rank terms, L and B
    // unused) over per-request caches kv_req_stride elements apart
    bool plain = false;
    int64_t kv_req_stride = 0;
    // paged mode: k_base / v_base / l_k / l_v are the page pools of lra_attn_decode
    // (page_size 16), read through one context's block table
    const int32_t* block_table = nullptr;  // non-NULL selects the paged mode
    int32_t max_blocks = 0, n_pages = 0;
};

lra_status launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);

// ----------------------------------------------------------------- fp32 path
// Straightforward fp32 kernels (one wavefront per query row) used for
// dtype == LRA_F32: exact fp32 arithmetic for any supported shape.
lra_status launch_decode_f32(const DecodeArgs& a, hipStream_t s);
lra_status launch_prefill_f32(const PrefillArgs& a, hipStream_t s);

// ----------------------------------------------------------------- LR build
struct LRBuildArgs {
    const void* x;
    const void* a_k;  // [n_lr, rank, d_model]
    const void* a_v;
    void* l_k;        // agent a's rows at a * lr_stride
    void* l_v;
    int32_t n_tok, d_model, rank, n_lr;
    int64_t row_offset, lr_stride;
    void* workspace;  // NULL: single-pass kernel; else >= lr_build_plan().ws_bytes, zeroed before first use
};

// d_model split of the bf16 LR build: ks ranges per 64-token block and agent
struct LRPlan {
    int ks, slices_per_split;
    long long units;
    size_t ws_counter_bytes, ws_bytes;
};
LRPlan lr_build_plan(int n_tok, int d_model, int rank, int n_lr);

lra_status launch_lr_build_bf16(const LRBuildArgs& a, hipStream_t s);
lra_status launch_lr_build_f32(const LRBuildArgs& a, hipStream_t s);

lra_status launch_rope_table(double theta, int head_dim, int n_pos, float* c, float* s,
                             hipStream_t st);

// ----------------------------------------------------------------- device ceilings
lra_status launch_ceiling_read(const void* buf, uint64_t n_bytes, int n_wg, bool nt, bool chunked,
                               uint32_t* sink, hipStream_t s);
lra_status launch_ceiling_mfma(int n_lds, int n_wg, int iters, uint32_t* sink, hipStream_t s);

// ----------------------------------------------------------------- naive baseline
// Materialised adapter terms (measurement baseline only; see naive_expand.hip).
struct ExpandArgs {
    const int32_t* ctx_req_start;
    const int32_t* req_agent;
    const void* k_pool;
    const void* v_pool;
    const void* lk_pool;
    const void* lv_pool;
    const int32_t* block_table;
    const int32_t* ctx_len;
    const void* b_k;
    const void* b_v;
    void* k_out;
    void* v_out;
    int64_t lr_stride = 0;  // elements between agents' LR pools (0: one shared pool)
    int32_t n_req, n_ctx, n_pages, max_blocks, n_agents, out_blocks;
    int32_t h_kv, head_dim, rank;
};

lra_status launch_naive_expand_bf16(const ExpandArgs& a, hipStream_t s);

// Contiguous expansion for the prefill baseline: per request, K_base + rot(L_k B_k)
// and V_base + L_v B_v into [n_req][H_kv][kv_len][d].
struct ExpandContigArgs {
    const int32_t* req_agent;
    const void* k_base;
    const void* v_base;
    const void* l_k;
    const void* l_v;
    const void* b_k;
    const void* b_v;
    const float* rope_cos;
    const float* rope_sin;
    void* k_out;
    void* v_out;
    int64_t lr_stride;
    int32_t n_req, kv_len, n_agents, h_kv, head_dim, rank;
};

lra_status launch_naive_expand_contig_bf16(const ExpandContigArgs& a, hipStream_t s);

// ----------------------------------------------------------------- paged cache
struct PagedArgs {
    const int64_t* slots;        // append
    const int32_t* block_table;  // gather: one context's row
    const void* k_rows;          // append sources
    const void* v_rows;
    const void* lk_rows;
    const void* lv_rows;
    void* k_pool;
    void* v_pool;
    void* lk_pool;
    void* lv_pool;
    void* k_out;  // gather destinations
    void* v_out;
    void* lk_out;
    void* lv_out;
    int32_t n_tok, n_pages, h_kv, kv_len, head_dim, rank;
    int32_t n_lr = 1;        // append: LR row sets (one per agent pool)
    int64_t lr_stride = 0;   // append: elements between agents' LR pools
};

lra_status launch_cache_append_bf16(const PagedArgs& a, hipStream_t s);
lra_status launch_cache_gather_bf16(const PagedArgs& a, hipStream_t s);

// bytes of the contiguous K/V/L staging of a paged prefill (each part 256-byte aligned)
size_t prefill_paged_workspace(int h_kv, int d, int r, int kv_len);

}  // namespace lra
