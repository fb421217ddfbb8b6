// C ABI: argument validation, work planning and dispatch to the gfx950 kernels.
// Declarations and the contract of every entry point are in include/lra_attn.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "lra_internal.h"

namespace {

thread_local char g_err[512] = "";

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int env_int(const char* name, int dflt) {
    const char* s = getenv(name);
    if (!s || !*s) return dflt;
    return atoi(s);
}

lra_status fail(lra_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

// Shared checks of the dims struct.  Returns LRA_OK or a status with detail.
lra_status check_dims(const lra_dims* d) {
    if (!d) return fail(LRA_ERR_NULL_PTR, "dims is NULL");
    if (d->n_q_heads <= 0 || d->n_kv_heads <= 0)
        return fail(LRA_ERR_BAD_SHAPE, "head counts must be positive (H_q=%d, H_kv=%d)", d->n_q_heads, d->n_kv_heads);
    if (d->n_q_heads % d->n_kv_heads != 0)
        return fail(LRA_ERR_BAD_SHAPE, "H_q=%d is not a multiple of H_kv=%d", d->n_q_heads, d->n_kv_heads);
    if (d->dtype != LRA_F32 && d->dtype != LRA_BF16)
        return fail(LRA_ERR_UNSUPPORTED, "dtype %d (expected LRA_F32=0 or LRA_BF16=1)", d->dtype);
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(LRA_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", d->head_dim);
    if (d->rank != 4 && d->rank != 8 && d->rank != 16 && d->rank != 32)
        return fail(LRA_ERR_UNSUPPORTED, "rank %d (supported: 4, 8, 16, 32)", d->rank);
    if (!(d->softmax_scale == d->softmax_scale) || isinf(d->softmax_scale))
        return fail(LRA_ERR_BAD_SHAPE, "softmax_scale is not finite");
    if (d->lr_agent_stride < 0)
        return fail(LRA_ERR_BAD_SHAPE, "lr_agent_stride %lld < 0", (long long)d->lr_agent_stride);
    return LRA_OK;
}

float eff_scale(const lra_dims* d) {
    return d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf((float)d->head_dim);
}

#define REQUIRE_PTR(p)                                                  \
    do {                                                                \
        if (!(p)) return fail(LRA_ERR_NULL_PTR, "%s is NULL", #p);      \
        if (!aligned16(p)) return fail(LRA_ERR_MISALIGNED, "%s is not 16-byte aligned", #p); \
    } while (0)

}  // namespace

namespace lra {

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

lra_status check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error("%s: %s", what, hipGetErrorString(e));
        return LRA_ERR_HIP;
    }
    return LRA_OK;
}

bool decode_plan(const lra_dims& d, int n_req, int n_ctx, int max_req_per_ctx, int max_ctx_len,
                 DecodePlan* p) {
    const int g = d.n_q_heads / d.n_kv_heads;
    if (g < 1 || g > 16 || n_ctx < 1 || max_req_per_ctx < 1 || max_ctx_len < 0 || n_req < 0) return false;
    p->g = g;
    // per-agent LR caches: one LR page stream per request slot, at most 4 per group
    p->rpg = d.lr_agent_stride != 0 ? (16 / g < 4 ? 16 / g : 4) : 16 / g;
    p->n_rg = (max_req_per_ctx + p->rpg - 1) / p->rpg;
    const long long units = (long long)n_ctx * p->n_rg * d.n_kv_heads;
    if (units > (1 << 26)) return false;
    p->n_units = (int)units;
    // Chunk length (tokens per workgroup, a power of two in [256, 4096] so the
    // kernel's per-wavefront step count is a compile-time constant): enough
    // workgroups to fill 256 CUs a few times over, each wavefront still
    // streaming several 32-token steps.
    int chunk = env_int("LRA_DECODE_CHUNK", 0);
    if (chunk != 256 && chunk != 512 && chunk != 1024 && chunk != 2048 && chunk != 4096) {
        // ~one workgroup per CU at the longest context; longer chunks amortise
        // each workgroup's fixed prologue/merge cost (measured best on MI355X:
        // 1024 tokens for 4 x 8192-token contexts, 4096 for 4k-64k contexts).
        const int target = env_int("LRA_DECODE_TARGET_WG", 256);
        const long long c = ((long long)max_ctx_len * units + target - 1) / (target > 0 ? target : 256);
        chunk = 256;
        while (chunk < 4096 && chunk < c) chunk *= 2;
    }
    p->chunk = chunk;
    p->n_split = max_ctx_len > 0 ? (max_ctx_len + chunk - 1) / chunk : 1;
    const long long wgs = units * p->n_split;
    if (wgs > 0x7ffffff0LL) return false;
    p->grid = (int)((wgs + 7) / 8 * 8);
    // Persistent workgroups (a queue of the chunks that exist) once the grid
    // would take several rounds of the GPU: the workgroup prologue and merge
    // tail then stop being paid per launch round, and missing chunks of
    // shorter contexts cost nothing.  Needs the workspace queue words and the
    // per-context prefix sums in LDS.
    const int per = env_int("LRA_DECODE_PERSISTENT", -1);
    p->persistent = p->n_split > 1 && n_ctx <= 1024 && (per == 1 || (per != 0 && wgs > 4 * 256));
    // partial row: [O_base | O_lr], then (m, l) padded to 16 bytes
    const int dr2 = d.head_dim + d.rank + 4;
    // per-unit merge counters, then the queue head and the workgroups-done count
    p->ws_counter_bytes = ((size_t)(p->n_units + 2) * sizeof(int32_t) + 255) / 256 * 256;
    p->ws_part_bytes = p->n_split > 1 ? (size_t)p->n_units * p->n_split * 16 * dr2 * sizeof(float) : 0;
    p->ws_total = p->n_split > 1 ? p->ws_counter_bytes + p->ws_part_bytes : 0;
    return true;
}

size_t prefill_paged_workspace(int h_kv, int d, int r, int kv_len) {
    auto al = [](size_t b) { return (b + 255) / 256 * 256; };
    return 2 * al((size_t)h_kv * kv_len * d * 2) + 2 * al((size_t)kv_len * r * 2);
}

}  // namespace lra

extern "C" {

int32_t lra_abi_version(void) { return LRA_ABI_VERSION; }

const char* lra_status_str(lra_status s) {
    switch (s) {
        case LRA_OK: return "LRA_OK";
        case LRA_ERR_NULL_PTR: return "LRA_ERR_NULL_PTR: a required pointer is NULL";
        case LRA_ERR_BAD_SHAPE: return "LRA_ERR_BAD_SHAPE: inconsistent or out-of-range sizes";
        case LRA_ERR_UNSUPPORTED: return "LRA_ERR_UNSUPPORTED: valid but not implemented";
        case LRA_ERR_MISALIGNED: return "LRA_ERR_MISALIGNED: device pointer not 16-byte aligned";
        case LRA_ERR_WORKSPACE_TOO_SMALL: return "LRA_ERR_WORKSPACE_TOO_SMALL: workspace below the queried size";
        case LRA_ERR_HIP: return "LRA_ERR_HIP: a HIP call or kernel launch failed";
        default: return "unknown lra_status";
    }
}

const char* lra_last_error(void) { return g_err; }

size_t lra_attn_decode_workspace_size(const lra_dims* dims, int32_t n_req, int32_t n_ctx,
                                      int32_t max_req_per_ctx, int32_t max_ctx_len) {
    if (check_dims(dims) != LRA_OK) return 0;
    if (dims->dtype != LRA_BF16) return 0;
    lra::DecodePlan p;
    if (!lra::decode_plan(*dims, n_req, n_ctx, max_req_per_ctx, max_ctx_len, &p)) return 0;
    return p.ws_total;
}

}  // extern "C"

namespace {

// ---- scratch of lra_attn_decode_noalloc: a file-scope device array, one copy
// per GPU.  Its first NOALLOC_COUNTER_BYTES hold the merge counters and the
// persistent queue words, the rest the chunk partials.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
constexpr size_t NOALLOC_COUNTER_BYTES = LRA_DECODE_NOALLOC_COUNTER_BYTES;
constexpr size_t NOALLOC_SCRATCH_BYTES = LRA_DECODE_NOALLOC_SCRATCH_BYTES;
static_assert(NOALLOC_COUNTER_BYTES % 256 == 0 && NOALLOC_SCRATCH_BYTES > NOALLOC_COUNTER_BYTES, "scratch layout");
__device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

// zero-fill of the counter words (a kernel, so callers under graph capture
// record no memset node)
__global__ void lra_zero_words_kernel(int32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// Device address of the current device's scratch.  The first call on a device
// looks the address up (with that device current) and clears the counter words
// on `stream`; every completed decode leaves them at zero again.
lra_status noalloc_scratch(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
        return fail(LRA_ERR_HIP, "decode_noalloc: no current device (or device index >= %d)", MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return fail(LRA_ERR_HIP, "decode_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
        const int n = (int)(NOALLOC_COUNTER_BYTES / sizeof(int32_t));
        hipLaunchKernelGGL(lra_zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, (int32_t*)ptr, n);
        const lra_status st = lra::check_launch("lra_zero_words_kernel");
        if (st != LRA_OK) return st;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return LRA_OK;
}

lra_status decode_entry(const lra_dims* dims, const void* q, int32_t n_req,
                        const int32_t* ctx_req_start, int32_t n_ctx, int32_t max_req_per_ctx,
                        const int32_t* req_agent, const void* k_pool, const void* v_pool,
                        const void* lk_pool, const void* lv_pool, int32_t n_pages,
                        int32_t page_size, const int32_t* block_table, int32_t max_blocks,
                        const int32_t* ctx_len, int32_t max_ctx_len, const void* b_k,
                        const void* b_v, int32_t n_agents, const float* rope_cos,
                        const float* rope_sin, int32_t rope_rows, void* out, void* workspace,
                        size_t workspace_bytes, bool noalloc, void* stream) {
    g_err[0] = 0;
    lra_status st = check_dims(dims);
    if (st != LRA_OK) return st;
    if (page_size != 16) return fail(LRA_ERR_UNSUPPORTED, "page_size %d (supported: 16)", page_size);
    if (n_req < 0) return fail(LRA_ERR_BAD_SHAPE, "n_req %d < 0", n_req);
    if (n_ctx < 1) return fail(LRA_ERR_BAD_SHAPE, "n_ctx %d < 1", n_ctx);
    if (max_req_per_ctx < 1 || max_req_per_ctx > (n_req > 0 ? n_req : 1))
        return fail(LRA_ERR_BAD_SHAPE, "max_req_per_ctx %d outside [1, n_req=%d]", max_req_per_ctx, n_req);
    if (n_pages < 1) return fail(LRA_ERR_BAD_SHAPE, "n_pages %d < 1", n_pages);
    if (max_blocks < 1) return fail(LRA_ERR_BAD_SHAPE, "max_blocks %d < 1", max_blocks);
    if (max_ctx_len < 0 || (long long)max_ctx_len > (long long)max_blocks * page_size)
        return fail(LRA_ERR_BAD_SHAPE, "max_ctx_len %d outside [0, max_blocks*page_size=%lld]",
                    max_ctx_len, (long long)max_blocks * page_size);
    if (n_agents < 1) return fail(LRA_ERR_BAD_SHAPE, "n_agents %d < 1", n_agents);
    const int g = dims->n_q_heads / dims->n_kv_heads;
    if (dims->dtype == LRA_BF16 && g > 16)
        return fail(LRA_ERR_UNSUPPORTED, "bf16 decode packs at most 16 query heads per KV head (g=%d)", g);
    REQUIRE_PTR(q);
    REQUIRE_PTR(ctx_req_start);
    REQUIRE_PTR(req_agent);
    REQUIRE_PTR(k_pool);
    REQUIRE_PTR(v_pool);
    REQUIRE_PTR(lk_pool);
    REQUIRE_PTR(lv_pool);
    REQUIRE_PTR(block_table);
    REQUIRE_PTR(ctx_len);
    REQUIRE_PTR(b_k);
    REQUIRE_PTR(b_v);
    REQUIRE_PTR(out);
    if ((rope_cos == nullptr) != (rope_sin == nullptr))
        return fail(LRA_ERR_NULL_PTR, "rope_cos and rope_sin must be both NULL or both set");
    if (rope_cos && (!aligned16(rope_cos) || !aligned16(rope_sin)))
        return fail(LRA_ERR_MISALIGNED, "rope tables are not 16-byte aligned");
    if (rope_cos && rope_rows < (max_ctx_len > 1 ? max_ctx_len : 1))
        return fail(LRA_ERR_BAD_SHAPE, "rope tables hold %d rows < max(max_ctx_len, 1) = %d", rope_rows,
                    max_ctx_len > 1 ? max_ctx_len : 1);
    if (dims->lr_agent_stride > 0 && dims->lr_agent_stride < (long long)n_pages * page_size * dims->rank)
        return fail(LRA_ERR_BAD_SHAPE, "lr_agent_stride %lld < one agent's LR pool (n_pages*page_size*r = %lld)",
                    (long long)dims->lr_agent_stride, (long long)n_pages * page_size * dims->rank);

    lra::DecodeArgs a;
    a.q = q;
    a.ctx_req_start = ctx_req_start;
    a.req_agent = req_agent;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.lk_pool = lk_pool;
    a.lv_pool = lv_pool;
    a.block_table = block_table;
    a.ctx_len = ctx_len;
    a.b_k = b_k;
    a.b_v = b_v;
    a.rope_cos = rope_cos;
    a.rope_sin = rope_sin;
    a.rope_rows = rope_cos ? rope_rows : 0;
    a.out = out;
    a.workspace = workspace;
    a.lr_stride = dims->lr_agent_stride;
    a.n_req = n_req;
    a.n_ctx = n_ctx;
    a.n_pages = n_pages;
    a.max_blocks = max_blocks;
    a.max_ctx_len = max_ctx_len;
    a.n_agents = n_agents;
    a.h_q = dims->n_q_heads;
    a.h_kv = dims->n_kv_heads;
    a.head_dim = dims->head_dim;
    a.rank = dims->rank;
    a.scale = eff_scale(dims);

    if (dims->dtype == LRA_F32) {
        if (n_req == 0) return LRA_OK;
        return lra::launch_decode_f32(a, (hipStream_t)stream);
    }
    lra::DecodePlan p;
    if (!lra::decode_plan(*dims, n_req, n_ctx, max_req_per_ctx, max_ctx_len, &p))
        return fail(LRA_ERR_BAD_SHAPE, "decode: problem too large to plan");
    if (noalloc) {
        // counters and partials at fixed offsets of the library's scratch
        if (p.ws_counter_bytes > NOALLOC_COUNTER_BYTES || p.ws_part_bytes > NOALLOC_SCRATCH_BYTES - NOALLOC_COUNTER_BYTES)
            return fail(LRA_ERR_WORKSPACE_TOO_SMALL,
                        "decode_noalloc: needs %zu counter and %zu partial bytes; the scratch holds %zu and %zu",
                        p.ws_counter_bytes, p.ws_part_bytes, NOALLOC_COUNTER_BYTES,
                        NOALLOC_SCRATCH_BYTES - NOALLOC_COUNTER_BYTES);
        if (n_req == 0) return LRA_OK;
        void* ptr = nullptr;
        const lra_status sst = noalloc_scratch((hipStream_t)stream, &ptr);
        if (sst != LRA_OK) return sst;
        a.workspace = ptr;
        p.ws_counter_bytes = NOALLOC_COUNTER_BYTES;
        return lra::launch_decode_bf16(a, p, (hipStream_t)stream);
    }
    if (p.ws_total > 0) {
        if (!workspace) return fail(LRA_ERR_NULL_PTR, "workspace is NULL (need %zu bytes)", p.ws_total);
        if (!aligned16(workspace)) return fail(LRA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
        if (workspace_bytes < p.ws_total)
            return fail(LRA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu", workspace_bytes, p.ws_total);
    }
    if (n_req == 0) return LRA_OK;
    return lra::launch_decode_bf16(a, p, (hipStream_t)stream);
}

}  // namespace

extern "C" {

lra_status lra_attn_decode(const lra_dims* dims, const void* q, int32_t n_req,
                           const int32_t* ctx_req_start, int32_t n_ctx, int32_t max_req_per_ctx,
                           const int32_t* req_agent, const void* k_pool, const void* v_pool,
                           const void* lk_pool, const void* lv_pool, int32_t n_pages,
                           int32_t page_size, const int32_t* block_table, int32_t max_blocks,
                           const int32_t* ctx_len, int32_t max_ctx_len, const void* b_k,
                           const void* b_v, int32_t n_agents, const float* rope_cos,
                           const float* rope_sin, int32_t rope_rows, void* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return decode_entry(dims, q, n_req, ctx_req_start, n_ctx, max_req_per_ctx, req_agent, k_pool, v_pool,
                        lk_pool, lv_pool, n_pages, page_size, block_table, max_blocks, ctx_len, max_ctx_len,
                        b_k, b_v, n_agents, rope_cos, rope_sin, rope_rows, out, workspace, workspace_bytes,
                        false, stream);
}

lra_status lra_attn_decode_noalloc(const lra_dims* dims, const void* q, int32_t n_req,
                                   const int32_t* ctx_req_start, int32_t n_ctx, int32_t max_req_per_ctx,
                                   const int32_t* req_agent, const void* k_pool, const void* v_pool,
                                   const void* lk_pool, const void* lv_pool, int32_t n_pages,
                                   int32_t page_size, const int32_t* block_table, int32_t max_blocks,
                                   const int32_t* ctx_len, int32_t max_ctx_len, const void* b_k,
                                   const void* b_v, int32_t n_agents, const float* rope_cos,
                                   const float* rope_sin, int32_t rope_rows, void* out, void* stream) {
    if (dims && dims->dtype != LRA_BF16) {
        g_err[0] = 0;
        return fail(LRA_ERR_UNSUPPORTED, "decode_noalloc: bf16 only (the fp32 path uses no scratch)");
    }
    return decode_entry(dims, q, n_req, ctx_req_start, n_ctx, max_req_per_ctx, req_agent, k_pool, v_pool,
                        lk_pool, lv_pool, n_pages, page_size, block_table, max_blocks, ctx_len, max_ctx_len,
                        b_k, b_v, n_agents, rope_cos, rope_sin, rope_rows, out, nullptr, 0, true, stream);
}

lra_status lra_attn_prefill(const lra_dims* dims, const void* q, int32_t n_req, int32_t q_len,
                            const int32_t* req_agent, const void* k_base, const void* v_base,
                            int32_t kv_len, const void* l_k, const void* l_v, const void* b_k,
                            const void* b_v, int32_t n_agents, const float* rope_cos,
                            const float* rope_sin, int32_t rope_rows, void* out, void* stream) {
    g_err[0] = 0;
    lra_status st = check_dims(dims);
    if (st != LRA_OK) return st;
    if (n_req < 0) return fail(LRA_ERR_BAD_SHAPE, "n_req %d < 0", n_req);
    if (q_len < 1) return fail(LRA_ERR_BAD_SHAPE, "q_len %d < 1", q_len);
    if (kv_len < q_len) return fail(LRA_ERR_BAD_SHAPE, "kv_len %d < q_len %d", kv_len, q_len);
    if (n_agents < 1) return fail(LRA_ERR_BAD_SHAPE, "n_agents %d < 1", n_agents);
    if ((rope_cos == nullptr) != (rope_sin == nullptr))
        return fail(LRA_ERR_NULL_PTR, "rope_cos and rope_sin must both be given or both NULL");
    REQUIRE_PTR(q);
    REQUIRE_PTR(req_agent);
    REQUIRE_PTR(k_base);
    REQUIRE_PTR(v_base);
    REQUIRE_PTR(l_k);
    REQUIRE_PTR(l_v);
    REQUIRE_PTR(b_k);
    REQUIRE_PTR(b_v);
    REQUIRE_PTR(out);
    if (rope_cos) {
        REQUIRE_PTR(rope_cos);
        REQUIRE_PTR(rope_sin);
        if (rope_rows < kv_len)
            return fail(LRA_ERR_BAD_SHAPE, "rope tables hold %d rows < kv_len %d", rope_rows, kv_len);
    }
    if (dims->lr_agent_stride > 0 && dims->lr_agent_stride < (long long)kv_len * dims->rank)
        return fail(LRA_ERR_BAD_SHAPE, "lr_agent_stride %lld < one agent's LR cache (kv_len*r = %lld)",
                    (long long)dims->lr_agent_stride, (long long)kv_len * dims->rank);
    lra::PrefillArgs a;
    a.q = q;
    a.req_agent = req_agent;
    a.k_base = k_base;
    a.v_base = v_base;
    a.l_k = l_k;
    a.l_v = l_v;
    a.b_k = b_k;
    a.b_v = b_v;
    a.rope_cos = rope_cos;
    a.rope_sin = rope_sin;
    a.out = out;
    a.lr_stride = dims->lr_agent_stride;
    a.n_req = n_req;
    a.q_len = q_len;
    a.kv_len = kv_len;
    a.n_agents = n_agents;
    a.h_q = dims->n_q_heads;
    a.h_kv = dims->n_kv_heads;
    a.head_dim = dims->head_dim;
    a.rank = dims->rank;
    a.scale = eff_scale(dims);
    if (n_req == 0) return LRA_OK;
    if (dims->dtype == LRA_F32) return lra::launch_prefill_f32(a, (hipStream_t)stream);
    return lra::launch_prefill_bf16(a, (hipStream_t)stream);
}

lra_status lra_attn_prefill_paged(const lra_dims* dims, const void* q, int32_t n_req, int32_t q_len,
                                  const int32_t* req_agent, const void* k_pool, const void* v_pool,
                                  const void* lk_pool, const void* lv_pool, int32_t n_pages,
                                  int32_t page_size, const int32_t* block_table, int32_t max_blocks,
                                  int32_t kv_len, const void* b_k, const void* b_v, int32_t n_agents,
                                  const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                                  void* out, void* stream) {
    g_err[0] = 0;
    lra_status st = check_dims(dims);
    if (st != LRA_OK) return st;
    if (dims->dtype != LRA_BF16) return fail(LRA_ERR_UNSUPPORTED, "paged prefill: bf16 only");
    if (page_size != 16) return fail(LRA_ERR_UNSUPPORTED, "page_size %d (supported: 16)", page_size);
    if (n_pages < 1) return fail(LRA_ERR_BAD_SHAPE, "n_pages %d < 1", n_pages);
    if (n_req < 0) return fail(LRA_ERR_BAD_SHAPE, "n_req %d < 0", n_req);
    if (q_len < 1) return fail(LRA_ERR_BAD_SHAPE, "q_len %d < 1", q_len);
    if (kv_len < q_len) return fail(LRA_ERR_BAD_SHAPE, "kv_len %d < q_len %d", kv_len, q_len);
    if (max_blocks < 1 || (long long)max_blocks * page_size < kv_len)
        return fail(LRA_ERR_BAD_SHAPE, "max_blocks %d cannot hold kv_len %d", max_blocks, kv_len);
    if (n_agents < 1) return fail(LRA_ERR_BAD_SHAPE, "n_agents %d < 1", n_agents);
    if ((rope_cos == nullptr) != (rope_sin == nullptr))
        return fail(LRA_ERR_NULL_PTR, "rope_cos and rope_sin must both be given or both NULL");
    if (dims->lr_agent_stride > 0 && dims->lr_agent_stride < (long long)n_pages * page_size * dims->rank)
        return fail(LRA_ERR_BAD_SHAPE, "lr_agent_stride %lld < one agent's LR pool (n_pages*page_size*r = %lld)",
                    (long long)dims->lr_agent_stride, (long long)n_pages * page_size * dims->rank);
    REQUIRE_PTR(q);
    REQUIRE_PTR(req_agent);
    REQUIRE_PTR(k_pool);
    REQUIRE_PTR(v_pool);
    REQUIRE_PTR(lk_pool);
    REQUIRE_PTR(lv_pool);
    REQUIRE_PTR(block_table);
    REQUIRE_PTR(b_k);
    REQUIRE_PTR(b_v);
    REQUIRE_PTR(out);
    if (rope_cos) {
        if (rope_rows < kv_len)
            return fail(LRA_ERR_BAD_SHAPE, "rope tables hold %d rows < kv_len %d", rope_rows, kv_len);
    }
    lra::PrefillArgs a;
    a.q = q;
    a.req_agent = req_agent;
    a.k_base = k_pool;
    a.v_base = v_pool;
    a.l_k = lk_pool;
    a.l_v = lv_pool;
    a.b_k = b_k;
    a.b_v = b_v;
    a.rope_cos = rope_cos;
    a.rope_sin = rope_sin;
    a.out = out;
    a.lr_stride = dims->lr_agent_stride;
    a.n_req = n_req;
    a.q_len = q_len;
    a.kv_len = kv_len;
    a.n_agents = n_agents;
    a.h_q = dims->n_q_heads;
    a.h_kv = dims->n_kv_heads;
    a.head_dim = dims->head_dim;
    a.rank = dims->rank;
    a.scale = eff_scale(dims);
    a.block_table = block_table;
    a.max_blocks = max_blocks;
    a.n_pages = n_pages;
    if (n_req == 0) return LRA_OK;
    return lra::launch_prefill_bf16(a, (hipStream_t)stream);
}

size_t lra_attn_prefill_paged_staged_workspace_size(const lra_dims* dims, int32_t kv_len) {
    if (check_dims(dims) != LRA_OK || dims->dtype != LRA_BF16 || kv_len < 0) return 0;
    return lra::prefill_paged_workspace(dims->n_kv_heads, dims->head_dim, dims->rank, kv_len);
}

lra_status lra_attn_prefill_paged_staged(const lra_dims* dims, const void* q, int32_t n_req, int32_t q_len,
                                         const int32_t* req_agent, const void* k_pool, const void* v_pool,
                                         const void* lk_pool, const void* lv_pool, int32_t n_pages,
                                         int32_t page_size, const int32_t* block_table, int32_t max_blocks,
                                         int32_t kv_len, const void* b_k, const void* b_v, int32_t n_agents,
                                         const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                                         void* out, void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    lra_status st = check_dims(dims);
    if (st != LRA_OK) return st;
    if (dims->dtype != LRA_BF16) return fail(LRA_ERR_UNSUPPORTED, "paged prefill: bf16 only");
    if (dims->lr_agent_stride != 0)
        return fail(LRA_ERR_UNSUPPORTED, "staged paged prefill: shared LR cache only (lr_agent_stride 0)");
    if (page_size != 16) return fail(LRA_ERR_UNSUPPORTED, "page_size %d (supported: 16)", page_size);
    if (n_pages < 1) return fail(LRA_ERR_BAD_SHAPE, "n_pages %d < 1", n_pages);
    if (q_len < 1) return fail(LRA_ERR_BAD_SHAPE, "q_len %d < 1", q_len);
    if (kv_len < q_len) return fail(LRA_ERR_BAD_SHAPE, "kv_len %d < q_len %d", kv_len, q_len);
    if (max_blocks < 1 || (long long)max_blocks * page_size < kv_len)
        return fail(LRA_ERR_BAD_SHAPE, "max_blocks %d cannot hold kv_len %d", max_blocks, kv_len);
    REQUIRE_PTR(k_pool);
    REQUIRE_PTR(v_pool);
    REQUIRE_PTR(lk_pool);
    REQUIRE_PTR(lv_pool);
    REQUIRE_PTR(block_table);
    REQUIRE_PTR(workspace);
    const size_t need = lra::prefill_paged_workspace(dims->n_kv_heads, dims->head_dim, dims->rank, kv_len);
    if (workspace_bytes < need)
        return fail(LRA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu", workspace_bytes, need);
    auto al = [](size_t b) { return (b + 255) / 256 * 256; };
    char* w = (char*)workspace;
    const size_t kvb = al((size_t)dims->n_kv_heads * kv_len * dims->head_dim * 2);
    const size_t lb = al((size_t)kv_len * dims->rank * 2);
    lra::PagedArgs g{};
    g.block_table = block_table;
    g.k_pool = (void*)k_pool;
    g.v_pool = (void*)v_pool;
    g.lk_pool = (void*)lk_pool;
    g.lv_pool = (void*)lv_pool;
    g.k_out = w;
    g.v_out = w + kvb;
    g.lk_out = w + 2 * kvb;
    g.lv_out = w + 2 * kvb + lb;
    g.n_pages = n_pages;
    g.h_kv = dims->n_kv_heads;
    g.kv_len = kv_len;
    g.head_dim = dims->head_dim;
    g.rank = dims->rank;
    // the staged rows feed the contiguous prefill: validate its arguments first
    // (a failing call launches nothing)
    if (n_req < 0) return fail(LRA_ERR_BAD_SHAPE, "n_req %d < 0", n_req);
    if (n_agents < 1) return fail(LRA_ERR_BAD_SHAPE, "n_agents %d < 1", n_agents);
    if ((rope_cos == nullptr) != (rope_sin == nullptr))
        return fail(LRA_ERR_NULL_PTR, "rope_cos and rope_sin must both be given or both NULL");
    REQUIRE_PTR(q);
    REQUIRE_PTR(req_agent);
    REQUIRE_PTR(b_k);
    REQUIRE_PTR(b_v);
    REQUIRE_PTR(out);
    if (rope_cos) {
        REQUIRE_PTR(rope_cos);
        REQUIRE_PTR(rope_sin);
        if (rope_rows < kv_len)
            return fail(LRA_ERR_BAD_SHAPE, "rope tables hold %d rows < kv_len %d", rope_rows, kv_len);
    }
    if (n_req == 0) return LRA_OK;
    st = lra::launch_cache_gather_bf16(g, (hipStream_t)stream);
    if (st != LRA_OK) return st;
    return lra_attn_prefill(dims, q, n_req, q_len, req_agent, g.k_out, g.v_out, kv_len, g.lk_out,
                            g.lv_out, b_k, b_v, n_agents, rope_cos, rope_sin, rope_rows, out, stream);
}

lra_status lra_cache_append(const lra_dims* dims, int32_t n_tok, const int64_t* slot_mapping,
                            const void* k_new, const void* v_new, const void* lk_new,
                            const void* lv_new, int32_t n_lr, void* k_pool, void* v_pool, void* lk_pool,
                            void* lv_pool, int32_t n_pages, int32_t page_size, void* stream) {
    g_err[0] = 0;
    lra_status st = check_dims(dims);
    if (st != LRA_OK) return st;
    if (dims->dtype != LRA_BF16) return fail(LRA_ERR_UNSUPPORTED, "cache append: bf16 only");
    if (page_size != 16) return fail(LRA_ERR_UNSUPPORTED, "page_size %d (supported: 16)", page_size);
    if (n_tok < 0) return fail(LRA_ERR_BAD_SHAPE, "n_tok %d < 0", n_tok);
    if (n_pages < 1) return fail(LRA_ERR_BAD_SHAPE, "n_pages %d < 1", n_pages);
    if (n_lr < 1) return fail(LRA_ERR_BAD_SHAPE, "n_lr %d < 1", n_lr);
    if (dims->lr_agent_stride == 0 && n_lr != 1)
        return fail(LRA_ERR_BAD_SHAPE, "n_lr %d LR row sets need per-agent pools (lr_agent_stride > 0)", n_lr);
    if (dims->lr_agent_stride > 0 && dims->lr_agent_stride < (long long)n_pages * page_size * dims->rank)
        return fail(LRA_ERR_BAD_SHAPE, "lr_agent_stride %lld < one agent's LR pool (n_pages*page_size*r = %lld)",
                    (long long)dims->lr_agent_stride, (long long)n_pages * page_size * dims->rank);
    REQUIRE_PTR(slot_mapping);
    REQUIRE_PTR(k_new);
    REQUIRE_PTR(v_new);
    REQUIRE_PTR(lk_new);
    REQUIRE_PTR(lv_new);
    REQUIRE_PTR(k_pool);
    REQUIRE_PTR(v_pool);
    REQUIRE_PTR(lk_pool);
    REQUIRE_PTR(lv_pool);
    if (n_tok == 0) return LRA_OK;
    lra::PagedArgs a{};
    a.slots = slot_mapping;
    a.k_rows = k_new;
    a.v_rows = v_new;
    a.lk_rows = lk_new;
    a.lv_rows = lv_new;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.lk_pool = lk_pool;
    a.lv_pool = lv_pool;
    a.n_tok = n_tok;
    a.n_pages = n_pages;
    a.h_kv = dims->n_kv_heads;
    a.head_dim = dims->head_dim;
    a.rank = dims->rank;
    a.n_lr = n_lr;
    a.lr_stride = dims->lr_agent_stride;
    return lra::launch_cache_append_bf16(a, (hipStream_t)stream);
}

size_t lra_lr_cache_build_workspace_size(int32_t dtype, int32_t n_tok, int32_t d_model, int32_t rank,
                                        int32_t n_lr) {
    if (dtype != LRA_BF16 || n_tok <= 0 || d_model <= 0 || d_model % 32 != 0 || n_lr < 1) return 0;
    if (rank != 4 && rank != 8 && rank != 16 && rank != 32) return 0;
    return lra::lr_build_plan(n_tok, d_model, rank, n_lr).ws_bytes;
}

lra_status lra_lr_cache_build(int32_t dtype, const void* x, int32_t n_tok, int32_t d_model,
                              const void* a_k, const void* a_v, int32_t rank, int32_t n_lr,
                              void* l_k, void* l_v, int64_t row_offset, int64_t lr_agent_stride,
                              void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    if (dtype != LRA_F32 && dtype != LRA_BF16)
        return fail(LRA_ERR_UNSUPPORTED, "dtype %d (expected LRA_F32=0 or LRA_BF16=1)", dtype);
    if (rank != 4 && rank != 8 && rank != 16 && rank != 32)
        return fail(LRA_ERR_UNSUPPORTED, "rank %d (supported: 4, 8, 16, 32)", rank);
    if (n_tok < 0) return fail(LRA_ERR_BAD_SHAPE, "n_tok %d < 0", n_tok);
    if (d_model <= 0) return fail(LRA_ERR_BAD_SHAPE, "d_model %d <= 0", d_model);
    if (d_model % 32 != 0) return fail(LRA_ERR_UNSUPPORTED, "d_model %d is not a multiple of 32", d_model);
    if (row_offset < 0) return fail(LRA_ERR_BAD_SHAPE, "row_offset %lld < 0", (long long)row_offset);
    if (n_lr < 1) return fail(LRA_ERR_BAD_SHAPE, "n_lr %d < 1", n_lr);
    if (n_lr > 1 && lr_agent_stride < (row_offset + n_tok) * (long long)rank)
        return fail(LRA_ERR_BAD_SHAPE, "lr_agent_stride %lld smaller than one cache's rows (%lld)",
                    (long long)lr_agent_stride, (long long)(row_offset + n_tok) * rank);
    REQUIRE_PTR(x);
    REQUIRE_PTR(a_k);
    REQUIRE_PTR(a_v);
    REQUIRE_PTR(l_k);
    REQUIRE_PTR(l_v);
    lra::LRBuildArgs a;
    a.x = x;
    a.a_k = a_k;
    a.a_v = a_v;
    a.l_k = l_k;
    a.l_v = l_v;
    a.n_tok = n_tok;
    a.d_model = d_model;
    a.rank = rank;
    a.n_lr = n_lr;
    a.row_offset = row_offset;
    a.lr_stride = n_lr > 1 ? lr_agent_stride : 0;
    a.workspace = nullptr;
    if (n_tok == 0) return LRA_OK;
    if (workspace != nullptr && dtype == LRA_BF16) {
        const size_t need = lra::lr_build_plan(n_tok, d_model, rank, n_lr).ws_bytes;
        if (need > 0) {
            if (!aligned16(workspace)) return fail(LRA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
            if (workspace_bytes < need)
                return fail(LRA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu", workspace_bytes, need);
            a.workspace = workspace;
        }
    }
    if (dtype == LRA_F32) return lra::launch_lr_build_f32(a, (hipStream_t)stream);
    return lra::launch_lr_build_bf16(a, (hipStream_t)stream);
}

lra_status lra_naive_expand_pages(const lra_dims* dims, int32_t n_req, const int32_t* ctx_req_start,
                                  int32_t n_ctx, const int32_t* req_agent, const void* k_pool,
                                  const void* v_pool, const void* lk_pool, const void* lv_pool,
                                  int32_t n_pages, int32_t page_size, const int32_t* block_table,
                                  int32_t max_blocks, const int32_t* ctx_len, const void* b_k,
                                  const void* b_v, int32_t n_agents, void* k_out, void* v_out,
                                  int32_t out_blocks, void* stream) {
    g_err[0] = 0;
    lra_status st = check_dims(dims);
    if (st != LRA_OK) return st;
    if (dims->dtype != LRA_BF16) return fail(LRA_ERR_UNSUPPORTED, "naive expand: bf16 only");
    if (dims->lr_agent_stride > 0 && dims->lr_agent_stride < (long long)n_pages * page_size * dims->rank)
        return fail(LRA_ERR_BAD_SHAPE, "lr_agent_stride %lld < one agent's LR pool (n_pages*page_size*r = %lld)",
                    (long long)dims->lr_agent_stride, (long long)n_pages * page_size * dims->rank);
    if (page_size != 16) return fail(LRA_ERR_UNSUPPORTED, "page_size %d (supported: 16)", page_size);
    if (n_req < 0) return fail(LRA_ERR_BAD_SHAPE, "n_req %d < 0", n_req);
    if (n_ctx < 1) return fail(LRA_ERR_BAD_SHAPE, "n_ctx %d < 1", n_ctx);
    if (n_pages < 1) return fail(LRA_ERR_BAD_SHAPE, "n_pages %d < 1", n_pages);
    if (max_blocks < 1) return fail(LRA_ERR_BAD_SHAPE, "max_blocks %d < 1", max_blocks);
    if (out_blocks < 1 || out_blocks > max_blocks)
        return fail(LRA_ERR_BAD_SHAPE, "out_blocks %d outside [1, max_blocks=%d]", out_blocks, max_blocks);
    if (n_agents < 1) return fail(LRA_ERR_BAD_SHAPE, "n_agents %d < 1", n_agents);
    REQUIRE_PTR(ctx_req_start);
    REQUIRE_PTR(req_agent);
    REQUIRE_PTR(k_pool);
    REQUIRE_PTR(v_pool);
    REQUIRE_PTR(lk_pool);
    REQUIRE_PTR(lv_pool);
    REQUIRE_PTR(block_table);
    REQUIRE_PTR(ctx_len);
    REQUIRE_PTR(b_k);
    REQUIRE_PTR(b_v);
    REQUIRE_PTR(k_out);
    REQUIRE_PTR(v_out);
    lra::ExpandArgs a;
    a.ctx_req_start = ctx_req_start;
    a.req_agent = req_agent;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.lk_pool = lk_pool;
    a.lv_pool = lv_pool;
    a.block_table = block_table;
    a.ctx_len = ctx_len;
    a.b_k = b_k;
    a.b_v = b_v;
    a.k_out = k_out;
    a.v_out = v_out;
    a.n_req = n_req;
    a.n_ctx = n_ctx;
    a.n_pages = n_pages;
    a.max_blocks = max_blocks;
    a.n_agents = n_agents;
    a.out_blocks = out_blocks;
    a.lr_stride = dims->lr_agent_stride;
    a.h_kv = dims->n_kv_heads;
    a.head_dim = dims->head_dim;
    a.rank = dims->rank;
    if (n_req == 0) return LRA_OK;
    return lra::launch_naive_expand_bf16(a, (hipStream_t)stream);
}

size_t lra_naive_prefill_workspace_size(const lra_dims* dims, int32_t n_req, int32_t kv_len) {
    if (check_dims(dims) != LRA_OK || dims->dtype != LRA_BF16 || n_req < 0 || kv_len < 0) return 0;
    return 2 * (((size_t)n_req * dims->n_kv_heads * kv_len * dims->head_dim * 2 + 255) / 256 * 256);
}

lra_status lra_naive_prefill(const lra_dims* dims, const void* q, int32_t n_req, int32_t q_len,
                             const int32_t* req_agent, const void* k_base, const void* v_base,
                             int32_t kv_len, const void* l_k, const void* l_v, const void* b_k,
                             const void* b_v, int32_t n_agents, const float* rope_cos,
                             const float* rope_sin, int32_t rope_rows, void* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    lra_status st = check_dims(dims);
    if (st != LRA_OK) return st;
    if (dims->dtype != LRA_BF16) return fail(LRA_ERR_UNSUPPORTED, "naive prefill: bf16 only");
    if (n_req < 0) return fail(LRA_ERR_BAD_SHAPE, "n_req %d < 0", n_req);
    if (q_len < 1) return fail(LRA_ERR_BAD_SHAPE, "q_len %d < 1", q_len);
    if (kv_len < q_len) return fail(LRA_ERR_BAD_SHAPE, "kv_len %d < q_len %d", kv_len, q_len);
    if (n_agents < 1) return fail(LRA_ERR_BAD_SHAPE, "n_agents %d < 1", n_agents);
    if ((rope_cos == nullptr) != (rope_sin == nullptr))
        return fail(LRA_ERR_NULL_PTR, "rope_cos and rope_sin must both be given or both NULL");
    REQUIRE_PTR(q);
    REQUIRE_PTR(req_agent);
    REQUIRE_PTR(k_base);
    REQUIRE_PTR(v_base);
    REQUIRE_PTR(l_k);
    REQUIRE_PTR(l_v);
    REQUIRE_PTR(b_k);
    REQUIRE_PTR(b_v);
    REQUIRE_PTR(out);
    REQUIRE_PTR(workspace);
    if (rope_cos) {
        REQUIRE_PTR(rope_cos);
        REQUIRE_PTR(rope_sin);
        if (rope_rows < kv_len)
            return fail(LRA_ERR_BAD_SHAPE, "rope tables hold %d rows < kv_len %d", rope_rows, kv_len);
    }
    if (dims->lr_agent_stride > 0 && dims->lr_agent_stride < (long long)kv_len * dims->rank)
        return fail(LRA_ERR_BAD_SHAPE, "lr_agent_stride %lld < one agent's LR cache (kv_len*r = %lld)",
                    (long long)dims->lr_agent_stride, (long long)kv_len * dims->rank);
    const size_t need = lra_naive_prefill_workspace_size(dims, n_req, kv_len);
    if (workspace_bytes < need)
        return fail(LRA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu", workspace_bytes, need);
    if ((long long)kv_len * 2 * dims->head_dim > 0x7fffffffLL)
        return fail(LRA_ERR_BAD_SHAPE, "naive prefill: kv_len %d too long", kv_len);
    if (n_req == 0) return LRA_OK;
    lra::ExpandContigArgs e;
    e.req_agent = req_agent;
    e.k_base = k_base;
    e.v_base = v_base;
    e.l_k = l_k;
    e.l_v = l_v;
    e.b_k = b_k;
    e.b_v = b_v;
    e.rope_cos = rope_cos;
    e.rope_sin = rope_sin;
    e.k_out = workspace;
    e.v_out = (char*)workspace + need / 2;
    e.lr_stride = dims->lr_agent_stride;
    e.n_req = n_req;
    e.kv_len = kv_len;
    e.n_agents = n_agents;
    e.h_kv = dims->n_kv_heads;
    e.head_dim = dims->head_dim;
    e.rank = dims->rank;
    st = lra::launch_naive_expand_contig_bf16(e, (hipStream_t)stream);
    if (st != LRA_OK) return st;
    lra::PrefillArgs a;
    a.q = q;
    a.req_agent = req_agent;
    a.k_base = e.k_out;
    a.v_base = e.v_out;
    a.l_k = l_k;  // unused by the plain mode
    a.l_v = l_v;
    a.b_k = b_k;
    a.b_v = b_v;
    a.rope_cos = nullptr;  // the expanded keys carry the rotation
    a.rope_sin = nullptr;
    a.out = out;
    a.lr_stride = 0;
    a.n_req = n_req;
    a.q_len = q_len;
    a.kv_len = kv_len;
    a.n_agents = n_agents;
    a.h_q = dims->n_q_heads;
    a.h_kv = dims->n_kv_heads;
    a.head_dim = dims->head_dim;
    a.rank = dims->rank;
    a.scale = eff_scale(dims);
    a.plain = true;
    a.kv_req_stride = (int64_t)dims->n_kv_heads * kv_len * dims->head_dim;
    return lra::launch_prefill_bf16(a, (hipStream_t)stream);
}

lra_status lra_rope_table_build(double theta, int32_t head_dim, int32_t n_pos, float* cos_out,
                                float* sin_out, void* stream) {
    g_err[0] = 0;
    if (!(theta > 0.0) || isinf(theta)) return fail(LRA_ERR_BAD_SHAPE, "theta must be finite and > 0");
    if (head_dim <= 0 || head_dim % 2 != 0) return fail(LRA_ERR_BAD_SHAPE, "head_dim %d must be even and > 0", head_dim);
    if (n_pos < 0) return fail(LRA_ERR_BAD_SHAPE, "n_pos %d < 0", n_pos);
    REQUIRE_PTR(cos_out);
    REQUIRE_PTR(sin_out);
    if (n_pos == 0) return LRA_OK;
    return lra::launch_rope_table(theta, head_dim, n_pos, cos_out, sin_out, (hipStream_t)stream);
}

lra_status lra_ceiling_hbm_read(const void* buf, size_t n_bytes, int32_t n_workgroups, int32_t flags,
                                uint32_t* sink, void* stream) {
    g_err[0] = 0;
    REQUIRE_PTR(buf);
    REQUIRE_PTR(sink);
    if (n_bytes == 0 || n_bytes % 16 != 0)
        return fail(LRA_ERR_BAD_SHAPE, "n_bytes %zu must be a positive multiple of 16", n_bytes);
    if (n_workgroups < 0 || n_workgroups > 65535)
        return fail(LRA_ERR_BAD_SHAPE, "n_workgroups %d outside [0, 65535]", n_workgroups);
    if (flags & ~(LRA_READ_NONTEMPORAL | LRA_READ_CHUNKED)) return fail(LRA_ERR_BAD_SHAPE, "unknown flags 0x%x", flags);
    int n_wg = n_workgroups;
    if (n_wg == 0) {  // 16 workgroups per CU of the 256, fewer when the buffer is small
        const uint64_t need = (n_bytes / 16 + 4095) / 4096;
        n_wg = (int)(need < 4096 ? need : 4096);
    }
    return lra::launch_ceiling_read(buf, n_bytes, n_wg, (flags & LRA_READ_NONTEMPORAL) != 0,
                                    (flags & LRA_READ_CHUNKED) != 0, sink, (hipStream_t)stream);
}

lra_status lra_ceiling_mfma_bf16(int32_t lds_operands, int32_t n_workgroups, int32_t iters, uint32_t* sink,
                                 void* stream) {
    g_err[0] = 0;
    REQUIRE_PTR(sink);
    if (lds_operands < 0 || lds_operands > 2) return fail(LRA_ERR_BAD_SHAPE, "lds_operands must be 0, 1 or 2");
    if (n_workgroups < 1 || n_workgroups > 65535)
        return fail(LRA_ERR_BAD_SHAPE, "n_workgroups %d outside [1, 65535]", n_workgroups);
    if (iters < 1 || iters > (1 << 20)) return fail(LRA_ERR_BAD_SHAPE, "iters %d outside [1, 2^20]", iters);
    return lra::launch_ceiling_mfma(lds_operands, n_workgroups, iters, sink, (hipStream_t)stream);
}

}  // extern "C"
