// fp32 Flash-LoRA-Attention (decode and prefill), one wavefront per query row.
//
// Serves dtype == LRA_F32: full fp32 arithmetic (no bf16 rounding anywhere),
// for small problems where latency, not bandwidth, dominates.  Same method as
// the bf16 kernels (LRAgent, arXiv 2602.01053v2, §3 and App. B): scores from
// q . k_base_j plus the pre-projected query against the shared rank-r row
// l_k_j (or, with RoPE, against the rebuilt key k_base_j + rot(l_k_j B_k^(h)),
// App. D.1, in decode and prefill alike), online softmax over 64-token chunks, value accumulation at head
// dimension for V_base and at rank r for L_v, and one B_v post-multiplication.
#include "lra_common.h"
#include "lra_internal.h"

namespace {

constexpr int PAGE = 16;

struct F32K {
    const float* q;
    const int32_t* ctx_req_start;  // decode only
    const int32_t* req_agent;
    const float* k;  // decode: pool [n_pages,H_kv,d/8,16,8]; prefill: [H_kv,kv_len,d]
    const float* v;  // decode: pool [n_pages,H_kv,d,16];     prefill: [H_kv,kv_len,d]
    const float* lk; // decode: pool [n_pages,16,r];          prefill: [kv_len,r]
    const float* lv; // decode: pool [n_pages,r,16];          prefill: [kv_len,r]
    const int32_t* block_table;
    const int32_t* ctx_len;
    const float* b_k;
    const float* b_v;
    const float* rope_cos;
    const float* rope_sin;
    float* out;
    int32_t n_req, n_ctx, n_pages, max_blocks, n_agents;
    int32_t q_len, kv_len;  // prefill
    int32_t max_len;        // decode: max_ctx_len (longer contexts are cut to it)
    int32_t h_q, h_kv, d, r;
    float scale;
    int64_t lr_stride;  // per-agent LR caches: elements between agents' caches (0: shared)
};

struct Paged {
    const F32K* a;
    const int32_t* bt;
    int h;
    size_t lr_off;  // this request's LR cache
    __device__ int pid(int j) const {
        int p = bt[j / PAGE];
        return min(max(p, 0), a->n_pages - 1);
    }
    __device__ float K(int j, int c) const {
        const int d = a->d;
        return a->k[(((size_t)pid(j) * a->h_kv + h) * (d / 8) + c / 8) * (PAGE * 8) + (j % PAGE) * 8 + c % 8];
    }
    __device__ float V(int j, int c) const {
        const int d = a->d;
        return a->v[(((size_t)pid(j) * a->h_kv + h) * d + c) * PAGE + j % PAGE];
    }
    __device__ float LK(int j, int t) const {
        return a->lk[lr_off + ((size_t)pid(j) * PAGE + j % PAGE) * a->r + t];
    }
    __device__ float LV(int j, int t) const {
        return a->lv[lr_off + ((size_t)pid(j) * a->r + t) * PAGE + j % PAGE];
    }
};

struct Contig {
    const F32K* a;
    int h;
    size_t lr_off;  // this request's LR cache
    __device__ float K(int j, int c) const { return a->k[((size_t)h * a->kv_len + j) * a->d + c]; }
    __device__ float V(int j, int c) const { return a->v[((size_t)h * a->kv_len + j) * a->d + c]; }
    __device__ float LK(int j, int t) const { return a->lk[lr_off + (size_t)j * a->r + t]; }
    __device__ float LV(int j, int t) const { return a->lv[lr_off + (size_t)j * a->r + t]; }
};

// One query row: q (length d) at absolute position `pos`, sees keys 0..pos.
template <typename Acc>
__device__ void row_attend(const F32K& a, const Acc& acc, const float* qrow, int agent, int h,
                           int pos, float* orow, bool rope) {
    __shared__ float s_q[128];
    __shared__ float s_qb[32];
    __shared__ float s_p[64];
    __shared__ float s_bk[32 * 128];  // B_k^(h) slice (rope path)
    __shared__ float s_olr[32];
    const int lane = threadIdx.x;
    const int d = a.d, r = a.r;
    const size_t bstride = (size_t)a.h_kv * d;
    const float* bk = a.b_k + (size_t)agent * r * bstride + (size_t)h * d;
    const float* bv = a.b_v + (size_t)agent * r * bstride + (size_t)h * d;
    for (int c = lane; c < d; c += 64) s_q[c] = qrow[c];
    // B_k^(h) slice, eight loads per lane in flight at a time (r * d is a multiple of 512)
    for (int e0 = lane; e0 < r * d; e0 += 512) {
        float bb[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + 64 * u;
            bb[u] = bk[(size_t)(e / d) * bstride + e % d];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) s_bk[e0 + 64 * u] = bb[u];
    }
    __syncthreads();
    if (lane < r) {
        float t = 0.f;
        for (int c = 0; c < d; ++c) t += s_q[c] * s_bk[lane * d + c];
        s_qb[lane] = t;
    }
    __syncthreads();

    float m = -INFINITY, l = 0.f;
    float o0 = 0.f, o1 = 0.f, olr = 0.f;
    const int n_vis = pos + 1;
    for (int c0 = 0; c0 < n_vis; c0 += 64) {
        const int j = c0 + lane;
        float s = -INFINITY;
        if (j < n_vis) {
            float dot = 0.f;
            if (!rope) {
                // loads requested eight (four) at a time; FMAs in dimension order
                for (int c = 0; c < d; c += 8) {  // d is a multiple of 8
                    float kv[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) kv[u] = acc.K(j, c + u);
#pragma unroll
                    for (int u = 0; u < 8; ++u) dot += s_q[c + u] * kv[u];
                }
                for (int t = 0; t < r; t += 4) {  // r is a multiple of 4
                    float lv[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) lv[u] = acc.LK(j, t + u);
#pragma unroll
                    for (int u = 0; u < 4; ++u) dot += s_qb[t + u] * lv[u];
                }
            } else {
                // rebuild the adapter key at head dimension, rotate it, add to K_base
                const int half = d / 2;
                for (int i = 0; i < half; ++i) {
                    float x1 = 0.f, x2 = 0.f;
                    for (int t = 0; t < r; ++t) {
                        const float lkv = acc.LK(j, t);
                        x1 += lkv * s_bk[t * d + i];
                        x2 += lkv * s_bk[t * d + i + half];
                    }
                    const float cs = a.rope_cos[(size_t)j * half + i];
                    const float sn = a.rope_sin[(size_t)j * half + i];
                    dot += s_q[i] * (acc.K(j, i) + x1 * cs - x2 * sn);
                    dot += s_q[i + half] * (acc.K(j, i + half) + x2 * cs + x1 * sn);
                }
            }
            s = dot * a.scale;
        }
        const float cm = wave_max(s);
        const float m_new = fmaxf(m, cm);
        const float alpha = expf(m - m_new);
        const float p = (j < n_vis) ? expf(s - m_new) : 0.f;
        l = l * alpha + wave_sum(p);
        m = m_new;
        s_p[lane] = p;
        __syncthreads();
        const int nk = min(64, n_vis - c0);
        o0 *= alpha;
        o1 *= alpha;
        olr *= alpha;
        // eight keys' values are requested before their FMAs (one memory round
        // trip per eight keys); the FMAs keep key order, so the result is the
        // same as key by key
        for (int jj0 = 0; jj0 < nk; jj0 += 8) {
            float v0[8], v1[8], vl[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = c0 + min(jj0 + u, nk - 1);
                v0[u] = lane < d ? acc.V(j, lane) : 0.f;
                v1[u] = lane + 64 < d ? acc.V(j, lane + 64) : 0.f;
                vl[u] = lane < r ? acc.LV(j, lane) : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (jj0 + u < nk) {
                    const float pj = s_p[jj0 + u];
                    if (lane < d) o0 += pj * v0[u];
                    if (lane + 64 < d) o1 += pj * v1[u];
                    if (lane < r) olr += pj * vl[u];
                }
            }
        }
        __syncthreads();
    }
    if (lane < r) s_olr[lane] = olr;
    __syncthreads();
    const float inv = 1.0f / l;
    for (int c = lane, k = 0; c < d; c += 64, ++k) {
        float o = (k == 0) ? o0 : o1;
        for (int t0 = 0; t0 < r; t0 += 4) {  // four B_v rows in flight; FMAs in rank order
            float bb[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) bb[u] = bv[(size_t)(t0 + u) * bstride + c];
#pragma unroll
            for (int u = 0; u < 4; ++u) o += s_olr[t0 + u] * bb[u];
        }
        orow[c] = o * inv;
    }
}

// grid: n_req * H_q blocks of 64 threads
__global__ __launch_bounds__(64) void lra_decode_f32_kernel(F32K a) {
    const int row = blockIdx.x;
    const int req = row / a.h_q, hq = row % a.h_q;
    const int g = a.h_q / a.h_kv;
    const int h = hq / g;
    // context of this request: largest c with ctx_req_start[c] <= req (binary search)
    int lo = 0, hi = a.n_ctx - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (a.ctx_req_start[mid] <= req) lo = mid; else hi = mid - 1;
    }
    const int ctx = lo;
    // clamped to max_ctx_len as well: the RoPE tables hold that many rows
    const int len = min(min(a.ctx_len[ctx], a.max_blocks * PAGE), a.max_len);
    float* orow = a.out + ((size_t)req * a.h_q + hq) * a.d;
    if (len <= 0) {
        for (int c = threadIdx.x; c < a.d; c += 64) orow[c] = 0.f;
        return;
    }
    int agent = min(max(a.req_agent[req], 0), a.n_agents - 1);
    Paged acc{&a, a.block_table + (size_t)ctx * a.max_blocks, h, (size_t)agent * a.lr_stride};
    row_attend(a, acc, a.q + ((size_t)req * a.h_q + hq) * a.d, agent, h, len - 1, orow,
               a.rope_cos != nullptr);
}

// grid: n_req * q_len * H_q blocks of 64 threads
__global__ __launch_bounds__(64) void lra_prefill_f32_kernel(F32K a) {
    const int row = blockIdx.x;
    const int hq = row % a.h_q;
    const int i = (row / a.h_q) % a.q_len;
    const int req = row / (a.h_q * a.q_len);
    const int g = a.h_q / a.h_kv;
    const int h = hq / g;
    const int agent = min(max(a.req_agent[req], 0), a.n_agents - 1);
    Contig acc{&a, h, (size_t)agent * a.lr_stride};
    const size_t off = (((size_t)req * a.q_len + i) * a.h_q + hq) * a.d;
    row_attend(a, acc, a.q + off, agent, h, a.kv_len - a.q_len + i, a.out + off, a.rope_cos != nullptr);
}

F32K common(const lra::DecodeArgs& d) {
    F32K k{};
    k.q = (const float*)d.q;
    k.ctx_req_start = d.ctx_req_start;
    k.req_agent = d.req_agent;
    k.k = (const float*)d.k_pool;
    k.v = (const float*)d.v_pool;
    k.lk = (const float*)d.lk_pool;
    k.lv = (const float*)d.lv_pool;
    k.block_table = d.block_table;
    k.ctx_len = d.ctx_len;
    k.b_k = (const float*)d.b_k;
    k.b_v = (const float*)d.b_v;
    k.rope_cos = d.rope_cos;
    k.rope_sin = d.rope_sin;
    k.out = (float*)d.out;
    k.n_req = d.n_req;
    k.n_ctx = d.n_ctx;
    k.n_pages = d.n_pages;
    k.max_blocks = d.max_blocks;
    k.max_len = d.max_ctx_len;
    k.n_agents = d.n_agents;
    k.h_q = d.h_q;
    k.h_kv = d.h_kv;
    k.d = d.head_dim;
    k.r = d.rank;
    k.scale = d.scale;
    k.lr_stride = d.lr_stride;
    return k;
}

}  // namespace

namespace lra {

lra_status launch_decode_f32(const DecodeArgs& d, hipStream_t s) {
    F32K k = common(d);
    if (d.n_req == 0) return LRA_OK;
    hipLaunchKernelGGL(lra_decode_f32_kernel, dim3(d.n_req * d.h_q), dim3(64), 0, s, k);
    return check_launch("lra_decode_f32_kernel");
}

lra_status launch_prefill_f32(const PrefillArgs& p, hipStream_t s) {
    F32K k{};
    k.q = (const float*)p.q;
    k.req_agent = p.req_agent;
    k.k = (const float*)p.k_base;
    k.v = (const float*)p.v_base;
    k.lk = (const float*)p.l_k;
    k.lv = (const float*)p.l_v;
    k.b_k = (const float*)p.b_k;
    k.b_v = (const float*)p.b_v;
    k.rope_cos = p.rope_cos;
    k.rope_sin = p.rope_sin;
    k.out = (float*)p.out;
    k.n_req = p.n_req;
    k.n_agents = p.n_agents;
    k.q_len = p.q_len;
    k.kv_len = p.kv_len;
    k.h_q = p.h_q;
    k.h_kv = p.h_kv;
    k.d = p.head_dim;
    k.r = p.rank;
    k.scale = p.scale;
    k.lr_stride = p.lr_stride;
    const long long blocks = (long long)p.n_req * p.q_len * p.h_q;
    if (blocks == 0) return LRA_OK;
    if (blocks > 0x7fffffffLL) {
        set_error("prefill f32: %lld query rows exceed the grid limit", blocks);
        return LRA_ERR_BAD_SHAPE;
    }
    hipLaunchKernelGGL(lra_prefill_f32_kernel, dim3((unsigned)blocks), dim3(64), 0, s, k);
    return check_launch("lra_prefill_f32_kernel");
}

}  // namespace lra
