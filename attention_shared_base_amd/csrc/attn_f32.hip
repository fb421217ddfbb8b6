// fp32 Flash-LoRA-Attention (decode and prefill), one workgroup of four
// wavefronts per query row.
//
// Serves dtype == LRA_F32: full fp32 arithmetic (no bf16 rounding anywhere),
// for small problems where latency, not bandwidth, dominates.  Same method as
// the bf16 kernels (LRAgent, arXiv 2602.01053v2, §3 and App. B): scores from
// q . k_base_j plus the pre-projected query against the shared rank-r row
// l_k_j (or, with RoPE, against the rebuilt key k_base_j + rot(l_k_j B_k^(h)),
// App. D.1, in decode and prefill alike), online softmax, value accumulation
// at head dimension for V_base and at rank r for L_v, and one B_v
// post-multiplication.
//
// Latency layout: a row's keys are dealt to the four wavefronts in 64-key
// chunks (wavefront w takes chunks w, w + 4, ...).  A wavefront requests a
// whole chunk's key rows at once (lane = key); its value columns (lane =
// column) go with them at head dim 64, and after the scores in two batches of
// 32 keys at 128; the next chunk's page ids are requested while a chunk runs.
// Each wavefront keeps its own online-softmax state; the four states are
// merged in LDS in wavefront order (the same bits on every call), then B_v is
// applied once.
#include "lra_common.h"
#include "lra_internal.h"

namespace {

constexpr int PAGE = 16;
constexpr int NW = 4;   // wavefronts per row
constexpr int CH = 64;  // keys per chunk: one per lane

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

// Paged pools.  chunk_pages: lane i < 4 gets the page id of keys c0 + 16 i ..
// (blocks past the last visible key repeat its block, so the block table is
// read only within the context).  Element accessors take the key's page id.
template <int D>
struct Paged {
    const F32K* a;
    const int32_t* bt;
    int h;
    size_t lr_off;  // this request's LR cache
    __device__ int chunk_pages(int c0, int n_vis, int lane) const {
        const int blk = min((c0 >> 4) + (lane & 3), (n_vis - 1) >> 4);
        return min(max(bt[blk], 0), a->n_pages - 1);
    }
    // dims 4 qd .. 4 qd + 3 of key j: half of one 8-dim group of the page
    __device__ f32x4 k4(int p, int j, int qd) const {
        return *(const f32x4*)(a->k + ((((size_t)p * a->h_kv + h) * (D / 8) + qd / 2) * PAGE + j % PAGE) * 8 +
                               4 * (qd & 1));
    }
    __device__ float lk(int p, int j, int t) const {
        return a->lk[lr_off + ((size_t)p * PAGE + j % PAGE) * a->r + t];
    }
    __device__ float v(int p, int j, int c) const {
        return a->v[(((size_t)p * a->h_kv + h) * D + c) * PAGE + j % PAGE];
    }
    __device__ float lv(int p, int j, int t) const {
        return a->lv[lr_off + ((size_t)p * a->r + t) * PAGE + j % PAGE];
    }
};

template <int D>
struct Contig {
    const F32K* a;
    int h;
    size_t lr_off;  // this request's LR cache
    __device__ int chunk_pages(int, int, int) const { return 0; }
    __device__ f32x4 k4(int, int j, int qd) const {
        return *(const f32x4*)(a->k + ((size_t)h * a->kv_len + j) * D + 4 * qd);
    }
    __device__ float lk(int, int j, int t) const { return a->lk[lr_off + (size_t)j * a->r + t]; }
    __device__ float v(int, int j, int c) const { return a->v[((size_t)h * a->kv_len + j) * D + c]; }
    __device__ float lv(int, int j, int t) const { return a->lv[lr_off + (size_t)j * a->r + t]; }
};

LRA_DEV float lane_value(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// One query row: q (length D) at absolute position `pos`, sees keys 0..pos.
// Block of NW wavefronts; every thread of the block calls it.  pg0: lanes 0..3
// hold the page ids of the wavefront's first chunk (paged pools).
template <int D, int R, bool ROPE, typename Acc>
__device__ void row_attend(const F32K& a, const Acc& acc, const float* qrow, int agent, int h,
                           int pos, int pg0, float* orow) {
    constexpr int HALF = D / 2;
    constexpr int NC = D / 64;             // value columns per lane
    constexpr int NB = R * D / (64 * NW);  // B elements per thread
    // keys per value batch; at D = 64 a chunk's values fit in registers beside its
    // keys and are requested with them
    constexpr int VB = D == 64 ? CH : 32;
    constexpr bool V_WITH_K = D == 64;
    __shared__ float s_q[D];
    __shared__ f32x4 s_bk4[R * D / 4];   // B_k^(h): [rank][dim]
    __shared__ float s_bv[R * D];        // B_v^(h): [rank][dim]
    __shared__ float s_qb[R];
    __shared__ float s_m[NW], s_l[NW];
    __shared__ float s_o[NW][D];
    __shared__ float s_olr[NW][R];
    __shared__ float s_olr_all[R];
    float* s_bk = (float*)s_bk4;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t bstride = (size_t)a.h_kv * D;
    const float* bk = a.b_k + (size_t)agent * R * bstride + (size_t)h * D;
    const float* bv = a.b_v + (size_t)agent * R * bstride + (size_t)h * D;
    const int n_vis = pos + 1;

    // A chunk's operands in registers: lane = key for its L_k row and (without
    // RoPE) its K_base row; lane = column for values.  Indices are clamped to the
    // row's last key, so a wavefront past the row's end reads in bounds (unused).
    f32x4 kv[ROPE ? 1 : D / 4];
    float lkv[R];
    float vv[NC][VB], vl[VB];
    auto load_keys = [&](int c0, int pgc) {
        const int jc = min(c0 + lane, n_vis - 1);
        const int pj = __shfl(pgc, max(jc - c0, 0) >> 4);
#pragma unroll
        for (int t = 0; t < R; ++t) lkv[t] = acc.lk(pj, jc, t);
        if constexpr (!ROPE) {
#pragma unroll
            for (int qd = 0; qd < D / 4; ++qd) kv[qd] = acc.k4(pj, jc, qd);
        }
    };
    auto load_values = [&](int c0, int pgc, int h0) {
        const int nk = min(CH, n_vis - c0);
#pragma unroll
        for (int u = 0; u < VB; ++u) {
            const int ku = nk > 0 ? min(h0 + u, nk - 1) : n_vis - 1 - c0;  // no keys: the row's last
            const int pu = __builtin_amdgcn_readlane(pgc, max(ku, 0) >> 4);
#pragma unroll
            for (int k = 0; k < NC; ++k) vv[k][u] = acc.v(pu, c0 + ku, lane + 64 * k);
            vl[u] = lane < R ? acc.lv(pu, c0 + ku, lane) : 0.f;
        }
    };

    // q and B requested first, then the first chunk's operands (unconditionally, so
    // waiting for B does not wait for them): both are in flight together
    float kb[NB], vb[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const int e = tid + 64 * NW * u;  // e = t * D + c
        kb[u] = bk[(size_t)(e / D) * bstride + e % D];
        vb[u] = bv[(size_t)(e / D) * bstride + e % D];
    }
    const float qv = tid < D ? qrow[tid] : 0.f;
    int c0 = CH * wave;
    int pgc = pg0;
    load_keys(c0, pgc);
    if constexpr (V_WITH_K) load_values(c0, pgc, 0);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const int e = tid + 64 * NW * u;
        s_bk[e] = kb[u];
        s_bv[e] = vb[u];
    }
    if (tid < D) s_q[tid] = qv;
    __syncthreads();
    if constexpr (!ROPE) {
        if (tid < R) {  // qB = q . B_k^(h) row t, in dimension order
            float t = 0.f;
            for (int c = 0; c < D; ++c) t += s_q[c] * s_bk[tid * D + c];
            s_qb[tid] = t;
        }
        __syncthreads();
    }

    float m = -INFINITY, l = 0.f, olr = 0.f;
    float o[NC];
#pragma unroll
    for (int k = 0; k < NC; ++k) o[k] = 0.f;
    for (; c0 < n_vis; c0 += CH * NW) {
        const int c1 = c0 + CH * NW;  // this wavefront's next chunk: its page ids now
        const int pg1 = c1 < n_vis ? acc.chunk_pages(c1, n_vis, lane) : 0;
        // ---- scores: lane = key (keys past the row's last repeat it, masked)
        const int j = c0 + lane;
        float dot = 0.f;
        if constexpr (!ROPE) {
#pragma unroll
            for (int c = 0; c < D; ++c) dot += s_q[c] * kv[c / 4][c % 4];
#pragma unroll
            for (int t = 0; t < R; ++t) dot += s_qb[t] * lkv[t];
        } else {
            // the adapter key rebuilt at head dimension and rotated by the key's
            // angle (pairs (i, i + D/2)), added to K_base; BI pairs per batch, the
            // rank sum of each dimension in rank order
            const int jc = min(j, n_vis - 1);
            const int pj = __shfl(pgc, (jc - c0) >> 4);
            const float* cs_row = a.rope_cos + (size_t)jc * HALF;
            const float* sn_row = a.rope_sin + (size_t)jc * HALF;
            constexpr int BI = 16;
#pragma unroll 1
            for (int i0 = 0; i0 < HALF; i0 += BI) {
                f32x4 cs[BI / 4], sn[BI / 4], k1[BI / 4], k2[BI / 4];
#pragma unroll
                for (int qd = 0; qd < BI / 4; ++qd) {
                    cs[qd] = *(const f32x4*)(cs_row + i0 + 4 * qd);
                    sn[qd] = *(const f32x4*)(sn_row + i0 + 4 * qd);
                    k1[qd] = acc.k4(pj, jc, i0 / 4 + qd);
                    k2[qd] = acc.k4(pj, jc, (HALF + i0) / 4 + qd);
                }
                f32x4 x1[BI / 4], x2[BI / 4];
#pragma unroll
                for (int qd = 0; qd < BI / 4; ++qd) x1[qd] = x2[qd] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < R; ++t) {
#pragma unroll
                    for (int qd = 0; qd < BI / 4; ++qd) {
                        const f32x4 b1 = s_bk4[(t * D + i0) / 4 + qd];
                        const f32x4 b2 = s_bk4[(t * D + HALF + i0) / 4 + qd];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            x1[qd][e] += lkv[t] * b1[e];
                            x2[qd][e] += lkv[t] * b2[e];
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < BI; ++i) {
                    const int c = i0 + i;
                    const float u1 = x1[i / 4][i % 4], u2 = x2[i / 4][i % 4];
                    const float csv = cs[i / 4][i % 4], snv = sn[i / 4][i % 4];
                    dot += s_q[c] * (k1[i / 4][i % 4] + u1 * csv - u2 * snv);
                    dot += s_q[c + HALF] * (k2[i / 4][i % 4] + u2 * csv + u1 * snv);
                }
            }
        }
        // ---- online softmax over the chunk
        const float s = j < n_vis ? dot * a.scale : -INFINITY;
        const float m_new = fmaxf(m, wave_max(s));  // finite: lane 0 is a visible key
        const float alpha = expf(m - m_new);
        const float p = j < n_vis ? expf(s - m_new) : 0.f;
        l = l * alpha + wave_sum(p);
        m = m_new;
#pragma unroll
        for (int k = 0; k < NC; ++k) o[k] *= alpha;
        olr *= alpha;
        // ---- values: lane = column (and rank, lanes < R); FMAs in key order
        const int nk = min(CH, n_vis - c0);
#pragma unroll
        for (int h0 = 0; h0 < CH; h0 += VB) {
            if (h0 >= nk) break;
            if (!V_WITH_K || h0 > 0) load_values(c0, pgc, h0);
#pragma unroll
            for (int u = 0; u < VB; ++u) {
                if (h0 + u < nk) {
                    const float pu = lane_value(p, h0 + u);
#pragma unroll
                    for (int k = 0; k < NC; ++k) o[k] += pu * vv[k][u];
                    olr += pu * vl[u];
                }
            }
        }
        // ---- the next chunk's operands
        if (c1 < n_vis) {
            pgc = pg1;
            load_keys(c1, pgc);
            if constexpr (V_WITH_K) load_values(c1, pgc, 0);
        }
    }

    // ---- merge the wavefronts' states (a wavefront without keys has m = -inf)
    if (lane == 0) {
        s_m[wave] = m;
        s_l[wave] = l;
    }
#pragma unroll
    for (int k = 0; k < NC; ++k) s_o[wave][lane + 64 * k] = o[k];
    if (lane < R) s_olr[wave][lane] = olr;
    __syncthreads();
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, s_m[w]);
    float wt[NW], L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        wt[w] = s_m[w] == -INFINITY ? 0.f : expf(s_m[w] - mx);
        L += wt[w] * s_l[w];
    }
    if (tid < R) {
        float x = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) x += wt[w] * s_olr[w][tid];
        s_olr_all[tid] = x;
    }
    __syncthreads();
    if (tid < D) {
        float x = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) x += wt[w] * s_o[w][tid];
#pragma unroll
        for (int t = 0; t < R; ++t) x += s_olr_all[t] * s_bv[t * D + tid];  // rank order
        orow[tid] = x * (1.0f / L);
    }
}

// grid: n_req * H_q blocks of NW wavefronts
template <int D, int R, bool ROPE>
__global__ __launch_bounds__(64 * NW) void lra_decode_f32_kernel(F32K a) {
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
    const int32_t* bt = a.block_table + (size_t)ctx * a.max_blocks;
    // the page ids of the wavefront's first chunk and the agent, requested with the
    // context length: blocks are clamped to the table row, which leaves the page of
    // every key the row uses unchanged
    const int blk0 = 4 * (int)(threadIdx.x >> 6) + (int)(threadIdx.x & 3);
    const int pg0 = min(max(bt[min(blk0, a.max_blocks - 1)], 0), a.n_pages - 1);
    const int agent = min(max(a.req_agent[req], 0), a.n_agents - 1);
    // clamped to max_ctx_len as well: the RoPE tables hold that many rows
    const int len = min(min(a.ctx_len[ctx], a.max_blocks * PAGE), a.max_len);
    float* orow = a.out + ((size_t)req * a.h_q + hq) * D;
    if (len <= 0) {  // the whole block leaves: len is the row's
        if (threadIdx.x < D) orow[threadIdx.x] = 0.f;
        return;
    }
    Paged<D> acc{&a, bt, h, (size_t)agent * a.lr_stride};
    row_attend<D, R, ROPE>(a, acc, a.q + ((size_t)req * a.h_q + hq) * D, agent, h, len - 1, pg0, orow);
}

// grid: n_req * q_len * H_q blocks of NW wavefronts
template <int D, int R, bool ROPE>
__global__ __launch_bounds__(64 * NW) void lra_prefill_f32_kernel(F32K a) {
    const int row = blockIdx.x;
    const int hq = row % a.h_q;
    const int i = (row / a.h_q) % a.q_len;
    const int req = row / (a.h_q * a.q_len);
    const int g = a.h_q / a.h_kv;
    const int h = hq / g;
    const int agent = min(max(a.req_agent[req], 0), a.n_agents - 1);
    Contig<D> acc{&a, h, (size_t)agent * a.lr_stride};
    const size_t off = (((size_t)req * a.q_len + i) * a.h_q + hq) * D;
    row_attend<D, R, ROPE>(a, acc, a.q + off, agent, h, a.kv_len - a.q_len + i, 0, a.out + off);
}

// head dim, rank and RoPE as template arguments (validated by the caller)
#define LRA_F32_KERNEL_TABLE(KERNEL)                                                         \
    template <int D, int R>                                                                  \
    void launch_##KERNEL##_dr(const F32K& k, bool rope, unsigned blocks, hipStream_t s) {     \
        if (rope)                                                                            \
            hipLaunchKernelGGL((KERNEL<D, R, true>), dim3(blocks), dim3(64 * NW), 0, s, k);  \
        else                                                                                 \
            hipLaunchKernelGGL((KERNEL<D, R, false>), dim3(blocks), dim3(64 * NW), 0, s, k); \
    }                                                                                        \
    void launch_##KERNEL(const F32K& k, unsigned blocks, hipStream_t s) {                    \
        const bool rope = k.rope_cos != nullptr;                                             \
        const int sel = (k.d == 128 ? 4 : 0) + (k.r == 4 ? 0 : k.r == 8 ? 1 : k.r == 16 ? 2 : 3); \
        switch (sel) {                                                                       \
            case 0: return launch_##KERNEL##_dr<64, 4>(k, rope, blocks, s);                  \
            case 1: return launch_##KERNEL##_dr<64, 8>(k, rope, blocks, s);                  \
            case 2: return launch_##KERNEL##_dr<64, 16>(k, rope, blocks, s);                 \
            case 3: return launch_##KERNEL##_dr<64, 32>(k, rope, blocks, s);                 \
            case 4: return launch_##KERNEL##_dr<128, 4>(k, rope, blocks, s);                 \
            case 5: return launch_##KERNEL##_dr<128, 8>(k, rope, blocks, s);                 \
            case 6: return launch_##KERNEL##_dr<128, 16>(k, rope, blocks, s);                \
            default: return launch_##KERNEL##_dr<128, 32>(k, rope, blocks, s);               \
        }                                                                                    \
    }
LRA_F32_KERNEL_TABLE(lra_decode_f32_kernel)
LRA_F32_KERNEL_TABLE(lra_prefill_f32_kernel)
#undef LRA_F32_KERNEL_TABLE

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
    launch_lra_decode_f32_kernel(k, (unsigned)(d.n_req * d.h_q), s);
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
    launch_lra_prefill_f32_kernel(k, (unsigned)blocks, s);
    return check_launch("lra_prefill_f32_kernel");
}

}  // namespace lra
