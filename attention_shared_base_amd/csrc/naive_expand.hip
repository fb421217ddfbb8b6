// Materialise the adapter terms at head dimension in HBM: the naive
// reconstruction that Flash-LoRA-Attention avoids (LRAgent, arXiv
// 2602.01053v2, §3 "Flash-LoRA-Attention" and App. B: expanding V_lr B before
// attention costs O(L r d_out) per step and d_out-sized traffic).  It exists
// only as the measured baseline of that comparison; no entry point of the
// method calls it.
//
// For request i (context c, agent a) and every page b of c's block table:
//   K_out[page i*out_blocks + b] = K_base[page] + L_k[page] B_k^(a)   (all KV heads)
//   V_out[page i*out_blocks + b] = V_base[page] + L_v[page] B_v^(a)
// (L_k, L_v from agent a's pools when the LR caches are per agent).
// in the decode page layouts (K [H_kv][d/8][16][8], V [H_kv][d][16]), bf16
// rounded to nearest even.  Plain decode attention over these per-request pages
// (one context per request, B = 0) then computes the same attention as the
// method, at N times the K/V bytes for N agents on a context.  The contiguous
// form below does the same for the prefill baseline (with the rotation of the
// adapter key when RoPE tables are given), followed by the prefill kernel's
// plain-attention mode over the per-request caches.
#include "lra_common.h"
#include "lra_internal.h"

namespace {

constexpr int PAGE = 16;
constexpr int PAGES_PER_WG = 16;

struct ExpandK {
    const int32_t* ctx_req_start;
    const int32_t* req_agent;
    const bf16* k_pool;
    const bf16* v_pool;
    const bf16* lk_pool;
    const bf16* lv_pool;
    const int32_t* block_table;
    const int32_t* ctx_len;
    const bf16* b_k;
    const bf16* b_v;
    bf16* k_out;
    bf16* v_out;
    int64_t lr_stride;  // per-agent LR pools: elements between agents' pools (0: shared)
    int32_t n_req, n_ctx, n_pages, max_blocks, n_agents, h_kv, out_blocks, groups;
};

// grid: n_req * H_kv * groups workgroups of 256 threads; workgroup = (request,
// KV head, PAGES_PER_WG consecutive blocks).  Per page, thread tid owns one K
// chunk (8 dims of one token) and one V chunk (8 tokens of one dim) when D = 128.
template <int D, int R>
__global__ __launch_bounds__(256) void lra_naive_expand_kernel(ExpandK a) {
    __shared__ float s_bk[R][D];
    __shared__ float s_bv[R][D];
    __shared__ float s_lk[PAGE][R];
    __shared__ float s_lv[R][PAGE];
    const int tid = threadIdx.x;
    const int grp = blockIdx.x % a.groups;
    const int h = (blockIdx.x / a.groups) % a.h_kv;
    const int req = blockIdx.x / (a.groups * a.h_kv);
    // context of the request: largest c with ctx_req_start[c] <= req
    int lo = 0, hi = a.n_ctx - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (a.ctx_req_start[mid] <= req) lo = mid; else hi = mid - 1;
    }
    const int ctx = lo;
    const int len = min(a.ctx_len[ctx], a.max_blocks * PAGE);
    const int n_blk = min((len + PAGE - 1) / PAGE, a.out_blocks);
    const int b0 = grp * PAGES_PER_WG;
    if (b0 >= n_blk) return;
    const int agent = min(max(a.req_agent[req], 0), a.n_agents - 1);
    const size_t bcols = (size_t)a.h_kv * D;
    for (int e = tid; e < R * D; e += 256) {
        const int rk = e / D, c = e % D;
        s_bk[rk][c] = (float)a.b_k[((size_t)agent * R + rk) * bcols + (size_t)h * D + c];
        s_bv[rk][c] = (float)a.b_v[((size_t)agent * R + rk) * bcols + (size_t)h * D + c];
    }
    const size_t kv_page = (size_t)a.h_kv * D * PAGE;
    const int* bt = a.block_table + (size_t)ctx * a.max_blocks;
    for (int b = b0; b < min(b0 + PAGES_PER_WG, n_blk); ++b) {
        const int pid = min(max(bt[b], 0), a.n_pages - 1);
        __syncthreads();  // previous page's L rows no longer read; B staged
        for (int e = tid; e < PAGE * R; e += 256) {
            s_lk[e / R][e % R] = (float)a.lk_pool[(size_t)agent * a.lr_stride + (size_t)pid * PAGE * R + e];
            s_lv[e / PAGE][e % PAGE] = (float)a.lv_pool[(size_t)agent * a.lr_stride + (size_t)pid * PAGE * R + e];
        }
        __syncthreads();
        const bf16* kin = a.k_pool + (size_t)pid * kv_page + (size_t)h * D * PAGE;
        const bf16* vin = a.v_pool + (size_t)pid * kv_page + (size_t)h * D * PAGE;
        const size_t opage = (size_t)req * a.out_blocks + b;
        bf16* kout = a.k_out + opage * kv_page + (size_t)h * D * PAGE;
        bf16* vout = a.v_out + opage * kv_page + (size_t)h * D * PAGE;
        // K chunks: (dim group dg, token t) -> 8 dims, layout [d/8][16][8]
        for (int ch = tid; ch < D / 8 * PAGE; ch += 256) {
            const int dg = ch / PAGE, t = ch % PAGE;
            const bf16x8 kb = *(const bf16x8*)(kin + ch * 8);
            float acc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = (float)kb[e];
#pragma unroll
            for (int rk = 0; rk < R; ++rk) {
                const float l = s_lk[t][rk];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += l * s_bk[rk][8 * dg + e];
            }
            bf16x8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = (bf16)acc[e];
            *(bf16x8*)(kout + ch * 8) = o;
        }
        // V chunks: (dim c, token half th) -> 8 tokens, layout [d][16]
        for (int ch = tid; ch < D * 2; ch += 256) {
            const int c = ch / 2, t0 = 8 * (ch % 2);
            const bf16x8 vb = *(const bf16x8*)(vin + ch * 8);
            float acc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = (float)vb[e];
#pragma unroll
            for (int rk = 0; rk < R; ++rk) {
                const float w = s_bv[rk][c];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += s_lv[rk][t0 + e] * w;
            }
            bf16x8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = (bf16)acc[e];
            *(bf16x8*)(vout + ch * 8) = o;
        }
    }
}

// Contiguous form for the prefill baseline: for request i (agent a = req_agent[i])
// and KV head h, rows j of a block of EX_KEYS keys:
//   K_out[i][h][j] = K_base[h][j] + rot_j(L_k[j] B_k^(a,h)),  V_out[i][h][j] = V_base[h][j] + L_v[j] B_v^(a,h)
// (rot_j: rotate-half by the angles of RoPE row j when tables are given), bf16
// rounded to nearest even, layout [n_req][H_kv][kv_len][D].  Thread t takes key
// t / 4 of the block and a quarter of its dims: D/8 rotation pairs (i, i + D/2)
// for K, D/4 consecutive dims for V.
constexpr int EX_KEYS = 64;

struct ExpandContigK {
    const int32_t* req_agent;
    const bf16* k_base;
    const bf16* v_base;
    const bf16* l_k;
    const bf16* l_v;
    const bf16* b_k;
    const bf16* b_v;
    const float* rope_cos;  // NULL: no rotation
    const float* rope_sin;
    bf16* k_out;
    bf16* v_out;
    int64_t lr_stride;  // per-agent LR caches: elements between agents' caches (0: shared)
    int32_t kv_len, n_agents, h_kv, n_blk;
};

template <int D, int R>
__global__ __launch_bounds__(256) void lra_naive_expand_contig_kernel(ExpandContigK a) {
    __shared__ float s_bk[R][D];
    __shared__ float s_bv[R][D];
    const int tid = threadIdx.x;
    const int blk = blockIdx.x % a.n_blk;
    const int h = (blockIdx.x / a.n_blk) % a.h_kv;
    const int req = blockIdx.x / (a.n_blk * a.h_kv);
    const int agent = min(max(a.req_agent[req], 0), a.n_agents - 1);
    const size_t bcols = (size_t)a.h_kv * D;
    for (int e = tid; e < R * D; e += 256) {
        const int rk = e / D, c = e % D;
        s_bk[rk][c] = (float)a.b_k[((size_t)agent * R + rk) * bcols + (size_t)h * D + c];
        s_bv[rk][c] = (float)a.b_v[((size_t)agent * R + rk) * bcols + (size_t)h * D + c];
    }
    __syncthreads();
    const int j = blk * EX_KEYS + tid / 4;
    if (j >= a.kv_len) return;
    const int part = tid % 4;
    float lk[R], lv[R];
    const size_t lr_off = (size_t)agent * a.lr_stride + (size_t)j * R;
#pragma unroll
    for (int rk = 0; rk < R; ++rk) {
        lk[rk] = (float)a.l_k[lr_off + rk];
        lv[rk] = (float)a.l_v[lr_off + rk];
    }
    const size_t row = ((size_t)h * a.kv_len + j) * D;
    const size_t orow = (((size_t)req * a.h_kv + h) * a.kv_len + j) * D;
    // K: pairs (i, i + D/2) for i in [part * D/8, (part + 1) * D/8)
    constexpr int NP = D / 8;
#pragma unroll
    for (int i0 = 0; i0 < NP; i0 += 8) {
        const int i = part * NP + i0;
        const bf16x8 k1 = *(const bf16x8*)(a.k_base + row + i);
        const bf16x8 k2 = *(const bf16x8*)(a.k_base + row + i + D / 2);
        float x1[8], x2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x1[e] = 0.f;
            x2[e] = 0.f;
        }
#pragma unroll
        for (int rk = 0; rk < R; ++rk)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                x1[e] += lk[rk] * s_bk[rk][i + e];
                x2[e] += lk[rk] * s_bk[rk][i + e + D / 2];
            }
        if (a.rope_cos != nullptr) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float c = a.rope_cos[(size_t)j * (D / 2) + i + e];
                const float sn = a.rope_sin[(size_t)j * (D / 2) + i + e];
                const float y1 = x1[e] * c - x2[e] * sn;
                const float y2 = x2[e] * c + x1[e] * sn;
                x1[e] = y1;
                x2[e] = y2;
            }
        }
        bf16x8 o1, o2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            o1[e] = (bf16)((float)k1[e] + x1[e]);
            o2[e] = (bf16)((float)k2[e] + x2[e]);
        }
        *(bf16x8*)(a.k_out + orow + i) = o1;
        *(bf16x8*)(a.k_out + orow + i + D / 2) = o2;
    }
    // V: dims [part * D/4, (part + 1) * D/4)
#pragma unroll
    for (int c0 = 0; c0 < D / 4; c0 += 8) {
        const int c = part * (D / 4) + c0;
        const bf16x8 vb = *(const bf16x8*)(a.v_base + row + c);
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float acc = (float)vb[e];
#pragma unroll
            for (int rk = 0; rk < R; ++rk) acc += lv[rk] * s_bv[rk][c + e];
            o[e] = (bf16)acc;
        }
        *(bf16x8*)(a.v_out + orow + c) = o;
    }
}

template <int D, int R>
lra_status launch_contig_t(const lra::ExpandContigArgs& p, hipStream_t s) {
    ExpandContigK k;
    k.req_agent = p.req_agent;
    k.k_base = (const bf16*)p.k_base;
    k.v_base = (const bf16*)p.v_base;
    k.l_k = (const bf16*)p.l_k;
    k.l_v = (const bf16*)p.l_v;
    k.b_k = (const bf16*)p.b_k;
    k.b_v = (const bf16*)p.b_v;
    k.rope_cos = p.rope_cos;
    k.rope_sin = p.rope_sin;
    k.k_out = (bf16*)p.k_out;
    k.v_out = (bf16*)p.v_out;
    k.lr_stride = p.lr_stride;
    k.kv_len = p.kv_len;
    k.n_agents = p.n_agents;
    k.h_kv = p.h_kv;
    k.n_blk = (p.kv_len + EX_KEYS - 1) / EX_KEYS;
    const long long grid = (long long)p.n_req * p.h_kv * k.n_blk;
    if (grid > 0x7fffffffLL) {
        lra::set_error("naive expand: grid of %lld workgroups too large", grid);
        return LRA_ERR_BAD_SHAPE;
    }
    hipLaunchKernelGGL((lra_naive_expand_contig_kernel<D, R>), dim3((unsigned)grid), dim3(256), 0, s, k);
    return lra::check_launch("lra_naive_expand_contig_kernel");
}

template <int D, int R>
lra_status launch_t(const lra::ExpandArgs& p, hipStream_t s) {
    ExpandK k;
    k.ctx_req_start = p.ctx_req_start;
    k.req_agent = p.req_agent;
    k.k_pool = (const bf16*)p.k_pool;
    k.v_pool = (const bf16*)p.v_pool;
    k.lk_pool = (const bf16*)p.lk_pool;
    k.lv_pool = (const bf16*)p.lv_pool;
    k.block_table = p.block_table;
    k.ctx_len = p.ctx_len;
    k.b_k = (const bf16*)p.b_k;
    k.b_v = (const bf16*)p.b_v;
    k.k_out = (bf16*)p.k_out;
    k.v_out = (bf16*)p.v_out;
    k.n_req = p.n_req;
    k.n_ctx = p.n_ctx;
    k.n_pages = p.n_pages;
    k.max_blocks = p.max_blocks;
    k.n_agents = p.n_agents;
    k.h_kv = p.h_kv;
    k.out_blocks = p.out_blocks;
    k.lr_stride = p.lr_stride;
    k.groups = (p.out_blocks + PAGES_PER_WG - 1) / PAGES_PER_WG;
    const long long grid = (long long)p.n_req * p.h_kv * k.groups;
    if (grid > 0x7fffffffLL) {
        lra::set_error("naive expand: grid of %lld workgroups too large", grid);
        return LRA_ERR_BAD_SHAPE;
    }
    hipLaunchKernelGGL((lra_naive_expand_kernel<D, R>), dim3((unsigned)grid), dim3(256), 0, s, k);
    return lra::check_launch("lra_naive_expand_kernel");
}

}  // namespace

namespace lra {

lra_status launch_naive_expand_bf16(const ExpandArgs& p, hipStream_t s) {
#define LRA_CASE(D_, R_) \
    if (p.head_dim == D_ && p.rank == R_) return launch_t<D_, R_>(p, s);
    LRA_CASE(128, 16)
    LRA_CASE(128, 32)
    LRA_CASE(128, 8)
    LRA_CASE(64, 16)
    LRA_CASE(64, 32)
    LRA_CASE(64, 8)
    LRA_CASE(128, 4)
    LRA_CASE(64, 4)
#undef LRA_CASE
    set_error("naive expand: unsupported head_dim %d / rank %d", p.head_dim, p.rank);
    return LRA_ERR_UNSUPPORTED;
}

lra_status launch_naive_expand_contig_bf16(const ExpandContigArgs& p, hipStream_t s) {
#define LRA_CASE(D_, R_) \
    if (p.head_dim == D_ && p.rank == R_) return launch_contig_t<D_, R_>(p, s);
    LRA_CASE(128, 16)
    LRA_CASE(128, 32)
    LRA_CASE(128, 8)
    LRA_CASE(64, 16)
    LRA_CASE(64, 32)
    LRA_CASE(64, 8)
    LRA_CASE(128, 4)
    LRA_CASE(64, 4)
#undef LRA_CASE
    set_error("naive expand: unsupported head_dim %d / rank %d", p.head_dim, p.rank);
    return LRA_ERR_UNSUPPORTED;
}

}  // namespace lra
