// Paged Flash-LoRA-Attention decode, bf16 storage / fp32 accumulation, gfx950.
//
// What is computed (LRAgent, arXiv 2602.01053v2, §3 and App. B): for every
// query row (request, query head hq, KV head h = hq / g)
//
//     s_j = (q . k_base_j + (q B_k^(h)T) . l_k_j) * scale
//     O   = (sum_j p_j v_base_j + (sum_j p_j l_v_j) B_v^(h)) / sum_j p_j
//
// with p_j = exp(s_j - m) under an online (streaming) maximum m.  The low-rank
// terms stay rank r through the whole pass: the key side is the pre-projected
// query qB = q B_k^(h)T (computed once per workgroup) against the shared
// l_k rows, the value side accumulates P L_v at rank r, and B_v^(h) is applied
// once per row in the epilogue.
//
// Decomposition.  A work unit is (context, row group, KV head).  A row group
// packs up to 16 query rows = (requests of one context) x (g query heads of
// the KV head), so every K/V page of a context is read once per KV head for
// all agents and all heads of the group (GQA + cross-agent sharing).  One
// workgroup (4 wavefronts) handles one chunk of a unit's tokens; each
// wavefront streams 32 tokens (two 16-token pages) per step with its own
// online-softmax state, and the four are merged through LDS.  When a unit has
// several chunks, partial (m, l, O_base[d], O_lr[r]) rows go to the workspace
// and the last workgroup to finish the unit merges them (log-sum-exp) and
// applies B_v — never a [tokens, d] expansion of the adapter term.
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16; 16 tokens x 16 rows per tile):
//   S^T[token][row] = K_tile[token][dims] . Qt[dims][row]      (A = keys)
//   S^T            += L_k[token][ranks] . qB^T[ranks][row]      (rank r, k padded to 32)
//   O^T[dim][row]  += V^T[dim][token] . P^T[token][row]         (A = values)
//   O_lr^T[rank][row] += L_v^T[rank][token] . P^T[token][row]
// The S^T accumulator layout (lane = row l%16, tokens 4*(l/16)+v of each page)
// is exactly the P^T operand layout the value MFMAs need, so P never leaves
// registers.  The page layouts of the boundary are chosen so every operand is
// one direct, coalesced global load: K pages [d/8][16][8], V pages dim-major
// [d][16], L_k [16][r], L_v rank-major [r][16].  No LDS in the streaming loop.
#include "lra_common.h"
#include "lra_internal.h"

namespace {

constexpr int PAGE = 16;
constexpr int ROWS = 16;
constexpr int WAVES = 4;
constexpr int KEYS_PER_STEP = 32;  // two pages per wavefront step

struct DecodeK {
    const bf16* q;
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
    bf16* out;
    int32_t* ws_count;
    float* ws_part;
    int32_t n_ctx, n_pages, max_blocks, n_agents;
    int32_t h_q, h_kv, g, rpg, n_rg, n_split, chunk;
    float scale_log2;
};

// The rank-r score term uses the same v_mfma_f32_16x16x32_bf16 as the base
// term it accumulates onto.  Every accumulator chain in this file stays on one
// MFMA shape: a 16x16x32 result fed straight into a dependent 16x16x16 on the
// same accumulator lost the first MFMA's contribution in the low accumulator
// elements on gfx950, so r <= 16 is zero-padded to k = 32 instead (slots 0-3
// of each k-group carry ranks 4*q4 + v, slots 4-7 carry ranks 16 + 4*q4 + v
// or zeros).

template <int D, int R>
struct Step {
    static constexpr int NJ = D / 32;          // score MFMAs (dims) per page
    static constexpr int NDT = D / 16;         // value tiles (dims)
    static constexpr int NRT = (R + 15) / 16;  // value tiles (ranks)
    bf16x8 k[2][NJ];
    bf16x8 lk[2];
    bf16x4 v[2][NDT];
    bf16x4 lv[2][NRT];
};

template <int D, int R>
__global__ __launch_bounds__(256) void lra_decode_bf16_kernel(DecodeK a) {
    constexpr int NJ = Step<D, R>::NJ;
    constexpr int NDT = Step<D, R>::NDT;
    constexpr int NRT = Step<D, R>::NRT;
    constexpr int DR = D + R;
    constexpr int SP = DR + 1;  // LDS row pitch (odd: no bank aliasing across rows)

    __shared__ float sm_o[WAVES][ROWS][SP];
    __shared__ float sm_m[WAVES][ROWS];
    __shared__ float sm_l[WAVES][ROWS];
    __shared__ float sm_M[ROWS];
    __shared__ float sm_L[ROWS];
    __shared__ int sm_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n16 = lane & 15;  // row (S^T / O^T column) of this lane
    const int q4 = lane >> 4;   // k-group of this lane

    // XCD-aware placement: workgroup b runs on XCD b % 8; remap so that the
    // KV heads of one (context, chunk) — which share its L_k/L_v pages — are
    // consecutive on one XCD and hit the same L2.
    const int nb = gridDim.x;
    const int b = blockIdx.x;
    const int bp = (b & 7) * (nb >> 3) + (b >> 3);
    const int h = bp % a.h_kv;
    int rest = bp / a.h_kv;
    const int split = rest % a.n_split;
    rest /= a.n_split;
    const int rg = rest % a.n_rg;
    const int ctx = rest / a.n_rg;
    if (ctx >= a.n_ctx) return;
    const int unit = (ctx * a.n_rg + rg) * a.h_kv + h;

    const int rs0 = a.ctx_req_start[ctx];
    const int rs1 = a.ctx_req_start[ctx + 1];
    const int req0 = rs0 + rg * a.rpg;
    const int nreq = min(a.rpg, rs1 - req0);
    if (nreq <= 0) return;
    const int g = a.g;
    const int nrows = nreq * g;
    const int len = min(a.ctx_len[ctx], a.max_blocks * PAGE);

    if (len <= 0) {  // empty context: defined as zero output
        if (split == 0) {
            for (int e = tid; e < nrows * D; e += blockDim.x) {
                const int n = e / D, c = e % D;
                a.out[((size_t)(req0 + n / g) * a.h_q + h * g + n % g) * D + c] = (bf16)0.0f;
            }
        }
        return;
    }
    const int n_active = (len + a.chunk - 1) / a.chunk;
    if (split >= n_active) return;
    const int kbeg = split * a.chunk;
    const int kend = min(len, kbeg + a.chunk);

    // ---- query operand (B of the score MFMA): lane holds dims 32j+8*q4.. of row n16
    const bool row_ok = n16 < nrows;
    bf16x8 qf[NJ];
    {
        const bf16* qp = a.q + ((size_t)(req0 + n16 / g) * a.h_q + h * g + n16 % g) * D + 8 * q4;
#pragma unroll
        for (int j = 0; j < NJ; ++j) qf[j] = row_ok ? ldg((const bf16x8*)(qp + 32 * j)) : zero8();
    }

    // ---- pre-projection qB = q B_k^(h)T, one MFMA tile per request of the group.
    // C lane layout: rank 16*rt + 4*q4 + v of row n16 — already the B operand
    // layout of the rank-r score MFMA.
    f32x4 qbacc[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) qbacc[rt] = zf4();
    for (int s = 0; s < nreq; ++s) {
        int agent = a.req_agent[req0 + s];
        agent = min(max(agent, 0), a.n_agents - 1);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const int rank = 16 * rt + n16;
            const bf16* bp_ = a.b_k + ((size_t)agent * R + rank) * ((size_t)a.h_kv * D) +
                              (size_t)h * D + 8 * q4;
            f32x4 c = zf4();
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                c = mfma16x16x32(rank < R ? ldg((const bf16x8*)(bp_ + 32 * j)) : zero8(), qf[j], c);
            if (n16 / g == s) qbacc[rt] = c;
        }
    }
    bf16x8 qb;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        qb[v] = (bf16)qbacc[0][v];
        qb[4 + v] = (R == 32) ? (bf16)qbacc[NRT - 1][v] : (bf16)0.0f;
    }

    // ---- streaming loop
    const int* bt = a.block_table + (size_t)ctx * a.max_blocks;
    const int n_steps = (kend - kbeg + KEYS_PER_STEP - 1) / KEYS_PER_STEP;
    const size_t kv_page = (size_t)a.h_kv * D * PAGE;  // elements per page (all heads)
    const bf16* kbase = a.k_pool + (size_t)h * D * PAGE;
    const bf16* vbase = a.v_pool + (size_t)h * D * PAGE;

    auto load = [&](Step<D, R>& T, int st) {
        const int key0 = kbeg + st * KEYS_PER_STEP;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int pg = (key0 >> 4) + t;
            const bool live = pg * PAGE < kend;
            int pid = live ? bt[pg] : 0;
            pid = min(max(pid, 0), a.n_pages - 1);
            const bf16* kp = kbase + (size_t)pid * kv_page;
            const bf16* vp = vbase + (size_t)pid * kv_page;
            const bf16* lkp = a.lk_pool + (size_t)pid * PAGE * R;
            const bf16* lvp = a.lv_pool + (size_t)pid * PAGE * R;
            if (live) {
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    T.k[t][j] = ldg_stream((const bf16x8*)(kp + ((4 * j + q4) * PAGE + n16) * 8));
                if constexpr (R == 32) {
                    const bf16x4 lo = ldg((const bf16x4*)(lkp + n16 * R + 4 * q4));
                    const bf16x4 hi = ldg((const bf16x4*)(lkp + n16 * R + 16 + 4 * q4));
                    T.lk[t] = cat4(lo, hi);
                } else if constexpr (R == 16) {
                    T.lk[t] = cat4(ldg((const bf16x4*)(lkp + n16 * R + 4 * q4)), zero4());
                } else {
                    T.lk[t] = cat4(q4 < 2 ? ldg((const bf16x4*)(lkp + n16 * R + 4 * q4)) : zero4(),
                                   zero4());
                }
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    T.v[t][dt] = ldg_stream((const bf16x4*)(vp + (16 * dt + n16) * PAGE + 4 * q4));
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) {
                    const int rank = 16 * rt + n16;
                    T.lv[t][rt] = rank < R ? ldg((const bf16x4*)(lvp + rank * PAGE + 4 * q4)) : zero4();
                }
            } else {
#pragma unroll
                for (int j = 0; j < NJ; ++j) T.k[t][j] = zero8();
                T.lk[t] = zero8();
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) T.v[t][dt] = zero4();
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) T.lv[t][rt] = zero4();
            }
        }
    };

    float m_run = -INFINITY;
    float l_run = 0.f;
    f32x4 acc[NDT];
    f32x4 acc_lr[NRT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = zf4();
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) acc_lr[rt] = zf4();
    const float sl2 = a.scale_log2;

    auto compute = [&](Step<D, R>& T, int st) {
        const int key0 = kbeg + st * KEYS_PER_STEP;
        f32x4 s[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            s[t] = zf4();
#pragma unroll
            for (int j = 0; j < NJ; ++j) s[t] = mfma16x16x32(T.k[t][j], qf[j], s[t]);
            s[t] = mfma16x16x32(T.lk[t], qb, s[t]);
        }
        const bool tail = key0 + KEYS_PER_STEP > kend;
        float x[8];
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float val = s[t][v] * sl2;
                if (tail && key0 + 16 * t + 4 * q4 + v >= kend) val = -INFINITY;
                x[4 * t + v] = val;
                mx = fmaxf(mx, val);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);  // finite: every step holds a live token
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        float ps = 0.f;
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = fast_exp2(x[i] - m_new);
            ps += p;
            pb[i] = (bf16)p;
        }
        l_run = l_run * alpha + ps;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) acc_lr[rt] *= alpha;
        if (tail) {
            // Tokens past the chunk end may hold anything (even NaN bits in
            // unused page slots): zero their values so 0 * NaN cannot appear.
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    if (key0 + 16 * t + 4 * q4 + v >= kend) {
#pragma unroll
                        for (int dt = 0; dt < NDT; ++dt) T.v[t][dt][v] = (bf16)0.0f;
#pragma unroll
                        for (int rt = 0; rt < NRT; ++rt) T.lv[t][rt][v] = (bf16)0.0f;
                    }
                }
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[dt] = mfma16x16x32(cat4(T.v[0][dt], T.v[1][dt]), pb, acc[dt]);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
            acc_lr[rt] = mfma16x16x32(cat4(T.lv[0][rt], T.lv[1][rt]), pb, acc_lr[rt]);
    };

    {
        Step<D, R> A, B;
        int st = wave;
        if (st < n_steps) load(A, st);
        while (st < n_steps) {
            const int nx = st + WAVES;
            if (nx < n_steps) load(B, nx);
            compute(A, st);
            if (nx >= n_steps) break;
            const int nx2 = nx + WAVES;
            if (nx2 < n_steps) load(A, nx2);
            compute(B, nx);
            st = nx2;
        }
    }
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);

    // ---- merge the four wavefronts through LDS
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int v = 0; v < 4; ++v) sm_o[wave][n16][16 * dt + 4 * q4 + v] = acc[dt][v];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int rank = 16 * rt + 4 * q4 + v;
            if (rank < R) sm_o[wave][n16][D + rank] = acc_lr[rt][v];
        }
    if (q4 == 0) {
        sm_m[wave][n16] = m_run;
        sm_l[wave][n16] = l_run;
    }
    __syncthreads();

    const int n = tid >> 4;   // row handled by this thread in the epilogues
    const int cl = tid & 15;  // column phase
    {
        float mw[WAVES];
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            mw[w] = sm_m[w][n];
            M = fmaxf(M, mw[w]);
        }
        float wt[WAVES];
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            wt[w] = (M == -INFINITY) ? 0.f : fast_exp2(mw[w] - M);
            L += wt[w] * sm_l[w][n];
        }
        for (int c = cl; c < DR; c += 16) {
            float o = 0.f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) o += wt[w] * sm_o[w][n][c];
            sm_o[0][n][c] = o;  // each (n, c) is read and written by this thread only
        }
        if (cl == 0) {
            sm_M[n] = M;
            sm_L[n] = L;
        }
    }

    if (a.n_split > 1) {
        // ---- partial row -> workspace; the last workgroup of the unit merges.
        __syncthreads();
        float* part = a.ws_part + ((size_t)unit * a.n_split + split) * ROWS * (DR + 2);
        if (n < nrows) {
            for (int c = cl; c < DR; c += 16) part[n * (DR + 2) + c] = sm_o[0][n][c];
            if (cl == 0) {
                part[n * (DR + 2) + DR] = sm_M[n];
                part[n * (DR + 2) + DR + 1] = sm_L[n];
            }
        }
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const int prev = atomicAdd(&a.ws_count[unit], 1);
            sm_last = (prev == n_active - 1);
        }
        __syncthreads();
        if (!sm_last) return;
        __threadfence();
        if (n < nrows) {
            const float* p0 = a.ws_part + (size_t)unit * a.n_split * ROWS * (DR + 2) + n * (DR + 2);
            const size_t sstride = (size_t)ROWS * (DR + 2);
            float M = -INFINITY;
            for (int sp = 0; sp < n_active; ++sp) M = fmaxf(M, p0[sp * sstride + DR]);
            float L = 0.f;
            for (int sp = 0; sp < n_active; ++sp) {
                const float w = fast_exp2(p0[sp * sstride + DR] - M);
                L += w * p0[sp * sstride + DR + 1];
            }
            for (int c = cl; c < DR; c += 16) {
                float o = 0.f;
                for (int sp = 0; sp < n_active; ++sp) {
                    const float w = fast_exp2(p0[sp * sstride + DR] - M);
                    o += w * p0[sp * sstride + c];
                }
                sm_o[0][n][c] = o;
            }
            if (cl == 0) {
                sm_M[n] = M;
                sm_L[n] = L;
            }
        }
        if (tid == 0) a.ws_count[unit] = 0;  // leave the workspace clean for the next call
    }
    __syncthreads();

    // ---- epilogue: O = (O_base + O_lr B_v^(h)) / l, one post-multiplication per row
    if (n < nrows) {
        const int req = req0 + n / g;
        int agent = a.req_agent[req];
        agent = min(max(agent, 0), a.n_agents - 1);
        const float L = sm_L[n];
        const float inv = L > 0.f ? 1.0f / L : 0.f;
        const bf16* bv = a.b_v + (size_t)agent * R * a.h_kv * D + (size_t)h * D;
        bf16* op = a.out + ((size_t)req * a.h_q + h * g + n % g) * D;
        for (int c = cl; c < D; c += 16) {
            float o = sm_o[0][n][c];
#pragma unroll
            for (int t = 0; t < R; ++t) o += sm_o[0][n][D + t] * (float)bv[(size_t)t * a.h_kv * D + c];
            op[c] = (bf16)(o * inv);
        }
    }
}

template <int D, int R>
lra_status launch_t(const lra::DecodeArgs& a, const lra::DecodePlan& p, hipStream_t s) {
    DecodeK k;
    k.q = (const bf16*)a.q;
    k.ctx_req_start = a.ctx_req_start;
    k.req_agent = a.req_agent;
    k.k_pool = (const bf16*)a.k_pool;
    k.v_pool = (const bf16*)a.v_pool;
    k.lk_pool = (const bf16*)a.lk_pool;
    k.lv_pool = (const bf16*)a.lv_pool;
    k.block_table = a.block_table;
    k.ctx_len = a.ctx_len;
    k.b_k = (const bf16*)a.b_k;
    k.b_v = (const bf16*)a.b_v;
    k.out = (bf16*)a.out;
    k.ws_count = (int32_t*)a.workspace;
    k.ws_part = (float*)((char*)a.workspace + p.ws_counter_bytes);
    k.n_ctx = a.n_ctx;
    k.n_pages = a.n_pages;
    k.max_blocks = a.max_blocks;
    k.n_agents = a.n_agents;
    k.h_q = a.h_q;
    k.h_kv = a.h_kv;
    k.g = p.g;
    k.rpg = p.rpg;
    k.n_rg = p.n_rg;
    k.n_split = p.n_split;
    k.chunk = p.chunk;
    k.scale_log2 = a.scale * LRA_LOG2E;
    hipLaunchKernelGGL((lra_decode_bf16_kernel<D, R>), dim3(p.grid), dim3(256), 0, s, k);
    return lra::check_launch("lra_decode_bf16_kernel");
}

}  // namespace

namespace lra {

lra_status launch_decode_bf16(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
    const int d = a.head_dim, r = a.rank;
#define LRA_CASE(D_, R_) \
    if (d == D_ && r == R_) return launch_t<D_, R_>(a, p, s);
    LRA_CASE(128, 16)
    LRA_CASE(128, 32)
    LRA_CASE(128, 8)
    LRA_CASE(64, 16)
    LRA_CASE(64, 32)
    LRA_CASE(64, 8)
#undef LRA_CASE
    set_error("decode: unsupported head_dim %d / rank %d", d, r);
    return LRA_ERR_UNSUPPORTED;
}

}  // namespace lra
