// Shared low-rank cache build L = X A for newly processed tokens.
//
// PReCache (PreLRShared) builds the adapters' low-rank caches when a context
// chunk is first processed by multiplying its hidden states with the adapters'
// input (down-projection) matrices; with a shared A (LRAgent §3 BaseLRShared)
// one product serves every agent.  Here both the key and the value
// down-projections are applied in one pass over X:  [L_k | L_v] = X [A_k | A_v].
//
// With one A per agent (PReCache PreLRShared with per-agent adapters, LRAgent
// §3 BaseShared) the same launch builds every agent's cache, X [A_1 .. A_n]:
// workgroups of neighbouring indices take the same 16 tokens for successive
// agents, so X is read from HBM about once and reused from the caches.
//
// The product is tall and skinny (d_model x 2r with 2r <= 64) and bound by
// reading X once from HBM.  A workgroup owns 16 tokens; its 8 wavefronts take
// interleaved 32-wide slices of d_model (so together they stream each X row
// contiguously) and each accumulates the full 16 x 2r tile with
// v_mfma_f32_16x16x32_bf16; the eight partial tiles are summed in LDS and
// rounded once to bf16.  Every wavefront issues the X and A loads of up to 16
// of its slices (8 for r = 32) before the first MFMA, so the whole product waits for about
// one memory round trip instead of one per slice.
#include "lra_common.h"
#include "lra_internal.h"

namespace {

constexpr int TOK = 16;
constexpr int WAVES = 8;

template <int R>
__global__ __launch_bounds__(512) void lra_lr_build_bf16_kernel(const bf16* __restrict__ x,
                                                                const bf16* __restrict__ a_k,
                                                                const bf16* __restrict__ a_v,
                                                                bf16* __restrict__ l_k,
                                                                bf16* __restrict__ l_v,
                                                                int n_tok, int d_model,
                                                                long long row_offset, int n_lr,
                                                                long long lr_stride) {
    constexpr int NT = 2 * R / 16;  // 16-column output tiles (R = 8, 16, 32)
    constexpr int NC = NT * 16;
    constexpr int BATCH = R == 32 ? 8 : 16;  // k-slices per wavefront in flight
    __shared__ float sm[WAVES][TOK][NC + 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, kq = lane >> 4;
    const int ag = blockIdx.x % n_lr;  // whose A / LR cache
    const int tok0 = (blockIdx.x / n_lr) * TOK;
    a_k += (size_t)ag * R * d_model;
    a_v += (size_t)ag * R * d_model;
    l_k += (size_t)ag * lr_stride;
    l_v += (size_t)ag * lr_stride;

    // rows past n_tok read a valid row; their results are never stored
    const bf16* xp = x + (size_t)min(tok0 + l16, n_tok - 1) * d_model + 8 * kq;
    const bf16* wp[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int col = nt * 16 + l16;
        wp[nt] = (col < R ? a_k + (size_t)col * d_model : a_v + (size_t)(col - R) * d_model) + 8 * kq;
    }

    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = zf4();

    // A wavefront takes two adjacent 32-wide slices at a time, so that its two
    // loads per token cover one whole 128-byte line of X.  Every workgroup reads
    // all of A_k and A_v; each starts at its own slice offset so that they do
    // not all request the same A lines (one L2 channel) at once.
    const int n_steps = d_model / 32;
    const int rot = (int)(((blockIdx.x / n_lr) * 16u) % (unsigned)n_steps) & ~1;
    for (int s0 = 2 * wave; s0 < n_steps; s0 += BATCH * WAVES) {
        bf16x8 xa[BATCH], wb[BATCH][NT];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            int sl = min(s0 + (u >> 1) * 2 * WAVES + (u & 1), n_steps - 1) + rot;
            sl = sl >= n_steps ? sl - n_steps : sl;
            const int k = sl * 32;
            xa[u] = ldg((const bf16x8*)(xp + k));
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) wb[u][nt] = ldg((const bf16x8*)(wp[nt] + k));
        }
        __builtin_amdgcn_sched_barrier(0);  // all loads of the batch in flight before the first wait
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            // slices past d_model contribute zero (branch-free: a branch here
            // would drain the loads in flight)
            const bf16x8 xv = s0 + (u >> 1) * 2 * WAVES + (u & 1) < n_steps ? xa[u] : zero8();
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma16x16x32(xv, wb[u][nt], acc[nt]);
        }
    }
    // C lane layout: tokens 4*kq + v, column l16 of each tile
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) sm[wave][4 * kq + v][nt * 16 + l16] = acc[nt][v];
    __syncthreads();
    for (int e = tid; e < TOK * 2 * R; e += blockDim.x) {
        const int t = e / (2 * R), c = e % (2 * R);
        if (tok0 + t >= n_tok) continue;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s += sm[w][t][c];
        const size_t row = (size_t)(row_offset + tok0 + t);
        if (c < R) l_k[row * R + c] = (bf16)s;
        else l_v[row * R + (c - R)] = (bf16)s;
    }
}

__global__ void lra_lr_build_f32_kernel(const float* __restrict__ x, const float* __restrict__ a_k,
                                        const float* __restrict__ a_v, float* __restrict__ l_k,
                                        float* __restrict__ l_v, int n_tok, int d_model, int r,
                                        long long row_offset, int n_lr, long long lr_stride) {
    long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (long long)n_tok * 2 * r * n_lr) return;
    const int ag = (int)(e / ((long long)n_tok * 2 * r));
    e %= (long long)n_tok * 2 * r;
    a_k += (size_t)ag * r * d_model;
    a_v += (size_t)ag * r * d_model;
    l_k += (size_t)ag * lr_stride;
    l_v += (size_t)ag * lr_stride;
    const int t = (int)(e / (2 * r)), c = (int)(e % (2 * r));
    const float* w = c < r ? a_k + (size_t)c * d_model : a_v + (size_t)(c - r) * d_model;
    const float* xr = x + (size_t)t * d_model;
    float s = 0.f;
    for (int k = 0; k < d_model; ++k) s += xr[k] * w[k];
    const size_t row = (size_t)(row_offset + t);
    if (c < r) l_k[row * r + c] = s;
    else l_v[row * r + (c - r)] = s;
}

__global__ void lra_rope_table_kernel(double theta, int head_dim, int n_pos, float* cs, float* sn) {
    const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int half = head_dim / 2;
    if (e >= (long long)n_pos * half) return;
    const int pos = (int)(e / half), i = (int)(e % half);
    const double ang = (double)pos * pow(theta, -2.0 * i / head_dim);
    cs[e] = (float)cos(ang);
    sn[e] = (float)sin(ang);
}

}  // namespace

namespace lra {

lra_status launch_lr_build_bf16(const LRBuildArgs& a, hipStream_t s) {
    if (a.n_tok == 0) return LRA_OK;
    const long long nb = (long long)(a.n_tok + TOK - 1) / TOK * a.n_lr;
    if (nb > 0x7fffffffLL) {
        set_error("lr build: grid of %lld workgroups too large", nb);
        return LRA_ERR_BAD_SHAPE;
    }
    const dim3 grid((unsigned)nb), block(64 * WAVES);
    const long long ro = (long long)a.row_offset, ls = (long long)a.lr_stride;
    const bf16* x = (const bf16*)a.x;
    const bf16* ak = (const bf16*)a.a_k;
    const bf16* av = (const bf16*)a.a_v;
    bf16* lk = (bf16*)a.l_k;
    bf16* lv = (bf16*)a.l_v;
    switch (a.rank) {
        case 8: hipLaunchKernelGGL(lra_lr_build_bf16_kernel<8>, grid, block, 0, s, x, ak, av, lk, lv, a.n_tok, a.d_model, ro, a.n_lr, ls); break;
        case 16: hipLaunchKernelGGL(lra_lr_build_bf16_kernel<16>, grid, block, 0, s, x, ak, av, lk, lv, a.n_tok, a.d_model, ro, a.n_lr, ls); break;
        case 32: hipLaunchKernelGGL(lra_lr_build_bf16_kernel<32>, grid, block, 0, s, x, ak, av, lk, lv, a.n_tok, a.d_model, ro, a.n_lr, ls); break;
        default: set_error("lr build: unsupported rank %d", a.rank); return LRA_ERR_UNSUPPORTED;
    }
    return check_launch("lra_lr_build_bf16_kernel");
}

lra_status launch_lr_build_f32(const LRBuildArgs& a, hipStream_t s) {
    const long long n = (long long)a.n_tok * 2 * a.rank * a.n_lr;
    if (n == 0) return LRA_OK;
    if ((n + 255) / 256 > 0x7fffffffLL) {
        set_error("lr build f32: %lld outputs too many", n);
        return LRA_ERR_BAD_SHAPE;
    }
    hipLaunchKernelGGL(lra_lr_build_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const float*)a.x, (const float*)a.a_k, (const float*)a.a_v, (float*)a.l_k,
                       (float*)a.l_v, a.n_tok, a.d_model, a.rank, (long long)a.row_offset, a.n_lr,
                       (long long)a.lr_stride);
    return check_launch("lra_lr_build_f32_kernel");
}

lra_status launch_rope_table(double theta, int head_dim, int n_pos, float* c, float* sn,
                             hipStream_t st) {
    const long long n = (long long)n_pos * (head_dim / 2);
    if (n == 0) return LRA_OK;
    hipLaunchKernelGGL(lra_rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       theta, head_dim, n_pos, c, sn);
    return check_launch("lra_rope_table_kernel");
}

}  // namespace lra
