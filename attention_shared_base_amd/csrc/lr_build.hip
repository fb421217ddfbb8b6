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
// reading X once from HBM.  Every workgroup also reads the A columns of its
// d_model range, and a CU streams only ~30-40 GB/s of loads (measured: one
// workgroup alone takes as long as 256 together), so the A bytes per token
// set the pace when every CU works on few tokens.
//
// Split kernel (with a workspace): a workgroup owns 64 tokens and one of KS
// ranges of d_model (KS chosen so the grid fills the GPU); each of its 8
// wavefronts takes pairs of 32-wide slices of the range for all four 16-token
// tiles, so an A fragment is loaded once per wavefront and used four times.
// The eight partial tiles are summed in LDS; with KS > 1 the fp32 partial goes
// to the workspace and the last workgroup of the 64 tokens (a counter per
// token block) adds the KS partials in range order and rounds once to bf16.
//
// LDS-staged kernel (the default when d_model is a multiple of its stage): see
// its definition below.
//
// Single-pass kernel (no workspace): a workgroup owns 16 tokens; its 8 wavefronts take
// interleaved 32-wide slices of d_model (so together they stream each X row
// contiguously) and each accumulates the full 16 x 2r tile with
// v_mfma_f32_16x16x32_bf16; the eight partial tiles are summed in LDS and
// rounded once to bf16.  Every wavefront issues the X and A loads of up to 16
// of its slices (8 for r = 32) before the first MFMA, so the whole product waits for about
// one memory round trip instead of one per slice.
#include <stdlib.h>
#include <string.h>

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
    constexpr int NT = (2 * R + 15) / 16;  // 16-column output tiles (R = 4 fills half of one)
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
    bool col_ok[NT];  // output columns past 2R (R = 4) take zero operands
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int col = min(nt * 16 + l16, 2 * R - 1);
        col_ok[nt] = nt * 16 + l16 < 2 * R;
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
            for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma16x16x32(xv, col_ok[nt] ? wb[u][nt] : zero8(), acc[nt]);
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

// LDS-staged kernel: a workgroup owns 16 tokens and the whole of d_model, so no
// partial crosses workgroups.  X rows and the agent's A rows stream through a
// ring of S LDS stages of KC values of k each, moved by buffer_load ... lds in
// 1 KB transfers that each cover whole 128-byte lines (halves or wholes of
// 512- / 1024-byte row pieces).  A CU fetches such transfers about three times
// as fast as the loads of MFMA fragments straight from memory, each of which
// touches 16 rows x 64 bytes.  In LDS the 16-byte chunks of a row sit
// XOR-swizzled by the row index mod 16: the fragment reads of 16 rows
// (ds_read_b128) meet 16 distinct bank groups, and every aligned group of 8
// DMA lanes still fetches one whole line.  The 8 wavefronts split each stage's
// k-steps; their partial 16 x 2R tiles are summed in LDS and rounded once.
template <int R>
struct LdsCfg {
    static constexpr int KC = R <= 8 ? 512 : 256;  // k values per stage (a multiple of d_model)
    static constexpr int CPR = KC / 8;             // 16-byte chunks of a row piece
    static constexpr int ROWS = TOK + 2 * R;       // X rows, then A_k rows, then A_v rows
    static constexpr int STAGE = ROWS * KC * 2;    // bytes of one stage
    static constexpr int S = (160 * 1024 / STAGE) < 6 ? (160 * 1024 / STAGE) : 6;  // ring depth: the LDS, at most 6
    static constexpr int NBLK = STAGE / 1024;      // 1 KB transfers per stage
    static constexpr int PER_WAVE = NBLK / WAVES;
    static constexpr int KPW = KC / 32 / WAVES;    // MFMA k-steps per wavefront per stage
    static_assert(NBLK % WAVES == 0 && (KC / 32) % WAVES == 0, "even split over the wavefronts");
    static_assert(1024 % (CPR * 16) == 0 || (CPR * 16) % 1024 == 0, "transfers hold whole row pieces");
    static_assert(PER_WAVE * (S - 2) < 16, "vmcnt immediate");
};

template <int N>
LRA_DEV void wait_vmcnt() { __builtin_amdgcn_s_waitcnt(0x0f70 | N); }

template <int R>
__global__ __launch_bounds__(512) void lra_lr_build_lds_kernel(const bf16* __restrict__ x,
                                                               const bf16* __restrict__ a_k,
                                                               const bf16* __restrict__ a_v,
                                                               bf16* __restrict__ l_k,
                                                               bf16* __restrict__ l_v,
                                                               int n_tok, int d_model,
                                                               long long row_offset, int n_lr,
                                                               long long lr_stride) {
    using C = LdsCfg<R>;
    constexpr int NT = (2 * R + 15) / 16;  // 16-column output tiles (R = 4 fills half of one)
    constexpr int NC = NT * 16;
    __shared__ __attribute__((aligned(1024))) char ring[C::S * C::STAGE];
    static_assert(WAVES * TOK * (NC + 1) * 4 <= C::S * C::STAGE, "reduction buffer fits the ring");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, kq = lane >> 4;
    const int ag = blockIdx.x % n_lr;  // whose A / LR cache
    const int tok0 = (blockIdx.x / n_lr) * TOK;
    const int rows = min(TOK, n_tok - tok0);
    const uint32_t rowb = (uint32_t)d_model * 2;
    // this block's X rows (rows past n_tok read as zero) and the agent's A_k, A_v
    const u32x4 rx = make_rsrc(x + (size_t)tok0 * d_model, (uint32_t)rows * rowb);
    const u32x4 rk = make_rsrc(a_k + (size_t)ag * R * d_model, (uint32_t)R * rowb);
    const u32x4 rv = make_rsrc(a_v + (size_t)ag * R * d_model, (uint32_t)R * rowb);
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)ring;

    // stage st into its ring slot: transfer b of the stage lands at slot + 1 KB * b;
    // its lane i fills 16-byte chunk p = 64 b + i, i.e. row p / CPR at swizzled
    // position p % CPR, and so reads that row's chunk (p % CPR) ^ (row % 16).
    // Every workgroup walks d_model in the same order: they all read the same A,
    // and requests of one line that arrive together are served by one fetch
    // (starting each block at another stage measured 20% slower).
    auto issue = [&](int st) {
        const uint32_t slot = ring_lds + (uint32_t)(st % C::S) * C::STAGE;
        const uint32_t k0b = (uint32_t)st * C::KC * 2;
#pragma unroll
        for (int u = 0; u < C::PER_WAVE; ++u) {
            const int b = wave + WAVES * u;
            const int p = 64 * b + lane;
            const int row = p / C::CPR;
            const int chunk = (p % C::CPR) ^ (row & 15);
            const int row0 = (64 * b) / C::CPR;  // first row of the transfer: picks the matrix
            const uint32_t inrow = k0b + 16u * chunk;
            if (row0 < TOK)
                dma_1k(rx, slot + 1024u * b, (uint32_t)row * rowb + inrow);
            else if (row0 < TOK + R)
                dma_1k(rk, slot + 1024u * b, (uint32_t)(row - TOK) * rowb + inrow);
            else
                dma_1k(rv, slot + 1024u * b, (uint32_t)(row - TOK - R) * rowb + inrow);
        }
    };

    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = zf4();
    auto compute = [&](int st) {
        const char* slot = ring + (st % C::S) * C::STAGE;
#pragma unroll
        for (int u = 0; u < C::KPW; ++u) {
            const int j = 4 * (wave + WAVES * u) + kq;  // chunk of this lane's 8 k values
            const bf16x8 xa = *(const bf16x8*)(slot + 16 * (l16 * C::CPR + (j ^ l16)));
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int c = nt * 16 + l16;  // output column = A row
                bf16x8 wb = zero8();
                if (c < 2 * R) wb = *(const bf16x8*)(slot + 16 * ((TOK + c) * C::CPR + (j ^ l16)));
                acc[nt] = mfma16x16x32(xa, wb, acc[nt]);
            }
        }
    };

    const int n_st = d_model / C::KC;
#pragma unroll
    for (int st = 0; st < C::S - 1; ++st)
        if (st < n_st) issue(st);
    for (int st = 0; st < n_st; ++st) {
        // this wavefront's transfers of stage st have landed; those of the (at
        // most S - 2) stages it issued after st may still be in flight
        if (st + C::S - 2 < n_st) wait_vmcnt<C::PER_WAVE * (C::S - 2)>();
        else wait_vmcnt<0>();
        __syncthreads();  // every wavefront's part of stage st is in LDS, and stage st - 1 is consumed
        if (st + C::S - 1 < n_st) issue(st + C::S - 1);  // into stage st - 1's slot
        compute(st);
    }

    __syncthreads();  // the ring becomes the reduction buffer
    float(*sm)[TOK][NC + 1] = reinterpret_cast<float(*)[TOK][NC + 1]>(ring);
    // C lane layout: tokens 4*kq + v, column l16 of each tile
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) sm[wave][4 * kq + v][nt * 16 + l16] = acc[nt][v];
    __syncthreads();
    l_k += (size_t)ag * lr_stride;
    l_v += (size_t)ag * lr_stride;
    for (int e = tid; e < TOK * 2 * R; e += blockDim.x) {
        const int t = e / (2 * R), c = e % (2 * R);
        if (t >= rows) continue;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) sum += sm[w][t][c];
        const size_t row = (size_t)(row_offset + tok0 + t);
        if (c < R) l_k[row * R + c] = (bf16)sum;
        else l_v[row * R + (c - R)] = (bf16)sum;
    }
}

// cache-policy bit sc1 (agent-coherent, as agent-scope atomic accesses) and
// the s_waitcnt immediate for vmcnt(0)
constexpr int LR_CPOL_SC1 = 16;
constexpr int LR_WAITCNT_VMCNT0 = 0x0f70;
constexpr int STOK = 64;  // tokens per workgroup of the split kernel

struct LRSplitK {
    const bf16* x;
    const bf16* a_k;
    const bf16* a_v;
    bf16* l_k;
    bf16* l_v;
    float* ws_part;   // [units][ks][STOK][2R]
    int32_t* ws_count;  // [units]
    long long row_offset, lr_stride;
    int32_t n_tok, d_model, n_lr, ks, slices_per_split;
};

template <int R>
__global__ __launch_bounds__(512) void lra_lr_build_split_kernel(LRSplitK p) {
    constexpr int NT = (2 * R + 15) / 16;  // 16-column output tiles (R = 4 fills half of one)
    constexpr int NC = NT * 16;            // = 2R, or 16 for R = 4
    constexpr int MT = STOK / 16;   // 16-token tiles
    constexpr int PB = 2;           // slice pairs per wavefront per batch
    __shared__ float sm[WAVES][STOK][NC + 1];
    __shared__ int sm_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, kq = lane >> 4;
    // neighbouring workgroups: the same tokens and range for successive agents
    // (X reused from the caches), then the ranges of one token block
    const int ag = blockIdx.x % p.n_lr;
    const int rest = blockIdx.x / p.n_lr;
    const int ks = rest % p.ks;
    const int tb = rest / p.ks;
    const int tok0 = tb * STOK;
    const int unit = tb * p.n_lr + ag;
    const bf16* a_k = p.a_k + (size_t)ag * R * p.d_model;
    const bf16* a_v = p.a_v + (size_t)ag * R * p.d_model;

    const bf16* xp[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)  // rows past n_tok read a valid row; never stored
        xp[m] = p.x + (size_t)min(tok0 + 16 * m + l16, p.n_tok - 1) * p.d_model + 8 * kq;
    const bf16* wp[NT];
    bool col_ok[NT];  // output columns past 2R (R = 4) take zero operands
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int col = min(nt * 16 + l16, 2 * R - 1);
        col_ok[nt] = nt * 16 + l16 < 2 * R;
        wp[nt] = (col < R ? a_k + (size_t)col * p.d_model : a_v + (size_t)(col - R) * p.d_model) + 8 * kq;
    }
    f32x4 acc[MT][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[m][nt] = zf4();

    // slices [s_beg, s_end) of this range; a wavefront takes two adjacent
    // slices at a time (its two loads per token row cover a 128-byte line)
    const int n_steps = p.d_model / 32;
    const int s_beg = ks * p.slices_per_split;
    const int s_end = min(s_beg + p.slices_per_split, n_steps);
    for (int s0 = s_beg + 2 * wave; s0 < s_end; s0 += 2 * WAVES * PB) {
        bf16x8 xa[MT][2 * PB], wb[2 * PB][NT];
#pragma unroll
        for (int u = 0; u < 2 * PB; ++u) {
            const int k = min(s0 + (u >> 1) * 2 * WAVES + (u & 1), n_steps - 1) * 32;
#pragma unroll
            for (int m = 0; m < MT; ++m) xa[m][u] = ldg((const bf16x8*)(xp[m] + k));
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) wb[u][nt] = ldg((const bf16x8*)(wp[nt] + k));
        }
        __builtin_amdgcn_sched_barrier(0);  // the batch's loads all in flight before the first wait
#pragma unroll
        for (int u = 0; u < 2 * PB; ++u) {
            // slices past the range contribute zero (branch-free)
            const bool ok = s0 + (u >> 1) * 2 * WAVES + (u & 1) < s_end;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const bf16x8 xv = ok ? xa[m][u] : zero8();
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[m][nt] = mfma16x16x32(xv, col_ok[nt] ? wb[u][nt] : zero8(), acc[m][nt]);
            }
        }
    }
    // C lane layout: tokens 16 m + 4 kq + v, column nt * 16 + l16
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v) sm[wave][16 * m + 4 * kq + v][nt * 16 + l16] = acc[m][nt][v];
    __syncthreads();
    // thread e: elements e, e + 512, ... of the [STOK][2R] tile
    constexpr int EPT = STOK * NC / 512;
    float sum[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int e = tid + 512 * j, t = e / NC, c = e % NC;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s += sm[w][t][c];
        sum[j] = s;
    }
    if (p.ks > 1) {
        // partial -> workspace with agent-coherent stores; every wavefront waits
        // for its store acknowledgements before the barrier, and only then is
        // the counter bumped; the last of the KS workgroups reads the others
        // with agent-coherent loads and adds all in range order
        float* part = p.ws_part + (size_t)unit * p.ks * STOK * NC;
#pragma unroll
        for (int j = 0; j < EPT; ++j)
            __hip_atomic_store(part + (size_t)ks * STOK * NC + tid + 512 * j, sum[j], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(LR_WAITCNT_VMCNT0);
        __syncthreads();
        if (tid == 0) {
            const int prev = __hip_atomic_fetch_add(p.ws_count + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sm_last = prev == p.ks - 1;
        }
        __syncthreads();
        if (!sm_last) return;
        float tot[EPT];
#pragma unroll
        for (int j = 0; j < EPT; ++j) tot[j] = 0.f;
        for (int r0 = 0; r0 < p.ks; r0 += 4) {
            float v[4][EPT];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int j = 0; j < EPT; ++j)
                    v[u][j] = (r0 + u < p.ks && r0 + u != ks)
                                  ? __hip_atomic_load(part + (size_t)(r0 + u) * STOK * NC + tid + 512 * j,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                  : sum[j];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int j = 0; j < EPT; ++j)
                    if (r0 + u < p.ks) tot[j] += v[u][j];
        }
#pragma unroll
        for (int j = 0; j < EPT; ++j) sum[j] = tot[j];
        if (tid == 0) __hip_atomic_store(p.ws_count + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    bf16* l_k = p.l_k + (size_t)ag * p.lr_stride;
    bf16* l_v = p.l_v + (size_t)ag * p.lr_stride;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int e = tid + 512 * j, t = e / NC, c = e % NC;
        if (tok0 + t < p.n_tok && c < 2 * R) {
            const size_t row = (size_t)(p.row_offset + tok0 + t);
            if (c < R) l_k[row * R + c] = (bf16)sum[j];
            else l_v[row * R + (c - R)] = (bf16)sum[j];
        }
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

LRPlan lr_build_plan(int n_tok, int d_model, int rank, int n_lr) {
    LRPlan pl{};
    const long long units = (long long)(n_tok + STOK - 1) / STOK * n_lr;
    const int n_steps = d_model / 32;
    // ranges of d_model: enough workgroups for every CU from one agent's token
    // blocks, each range still >= 16 slices (two per wavefront).  The split
    // does not depend on n_lr, so a build of n caches in one call gives the
    // bits of n single-cache builds.
    const long long blocks = (long long)(n_tok + STOK - 1) / STOK;
    int ks = 1;
    while (ks < 8 && blocks * ks < 256 && n_steps / (2 * ks) >= 16) ks *= 2;
    pl.ks = ks;
    pl.slices_per_split = ((n_steps + ks - 1) / ks + 1) / 2 * 2;
    pl.units = units;
    pl.ws_counter_bytes = ((size_t)units * sizeof(int32_t) + 255) / 256 * 256;
    const int nc = 2 * rank < 16 ? 16 : 2 * rank;  // fp32 columns of a partial row
    pl.ws_bytes = ks > 1 ? pl.ws_counter_bytes + (size_t)units * ks * STOK * nc * sizeof(float) : 0;
    return pl;
}

lra_status launch_lr_build_bf16(const LRBuildArgs& a, hipStream_t s) {
    if (a.n_tok == 0) return LRA_OK;
    const bf16* x = (const bf16*)a.x;
    const bf16* ak = (const bf16*)a.a_k;
    const bf16* av = (const bf16*)a.a_v;
    bf16* lk = (bf16*)a.l_k;
    bf16* lv = (bf16*)a.l_v;
    const long long ro = (long long)a.row_offset, ls = (long long)a.lr_stride;
    // The LDS-staged kernel whenever d_model is a multiple of its stage (256, or
    // 512 for ranks <= 8); it needs no workspace.  LRA_LR_BUILD_PATH = split or
    // single selects one of the other two kernels instead (comparisons, tests).
    const char* path = getenv("LRA_LR_BUILD_PATH");
    const bool want_split = path && strcmp(path, "split") == 0;
    const bool want_single = path && strcmp(path, "single") == 0;
    const int kc = a.rank <= 8 ? 512 : 256;
    // its buffer ranges and offsets are 32-bit byte counts: X rows of a block and
    // the 2 * rank A rows must stay below 2^31 bytes
    const bool fits = (long long)(TOK > 2 * a.rank ? TOK : 2 * a.rank) * a.d_model * 2 < (1LL << 31);
    if (!want_split && !want_single && a.d_model % kc == 0 && fits) {
        const long long nb = (long long)(a.n_tok + TOK - 1) / TOK * a.n_lr;
        if (nb > 0x7fffffffLL) {
            set_error("lr build: grid of %lld workgroups too large", nb);
            return LRA_ERR_BAD_SHAPE;
        }
        const dim3 grid((unsigned)nb), block(64 * WAVES);
        switch (a.rank) {
            case 4: hipLaunchKernelGGL(lra_lr_build_lds_kernel<4>, grid, block, 0, s, x, ak, av, lk, lv, a.n_tok, a.d_model, ro, a.n_lr, ls); break;
            case 8: hipLaunchKernelGGL(lra_lr_build_lds_kernel<8>, grid, block, 0, s, x, ak, av, lk, lv, a.n_tok, a.d_model, ro, a.n_lr, ls); break;
            case 16: hipLaunchKernelGGL(lra_lr_build_lds_kernel<16>, grid, block, 0, s, x, ak, av, lk, lv, a.n_tok, a.d_model, ro, a.n_lr, ls); break;
            case 32: hipLaunchKernelGGL(lra_lr_build_lds_kernel<32>, grid, block, 0, s, x, ak, av, lk, lv, a.n_tok, a.d_model, ro, a.n_lr, ls); break;
            default: set_error("lr build: unsupported rank %d", a.rank); return LRA_ERR_UNSUPPORTED;
        }
        return check_launch("lra_lr_build_lds_kernel");
    }
    const LRPlan pl = lr_build_plan(a.n_tok, a.d_model, a.rank, a.n_lr);
    if (!want_single && (pl.ks == 1 || a.workspace != nullptr)) {
        const long long nb = pl.units * pl.ks;
        if (nb > 0x7fffffffLL) {
            set_error("lr build: grid of %lld workgroups too large", nb);
            return LRA_ERR_BAD_SHAPE;
        }
        LRSplitK k{};
        k.x = x;
        k.a_k = ak;
        k.a_v = av;
        k.l_k = lk;
        k.l_v = lv;
        k.ws_count = (int32_t*)a.workspace;
        k.ws_part = a.workspace ? (float*)((char*)a.workspace + pl.ws_counter_bytes) : nullptr;
        k.row_offset = ro;
        k.lr_stride = ls;
        k.n_tok = a.n_tok;
        k.d_model = a.d_model;
        k.n_lr = a.n_lr;
        k.ks = pl.ks;
        k.slices_per_split = pl.slices_per_split;
        const dim3 grid((unsigned)nb), block(64 * WAVES);
        switch (a.rank) {
            case 4: hipLaunchKernelGGL(lra_lr_build_split_kernel<4>, grid, block, 0, s, k); break;
            case 8: hipLaunchKernelGGL(lra_lr_build_split_kernel<8>, grid, block, 0, s, k); break;
            case 16: hipLaunchKernelGGL(lra_lr_build_split_kernel<16>, grid, block, 0, s, k); break;
            case 32: hipLaunchKernelGGL(lra_lr_build_split_kernel<32>, grid, block, 0, s, k); break;
            default: set_error("lr build: unsupported rank %d", a.rank); return LRA_ERR_UNSUPPORTED;
        }
        return check_launch("lra_lr_build_split_kernel");
    }
    // no workspace: 16-token workgroups over the whole of d_model
    const long long nb = (long long)(a.n_tok + TOK - 1) / TOK * a.n_lr;
    if (nb > 0x7fffffffLL) {
        set_error("lr build: grid of %lld workgroups too large", nb);
        return LRA_ERR_BAD_SHAPE;
    }
    const dim3 grid((unsigned)nb), block(64 * WAVES);
    switch (a.rank) {
        case 4: hipLaunchKernelGGL(lra_lr_build_bf16_kernel<4>, grid, block, 0, s, x, ak, av, lk, lv, a.n_tok, a.d_model, ro, a.n_lr, ls); break;
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
