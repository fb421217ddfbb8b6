// Paged Flash-LoRA-Attention decode, bf16 storage / fp32 accumulation, gfx950.
// (kernel template; instantiated by decode_bf16.hip and decode_rope_bf16.hip)
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
// and the last workgroup of the unit to finish merges them (log-sum-exp) and
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
//
// RoPE on the adapter key (LRAgent App. D.1).  When the model rotates keys,
// the adapter term must be rotated with its key's position before it meets
// the query, s_j = q . (k_base_j + rot_j(l_k_j B_k^(h))), so the key side
// cannot stay at rank r: per page and per request of the group the kernel
// rebuilds dK^T = B_k^(h)T L_k^T on the matrix cores (lane = token, 4 dims per
// 16-dim tile), rotates the pairs (i, i + d/2) lane-locally with the page's
// cos/sin rows, rounds the rotated term to bf16 and adds its product with the
// query rows of that request to the base scores.  The rebuilt key never
// leaves registers; the value side is unchanged.  B_k^(h) of every request
// in the group is staged once per work item in LDS, already in the operand
// layout.
#pragma once

#include "lra_common.h"
#include "lra_internal.h"

namespace {

constexpr int PAGE = 16;
constexpr int ROWS = 16;
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
    int32_t h_q, h_kv, g, rpg, n_rg, n_split;
    int32_t n_units;
    int32_t n_req;
    int32_t persistent;  // 1: workgroups pull (context, row group, head, chunk) items from a queue
    float scale_log2;
    const float* rope_cos;  // RoPE: [rope_rows, D/2] tables of the keys' positions
    const float* rope_sin;
    int32_t rope_rows;
    int32_t max_len;    // max_ctx_len: longer contexts are cut to it (the workspace is sized for it)
    int64_t lr_stride;  // per-agent LR caches: elements between agents' pools (0: one shared cache)
};

// Persistent mode keeps the per-context item prefix sums in LDS.
constexpr int MAX_CTX_PERSISTENT = 1024;

// The rank-r score term uses the same v_mfma_f32_16x16x32_bf16 as the base
// term it accumulates onto.  Every accumulator chain in this file stays on one
// MFMA shape: a 16x16x32 result fed straight into a dependent 16x16x16 on the
// same accumulator lost the first MFMA's contribution in the low accumulator
// elements on gfx950, so r <= 16 is zero-padded to k = 32 instead (slots 0-3
// of each k-group carry ranks 4*q4 + v, slots 4-7 carry ranks 16 + 4*q4 + v
// or zeros).

// B_v^(h) columns c0 .. c0 + D/16 - 1 of every rank, for one output thread
template <int D, int R>
struct BvCols {
    typedef __bf16 vec __attribute__((ext_vector_type(D / 16)));
    vec r[R];
};

template <int D, int R, int SP>
__device__ __forceinline__ void finalize_rows(const DecodeK& a, const float (*o)[SP], const float* L_row,
                                              int n, int cl, int nrows, int req0, int h,
                                              const BvCols<D, R>& bv);

// cache-policy bit sc1 of buffer loads/stores (agent-coherent, as the
// agent-scope atomic loads/stores the compiler emits); s_waitcnt immediate for
// vmcnt(0) with the other counters left unconstrained
constexpr int CPOL_SC1 = 16;
constexpr int WAITCNT_VMCNT0 = 0x0f70;
// 16-byte groups per partial row ([O_base | O_lr], then (m, l)) handled by each
// of the 16 threads of a row
template <int DR>
constexpr int MERGE_NG = (DR / 4 + 1 + 15) / 16;

template <int D, int R, int SP, int NG>
__device__ __forceinline__ void merge_partials(const DecodeK& a, int unit, int own, int n_active, int nrows,
                                               int n, int cl, const f32x4 (&own_o)[NG], float own_m,
                                               float own_l, float (*o)[SP], float* L_row);

// NQ: LR caches read per step (1 shared; 4 = one per request slot of the group)
template <int D, int R, int NQ = 1>
struct Step {
    static constexpr int NJ = D / 32;          // score MFMAs (dims) per page
    static constexpr int NDT = D / 16;         // value tiles (dims)
    static constexpr int NRT = (R + 15) / 16;  // value tiles (ranks)
    bf16x8 k[2][NJ];
    bf16x8 lk[NQ][2];
    bf16x4 v[2][NDT];
    bf16x4 lv[NQ][2][NRT];
};

// Modes of the decode kernel: the rank-r score term on the shared LR cache; the
// adapter key rebuilt and rotated (RoPE); one LR cache per agent (the agent's
// L_k, L_v rows for its own requests' rows, at most PA_REQ requests per group).
constexpr int MODE_SHARED = 0, MODE_ROPE = 1, MODE_PER_AGENT = 2, MODE_ROPE_PER_AGENT = 3;
constexpr int PA_REQ = 4;

// RoPE: cos, sin of one step's keys (page t, token n16), dims 16*ht + 4*q4 .. +3
template <int D>
struct StepRope {
    f32x4 cs[2][D / 32][2];
};

// WAVES wavefronts per workgroup; SPW = 32-token steps per wavefront; a
// workgroup covers WAVES * SPW * 32 tokens.  DEPTH = step buffers per
// wavefront (DEPTH - 1 steps of loads in flight).  MODE: see MODE_SHARED ..
template <int D, int R, int SPW, int DEPTH, int WAVES, int MODE>
__global__ __launch_bounds__(64 * WAVES) void lra_decode_bf16_kernel(DecodeK a) {
    constexpr bool ROPE = MODE == MODE_ROPE || MODE == MODE_ROPE_PER_AGENT;
    constexpr bool PA = MODE == MODE_PER_AGENT || MODE == MODE_ROPE_PER_AGENT;
    // RoPE: later steps' cos / sin by angle addition from step 0's rows, except
    // in the per-agent instances of ranks 8 and 32, whose registers are full (the
    // angle update spills there): those load every step's rows
    constexpr bool RADV = MODE == MODE_ROPE || (MODE == MODE_ROPE_PER_AGENT && R != 8 && R != 32);
    constexpr int NQ = PA ? PA_REQ : 1;
    // request -> agent table fetched at kernel start (see below); the RoPE and
    // per-agent rank-32 instances keep scalar loads, as their registers are full
    constexpr bool AGENT_TAB = !ROPE && !(PA && R == 32);
    using StepT = Step<D, R, NQ>;
    constexpr int NJ = StepT::NJ;
    constexpr int NDT = StepT::NDT;
    constexpr int NRT = StepT::NRT;
    constexpr int DR = D + R;
    // LDS row pitch: 4 x an odd number of floats, so rows start 16-byte aligned
    // (vector reads and writes) and the 16 rows of a 16-byte access fall on 16
    // distinct 4-bank groups (an odd multiplier is invertible mod 16)
    constexpr int SP = ((DR / 4 + 1) | 1) * 4;
    static_assert(DR % 4 == 0 && SP > DR, "row pitch");
    constexpr int CHUNK = WAVES * SPW * KEYS_PER_STEP;

    // RoPE: B_k^(h)T operands of up to ROWS requests (one per row when g = 1),
    // [request][dim tile][lane] x 16 bytes (unused rank slots hold zeros).
    // They are needed only while streaming and the wavefront merge buffer only
    // after it, so the two share one LDS block (a barrier separates the uses).
    constexpr int BKW = 16;
    constexpr int SMO_BYTES = WAVES * ROWS * SP * 4;
    constexpr int BK_BYTES = ROPE ? ROWS * NDT * 64 * BKW : 0;
    __shared__ __attribute__((aligned(16))) char sm_raw[SMO_BYTES > BK_BYTES ? SMO_BYTES : BK_BYTES];
    float(*const sm_o)[ROWS][SP] = reinterpret_cast<float(*)[ROWS][SP]>(sm_raw);
    char* const sm_bk = sm_raw;
    __shared__ int sm_pid[ROPE ? CHUNK / PAGE : 1];
    // RoPE: cos / sin of the angle of WAVES * 32 positions (table row WAVES * 32),
    // [dim tile ht][cos, sin][k-group q4]: dims 16*ht + 4*q4 .. + 3
    __shared__ f32x4 sm_radv[RADV ? D / 32 : 1][2][4];
    __shared__ float sm_m[WAVES][ROWS];
    __shared__ float sm_l[WAVES][ROWS];
    __shared__ float sm_L[ROWS];
    __shared__ int sm_last;
    // agent ids of the row group's requests.  Every thread writes every entry
    // (the same uniform values), so each thread reads back its own writes and
    // no barrier is needed between the prologue and the epilogue's reads.
    __shared__ int sm_agent[ROWS];
    __shared__ int sm_pref[MAX_CTX_PERSISTENT + 1];
    __shared__ int sm_item;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform by construction; readfirstlane lets the compiler see it, so
    // page-table reads become scalar loads that never wait on the vector loads
    // in flight (a vector page-id load would force a full vmcnt(0) drain).
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15;  // row (S^T / O^T column) of this lane
    const int q4 = lane >> 4;   // k-group of this lane

    // all kernel arguments in one scalar round trip (the compiler would otherwise
    // fetch them piecemeal between the dependent loads below)
    asm volatile("" ::"s"(a.k_pool), "s"(a.v_pool), "s"(a.lk_pool), "s"(a.lv_pool), "s"(a.block_table),
                 "s"(a.ctx_len), "s"(a.ctx_req_start), "s"(a.q), "s"(a.b_k), "s"(a.req_agent));
    asm volatile("" ::"s"(a.n_ctx), "s"(a.n_pages), "s"(a.max_blocks), "s"(a.n_agents), "s"(a.h_q),
                 "s"(a.h_kv), "s"(a.g), "s"(a.rpg), "s"(a.n_rg), "s"(a.n_split));
    // agent ids of requests 0..63 (lane i: request i), fetched by one vector load
    // before any cache load.  With up to 64 requests the prologue takes its
    // group's ids from here instead of a dependent scalar load, which would queue
    // behind every CU's first cache loads; a wait for this load never waits for
    // those.  Entries past n_req read as zero through the buffer range.
    int agent_tab = 0;
    if constexpr (AGENT_TAB)
        agent_tab = (int)__builtin_amdgcn_raw_buffer_load_b32(
            __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(a.req_agent), (short)0, 4 * min(a.n_req, 64), 0x00020000),
            4 * lane, 0, 0);

    // ---- one work item: chunk `split` of row group rg of context ctx, KV head h
    // `queue`: persistent mode's queue (NULL otherwise); the next item's index is
    // requested into *next once this item's streaming is done, so the round trip
    // overlaps the merge tail without reserving work early
    auto process = [&](const int ctx, const int rg, const int h, const int split, int* queue,
                       int* next) __attribute__((always_inline)) {
    const int unit = (ctx * a.n_rg + rg) * a.h_kv + h;
    auto grab_next = [&]() {
        if (queue != nullptr && tid == 0)
            *next = __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    // ---- every scalar load the step addresses depend on goes out at once,
    // before any branch on their values: request range and length of the
    // context, and the raw page-table entries of this wavefront's steps (rows
    // clamped to the table; pages past the chunk end are replaced below).
    const int* bt = a.block_table + (size_t)ctx * a.max_blocks;
    const int kbeg = split * CHUNK;
    const int rs0 = a.ctx_req_start[ctx];
    const int rs1 = a.ctx_req_start[ctx + 1];
    const int len_raw = a.ctx_len[ctx];
    const int first_raw = bt[min(kbeg >> 4, a.max_blocks - 1)];
    // (RoPE: the first step only; its stream reads later steps' ids as it goes)
    constexpr int NPRE = ROPE ? 1 : SPW;
    int praw[NPRE][2];
#pragma unroll
    for (int i = 0; i < NPRE; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
            praw[i][t] = bt[min((kbeg >> 4) + 2 * (wave + WAVES * i) + t, a.max_blocks - 1)];
    asm volatile("" ::"s"(rs0), "s"(rs1), "s"(len_raw), "s"(first_raw));
#pragma unroll
    for (int i = 0; i < NPRE; ++i) asm volatile("" ::"s"(praw[i][0]), "s"(praw[i][1]));

    const int req0 = rs0 + rg * a.rpg;
    const int nreq = min(a.rpg, rs1 - req0);
    if (nreq <= 0) {
        grab_next();
        return;
    }
    const int g = a.g;
    const int nrows = nreq * g;
    // lengths are clamped to max_ctx_len: the host sized the chunk count and the
    // workspace for it, and a longer context must not add chunks past them
    const int len = min(min(len_raw, a.max_blocks * PAGE), a.max_len);

    if (len <= 0) {  // empty context: defined as zero output
        if (split == 0) {
            for (int e = tid; e < nrows * D; e += blockDim.x) {
                const int n = e / D, c = e % D;
                a.out[((size_t)(req0 + n / g) * a.h_q + h * g + n % g) * D + c] = (bf16)0.0f;
            }
        }
        grab_next();
        return;
    }
    const int n_active = (len + CHUNK - 1) / CHUNK;
    if (split >= n_active) {
        grab_next();
        return;
    }
    const int kend = min(len, kbeg + CHUNK);

    // ---- page ids of this wavefront's steps.  Pages past the chunk end take
    // the chunk's first page: those steps load cached data and are never
    // computed, so the loads can stay unconditional.
    const int last_pg = (kend - 1) >> 4;
    auto page_of = [&](int i, int t, int raw) {
        const int pg = (kbeg >> 4) + 2 * (wave + WAVES * i) + t;
        return min(max(pg <= last_pg ? raw : first_raw, 0), a.n_pages - 1);
    };
    int pid[NPRE][2];
#pragma unroll
    for (int i = 0; i < NPRE; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t) pid[i][t] = page_of(i, t, praw[i][t]);
    // RoPE stream: the chunk's raw page ids are staged in LDS with the B_k
    // operands (one vector load per thread) and read back per step
    if constexpr (ROPE) {
        if (tid < CHUNK / PAGE) sm_pid[tid] = bt[min((kbeg >> 4) + tid, a.max_blocks - 1)];
    }
    auto page_now = [&](int i, int t) {
        const int raw = __builtin_amdgcn_readfirstlane(sm_pid[2 * (wave + WAVES * i) + t]);
        return page_of(i, t, raw);
    };

    const size_t kv_page = (size_t)a.h_kv * D * PAGE;  // elements per page (all heads)
    const bf16* kbase = a.k_pool + (size_t)h * D * PAGE;
    const bf16* vbase = a.v_pool + (size_t)h * D * PAGE;

    // agent ids of the group's first four requests, from the table above; with
    // more than 64 requests, from a table reloaded at the group's first request
    int agent0[4];
    if constexpr (AGENT_TAB) {
        int tab = agent_tab, tab0 = 0;
        if (a.n_req > 64) {
            tab = (int)__builtin_amdgcn_raw_buffer_load_b32(
                __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(a.req_agent), (short)0, 4 * a.n_req, 0x00020000),
                4 * (req0 + lane), 0, 0);
            tab0 = req0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) agent0[u] = __builtin_amdgcn_readlane(tab, req0 - tab0 + min(u, nreq - 1));
    } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) agent0[u] = a.req_agent[req0 + min(u, nreq - 1)];
    }
    // per-agent LR caches: the step loads address the agents' pools
    int agent_of[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) agent_of[u] = PA ? min(max(agent0[u], 0), a.n_agents - 1) : 0;

    // Loads of one step: no data-dependent branches; dead slots are masked later.
    auto load = [&](StepT& T, const int (&pids)[2]) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const bf16* kp = kbase + (size_t)pids[t] * kv_page;
            const bf16* vp = vbase + (size_t)pids[t] * kv_page;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                T.k[t][j] = ldg_stream((const bf16x8*)(kp + ((4 * j + q4) * PAGE + n16) * 8));
#pragma unroll
            for (int u = 0; u < NQ; ++u) {
                // per-agent LR caches: request slot u reads its agent's pages
                // (slots past the group repeat its last request; never used)
                const size_t lr_off = PA ? (size_t)agent_of[u] * a.lr_stride : 0;
                const bf16* lkp = a.lk_pool + lr_off + (size_t)pids[t] * PAGE * R;
                const bf16* lvp = a.lv_pool + lr_off + (size_t)pids[t] * PAGE * R;
                if constexpr (R == 32) {
                    T.lk[u][t] = cat4(ldg((const bf16x4*)(lkp + n16 * R + 4 * q4)),
                                      ldg((const bf16x4*)(lkp + n16 * R + 16 + 4 * q4)));
                } else if constexpr (R == 16) {
                    T.lk[u][t] = cat4(ldg((const bf16x4*)(lkp + n16 * R + 4 * q4)), zero4());
                } else {
                    // R = 8 / 4: k-groups past R/4 hold zero ranks (loads stay in the row)
                    T.lk[u][t] = cat4(ldg((const bf16x4*)(lkp + n16 * R + 4 * (q4 % (R / 4)))), zero4());
                    if (q4 >= R / 4) T.lk[u][t] = zero8();
                }
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) {
                    const int rank = min(16 * rt + n16, R - 1);
                    T.lv[u][t][rt] = ldg((const bf16x4*)(lvp + rank * PAGE + 4 * q4));
                }
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                T.v[t][dt] = ldg_stream((const bf16x4*)(vp + (16 * dt + n16) * PAGE + 4 * q4));
        }
    };
    // RoPE tables of step i's keys: the key's position in its context is its
    // token index.  With RADV only step 0's rows are loaded: every later step's
    // keys sit WAVES * 32 positions after the previous step's, so their cos /
    // sin follow by angle addition with the table row of that distance
    // (sm_radv), and the stream issues no table loads.  Otherwise step i+1's
    // rows are requested when step i is done with its own (one buffer).  Rows
    // are read through a buffer range starting at the page's first key, so the
    // address stays scalar; rows past the table read as zero (keys there are
    // past the context and masked).
    const uint32_t rope_voff = (uint32_t)(n16 * (D / 2) + 4 * q4) * 4;
    auto load_rope = [&](StepRope<D>& C, int i) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int row0 = kbeg + (wave + WAVES * i) * KEYS_PER_STEP + PAGE * t;
            const uint32_t bytes = (uint32_t)max(a.rope_rows - row0, 0) * (D / 2) * 4;
            const __amdgpu_buffer_rsrc_t rc =
                __builtin_amdgcn_make_buffer_rsrc((void*)(a.rope_cos + (size_t)row0 * (D / 2)), (short)0, bytes, 0x00020000);
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc((void*)(a.rope_sin + (size_t)row0 * (D / 2)), (short)0, bytes, 0x00020000);
#pragma unroll
            for (int ht = 0; ht < D / 32; ++ht) {
                C.cs[t][ht][0] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, rope_voff + 64 * ht, 0, 0));
                C.cs[t][ht][1] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, rope_voff + 64 * ht, 0, 0));
            }
        }
    };


    // ---- query operand (B of the score MFMA): lane holds dims 32j+8*q4.. of row
    // n16.  Loaded unconditionally (rows past nrows read row 0 and are zeroed
    // just before use): a branch here would drain the step loads in flight.
    const bool row_ok = n16 < nrows;
    bf16x8 qf[NJ];
    // RoPE: the same query rows with the dims of k-step j in the order of the
    // rebuilt key operand: slots 0-3 = dims 32j + 4*q4 .., slots 4-7 = 32j + 16 + 4*q4 ..
    bf16x8 qfp[NJ];
    {
        const int qr = row_ok ? n16 : 0;
        const bf16* qp = a.q + ((size_t)(req0 + qr / g) * a.h_q + h * g + qr % g) * D;
#pragma unroll
        for (int j = 0; j < NJ; ++j) qf[j] = ldg((const bf16x8*)(qp + 32 * j + 8 * q4));
        if constexpr (ROPE) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                qfp[j] = cat4(ldg((const bf16x4*)(qp + 32 * j + 4 * q4)),
                              ldg((const bf16x4*)(qp + 32 * j + 16 + 4 * q4)));
        }
    }

    // ---- B_k rows of one group of four requests (operands of the pre-projection
    // below).  With the agent table the first group's go out here, with the
    // query, ahead of the first step's cache loads: loads complete in issue
    // order, so the pre-projection then waits for neither the stream nor a
    // scalar round trip queued behind it.
    const size_t bcols = (size_t)a.h_kv * D;
    auto bk_issue = [&](const int s0, bf16x8 (&bk)[4][NRT][NJ]) __attribute__((always_inline)) {
        int agent[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) agent[u] = s0 == 0 ? agent0[u] : a.req_agent[req0 + min(s0 + u, nreq - 1)];
        asm volatile("" ::"s"(agent[0]), "s"(agent[1]), "s"(agent[2]), "s"(agent[3]));
#pragma unroll
        for (int u = 0; u < 4; ++u) sm_agent[s0 + u] = agent[u];  // s0 + u < 16: s0 < nreq <= 16
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int ag = min(max(agent[u], 0), a.n_agents - 1);
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                const int rank = 16 * rt + n16;
                const bf16* bp_ = a.b_k + ((size_t)ag * R + min(rank, R - 1)) * bcols + (size_t)h * D + 8 * q4;
#pragma unroll
                for (int j = 0; j < NJ; ++j) bk[u][rt][j] = ldg((const bf16x8*)(bp_ + 32 * j));
            }
        }
    };
    bf16x8 bk0[4][NRT][NJ];
    if constexpr (AGENT_TAB) bk_issue(0, bk0);

    // ---- then the first DEPTH-1 steps' loads, before the prologue's dependent chain
    StepT buf[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH - 1; ++i)
        if (i < NPRE) load(buf[i], pid[i]);
    StepRope<D> rope_buf;
    if constexpr (ROPE) load_rope(rope_buf, 0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- pre-projection qB = q B_k^(h)T, one MFMA tile per request of the group.
    // C lane layout: rank 16*rt + 4*q4 + v of row n16 — already the B operand
    // layout of the rank-r score MFMA.  The agent ids of up to four requests
    // are fetched together, then all their B_k rows: two memory round trips in
    // all, overlapping the first step's loads.
    f32x4 qbacc[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) qbacc[rt] = zf4();
    if constexpr (ROPE) {
        // ---- RoPE: stage B_k^(h)T of every request of the group in LDS as the A
        // operand of dK^T = B_k^(h)T L_k^T: entry (request u, dim tile, lane l)
        // holds dim 16*tile + l%16, ranks 4*(l/16) + v in slots 0-3 and
        // 16 + 4*(l/16) + v in slots 4-7 (rank 32 only) — the rank order of the
        // L_k operand.  Each thread fetches 16-byte pieces of B_k rows (8 dims of
        // one rank) for four requests at a time, then scatters them.
        constexpr int PIECES = R * D / 8;  // per request
        constexpr int PPT = (PIECES + 64 * WAVES - 1) / (64 * WAVES);
        // the angle-advance row: thread e < 8 * D / 32 fetches entry (ht, cos / sin,
        // q4) = (e / 8, (e / 4) % 2, e % 4)
        constexpr int ADV = WAVES * KEYS_PER_STEP;
        f32x4 radv = zf4();
        if constexpr (RADV) {
            const int e = min(tid, 8 * (D / 32) - 1);
            const float* tab = ((e >> 2) & 1) ? a.rope_sin : a.rope_cos;
            const uint32_t bytes = (uint32_t)max(a.rope_rows - ADV, 0) * (D / 2) * 4;
            const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(tab + (size_t)ADV * (D / 2)), (short)0, bytes, 0x00020000);
            radv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rt, (16 * (e >> 3) + 4 * (e & 3)) * 4, 0, 0));
        }
        for (int s0 = 0; s0 < nreq; s0 += 4) {
            int agent[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) agent[u] = s0 == 0 ? agent0[u] : a.req_agent[req0 + min(s0 + u, nreq - 1)];
            asm volatile("" ::"s"(agent[0]), "s"(agent[1]), "s"(agent[2]), "s"(agent[3]));
#pragma unroll
            for (int u = 0; u < 4; ++u) sm_agent[s0 + u] = agent[u];  // s0 + u < 16: s0 < nreq <= 16
            bf16x8 raw[4][PPT];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int ag = min(max(agent[u], 0), a.n_agents - 1);
#pragma unroll
                for (int k = 0; k < PPT; ++k) {
                    const int pc = min(tid + 64 * WAVES * k, PIECES - 1);
                    const int rank = pc / (D / 8), c0 = 8 * (pc % (D / 8));
                    raw[u][k] = ldg((const bf16x8*)(a.b_k + ((size_t)ag * R + rank) * bcols + (size_t)h * D + c0));
                }
            }
            __builtin_amdgcn_sched_barrier(0);  // every B_k load issued before the first wait
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
                for (int k = 0; k < PPT; ++k) {
                    const int pc = tid + 64 * WAVES * k;
                    if (s0 + u < nreq && pc < PIECES) {
                        const int rank = pc / (D / 8), c0 = 8 * (pc % (D / 8));
                        const int slot = (rank & 3) + (rank >= 16 ? 4 : 0);
                        const int grp = (rank & 15) >> 2;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int c = c0 + e;
                            char* ent = sm_bk + (((s0 + u) * NDT + (c >> 4)) * 64 + (c & 15) + 16 * grp) * BKW;
                            *(bf16*)(ent + 2 * slot) = raw[u][k][e];
                            // the zero slots: ranks 16.. (R < 32) and the k-groups
                            // R/4 .. 3 that hold no rank (R < 16; written by rank 0)
                            if (R < 32 && (rank & 3) == 0) *(bf16x4*)(ent + 8) = zero4();
                            if (R < 16 && rank == 0) {
#pragma unroll
                                for (int gz = R / 4; gz < 4; ++gz) *(bf16x8*)(ent + 16 * gz * BKW) = zero8();
                            }
                        }
                    }
                }
            }
        }
        if (RADV && tid < 8 * (D / 32)) sm_radv[tid >> 3][(tid >> 2) & 1][tid & 3] = radv;
        __syncthreads();
    } else {
    auto bk_mfma = [&](const int s0, const bf16x8 (&bk)[4][NRT][NJ]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                f32x4 c = zf4();
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    c = mfma16x16x32(16 * rt + n16 < R ? bk[u][rt][j] : zero8(), qf[j], c);
                if (n16 / g == s0 + u) qbacc[rt] = c;
            }
    };
    if constexpr (!AGENT_TAB) {
        bk_issue(0, bk0);
        __builtin_amdgcn_sched_barrier(0);  // every B_k load issued before the first wait
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) qf[j] = row_ok ? qf[j] : zero8();
    bk_mfma(0, bk0);
    for (int s0 = 4; s0 < nreq; s0 += 4) {
        bf16x8 bk[4][NRT][NJ];
        bk_issue(s0, bk);
        __builtin_amdgcn_sched_barrier(0);  // every B_k load issued before the first wait
        bk_mfma(s0, bk);
    }
    }
    bf16x8 qb;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        qb[v] = (bf16)qbacc[0][v];
        qb[4 + v] = (R == 32) ? (bf16)qbacc[NRT - 1][v] : (bf16)0.0f;
    }

    float m_run = -INFINITY;
    float l_run = 0.f;
    f32x4 acc[NDT];
    f32x4 acc_lr[NRT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = zf4();
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) acc_lr[rt] = zf4();
    const float sl2 = a.scale_log2;

    const int my_req = n16 / g;  // request (within the group) of this lane's row
    auto compute = [&](StepT& T, int key0) {
        f32x4 s[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            s[t] = zf4();
#pragma unroll
            for (int j = 0; j < NJ; ++j) s[t] = mfma16x16x32(T.k[t][j], qf[j], s[t]);
            if constexpr (MODE == MODE_SHARED) s[t] = mfma16x16x32(T.lk[0][t], qb, s[t]);
            if constexpr (PA && !ROPE) {
                // each request slot's LR rows meet only that request's rows
#pragma unroll
                for (int u = 0; u < NQ; ++u) s[t] = mfma16x16x32(T.lk[u][t], my_req == u ? qb : zero8(), s[t]);
            }
        }
        if constexpr (ROPE) {
            // adapter key term of each request: dK^T = B_k^(h)T L_k^T (lane =
            // token n16, dims 16*tile + 4*q4 + v), rotated by the token's
            // position, rounded to bf16, contracted with the query rows (all
            // rows computed, only the request's rows kept).  With per-agent LR
            // caches request slot u's own L_k rows are used.
            auto rebuild_req = [&](int u, const bf16x8 (&lkt)[2]) {
                const char* bkp = sm_bk + (u * NDT * 64 + lane) * BKW;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    f32x4 dk[NDT];
#pragma unroll
                    for (int tile = 0; tile < NDT; ++tile) {
                        const bf16x8 bop = *(const bf16x8*)(bkp + tile * 64 * BKW);
                        dk[tile] = mfma16x16x32(bop, lkt[t], zf4());
                    }
#pragma unroll
                    for (int ht = 0; ht < NDT / 2; ++ht) {
                        const f32x4 c = rope_buf.cs[t][ht][0], sn = rope_buf.cs[t][ht][1];
                        const f32x4 x1 = dk[ht], x2 = dk[ht + NDT / 2];
                        dk[ht] = x1 * c - x2 * sn;
                        dk[ht + NDT / 2] = x2 * c + x1 * sn;
                    }
                    f32x4 acc_u = s[t];
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        bf16x8 op;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            op[v] = (bf16)dk[2 * j][v];
                            op[4 + v] = (bf16)dk[2 * j + 1][v];
                        }
                        acc_u = mfma16x16x32(op, qfp[j], acc_u);
                    }
                    if (my_req == u) s[t] = acc_u;
                }
            };
            if constexpr (PA) {
                // at most NQ requests per row group (the plan's packing)
#pragma unroll
                for (int u = 0; u < NQ; ++u)
                    if (u < nreq) rebuild_req(u, T.lk[u]);
            } else {
                for (int u = 0; u < nreq; ++u) rebuild_req(u, T.lk[0]);
            }
        }
        // Tokens at or past the chunk end: score -inf, and their values zeroed
        // (unused page slots may hold anything, even NaN bits, and 0 * NaN is
        // NaN).  Branch-free on purpose: a branch here makes the compiler drain
        // every load in flight before the value MFMAs.
        float x[8];
        float mx = -INFINITY;
        uint32_t keep[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            bool ok[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                ok[v] = key0 + 16 * t + 4 * q4 + v < kend;
                const float val = ok[v] ? s[t][v] * sl2 : -INFINITY;
                x[4 * t + v] = val;
                mx = fmaxf(mx, val);
            }
            keep[t][0] = (ok[0] ? 0x0000ffffu : 0u) | (ok[1] ? 0xffff0000u : 0u);
            keep[t][1] = (ok[2] ? 0x0000ffffu : 0u) | (ok[3] ? 0xffff0000u : 0u);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // A step past the chunk end (all tokens dead) leaves the state as it
        // is: alpha = 1 and p = 0, also while nothing has been seen yet.
        const float m_new = fmaxf(m_run, mx);
        const bool none = m_new == -INFINITY;
        const float alpha = none ? 1.0f : fast_exp2(m_run - m_new);
        m_run = m_new;
        float ps = 0.f;
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = x[i] == -INFINITY ? 0.f : fast_exp2(x[i] - m_new);
            ps += p;
            pb[i] = (bf16)p;
        }
        l_run = l_run * alpha + ps;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) acc_lr[rt] *= alpha;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) T.v[t][dt] = and_mask(T.v[t][dt], keep[t][0], keep[t][1]);
#pragma unroll
            for (int u = 0; u < NQ; ++u)
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
                    T.lv[u][t][rt] = and_mask(T.lv[u][t][rt], keep[t][0], keep[t][1]);
        }
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            // per-agent LR caches: request slot u's L_v rows against its rows' P only
            const bf16x8 pu = (!PA || my_req == u) ? pb : zero8();
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                bf16x8 lvop = cat4(T.lv[u][0][rt], T.lv[u][1][rt]);
                if (16 * rt + n16 >= R) lvop = zero8();
                acc_lr[rt] = mfma16x16x32(lvop, pu, acc_lr[rt]);
            }
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[dt] = mfma16x16x32(cat4(T.v[0][dt], T.v[1][dt]), pb, acc[dt]);
    };

    // ---- streaming: the loads of steps i+1 .. i+DEPTH-1 are in flight while step i
    // computes (fully unrolled, so every buffer index is static and the step
    // buffers live in VGPRs/AGPRs without copies).
    // No branches in this loop and a scheduling barrier after each batch of
    // loads: the compiler may neither sink the loads towards their use nor
    // merge control flow (either makes it drain every load in flight).
    if constexpr (!ROPE) {
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            if (i + DEPTH - 1 < SPW) load(buf[(i + DEPTH - 1) % DEPTH], pid[i + DEPTH - 1]);
            __builtin_amdgcn_sched_barrier(0);
            compute(buf[i % DEPTH], kbeg + (wave + WAVES * i) * KEYS_PER_STEP);
        }
    } else {
        // RoPE: each step carries the per-request key rebuild, so the stream is a
        // runtime loop over step pairs (bounded registers and code size).  Loads
        // stay unconditional: past the last step they repeat it (never used).
        static_assert(DEPTH == 2 && SPW % 2 == 0, "RoPE stream: two step buffers, even step count");
        auto rstep = [&](int i, StepT& cur, StepT& nxt) {
            const int in = min(i + 1, SPW - 1);
            const int pn[2] = {page_now(in, 0), page_now(in, 1)};
            load(nxt, pn);
            __builtin_amdgcn_sched_barrier(0);
            compute(cur, kbeg + (wave + WAVES * i) * KEYS_PER_STEP);
            // cos / sin of the next step's keys: angle + WAVES * 32 positions
            if constexpr (!RADV) {
                load_rope(rope_buf, in);
            } else {
#pragma unroll
                for (int ht = 0; ht < D / 32; ++ht) {
                    const f32x4 ca = sm_radv[ht][0][q4], sa = sm_radv[ht][1][q4];
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const f32x4 c = rope_buf.cs[t][ht][0], sn = rope_buf.cs[t][ht][1];
                        rope_buf.cs[t][ht][0] = c * ca - sn * sa;
                        rope_buf.cs[t][ht][1] = sn * ca + c * sa;
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        };
#pragma unroll 1
        for (int i = 0; i < SPW; i += 2) {
            rstep(i, buf[0], buf[1]);
            rstep(i + 1, buf[1], buf[0]);
        }
    }
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    grab_next();

    // ---- merge the four wavefronts through LDS
    if constexpr (ROPE) __syncthreads();  // every B_k operand read before sm_o (same LDS) is written
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) *(f32x4*)&sm_o[wave][n16][16 * dt + 4 * q4] = acc[dt];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)  // ranks 16 rt + 4 q4 .. + 3 (R is a multiple of 4)
        if (16 * rt + 4 * q4 < R) *(f32x4*)&sm_o[wave][n16][D + 16 * rt + 4 * q4] = acc_lr[rt];
    if (q4 == 0) {
        sm_m[wave][n16] = m_run;
        sm_l[wave][n16] = l_run;
    }
    __syncthreads();

    // Thread (row n, phase cl) combines the wavefronts' partials for the
    // 16-byte column groups cl, cl + 16, ... of its row (every column belongs
    // to one thread) and keeps them in registers: the chunk partial goes to
    // the workspace straight from there, and the merging workgroup starts from
    // them.  static_assert: 256 threads = ROWS rows x 16 phases.
    static_assert(64 * WAVES == ROWS * 16, "one thread per (row, column phase)");
    const int n = tid >> 4;   // row handled by this thread in the epilogues
    const int cl = tid & 15;  // column phase
    constexpr int NG = MERGE_NG<DR>;
    f32x4 og[NG];
    float M = -INFINITY, L = 0.f;
    {
        float mw[WAVES];
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            mw[w] = sm_m[w][n];
            M = fmaxf(M, mw[w]);
        }
        float wt[WAVES];
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            wt[w] = (M == -INFINITY) ? 0.f : fast_exp2(mw[w] - M);
            L += wt[w] * sm_l[w][n];
        }
        // unrolled: the LDS reads of every column go out before the first wait
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            const int gi = min(cl + 16 * k, DR / 4 - 1);
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < WAVES; ++w) o += wt[w] * *(const f32x4*)&sm_o[w][n][4 * gi];
            og[k] = o;
        }
    }
    // the combined partial into LDS (columns 4 gi .. of this thread only), for
    // the epilogue of a unit of one chunk
    auto og_to_lds = [&]() {
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            const int gi = cl + 16 * k;
            if (gi < DR / 4) *(f32x4*)&sm_o[0][n][4 * gi] = og[k];
        }
        if (cl == 0) sm_L[n] = L;
    };

    // B_v^(h) columns of this thread's output row (agent ids from LDS, so one
    // memory round trip).  Only the workgroup that finalizes the unit needs
    // them: the merging one requests them together with the partials.
    BvCols<D, R> bvc;
    auto load_bv = [&]() {
        if (n < nrows) {
            const int agent = min(max(sm_agent[n / g], 0), a.n_agents - 1);
            const bf16* bv = a.b_v + (size_t)agent * R * a.h_kv * D + (size_t)h * D + cl * (D / 16);
#pragma unroll
            for (int t = 0; t < R; ++t)
                bvc.r[t] = ldg((const typename BvCols<D, R>::vec*)(bv + (size_t)t * a.h_kv * D));
        }
    };

    if (n_active > 1) {
        // ---- partial row -> workspace; the last workgroup of the unit merges.
        //
        // Cross-workgroup protocol without an L2 write-back.  Partial rows are
        // written with stores that carry the agent-coherence bit (sc1, what
        // agent-scope atomic stores use), and every wavefront waits until its
        // stores have completed (vmcnt(0): the store acknowledgements) before
        // the barrier; only then is the unit's counter bumped.  The workgroup
        // that sees the count reach n_active - 1 reads the other partials with
        // sc1 loads (agent-coherent, as agent-scope atomic loads).  A
        // workgroup-scope release would not wait for the acknowledgements, and
        // an agent-scope release would write back the whole L2 once per
        // workgroup, which serialises across the GPU.
        constexpr int PW = DR + 4;
        // buffer descriptors must be wave-uniform (scalar registers): a
        // per-lane base makes the compiler loop over the distinct values
        // ("waterfall"), so the row goes into the per-lane offset
        const int unit_s = __builtin_amdgcn_readfirstlane(unit);
        const int split_s = __builtin_amdgcn_readfirstlane(split);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            a.ws_part + ((size_t)unit_s * a.n_split + split_s) * ROWS * PW, (short)0, ROWS * PW * 4, 0x00020000);
        if (n < nrows) {
#pragma unroll
            for (int k = 0; k < NG; ++k) {
                const int gi = cl + 16 * k;  // 16-byte group of the row: columns 4 gi .. 4 gi + 3, then (m, l)
                if (gi <= DR / 4) {
                    const f32x4 v = gi < DR / 4 ? og[k] : f32x4{M, L, 0.f, 0.f};
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, (n * PW + 4 * gi) * 4, 0, CPOL_SC1);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(WAITCNT_VMCNT0);
        __syncthreads();
        if (tid == 0) {
            const int prev = __hip_atomic_fetch_add(a.ws_count + unit, 1, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
            sm_last = prev == n_active - 1;
        }
        __syncthreads();
        if (!sm_last) return;
        load_bv();
        merge_partials<D, R, SP, NG>(a, unit_s, split_s, n_active, nrows, n, cl, og, M, L, sm_o[0], sm_L);
        if (tid == 0) __hip_atomic_store(a.ws_count + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        load_bv();
        og_to_lds();
    }
    __syncthreads();
    finalize_rows<D, R, SP>(a, sm_o[0], sm_L, n, cl, nrows, req0, h, bvc);
    };

    if (!a.persistent) {
        // one item per workgroup.  XCD-aware placement: workgroup b runs on XCD
        // b % 8; remap so that the KV heads and row groups of one (context,
        // chunk) — which share its L_k/L_v pages, and per head its K/V pages —
        // are consecutive on one XCD and hit the same L2 at about the same time.
        const int nb = gridDim.x;
        const int b = blockIdx.x;
        const int bp = (b & 7) * (nb >> 3) + (b >> 3);
        const int h = bp % a.h_kv;
        int rest = bp / a.h_kv;
        const int rg = rest % a.n_rg;
        rest /= a.n_rg;
        const int split = rest % a.n_split;
        const int ctx = rest / a.n_split;
        if (ctx < a.n_ctx) process(ctx, rg, h, split, nullptr, nullptr);
        return;
    }

    // ---- persistent: one workgroup per CU pulls items from a queue in the
    // workspace.  Items are only the chunks that exist (a context of length len
    // has ceil(len / CHUNK) chunks per row group and KV head; an empty one has
    // one item, which writes its zero rows), enumerated context by context,
    // then chunk, row group, head.  The next item's index is requested when an
    // item's streaming ends, so the queue's round trip overlaps its merge tail.
    int* queue = a.ws_count + a.n_units;  // [0] next item, [1] workgroups done
    if (wave == 0) {
        int run = 0;
        for (int base = 0; base < a.n_ctx; base += 64) {
            const int c = base + lane;
            int v = 0;
            if (c < a.n_ctx) {
                const int len = min(min(a.ctx_len[c], a.max_blocks * PAGE), a.max_len);
                v = (len > 0 ? (len + CHUNK - 1) / CHUNK : 1) * a.n_rg * a.h_kv;
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int t = __shfl_up(v, off);
                if (lane >= off) v += t;
            }
            if (c < a.n_ctx) sm_pref[c + 1] = run + v;
            run += __shfl(v, 63);
        }
        if (lane == 0) {
            sm_pref[0] = 0;
            sm_item = __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    const int total = sm_pref[a.n_ctx];
    int item = sm_item;
    while (item < total) {
        int next = total;
        int ctx = 0;
        for (int base = 0; base < a.n_ctx; base += 64) {
            const int c = base + lane;
            const bool hit = c < a.n_ctx && sm_pref[c] <= item && item < sm_pref[c + 1];
            const unsigned long long m = __builtin_amdgcn_ballot_w64(hit);
            if (m != 0) {
                ctx = base + __builtin_ctzll(m);
                break;
            }
        }
        ctx = __builtin_amdgcn_readfirstlane(ctx);
        const int local = item - sm_pref[ctx];
        const int h = local % a.h_kv;
        const int rest = local / a.h_kv;
        process(ctx, rest % a.n_rg, h, rest / a.n_rg, queue, &next);
        __syncthreads();  // every thread is done with this item's LDS
        if (tid == 0) sm_item = next;
        __syncthreads();
        item = sm_item;
    }
    // the last workgroup out resets the queue (no grab can follow: every
    // workgroup's final grab returned before it got here)
    if (tid == 0) {
        const int done = __hip_atomic_fetch_add(queue + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == (int)gridDim.x - 1) {
            __hip_atomic_store(queue, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(queue + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Log-sum-exp merge of the chunk partials of one work unit into o[row][0..DR)
// and L[row].  Runs in the last workgroup to finish, whose own partial (chunk
// `own`) is still in registers (own_o: this thread's column groups, own_m,
// own_l) and is taken from there; the others are read from the workspace.  Chunks are combined in chunk order whichever
// workgroup merges, so repeated calls give identical bits.  Thread (row n,
// phase cl) owns the 16-byte column groups cl, cl + 16, ... of the row and
// reads every partial's (m, l); the partials of up to GB chunks are requested
// together, so a merge of <= GB chunks waits for one memory round trip.
template <int D, int R, int SP, int NG>
__device__ __forceinline__ void merge_partials(const DecodeK& a, int unit, int own, int n_active, int nrows,
                                               int n, int cl, const f32x4 (&own_o)[NG], float own_m,
                                               float own_l, float (*o)[SP], float* L_row) {
    constexpr int DR = D + R;
    constexpr int PW = DR + 4;
    static_assert(NG == MERGE_NG<DR>, "column groups per thread");
    constexpr int GB = 8;  // chunks per batch
    // `unit` and `own` are wave-uniform (scalar): the descriptor stays in
    // scalar registers and the row is part of the per-lane offset
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        a.ws_part + (size_t)unit * a.n_split * ROWS * PW, (short)0,
        (uint32_t)((size_t)a.n_split * ROWS * PW * 4), 0x00020000);
    if (n >= nrows) return;
    const uint32_t sstride = ROWS * PW * 4;  // bytes between chunks
    const uint32_t row_off = (uint32_t)n * PW * 4;
    // the own partial, in the layout of a loaded one
    const f32x4 own_ml = f32x4{own_m, own_l, 0.f, 0.f};
    float M = -INFINITY, L = 0.f;
    f32x4 acc[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int g0 = 0; g0 < n_active; g0 += GB) {
        f32x4 ml[GB], ov[GB][NG];
#pragma unroll
        for (int u = 0; u < GB; ++u) {
            // chunks past n_active re-read the own slot (weight 0); the own
            // chunk's loaded values are replaced by the LDS ones
            const int c = g0 + u < n_active ? g0 + u : own;
            ml[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, c * sstride + row_off + 16 * (DR / 4), 0, CPOL_SC1));
#pragma unroll
            for (int k = 0; k < NG; ++k)
                ov[u][k] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, c * sstride + row_off + 16 * min(cl + 16 * k, DR / 4 - 1), 0, CPOL_SC1));
        }
#pragma unroll
        for (int u = 0; u < GB; ++u) {
            if (g0 + u == own) {
                ml[u] = own_ml;
#pragma unroll
                for (int k = 0; k < NG; ++k) ov[u][k] = own_o[k];
            }
        }
        float mv[GB];
#pragma unroll
        for (int u = 0; u < GB; ++u) mv[u] = g0 + u < n_active ? ml[u][0] : -INFINITY;
        float M_new = M;
#pragma unroll
        for (int u = 0; u < GB; ++u) M_new = fmaxf(M_new, mv[u]);
        const float resc = M == -INFINITY ? 0.f : fast_exp2(M - M_new);
        L *= resc;
#pragma unroll
        for (int k = 0; k < NG; ++k) acc[k] *= resc;
#pragma unroll
        for (int u = 0; u < GB; ++u) {
            const float w = mv[u] == -INFINITY ? 0.f : fast_exp2(mv[u] - M_new);
            L += w * ml[u][1];
#pragma unroll
            for (int k = 0; k < NG; ++k) acc[k] += w * ov[u][k];
        }
        M = M_new;
    }
#pragma unroll
    for (int k = 0; k < NG; ++k) {
        const int gi = cl + 16 * k;
        if (gi < DR / 4) {
            *(f32x4*)&o[n][4 * gi] = acc[k];
        }
    }
    if (cl == 0) L_row[n] = L;
}

// O = (O_base + O_lr B_v^(h)) / l for the rows of one work unit: the single
// post-multiplication by B_v per query row.  `o` holds [O_base | O_lr] per row;
// thread (n, cl) owns D/16 contiguous output columns (one vector store).
template <int D, int R, int SP>
__device__ __forceinline__ void finalize_rows(const DecodeK& a, const float (*o)[SP], const float* L_row,
                                              int n, int cl, int nrows, int req0, int h,
                                              const BvCols<D, R>& bv) {
    if (n >= nrows) return;
    constexpr int CPT = D / 16;
    const int g = a.g;
    const int req = req0 + n / g;
    const float L = L_row[n];
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    const int c0 = cl * CPT;
    // 16-byte LDS reads: the row pitch is a multiple of 4 floats, c0 of CPT
    float acc[CPT];
#pragma unroll
    for (int k = 0; k < CPT; k += 4) {
        const f32x4 v = *(const f32x4*)&o[n][c0 + k];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[k + e] = v[e];
    }
#pragma unroll
    for (int t4 = 0; t4 < R; t4 += 4) {
        const f32x4 w4 = *(const f32x4*)&o[n][D + t4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int k = 0; k < CPT; ++k) acc[k] += w4[e] * (float)bv.r[t4 + e][k];
    }
    typename BvCols<D, R>::vec res;
#pragma unroll
    for (int k = 0; k < CPT; ++k) res[k] = (bf16)(acc[k] * inv);
    *(typename BvCols<D, R>::vec*)(a.out + ((size_t)req * a.h_q + h * g + n % g) * D + c0) = res;
}

template <int D, int R, int SPW, int MODE>
lra_status launch_t(const lra::DecodeArgs& a, const lra::DecodePlan& p, hipStream_t s) {
    constexpr int DEPTH = 2;  // one step of loads in flight per wavefront
    constexpr int W = 4;      // wavefronts per workgroup
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
    k.n_units = p.n_units;
    k.n_req = a.n_req;
    k.persistent = p.persistent;
    k.scale_log2 = a.scale * LRA_LOG2E;
    k.rope_cos = a.rope_cos;
    k.rope_sin = a.rope_sin;
    k.rope_rows = a.rope_rows;
    k.max_len = a.max_ctx_len;
    k.lr_stride = a.lr_stride;
    int grid = p.grid;
    if (p.persistent) {
        // one workgroup per CU of the current device
        int dev = 0, n_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0) {
            lra::set_error("decode: cannot query the device's compute units");
            return LRA_ERR_HIP;
        }
        grid = min(n_cu, p.grid);
    }
    hipLaunchKernelGGL((lra_decode_bf16_kernel<D, R, SPW, DEPTH, W, MODE>), dim3(grid), dim3(64 * W), 0, s, k);
    return lra::check_launch("lra_decode_bf16_kernel");
}

template <int D, int R, int MODE>
lra_status launch_dr(const lra::DecodeArgs& a, const lra::DecodePlan& p, hipStream_t s) {
    // chunk = 4 wavefronts x SPW steps x 32 tokens
    switch (p.chunk) {
        case 256: return launch_t<D, R, 2, MODE>(a, p, s);
        case 512: return launch_t<D, R, 4, MODE>(a, p, s);
        case 1024: return launch_t<D, R, 8, MODE>(a, p, s);
        case 2048: return launch_t<D, R, 16, MODE>(a, p, s);
        case 4096: return launch_t<D, R, 32, MODE>(a, p, s);
        default: break;
    }
    lra::set_error("decode: unsupported chunk %d", p.chunk);
    return LRA_ERR_UNSUPPORTED;
}

}  // namespace

