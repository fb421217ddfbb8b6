// Chunked-prefill Flash-LoRA-Attention, bf16 storage / fp32 accumulation, gfx950.
//
// What is computed (LRAgent, arXiv 2602.01053v2, §3, App. B, App. D.1): every
// new token i of a request (position kv_len - q_len + i) attends causally to
// the shared base cache and the shared rank-r LR cache through its agent's
// B_k, B_v:
//
//   without RoPE on the adapter key:  s_j = q . k_base_j + (q B_k^(h)T) . l_k_j
//   with RoPE:                         s_j = q . (k_base_j + rot_j(l_k_j B_k^(h)))
//   O = (sum_j p_j v_base_j + (sum_j p_j l_v_j) B_v^(h)) / sum_j p_j
//
// The value side always stays at rank r until one post-multiplication by B_v
// per row.  With RoPE the position-dependent rotation blocks the reordering on
// the key side (App. D.1), so the adapted key tile is rebuilt at head dimension
// in LDS, once per (workgroup, key tile), and never written to HBM.
//
// Decomposition: a workgroup = (request, KV head h, block of 8*TW new tokens);
// its 8 wavefronts each own 32 rows = TW tokens x g query heads of h (GQA
// packing: one K/V tile serves all g heads).  All products run on
// v_mfma_f32_32x32x16_bf16:
//
//   S^T[key][row]  = K[key][dim] . Q^T[dim][row]  (+ L_k . qB^T, rank r)
//   O^T[dim][row] += V^T[dim][key] . P^T[key][row]
//   O_lr^T[rank][row] += L_v^T[rank][key] . P^T[key][row]   (+ a ones row: sum_j p_j)
//   O^T           += B_v^T[dim][rank] . O_lr^T[rank][row]  (epilogue)
//
// Key order inside a 32-key score tile: MFMA row m of S^T holds key sigma(m),
// m with bits 2 and 3 swapped (the K operand rows are read in that order).  The
// accumulator layout (lane = row l%32, M rows 8*(v/4) + 4*(l/32) + v%4) then
// gives the lane of k-group hh, in P^T slot e of k-step ks, key 16*ks + 8*hh + e:
// P stays in registers as the B operand of the value products, and each lane's
// V^T / L_v^T operand is 8 consecutive keys.  From the row-major LDS tiles
// those come through the gfx950 transposing read ds_read_b64_tr_b16 (16 lanes
// turn a 4 x 16 block into 16 columns of 4); from the dim-major tiles of the
// paged mode they are one 16-byte row read.
//
// Data movement.  64-key tiles go HBM -> LDS by buffer_load ... lds (no
// register staging): one instruction moves 1 KB, lane i's 16 bytes landing at
// 16*i, and keys past kv_len read as zero through the buffer range.  Each 1 KB
// block of a K / V tile (and of the cos / sin rows of key offsets 0..63) holds
// the rows key = i + NI*m of block i,
// and consecutive blocks sit 1040 B (K, cos, sin) or 1088 B (V) apart: that
// spreads the 16 rows a 16-lane row read touches over all 64 banks, and the
// 4 rows of a transposing read over the four 64-byte bank quarters, with LDS
// addresses that stay linear in the key (one base register per operand).
// L tiles are chunk-major ([16-byte rank chunk][key]); the L_v tile carries
// constant chunks after the ranks (the ones row, zeros) written once.
//
// Paged mode: the caches are page pools (16 tokens a page) reached through one
// context's block table, read in place.  A 64-key tile is 4 pages, gathered by
// global_load_lds_dwordx4 (each lane its own 64-bit address, so one 1 KB block
// can draw on 4 pages); every DMA reads runs of 256 contiguous bytes or more of
// a page.  The K tile is chunk-major in LDS ([8-dim chunk][key], as the L
// tiles), matching the page's [d/8][16 keys][8] order.  V and L_v pages are
// dim- / rank-major ([dim][16 keys]) in HBM and stay so in LDS: [page][dim][key
// half][8 keys], the two halves of a dim swapped when its bit 3 is set (16
// lanes reading one half of 16 dims then meet 16 different bank groups); one
// 16-byte LDS read per operand, no transposing read.  Lanes of L_v^T past the
// rank read a constant region of ones (the ones row gives the row sums; the
// other rows are never used).  Pages past the context read page 0 and their
// keys, like every key past kv_len, are masked in the scores; the value rows
// of those keys are zeroed in LDS after the DMA (a pool may hold any bits
// there), so the results equal those of the contiguous mode bit for bit.
//
// Pipeline per tile t: K is loaded two tiles ahead and V one tile ahead, so
// S(t+1) is on the matrix cores while the softmax of S(t) runs on the VALU,
// followed by P(t)V(t) with the row max of S(t+1) in its shadow; one barrier
// per tile.  With RoPE, K is loaded three tiles ahead into a ring of three
// buffers and each raw tile is rebuilt in place (K' = K_base + rot(L_k B_k))
// in the step before its score MFMAs; the rotation angle of a key is that of
// its tile's first position plus that of its offset in the tile (angle
// addition from cos / sin rows held in LDS and registers).
#include <algorithm>
#include <type_traits>

#include "lra_common.h"
#include "lra_internal.h"

namespace {

constexpr int WAVES = 8;
constexpr int KT = 64;  // keys per tile

struct PrefillK {
    const bf16* q;
    const int32_t* req_agent;
    const bf16* k_base;
    const bf16* v_base;
    const bf16* l_k;
    const bf16* l_v;
    const bf16* b_k;
    const bf16* b_v;
    const float* rope_cos;
    const float* rope_sin;
    bf16* out;
    int32_t n_req, q_len, kv_len, n_agents, h_q, h_kv, g, n_qblk;
    float scale_log2;
    int64_t lr_stride;  // per-agent LR caches: elements between agents' caches (0: shared)
    int64_t kv_req_stride;  // plain mode: elements between requests' K / V caches
    // paged mode: k_base / v_base / l_k / l_v are the page pools
    const int32_t* block_table;  // the context's row: page of tokens 16 b .. 16 b + 15
    int32_t n_blk;               // entries in use: min(max_blocks, ceil(kv_len / 16))
    int32_t n_pages;
    uint32_t page_bytes;         // bytes per page of the K / V pools (all heads)
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Transposing LDS read: the 16 lanes of a group each name one 8-byte row piece
// (lane a + 4*s -> row k0+s, columns n0+4a .. n0+4a+3); lane i of the group
// receives column n0+i of rows k0 .. k0+3.
LRA_DEV bf16x4 lds_read_tr(const char* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// The same with 4 bytes per lane (lane i -> lds + 4 i): the rank-4 L rows, 8
// bytes each, spread over 16-byte LDS slots.
LRA_DEV void dma_256(u32x4 r, uint32_t lds, uint32_t voff) {
    uint32_t keep;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(keep)
        : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(r)
        : "memory");
}

// Gathers into LDS (global_load_lds_dwordx4 / _dword): lane i reads 16 (4)
// bytes at its own 64-bit address src; they land at lds + 16*i (4*i).
LRA_DEV void dma_g16(uint32_t lds, const void* src) {
    uint32_t keep;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(keep)
        : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src)
        : "memory");
}

LRA_DEV void dma_g4(uint32_t lds, const void* src) {
    uint32_t keep;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(keep)
        : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src)
        : "memory");
}

// s_waitcnt vmcnt(0): this wavefront's LDS DMA has landed.
LRA_DEV void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// v_max3_f32 (operands are finite or -inf; no NaN canonicalisation needed)
LRA_DEV float max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// PLAIN (measurement baseline only): plain attention over per-request K / V
// caches kv_req_stride elements apart, with no low-rank terms (L, B unused); the
// row sums still come from the ones row of the value-side tile.
// PAGED: the caches are read from page pools through a block table.
template <int D, int R, bool ROPE, bool PLAIN, bool PAGED>
__global__ __launch_bounds__(512) void lra_prefill_bf16_kernel(PrefillK a) {
    constexpr int RB = 2 * D;                 // bytes per K / V row (and per cos / sin row)
    constexpr int CPR = D / 8;                // 16-byte chunks per row
    constexpr int NI = KT * RB / 1024;        // 1 KB blocks per tile
    constexpr int NU = NI / WAVES;            // blocks per wavefront per tile
    constexpr int KBS = 1024 + 16;            // block stride: K, cos, sin
    constexpr int VBS = 1024 + 64;            // block stride: V, L_v chunks
    constexpr int TC = NI * KBS;              // cos / sin table of 64 key offsets
    // K tile: row blocks as above; paged: chunk-major [dim chunk][key][8 dims] (NI chunks)
    constexpr int TK = PAGED ? NI * 1024 : NI * KBS;
    // paged V tile: [page][key half][dim][8 keys], 1 KB blocks back to back
    constexpr int TV = PAGED ? NI * 1024 : NI * VBS;
    constexpr int RW = R < 16 ? 16 : R;       // ranks held per L row (zero padded)
    constexpr int NKS = D / 16;               // k-steps over head dim
    constexpr int NDT = D / 32;               // 32-wide dim tiles
    constexpr int NKR = RW / 16;              // k-steps over rank
    // 16-byte rank chunks of an L tile that come from HBM (rank 4: one chunk,
    // ranks 4-7 zero); the ones row is the first rank of the next chunk
    constexpr int RCH = PLAIN ? 0 : (R < 8 ? 1 : R / 8);
    constexpr int ONES_RANK = 8 * RCH;        // = R for R >= 8
    constexpr int NLT = (ONES_RANK + 1 + 31) / 32;  // rank tiles of O_lr incl. the ones row
    constexpr int ONES_T = ONES_RANK / 32;    // tile holding the ones row
    constexpr int ONES_M = ONES_RANK % 32;    // its row inside the tile
    constexpr int NLK = PLAIN ? 0 : RW / 8;   // L_k chunks held
    constexpr int NLV = 4 * NLT;              // L_v chunks held (ranks, ones row, zeros)
    constexpr int TLK = NLK * 1024;
    // paged L_v tile: the DMA'd blocks (at least one) of [page][rank][key half],
    // then 1 KB of ones read by the lanes past the rank
    constexpr int NLVB = R < 8 ? 1 : R / 8;   // paged: L_v DMA blocks per tile
    constexpr int LVD = NLVB * 1024;          // paged: offset of the ones region
    constexpr int TLV = PAGED ? LVD + 1024 : NLV * VBS;
    // K / L_k tile buffers: two, or with RoPE a ring of three (a raw key tile is
    // rebuilt in place one step before the step whose score MFMAs read it)
    constexpr int NKB = ROPE ? 3 : 2;
    constexpr int OFF_K = 0;
    constexpr int OFF_V = OFF_K + NKB * TK;
    constexpr int OFF_LK = OFF_V + 2 * TV;
    constexpr int OFF_LV = OFF_LK + NKB * TLK;
    constexpr int OFF_CS = OFF_LV + 2 * TLV;  // RoPE: cos / sin of key offsets 0..63 (whole kernel)
    constexpr int OFF_CB = OFF_CS + 2 * TC;   // RoPE: cos / sin rows of each tile's first key, ring of 3
    constexpr int LDS_BYTES = ROPE ? OFF_CB + NKB * 2048 : OFF_CS;
    constexpr int KMT = PAGED ? 512 : (32 / NI) * RB;  // K tile offset of keys 32..63
    constexpr int KKS = PAGED ? 2048 : 32;    // K tile offset of the next 16 dims
    constexpr int VKS = (D == 128) ? RB : 2 * RB;   // V offset of the next 16 keys
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    static_assert((R % 8 == 0 && R <= 32) || R == 4, "rank 4, 8, 16, 24 or 32");
    static_assert(NU >= 1 && NI % WAVES == 0, "tile blocks divide over the wavefronts");
    static_assert(RCH <= 4, "L_v DMA uses wavefronts 4..7");
    static_assert(!(PLAIN && ROPE), "the plain baseline takes pre-rotated keys");
    static_assert(!(PLAIN && PAGED), "the plain baseline reads contiguous caches");
    static_assert(NLVB <= 4, "paged L_v DMA uses wavefronts 4..7");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
    const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n32 = lane & 31;  // row of this lane (S^T / O^T column)
    const int hh = lane >> 5;   // k-group of this lane
    const int i16 = lane & 15;  // lane inside its 16-lane group (transposing reads)
    const int g16 = lane >> 4;  // 16-lane group
    const int sa = i16 & 3;     // transposing read: 8-byte piece
    const int ss = i16 >> 2;    // transposing read: row

    const int g = a.g;
    const int TW = 32 / g;  // tokens per wavefront
    // Work item: KV head outermost, then request, then query block.  Workgroup b
    // runs on XCD b % 8, one workgroup per CU.  With RoPE, or a grid of one
    // round (at most 256 workgroups), and a grid that divides by 8, XCD x takes
    // the x-th eighth of the items, so the workgroups that stream one head's K /
    // V tiles (every request and query block of it) share one XCD's L2.  A grid
    // of many rounds without RoPE goes in plain order: all XCDs stream the same
    // head at about the same time, so a long context's K / V of one head (69 MB
    // at 135168 tokens) is served by the 256 MB Infinity Cache instead of eight
    // heads at once (the 8-agent 4096 x 135168 prefill: 0.6-0.8% faster than an
    // eighth of the grid or of each round per XCD, 30% fewer L2 misses).
    const int nb = gridDim.x;
    const int bi = blockIdx.x;
    const int bp = ((nb & 7) == 0 && (ROPE || nb <= 256)) ? (bi & 7) * (nb >> 3) + (bi >> 3) : bi;
    const int qb = bp % a.n_qblk;
    const int req = (bp / a.n_qblk) % a.n_req;
    const int h = bp / (a.n_qblk * a.n_req);
    const int tok_wg = qb * WAVES * TW;
    const int q_len = a.q_len, kv_len = a.kv_len;
    int agent = a.req_agent[req];
    agent = min(max(agent, 0), a.n_agents - 1);
    // the LR cache this request reads: the shared one, or its agent's
    const bf16* lk_ag = a.l_k + (size_t)agent * a.lr_stride;
    const bf16* lv_ag = a.l_v + (size_t)agent * a.lr_stride;

    // this lane's row: token tok (chunk-local), query head h*g + (n32 % g)
    const int tok = tok_wg + wave * TW + n32 / g;
    const bool row_ok = tok < q_len;
    const int qpos = row_ok ? kv_len - q_len + tok : -1;  // absolute position (causal bound)
    const int hq = h * g + n32 % g;

    // keys needed by the workgroup: up to the last valid token's position
    const int last_tok = min(q_len - 1, tok_wg + WAVES * TW - 1);
    const int n_tiles = (kv_len - q_len + last_tok) / KT + 1;

    // contiguous: head h's [kv_len, D] rows; paged: head h's [D/8 or D, 16] part
    // of a page (the page itself is added per tile)
    const size_t hstride = PAGED ? (size_t)16 * D : (size_t)kv_len * D;
    const bf16* kb = a.k_base + (size_t)req * a.kv_req_stride + (size_t)h * hstride;
    const bf16* vb = a.v_base + (size_t)req * a.kv_req_stride + (size_t)h * hstride;

    // ---- HBM -> LDS tile DMA.  Block i of a K / V / cos / sin tile: lane l carries
    // row key = i + NI*(l / CPR), chunk l % CPR.  L chunk c: lane l carries key l.
    uint32_t voff_row[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u)
        voff_row[u] = (uint32_t)((wave + WAVES * u) + NI * (lane / CPR)) * RB + (lane % CPR) * 16;
    const uint32_t voff_l = (uint32_t)lane * (2 * R);
    // rank 4: dword DMA j (of 4) fills keys 16j .. 16j+15; lane -> key 16j + lane/4,
    // dword lane%4 of its 16-byte slot: the row's two dwords, then two zeros
    // (an offset past every buffer range reads as zero)
    const uint32_t voff_l4 = (lane & 3) < 2 ? (uint32_t)(lane >> 2) * 8 + 4 * (lane & 3) : 0x80000000u;

    // ---- paged mode: page ids.  Lane l holds the id of page l / 16 of a tile: every
    // paged DMA gives lanes 16p .. 16p+15 page p's bytes.  The raw entries a step
    // uses are loaded (from the cached block table) one step ahead, and nothing
    // reads them before that step: a use right after the load would wait for the
    // tile DMAs issued with it.  Pages past the context take the context's last
    // block (their keys are masked, their value rows zeroed); ids outside the pool
    // are clamped.
    auto pid_load = [&](int T) { return a.block_table[min(4 * T + (lane >> 4), a.n_blk - 1)]; };
    auto pid_use = [&](int raw) {
        asm volatile("" : "+v"(raw));
        return min(max(raw, 0), a.n_pages - 1);
    };
    // per-lane byte offsets inside a page (the tile and the page id add to them):
    // K block c (= wave + 8u): dims 8c.. of slot (lane % 16), 256 contiguous bytes
    // per page; V block i: page-local slots 16 i + lane % 16; L_v block c likewise
    const int q16 = lane & 15;
    const int kg_lane = q16 * 16 + wave * 256;
    const int vg_lane = (8 * wave + (q16 >> 1)) * 32 + ((q16 & 1) ^ (wave & 1)) * 16;
    const int lvg_c = max(wave - 4, 0);
    const int lvg_q = R < 8 ? (q16 & 7) : q16;  // rank 4: 8 slots a page, lanes 8.. repeat
    const int lvg_lane = (8 * lvg_c + (lvg_q >> 1)) * 32 + ((lvg_q & 1) ^ (lvg_c & 1)) * 16;
    // Paged V / L_v tiles: page-local slot s of page p (s = 2 * dim + stored half)
    // sits in block s / 16 at 256 p + 16 (s % 16); the stored half is the key half
    // hv ^ bit 3 of the dim (rank), so that 16 lanes reading one half of 16
    // consecutive dims hit 16 different bank groups.  Source half of slot s:
    auto vhalf = [](int s) { return (s & 1) ^ ((s >> 4) & 1); };

    auto dma_k = [&](int T, int b, int pid) {
        const int key0 = T * KT;
        const uint32_t rem = (uint32_t)(kv_len - key0);
        if constexpr (PAGED) {
            // K block c = dims 8c .. 8c+7 of the tile's 64 keys: lane l reads key l
            // (page l / 16, slot l % 16)
            const char* kp = (const char*)kb + (uint64_t)(uint32_t)pid * a.page_bytes + kg_lane;
#pragma unroll
            for (int u = 0; u < NU; ++u)
                dma_g16(smem_lds + OFF_K + b * TK + (wave + WAVES * u) * 1024, kp + WAVES * u * 256);
            // L_k [page][16 keys][R]: chunk c of key l (page l / 16) lands at 16 l of chunk c
            if constexpr (R < 8) {
                if (wave < 4) {
                    const int pj = __builtin_amdgcn_readlane(pid, 16 * wave);
                    // lanes 4k+2, 4k+3 repeat the row's two dwords (ranks 4..7 meet zero qB / B_k)
                    dma_g4(smem_lds + OFF_LK + b * TLK + wave * 256,
                           (const char*)lk_ag + (uint64_t)(uint32_t)pj * (32 * R) + (lane >> 2) * 8 + 4 * (lane & 1));
                }
            } else if (wave < RCH) {
                dma_g16(smem_lds + OFF_LK + b * TLK + wave * 1024,
                        (const char*)lk_ag + (uint64_t)(uint32_t)pid * (32 * R) + (lane & 15) * (2 * R) + 16 * wave);
            }
        } else {
            const auto rk = make_rsrc(kb + (size_t)key0 * D, rem * RB);
#pragma unroll
            for (int u = 0; u < NU; ++u) dma_1k(rk, smem_lds + OFF_K + b * TK + (wave + WAVES * u) * KBS, voff_row[u]);
            if constexpr (PLAIN) {
            } else if constexpr (R < 8) {
                if (wave < 4)
                    dma_256(make_rsrc(lk_ag + (size_t)(key0 + 16 * wave) * R,
                                      (uint32_t)max((int)rem - 16 * wave, 0) * (2 * R)),
                            smem_lds + OFF_LK + b * TLK + wave * 256, voff_l4);
            } else if (wave < RCH) {
                dma_1k(make_rsrc(lk_ag + (size_t)key0 * R, rem * (2 * R)), smem_lds + OFF_LK + b * TLK + wave * 1024,
                       voff_l + 16 * wave);
            }
        }
        if constexpr (ROPE) {
            // The cos / sin rows of the tile's first key.  Lanes 0 .. CPR-1 of the K
            // offsets voff_row[0] read row `wave` of a resource, so the resource
            // starts `wave` rows before row key0 (only the first RB bytes of each
            // 1 KB block are used).
            if (wave >= WAVES - 2) {
                const float* tab = wave == WAVES - 2 ? a.rope_cos : a.rope_sin;
                const uintptr_t base = (uintptr_t)(tab + (size_t)key0 * (D / 2)) - (uintptr_t)wave * RB;
                dma_1k(make_rsrc((const void*)base, (rem + wave) * RB),
                       smem_lds + OFF_CB + b * 2048 + (wave - (WAVES - 2)) * 1024, voff_row[0]);
            }
        }
    };
    auto dma_v = [&](int T, int b, int pid) {
        const int key0 = T * KT;
        const uint32_t rem = (uint32_t)(kv_len - key0);
        const int c = wave - 4;
        if constexpr (PAGED) {
            const char* vp = (const char*)vb + (uint64_t)(uint32_t)pid * a.page_bytes + vg_lane;
#pragma unroll
            for (int u = 0; u < NU; ++u)
                dma_g16(smem_lds + OFF_V + b * TV + (wave + WAVES * u) * 1024, vp + WAVES * u * 256);
            if (c >= 0 && c < NLVB)
                dma_g16(smem_lds + OFF_LV + b * TLV + c * 1024,
                        (const char*)lv_ag + (uint64_t)(uint32_t)pid * (32 * R) + lvg_lane);
        } else {
            const auto rv = make_rsrc(vb + (size_t)key0 * D, rem * RB);
#pragma unroll
            for (int u = 0; u < NU; ++u) dma_1k(rv, smem_lds + OFF_V + b * TV + (wave + WAVES * u) * VBS, voff_row[u]);
            if constexpr (PLAIN) {
            } else if constexpr (R < 8) {
                if (c >= 0)
                    dma_256(make_rsrc(lv_ag + (size_t)(key0 + 16 * c) * R,
                                      (uint32_t)max((int)rem - 16 * c, 0) * (2 * R)),
                            smem_lds + OFF_LV + b * TLV + c * 256, voff_l4);
            } else if (c >= 0 && c < RCH) {
                dma_1k(make_rsrc(lv_ag + (size_t)key0 * R, rem * (2 * R)), smem_lds + OFF_LV + b * TLV + c * VBS,
                       voff_l + 16 * c);
            }
        }
    };
    // paged: the value rows (V, L_v) of keys past kv_len in the tile holding
    // kv_len, zeroed after this wavefront's own DMA of them has landed
    auto zero_dead = [&](int T, int b) {
        const int live = kv_len - T * KT;
        auto fix = [&](int off, int k0) {
            if (k0 + 8 > live) {
                bf16x8 v = *(bf16x8*)(smem + off);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (k0 + e >= live) v[e] = (bf16)0.0f;
                *(bf16x8*)(smem + off) = v;
            }
        };
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int i = wave + WAVES * u;
            fix(OFF_V + b * TV + 1024 * i + 16 * lane, 16 * (lane >> 4) + 8 * vhalf(16 * i + q16));
        }
        const int c = wave - 4;
        if (c >= 0 && c < NLVB)
            fix(OFF_LV + b * TLV + 1024 * c + 16 * lane, 16 * (lane >> 4) + 8 * vhalf(16 * c + lvg_q));
    };

    // constant chunks: L_v rank ONES_RANK = ones, further ranks zero (paged: the
    // region of ones); L_k padding zero
    if constexpr (PAGED) {
        bf16x8 ones;
#pragma unroll
        for (int e = 0; e < 8; ++e) ones[e] = (bf16)1.0f;
        for (int e = tid; e < 2 * 64; e += 512)
            *(bf16x8*)(smem + OFF_LV + (e / 64) * TLV + LVD + (e % 64) * 16) = ones;
    } else {
        for (int e = tid; e < 2 * (NLV - RCH) * KT; e += 512) {
            const int b = e / ((NLV - RCH) * KT);
            const int c = RCH + (e / KT) % (NLV - RCH);
            bf16x8 v = zero8();
            if (c == RCH) v[0] = (bf16)1.0f;
            *(bf16x8*)(smem + OFF_LV + b * TLV + c * VBS + (e % KT) * 16) = v;
        }
    }
    if constexpr (NLK > RCH) {
        for (int e = tid; e < NKB * (NLK - RCH) * KT; e += 512) {
            const int b = e / ((NLK - RCH) * KT);
            const int c = RCH + (e / KT) % (NLK - RCH);
            *(bf16x8*)(smem + OFF_LK + b * TLK + c * 1024 + (e % KT) * 16) = zero8();
        }
    }

    // page ids (paged mode; otherwise unused) of tiles 0..2, then the loads in
    // flight for the K and V tiles of the next step
    int pid_k = 0, pid_v = 0, pid_2 = 0;
    if constexpr (PAGED) {
        pid_k = pid_use(pid_load(0));
        pid_v = pid_use(pid_load(1));
        if constexpr (ROPE) pid_2 = pid_use(pid_load(2));
    }
    // the tile holding kv_len when it is not full (paged: its value rows past
    // kv_len are zeroed after their DMA)
    const int t_dead = PAGED && kv_len % KT != 0 ? kv_len / KT : -1;
    dma_k(0, 0, pid_k);
    dma_v(0, 0, pid_k);
    if (n_tiles > 1) dma_k(1, 1, pid_v);
    if constexpr (ROPE) {
        if (n_tiles > 2) dma_k(2, 2, pid_2);
        // cos / sin rows 0..63 (the angles of the key offsets inside a tile), kept for
        // the whole kernel; rows past kv_len read as zero
        const auto rc = make_rsrc(a.rope_cos, (uint32_t)kv_len * RB);
        const auto rs = make_rsrc(a.rope_sin, (uint32_t)kv_len * RB);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            dma_1k(rc, smem_lds + OFF_CS + (wave + WAVES * u) * KBS, voff_row[u]);
            dma_1k(rs, smem_lds + OFF_CS + TC + (wave + WAVES * u) * KBS, voff_row[u]);
        }
    }
    // the next step loads V(1) and K(2) (with RoPE: K(3)): raw ids in flight
    if constexpr (PAGED) {
        pid_k = pid_load(ROPE ? 3 : 2);
        pid_v = pid_load(1);
    }

    // ---- query operand (B of S^T): lane holds dims 16*ks + 8*hh .. +7 of its row
    bf16x8 qf[NKS];
    {
        const bf16* qp = a.q + (((size_t)req * q_len + (row_ok ? tok : 0)) * a.h_q + hq) * D + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = row_ok ? ldg((const bf16x8*)(qp + 16 * ks)) : zero8();
    }
    const size_t bcols = (size_t)a.h_kv * D;
    const bf16* bk_ag = a.b_k + (size_t)agent * R * bcols + (size_t)h * D;
    const bf16* bv_ag = a.b_v + (size_t)agent * R * bcols + (size_t)h * D;

    // Rank k-slots.  In the loop a lane of k-group hh carries ranks
    // 16*kr + 8*hh .. +7 (one 16-byte L chunk).  The epilogue follows the O_lr
    // accumulator layout instead: slot e of k-group hh is rank_of(kr, e).
    auto rank_of = [&](int kr, int e) { return 16 * kr + 8 * (e >> 2) + 4 * hh + (e & 3); };

    // ---- qB^T = B_k^(h) Q^T (no RoPE).  A row rho takes rank 16kr + rho with
    // bits 2 and 3 swapped, so that C lane (row, hh) slot e holds rank 16kr + 8hh + e.
    bf16x8 qbf[NKR];
    if constexpr (!ROPE && !PLAIN) {
#pragma unroll
        for (int kr = 0; kr < NKR; ++kr) {
            f32x16 c = {};
            const int rank = 16 * kr + ((n32 & 3) | ((n32 & 4) << 1) | ((n32 & 8) >> 1));
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                bf16x8 av = zero8();
                if (n32 < 16 && rank < R) av = ldg((const bf16x8*)(bk_ag + (size_t)rank * bcols + 16 * ks + 8 * hh));
                c = mfma32x32x16(av, qf[ks], c);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) qbf[kr][e] = (bf16)c[e];
        }
    }

    // ---- RoPE key rebuild K' = K_base + rot_key(L_k B_k^(h)) of one buffer, in place.
    // On 16x16 MFMA tiles (16 dims x 16 keys, ranks as k, zero padded to 16 or
    // 32): the tile's 64 keys x D/2 rotation pairs make D/8 (dim tile, key tile)
    // items, RC = D/64 per wavefront: dim tile r_dt = wave % (D/32) (dims
    // 16 r_dt .. and D/2 + 16 r_dt ..), key tiles RC (wave / (D/32)) + c.  The C
    // layout gives lane l dims 16 r_dt + 4 (l/16) + v of key 16 kt + l % 16, so a
    // lane rotates four (i, i + D/2) pairs of one key per item.
    // The angle of key offset o of tile T is that of position 64T plus that of o:
    //   cos = cos_b cos_o - sin_b sin_o,  sin = sin_b cos_o + cos_b sin_o,
    // with the offset rows o = 0..63 in LDS for the whole kernel and the tile's
    // base row 64T DMA'd beside its keys.
    constexpr int RC = D / 64;
    constexpr int RK = R <= 16 ? 16 : 32;
    typedef __bf16 bfk __attribute__((ext_vector_type(RK / 4)));
    const int r_dt = wave % (D / 32);
    const int r_kt0 = (wave / (D / 32)) * RC;
    const int r_i0 = 16 * r_dt + 4 * g16;  // this lane's first pair index
    bfk rbk1, rbk2;  // B_k^T operands: dim 16 r_dt + i16 (and + D/2), ranks (RK/4) g16 ..
    if constexpr (ROPE) {
#pragma unroll
        for (int e = 0; e < RK / 4; ++e) {
            const int rk = (RK / 4) * g16 + e;
            const bool ok = rk < R;
            const bf16* bp = bk_ag + (size_t)(ok ? rk : 0) * bcols + 16 * r_dt + i16;
            rbk1[e] = ok ? bp[0] : (bf16)0.0f;
            rbk2[e] = ok ? bp[D / 2] : (bf16)0.0f;
        }
    }
    auto rebuild_item = [&](int b, int c) {
        const int key_l = 16 * (r_kt0 + c) + i16;
        const char* lrow = smem + OFF_LK + b * TLK + key_l * 16;
        f32x4 x1, x2;
        if constexpr (RK == 16) {
            const bf16x4 lb = *(const bf16x4*)(lrow + (g16 >> 1) * 1024 + (g16 & 1) * 8);
            x1 = mfma16x16x16(rbk1, lb, zf4());
            x2 = mfma16x16x16(rbk2, lb, zf4());
        } else {
            const bf16x8 lb = *(const bf16x8*)(lrow + g16 * 1024);
            x1 = mfma16x16x32(rbk1, lb, zf4());
            x2 = mfma16x16x32(rbk2, lb, zf4());
        }
        // dims r_i0 .. r_i0+3 and D/2 + r_i0 .. of key key_l
        char* k1p = PAGED ? smem + OFF_K + b * TK + (r_i0 / 8) * 1024 + key_l * 16 + (r_i0 % 8) * 2
                          : smem + OFF_K + b * TK + (key_l % NI) * KBS + (key_l / NI) * RB + 2 * r_i0;
        char* k2p = k1p + (PAGED ? (D / 16) * 1024 : D);
        const char* crow = smem + OFF_CS + (key_l % NI) * KBS + (key_l / NI) * RB;
        const f32x4 co = *(const f32x4*)(crow + 4 * r_i0);
        const f32x4 so = *(const f32x4*)(crow + TC + 4 * r_i0);
        const f32x4 cb = *(const f32x4*)(smem + OFF_CB + b * 2048 + 4 * r_i0);
        const f32x4 sb = *(const f32x4*)(smem + OFF_CB + b * 2048 + 1024 + 4 * r_i0);
        const f32x4 cs = cb * co - sb * so;
        const f32x4 sn = sb * co + cb * so;
        bf16x4* r1 = (bf16x4*)k1p;
        bf16x4* r2 = (bf16x4*)k2p;
        bf16x4 k1 = *r1, k2 = *r2;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            k1[v] = (bf16)((float)k1[v] + (x1[v] * cs[v] - x2[v] * sn[v]));
            k2[v] = (bf16)((float)k2[v] + (x2[v] * cs[v] + x1[v] * sn[v]));
        }
        *r1 = k1;
        *r2 = k2;
    };
    auto rebuild = [&](int b) {
#pragma unroll
        for (int c = 0; c < RC; ++c) rebuild_item(b, c);
    };

    // ---- per-lane LDS operand bases (all further offsets are immediates)
    // score row n32 reads key sigma(n32) (bits 2 and 3 swapped); the value-side
    // reads of k-group hh take keys 8 hh .. 8 hh + 7 of each 16
    const int sk = (n32 & 0x13) | ((n32 & 4) << 1) | ((n32 & 8) >> 1);
    const int rtr = 8 * hh + ss;  // first row of this lane's transposing reads
    const int lds_k = PAGED ? hh * 1024 + sk * 16                              // K row read
                            : (sk % NI) * KBS + (sk / NI) * RB + 16 * hh;
    const int lds_lk = hh * 1024 + sk * 16;                                    // L_k chunk read
    const int lds_v = (rtr % NI) * VBS + (rtr / NI) * RB + 32 * (g16 & 1) + 8 * sa;  // V transposing read
    const int lds_lv = (2 * (g16 & 1) + (sa >> 1)) * VBS + rtr * 16 + 8 * (sa & 1);
    // paged: V^T row (dim n32 of a 32-dim tile, keys 8 hh ..) and L_v^T row (rank
    // 32 lt + n32; past the rank: the ones region)
    // (slot s = 2 * dim + (hh ^ bit 3 of dim) -> block s / 16, 16 (s % 16); the
    // page ks and the dim tile add 256 ks + 4096 dt)
    const int lds_vp = (n32 >> 3) * 1024 + (2 * (n32 & 7) + (hh ^ ((n32 >> 3) & 1))) * 16;
    int lds_lvp[NLT];
#pragma unroll
    for (int lt = 0; lt < NLT; ++lt) {
        const int rho = 32 * lt + n32;
        lds_lvp[lt] = rho < R ? (rho >> 3) * 1024 + (2 * (rho & 7) + (hh ^ ((rho >> 3) & 1))) * 16
                              : LVD + 16 * hh;
    }

    auto s_tile = [&](int b, f32x16 (&s)[2]) {
        const char* kp = smem + OFF_K + b * TK + lds_k;
        const char* lp = smem + OFF_LK + b * TLK + lds_lk;
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                s[mt] = mfma32x32x16(*(const bf16x8*)(kp + mt * KMT + ks * KKS), qf[ks], s[mt]);
        if constexpr (!ROPE && !PLAIN) {
#pragma unroll
            for (int kr = 0; kr < NKR; ++kr)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    s[mt] = mfma32x32x16(*(const bf16x8*)(lp + kr * 2048 + mt * 512), qbf[kr], s[mt]);
        }
    };
    // keys above the row's causal bound -> -inf
    // (slot v of k-group hh in score tile mt: key 32 mt + sigma(8 (v/4) + 4 hh + v%4))
    auto mask_tile = [&](int T, f32x16 (&s)[2]) {
        const int lim = qpos - T * KT - 8 * hh;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                s[mt][v] = 32 * mt + 16 * (v >> 3) + 4 * ((v >> 2) & 1) + (v & 3) > lim ? -INFINITY : s[mt][v];
    };
    // every key of the tile visible to the workgroup's first token
    auto full_tile = [&](int T) { return T * KT + KT - 1 <= kv_len - q_len + tok_wg; };
    const float sl2 = a.scale_log2;
    // row max of a score tile, in log2 units
    auto tile_max = [&](const f32x16 (&s)[2]) {
        float m0 = max3(s[0][0], s[0][1], s[0][2]);
        float m1 = max3(s[1][0], s[1][1], s[1][2]);
#pragma unroll
        for (int v = 3; v < 15; v += 2) {
            m0 = max3(m0, s[0][v], s[0][v + 1]);
            m1 = max3(m1, s[1][v], s[1][v + 1]);
        }
        float m = max3(m0, m1, s[0][15]);
        m = max3(m, s[1][15], s[1][15]);
        // v_permlane32_swap of (m, m): lane l sees m of lanes l and l ^ 32
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
        return max3(__uint_as_float(sw[0]), __uint_as_float(sw[1]), __uint_as_float(sw[1])) * sl2;
    };

    f32x16 acc_o[NDT];
    f32x16 acc_lr[NLT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc_o[dt] = f32x16{};
#pragma unroll
    for (int lt = 0; lt < NLT; ++lt) acc_lr[lt] = f32x16{};

    auto pv_tile = [&](int b, const bf16x8 (&pb)[4]) {
        if constexpr (PAGED) {
            // k-step ks = page ks of the tile
            const char* vp = smem + OFF_V + b * TV + lds_vp;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    acc_o[dt] = mfma32x32x16(*(const bf16x8*)(vp + ks * 256 + dt * 4096), pb[ks], acc_o[dt]);
#pragma unroll
                for (int lt = 0; lt < NLT; ++lt)
                    acc_lr[lt] = mfma32x32x16(*(const bf16x8*)(smem + OFF_LV + b * TLV + lds_lvp[lt] + ks * 256),
                                              pb[ks], acc_lr[lt]);
            }
        } else {
            const char* vp = smem + OFF_V + b * TV + lds_v;
            const char* lp = smem + OFF_LV + b * TLV + lds_lv;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const char* p = vp + ks * VKS + dt * 64;
                    acc_o[dt] = mfma32x32x16(cat4(lds_read_tr(p), lds_read_tr(p + 4 * VBS)), pb[ks], acc_o[dt]);
                }
#pragma unroll
                for (int lt = 0; lt < NLT; ++lt) {
                    const char* p = lp + lt * 4 * VBS + ks * 256;
                    acc_lr[lt] = mfma32x32x16(cat4(lds_read_tr(p), lds_read_tr(p + 64)), pb[ks], acc_lr[lt]);
                }
            }
        }
    };

    // ---- prologue: tiles 0 (K, V) and 1 (K) resident, S(0) and its row max
    wait_dma();
    if (t_dead == 0) zero_dead(0, 0);
    __syncthreads();
    if constexpr (ROPE) {
        // K'(0), K'(1) rebuilt; K(2) is in its buffer already
        rebuild(0);
        if (n_tiles > 1) rebuild(1);
        __syncthreads();
    }
    f32x16 sA[2], sB[2];
    s_tile(0, sA);
    if (!full_tile(0)) mask_tile(0, sA);
    // Running max, lazily updated: rescale only when a row's tile max exceeds it
    // by more than 8 (log2 units), so p = exp2(s*scale - m) <= 2^8 -- exact after
    // the final division, and bf16 / fp32 hold that range.  The floor keeps rows
    // past q_len (Q = 0, everything masked) free of inf - inf.
    float m_run = __builtin_fmaxf(tile_max(sA), -1e30f);
    __syncthreads();  // every S(0) read done before the next key tile lands in buffer 0

    // instruction counts of the two overlapped phases (scheduling hints only)
    constexpr int NS_MFMA = 2 * NKS + (ROPE || PLAIN ? 0 : 2 * NKR);
    constexpr int NP_MFMA = 4 * (NDT + NLT);
    constexpr int DSV = PAGED ? 1 : 2;  // LDS reads per value-side MFMA operand

    // phase 1 of tile t: S(t+1) from K buffer kb on the matrix cores (a stale
    // buffer on the last tile: unused) while P(t) = exp2(S(t)*scale*log2e - m)
    // of keys 0 .. 16*n_exp - 1 runs on the VALU
    auto exp_p = [&](const f32x16 (&sc)[2], bf16x8 (&pb)[4], int ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            pb[ks][e] = (bf16)fast_exp2(__builtin_fmaf(sc[ks >> 1][8 * (ks & 1) + e], sl2, -m_run));
    };
    // extra work placed into the phases (RoPE: one key-rebuild item each): its
    // MFMAs join the MFMA slots of the scheduling hints; its VALU ops are left to
    // the scheduler (pinning them to MFMA slots measured no faster)
    constexpr int XM1 = ROPE ? 2 : 0, XV1 = 0;
    constexpr int XM2 = ROPE && RC > 1 ? 2 : 0, XV2 = 0;
    auto phase1 = [&](int kb, const f32x16 (&sc)[2], f32x16 (&sn)[2], bf16x8 (&pb)[4], auto n_exp_c,
                      auto&& extra) {
        constexpr int n_exp = decltype(n_exp_c)::value;
        s_tile(kb, sn);
        extra();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            if (ks < n_exp) exp_p(sc, pb, ks);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // DS read
#pragma unroll
        for (int i = 0; i < NS_MFMA + XM1; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                     // MFMA
            __builtin_amdgcn_sched_group_barrier(0x402, 2 * n_exp - 1 + XV1, 0);  // VALU / transcendental
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                     // DS read
        }
    };
    // phase 2 of tile t: O += P(t) V(t) from V buffer vb on the matrix cores
    // (exp of keys 16*n_done.. first), row max of S(t+1) on the VALU, then the
    // lazy rescale
    auto phase2 = [&](int t, int vb, const f32x16 (&sc)[2], f32x16 (&sn)[2], bf16x8 (&pb)[4], auto n_done_c,
                      auto&& extra) {
        constexpr int n_done = decltype(n_done_c)::value;
        const bool nxt = t + 1 < n_tiles;
        if (nxt && !full_tile(t + 1)) mask_tile(t + 1, sn);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            if (ks >= n_done) exp_p(sc, pb, ks);
        pv_tile(vb, pb);
        extra();
        const float mx = tile_max(sn);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * DSV, 0);
#pragma unroll
        for (int i = 0; i < (NP_MFMA + XM2) / 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x402, (n_done < 4 ? 4 : 1) + XV2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, DSV, 0);
        }
#pragma unroll
        for (int i = (NP_MFMA + XM2) / 2; i < NP_MFMA + XM2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x402, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, DSV, 0);
        }
        if (nxt && __builtin_amdgcn_ballot_w64(mx > m_run + 8.0f) != 0) {
            const float m_new = __builtin_fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - m_new);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) acc_o[dt] *= alpha;
#pragma unroll
            for (int lt = 0; lt < NLT; ++lt) acc_lr[lt] *= alpha;
            m_run = m_new;
        }
    };

    using I2 = std::integral_constant<int, 2>;
    bf16x8 pb[4];
    if constexpr (!ROPE) {
        // one tile per barrier interval: K(t+2) and V(t+1) land while tile t runs
        auto step = [&](int t, int B, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
            if constexpr (PAGED) {
                pid_k = pid_use(pid_k);
                pid_v = pid_use(pid_v);
            }
            if (t + 2 < n_tiles) dma_k(t + 2, B, pid_k);
            if (t + 1 < n_tiles) dma_v(t + 1, B ^ 1, pid_v);
            if constexpr (PAGED) {
                pid_k = pid_load(t + 3);
                pid_v = pid_load(t + 2);
            }
            phase1(B ^ 1, sc, sn, pb, I2{}, [] {});
            asm volatile("" ::"v"(pb[0]), "v"(pb[1]));  // keys 0..31 of P(t) complete here
            phase2(t, B, sc, sn, pb, I2{}, [] {});
            wait_dma();
            if (t + 1 == t_dead && t + 1 < n_tiles) zero_dead(t + 1, B ^ 1);
            __syncthreads();
        };
        for (int t = 0; t < n_tiles; t += 2) {
            step(t, 0, sA, sB);
            if (t + 1 < n_tiles) step(t + 1, 1, sB, sA);
        }
    } else {
        // RoPE: key tiles go through a ring of three buffers.  Step t issues the
        // DMA of raw K(t+3) (into the buffer K'(t) held) and V(t+1), computes
        // S(t+1) from K'(t+1) on the matrix cores with P(t) on the VALU, then
        // P(t) V(t), and rebuilds K'(t+2) = K(t+2) + rot(L_k B_k) in place (raw
        // K(t+2) landed in step t-1) in the shadow of those MFMAs; one barrier per
        // step, as without RoPE.  The ring index is a run-time, wave-uniform value.
        int kb0 = 0;  // t % 3
        auto step = [&](int t, int B, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
            int k0 = kb0;
            asm volatile("" : "+s"(k0));  // opaque: one address per buffer use, no per-buffer copies
            const int k1 = k0 == 2 ? 0 : k0 + 1;
            const int k2 = k1 == 2 ? 0 : k1 + 1;
            if constexpr (PAGED) {
                pid_k = pid_use(pid_k);
                pid_v = pid_use(pid_v);
            }
            if (t + 3 < n_tiles) dma_k(t + 3, k0, pid_k);
            if (t + 1 < n_tiles) dma_v(t + 1, B ^ 1, pid_v);
            if constexpr (PAGED) {
                pid_k = pid_load(t + 4);
                pid_v = pid_load(t + 2);
            }
            // the rebuild of K'(t+2) is interleaved with the score and value MFMAs
            // (a tile past the end rebuilds a stale buffer that is never read)
            phase1(k1, sc, sn, pb, I2{}, [&] { rebuild_item(k2, 0); });
            asm volatile("" ::"v"(pb[0]), "v"(pb[1]));  // keys 0..31 of P(t) complete here
            phase2(t, B, sc, sn, pb, I2{}, [&] {
                if constexpr (RC > 1) rebuild_item(k2, 1);
            });
            wait_dma();
            if (t + 1 == t_dead && t + 1 < n_tiles) zero_dead(t + 1, B ^ 1);
            __syncthreads();
            kb0 = k1;
        };
        for (int t = 0; t < n_tiles; t += 2) {
            step(t, 0, sA, sB);
            if (t + 1 < n_tiles) step(t + 1, 1, sB, sA);
        }
    }

    // ---- epilogue: l from the ones row; O^T += B_v^T O_lr^T; divide; store
    // ones row sits at M-row ONES_M of tile ONES_T: v with 8(v/4)+4hh+v%4 == ONES_M
    constexpr int OV = 4 * (ONES_M / 8) + (ONES_M % 4);
    constexpr int OH = (ONES_M / 4) % 2;
    const float l_mine = acc_lr[ONES_T][OV];
    const float l_row = __shfl(l_mine, n32 + 32 * OH);
#pragma unroll
    for (int kr = 0; kr < (PLAIN ? 0 : NKR); ++kr) {
        // B_v^T operand: lane (dim 32dt + n32, k-group hh) -> ranks rank_of(kr, e)
        bf16x8 bvt[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int rk = rank_of(kr, e);
                bvt[dt][e] = rk < R ? bv_ag[(size_t)rk * bcols + 32 * dt + n32] : (bf16)0.0f;
            }
        // O_lr^T as B operand: slots e -> ranks rank_of(kr, e) = C rows 16kr + 8(e/4) + 4hh + e%4
        bf16x8 ob;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int rk = rank_of(kr, e);
            ob[e] = rk < R ? (bf16)acc_lr[rk / 32][(8 * kr + e) % 16] : (bf16)0.0f;
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc_o[dt] = mfma32x32x16(bvt[dt], ob, acc_o[dt]);
    }
    if (row_ok) {
        const float inv = l_row > 0.f ? 1.0f / l_row : 0.f;
        bf16* op = a.out + (((size_t)req * q_len + tok) * a.h_q + hq) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int b4 = 0; b4 < 4; ++b4) {
                bf16x4 o;
#pragma unroll
                for (int c = 0; c < 4; ++c) o[c] = (bf16)(acc_o[dt][4 * b4 + c] * inv);
                *(bf16x4*)(op + 32 * dt + 8 * b4 + 4 * hh) = o;
            }
    }
}

template <int D, int R, bool ROPE, bool PLAIN = false, bool PAGED = false>
lra_status launch_t(const lra::PrefillArgs& p, hipStream_t s) {
    PrefillK k;
    k.q = (const bf16*)p.q;
    k.req_agent = p.req_agent;
    k.k_base = (const bf16*)p.k_base;
    k.v_base = (const bf16*)p.v_base;
    k.l_k = (const bf16*)p.l_k;
    k.l_v = (const bf16*)p.l_v;
    k.b_k = (const bf16*)p.b_k;
    k.b_v = (const bf16*)p.b_v;
    k.rope_cos = p.rope_cos;
    k.rope_sin = p.rope_sin;
    k.out = (bf16*)p.out;
    k.n_req = p.n_req;
    k.q_len = p.q_len;
    k.kv_len = p.kv_len;
    k.n_agents = p.n_agents;
    k.h_q = p.h_q;
    k.h_kv = p.h_kv;
    k.g = p.h_q / p.h_kv;
    const int tw = 32 / k.g;
    k.n_qblk = (p.q_len + WAVES * tw - 1) / (WAVES * tw);
    k.scale_log2 = p.scale * LRA_LOG2E;
    k.lr_stride = p.lr_stride;
    k.kv_req_stride = PLAIN ? p.kv_req_stride : 0;
    k.block_table = p.block_table;
    k.n_blk = PAGED ? (int)std::min<long long>(p.max_blocks, ((long long)p.kv_len + 15) / 16) : 0;
    k.n_pages = p.n_pages;
    k.page_bytes = (uint32_t)p.h_kv * D * 16 * 2;
    // tiles (and with RoPE the cos / sin rows) are addressed through 32-bit
    // buffer ranges of kv_len rows of 2*D bytes
    if ((long long)p.kv_len * 2 * D > 0x7fffffffLL) {
        lra::set_error("prefill: kv_len %d too long for 32-bit tile addressing", p.kv_len);
        return LRA_ERR_BAD_SHAPE;
    }
    const long long grid = (long long)p.n_req * p.h_kv * k.n_qblk;
    if (grid > 0x7fffffffLL) {
        lra::set_error("prefill: grid of %lld workgroups too large", grid);
        return LRA_ERR_BAD_SHAPE;
    }
    hipLaunchKernelGGL((lra_prefill_bf16_kernel<D, R, ROPE, PLAIN, PAGED>), dim3((unsigned)grid), dim3(512), 0, s, k);
    return lra::check_launch("lra_prefill_bf16_kernel");
}

template <bool ROPE, bool PAGED>
lra_status launch_rope(const lra::PrefillArgs& p, hipStream_t s) {
#define LRA_CASE(D_, R_) \
    if (p.head_dim == D_ && p.rank == R_) return launch_t<D_, R_, ROPE, false, PAGED>(p, s);
    LRA_CASE(128, 16)
    LRA_CASE(128, 32)
    LRA_CASE(128, 8)
    LRA_CASE(64, 16)
    LRA_CASE(64, 32)
    LRA_CASE(64, 8)
    LRA_CASE(128, 4)
    LRA_CASE(64, 4)
#undef LRA_CASE
    lra::set_error("prefill: unsupported head_dim %d / rank %d", p.head_dim, p.rank);
    return LRA_ERR_UNSUPPORTED;
}

}  // namespace

namespace lra {

lra_status launch_prefill_bf16(const PrefillArgs& p, hipStream_t s) {
    const int g = p.h_q / p.h_kv;
    if (32 % g != 0) {
        set_error("bf16 prefill packs 32 rows per wavefront: H_q/H_kv = %d must divide 32", g);
        return LRA_ERR_UNSUPPORTED;
    }
    if (p.plain) {
        if (p.rope_cos) {
            set_error("plain prefill takes pre-rotated keys (no RoPE tables)");
            return LRA_ERR_UNSUPPORTED;
        }
        if (p.head_dim == 128) return launch_t<128, 8, false, true>(p, s);
        if (p.head_dim == 64) return launch_t<64, 8, false, true>(p, s);
        set_error("prefill: unsupported head_dim %d", p.head_dim);
        return LRA_ERR_UNSUPPORTED;
    }
    if (p.block_table)
        return p.rope_cos ? launch_rope<true, true>(p, s) : launch_rope<false, true>(p, s);
    return p.rope_cos ? launch_rope<true, false>(p, s) : launch_rope<false, false>(p, s);
}

}  // namespace lra
