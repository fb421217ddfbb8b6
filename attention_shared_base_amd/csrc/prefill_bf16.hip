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
// S^T's accumulator layout (lane = row l%32, keys 8*(v/4) + 4*(l/32) + v%4) is
// already the P^T operand layout, so P stays in registers.  V^T and L_v^T
// operands come from the row-major LDS tiles through the gfx950 transposing
// read ds_read_b64_tr_b16 (16 lanes turn a 4 x 16 block into 16 columns of 4).
//
// Data movement.  64-key tiles go HBM -> LDS by buffer_load ... lds (no
// register staging): one instruction moves 1 KB, lane i's 16 bytes landing at
// 16*i, and keys past kv_len read as zero through the buffer range.  Each 1 KB
// block of a K / V / cos / sin tile holds the rows key = i + NI*m of block i,
// and consecutive blocks sit 1040 B (K, cos, sin) or 1088 B (V) apart: that
// spreads the 16 rows a 16-lane row read touches over all 64 banks, and the
// 4 rows of a transposing read over the four 64-byte bank quarters, with LDS
// addresses that stay linear in the key (one base register per operand).
// L tiles are chunk-major ([16-byte rank chunk][key]); the L_v tile carries
// constant chunks after the ranks (the ones row, zeros) written once.
//
// Pipeline per tile t: K is loaded two tiles ahead and V one tile ahead, so
// S(t+1) is on the matrix cores while the softmax of S(t) runs on the VALU,
// followed by P(t)V(t) with the row max of S(t+1) in its shadow; one barrier
// per tile (two with RoPE: raw K(t+2) lands, K'(t+2) is rebuilt in place).
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

// One 1 KB HBM -> LDS block (buffer_load_dwordx4 ... lds): lane i reads 16
// bytes at byte offset voff of the resource and they land at LDS address
// lds + 16*i.  Issued from asm so that the compiler does not serialise the
// transfer against unrelated LDS reads; completion is awaited explicitly
// (wait_dma) before the barrier that publishes the tile.  M0 is restored.
LRA_DEV void dma_1k(u32x4 r, uint32_t lds, uint32_t voff) {
    uint32_t keep;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(keep)
        : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(r)
        : "memory");
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

// s_waitcnt vmcnt(0): this wavefront's LDS DMA has landed.
LRA_DEV void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// v_max3_f32 (operands are finite or -inf; no NaN canonicalisation needed)
LRA_DEV float max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

template <int D, int R, bool ROPE>
__global__ __launch_bounds__(512) void lra_prefill_bf16_kernel(PrefillK a) {
    constexpr int RB = 2 * D;                 // bytes per K / V row (and per cos / sin row)
    constexpr int CPR = D / 8;                // 16-byte chunks per row
    constexpr int NI = KT * RB / 1024;        // 1 KB blocks per tile
    constexpr int NU = NI / WAVES;            // blocks per wavefront per tile
    constexpr int KBS = 1024 + 16;            // block stride: K, cos, sin
    constexpr int VBS = 1024 + 64;            // block stride: V, L_v chunks
    constexpr int TK = NI * KBS;
    constexpr int TV = NI * VBS;
    constexpr int RW = R < 16 ? 16 : R;       // ranks held per L row (zero padded)
    constexpr int NKS = D / 16;               // k-steps over head dim
    constexpr int NDT = D / 32;               // 32-wide dim tiles
    constexpr int NKR = RW / 16;              // k-steps over rank
    // 16-byte rank chunks of an L tile that come from HBM (rank 4: one chunk,
    // ranks 4-7 zero); the ones row is the first rank of the next chunk
    constexpr int RCH = R < 8 ? 1 : R / 8;
    constexpr int ONES_RANK = 8 * RCH;        // = R for R >= 8
    constexpr int NLT = (ONES_RANK + 1 + 31) / 32;  // rank tiles of O_lr incl. the ones row
    constexpr int ONES_T = ONES_RANK / 32;    // tile holding the ones row
    constexpr int ONES_M = ONES_RANK % 32;    // its row inside the tile
    constexpr int NLK = RW / 8;               // L_k chunks held
    constexpr int NLV = 4 * NLT;              // L_v chunks held (ranks, ones row, zeros)
    constexpr int TLK = NLK * 1024;
    constexpr int TLV = NLV * VBS;
    constexpr int OFF_K = 0;
    constexpr int OFF_V = OFF_K + 2 * TK;
    constexpr int OFF_LK = OFF_V + 2 * TV;
    constexpr int OFF_LV = OFF_LK + 2 * TLK;
    constexpr int OFF_CS = OFF_LV + 2 * TLV;  // RoPE: cos / sin tiles, two buffers
    constexpr int LDS_BYTES = OFF_CS + (ROPE ? 4 * TK : 0);
    constexpr int KMT = (32 / NI) * RB;       // K tile offset of keys 32..63
    constexpr int VKS = (D == 128) ? RB : 2 * RB;   // V offset of the next 16 keys
    constexpr int V8 = (D == 128) ? 8 * VBS : RB;   // V offset of rows +8
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    static_assert((R % 8 == 0 && R <= 32) || R == 4, "rank 4, 8, 16, 24 or 32");
    static_assert(NU >= 1 && NI % WAVES == 0, "tile blocks divide over the wavefronts");
    static_assert(RCH <= 4, "L_v DMA uses wavefronts 4..7");
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
    const int qb = blockIdx.x % a.n_qblk;
    const int h = (blockIdx.x / a.n_qblk) % a.h_kv;
    const int req = blockIdx.x / (a.n_qblk * a.h_kv);
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

    const size_t hstride = (size_t)kv_len * D;
    const bf16* kb = a.k_base + (size_t)h * hstride;
    const bf16* vb = a.v_base + (size_t)h * hstride;

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

    auto dma_k = [&](int T, int b) {
        const int key0 = T * KT;
        const uint32_t rem = (uint32_t)(kv_len - key0);
        const auto rk = make_rsrc(kb + (size_t)key0 * D, rem * RB);
#pragma unroll
        for (int u = 0; u < NU; ++u) dma_1k(rk, smem_lds + OFF_K + b * TK + (wave + WAVES * u) * KBS, voff_row[u]);
        if constexpr (R < 8) {
            if (wave < 4)
                dma_256(make_rsrc(lk_ag + (size_t)(key0 + 16 * wave) * R,
                                  (uint32_t)max((int)rem - 16 * wave, 0) * (2 * R)),
                        smem_lds + OFF_LK + b * TLK + wave * 256, voff_l4);
        } else if (wave < RCH) {
            dma_1k(make_rsrc(lk_ag + (size_t)key0 * R, rem * (2 * R)), smem_lds + OFF_LK + b * TLK + wave * 1024,
                   voff_l + 16 * wave);
        }
        if constexpr (ROPE) {
            const auto rc = make_rsrc(a.rope_cos + (size_t)key0 * (D / 2), rem * RB);
            const auto rs = make_rsrc(a.rope_sin + (size_t)key0 * (D / 2), rem * RB);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                dma_1k(rc, smem_lds + OFF_CS + (2 * b) * TK + (wave + WAVES * u) * KBS, voff_row[u]);
                dma_1k(rs, smem_lds + OFF_CS + (2 * b + 1) * TK + (wave + WAVES * u) * KBS, voff_row[u]);
            }
        }
    };
    auto dma_v = [&](int T, int b) {
        const int key0 = T * KT;
        const uint32_t rem = (uint32_t)(kv_len - key0);
        const auto rv = make_rsrc(vb + (size_t)key0 * D, rem * RB);
#pragma unroll
        for (int u = 0; u < NU; ++u) dma_1k(rv, smem_lds + OFF_V + b * TV + (wave + WAVES * u) * VBS, voff_row[u]);
        const int c = wave - 4;
        if constexpr (R < 8) {
            if (c >= 0)
                dma_256(make_rsrc(lv_ag + (size_t)(key0 + 16 * c) * R,
                                  (uint32_t)max((int)rem - 16 * c, 0) * (2 * R)),
                        smem_lds + OFF_LV + b * TLV + c * 256, voff_l4);
        } else if (c >= 0 && c < RCH) {
            dma_1k(make_rsrc(lv_ag + (size_t)key0 * R, rem * (2 * R)), smem_lds + OFF_LV + b * TLV + c * VBS,
                   voff_l + 16 * c);
        }
    };

    // constant chunks: L_v rank ONES_RANK = ones, further ranks zero; L_k padding zero
    for (int e = tid; e < 2 * (NLV - RCH) * KT; e += 512) {
        const int b = e / ((NLV - RCH) * KT);
        const int c = RCH + (e / KT) % (NLV - RCH);
        bf16x8 v = zero8();
        if (c == RCH) v[0] = (bf16)1.0f;
        *(bf16x8*)(smem + OFF_LV + b * TLV + c * VBS + (e % KT) * 16) = v;
    }
    if constexpr (NLK > RCH) {
        for (int e = tid; e < 2 * (NLK - RCH) * KT; e += 512) {
            const int b = e / ((NLK - RCH) * KT);
            const int c = RCH + (e / KT) % (NLK - RCH);
            *(bf16x8*)(smem + OFF_LK + b * TLK + c * 1024 + (e % KT) * 16) = zero8();
        }
    }

    dma_k(0, 0);
    dma_v(0, 0);
    if (n_tiles > 1) dma_k(1, 1);

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
    if constexpr (!ROPE) {
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
    // Wavefront -> key half kt, dim tile dt (paired with dt + D/64), and a part of
    // the 8-dim groups b4.  x1/x2 = B_k^T L_k^T for dims 32dt.. and 32dt + D/2..
    constexpr int HALF_T = D / 64;
    const int rb_kt = wave & 1;
    const int rb_dt = (wave >> 1) % HALF_T;
    const int rb_part = (wave >> 1) / HALF_T;
    bf16x8 bk1[NKR], bk2[NKR];
    if constexpr (ROPE) {
#pragma unroll
        for (int kr = 0; kr < NKR; ++kr)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int rk = 16 * kr + 8 * hh + e;
                const bool ok = rk < R;
                const bf16* bp = bk_ag + (size_t)(ok ? rk : 0) * bcols + 32 * rb_dt + n32;
                bk1[kr][e] = ok ? bp[0] : (bf16)0.0f;
                bk2[kr][e] = ok ? bp[D / 2] : (bf16)0.0f;
            }
    }
    auto rebuild = [&](int T, int b) {
        const int key_l = 32 * rb_kt + n32;
        f32x16 x1 = {}, x2 = {};
#pragma unroll
        for (int kr = 0; kr < NKR; ++kr) {
            const bf16x8 lb = *(const bf16x8*)(smem + OFF_LK + b * TLK + (2 * kr + hh) * 1024 + key_l * 16);
            x1 = mfma32x32x16(bk1[kr], lb, x1);
            x2 = mfma32x32x16(bk2[kr], lb, x2);
        }
        char* krow = smem + OFF_K + b * TK + (key_l % NI) * KBS + (key_l / NI) * RB;
        const char* crow = smem + OFF_CS + (2 * b) * TK + (key_l % NI) * KBS + (key_l / NI) * RB;
        const char* srow = crow + TK;
#pragma unroll
        for (int j = 0; j < HALF_T; ++j) {
            const int b4 = rb_part * HALF_T + j;
            const int i0 = 32 * rb_dt + 8 * b4 + 4 * hh;
            const f32x4 cs = *(const f32x4*)(crow + 4 * i0);
            const f32x4 sn = *(const f32x4*)(srow + 4 * i0);
            bf16x4* r1 = (bf16x4*)(krow + 2 * i0);
            bf16x4* r2 = (bf16x4*)(krow + 2 * (i0 + D / 2));
            bf16x4 k1 = *r1, k2 = *r2;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float u1 = x1[4 * b4 + c], u2 = x2[4 * b4 + c];
                k1[c] = (bf16)((float)k1[c] + (u1 * cs[c] - u2 * sn[c]));
                k2[c] = (bf16)((float)k2[c] + (u2 * cs[c] + u1 * sn[c]));
            }
            *r1 = k1;
            *r2 = k2;
        }
        (void)T;
    };

    // ---- per-lane LDS operand bases (all further offsets are immediates)
    const int lds_k = (n32 % NI) * KBS + (n32 / NI) * RB + 16 * hh;            // K row read
    const int lds_lk = hh * 1024 + n32 * 16;                                   // L_k chunk read
    const int lds_v = (4 * hh + ss) * VBS + 32 * (g16 & 1) + 8 * sa;           // V transposing read
    const int lds_lv = (2 * (g16 & 1) + (sa >> 1)) * VBS + (4 * hh + ss) * 16 + 8 * (sa & 1);

    auto s_tile = [&](int b, f32x16 (&s)[2]) {
        const char* kp = smem + OFF_K + b * TK + lds_k;
        const char* lp = smem + OFF_LK + b * TLK + lds_lk;
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                s[mt] = mfma32x32x16(*(const bf16x8*)(kp + mt * KMT + ks * 32), qf[ks], s[mt]);
        if constexpr (!ROPE) {
#pragma unroll
            for (int kr = 0; kr < NKR; ++kr)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    s[mt] = mfma32x32x16(*(const bf16x8*)(lp + kr * 2048 + mt * 512), qbf[kr], s[mt]);
        }
    };
    // keys above the row's causal bound -> -inf
    auto mask_tile = [&](int T, f32x16 (&s)[2]) {
        const int lim = qpos - T * KT - 4 * hh;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                s[mt][v] = 32 * mt + 8 * (v >> 2) + (v & 3) > lim ? -INFINITY : s[mt][v];
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
        const char* vp = smem + OFF_V + b * TV + lds_v;
        const char* lp = smem + OFF_LV + b * TLV + lds_lv;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const char* p = vp + ks * VKS + dt * 64;
                acc_o[dt] = mfma32x32x16(cat4(lds_read_tr(p), lds_read_tr(p + V8)), pb[ks], acc_o[dt]);
            }
#pragma unroll
            for (int lt = 0; lt < NLT; ++lt) {
                const char* p = lp + lt * 4 * VBS + ks * 256;
                acc_lr[lt] = mfma32x32x16(cat4(lds_read_tr(p), lds_read_tr(p + 128)), pb[ks], acc_lr[lt]);
            }
        }
    };

    // ---- prologue: tiles 0 (K, V) and 1 (K) resident, S(0) and its row max
    wait_dma();
    __syncthreads();
    if constexpr (ROPE) {
        rebuild(0, 0);
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
    __syncthreads();  // every S(0) read done before K(2) lands in buffer 0

    // instruction counts of the two overlapped phases (scheduling hints only)
    constexpr int NS_MFMA = 2 * NKS + (ROPE ? 0 : 2 * NKR);
    constexpr int NP_MFMA = 4 * (NDT + NLT);

    // phase 1 of tile t: S(t+1) from K buffer kb on the matrix cores (a stale
    // buffer on the last tile: unused) while P(t) = exp2(S(t)*scale*log2e - m)
    // of keys 0 .. 16*n_exp - 1 runs on the VALU
    auto exp_p = [&](const f32x16 (&sc)[2], bf16x8 (&pb)[4], int ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            pb[ks][e] = (bf16)fast_exp2(__builtin_fmaf(sc[ks >> 1][8 * (ks & 1) + e], sl2, -m_run));
    };
    auto phase1 = [&](int kb, const f32x16 (&sc)[2], f32x16 (&sn)[2], bf16x8 (&pb)[4], auto n_exp_c) {
        constexpr int n_exp = decltype(n_exp_c)::value;
        s_tile(kb, sn);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            if (ks < n_exp) exp_p(sc, pb, ks);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // DS read
#pragma unroll
        for (int i = 0; i < NS_MFMA; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
            __builtin_amdgcn_sched_group_barrier(0x402, 2 * n_exp - 1, 0);  // VALU / transcendental
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);               // DS read
        }
    };
    // phase 2 of tile t: O += P(t) V(t) from V buffer vb on the matrix cores
    // (exp of keys 16*n_done.. first), row max of S(t+1) on the VALU, then the
    // lazy rescale
    auto phase2 = [&](int t, int vb, const f32x16 (&sc)[2], f32x16 (&sn)[2], bf16x8 (&pb)[4], auto n_done_c) {
        constexpr int n_done = decltype(n_done_c)::value;
        const bool nxt = t + 1 < n_tiles;
        if (nxt && !full_tile(t + 1)) mask_tile(t + 1, sn);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            if (ks >= n_done) exp_p(sc, pb, ks);
        pv_tile(vb, pb);
        const float mx = tile_max(sn);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < NP_MFMA / 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x402, n_done < 4 ? 4 : 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
#pragma unroll
        for (int i = NP_MFMA / 2; i < NP_MFMA; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x402, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
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
    using I4 = std::integral_constant<int, 4>;
    bf16x8 pb[4];
    if constexpr (!ROPE) {
        // one tile per barrier interval: K(t+2) and V(t+1) land while tile t runs
        auto step = [&](int t, int B, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
            if (t + 2 < n_tiles) dma_k(t + 2, B);
            if (t + 1 < n_tiles) dma_v(t + 1, B ^ 1);
            phase1(B ^ 1, sc, sn, pb, I2{});
            asm volatile("" ::"v"(pb[0]), "v"(pb[1]));  // keys 0..31 of P(t) complete here
            phase2(t, B, sc, sn, pb, I2{});
            wait_dma();
            __syncthreads();
        };
        for (int t = 0; t < n_tiles; t += 2) {
            step(t, 0, sA, sB);
            if (t + 1 < n_tiles) step(t + 1, 1, sB, sA);
        }
    } else {
        // RoPE: the key tile has to be rebuilt (K' = K + rot(L_k B_k)) between its
        // arrival and its score MFMAs.  Step t runs
        //   A: O += P(t-1) V(t-1) on the matrix cores, with the row max of S(t)
        //      and the rebuild of K'(t+1) on the VALU;  barrier;
        //   B: S(t+1) from K'(t+1) on the matrix cores, P(t) on the VALU.
        // Step t loads K(t+2) (with its L_k rows and cos / sin tiles) and V(t).
        // step 0: no P V yet
        if (n_tiles > 2) dma_k(2, 0);
        rebuild(1, 1);  // a stale buffer when n_tiles == 1: never read
        __syncthreads();
        phase1(1, sA, sB, pb, I4{});
        wait_dma();
        __syncthreads();
        auto step = [&](int t, int B, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
            if (t + 2 < n_tiles) dma_k(t + 2, B);
            dma_v(t, B);
            if (!full_tile(t)) mask_tile(t, sc);
            pv_tile(B ^ 1, pb);
            const float mx = tile_max(sc);
            rebuild(t + 1, B ^ 1);  // a stale buffer on the last tile: never read
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < NP_MFMA + 2 * NKR; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.0f) != 0) {
                const float m_new = __builtin_fmaxf(m_run, mx);
                const float alpha = fast_exp2(m_run - m_new);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) acc_o[dt] *= alpha;
#pragma unroll
                for (int lt = 0; lt < NLT; ++lt) acc_lr[lt] *= alpha;
                m_run = m_new;
            }
            __syncthreads();
            phase1(B ^ 1, sc, sn, pb, I4{});
            wait_dma();
            __syncthreads();
        };
        for (int t = 1; t < n_tiles; t += 2) {
            step(t, 1, sB, sA);
            if (t + 1 < n_tiles) step(t + 1, 0, sA, sB);
        }
        pv_tile((n_tiles - 1) & 1, pb);
    }

    // ---- epilogue: l from the ones row; O^T += B_v^T O_lr^T; divide; store
    // ones row sits at M-row ONES_M of tile ONES_T: v with 8(v/4)+4hh+v%4 == ONES_M
    constexpr int OV = 4 * (ONES_M / 8) + (ONES_M % 4);
    constexpr int OH = (ONES_M / 4) % 2;
    const float l_mine = acc_lr[ONES_T][OV];
    const float l_row = __shfl(l_mine, n32 + 32 * OH);
#pragma unroll
    for (int kr = 0; kr < NKR; ++kr) {
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

template <int D, int R, bool ROPE>
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
    // tiles are addressed through 32-bit buffer ranges of kv_len rows of 2*D bytes
    if ((long long)p.kv_len * 2 * D > 0x7fffffffLL) {
        lra::set_error("prefill: kv_len %d too long for 32-bit tile addressing", p.kv_len);
        return LRA_ERR_BAD_SHAPE;
    }
    const long long grid = (long long)p.n_req * p.h_kv * k.n_qblk;
    if (grid > 0x7fffffffLL) {
        lra::set_error("prefill: grid of %lld workgroups too large", grid);
        return LRA_ERR_BAD_SHAPE;
    }
    hipLaunchKernelGGL((lra_prefill_bf16_kernel<D, R, ROPE>), dim3((unsigned)grid), dim3(512), 0, s, k);
    return lra::check_launch("lra_prefill_bf16_kernel");
}

template <bool ROPE>
lra_status launch_rope(const lra::PrefillArgs& p, hipStream_t s) {
#define LRA_CASE(D_, R_) \
    if (p.head_dim == D_ && p.rank == R_) return launch_t<D_, R_, ROPE>(p, s);
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
    return p.rope_cos ? launch_rope<true>(p, s) : launch_rope<false>(p, s);
}

}  // namespace lra
