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
// packing: one K/V tile serves all g heads).  64-token K/V/L tiles stream
// through double-buffered LDS.  All products run on v_mfma_f32_32x32x16_bf16:
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
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

LRA_DEV bf16x8 ones8() {
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (bf16)1.0f;
    return o;
}

// Transposing LDS read: the 16 lanes of a group each name one 8-byte row piece
// (lane a + 4*s -> row k0+s, columns n0+4a .. n0+4a+3); lane i of the group
// receives column n0+i of rows k0 .. k0+3.
LRA_DEV bf16x4 lds_read_tr(const bf16* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

template <int D, int R, bool ROPE>
__global__ __launch_bounds__(512) void lra_prefill_bf16_kernel(PrefillK a) {
    // LDS row pitches (elements), measured conflict-free on gfx950: 16-byte row
    // reads need a pitch of 16 (mod 256) bytes, the transposing reads (two
    // 16-lane groups side by side, 4 rows each) 64 (mod 256) bytes, and the
    // 8-byte rank reads of 32 rows an odd number of 8-byte words.
    constexpr int KP = D + 8;                    // K tile: 272 B for d = 128
    constexpr int VP = D + 32;                   // V tile: 320 B for d = 128
    constexpr int RW = R < 16 ? 16 : R;          // rank columns held per L row (zero padded)
    constexpr int RP = RW + 4;                   // L_k tile: 40 B (r <= 16) / 72 B (r = 32)
    constexpr int RV = RW;                       // L_v tile: transposing reads, contiguous rows
    constexpr int NKS = D / 16;                  // k-steps over head dim
    constexpr int NDT = D / 32;                  // 32-wide dim tiles
    constexpr int NKR = (R + 15) / 16;           // k-steps over rank
    constexpr int NLT = (R + 1 + 31) / 32;       // rank tiles of O_lr incl. the ones row
    constexpr int ONES_T = R / 32;               // tile holding the ones row
    constexpr int ONES_M = R % 32;               // its row inside the tile
    constexpr int CH_K = KT * D / 8;             // 16-byte chunks per K (or V) tile
    constexpr int CH_L = KT * RW / 8;            // 16-byte chunks per L tile
    constexpr int CH = 2 * CH_K + 2 * CH_L;
    constexpr int LPT = (CH + 511) / 512;        // chunks per thread

    __shared__ __attribute__((aligned(16))) bf16 sK[2][KT][KP];
    __shared__ __attribute__((aligned(16))) bf16 sV[2][KT][VP];
    __shared__ __attribute__((aligned(16))) bf16 sLk[2][KT][RP];
    __shared__ __attribute__((aligned(16))) bf16 sLv[2][KT][RV];
    __shared__ __attribute__((aligned(16))) bf16 sBk[ROPE ? R : 1][ROPE ? D : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n32 = lane & 31;  // row of this lane (S^T / O^T column)
    const int hh = lane >> 5;   // k-group of this lane
    const int i16 = lane & 15;  // lane inside its 16-lane group (transposing reads)
    const int g16 = lane >> 4;  // 16-lane group

    const int g = a.g;
    const int TW = 32 / g;  // tokens per wavefront
    const int qb = blockIdx.x % a.n_qblk;
    const int h = (blockIdx.x / a.n_qblk) % a.h_kv;
    const int req = blockIdx.x / (a.n_qblk * a.h_kv);
    const int tok_wg = qb * WAVES * TW;
    const int q_len = a.q_len, kv_len = a.kv_len;
    int agent = a.req_agent[req];
    agent = min(max(agent, 0), a.n_agents - 1);

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

    // ---- global -> register -> LDS tile copies (16-byte chunks)
    bf16x8 stage[LPT];
    auto gload = [&](int tile) {
        const int key0 = tile * KT;
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int c = tid + 512 * u;
            bf16x8 v = zero8();
            if (c < CH) {
                if (c < 2 * CH_K) {
                    const int cc = c % CH_K;
                    const int key = key0 + cc / (D / 8);
                    const int col = (cc % (D / 8)) * 8;
                    if (key < kv_len) v = ldg_stream((const bf16x8*)((c < CH_K ? kb : vb) + (size_t)key * D + col));
                } else {
                    const int cc = (c - 2 * CH_K) % CH_L;
                    const int key = key0 + cc / (RW / 8);
                    const int col = (cc % (RW / 8)) * 8;
                    if (key < kv_len && col < R)
                        v = ldg((const bf16x8*)((c < 2 * CH_K + CH_L ? a.l_k : a.l_v) + (size_t)key * R + col));
                }
            }
            stage[u] = v;
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int c = tid + 512 * u;
            if (c < CH) {
                if (c < CH_K) {
                    const int cc = c;
                    *(bf16x8*)(&sK[buf][0][0] + (cc / (D / 8)) * KP + (cc % (D / 8)) * 8) = stage[u];
                } else if (c < 2 * CH_K) {
                    const int cc = c - CH_K;
                    *(bf16x8*)(&sV[buf][0][0] + (cc / (D / 8)) * VP + (cc % (D / 8)) * 8) = stage[u];
                } else if (c < 2 * CH_K + CH_L) {
                    // 8-byte aligned rows: two 8-byte stores
                    const int cc = c - 2 * CH_K;
                    bf16* dst = &sLk[buf][0][0] + (cc / (RW / 8)) * RP + (cc % (RW / 8)) * 8;
                    *(bf16x4*)dst = __builtin_shufflevector(stage[u], stage[u], 0, 1, 2, 3);
                    *(bf16x4*)(dst + 4) = __builtin_shufflevector(stage[u], stage[u], 4, 5, 6, 7);
                } else {
                    const int cc = c - 2 * CH_K - CH_L;
                    *(bf16x8*)(&sLv[buf][0][0] + (cc / (RW / 8)) * RV + (cc % (RW / 8)) * 8) = stage[u];
                }
            }
        }
    };

    gload(0);

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
    // rank carried by k-slot e of rank step kr for a lane in k-group hh
    auto rank_of = [&](int kr, int e) { return 16 * kr + 8 * (e >> 2) + 4 * hh + (e & 3); };

    // ---- qB^T = B_k^(h) Q^T (no RoPE): ranks on M, rows on N
    bf16x8 qbf[NKR];
    if constexpr (!ROPE) {
#pragma unroll
        for (int kr = 0; kr < NKR; ++kr) {
            f32x16 c = {};
            const int rank = 16 * kr + n32;  // A row: rank
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                bf16x8 av = zero8();
                if (n32 < 16 && rank < R) av = ldg((const bf16x8*)(bk_ag + (size_t)rank * bcols + 16 * ks + 8 * hh));
                c = mfma32x32x16(av, qf[ks], c);
            }
            // C lane holds ranks 16kr + 8(v/4) + 4hh + v%4 (v < 8 carry ranks < 16kr + 16)
#pragma unroll
            for (int e = 0; e < 8; ++e) qbf[kr][e] = (bf16)c[e];
        }
    }
    // ---- B_k^(h) of the RoPE key rebuild, staged once in LDS as [rank][dim]
    if constexpr (ROPE) {
        for (int e = tid; e < R * D; e += 512) sBk[e / D][e % D] = bk_ag[(size_t)(e / D) * bcols + e % D];
    }

    f32x16 acc_o[NDT];
    f32x16 acc_lr[NLT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc_o[dt] = f32x16{};
#pragma unroll
    for (int lt = 0; lt < NLT; ++lt) acc_lr[lt] = f32x16{};
    float m_run = -INFINITY;
    const float sl2 = a.scale_log2;

    lstore(0);
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
        const int buf = t & 1;
        const int key0 = t * KT;
        if (t + 1 < n_tiles) gload(t + 1);

        if constexpr (ROPE) {
            // rebuild K'[key][dim] = K_base + rot_key(L_k B_k^(h)) in place, waves 0..2*D/64-1:
            // wave -> (key tile kt, dim tile dt paired with dt + D/64)
            constexpr int HALF_T = D / 64;
            if (wave < 2 * HALF_T) {
                const int kt = wave / HALF_T;
                const int dt = wave % HALF_T;
                f32x16 x1 = {}, x2 = {};
#pragma unroll
                for (int kr = 0; kr < NKR; ++kr) {
                    // B_k^T operand: lane (dim 32dt + n32, k-group hh) -> ranks rank_of(kr, e)
                    bf16x8 b1, b2;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int rk = min(rank_of(kr, e), R - 1);
                        const bool ok = rank_of(kr, e) < R;
                        b1[e] = ok ? sBk[rk][32 * dt + n32] : (bf16)0.0f;
                        b2[e] = ok ? sBk[rk][32 * (dt + HALF_T) + n32] : (bf16)0.0f;
                    }
                    // L_k^T operand: lane (key n32, k-group hh) -> ranks rank_of(kr, e)
                    const bf16* lp = &sLk[buf][32 * kt + n32][16 * kr + 4 * hh];
                    bf16x8 lb = cat4(*(const bf16x4*)lp, *(const bf16x4*)(lp + 8));
                    if (16 * kr + 4 * hh >= R) lb = zero8();
                    x1 = mfma32x32x16(b1, lb, x1);
                    x2 = mfma32x32x16(b2, lb, x2);
                }
                // C lane (key n32, hh): dims 32dt + 8(v/4) + 4hh + v%4 (x1) and +D/2 (x2)
                const int key = key0 + 32 * kt + n32;
                const int kc = min(key, kv_len - 1);
#pragma unroll
                for (int b4 = 0; b4 < 4; ++b4) {
                    const int i0 = 32 * dt + 8 * b4 + 4 * hh;
                    const f32x4 cs = *(const f32x4*)(a.rope_cos + (size_t)kc * (D / 2) + i0);
                    const f32x4 sn = *(const f32x4*)(a.rope_sin + (size_t)kc * (D / 2) + i0);
                    bf16* r1 = &sK[buf][32 * kt + n32][i0];
                    bf16* r2 = r1 + D / 2;
                    bf16x4 k1 = *(bf16x4*)r1, k2 = *(bf16x4*)r2;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const float u1 = x1[4 * b4 + c], u2 = x2[4 * b4 + c];
                        k1[c] = (bf16)((float)k1[c] + (u1 * cs[c] - u2 * sn[c]));
                        k2[c] = (bf16)((float)k2[c] + (u2 * cs[c] + u1 * sn[c]));
                    }
                    *(bf16x4*)r1 = k1;
                    *(bf16x4*)r2 = k2;
                }
            }
            __syncthreads();
        }

        // ---- S^T for two 32-key halves
        f32x16 s[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            s[mt] = f32x16{};
            const bf16* kp = &sK[buf][32 * mt + n32][8 * hh];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) s[mt] = mfma32x32x16(*(const bf16x8*)(kp + 16 * ks), qf[ks], s[mt]);
            if constexpr (!ROPE) {
#pragma unroll
                for (int kr = 0; kr < NKR; ++kr) {
                    const bf16* lp = &sLk[buf][32 * mt + n32][16 * kr + 4 * hh];
                    bf16x8 lb = cat4(*(const bf16x4*)lp, *(const bf16x4*)(lp + 8));
                    if (16 * kr + 4 * hh >= R) lb = zero8();
                    s[mt] = mfma32x32x16(lb, qbf[kr], s[mt]);
                }
            }
        }
        // ---- online softmax (row = lane % 32; the two k-groups hold disjoint keys).
        // Tiles entirely below the causal diagonal of the workgroup's first token
        // skip the mask.  The running max is updated lazily: only when some row's
        // tile max exceeds it by more than 8 (log2 units) are the accumulators
        // rescaled, so p = exp2(s*scale - m) <= 2^8 — exact after the final
        // division, and bf16 / fp32 hold that range.  Rows past q_len (Q = 0) never
        // reach the output.
        const bool full = key0 + KT - 1 <= kv_len - q_len + tok_wg;
        if (!full) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = key0 + 32 * mt + 8 * (v >> 2) + 4 * hh + (v & 3);
                    s[mt][v] = key <= qpos ? s[mt][v] : -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int v = 0; v < 16; v += 2) mx = fmaxf(mx, fmaxf(s[mt][v], s[mt][v + 1]));
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
        if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.0f) != 0) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - m_new);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) acc_o[dt] *= alpha;
#pragma unroll
            for (int lt = 0; lt < NLT; ++lt) acc_lr[lt] *= alpha;
            m_run = m_new;
        }
        bf16x8 pb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pb[ks][e] = (bf16)fast_exp2(__builtin_fmaf(s[ks >> 1][8 * (ks & 1) + e], sl2, -m_run));

        // ---- O^T += V^T P^T and O_lr^T += L_v^T P^T (16 keys per k-step)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int k0 = 32 * (ks >> 1) + 16 * (ks & 1) + 4 * hh;  // keys of slots 0..3; +8 for 4..7
            const int srow = k0 + (i16 >> 2);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const bf16* vp = &sV[buf][srow][32 * dt + 16 * (g16 & 1) + 4 * (i16 & 3)];
                const bf16x8 va = cat4(lds_read_tr(vp), lds_read_tr(vp + 8 * VP));
                acc_o[dt] = mfma32x32x16(va, pb[ks], acc_o[dt]);
            }
#pragma unroll
            for (int lt = 0; lt < NLT; ++lt) {
                // A rows m = 32lt + lane%32: ranks (< R) from L_v^T, then the ones
                // row (m == R, giving sum_j p_j), then zeros.  The transposing read
                // runs on every lane (rows >= R read an in-bounds dummy column and
                // are overwritten after): under a lane-divergent branch it also
                // overwrote the inactive lanes' destination registers.
                const int col = 32 * lt + 16 * (g16 & 1);
                const bf16* lp = &sLv[buf][srow][(col < R ? col : 0) + 4 * (i16 & 3)];
                bf16x8 la = cat4(lds_read_tr(lp), lds_read_tr(lp + 8 * RV));
                const int m = 32 * lt + n32;
                if (m >= R) la = m == R ? ones8() : zero8();
                acc_lr[lt] = mfma32x32x16(la, pb[ks], acc_lr[lt]);
            }
        }

        if (t + 1 < n_tiles) {
            lstore(buf ^ 1);
        }
        __syncthreads();
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
