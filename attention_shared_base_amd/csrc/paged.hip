// Paged cache maintenance around the attention kernels (LRAgent §3: agents
// compute only the newly appended context; App. B: the accumulated context is
// L = L_p + L_c).
//
// * Append: the base K/V rows and the LR rows of new tokens (a prefill chunk or
//   one decode token per request; one LR row set per agent pool when the LR
//   caches are per agent) are written into the page pools at the slots a slot
//   mapping names (slot = page * 16 + offset; negative = skip).
//   Page layouts are the decode kernel's: K [H_kv][d/8][16][8], V [H_kv][d][16],
//   L_k [16][r], L_v [r][16].
// * Gather: one context's pages back to the contiguous per-head rows of the
//   contiguous prefill ([H_kv, kv_len, d], [kv_len, r]): the staged paged
//   prefill, kept as a fallback and cross-check of the prefill that reads the
//   pages in place.
#include "lra_common.h"
#include "lra_internal.h"

namespace {

constexpr int PAGE = 16;

struct PagedK {
    const int64_t* slots;       // append: [n_tok]
    const int32_t* block_table; // gather: one context's row
    const bf16* k_rows;         // append source / gather destination (contiguous)
    const bf16* v_rows;
    const bf16* lk_rows;
    const bf16* lv_rows;
    bf16* k_pool;
    bf16* v_pool;
    bf16* lk_pool;
    bf16* lv_pool;
    bf16* k_out;  // gather outputs
    bf16* v_out;
    bf16* lk_out;
    bf16* lv_out;
    int64_t lr_stride;  // append: elements between agents' LR pools
    int32_t n_tok, n_pages, h_kv, kv_len, max_blocks, n_lr;
};

// Append: workgroup = one token, 256 threads.  Rows k_rows/v_rows are
// [n_tok, H_kv, d] (the layout a K/V projection produces), lk_rows/lv_rows
// [n_lr, n_tok, r]: row set a goes to the LR pools of agent a (one set for a
// shared LR cache).
template <int D, int R>
__global__ __launch_bounds__(256) void lra_cache_append_kernel(PagedK a) {
    const int tok = blockIdx.x;
    const int64_t slot = a.slots[tok];
    if (slot < 0 || slot >= (int64_t)a.n_pages * PAGE) return;
    const int64_t pid = slot / PAGE;
    const int t = (int)(slot % PAGE);
    const size_t kv_page = (size_t)a.h_kv * D * PAGE;
    // K: 16-byte chunks (head, dim group); V: single elements (dim-major page)
    for (int e = threadIdx.x; e < a.h_kv * (D / 8); e += blockDim.x) {
        const int h = e / (D / 8), dg = e % (D / 8);
        const bf16x8 v = *(const bf16x8*)(a.k_rows + ((size_t)tok * a.h_kv + h) * D + 8 * dg);
        *(bf16x8*)(a.k_pool + pid * kv_page + (size_t)h * D * PAGE + ((size_t)dg * PAGE + t) * 8) = v;
    }
    for (int e = threadIdx.x; e < a.h_kv * D; e += blockDim.x) {
        const int h = e / D, c = e % D;
        a.v_pool[pid * kv_page + (size_t)h * D * PAGE + (size_t)c * PAGE + t] =
            a.v_rows[((size_t)tok * a.h_kv + h) * D + c];
    }
    for (int e = threadIdx.x; e < a.n_lr * R; e += blockDim.x) {
        const int ag = e / R, k = e % R;
        const size_t src = ((size_t)ag * a.n_tok + tok) * R + k;
        a.lk_pool[ag * a.lr_stride + (pid * PAGE + t) * R + k] = a.lk_rows[src];
        a.lv_pool[ag * a.lr_stride + (pid * R + k) * PAGE + t] = a.lv_rows[src];
    }
}

// Gather: workgroup = (block b of the context, KV head h), 256 threads.  Every
// access is 16 bytes: K chunks move as they are; the dim-major V page (32
// bytes per dim) is turned into rows through LDS (a 16-byte read of 8 tokens
// of one dim, scattered to the 8 rows; then each thread writes 8 dims of one
// row); the LR rows of the block go with head 0.
template <int D, int R>
__global__ __launch_bounds__(256) void lra_cache_gather_kernel(PagedK a) {
    __shared__ __attribute__((aligned(16))) bf16 s_v[PAGE][D + 8];  // row pitch D + 8: 16-byte aligned rows
    const int b = blockIdx.x / a.h_kv;
    const int h = blockIdx.x % a.h_kv;
    const int key0 = b * PAGE;
    const int n = min(PAGE, a.kv_len - key0);
    const int pid = min(max(a.block_table[b], 0), a.n_pages - 1);
    const size_t kv_page = (size_t)a.h_kv * D * PAGE;
    const bf16* kp = a.k_pool + (size_t)pid * kv_page + (size_t)h * D * PAGE;
    const bf16* vp = a.v_pool + (size_t)pid * kv_page + (size_t)h * D * PAGE;
    const int tid = threadIdx.x;
    // K: chunk e = (dim group e / PAGE, token e % PAGE)
    for (int e = tid; e < (D / 8) * PAGE; e += blockDim.x) {
        const int dg = e / PAGE, t = e % PAGE;
        const bf16x8 v = *(const bf16x8*)(kp + (size_t)e * 8);
        if (t < n) *(bf16x8*)(a.k_out + ((size_t)h * a.kv_len + key0 + t) * D + 8 * dg) = v;
    }
    // V: chunk e = (dim e / 2, tokens 8 (e % 2) ..)
    for (int e = tid; e < D * 2; e += blockDim.x) {
        const int c = e / 2, t0 = 8 * (e % 2);
        const bf16x8 v = *(const bf16x8*)(vp + (size_t)e * 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) s_v[t0 + j][c] = v[j];
    }
    __syncthreads();
    for (int e = tid; e < PAGE * (D / 8); e += blockDim.x) {
        const int t = e / (D / 8), cg = e % (D / 8);
        if (t < n)
            *(bf16x8*)(a.v_out + ((size_t)h * a.kv_len + key0 + t) * D + 8 * cg) = *(const bf16x8*)&s_v[t][8 * cg];
    }
    if (h == 0) {
        for (int e = tid; e < PAGE * R; e += blockDim.x) {
            const int t = e / R, rk = e % R;
            if (t < n) {
                a.lk_out[(size_t)(key0 + t) * R + rk] = a.lk_pool[((size_t)pid * PAGE + t) * R + rk];
                a.lv_out[(size_t)(key0 + t) * R + rk] = a.lv_pool[((size_t)pid * R + rk) * PAGE + t];
            }
        }
    }
}

template <int D, int R>
lra_status launch_append_t(const lra::PagedArgs& p, hipStream_t s) {
    PagedK k{};
    k.slots = p.slots;
    k.k_rows = (const bf16*)p.k_rows;
    k.v_rows = (const bf16*)p.v_rows;
    k.lk_rows = (const bf16*)p.lk_rows;
    k.lv_rows = (const bf16*)p.lv_rows;
    k.k_pool = (bf16*)p.k_pool;
    k.v_pool = (bf16*)p.v_pool;
    k.lk_pool = (bf16*)p.lk_pool;
    k.lv_pool = (bf16*)p.lv_pool;
    k.n_tok = p.n_tok;
    k.n_pages = p.n_pages;
    k.h_kv = p.h_kv;
    k.n_lr = p.n_lr;
    k.lr_stride = p.lr_stride;
    hipLaunchKernelGGL((lra_cache_append_kernel<D, R>), dim3(p.n_tok), dim3(256), 0, s, k);
    return lra::check_launch("lra_cache_append_kernel");
}

template <int D, int R>
lra_status launch_gather_t(const lra::PagedArgs& p, hipStream_t s) {
    PagedK k{};
    k.block_table = p.block_table;
    k.k_pool = (bf16*)p.k_pool;
    k.v_pool = (bf16*)p.v_pool;
    k.lk_pool = (bf16*)p.lk_pool;
    k.lv_pool = (bf16*)p.lv_pool;
    k.k_out = (bf16*)p.k_out;
    k.v_out = (bf16*)p.v_out;
    k.lk_out = (bf16*)p.lk_out;
    k.lv_out = (bf16*)p.lv_out;
    k.n_pages = p.n_pages;
    k.h_kv = p.h_kv;
    k.kv_len = p.kv_len;
    const long long grid = (long long)((p.kv_len + PAGE - 1) / PAGE) * p.h_kv;
    if (grid > 0x7fffffffLL) {
        lra::set_error("paged gather: grid of %lld workgroups too large", grid);
        return LRA_ERR_BAD_SHAPE;
    }
    hipLaunchKernelGGL((lra_cache_gather_kernel<D, R>), dim3((unsigned)grid), dim3(256), 0, s, k);
    return lra::check_launch("lra_cache_gather_kernel");
}

}  // namespace

namespace lra {

#define LRA_DISPATCH(FN)                                                         \
    if (p.head_dim == 128 && p.rank == 16) return FN<128, 16>(p, s);             \
    if (p.head_dim == 128 && p.rank == 32) return FN<128, 32>(p, s);             \
    if (p.head_dim == 128 && p.rank == 8) return FN<128, 8>(p, s);               \
    if (p.head_dim == 64 && p.rank == 16) return FN<64, 16>(p, s);               \
    if (p.head_dim == 64 && p.rank == 32) return FN<64, 32>(p, s);               \
    if (p.head_dim == 64 && p.rank == 8) return FN<64, 8>(p, s);                 \
    if (p.head_dim == 128 && p.rank == 4) return FN<128, 4>(p, s);               \
    if (p.head_dim == 64 && p.rank == 4) return FN<64, 4>(p, s);                 \
    set_error("paged cache: unsupported head_dim %d / rank %d", p.head_dim, p.rank); \
    return LRA_ERR_UNSUPPORTED;

lra_status launch_cache_append_bf16(const PagedArgs& p, hipStream_t s) { LRA_DISPATCH(launch_append_t) }

lra_status launch_cache_gather_bf16(const PagedArgs& p, hipStream_t s) { LRA_DISPATCH(launch_gather_t) }

#undef LRA_DISPATCH

}  // namespace lra
