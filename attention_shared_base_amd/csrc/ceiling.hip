// Device ceilings for the roofline figures: a plain HBM read stream and a bf16 MFMA
// stream.  Neither is part of the attention path.  They measure what this device
// sustains (at the clock it holds under that load), so a kernel's rate can be set
// against a rate reached on the same chip as well as against the published peaks.
#include "lra_common.h"
#include "lra_internal.h"

namespace {

// Two layouts of a plain read, 16-byte loads, sixteen in flight per lane (NT:
// non-temporal loads, else ordinary cached loads):
//   grid-stride  lane g of the grid reads words g, g + S, g + 2S, ... (S = lanes in
//                the grid), so each wavefront instruction covers 1 KB and the whole
//                grid sweeps the buffer front to back;
//   chunked      workgroup b reads words [b c, (b + 1) c) (c = chunk, a multiple of
//                64 words), 4 KB per round of its 256 lanes.
// The words are folded by XOR and written only when the fold hits a value the host
// never plants, which keeps the loads from being dropped as dead code.
constexpr int kReadInFlight = 16;

template <bool NT>
LRA_DEV u32x4 ld16(const u32x4* p) {
    if constexpr (NT) return ldg_stream(p);
    return *p;
}

LRA_DEV void fold_to_sink(u32x4 x, uint32_t* sink) {
    const uint32_t f = x[0] ^ x[1] ^ x[2] ^ x[3];
    if (f == 0x6a09e667u) sink[0] = f;
}

template <bool NT>
__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4* __restrict__ p, uint64_t n16,
                                                       uint32_t* __restrict__ sink) {
    constexpr int U = kReadInFlight;
    const uint64_t s = (uint64_t)gridDim.x * 256u;
    uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    u32x4 x = {0u, 0u, 0u, 0u};
    for (; i + (U - 1) * s < n16; i += U * s) {
        u32x4 v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) v[j] = ld16<NT>(p + i + j * s);
#pragma unroll
        for (int j = 0; j < U; ++j) x ^= v[j];
    }
    for (; i < n16; i += s) x ^= ld16<NT>(p + i);
    fold_to_sink(x, sink);
}

template <bool NT>
__global__ __launch_bounds__(256) void hbm_read_chunked_kernel(const u32x4* __restrict__ p, uint64_t n16,
                                                               uint64_t chunk, uint32_t* __restrict__ sink) {
    constexpr int U = kReadInFlight;
    const uint64_t b0 = (uint64_t)blockIdx.x * chunk;
    const uint64_t e = b0 + chunk < n16 ? b0 + chunk : n16;
    uint64_t i = b0 + threadIdx.x;
    u32x4 x = {0u, 0u, 0u, 0u};
    for (; i + (U - 1) * 256 < e; i += U * 256) {
        u32x4 v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) v[j] = ld16<NT>(p + i + j * 256);
#pragma unroll
        for (int j = 0; j < U; ++j) x ^= v[j];
    }
    for (; i < e; i += 256) x ^= ld16<NT>(p + i);
    fold_to_sink(x, sink);
}

// Each wavefront runs four independent accumulation chains of
// v_mfma_f32_32x32x16_bf16 (2 x 32 x 32 x 16 flops each) for `iters` rounds.
// NLDS operands of every MFMA come from a fresh ds_read_b128 (1 KB per wavefront
// per operand): 0 keeps both in registers, 1 reads B (the operand traffic of an
// attention tile whose keys sit in LDS), 2 reads A and B.  The slot index
// advances by a runtime step so the reads cannot be hoisted.
template <int NLDS>
__global__ __launch_bounds__(256) void mfma_bf16_kernel(int32_t iters, int32_t step,
                                                        uint32_t* __restrict__ sink) {
    __shared__ bf16x8 tile[NLDS ? 8 * 256 : 1];
    const int t = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (bf16)((float)((t + e) & 7) * 0.125f);
        b[e] = (bf16)((float)((3 * t + e) & 7) * -0.0625f);
    }
    if constexpr (NLDS > 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) tile[j * 256 + t] = j & 1 ? a : b;
        __syncthreads();
    }
    f32x16 c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) c[j][v] = 0.f;
    int slot = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x8 aj = a, bj = b;
            if constexpr (NLDS >= 1) bj = tile[((slot + j) & 7) * 256 + t];
            if constexpr (NLDS >= 2) aj = tile[((slot + j + 4) & 7) * 256 + t];
            c[j] = mfma32x32x16(aj, bj, c[j]);
        }
        slot += step;
    }
    float f = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) f += c[j][v];
    if (f == 1234567.0f) sink[0] = __float_as_uint(f);
}

}  // namespace

namespace lra {

lra_status launch_ceiling_read(const void* buf, uint64_t n_bytes, int n_wg, bool nt, bool chunked,
                               uint32_t* sink, hipStream_t s) {
    const u32x4* p = (const u32x4*)buf;
    const uint64_t n16 = n_bytes / 16u;
    if (chunked) {
        const uint64_t chunk = ((n16 + n_wg - 1) / n_wg + 63) / 64 * 64;
        if (nt)
            hipLaunchKernelGGL(hbm_read_chunked_kernel<true>, dim3(n_wg), dim3(256), 0, s, p, n16, chunk, sink);
        else
            hipLaunchKernelGGL(hbm_read_chunked_kernel<false>, dim3(n_wg), dim3(256), 0, s, p, n16, chunk, sink);
    } else if (nt) {
        hipLaunchKernelGGL(hbm_read_kernel<true>, dim3(n_wg), dim3(256), 0, s, p, n16, sink);
    } else {
        hipLaunchKernelGGL(hbm_read_kernel<false>, dim3(n_wg), dim3(256), 0, s, p, n16, sink);
    }
    return check_launch("hbm_read_kernel");
}

lra_status launch_ceiling_mfma(int n_lds, int n_wg, int iters, uint32_t* sink, hipStream_t s) {
    if (n_lds == 2)
        hipLaunchKernelGGL(mfma_bf16_kernel<2>, dim3(n_wg), dim3(256), 0, s, iters, 1, sink);
    else if (n_lds == 1)
        hipLaunchKernelGGL(mfma_bf16_kernel<1>, dim3(n_wg), dim3(256), 0, s, iters, 1, sink);
    else
        hipLaunchKernelGGL(mfma_bf16_kernel<0>, dim3(n_wg), dim3(256), 0, s, iters, 1, sink);
    return check_launch("mfma_bf16_kernel");
}

}  // namespace lra
