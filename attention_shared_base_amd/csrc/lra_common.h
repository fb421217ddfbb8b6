// Device-side building blocks shared by the gfx950 kernels: vector types, MFMA
// wrappers and small wave-level helpers.  CDNA4 only (wave64, gfx950 MFMA).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lra_attn.h"

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define LRA_DEV __device__ __forceinline__

// log2(e): softmax is evaluated with exp2 on scores pre-multiplied by scale*log2(e).
#define LRA_LOG2E 1.4426950408889634f

// ---------------------------------------------------------------------------
// MFMA.  Operand lane layouts used throughout (wave64, l = lane id):
//   16x16xK : A lane l holds row (l % 16), k-group (l / 16);
//             B lane l holds column (l % 16), k-group (l / 16);
//             C lane l holds rows 4*(l/16) + v (v = 0..3) of column (l % 16).
//   32x32x16: A row (l % 32), k-group (l / 32); B column (l % 32);
//             C lane l holds rows 8*(v/4) + 4*(l/32) + (v%4) of column (l % 32).
// The k index inside a group only has to agree between A and B, so callers are
// free to choose which physical column each (group, slot) pair carries.

LRA_DEV f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

LRA_DEV f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

LRA_DEV f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// vector helpers

LRA_DEV bf16x8 cat4(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

LRA_DEV bf16x8 zero8() {
    bf16x8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
    return z;
}

LRA_DEV bf16x4 zero4() {
    bf16x4 z;
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = (bf16)0.0f;
    return z;
}

LRA_DEV f32x4 zf4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Bitwise AND of the four bf16 lanes with two 32-bit masks (elements 0-1 / 2-3).
LRA_DEV bf16x4 and_mask(bf16x4 x, uint32_t lo, uint32_t hi) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x2 u = __builtin_bit_cast(u32x2, x);
    u.x &= lo;
    u.y &= hi;
    return __builtin_bit_cast(bf16x4, u);
}

template <typename T>
LRA_DEV T ldg(const T* p) { return *p; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes): stride 0, reads past the end
// return 0.
LRA_DEV u32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t p = (uint64_t)base;
    u32x4 r;
    r[0] = (uint32_t)p;
    r[1] = (uint32_t)(p >> 32) & 0xffffu;
    r[2] = bytes;
    r[3] = 0x00020000u;
    return r;
}

// One 1 KB HBM -> LDS block (buffer_load_dwordx4 ... lds): lane i reads 16
// bytes at byte offset voff of the resource and they land at LDS address
// lds + 16*i.  Issued from asm so that the compiler does not serialise the
// transfer against unrelated LDS reads; the caller awaits completion with
// s_waitcnt vmcnt before the barrier that publishes the data.  M0 is restored.
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

// Streaming (read-once) load: bypasses reuse in the caches it can.
template <typename T>
LRA_DEV T ldg_stream(const T* p) { return __builtin_nontemporal_load(p); }

LRA_DEV float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

LRA_DEV float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// exp2 with the hardware instruction (v_exp_f32); exp2(-inf) = 0.
LRA_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// host-side launch helpers shared by the translation units

namespace lra {

// Set the thread's error text (defined in api.hip).
void set_error(const char* fmt, ...);

// Convert a failed launch into a status with detail text.
lra_status check_launch(const char* what);

}  // namespace lra
