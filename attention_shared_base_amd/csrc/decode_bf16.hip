// Paged decode entry: the shared-LR mode of the decode kernel (decode_kernel.h);
// the per-agent-LR mode is built in decode_pa_bf16.hip, the RoPE mode in
// decode_rope_bf16.hip and RoPE with per-agent LR in decode_rope_pa_bf16.hip
// (translation units of their own, compiled in parallel).
#include "decode_kernel.h"

namespace lra {

lra_status launch_decode_rope_bf16(const DecodeArgs& a, const DecodePlan& p, hipStream_t s);
lra_status launch_decode_pa_bf16(const DecodeArgs& a, const DecodePlan& p, hipStream_t s);
lra_status launch_decode_rope_pa_bf16(const DecodeArgs& a, const DecodePlan& p, hipStream_t s);

lra_status launch_decode_bf16(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
    const int d = a.head_dim, r = a.rank;
    if (a.rope_cos != nullptr) {
        // The RoPE modes always run one workgroup per chunk.  Their persistent
        // (chunk-queue) form is switched off: a GPU memory fault was observed
        // with it (rank 32, 512-token chunks) whose cause has not been found.
        DecodePlan q = p;
        q.persistent = 0;
        if (a.lr_stride != 0) return launch_decode_rope_pa_bf16(a, q, s);
        return launch_decode_rope_bf16(a, q, s);
    }
    if (a.lr_stride != 0) return launch_decode_pa_bf16(a, p, s);
#define LRA_CASE(D_, R_) \
    if (d == D_ && r == R_) return launch_dr<D_, R_, MODE_SHARED>(a, p, s);
    LRA_CASE(128, 16)
    LRA_CASE(128, 32)
    LRA_CASE(128, 8)
    LRA_CASE(64, 16)
    LRA_CASE(64, 32)
    LRA_CASE(64, 8)
    LRA_CASE(128, 4)
    LRA_CASE(64, 4)
#undef LRA_CASE
    set_error("decode: unsupported head_dim %d / rank %d", d, r);
    return LRA_ERR_UNSUPPORTED;
}

}  // namespace lra
