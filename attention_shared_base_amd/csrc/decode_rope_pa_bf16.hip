// Paged decode with RoPE on the adapter key term and one LR cache per agent
// (LRAgent §3 BaseShared with the rotated key of App. D.1): the RoPE + per-agent
// mode of the decode kernel (decode_kernel.h), in a translation unit of its own
// (built, like the RoPE mode, with the MFMA results kept in VGPRs).
#include "decode_kernel.h"

namespace lra {

lra_status launch_decode_rope_pa_bf16(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
    const int d = a.head_dim, r = a.rank;
#define LRA_CASE(D_, R_) \
    if (d == D_ && r == R_) return launch_dr<D_, R_, MODE_ROPE_PER_AGENT>(a, p, s);
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
