// placeholder, replaced by the MFMA prefill kernel
#include "lra_common.h"
#include "lra_internal.h"
namespace lra {
lra_status launch_prefill_bf16(const PrefillArgs&, hipStream_t) {
    set_error("bf16 prefill not built yet");
    return LRA_ERR_UNSUPPORTED;
}
}  // namespace lra
