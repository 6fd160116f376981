// Masked causal prefill attention on MFMA (gfx950).
#include "dms_internal.h"

namespace dms {

hipError_t launch_prefill_attend(const PrefillArgs& a, hipStream_t s) {
    (void)a;
    (void)s;
    return hipErrorNotSupported;
}

}  // namespace dms
