// Instantiations of the verify / fold kernel for f32 token inputs.
#include "verify_kernel.h"

namespace mil {

hipError_t dispatch_verify_f32(const VerifyParams &vp, int kt, int batch, hipStream_t s) {
    if (kt == 4) return dispatch_rows<float, 4>(vp, batch, s);
    if (kt == 8) return dispatch_rows<float, 8>(vp, batch, s);
    if (kt == 16) return dispatch_rows<float, 16>(vp, batch, s);
    return hipErrorInvalidValue;
}

}  // namespace mil
