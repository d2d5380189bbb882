// Instantiations of the verify / fold kernel for f32 token inputs.
#include "verify_kernel.h"

namespace mil {

hipError_t dispatch_verify_f32(const VerifyParams &vp, int batch, hipStream_t s) {
    return dispatch_rows<float>(vp, batch, s);
}

}  // namespace mil
