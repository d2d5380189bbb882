// Instantiations of the verify / fold kernel for bf16 token inputs.
#include "verify_kernel.h"

namespace mil {

hipError_t dispatch_verify_bf16(const VerifyParams &vp, int batch, hipStream_t s) {
    return dispatch_rows<uint16_t>(vp, batch, s);
}

}  // namespace mil
