// Launcher of the speculative verify / fold kernel (kernel in verify_kernel.h).
#include "verify_kernel.h"

namespace mil {

bool verify_supported(int P, int N, int kt) {
    (void)kt;
    return (P == 16 || P == 32 || P == 64 || P == 128 || P == 256) &&
           (N == 16 || N == 32 || N == 64 || N == 128 || N == 256) && shape_known(P, N);
}

hipError_t launch_verify(const CacheImpl &c, int K, const void *x, const void *B, const void *C,
                         const void *dt, const float *A, const float *D, float *y, hipStream_t s) {
    VerifyParams vp;
    vp.state = cache_state(c);
    vp.head_stride = c.lay.state_head_stride / 4;
    vp.pend_x = cache_pend_x(c);
    vp.pend_B = cache_pend_B(c);
    vp.pend_dt = cache_pend_dt(c);
    vp.pending = cache_pending(c);
    vp.x = x;
    vp.B = B;
    vp.C = C;
    vp.dt = dt;
    vp.A = A;
    vp.D = D;
    vp.y = y;
    vp.H = c.dims.nheads;
    vp.P = c.dims.headdim;
    vp.N = c.dims.dstate;
    vp.G = c.dims.ngroups;
    vp.K = K;
    vp.k_max = c.k_max;
    const int kt = c.k_max <= 4 ? 4 : (c.k_max <= 8 ? 8 : 16);  // bounds both K and pending
    const int batch = c.dims.batch;
    const int id = K > 0 ? MIL_TRACE_VERIFY : MIL_TRACE_FOLD;
    trace_begin(c, id, s);
    const hipError_t e = c.dtype == MIL_BF16 ? dispatch_verify_bf16(vp, kt, batch, s)
                                             : dispatch_verify_f32(vp, kt, batch, s);
    trace_end(c, id, s);
    return e;
}

}  // namespace mil
