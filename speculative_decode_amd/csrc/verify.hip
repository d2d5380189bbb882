// Launcher of the speculative verify / fold kernel (kernel in verify_kernel.h).
#include "verify_kernel.h"

namespace mil {

bool verify_supported(int batch, int H, int P, int N, int K, int kmax) {
    return shape_for(batch, H, P, N, K, kmax).S > 0;
}

hipError_t launch_verify(const CacheImpl &c, int K, const void *x, const void *B, const void *C,
                         const void *dt, const float *A, const float *D, float *y, hipStream_t s,
                         const int32_t *parent) {
    VerifyParams vp;
    vp.state = cache_state(c);
    vp.head_stride = c.lay.state_head_stride / 4;
    vp.pend_x = cache_pend_x(c);
    vp.pend_B = cache_pend_B(c);
    vp.pend_dt = cache_pend_dt(c);
    vp.pending = cache_pending(c);
    vp.append = cache_append(c);
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
    vp.cs = 1;  // set by the launcher from the chosen shape
    vp.vec = (((uintptr_t)x | (uintptr_t)B | (uintptr_t)C) & 15) == 0;
    vp.parent = parent;
    vp.err = cache_err(c);
    const int batch = c.dims.batch;
    const int id = K > 0 ? MIL_TRACE_VERIFY : MIL_TRACE_FOLD;
    trace_begin(c, id, s);
    const hipError_t e = c.dtype == MIL_BF16 ? dispatch_verify_bf16(vp, batch, s)
                                             : dispatch_verify_f32(vp, batch, s);
    trace_end(c, id, s);
    return e;
}

}  // namespace mil
