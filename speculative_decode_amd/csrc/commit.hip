// Accepted-length bookkeeping for the speculative step, and small utility kernels.
//
// QbitAI article "Llama 3+Mamba 强强联手", speculative-decoding walkthrough: accepted
// drafts are appended to the output and the state advances through them only; at the
// first rejection the rest is cut and drafting restarts from the last accepted token.
// The commit kernel records that decision for each slot: it checks the accepted length
// j in 0..K, copies the j accepted token rows (x, B, dt) into the cache's pending area,
// and sets pending = j, pos += j.  The state itself is not touched here; the next
// verify (or an immediate fold) applies the pending rows.  Integer work only: exact.
#include "ssm_internal.h"

namespace mil {
namespace {

__global__ void fill_zero_kernel(uint32_t *p, int64_t words) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride) p[i] = 0u;
}

struct CommitParams {
    const int32_t *accepted;
    const char *x, *B, *dt;           // drafts [batch][K][row]
    char *px, *pB, *pdt;              // pending rows [batch][k_max][row]
    int32_t *pos, *pending, *err;
    int x_row, B_row, dt_row;         // bytes per token row (H*P, G*N, H elements)
    int K, k_max;
};

// Copy `bytes` (a multiple of sizeof(V)) with one vector per thread per pass.
template <typename V>
__device__ __forceinline__ void copy_row(char *dst, const char *src, int bytes) {
    const V *s = reinterpret_cast<const V *>(src);
    V *d = reinterpret_cast<V *>(dst);
    const int n = bytes / (int)sizeof(V);
    for (int i = threadIdx.x; i < n; i += blockDim.x) d[i] = s[i];
}

// grid (K, batch): workgroup (k, b) copies accepted row k of slot b (if k < j); the
// k = 0 workgroup also does the slot's bookkeeping.  A rejected value (j outside 0..K)
// is reported in err[b] and leaves pos and the pending rows alone; pending becomes 0
// because the verify that preceded this commit has already folded the previous rows.
template <typename V>
__global__ __launch_bounds__(256) void ssm_commit_kernel(const CommitParams p) {
    const int k = blockIdx.x, b = blockIdx.y;
    const int j = p.accepted[b];
    const bool ok = j >= 0 && j <= p.K;
    if (k == 0 && threadIdx.x == 0) {
        if (ok) {
            p.pending[b] = j;
            p.pos[b] += j;
        } else {
            p.err[b] = MIL_DEVERR_ACCEPT;
            p.pending[b] = 0;
        }
    }
    if (!ok || k >= j) return;
    const size_t src = (size_t)b * p.K + k, dst = (size_t)b * p.k_max + k;
    copy_row<V>(p.px + dst * p.x_row, p.x + src * p.x_row, p.x_row);
    copy_row<V>(p.pB + dst * p.B_row, p.B + src * p.B_row, p.B_row);
    // dt rows (H elements) need not be a whole number of vectors
    const char *ds = p.dt + src * p.dt_row;
    char *dd = p.pdt + dst * p.dt_row;
    for (int i = threadIdx.x; i < p.dt_row / 2; i += blockDim.x)
        reinterpret_cast<uint16_t *>(dd)[i] = reinterpret_cast<const uint16_t *>(ds)[i];
}

__global__ void clear_pending_kernel(int32_t *pending, int batch) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < batch) pending[i] = 0;
}

}  // namespace

hipError_t launch_fill_zero(void *p, int64_t words, hipStream_t s) {
    if (words <= 0) return hipSuccess;
    int64_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint32_t *>(p), words);
    return hipGetLastError();
}

hipError_t launch_commit(const CacheImpl &c, int K, const int32_t *accepted, const void *x,
                         const void *B, const void *dt, hipStream_t s) {
    const int e = elt_bytes(c.dtype);
    CommitParams p;
    p.accepted = accepted;
    p.x = static_cast<const char *>(x);
    p.B = static_cast<const char *>(B);
    p.dt = static_cast<const char *>(dt);
    p.px = static_cast<char *>(cache_pend_x(c));
    p.pB = static_cast<char *>(cache_pend_B(c));
    p.pdt = static_cast<char *>(cache_pend_dt(c));
    p.pos = cache_pos(c);
    p.pending = cache_pending(c);
    p.err = cache_err(c);
    p.x_row = c.dims.nheads * c.dims.headdim * e;   // multiples of 32 bytes (P, N >= 16)
    p.B_row = c.dims.ngroups * c.dims.dstate * e;
    p.dt_row = c.dims.nheads * e;                    // even number of bytes
    p.K = K;
    p.k_max = c.k_max;
    // pending rows are 256-B aligned; 16-byte copies when the draft rows are too
    const bool v16 = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(B)) & 15) == 0;
    trace_begin(c, MIL_TRACE_COMMIT, s);
    if (v16)
        hipLaunchKernelGGL(ssm_commit_kernel<uint4>, dim3(K, c.dims.batch), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(ssm_commit_kernel<uint32_t>, dim3(K, c.dims.batch), dim3(256), 0, s, p);
    trace_end(c, MIL_TRACE_COMMIT, s);
    return hipGetLastError();
}

hipError_t launch_clear_pending(const CacheImpl &c, hipStream_t s) {
    const int n = c.dims.batch;
    hipLaunchKernelGGL(clear_pending_kernel, dim3((n + 255) / 256), dim3(256), 0, s, cache_pending(c), n);
    return hipGetLastError();
}

}  // namespace mil
