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
    const uint32_t *x, *B, *dt;        // drafts, viewed as 32-bit words
    uint32_t *px, *pB, *pdt;           // pending rows, viewed as 32-bit words
    int32_t *pos, *pending, *err;
    int x_row_words, B_row_words;  // 32-bit words per token row (H*P, G*N elements)
    int dt_elems;                  // elements per token row of dt (H)
    int K, k_max, dt_elt;
};

// One workgroup per slot.  A rejected value (j outside 0..K) is reported in err[b]
// and leaves pos and the pending rows alone; pending becomes 0 because the verify
// that preceded this commit has already folded the previous rows into the state.
__global__ __launch_bounds__(256) void ssm_commit_kernel(const CommitParams p) {
    const int b = blockIdx.x;
    const int j = p.accepted[b];
    if (j < 0 || j > p.K) {
        if (threadIdx.x == 0) {
            p.err[b] = MIL_DEVERR_ACCEPT;
            p.pending[b] = 0;
        }
        return;
    }
    // accepted rows k < j: [b][k][row] -> [b][k][row] of the pending area (32-bit words)
    const int xw = p.x_row_words, bw = p.B_row_words, de = p.dt_elems;
    for (int k = 0; k < j; ++k) {
        const uint32_t *xs = p.x + ((int64_t)b * p.K + k) * xw;
        uint32_t *xd = p.px + ((int64_t)b * p.k_max + k) * xw;
        for (int i = threadIdx.x; i < xw; i += blockDim.x) xd[i] = xs[i];
        const uint32_t *bs = p.B + ((int64_t)b * p.K + k) * bw;
        uint32_t *bd = p.pB + ((int64_t)b * p.k_max + k) * bw;
        for (int i = threadIdx.x; i < bw; i += blockDim.x) bd[i] = bs[i];
        // dt rows can be an odd number of bf16 elements long: copied element by element
        const int64_t src = ((int64_t)b * p.K + k) * de, dst = ((int64_t)b * p.k_max + k) * de;
        for (int i = threadIdx.x; i < de; i += blockDim.x) {
            if (p.dt_elt == 2)
                reinterpret_cast<uint16_t *>(p.pdt)[dst + i] = reinterpret_cast<const uint16_t *>(p.dt)[src + i];
            else
                p.pdt[dst + i] = p.dt[src + i];
        }
    }
    if (threadIdx.x == 0) {
        p.pending[b] = j;
        p.pos[b] += j;
    }
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
    p.x = static_cast<const uint32_t *>(x);
    p.B = static_cast<const uint32_t *>(B);
    p.dt = static_cast<const uint32_t *>(dt);
    p.px = static_cast<uint32_t *>(cache_pend_x(c));
    p.pB = static_cast<uint32_t *>(cache_pend_B(c));
    p.pdt = static_cast<uint32_t *>(cache_pend_dt(c));
    p.pos = cache_pos(c);
    p.pending = cache_pending(c);
    p.err = cache_err(c);
    // H*P and G*N are multiples of 16 (P, N >= 16), so these rows are whole words
    p.x_row_words = c.dims.nheads * c.dims.headdim * e / 4;
    p.B_row_words = c.dims.ngroups * c.dims.dstate * e / 4;
    p.dt_elems = c.dims.nheads;
    p.K = K;
    p.k_max = c.k_max;
    p.dt_elt = e;
    trace_begin(c, MIL_TRACE_COMMIT, s);
    hipLaunchKernelGGL(ssm_commit_kernel, dim3(c.dims.batch), dim3(256), 0, s, p);
    trace_end(c, MIL_TRACE_COMMIT, s);
    return hipGetLastError();
}

hipError_t launch_clear_pending(const CacheImpl &c, hipStream_t s) {
    const int n = c.dims.batch;
    hipLaunchKernelGGL(clear_pending_kernel, dim3((n + 255) / 256), dim3(256), 0, s, cache_pending(c), n);
    return hipGetLastError();
}

}  // namespace mil
