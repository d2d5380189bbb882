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
    int64_t x_row_words, B_row_words;  // words per token row (H*P, G*N elements)
    int64_t dt_row_bytes;              // bytes per token row of dt (H elements)
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
    // x rows: [b][k][H*P] -> [b][k_max slot k][H*P]
    for (int64_t i = threadIdx.x; i < (int64_t)j * p.x_row_words; i += blockDim.x) {
        const int64_t k = i / p.x_row_words, w = i % p.x_row_words;
        p.px[((int64_t)b * p.k_max + k) * p.x_row_words + w] = p.x[((int64_t)b * p.K + k) * p.x_row_words + w];
    }
    for (int64_t i = threadIdx.x; i < (int64_t)j * p.B_row_words; i += blockDim.x) {
        const int64_t k = i / p.B_row_words, w = i % p.B_row_words;
        p.pB[((int64_t)b * p.k_max + k) * p.B_row_words + w] = p.B[((int64_t)b * p.K + k) * p.B_row_words + w];
    }
    // dt rows can be an odd number of bf16 elements long: copy element by element
    const int64_t dt_elems = p.dt_row_bytes / p.dt_elt;
    for (int64_t i = threadIdx.x; i < (int64_t)j * dt_elems; i += blockDim.x) {
        const int64_t k = i / dt_elems, e = i % dt_elems;
        const int64_t src = ((int64_t)b * p.K + k) * dt_elems + e;
        const int64_t dst = ((int64_t)b * p.k_max + k) * dt_elems + e;
        if (p.dt_elt == 2)
            reinterpret_cast<uint16_t *>(p.pdt)[dst] = reinterpret_cast<const uint16_t *>(p.dt)[src];
        else
            p.pdt[dst] = p.dt[src];
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

__global__ void prefill_counters_kernel(int32_t *pos, int32_t *pending, int slot0, int nseq, int L, int cont) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nseq) {
        pos[slot0 + i] = cont ? pos[slot0 + i] + L : L;
        pending[slot0 + i] = 0;
    }
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
    p.x_row_words = (int64_t)c.dims.nheads * c.dims.headdim * e / 4;
    p.B_row_words = (int64_t)c.dims.ngroups * c.dims.dstate * e / 4;
    p.dt_row_bytes = (int64_t)c.dims.nheads * e;
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

hipError_t launch_prefill_counters(const CacheImpl &c, int slot0, int nseq, int L, bool cont, hipStream_t s) {
    hipLaunchKernelGGL(prefill_counters_kernel, dim3((nseq + 255) / 256), dim3(256), 0, s, cache_pos(c),
                       cache_pending(c), slot0, nseq, L, cont ? 1 : 0);
    return hipGetLastError();
}

}  // namespace mil
