// Accepted-length bookkeeping for the speculative step, and small utility kernels.
//
// QbitAI article "Llama 3+Mamba 强强联手", speculative-decoding walkthrough: accepted
// drafts are appended to the output and the state advances through them only; at the
// first rejection the rest is cut and drafting restarts from the last accepted token.
// The commit kernel records that decision for each slot: it checks the accepted length
// j in 0..K, copies the j accepted token rows (x, B, dt) into the cache's pending area,
// and sets pending = j, pos += j.  The state itself is not touched here; the next
// verify (or an immediate fold) applies the pending rows.  Integer work only: exact.
#include <algorithm>

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
// The row is read into registers before j is known, so that the two reads overlap
// instead of the copy waiting for j first (a row past j is read and dropped); rows
// longer than kCommitRegs vectors per thread copy their remainder afterwards.
constexpr int kCommitRegs = 4;
typedef int i32x4v __attribute__((ext_vector_type(4)));  // 16 bytes that arrays keep in registers
template <typename V> struct RegVec { typedef V type; };
template <> struct RegVec<uint4> { typedef i32x4v type; };

template <typename VM>
__global__ __launch_bounds__(256) void ssm_commit_kernel(const CommitParams p) {
    typedef typename RegVec<VM>::type V;
    const int k = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, nt = blockDim.x;
    const size_t src = (size_t)b * p.K + k, dst = (size_t)b * p.k_max + k;
    const V *xs = reinterpret_cast<const V *>(p.x + src * p.x_row);
    const V *bs = reinterpret_cast<const V *>(p.B + src * p.B_row);
    const uint16_t *ds = reinterpret_cast<const uint16_t *>(p.dt + src * p.dt_row);
    const int nx = p.x_row / (int)sizeof(V), nb = p.B_row / (int)sizeof(V), nd = p.dt_row / 2;
    // every index clamped into the row (rows are never empty), so no load waits on a branch
    V vx[kCommitRegs], vb[kCommitRegs];
#pragma unroll
    for (int i = 0; i < kCommitRegs; ++i) {
        vx[i] = xs[min(tid + i * nt, nx - 1)];
        vb[i] = bs[min(tid + i * nt, nb - 1)];
    }
    const uint16_t vd = ds[min(tid, nd - 1)];
    const int j = p.accepted[b];
    const bool ok = j >= 0 && j <= p.K;
    if (k == 0 && tid == 0) {
        if (ok) {
            p.pending[b] = j;
            p.pos[b] += j;
        } else {
            p.err[b] = MIL_DEVERR_ACCEPT;
            p.pending[b] = 0;
        }
    }
    if (!ok || k >= j) return;
    V *xd = reinterpret_cast<V *>(p.px + dst * p.x_row);
    V *bd = reinterpret_cast<V *>(p.pB + dst * p.B_row);
    uint16_t *dd = reinterpret_cast<uint16_t *>(p.pdt + dst * p.dt_row);
#pragma unroll
    for (int i = 0; i < kCommitRegs; ++i) {
        if (tid + i * nt < nx) xd[tid + i * nt] = vx[i];
        if (tid + i * nt < nb) bd[tid + i * nt] = vb[i];
    }
    for (int e = tid + kCommitRegs * nt; e < nx; e += nt) xd[e] = xs[e];
    for (int e = tid + kCommitRegs * nt; e < nb; e += nt) bd[e] = bs[e];
    // dt rows (H elements) need not be a whole number of vectors
    if (tid < nd) dd[tid] = vd;
    for (int e = tid + nt; e < nd; e += nt) dd[e] = ds[e];
}

// ------------------------------------------------------------------ tree drafts
// The commit of a tree round (tree-organised candidates; skycaiji.com summary,
// related-work paragraph): the accepted branch is the root path of one node, and its
// tokens, root first, become the pending rows, exactly as the j accepted drafts of a
// chain do.  grid (K, batch): every workgroup of slot b walks the parent links up from
// accepted_node[b] (at most K steps, each link checked to lie in -1..i-1); workgroup k
// copies the path's k-th token row, workgroup 0 does the bookkeeping.  A node outside
// -1..K-1 or a bad link on the path sets err[b] and pending = 0 and leaves pos alone.
struct TreeCommitParams {
    CommitParams c;
    const int32_t *parent;         // [batch][K]
    const int32_t *accepted_node;  // [batch]
};

template <typename V>
__global__ __launch_bounds__(256) void ssm_commit_tree_kernel(const TreeCommitParams tp) {
    const CommitParams &p = tp.c;
    __shared__ int spath[MIL_KMAX_LIMIT];
    __shared__ int sj, sbad;
    const int k = blockIdx.x, b = blockIdx.y;
    if (threadIdx.x == 0) {
        const int a = tp.accepted_node[b];
        int bad = (a < -1 || a >= p.K) ? MIL_DEVERR_ACCEPT : 0;
        int depth = 0;
        // first walk: the depth (links strictly decrease, so at most K steps)
        for (int i = a; !bad && i >= 0; ++depth) {
            const int q = tp.parent[(size_t)b * p.K + i];
            if (q < -1 || q >= i) bad = MIL_DEVERR_TREE;
            i = q;
        }
        // second walk: the path, root first
        if (!bad)
            for (int i = a, d = depth - 1; i >= 0; --d) {
                spath[d] = i;
                i = tp.parent[(size_t)b * p.K + i];
            }
        sj = bad ? 0 : depth;
        sbad = bad;
    }
    __syncthreads();
    const int j = sj;
    if (k == 0 && threadIdx.x == 0) {
        if (!sbad) {
            p.pending[b] = j;
            p.pos[b] += j;
        } else {
            p.err[b] = sbad;
            p.pending[b] = 0;
        }
    }
    if (k >= j) return;
    const size_t src = (size_t)b * p.K + spath[k], dst = (size_t)b * p.k_max + k;
    copy_row<V>(p.px + dst * p.x_row, p.x + src * p.x_row, p.x_row);
    copy_row<V>(p.pB + dst * p.B_row, p.B + src * p.B_row, p.B_row);
    const char *ds = p.dt + src * p.dt_row;
    char *dd = p.pdt + dst * p.dt_row;
    for (int i = threadIdx.x; i < p.dt_row / 2; i += blockDim.x)
        reinterpret_cast<uint16_t *>(dd)[i] = reinterpret_cast<const uint16_t *>(ds)[i];
}

// ------------------------------------------------------------------ greedy acceptance
// The same commit with the accepted lengths decided on the device (QbitAI walkthrough:
// keep the drafts the verifier confirms, cut at the first one it rejects; read here as
// greedy verification, a draft being confirmed when it is the argmax of the verifier's
// logits at its position).  Two launches:
//   1. greedy_argmax_kernel, grid (S, K, batch): split s of row (b, k) of the logits
//      reduces its slice to one 64-bit key, written to ws[b][k][s];
//   2. greedy_commit_kernel, grid (K, batch): every workgroup of slot b takes the max of
//      the S keys per position (the argmax token), compares with the drafts, finds the
//      accepted length j, and then does what ssm_commit_kernel does with it.
// Key = (order-preserving bits of the value) << 32 | (0xFFFFFFFF - index): the largest
// key is the largest value, ties going to the lowest index, so the result does not depend
// on how the vocabulary is split or in which order partial maxima meet.  Integer and
// compare-only work: exact.
constexpr int kGreedySplitsMax = 64;

__device__ __forceinline__ uint32_t ordered(float v) {  // monotonic in v
    const uint32_t u = __float_as_uint(v);
    return u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
}
__device__ __forceinline__ uint64_t argmax_key(uint32_t o, uint32_t idx) {
    return ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ uint64_t kmax(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ float logit(float v) { return v; }
__device__ __forceinline__ float logit(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
// Element q of 16 loaded bytes (q known at compile time after unrolling), as a float.
__device__ __forceinline__ uint32_t word(const uint4 &w, int i) { return i == 0 ? w.x : i == 1 ? w.y : i == 2 ? w.z : w.w; }
__device__ __forceinline__ float element(const uint4 &w, int q, const float *) { return __uint_as_float(word(w, q)); }
__device__ __forceinline__ float element(const uint4 &w, int q, const uint16_t *) {
    const uint32_t u = word(w, q >> 1);
    return __uint_as_float((q & 1) ? (u & 0xffff0000u) : (u << 16));
}

// Largest key over the workgroup (256 threads), returned to every thread.
__device__ __forceinline__ uint64_t block_max_key(uint64_t v, uint64_t *sred) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const uint32_t h = __shfl_xor(static_cast<int>(v >> 32), d);
        const uint32_t l = __shfl_xor(static_cast<int>(static_cast<uint32_t>(v)), d);
        v = kmax(v, (static_cast<uint64_t>(h) << 32) | l);
    }
    if ((threadIdx.x & 63) == 0) sred[threadIdx.x >> 6] = v;
    __syncthreads();
    v = kmax(kmax(sred[0], sred[1]), kmax(sred[2], sred[3]));
    return v;
}

struct ArgmaxParams {
    const void *logits;  // [batch][K][vocab]
    uint64_t *part;      // [batch][K][S]
    int64_t vocab;
    int K, S;
    int64_t chunk;       // elements per split, a multiple of 8
    int vec;             // rows start on 16-byte boundaries: 16-byte loads
};

template <typename T>
__global__ __launch_bounds__(256) void greedy_argmax_kernel(const ArgmaxParams p) {
    __shared__ uint64_t sred[4];
    const int s = blockIdx.x, k = blockIdx.y, b = blockIdx.z;
    const T *row = static_cast<const T *>(p.logits) + ((int64_t)b * p.K + k) * p.vocab;
    const int64_t lo = (int64_t)s * p.chunk, hi = min(lo + p.chunk, p.vocab);
    // this thread's largest value (order-preserving bits) and its index; each thread walks
    // its indices upwards and keeps a value only when strictly larger, so the lowest index
    // of equal values stays
    uint32_t bo = 0, bi = 0xFFFFFFFFu;
    int64_t tail = lo;
    if (p.vec) {
        constexpr int E = 16 / sizeof(T);  // lo is a multiple of 8, so of E
        constexpr int U = 4;               // 16-byte loads in flight per thread
        const uint4 *row4 = reinterpret_cast<const uint4 *>(row);
        const int64_t v0 = lo / E, v1 = hi / E;
        for (int64_t base = v0 + threadIdx.x; base < v1; base += 256 * U) {
            uint4 w[U];
#pragma unroll
            for (int u = 0; u < U; ++u) w[u] = row4[min(base + u * 256, v1 - 1)];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = base + u * 256;
                if (i < v1) {
#pragma unroll
                    for (int q = 0; q < E; ++q) {
                        const uint32_t o = ordered(element(w[u], q, static_cast<const T *>(nullptr)));
                        if (o > bo) {
                            bo = o;
                            bi = (uint32_t)(i * E + q);
                        }
                    }
                }
            }
        }
        tail = v1 * E;
    }
    for (int64_t i = tail + threadIdx.x; i < hi; i += 256) {
        const uint32_t o = ordered(logit(row[i]));
        if (o > bo) {
            bo = o;
            bi = (uint32_t)i;
        }
    }
    const uint64_t best = block_max_key(argmax_key(bo, bi), sred);
    if (threadIdx.x == 0) p.part[((int64_t)b * p.K + k) * p.S + s] = best;
}

struct GreedyParams {
    CommitParams c;
    const uint64_t *part;   // [batch][K][S]
    const int32_t *draft;   // [batch][K]
    int32_t *accepted;      // [batch] out
    int32_t *tokens;        // [batch][K] out, or null
    int S;
};

template <typename V>
__global__ __launch_bounds__(256) void greedy_commit_kernel(const GreedyParams g) {
    __shared__ uint64_t skey[MIL_KMAX_LIMIT * kGreedySplitsMax];
    __shared__ int32_t stok[MIL_KMAX_LIMIT];
    __shared__ int sj;
    const CommitParams &p = g.c;
    const int k = blockIdx.x, b = blockIdx.y, K = p.K, S = g.S;
    for (int i = threadIdx.x; i < K * S; i += blockDim.x) skey[i] = g.part[(int64_t)b * K * S + i];
    __syncthreads();
    if (threadIdx.x < K) {
        uint64_t m = 0;
        for (int q = 0; q < S; ++q) m = kmax(m, skey[threadIdx.x * S + q]);
        stok[threadIdx.x] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(m));
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int j = 0;
        while (j < K && g.draft[(int64_t)b * K + j] == stok[j]) ++j;
        sj = j;
    }
    __syncthreads();
    const int j = sj;
    if (k == 0) {
        if (threadIdx.x == 0) {
            g.accepted[b] = j;
            p.pending[b] = j;
            p.pos[b] += j;
        }
        if (g.tokens && threadIdx.x < K) g.tokens[(int64_t)b * K + threadIdx.x] = stok[threadIdx.x];
    }
    if (k >= j) return;
    const size_t src = (size_t)b * K + k, dst = (size_t)b * p.k_max + k;
    copy_row<V>(p.px + dst * p.x_row, p.x + src * p.x_row, p.x_row);
    copy_row<V>(p.pB + dst * p.B_row, p.B + src * p.B_row, p.B_row);
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

namespace {
CommitParams commit_params(const CacheImpl &c, int K, const int32_t *accepted, const void *x, const void *B,
                           const void *dt) {
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
    return p;
}
}  // namespace

hipError_t launch_commit_tree(const CacheImpl &c, int K, const int32_t *parent, const int32_t *accepted_node,
                              const void *x, const void *B, const void *dt, hipStream_t s) {
    TreeCommitParams tp;
    tp.c = commit_params(c, K, nullptr, x, B, dt);
    tp.parent = parent;
    tp.accepted_node = accepted_node;
    const bool v16 = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(B)) & 15) == 0;
    trace_begin(c, MIL_TRACE_COMMIT, s);
    if (v16)
        hipLaunchKernelGGL(ssm_commit_tree_kernel<uint4>, dim3(K, c.dims.batch), dim3(256), 0, s, tp);
    else
        hipLaunchKernelGGL(ssm_commit_tree_kernel<uint32_t>, dim3(K, c.dims.batch), dim3(256), 0, s, tp);
    trace_end(c, MIL_TRACE_COMMIT, s);
    return hipGetLastError();
}

hipError_t launch_commit(const CacheImpl &c, int K, const int32_t *accepted, const void *x,
                         const void *B, const void *dt, hipStream_t s) {
    const CommitParams p = commit_params(c, K, accepted, x, B, dt);
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

// Vocabulary splits per (slot, draft) row: enough workgroups to spread over the chip
// (about 2048 in all), each split at least 2048 logits.
int greedy_splits(int batch, int K, int64_t vocab) {
    const int64_t rows = (int64_t)batch * K;
    int64_t S = (2048 + rows - 1) / rows;
    S = std::min<int64_t>(S, (vocab + 2047) / 2048);
    return (int)std::max<int64_t>(1, std::min<int64_t>(S, kGreedySplitsMax));
}

int64_t greedy_workspace_bytes(int batch, int K) {
    return ((int64_t)batch * K * kGreedySplitsMax * 8 + 255) / 256 * 256;
}

hipError_t launch_commit_greedy(const CacheImpl &c, int K, const int32_t *draft, const void *logits, int vocab,
                                int logits_dtype, int32_t *accepted, int32_t *tokens, const void *x, const void *B,
                                const void *dt, void *ws, hipStream_t s) {
    const int batch = c.dims.batch;
    const int S = greedy_splits(batch, K, vocab);
    const int le = logits_dtype == MIL_BF16 ? 2 : 4;
    ArgmaxParams a;
    a.logits = logits;
    a.part = static_cast<uint64_t *>(ws);
    a.vocab = vocab;
    a.K = K;
    a.S = S;
    a.chunk = ((vocab + S - 1) / S + 7) / 8 * 8;
    a.vec = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) && ((int64_t)vocab * le % 16 == 0);
    trace_begin(c, MIL_TRACE_ACCEPT, s);
    if (logits_dtype == MIL_BF16)
        hipLaunchKernelGGL(greedy_argmax_kernel<uint16_t>, dim3(S, K, batch), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(greedy_argmax_kernel<float>, dim3(S, K, batch), dim3(256), 0, s, a);
    trace_end(c, MIL_TRACE_ACCEPT, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    GreedyParams g;
    g.c = commit_params(c, K, nullptr, x, B, dt);
    g.part = a.part;
    g.draft = draft;
    g.accepted = accepted;
    g.tokens = tokens;
    g.S = S;
    const bool v16 = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(B)) & 15) == 0;
    trace_begin(c, MIL_TRACE_COMMIT, s);
    if (v16)
        hipLaunchKernelGGL(greedy_commit_kernel<uint4>, dim3(K, batch), dim3(256), 0, s, g);
    else
        hipLaunchKernelGGL(greedy_commit_kernel<uint32_t>, dim3(K, batch), dim3(256), 0, s, g);
    trace_end(c, MIL_TRACE_COMMIT, s);
    return hipGetLastError();
}

hipError_t launch_clear_pending(const CacheImpl &c, hipStream_t s) {
    const int n = c.dims.batch;
    hipLaunchKernelGGL(clear_pending_kernel, dim3((n + 255) / 256), dim3(256), 0, s, cache_pending(c), n);
    return hipGetLastError();
}

}  // namespace mil
