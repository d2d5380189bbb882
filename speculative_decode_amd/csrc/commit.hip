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
#include <mutex>

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
    const int32_t *append;            // [batch] first pending row this commit writes (set by the verify)
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
// is reported in err[b] and leaves pos alone; pending becomes the rows still pending (0
// after the verify wrote the state back, else its pending count): nothing of this round
// is kept.
// The row is read into registers before j is known, so that the two reads overlap
// instead of the copy waiting for j first (a row past j is read and dropped); rows
// longer than kCommitRegs vectors per thread copy their remainder afterwards.
constexpr int kCommitRegs = 4;
typedef int i32x4v __attribute__((ext_vector_type(4)));  // 16 bytes that arrays keep in registers
template <typename V> struct RegVec { typedef V type; };
template <> struct RegVec<uint4> { typedef i32x4v type; };

template <typename VM>
__device__ __forceinline__ void commit_rows(const CommitParams &p, const int k, const int b) {
    typedef typename RegVec<VM>::type V;
    const int tid = threadIdx.x, nt = blockDim.x;
    // 0 when the verify wrote the state back, else its pending count (at most k_max - K by
    // the verify's rule; clamped so that no value in the buffer can place a row outside it)
    const int base = min(max(p.append[b], 0), p.k_max - p.K);
    const size_t src = (size_t)b * p.K + k, dst = (size_t)b * p.k_max + base + k;
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
            p.pending[b] = base + j;
            p.pos[b] += j;
        } else {
            atomicOr(p.err + b, MIL_DEVERR_ACCEPT);  // keeps bits set by earlier calls
            p.pending[b] = base;  // the rows still pending stay
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

template <typename VM>
__global__ __launch_bounds__(256) void ssm_commit_kernel(const CommitParams p) {
    commit_rows<VM>(p, blockIdx.x, blockIdx.y);
}

// The commit of several layers' caches in one launch, grid (K, batch, layers): layer z's
// workgroups do exactly what ssm_commit_kernel's do for its cache.  The per-layer pointers
// travel in the kernel arguments (MIL_COMMIT_LAYERS_MAX layers, under 2.5 KB).
struct LayerPtrs {
    const char *x, *B, *dt;
    char *px, *pB, *pdt;
    int32_t *pos, *pending, *err;
    const int32_t *append;
};
struct LayersCommitParams {
    CommitParams shared;  // accepted, row sizes, K, k_max (the pointers are per layer)
    LayerPtrs layer[MIL_COMMIT_LAYERS_MAX];
};
static_assert(sizeof(LayersCommitParams) <= 4096, "kernel arguments are limited to 4 KB");

template <typename VM>
__global__ __launch_bounds__(256) void ssm_commit_layers_kernel(const LayersCommitParams lp) {
    const LayerPtrs &l = lp.layer[blockIdx.z];
    CommitParams p = lp.shared;
    p.x = l.x;
    p.B = l.B;
    p.dt = l.dt;
    p.px = l.px;
    p.pB = l.pB;
    p.pdt = l.pdt;
    p.pos = l.pos;
    p.pending = l.pending;
    p.err = l.err;
    p.append = l.append;
    commit_rows<VM>(p, blockIdx.x, blockIdx.y);
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
    // 0 when the verify wrote the state back, else its pending count (at most k_max - K by
    // the verify's rule; clamped so that no value in the buffer can place a row outside it)
    const int base = min(max(p.append[b], 0), p.k_max - p.K);
    if (k == 0 && threadIdx.x == 0) {
        if (!sbad) {
            p.pending[b] = base + j;
            p.pos[b] += j;
        } else {
            atomicOr(p.err + b, sbad);  // keeps bits set by earlier calls
            p.pending[b] = base;        // the rows still pending stay
        }
    }
    if (k >= j) return;
    const size_t src = (size_t)b * p.K + spath[k], dst = (size_t)b * p.k_max + base + k;
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
// logits at its position).  One launch, grid (S, K, batch); workgroup (s, k, b):
//   1. reduces split s of logits row (b, k) to one 64-bit key and publishes it in
//      ws[b][k][s];
//   2. counts itself in the slot's arrival word;
//   3. copies its share (1/S) of draft row k of slot b into the pending area, after the
//      rows still pending: every draft is copied, and the rows past the accepted ones lie
//      beyond the new pending count, where nothing reads them;
//   4. if it was the slot's last workgroup, takes the max of the S keys per position (the
//      argmax token), compares the drafts with them, finds the accepted length j and does
//      the slot's bookkeeping.
// Keys and arrival words cross workgroups through agent-coherent accesses (relaxed
// agent-scope atomics, which bypass the non-coherent cache levels), and a key's store
// completes before its workgroup counts itself; the last workgroup sets the word back to
// 0, so that every call (and every replay of a captured one) starts from zero.  The
// copies need no ordering: the verify before this commit has finished reading the area.
// Key = (order-preserving bits of the value) << 32 | (0xFFFFFFFF - index): the largest
// key is the largest value, ties going to the lowest index, so the result does not depend
// on how the vocabulary is split or in which order partial maxima meet.  Integer and
// compare-only work: exact.  The argmax rule: -0 and +0 are one value, and every NaN
// (either sign, any payload) ranks above every number, the lowest id first among NaNs.
constexpr int kGreedySplitsMax = 64;

__device__ __forceinline__ uint32_t ordered(float v) {  // monotonic in v, +-0 and NaNs canonical
    const uint32_t u = __float_as_uint(v);
    const uint32_t mag = u & 0x7fffffffu;
    if (mag > 0x7f800000u) return 0xffffffffu;  // any NaN: above +inf (0xff800000)
    if (mag == 0u) return 0x80000000u;          // -0 keyed as +0
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

struct GreedyParams {
    CommitParams c;          // the drafts' rows, the pending area, pos / pending / append
    const void *logits;      // [batch][K][vocab]
    uint64_t *part;          // [batch][K][S] published keys
    int32_t *arrive;         // slot b's arrival word: arrive[b * arrive_stride]
    int64_t arrive_stride;
    const int32_t *draft;    // [batch][K]
    int32_t *accepted;       // [batch] out
    int32_t *tokens;         // [batch][K] out, or null
    int64_t vocab;
    int64_t chunk;           // logits per split, a multiple of 8
    int S;
    int vec;                 // logits rows start on 16-byte boundaries: 16-byte loads
};

// Share s of S of a row of `bytes` (a multiple of sizeof(V)), one vector per thread per pass.
template <typename V>
__device__ __forceinline__ void copy_share(char *dst, const char *src, int bytes, int s, int S) {
    const V *sv = reinterpret_cast<const V *>(src);
    V *dv = reinterpret_cast<V *>(dst);
    const int n = bytes / (int)sizeof(V), per = (n + S - 1) / S, lo = s * per, hi = min(n, lo + per);
    for (int i = lo + threadIdx.x; i < hi; i += blockDim.x) dv[i] = sv[i];
}

template <typename T, typename V>
__global__ __launch_bounds__(256) void greedy_accept_kernel(const GreedyParams g) {
    __shared__ uint64_t sred[4];
    __shared__ uint64_t skey[MIL_KMAX_LIMIT * kGreedySplitsMax];
    __shared__ int32_t stok[MIL_KMAX_LIMIT], sdraft[MIL_KMAX_LIMIT];
    __shared__ int slast;
    const CommitParams &p = g.c;
    const int s = blockIdx.x, k = blockIdx.y, b = blockIdx.z, K = p.K, S = g.S;
    // the slot's draft tokens, read up front by every workgroup (a few bytes), so that the
    // last one compares them without a global read per position
    const int32_t mydraft = threadIdx.x < K ? g.draft[(int64_t)b * K + threadIdx.x] : 0;
    // where this slot's rows of the round go: 0 when the verify wrote the state back, else
    // its pending count (at most k_max - K by the verify's rule; clamped so that no value
    // in the buffer can place a row outside the area)
    const int base = min(max(p.append[b], 0), p.k_max - K);

    // ---- 1. this split's largest logit, as a key ----
    const T *row = static_cast<const T *>(g.logits) + ((int64_t)b * K + k) * g.vocab;
    const int64_t lo = (int64_t)s * g.chunk, hi = min(lo + g.chunk, g.vocab);
    // this thread's largest value (order-preserving bits) and its index; each thread walks
    // its indices upwards and keeps a value only when strictly larger, so the lowest index
    // of equal values stays
    uint32_t bo = 0, bi = 0xFFFFFFFFu;
    int64_t tail = lo;
    if (g.vec) {
        constexpr int E = 16 / sizeof(T);  // lo is a multiple of 8, so of E
        constexpr int U = 8;               // 16-byte loads in flight per thread
        const uint4 *row4 = reinterpret_cast<const uint4 *>(row);
        const int64_t v0 = lo / E, v1 = hi / E;
        for (int64_t base4 = v0 + threadIdx.x; base4 < v1; base4 += 256 * U) {
            uint4 w[U];
#pragma unroll
            for (int u = 0; u < U; ++u) w[u] = row4[min(base4 + u * 256, v1 - 1)];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = base4 + u * 256;
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

    // ---- 2. publish the key and count in (the key's store complete first: the wait comes
    // before the copies below, which need no order, so it does not wait for them) ----
    int32_t *arrive = g.arrive + (size_t)b * g.arrive_stride;
    const size_t src = (size_t)b * K + k, dst = (size_t)b * p.k_max + base + k;
    if (threadIdx.x == 0) {
        __hip_atomic_store(g.part + src * S + s, best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        slast = __hip_atomic_fetch_add(arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == K * S - 1;
    }
    // ---- 3. this split's share of draft row k, after the rows still pending: at once in
    // every workgroup but the slot's last, which copies after deciding (its key reads would
    // otherwise wait behind these stores) ----
    auto copy = [&]() {
        copy_share<V>(p.px + dst * p.x_row, p.x + src * p.x_row, p.x_row, s, S);
        copy_share<V>(p.pB + dst * p.B_row, p.B + src * p.B_row, p.B_row, s, S);
        if (s == 0) {
            const uint16_t *ds = reinterpret_cast<const uint16_t *>(p.dt + src * p.dt_row);
            uint16_t *dd = reinterpret_cast<uint16_t *>(p.pdt + dst * p.dt_row);
            for (int i = threadIdx.x; i < p.dt_row / 2; i += blockDim.x) dd[i] = ds[i];
        }
    };
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // slast is visible
    if (!slast) {
        copy();
        return;
    }
    // ---- 4. the slot's last workgroup decides ----
    if (threadIdx.x == 0) __hip_atomic_store(arrive, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = threadIdx.x; i < K * S; i += blockDim.x)
        skey[i] = __hip_atomic_load(g.part + (size_t)b * K * S + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x < K) sdraft[threadIdx.x] = mydraft;
    __syncthreads();
    if (threadIdx.x < K) {
        uint64_t m = 0;
        for (int q = 0; q < S; ++q) m = kmax(m, skey[threadIdx.x * S + q]);
        stok[threadIdx.x] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(m));
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int j = 0;
        while (j < K && sdraft[j] == stok[j]) ++j;
        g.accepted[b] = j;
        p.pending[b] = base + j;
        p.pos[b] += j;
    }
    if (g.tokens && threadIdx.x < K) g.tokens[(int64_t)b * K + threadIdx.x] = stok[threadIdx.x];
    copy();
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
    p.append = cache_append(c);
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

hipError_t launch_commit_layers(const CacheImpl *const *cs, int n, int K, const int32_t *accepted,
                                const void *const *x, const void *const *B, const void *const *dt, hipStream_t s) {
    bool v16 = true;
    for (int l = 0; l < n; ++l)
        v16 = v16 && ((reinterpret_cast<uintptr_t>(x[l]) | reinterpret_cast<uintptr_t>(B[l])) & 15) == 0;
    for (int l0 = 0; l0 < n; l0 += MIL_COMMIT_LAYERS_MAX) {
        const int nl = std::min(n - l0, MIL_COMMIT_LAYERS_MAX);
        LayersCommitParams lp;
        lp.shared = commit_params(*cs[l0], K, accepted, nullptr, nullptr, nullptr);
        for (int l = 0; l < MIL_COMMIT_LAYERS_MAX; ++l) {
            const int li = l0 + std::min(l, nl - 1);  // unused entries repeat the last layer
            const CommitParams q = commit_params(*cs[li], K, accepted, x[li], B[li], dt[li]);
            lp.layer[l] = LayerPtrs{q.x, q.B, q.dt, q.px, q.pB, q.pdt, q.pos, q.pending, q.err, q.append};
        }
        const CacheImpl &c0 = *cs[l0];
        trace_begin(c0, MIL_TRACE_COMMIT, s);
        if (v16)
            hipLaunchKernelGGL(ssm_commit_layers_kernel<uint4>, dim3(K, c0.dims.batch, nl), dim3(256), 0, s, lp);
        else
            hipLaunchKernelGGL(ssm_commit_layers_kernel<uint32_t>, dim3(K, c0.dims.batch, nl), dim3(256), 0, s, lp);
        trace_end(c0, MIL_TRACE_COMMIT, s);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
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
// (about 1024 in all, four per compute unit: against 2048 smaller ones, a shorter dispatch
// ramp with as many loads in flight), each split at least 2048 logits.
int greedy_splits(int batch, int K, int64_t vocab) {
    const int64_t rows = (int64_t)batch * K;
    int64_t S = (1024 + rows - 1) / rows;
    S = std::min<int64_t>(S, (vocab + 2047) / 2048);
    return (int)std::max<int64_t>(1, std::min<int64_t>(S, kGreedySplitsMax));
}

int64_t greedy_workspace_bytes(int batch, int K) {
    return ((int64_t)batch * K * kGreedySplitsMax * 8 + 255) / 256 * 256;
}

// ---- the greedy commit's scratch for callers that cannot allocate ----
// One array per GPU, in the library's own device memory (held until the process ends).
// Host code never passes `scratch` itself to a kernel: its name is a host-side stand-in,
// not a device address.  The device address is looked up once per device, with that
// device current, and kept; kernels get that address, as they get a workspace.
static __device__ __align__(256) uint64_t scratch[MIL_GREEDY_NOALLOC_SCRATCH_BYTES / 8];
static_assert(MIL_GREEDY_NOALLOC_MAX_ROWS * kGreedySplitsMax * 8 <= MIL_GREEDY_NOALLOC_SCRATCH_BYTES,
              "the no-alloc scratch holds the partial keys of its largest accepted size");

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t greedy_noalloc_scratch(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_commit_greedy(const CacheImpl &c, int K, const int32_t *draft, const void *logits, int vocab,
                                int logits_dtype, int32_t *accepted, int32_t *tokens, const void *x, const void *B,
                                const void *dt, void *ws, hipStream_t s) {
    const int batch = c.dims.batch;
    const int S = greedy_splits(batch, K, vocab);
    const int le = logits_dtype == MIL_BF16 ? 2 : 4;
    GreedyParams g;
    g.c = commit_params(c, K, nullptr, x, B, dt);
    g.logits = logits;
    g.part = static_cast<uint64_t *>(ws);
    // slot b's arrival word: a spare word of its first prefill handoff row (head 0, slab 0)
    g.arrive = cache_scan(c) + kGreedyArriveWord;
    g.arrive_stride = (int64_t)c.dims.nheads * kScanSlabs * kScanRow;
    g.draft = draft;
    g.accepted = accepted;
    g.tokens = tokens;
    g.vocab = vocab;
    g.S = S;
    g.chunk = ((vocab + S - 1) / S + 7) / 8 * 8;
    g.vec = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) && ((int64_t)vocab * le % 16 == 0);
    // draft rows copied 16 bytes at a time when x and B are 16-byte aligned
    const bool v16 = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(B)) & 15) == 0;
    const dim3 grid(S, K, batch);
    trace_begin(c, MIL_TRACE_ACCEPT, s);
    if (logits_dtype == MIL_BF16) {
        if (v16)
            hipLaunchKernelGGL((greedy_accept_kernel<uint16_t, uint4>), grid, dim3(256), 0, s, g);
        else
            hipLaunchKernelGGL((greedy_accept_kernel<uint16_t, uint32_t>), grid, dim3(256), 0, s, g);
    } else {
        if (v16)
            hipLaunchKernelGGL((greedy_accept_kernel<float, uint4>), grid, dim3(256), 0, s, g);
        else
            hipLaunchKernelGGL((greedy_accept_kernel<float, uint32_t>), grid, dim3(256), 0, s, g);
    }
    trace_end(c, MIL_TRACE_ACCEPT, s);
    return hipGetLastError();
}

hipError_t launch_clear_pending(const CacheImpl &c, hipStream_t s) {
    const int n = c.dims.batch;
    hipLaunchKernelGGL(clear_pending_kernel, dim3((n + 255) / 256), dim3(256), 0, s, cache_pending(c), n);
    return hipGetLastError();
}

}  // namespace mil
