// Internal declarations shared by the host ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mil_ssm.h"

namespace mil {

constexpr uint32_t kCacheMagic = 0x4d494c53u;  // "MILS"
enum Phase : int32_t { kUninit = 0, kReady = 1, kVerified = 2 };

// Host-side view of a cache descriptor (lives inside mil_ssm_cache::opaque).
struct CacheImpl {
    uint32_t magic;
    int32_t phase;
    mil_ssm_dims dims;
    int32_t k_max;
    int32_t dtype;
    int32_t verified_k;
    int32_t pad_;
    char *base;
    int64_t bytes;
    mil_ssm_layout lay;
    int32_t trace_kernel;  // mil_trace_kernel, MIL_TRACE_OFF when not tracing
    int32_t pad2_;
    hipEvent_t trace_start, trace_stop;
};

// Event records around one launch of kernel `id` when the descriptor traces it.
inline void trace_begin(const CacheImpl &c, int id, hipStream_t s) {
    if (c.trace_kernel == id && c.trace_start) (void)hipEventRecord(c.trace_start, s);
}
inline void trace_end(const CacheImpl &c, int id, hipStream_t s) {
    if (c.trace_kernel == id && c.trace_stop) (void)hipEventRecord(c.trace_stop, s);
}
static_assert(sizeof(CacheImpl) <= sizeof(mil_ssm_cache), "cache descriptor too large");

inline float *cache_state(const CacheImpl &c) { return reinterpret_cast<float *>(c.base + c.lay.state_off); }
inline void *cache_pend_x(const CacheImpl &c) { return c.base + c.lay.pend_x_off; }
inline void *cache_pend_B(const CacheImpl &c) { return c.base + c.lay.pend_B_off; }
inline void *cache_pend_dt(const CacheImpl &c) { return c.base + c.lay.pend_dt_off; }
inline int32_t *cache_pos(const CacheImpl &c) { return reinterpret_cast<int32_t *>(c.base + c.lay.pos_off); }
inline int32_t *cache_pending(const CacheImpl &c) { return reinterpret_cast<int32_t *>(c.base + c.lay.pending_off); }
inline int32_t *cache_err(const CacheImpl &c) { return reinterpret_cast<int32_t *>(c.base + c.lay.err_off); }
// single-launch prefill handoff words: [slot][head][kScanSlabs][kScanRow], zeroed when the
// cache is set up.  Per row: kScanChunks chunk flags, then the row's epoch (the epoch of
// the row's last launch, 1..2^30-1).  A launch takes the next epoch e, writes its flags
// as (e << 2) | kind and stores e as the row's epoch once every flag of the launch is up,
// so the value that marks a launch lives on the device with the cache (graph replays and
// byte copies of a cache carry it along)
constexpr int kScanSlabs = 8;
constexpr int kScanChunks = 64;  // chunks per launch of the single-launch prefill (longer prompts: more launches)
constexpr int kScanRow = kScanChunks + 4;  // words per (slot, head, slab) row: flags, epoch, pad
constexpr int kScanEpoch = kScanChunks;    // index of the epoch word in a row
// the next word of each slot's first row (head 0, slab 0): the arrival count of a greedy
// commit's workgroups for that slot, 0 between calls (the last arrival resets it)
constexpr int kGreedyArriveWord = kScanEpoch + 1;
inline int32_t *cache_scan(const CacheImpl &c) { return reinterpret_cast<int32_t *>(c.base + c.lay.scan_off); }
inline int32_t *cache_append(const CacheImpl &c) { return reinterpret_cast<int32_t *>(c.base + c.lay.append_off); }
inline int elt_bytes(int32_t dtype) { return dtype == MIL_BF16 ? 2 : 4; }

// ---- launchers (each returns the launch's hipError_t) ----

// Zero `words` 32-bit words starting at p (a plain fill kernel, safe under graph capture).
hipError_t launch_fill_zero(void *p, int64_t words, hipStream_t s);

// Fold every slot's pending rows into the stored state, then, when K > 0, emit y for
// K drafts from that state.  K == 0 is the fold alone (x/B/C/dt/y unused).
// With `parent` ([batch][K], -1..k-1), the drafts form a tree and each one's output runs
// over its root path; null means a chain.
hipError_t launch_verify(const CacheImpl &c, int K, const void *x, const void *B, const void *C,
                         const void *dt, const float *A, const float *D, float *y, hipStream_t s,
                         const int32_t *parent = nullptr);
// A verify launch shape exists for these sizes (K drafts, up to kmax pending rows).
bool verify_supported(int batch, int H, int P, int N, int K, int kmax);

// Check accepted[b] in 0..K, copy the accepted draft rows into the pending area,
// set pending[b] = accepted[b], pos[b] += accepted[b]; a bad value sets err[b] and pending[b] = 0.
hipError_t launch_commit_layers(const CacheImpl *const *cs, int n, int K, const int32_t *accepted,
                                const void *const *x, const void *const *B, const void *const *dt, hipStream_t s);
hipError_t launch_commit(const CacheImpl &c, int K, const int32_t *accepted, const void *x,
                         const void *B, const void *dt, hipStream_t s);

// The commit of a tree round: the root path of accepted_node[b] (-1..K-1, -1 = none)
// becomes the pending rows in root-first order; a bad node or parent link sets err[b].
hipError_t launch_commit_tree(const CacheImpl &c, int K, const int32_t *parent, const int32_t *accepted_node,
                              const void *x, const void *B, const void *dt, hipStream_t s);

// pending[b] = 0 for every slot (after a fold that has consumed them).
hipError_t launch_clear_pending(const CacheImpl &c, hipStream_t s);
// Greedy acceptance fused into the commit (argmax over the vocabulary per draft position).
int64_t greedy_workspace_bytes(int batch, int K);
hipError_t launch_commit_greedy(const CacheImpl &c, int K, const int32_t *draft, const void *logits, int vocab,
                                int logits_dtype, int32_t *accepted, int32_t *tokens, const void *x, const void *B,
                                const void *dt, void *ws, hipStream_t s);
// Device address of the calling thread's current device's no-alloc greedy scratch
// (MIL_GREEDY_NOALLOC_SCRATCH_BYTES), looked up on the first call per device.
hipError_t greedy_noalloc_scratch(void **out);

// Chunked prefill (three phases: chunk states, inter-chunk pass, chunk outputs).  The
// inter-chunk pass also sets pos[slot] = L (or += L when cont) for the prefilled slots
// and pending = 0 (for every slot when cont: the fold before it consumed them all).
int64_t prefill_workspace_bytes(const mil_ssm_dims &d, int nseq, int L, int chunk);
hipError_t launch_prefill(const CacheImpl &c, int slot0, int nseq, int L, int chunk, const void *x,
                          const void *B, const void *C, const void *dt, const float *A,
                          const float *D, float *y, void *ws, bool cont, hipStream_t s);

// Matrix-core form of the three prefill phases (bf16 inputs; see prefill_mfma_supported).
bool prefill_mfma_supported(int Q, int N, int P);
// The matrix-core prefill of these sizes runs as one launch (chunk states, handoff, outputs).
bool prefill_single_launch(int nseq, int L, int chunk, int H, int P, int N);
hipError_t launch_prefill_mfma(const CacheImpl &c, int slot0, int nseq, int L, int chunk, const void *x,
                               const void *B, const void *C, const void *dt, const float *A,
                               const float *D, float *y, void *ws, bool cont, hipStream_t s);

// Input projections x, B, C, dt = softplus(.) of T rows of width d (one bf16 GEMM over four
// weight blocks; fp32 partial sums in `ws` when the inputs are split over workgroups).
bool project_supported(const mil_ssm_dims &d, int T, int dmodel);
int64_t project_workspace_bytes(const mil_ssm_dims &d, int T, int dmodel);
hipError_t launch_project(const mil_ssm_dims &d, int T, int dmodel, const void *u, const void *const w[4],
                          const float *bias, bool out_bf16, void *const out[4], void *ws, hipStream_t s);

}  // namespace mil
