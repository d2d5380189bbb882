// C ABI entry points: argument and protocol checks, cache carving, dispatch to the
// kernel launchers.  Every check runs before any work is enqueued.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "ssm_internal.h"

using namespace mil;

namespace {

constexpr int64_t kAlign = 256;

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

int check_dims(const mil_ssm_dims *d) {
    if (!d) return MIL_E_INVALID;
    if (d->batch < 1 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 || d->ngroups < 1)
        return MIL_E_INVALID;
    if (d->nheads % d->ngroups != 0) return MIL_E_INVALID;
    if (!pow2_in(d->headdim, 16, 256) || !pow2_in(d->dstate, 16, 256)) return MIL_E_UNSUPPORTED;
    return MIL_OK;
}

int check_dtype(int32_t dtype) { return (dtype == MIL_F32 || dtype == MIL_BF16) ? MIL_OK : MIL_E_INVALID; }


CacheImpl *impl(mil_ssm_cache *c) {
    if (!c) return nullptr;
    CacheImpl *ci = reinterpret_cast<CacheImpl *>(c->opaque);
    return ci->magic == kCacheMagic ? ci : nullptr;
}
const CacheImpl *impl(const mil_ssm_cache *c) {
    if (!c) return nullptr;
    const CacheImpl *ci = reinterpret_cast<const CacheImpl *>(c->opaque);
    return ci->magic == kCacheMagic ? ci : nullptr;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? MIL_OK : MIL_E_HIP; }

// MIL_SSM_DEBUG=1 (any value but "0"): verbose host checks.  A call that fails prints its
// name and status on stderr; a call that enqueued work then synchronizes its stream
// (unless the stream is being captured into a graph), reports a failed launch as
// MIL_E_HIP, and prints every slot whose device error word is set in the caches it used
// (the status returned stays the call's own).
bool debug_on() {
    static const bool on = [] {
        const char *e = getenv("MIL_SSM_DEBUG");
        return e != nullptr && e[0] != '\0' && strcmp(e, "0") != 0;
    }();
    return on;
}

int debug_after(const char *fn, int st, bool enqueued, mil_stream_t stream, mil_ssm_cache *const *caches, int n);

}  // namespace

extern "C" {

const char *mil_status_string(int status) {
    switch (status) {
        case MIL_OK: return "ok";
        case MIL_E_INVALID: return "invalid argument";
        case MIL_E_ALIGN: return "misaligned device buffer";
        case MIL_E_ORDER: return "call out of protocol order";
        case MIL_E_UNSUPPORTED: return "unsupported shape";
        case MIL_E_HIP: return "HIP runtime error";
        case MIL_E_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

static int mil_ssm_supported_impl(const mil_ssm_dims *dims, int32_t dtype) {
    int st = check_dims(dims);
    if (st != MIL_OK) return st;
    st = check_dtype(dtype);
    if (st != MIL_OK) return st;
    if (!verify_supported(dims->batch, dims->nheads, dims->headdim, dims->dstate, 1, 1))
        return MIL_E_UNSUPPORTED;
    return MIL_OK;
}

int mil_ssm_supported(const mil_ssm_dims *dims, int32_t dtype) {
    const int st = mil_ssm_supported_impl(dims, dtype);
    return debug_after("mil_ssm_supported", st, false, nullptr, nullptr, 0);
}

static int mil_ssm_cache_layout_impl(const mil_ssm_dims *d, int32_t k_max, int32_t dtype, mil_ssm_layout *out) {
    int st = check_dims(d);
    if (st != MIL_OK) return st;
    if ((st = check_dtype(dtype)) != MIL_OK) return st;
    if (!out || k_max < 1 || k_max > MIL_KMAX_LIMIT) return MIL_E_INVALID;
    const int64_t e = elt_bytes(dtype);
    const int64_t Bt = d->batch, H = d->nheads, P = d->headdim, N = d->dstate, G = d->ngroups;
    mil_ssm_layout L;
    int64_t off = 0;
    L.state_off = off;
    L.state_head_stride = round_up(N * P * 4, kAlign);
    off += Bt * H * L.state_head_stride;
    L.pend_x_off = off = round_up(off, kAlign);
    off += Bt * k_max * H * P * e;
    L.pend_B_off = off = round_up(off, kAlign);
    off += Bt * k_max * G * N * e;
    L.pend_dt_off = off = round_up(off, kAlign);
    off += Bt * k_max * H * e;
    L.pos_off = off = round_up(off, kAlign);
    off += Bt * 4;
    L.pending_off = off = round_up(off, kAlign);
    off += Bt * 4;
    L.err_off = off = round_up(off, kAlign);
    off += Bt * 4;
    L.scan_off = off = round_up(off, kAlign);
    off += Bt * H * kScanSlabs * kScanRow * 4;
    L.append_off = off = round_up(off, kAlign);
    off += Bt * 4;
    L.bytes = round_up(off, kAlign);
    *out = L;
    return MIL_OK;
}

int mil_ssm_cache_layout(const mil_ssm_dims *d, int32_t k_max, int32_t dtype, mil_ssm_layout *out) {
    const int st = mil_ssm_cache_layout_impl(d, k_max, dtype, out);
    return debug_after("mil_ssm_cache_layout", st, false, nullptr, nullptr, 0);
}

size_t mil_ssm_cache_bytes(const mil_ssm_dims *d, int32_t k_max, int32_t dtype) {
    mil_ssm_layout L;
    return mil_ssm_cache_layout(d, k_max, dtype, &L) == MIL_OK ? (size_t)L.bytes : 0;
}

namespace {
int describe(mil_ssm_cache *cache, const mil_ssm_dims *d, int32_t k_max, int32_t dtype, void *dev_buf,
             size_t bytes) {
    if (!cache || !dev_buf) return MIL_E_INVALID;
    mil_ssm_layout L;
    int st = mil_ssm_cache_layout(d, k_max, dtype, &L);
    if (st != MIL_OK) return st;
    if ((st = mil_ssm_supported(d, dtype)) != MIL_OK) return st;
    // every K up to k_max needs a verify shape (its LDS grows with K and k_max)
    if (!verify_supported(d->batch, d->nheads, d->headdim, d->dstate, k_max, k_max)) return MIL_E_UNSUPPORTED;
    if (!aligned(dev_buf, kAlign)) return MIL_E_ALIGN;
    if ((int64_t)bytes < L.bytes) return MIL_E_INVALID;
    memset(cache->opaque, 0, sizeof(cache->opaque));
    CacheImpl *c = reinterpret_cast<CacheImpl *>(cache->opaque);
    c->dims = *d;
    c->k_max = k_max;
    c->dtype = dtype;
    c->verified_k = 0;
    c->base = static_cast<char *>(dev_buf);
    c->bytes = L.bytes;
    c->lay = L;
    return MIL_OK;
}
}  // namespace

static int mil_ssm_cache_attach_impl(mil_ssm_cache *cache, const mil_ssm_dims *d, int32_t k_max, int32_t dtype,
                         void *dev_buf, size_t bytes) {
    const int st = describe(cache, d, k_max, dtype, dev_buf, bytes);
    if (st != MIL_OK) return st;
    CacheImpl *c = reinterpret_cast<CacheImpl *>(cache->opaque);
    c->magic = kCacheMagic;
    c->phase = kReady;
    return MIL_OK;
}

int mil_ssm_cache_attach(mil_ssm_cache *cache, const mil_ssm_dims *d, int32_t k_max, int32_t dtype,
                         void *dev_buf, size_t bytes) {
    const int st = mil_ssm_cache_attach_impl(cache, d, k_max, dtype, dev_buf, bytes);
    return debug_after("mil_ssm_cache_attach", st, false, nullptr, nullptr, 0);
}

static int mil_ssm_cache_init_impl(mil_ssm_cache *cache, const mil_ssm_dims *d, int32_t k_max, int32_t dtype,
                       void *dev_buf, size_t bytes, mil_stream_t stream) {
    const int st = describe(cache, d, k_max, dtype, dev_buf, bytes);
    if (st != MIL_OK) return st;
    CacheImpl *c = reinterpret_cast<CacheImpl *>(cache->opaque);
    const mil_ssm_layout &L = c->lay;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // zero the state block and the three counter arrays (the pending token rows are
    // never read before a commit writes them)
    hipError_t e = launch_fill_zero(c->base + L.state_off, (L.pend_x_off - L.state_off) / 4, s);
    if (e == hipSuccess) e = launch_fill_zero(c->base + L.pos_off, (L.bytes - L.pos_off) / 4, s);
    if (e != hipSuccess) return MIL_E_HIP;
    c->magic = kCacheMagic;
    c->phase = kReady;
    return MIL_OK;
}

int mil_ssm_cache_init(mil_ssm_cache *cache, const mil_ssm_dims *d, int32_t k_max, int32_t dtype,
                       void *dev_buf, size_t bytes, mil_stream_t stream) {
    const int st = mil_ssm_cache_init_impl(cache, d, k_max, dtype, dev_buf, bytes, stream);
    return debug_after("mil_ssm_cache_init", st, true, stream, &cache, 1);
}

size_t mil_ssm_prefill_workspace_bytes(const mil_ssm_dims *d, int32_t nseq, int32_t L, int32_t chunk) {
    if (check_dims(d) != MIL_OK || nseq < 1 || L < 1) return 0;
    if (chunk != 64 && chunk != 128 && chunk != 256) return 0;
    return (size_t)prefill_workspace_bytes(*d, nseq, L, chunk);
}

static int mil_ssm_prefill_impl(mil_ssm_cache *cache, int32_t slot0, int32_t nseq, int32_t L, int32_t chunk,
                    const void *x, const void *B, const void *C, const void *dt, const float *A,
                    const float *D, float *y, void *ws, size_t ws_bytes, uint32_t flags,
                    mil_stream_t stream) {
    CacheImpl *c = impl(cache);
    if (!c) return MIL_E_INVALID;
    if (c->phase != kReady) return MIL_E_ORDER;
    if (flags & ~MIL_PREFILL_CONTINUE) return MIL_E_INVALID;
    if (nseq < 1 || slot0 < 0 || slot0 + nseq > c->dims.batch || L < 1) return MIL_E_INVALID;
    if (chunk != 64 && chunk != 128 && chunk != 256) return MIL_E_INVALID;
    if (!x || !B || !C || !dt || !A || !D) return MIL_E_INVALID;
    const int eb = elt_bytes(c->dtype);
    if (!aligned(x, eb) || !aligned(B, eb) || !aligned(C, eb) || !aligned(dt, eb) || !aligned(A, 4) ||
        !aligned(D, 4) || (y && !aligned(y, 4)))
        return MIL_E_ALIGN;
    const int64_t need = prefill_workspace_bytes(c->dims, nseq, L, chunk);
    if (!ws || (int64_t)ws_bytes < need) return MIL_E_WORKSPACE;
    if (!aligned(ws, kAlign)) return MIL_E_ALIGN;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool cont = (flags & MIL_PREFILL_CONTINUE) != 0;
    hipError_t e = hipSuccess;
    if (cont) {
        // fold pending accepted rows of every slot (a no-op where pending == 0)
        e = launch_verify(*c, 0, nullptr, nullptr, nullptr, nullptr, A, D, nullptr, s);
    }
    if (e == hipSuccess) e = launch_prefill(*c, slot0, nseq, L, chunk, x, B, C, dt, A, D, y, ws, cont, s);
    return hip_status(e);
}

int mil_ssm_prefill(mil_ssm_cache *cache, int32_t slot0, int32_t nseq, int32_t L, int32_t chunk,
                    const void *x, const void *B, const void *C, const void *dt, const float *A,
                    const float *D, float *y, void *ws, size_t ws_bytes, uint32_t flags,
                    mil_stream_t stream) {
    const int st = mil_ssm_prefill_impl(cache, slot0, nseq, L, chunk, x, B, C, dt, A, D, y, ws, ws_bytes, flags, stream);
    return debug_after("mil_ssm_prefill", st, true, stream, &cache, 1);
}

static int mil_ssm_verify_impl(mil_ssm_cache *cache, int32_t K, const void *x, const void *B, const void *C,
                   const void *dt, const float *A, const float *D, float *y, mil_stream_t stream) {
    CacheImpl *c = impl(cache);
    if (!c) return MIL_E_INVALID;
    if (c->phase != kReady) return MIL_E_ORDER;
    if (K < 1 || K > c->k_max) return MIL_E_INVALID;
    if (!x || !B || !C || !dt || !A || !D || !y) return MIL_E_INVALID;
    const int eb = elt_bytes(c->dtype);
    if (!aligned(x, eb) || !aligned(B, eb) || !aligned(C, eb) || !aligned(dt, eb) || !aligned(A, 4) ||
        !aligned(D, 4) || !aligned(y, 4))
        return MIL_E_ALIGN;
    hipError_t e = launch_verify(*c, K, x, B, C, dt, A, D, y, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return MIL_E_HIP;
    c->phase = kVerified;
    c->verified_k = K;
    return MIL_OK;
}

int mil_ssm_verify(mil_ssm_cache *cache, int32_t K, const void *x, const void *B, const void *C,
                   const void *dt, const float *A, const float *D, float *y, mil_stream_t stream) {
    const int st = mil_ssm_verify_impl(cache, K, x, B, C, dt, A, D, y, stream);
    return debug_after("mil_ssm_verify", st, true, stream, &cache, 1);
}

static int mil_ssm_commit_impl(mil_ssm_cache *cache, int32_t K, const int32_t *accepted, const void *x,
                   const void *B, const void *dt, const float *A, const float *D, uint32_t flags,
                   mil_stream_t stream) {
    CacheImpl *c = impl(cache);
    if (!c) return MIL_E_INVALID;
    if (c->phase != kVerified) return MIL_E_ORDER;
    if (flags & ~MIL_COMMIT_MATERIALIZE) return MIL_E_INVALID;
    if (K != c->verified_k) return MIL_E_INVALID;
    if (!accepted || !x || !B || !dt) return MIL_E_INVALID;
    const bool mat = (flags & MIL_COMMIT_MATERIALIZE) != 0;
    if (mat && (!A || !D)) return MIL_E_INVALID;
    const int eb = elt_bytes(c->dtype);
    // x and B rows are copied as 32-bit words
    if (!aligned(accepted, 4) || !aligned(x, 4) || !aligned(B, 4) || !aligned(dt, eb))
        return MIL_E_ALIGN;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = launch_commit(*c, K, accepted, x, B, dt, s);
    if (e == hipSuccess && mat) {
        e = launch_verify(*c, 0, nullptr, nullptr, nullptr, nullptr, A, D, nullptr, s);
        if (e == hipSuccess) e = launch_clear_pending(*c, s);
    }
    if (e != hipSuccess) return MIL_E_HIP;
    c->phase = kReady;
    c->verified_k = 0;
    return MIL_OK;
}

int mil_ssm_commit(mil_ssm_cache *cache, int32_t K, const int32_t *accepted, const void *x,
                   const void *B, const void *dt, const float *A, const float *D, uint32_t flags,
                   mil_stream_t stream) {
    const int st = mil_ssm_commit_impl(cache, K, accepted, x, B, dt, A, D, flags, stream);
    return debug_after("mil_ssm_commit", st, true, stream, &cache, 1);
}

static int mil_ssm_commit_layers_impl(mil_ssm_cache *const *caches, int32_t n, int32_t K, const int32_t *accepted,
                          const void *const *x, const void *const *B, const void *const *dt,
                          mil_stream_t stream) {
    if (!caches || n < 1 || !accepted || !x || !B || !dt) return MIL_E_INVALID;
    std::vector<CacheImpl *> cs((size_t)n);
    for (int l = 0; l < n; ++l) {
        cs[l] = impl(caches[l]);
        if (!cs[l] || !x[l] || !B[l] || !dt[l]) return MIL_E_INVALID;
        for (int q = 0; q < l; ++q)
            if (cs[q] == cs[l]) return MIL_E_INVALID;  // each cache once
    }
    const CacheImpl &c0 = *cs[0];
    for (int l = 0; l < n; ++l) {
        const CacheImpl &c = *cs[l];
        if (c.dims.batch != c0.dims.batch || c.dims.nheads != c0.dims.nheads || c.dims.headdim != c0.dims.headdim ||
            c.dims.dstate != c0.dims.dstate || c.dims.ngroups != c0.dims.ngroups || c.dtype != c0.dtype ||
            c.k_max != c0.k_max)
            return MIL_E_INVALID;
    }
    for (int l = 0; l < n; ++l)
        if (cs[l]->phase != kVerified) return MIL_E_ORDER;
    for (int l = 0; l < n; ++l)
        if (K != cs[l]->verified_k) return MIL_E_INVALID;
    const int eb = elt_bytes(c0.dtype);
    if (!aligned(accepted, 4)) return MIL_E_ALIGN;
    for (int l = 0; l < n; ++l)
        if (!aligned(x[l], 4) || !aligned(B[l], 4) || !aligned(dt[l], eb)) return MIL_E_ALIGN;
    const hipError_t e = launch_commit_layers(cs.data(), n, K, accepted, x, B, dt, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return MIL_E_HIP;
    for (int l = 0; l < n; ++l) {
        cs[l]->phase = kReady;
        cs[l]->verified_k = 0;
    }
    return MIL_OK;
}

int mil_ssm_commit_layers(mil_ssm_cache *const *caches, int32_t n, int32_t K, const int32_t *accepted,
                          const void *const *x, const void *const *B, const void *const *dt,
                          mil_stream_t stream) {
    const int st = mil_ssm_commit_layers_impl(caches, n, K, accepted, x, B, dt, stream);
    return debug_after("mil_ssm_commit_layers", st, true, stream, caches, n);
}

static int mil_ssm_verify_tree_impl(mil_ssm_cache *cache, int32_t K, const int32_t *parent, const void *x, const void *B,
                        const void *C, const void *dt, const float *A, const float *D, float *y,
                        mil_stream_t stream) {
    CacheImpl *c = impl(cache);
    if (!c) return MIL_E_INVALID;
    if (c->phase != kReady) return MIL_E_ORDER;
    if (K < 1 || K > c->k_max) return MIL_E_INVALID;
    if (!parent || !x || !B || !C || !dt || !A || !D || !y) return MIL_E_INVALID;
    const int eb = elt_bytes(c->dtype);
    if (!aligned(parent, 4) || !aligned(x, eb) || !aligned(B, eb) || !aligned(C, eb) || !aligned(dt, eb) ||
        !aligned(A, 4) || !aligned(D, 4) || !aligned(y, 4))
        return MIL_E_ALIGN;
    hipError_t e = launch_verify(*c, K, x, B, C, dt, A, D, y, reinterpret_cast<hipStream_t>(stream), parent);
    if (e != hipSuccess) return MIL_E_HIP;
    c->phase = kVerified;
    c->verified_k = K;
    return MIL_OK;
}

int mil_ssm_verify_tree(mil_ssm_cache *cache, int32_t K, const int32_t *parent, const void *x, const void *B,
                        const void *C, const void *dt, const float *A, const float *D, float *y,
                        mil_stream_t stream) {
    const int st = mil_ssm_verify_tree_impl(cache, K, parent, x, B, C, dt, A, D, y, stream);
    return debug_after("mil_ssm_verify_tree", st, true, stream, &cache, 1);
}

static int mil_ssm_commit_tree_impl(mil_ssm_cache *cache, int32_t K, const int32_t *parent, const int32_t *accepted_node,
                        const void *x, const void *B, const void *dt, const float *A, const float *D,
                        uint32_t flags, mil_stream_t stream) {
    CacheImpl *c = impl(cache);
    if (!c) return MIL_E_INVALID;
    if (c->phase != kVerified) return MIL_E_ORDER;
    if (flags & ~MIL_COMMIT_MATERIALIZE) return MIL_E_INVALID;
    if (K != c->verified_k) return MIL_E_INVALID;
    if (!parent || !accepted_node || !x || !B || !dt) return MIL_E_INVALID;
    const bool mat = (flags & MIL_COMMIT_MATERIALIZE) != 0;
    if (mat && (!A || !D)) return MIL_E_INVALID;
    const int eb = elt_bytes(c->dtype);
    if (!aligned(parent, 4) || !aligned(accepted_node, 4) || !aligned(x, 4) || !aligned(B, 4) || !aligned(dt, eb))
        return MIL_E_ALIGN;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = launch_commit_tree(*c, K, parent, accepted_node, x, B, dt, s);
    if (e == hipSuccess && mat) {
        e = launch_verify(*c, 0, nullptr, nullptr, nullptr, nullptr, A, D, nullptr, s);
        if (e == hipSuccess) e = launch_clear_pending(*c, s);
    }
    if (e != hipSuccess) return MIL_E_HIP;
    c->phase = kReady;
    c->verified_k = 0;
    return MIL_OK;
}

int mil_ssm_commit_tree(mil_ssm_cache *cache, int32_t K, const int32_t *parent, const int32_t *accepted_node,
                        const void *x, const void *B, const void *dt, const float *A, const float *D,
                        uint32_t flags, mil_stream_t stream) {
    const int st = mil_ssm_commit_tree_impl(cache, K, parent, accepted_node, x, B, dt, A, D, flags, stream);
    return debug_after("mil_ssm_commit_tree", st, true, stream, &cache, 1);
}

size_t mil_ssm_greedy_workspace_bytes(const mil_ssm_dims *d, int32_t K, int32_t vocab) {
    if (check_dims(d) != MIL_OK || K < 1 || K > MIL_KMAX_LIMIT || vocab < 1) return 0;
    return (size_t)greedy_workspace_bytes(d->batch, K);
}

}  // extern "C"

namespace {
// mil_ssm_commit_greedy with its workspace given; `noalloc`: the workspace is the
// library's scratch (checked for size against the batch and K, not against ws_bytes).
int commit_greedy(mil_ssm_cache *cache, int32_t K, const int32_t *draft_tokens, const void *logits, int32_t vocab,
                  int32_t logits_dtype, int32_t *accepted, int32_t *verifier_tokens, const void *x, const void *B,
                  const void *dt, const float *A, const float *D, void *ws, size_t ws_bytes, uint32_t flags,
                  mil_stream_t stream, bool noalloc) {
    CacheImpl *c = impl(cache);
    if (!c) return MIL_E_INVALID;
    if (c->phase != kVerified) return MIL_E_ORDER;
    if (flags & ~MIL_COMMIT_MATERIALIZE) return MIL_E_INVALID;
    if (K != c->verified_k) return MIL_E_INVALID;
    if (!draft_tokens || !logits || !accepted || !x || !B || !dt || vocab < 1) return MIL_E_INVALID;
    if (check_dtype(logits_dtype) != MIL_OK) return MIL_E_INVALID;
    const bool mat = (flags & MIL_COMMIT_MATERIALIZE) != 0;
    if (mat && (!A || !D)) return MIL_E_INVALID;
    const int64_t need = greedy_workspace_bytes(c->dims.batch, K);
    if (noalloc) {
        if ((int64_t)c->dims.batch * K > MIL_GREEDY_NOALLOC_MAX_ROWS) return MIL_E_WORKSPACE;
        if (greedy_noalloc_scratch(&ws) != hipSuccess) return MIL_E_HIP;
        ws_bytes = MIL_GREEDY_NOALLOC_SCRATCH_BYTES;
    }
    if (!ws || (int64_t)ws_bytes < need) return MIL_E_WORKSPACE;
    const int eb = elt_bytes(c->dtype);
    if (!aligned(draft_tokens, 4) || !aligned(accepted, 4) || (verifier_tokens && !aligned(verifier_tokens, 4)) ||
        !aligned(logits, elt_bytes(logits_dtype)) || !aligned(ws, kAlign) || !aligned(x, 4) || !aligned(B, 4) ||
        !aligned(dt, eb))
        return MIL_E_ALIGN;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = launch_commit_greedy(*c, K, draft_tokens, logits, vocab, logits_dtype, accepted, verifier_tokens,
                                        x, B, dt, ws, s);
    if (e == hipSuccess && mat) {
        e = launch_verify(*c, 0, nullptr, nullptr, nullptr, nullptr, A, D, nullptr, s);
        if (e == hipSuccess) e = launch_clear_pending(*c, s);
    }
    if (e != hipSuccess) return MIL_E_HIP;
    c->phase = kReady;
    c->verified_k = 0;
    return MIL_OK;
}
}  // namespace

extern "C" {

static int mil_ssm_commit_greedy_impl(mil_ssm_cache *cache, int32_t K, const int32_t *draft_tokens, const void *logits,
                          int32_t vocab, int32_t logits_dtype, int32_t *accepted, int32_t *verifier_tokens,
                          const void *x, const void *B, const void *dt, const float *A, const float *D, void *ws,
                          size_t ws_bytes, uint32_t flags, mil_stream_t stream) {
    return commit_greedy(cache, K, draft_tokens, logits, vocab, logits_dtype, accepted, verifier_tokens, x, B, dt, A,
                         D, ws, ws_bytes, flags, stream, false);
}

int mil_ssm_commit_greedy(mil_ssm_cache *cache, int32_t K, const int32_t *draft_tokens, const void *logits,
                          int32_t vocab, int32_t logits_dtype, int32_t *accepted, int32_t *verifier_tokens,
                          const void *x, const void *B, const void *dt, const float *A, const float *D, void *ws,
                          size_t ws_bytes, uint32_t flags, mil_stream_t stream) {
    const int st = mil_ssm_commit_greedy_impl(cache, K, draft_tokens, logits, vocab, logits_dtype, accepted, verifier_tokens, x, B, dt, A, D, ws, ws_bytes, flags, stream);
    return debug_after("mil_ssm_commit_greedy", st, true, stream, &cache, 1);
}

static int mil_ssm_commit_greedy_noalloc_impl(mil_ssm_cache *cache, int32_t K, const int32_t *draft_tokens, const void *logits,
                                  int32_t vocab, int32_t logits_dtype, int32_t *accepted, int32_t *verifier_tokens,
                                  const void *x, const void *B, const void *dt, const float *A, const float *D,
                                  uint32_t flags, mil_stream_t stream) {
    return commit_greedy(cache, K, draft_tokens, logits, vocab, logits_dtype, accepted, verifier_tokens, x, B, dt, A,
                         D, nullptr, 0, flags, stream, true);
}

int mil_ssm_commit_greedy_noalloc(mil_ssm_cache *cache, int32_t K, const int32_t *draft_tokens, const void *logits,
                                  int32_t vocab, int32_t logits_dtype, int32_t *accepted, int32_t *verifier_tokens,
                                  const void *x, const void *B, const void *dt, const float *A, const float *D,
                                  uint32_t flags, mil_stream_t stream) {
    const int st = mil_ssm_commit_greedy_noalloc_impl(cache, K, draft_tokens, logits, vocab, logits_dtype, accepted, verifier_tokens, x, B, dt, A, D, flags, stream);
    return debug_after("mil_ssm_commit_greedy_noalloc", st, true, stream, &cache, 1);
}

size_t mil_ssm_project_workspace_bytes(const mil_ssm_dims *d, int32_t T, int32_t d_model) {
    if (check_dims(d) != MIL_OK || !project_supported(*d, T, d_model)) return 0;
    return (size_t)project_workspace_bytes(*d, T, d_model);
}

static int mil_ssm_project_impl(const mil_ssm_dims *d, int32_t T, int32_t d_model, const void *u, const void *w_x,
                    const void *w_B, const void *w_C, const void *w_dt, const float *dt_bias, int32_t out_dtype,
                    void *x, void *B, void *C, void *dt, void *ws, size_t ws_bytes, mil_stream_t stream) {
    int st = check_dims(d);
    if (st != MIL_OK) return st;
    if (check_dtype(out_dtype) != MIL_OK) return MIL_E_INVALID;
    if (T < 1 || d_model < 1) return MIL_E_INVALID;
    if (!u || !w_x || !w_B || !w_C || !w_dt || !x || !B || !C || !dt) return MIL_E_INVALID;
    if (!project_supported(*d, T, d_model)) return MIL_E_UNSUPPORTED;
    const int64_t need = project_workspace_bytes(*d, T, d_model);
    if (need > 0 && (!ws || (int64_t)ws_bytes < need)) return MIL_E_WORKSPACE;
    const int eb = elt_bytes(out_dtype);
    if (!aligned(u, 16) || !aligned(w_x, 16) || !aligned(w_B, 16) || !aligned(w_C, 16) || !aligned(w_dt, 16) ||
        (dt_bias && !aligned(dt_bias, 4)) || !aligned(x, eb) || !aligned(B, eb) || !aligned(C, eb) ||
        !aligned(dt, eb) || (need > 0 && !aligned(ws, kAlign)))
        return MIL_E_ALIGN;
    const void *w[4] = {w_x, w_B, w_C, w_dt};
    void *out[4] = {x, B, C, dt};
    return hip_status(launch_project(*d, T, d_model, u, w, dt_bias, out_dtype == MIL_BF16, out, ws,
                                     reinterpret_cast<hipStream_t>(stream)));
}

int mil_ssm_project(const mil_ssm_dims *d, int32_t T, int32_t d_model, const void *u, const void *w_x,
                    const void *w_B, const void *w_C, const void *w_dt, const float *dt_bias, int32_t out_dtype,
                    void *x, void *B, void *C, void *dt, void *ws, size_t ws_bytes, mil_stream_t stream) {
    const int st = mil_ssm_project_impl(d, T, d_model, u, w_x, w_B, w_C, w_dt, dt_bias, out_dtype, x, B, C, dt, ws, ws_bytes, stream);
    return debug_after("mil_ssm_project", st, true, stream, nullptr, 0);
}

int mil_ssm_cache_status(const mil_ssm_cache *cache, int32_t *bad_slot, int32_t clear, mil_stream_t stream) {
    const CacheImpl *c = impl(cache);
    if (!c || !bad_slot) return MIL_E_INVALID;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int Bt = c->dims.batch;
    int32_t *host = static_cast<int32_t *>(malloc(sizeof(int32_t) * Bt));
    if (!host) return MIL_E_INVALID;
    hipError_t e = hipMemcpyAsync(host, cache_err(*c), sizeof(int32_t) * Bt, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        free(host);
        return MIL_E_HIP;
    }
    *bad_slot = -1;
    for (int b = 0; b < Bt; ++b)
        if (host[b] != 0) {
            *bad_slot = b;
            break;
        }
    free(host);
    if (clear) {
        e = launch_fill_zero(cache_err(*c), Bt, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return MIL_E_HIP;
    }
    return *bad_slot < 0 ? MIL_OK : MIL_E_INVALID;
}

int mil_ssm_prefill_kernels(const mil_ssm_cache *cache, int32_t nseq, int32_t L, int32_t chunk) {
    const CacheImpl *c = impl(cache);
    if (!c || nseq < 1 || nseq > c->dims.batch || L < 1 || (chunk != 64 && chunk != 128 && chunk != 256)) return 0;
    const mil_ssm_dims &d = c->dims;
    if (c->dtype == MIL_BF16 && prefill_single_launch(nseq, L, chunk, d.nheads, d.headdim, d.dstate))
        return 1 << MIL_TRACE_PREFILL_SCAN;
    return (1 << MIL_TRACE_PREFILL_STATE) | (1 << MIL_TRACE_PREFILL_PASS) | (1 << MIL_TRACE_PREFILL_OUT);
}

int mil_ssm_cache_phase(const mil_ssm_cache *cache) {
    const CacheImpl *c = impl(cache);
    return c ? c->phase : kUninit;
}

static int mil_ssm_cache_trace_impl(mil_ssm_cache *cache, int32_t kernel, void *ev_start, void *ev_stop) {
    CacheImpl *c = impl(cache);
    if (!c || kernel < MIL_TRACE_OFF || kernel > MIL_TRACE_PREFILL_SCAN) return MIL_E_INVALID;
    if (kernel == MIL_TRACE_OFF || !ev_start || !ev_stop) {
        c->trace_kernel = MIL_TRACE_OFF;
        c->trace_start = c->trace_stop = nullptr;
        return MIL_OK;
    }
    c->trace_kernel = kernel;
    c->trace_start = static_cast<hipEvent_t>(ev_start);
    c->trace_stop = static_cast<hipEvent_t>(ev_stop);
    return MIL_OK;
}

int mil_ssm_cache_trace(mil_ssm_cache *cache, int32_t kernel, void *ev_start, void *ev_stop) {
    const int st = mil_ssm_cache_trace_impl(cache, kernel, ev_start, ev_stop);
    return debug_after("mil_ssm_cache_trace", st, false, nullptr, nullptr, 0);
}

}  // extern "C"

namespace {
int debug_after(const char *fn, int st, bool enqueued, mil_stream_t stream, mil_ssm_cache *const *caches, int n) {
    if (!debug_on()) return st;
    if (st != MIL_OK) {
        fprintf(stderr, "mil_ssm debug: %s returned %d (%s)\n", fn, st, mil_status_string(st));
        return st;
    }
    if (!enqueued) return st;
    // a stream being captured into a graph cannot be synchronized (that would end the
    // capture): the work runs only when the graph is launched, so there is nothing to check
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(reinterpret_cast<hipStream_t>(stream), &cap) == hipSuccess &&
        cap != hipStreamCaptureStatusNone)
        return st;
    hipError_t e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) {
        fprintf(stderr, "mil_ssm debug: %s: the enqueued work failed: %s\n", fn, hipGetErrorString(e));
        return MIL_E_HIP;
    }
    for (int l = 0; l < n; ++l) {
        const CacheImpl *c = impl(caches[l]);
        if (!c) continue;
        std::vector<int32_t> err((size_t)c->dims.batch);
        e = hipMemcpy(err.data(), cache_err(*c), sizeof(int32_t) * err.size(), hipMemcpyDeviceToHost);
        if (e != hipSuccess) {
            fprintf(stderr, "mil_ssm debug: %s: reading the error words failed: %s\n", fn, hipGetErrorString(e));
            return MIL_E_HIP;
        }
        for (size_t b = 0; b < err.size(); ++b)
            if (err[b] != 0)
                fprintf(stderr, "mil_ssm debug: %s: cache %d slot %zu error word 0x%x (accept %d, tree %d, scan %d)\n",
                        fn, l, b, (unsigned)err[b], (err[b] & MIL_DEVERR_ACCEPT) != 0, (err[b] & MIL_DEVERR_TREE) != 0,
                        (err[b] & MIL_DEVERR_SCAN) != 0);
    }
    return st;
}
}  // namespace
