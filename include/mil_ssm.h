/*
 * mil_ssm.h -- C ABI of the MI355X (gfx950) library for the selective SSM layer
 * of "The Mamba in the Llama: Distilling and Accelerating Hybrid Models", in its
 * two inference modes: a chunked full-sequence prefill, and the speculative
 * verify / commit step that advances a cached state through K draft tokens and
 * rolls back to the accepted prefix by recomputing from the cached state.
 *
 * The layer (one sequence b, head h, group g = h / (H/G); abstract of the paper:
 * attention is distilled into a linear RNN reusing the attention projections, so
 * x comes from V, B from K and C from Q; skycaiji.com summary, method paragraph:
 * a continuous-time SSM with an expanded state, discretised per token):
 *     h_t = exp(dt_t * A_h) * h_{t-1} + (dt_t * B_t) x_t^T      (N x P, fp32)
 *     y_t = C_t^T h_t + D_h * x_t                               (P, fp32)
 *
 * The decoding protocol (QbitAI article "Llama 3+Mamba 强强联手", speculative-
 * decoding walkthrough): a draft model proposes K tokens; the Mamba layer takes
 * them one after another; the state moves forward only through the accepted
 * ones; no intermediate state is stored; on a rejection the state goes back to
 * the last accepted token and drafting restarts from there.
 *
 * Conventions for every function below:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates no device memory.  Its only global state is the static scratch of
 *     mil_ssm_commit_greedy_noalloc (one array per GPU) and per-device values it
 *     looks up once (that array's address, the compute-unit count).
 *   - Token tensors are row-major with the last dimension contiguous:
 *       x  [seq][T][H][P],  B, C [seq][T][G][N],  dt [seq][T][H]   (dtype of the cache)
 *       A, D [H] fp32,  y [seq][T][H][P] fp32.
 *     dt is the step size after any softplus (dt > 0); A is the continuous decay
 *     rate (A <= 0 for a stable layer; any finite value is accepted).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the functions return without synchronising, except mil_ssm_cache_status.
 *   - Argument errors are reported synchronously as a status code before any
 *     work is enqueued; nothing is modified then.  A failing HIP launch returns
 *     MIL_E_HIP.  No function throws or aborts.
 *   - Calls on one cache must be issued from one host thread in order; calls on
 *     different caches are independent and reentrant.
 *   - Debugging: with MIL_SSM_DEBUG set in the environment (any value but "0"),
 *     every call that fails prints its name and status on stderr, and every call
 *     that enqueues work (on a stream not being captured into a graph) then
 *     synchronizes its stream, returns MIL_E_HIP if that
 *     work failed, and prints each slot whose device error word is set in the
 *     caches it used (its own status is unchanged).  For debugging only: the
 *     synchronization serializes the host with the GPU.
 */
#ifndef MIL_SSM_H
#define MIL_SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t *mil_stream_t;

enum mil_status {
    MIL_OK = 0,
    MIL_E_INVALID = 1,     /* null pointer, bad size, bad dtype, value out of range */
    MIL_E_ALIGN = 2,       /* a device buffer is not aligned as required (256 B for the cache) */
    MIL_E_ORDER = 3,       /* call out of protocol order (see mil_ssm_verify / mil_ssm_commit) */
    MIL_E_UNSUPPORTED = 4, /* a shape this build has no kernel for (see mil_ssm_supported) */
    MIL_E_HIP = 5,         /* the HIP runtime reported an error */
    MIL_E_WORKSPACE = 6    /* workspace missing or too small */
};

enum mil_dtype {
    MIL_F32 = 0,  /* x, B, C, dt stored as IEEE fp32 */
    MIL_BF16 = 1  /* x, B, C, dt stored as bfloat16 */
};

/* Layer shape.  H % G == 0; heads h and h' share B and C when h/(H/G) == h'/(H/G). */
typedef struct {
    int32_t batch;   /* number of sequence slots in a cache */
    int32_t nheads;  /* H */
    int32_t headdim; /* P: columns of the state, width of x and y per head */
    int32_t dstate;  /* N: rows of the state, width of B and C per group */
    int32_t ngroups; /* G */
} mil_ssm_dims;

/*
 * Byte layout of a cache buffer (all offsets from its start, each a multiple of 256).
 *   state   fp32 [batch][H][N][P]: head block (slot, h) starts at
 *           state_off + (slot*H + h) * state_head_stride; p is contiguous.
 *   pend_x  [batch][k_max][H][P], pend_B [batch][k_max][G][N], pend_dt [batch][k_max][H]
 *           (cache dtype): accepted draft tokens not yet folded into `state`.
 *   pos     int32 [batch]: tokens the sequence has absorbed (prefill + accepted drafts).
 *   pending int32 [batch]: how many rows of pend_* are accepted but not yet folded in.
 *   err     int32 [batch]: 0, or the OR of MIL_DEVERR_ACCEPT (an out-of-range accepted
 *           length or node), MIL_DEVERR_TREE (a tree link outside -1..k-1) and
 *           MIL_DEVERR_SCAN (a prefill's chunk-to-chunk handoff timed out; the slot's
 *           prefill results are then wrong).
 *   scan    int32 [batch][H][8][68]: single-launch prefill handoff words, one row per
 *           (slot, head, column slab): 64 chunk flags, then the row's epoch (that of the
 *           row's last launch), then padding.  mil_ssm_cache_init zeroes them; a launch
 *           takes epoch e = the row's epoch + 1, writes its flags as (e << 2) | kind and
 *           then stores e as the row's epoch, so the value that marks a launch lives in the
 *           buffer itself: graph replays and byte copies of a cache (mil_ssm_cache_attach)
 *           stay correct.  A buffer whose rows hold a flag of a later epoch than their own
 *           is not a cache this library wrote.  The word after the epoch in each slot's
 *           first row (head 0, slab 0) counts the workgroups of a greedy commit that have
 *           finished for that slot; it is 0 between calls (the last one resets it).
 *   append  int32 [batch]: the pend_* row at which the next commit puts its first accepted
 *           row: 0 when the verify before it wrote the folded state back, else that
 *           verify's pending count (written by verify, read by commit).
 * The logical state of slot b is `state` advanced through its `pending` rows.  A verify
 * folds all of them (in registers) for its outputs, but writes the folded state back only
 * when the next commit could overflow the pending area (pending + K > k_max; always with
 * K = 0); otherwise the accepted rows stay pending and the next commit appends to them.
 * With k_max = K every verify that has pending rows writes the state back; a larger k_max
 * trades a few more rows folded per verify for fewer state writes.
 */
typedef struct {
    int64_t bytes;
    int64_t state_off, state_head_stride;
    int64_t pend_x_off, pend_B_off, pend_dt_off;
    int64_t pos_off, pending_off, err_off;
    int64_t scan_off;
    int64_t append_off;
} mil_ssm_layout;

#define MIL_DEVERR_ACCEPT 1
#define MIL_DEVERR_TREE 2      /* a tree link outside -1..k-1 (verify_tree / commit_tree) */
#define MIL_DEVERR_SCAN 4      /* a prefill chunk waited too long for the state of the chunk before it */

/* Host-side cache descriptor.  The caller provides the storage; mil_ssm_cache_init
 * fills it.  It holds the device buffer address, the shape and the protocol phase. */
typedef struct {
    uint64_t opaque[24];
} mil_ssm_cache;

#define MIL_KMAX_LIMIT 16          /* largest K (drafts per round) and k_max supported */
#define MIL_PREFILL_CONTINUE 1u    /* prefill: start from the slot's logical state instead of zeros */
#define MIL_COMMIT_MATERIALIZE 1u  /* commit: fold the accepted tokens into `state` now */

/* Text for a status code (static storage). */
const char *mil_status_string(int status);

/* MIL_OK if this build has kernels for the shape and dtype, else MIL_E_UNSUPPORTED
 * (or MIL_E_INVALID for a malformed shape).  Supported: P and N in {16,32,64,128,256},
 * H % G == 0, batch >= 1, dtype MIL_F32 or MIL_BF16. */
int mil_ssm_supported(const mil_ssm_dims *dims, int32_t dtype);

/* Fill *out with the layout of a cache for `dims`, k_max (1..MIL_KMAX_LIMIT) and dtype. */
int mil_ssm_cache_layout(const mil_ssm_dims *dims, int32_t k_max, int32_t dtype, mil_ssm_layout *out);

/* Bytes a cache needs (0 if the arguments are invalid). */
size_t mil_ssm_cache_bytes(const mil_ssm_dims *dims, int32_t k_max, int32_t dtype);

/* Carve a caller-owned device buffer (256-B aligned, >= mil_ssm_cache_bytes) into a
 * cache and enqueue zeroing of the state, pos, pending and err arrays.  The descriptor
 * starts in the READY phase.  The buffer must outlive every call that uses the cache. */
int mil_ssm_cache_init(mil_ssm_cache *cache, const mil_ssm_dims *dims, int32_t k_max, int32_t dtype,
                       void *dev_buf, size_t bytes, mil_stream_t stream);

/* Describe a buffer that already holds a cache of this shape (for instance a byte copy
 * of one set up by mil_ssm_cache_init, used to snapshot and restore sequences).  Same
 * checks as mil_ssm_cache_init; nothing is enqueued and the contents are not touched.
 * The descriptor starts in the READY phase. */
int mil_ssm_cache_attach(mil_ssm_cache *cache, const mil_ssm_dims *dims, int32_t k_max, int32_t dtype,
                         void *dev_buf, size_t bytes);

/* Workspace bytes mil_ssm_prefill needs for nseq sequences of L tokens with chunk length `chunk`. */
size_t mil_ssm_prefill_workspace_bytes(const mil_ssm_dims *dims, int32_t nseq, int32_t L, int32_t chunk);

/*
 * Full-sequence scan of L tokens for slots [slot0, slot0+nseq).
 * Computes y for every token (skipped when y is NULL) and sets each slot's logical
 * state to h_L.  It starts from zeros, or with MIL_PREFILL_CONTINUE from the slot's
 * logical state (pending rows are folded in first).  pos becomes L (or pos + L);
 * pending becomes 0.  The sequence is cut into chunks of `chunk` tokens (the last may
 * be shorter): within a chunk the layer is evaluated in its matrix (quadratic) form on
 * the matrix cores, and a short sequential pass carries the state across chunks.
 * chunk must be 64, 128 or 256.  ws: device workspace of at least
 * mil_ssm_prefill_workspace_bytes(); it is scratch and may be reused after the call's
 * work completes in stream order.
 * Order: the cache must be READY (not between verify and commit) -> MIL_E_ORDER.
 */
int mil_ssm_prefill(mil_ssm_cache *cache, int32_t slot0, int32_t nseq, int32_t L, int32_t chunk,
                    const void *x, const void *B, const void *C, const void *dt,
                    const float *A, const float *D, float *y,
                    void *ws, size_t ws_bytes, uint32_t flags, mil_stream_t stream);

/*
 * Speculative verify of K draft tokens (1 <= K <= k_max) for every slot of the cache.
 * x, B, C, dt hold the drafts, [batch][K][...]; y [batch][K][H][P] receives, for each
 * draft k, the output the layer gives when drafts 0..k follow the slot's logical state.
 * The logical state is NOT changed (a draft is folded in only by a later commit).
 * Each (slot, head) state block is read from HBM once; the pending accepted rows are
 * folded in on the way (in registers), and the folded state is written back once, only if
 * pending + K > k_max (the next commit could overflow the pending area); otherwise the
 * rows stay pending and the next commit appends to them (see the cache layout above).
 * Order: READY -> VERIFIED.  A second verify without a commit returns MIL_E_ORDER.
 */
int mil_ssm_verify(mil_ssm_cache *cache, int32_t K,
                   const void *x, const void *B, const void *C, const void *dt,
                   const float *A, const float *D, float *y, mil_stream_t stream);

/*
 * Accept the first accepted[b] drafts of slot b (device int32 [batch], each 0..K) from
 * the round verified just before.  x, B, dt are the same draft buffers given to that
 * verify (C is not needed).  The logical state of slot b becomes the state after its
 * accepted drafts; pos[b] += accepted[b].  The accepted rows are copied into the cache,
 * so the draft buffers may be reused once this call is enqueued.  By default the rows are
 * folded into `state` by a later verify (when it writes the state back) or prefill;
 * MIL_COMMIT_MATERIALIZE folds every pending row in now (same arithmetic, bit-identical
 * state).  An accepted[b] outside 0..K sets
 * err[b] = MIL_DEVERR_ACCEPT and leaves slot b's logical state and pos unchanged.
 * A and D are needed only with MIL_COMMIT_MATERIALIZE (may be NULL otherwise).
 * Order: VERIFIED -> READY (MIL_E_ORDER otherwise); K must equal the verified K.
 */
int mil_ssm_commit(mil_ssm_cache *cache, int32_t K, const int32_t *accepted,
                   const void *x, const void *B, const void *dt,
                   const float *A, const float *D, uint32_t flags, mil_stream_t stream);

/*
 * The commit of one decoding round for several layers at once.  In a round every layer
 * verifies the same K drafts and the verifier decides from the last layer's output how
 * many are accepted, so each layer's cache takes the same accepted lengths (QbitAI
 * article, speculative-decoding walkthrough: the Mamba layers keep the accepted tokens
 * and go back to the last accepted one).  Equivalent to mil_ssm_commit(caches[l], K,
 * accepted, x[l], B[l], dt[l], NULL, NULL, 0, stream) for l = 0 .. n-1 (deferred fold, the
 * same copies and bookkeeping, bit for bit), issued as one launch per
 * MIL_COMMIT_LAYERS_MAX layers.
 * caches: host array of n descriptors (1 <= n); x, B, dt: host arrays of n device pointers,
 * layer l's draft buffers as given to its verify; accepted: device int32 [batch], 0..K.
 * Every cache must have the same batch, heads, head dim, state size, groups, dtype and
 * k_max, be VERIFIED with this K, and appear once.  Nothing is launched and no cache
 * changes phase when any check fails: MIL_E_INVALID (null pointers, n < 1, a repeated
 * cache, shapes, dtypes or K that differ), MIL_E_ORDER (a cache not VERIFIED), MIL_E_ALIGN.
 * An accepted[b] outside 0..K sets err[b] = MIL_DEVERR_ACCEPT in every cache and leaves
 * slot b's logical state and pos unchanged, as mil_ssm_commit does.
 */
#define MIL_COMMIT_LAYERS_MAX 32
int mil_ssm_commit_layers(mil_ssm_cache *const *caches, int32_t n, int32_t K, const int32_t *accepted,
                          const void *const *x, const void *const *B, const void *const *dt,
                          mil_stream_t stream);

/*
 * Greedy acceptance on the device, fused into the commit.
 * QbitAI article "Llama 3+Mamba 强强联手", speculative-decoding walkthrough: the verifier
 * checks the K drafted tokens in order, the accepted ones are kept and the sequence is
 * cut at the first rejected one.  The pages do not say what makes a draft "correct"; the
 * reading taken here is greedy verification: draft k of slot b is correct when it equals
 * the verifier's most likely token at that position, the argmax over the vocabulary of
 * logits[b][k][:]: among equal values the lowest token id wins, -0 and +0 are one value,
 * and every NaN (either sign, any payload) ranks above every number, the lowest id first
 * among NaNs.  accepted[b] = the number of leading correct drafts (0..K).
 *
 * draft_tokens  device int32 [batch][K], token ids the drafts stand for;
 * logits        device [batch][K][vocab], MIL_F32 or MIL_BF16 (logits_dtype, independent
 *               of the cache dtype), the verifier's scores at the K draft positions;
 * accepted      device int32 [batch], written with accepted[b];
 * verifier_tokens  device int32 [batch][K] written with the argmax per position, or NULL;
 * ws            caller-owned device workspace of at least mil_ssm_greedy_workspace_bytes
 *               bytes, 256-byte aligned (partial maxima; no state is kept in it).
 * Everything else (x, B, dt, A, D, flags, order, K) is as for mil_ssm_commit, with
 * accepted[b] computed here instead of given; the cache ends up as after mil_ssm_commit
 * with those accepted lengths (the same logical state, pos and pending; the pending rows
 * past the new count may hold the rejected drafts, which nothing reads).  One launch does
 * the argmax, the decision and the copies.
 */
size_t mil_ssm_greedy_workspace_bytes(const mil_ssm_dims *dims, int32_t K, int32_t vocab);
int mil_ssm_commit_greedy(mil_ssm_cache *cache, int32_t K, const int32_t *draft_tokens,
                          const void *logits, int32_t vocab, int32_t logits_dtype,
                          int32_t *accepted, int32_t *verifier_tokens,
                          const void *x, const void *B, const void *dt,
                          const float *A, const float *D, void *ws, size_t ws_bytes,
                          uint32_t flags, mil_stream_t stream);

/*
 * mil_ssm_commit_greedy for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  Same arguments,
 * results and errors, without ws / ws_bytes: the partial maxima go to a scratch array the
 * library owns, MIL_GREEDY_NOALLOC_SCRATCH_BYTES in every GPU's memory, held until the
 * process ends.  Nothing is allocated by this call (its first call on a device looks up
 * that device's array).  batch * K above MIL_GREEDY_NOALLOC_MAX_ROWS returns
 * MIL_E_WORKSPACE and enqueues nothing.  Every call on one GPU shares that GPU's array
 * and leaves its contents behind (nothing in it needs clearing: each call writes every
 * entry it reads), so calls that may overlap on one GPU (other streams, other threads)
 * race and must not be made.
 */
#define MIL_GREEDY_NOALLOC_MAX_ROWS 512
#define MIL_GREEDY_NOALLOC_SCRATCH_BYTES (256 * 1024)
int mil_ssm_commit_greedy_noalloc(mil_ssm_cache *cache, int32_t K, const int32_t *draft_tokens,
                                  const void *logits, int32_t vocab, int32_t logits_dtype,
                                  int32_t *accepted, int32_t *verifier_tokens,
                                  const void *x, const void *B, const void *dt,
                                  const float *A, const float *D, uint32_t flags, mil_stream_t stream);

/* ---- Tree drafts ----
 *
 * Speculative decoding with tree-organised candidates (named among the variants in the
 * skycaiji.com summary, related-work paragraph): the K drafts of a sequence form a tree,
 * draft k following draft parent[b][k] instead of draft k-1, parent -1 meaning the
 * committed state itself; parents are numbered before their children (parent[b][k] in
 * -1..k-1).  Every branch starts from the same cached state, which is read once.
 *
 * mil_ssm_verify_tree: as mil_ssm_verify, with y[b][k] the output at draft k after the
 *   recurrence has run over k's root path (the drafts from the state to k, root first).
 *   A chain (parent[b][k] = k-1) gives exactly mil_ssm_verify's results, and draft k's
 *   output is bit-identical to a chain verify of its path's tokens.  A link outside
 *   -1..k-1 is taken as -1 and reported as MIL_DEVERR_TREE in err[b].
 * mil_ssm_commit_tree: as mil_ssm_commit, with the accepted branch given as one node,
 *   accepted_node[b] in -1..K-1 (device int32; -1 accepts nothing): the tokens on its
 *   root path, root first, are accepted (j = the path's length).  An out-of-range node
 *   (MIL_DEVERR_ACCEPT) or a bad link on the path (MIL_DEVERR_TREE) sets err[b] and
 *   leaves slot b's logical state and pos unchanged.
 * parent   device int32 [batch][K], 4-byte aligned; the same array for both calls of a round.
 * Everything else (buffers, order, K, flags) is as for mil_ssm_verify and mil_ssm_commit.
 */
int mil_ssm_verify_tree(mil_ssm_cache *cache, int32_t K, const int32_t *parent,
                        const void *x, const void *B, const void *C, const void *dt,
                        const float *A, const float *D, float *y, mil_stream_t stream);
int mil_ssm_commit_tree(mil_ssm_cache *cache, int32_t K, const int32_t *parent,
                        const int32_t *accepted_node, const void *x, const void *B, const void *dt,
                        const float *A, const float *D, uint32_t flags, mil_stream_t stream);

/* ---- Input projections (the step before the layer) ----
 *
 * "The Mamba in the Llama" builds the layer out of an attention layer's own linear
 * projection weights (arXiv abstract; skycaiji.com summary, method paragraph: the
 * modified Mamba is initialised from the attention module).  Reading used here: the
 * value projection gives x, the key projection B, the query projection C, and one more
 * projection per head gives the step size through softplus, so that dt > 0:
 *   x[t][h*P+p]  = sum_k u[t][k] w_x[h*P+p][k]
 *   B[t][g*N+n]  = sum_k u[t][k] w_B[g*N+n][k]      C likewise with w_C
 *   dt[t][h]     = softplus(sum_k u[t][k] w_dt[h][k] + dt_bias[h])
 * for T input rows u of width d_model.  The outputs are laid out exactly as
 * mil_ssm_verify / mil_ssm_prefill take them (x [T][H][P], B and C [T][G][N], dt [T][H],
 * with T = batch*K or nseq*L rows), so they feed those calls directly.
 *
 * dims          H, P, N, G as for the cache (dims->batch is not used).
 * T, d_model    rows and row width; d_model a multiple of 64, T >= 1.
 * u             bf16 [T][d_model]; w_x bf16 [H*P][d_model]; w_B, w_C bf16 [G*N][d_model];
 *               w_dt bf16 [H][d_model]: device pointers, 16-byte aligned, row-major (a
 *               weight row is one output feature).  Each weight block must be under 2 GiB.
 * dt_bias       fp32 [H] or NULL (no bias).
 * out_dtype     MIL_BF16 or MIL_F32 for x, B, C, dt (products are summed in fp32; bf16
 *               outputs are rounded to nearest even once, at the end).
 * ws            caller-owned device workspace, 256-byte aligned, of at least
 *               mil_ssm_project_workspace_bytes() bytes; may be NULL when that is 0.  It holds
 *               fp32 partial sums when the d_model inputs are split over several
 *               workgroups (few rows); they are added in a fixed order, so results are
 *               reproducible.
 * Returns MIL_E_INVALID (null pointer, bad size or dtype), MIL_E_UNSUPPORTED (d_model not
 * a multiple of 64, a weight block over 2 GiB), MIL_E_WORKSPACE, MIL_E_ALIGN or MIL_E_HIP;
 * nothing is enqueued on an error.  No cache is involved: it may run on any stream.
 */
size_t mil_ssm_project_workspace_bytes(const mil_ssm_dims *dims, int32_t T, int32_t d_model);
int mil_ssm_project(const mil_ssm_dims *dims, int32_t T, int32_t d_model, const void *u,
                    const void *w_x, const void *w_B, const void *w_C, const void *w_dt,
                    const float *dt_bias, int32_t out_dtype, void *x, void *B, void *C, void *dt,
                    void *ws, size_t ws_bytes, mil_stream_t stream);

/* Synchronise `stream`, then report device-side errors: *bad_slot = first slot with
 * err != 0, or -1.  Returns MIL_OK, or MIL_E_INVALID when a slot has an error.
 * With clear != 0 the err words are zeroed afterwards. */
int mil_ssm_cache_status(const mil_ssm_cache *cache, int32_t *bad_slot, int32_t clear, mil_stream_t stream);

/* Protocol phase of a cache descriptor: 0 = uninitialised, 1 = READY, 2 = VERIFIED. */
int mil_ssm_cache_phase(const mil_ssm_cache *cache);

/* Kernels that can be traced with mil_ssm_cache_trace. */
enum mil_trace_kernel {
    MIL_TRACE_OFF = 0,
    MIL_TRACE_VERIFY = 1,        /* verify: fold pending rows + K draft outputs */
    MIL_TRACE_FOLD = 2,          /* fold-only pass (commit with MIL_COMMIT_MATERIALIZE, prefill continue) */
    MIL_TRACE_COMMIT = 3,        /* accepted-length bookkeeping (a greedy commit is MIL_TRACE_ACCEPT) */
    MIL_TRACE_PREFILL_STATE = 4, /* prefill phase 1: per-chunk states */
    MIL_TRACE_PREFILL_PASS = 5,  /* prefill phase 2: sequential pass across chunks */
    MIL_TRACE_PREFILL_OUT = 6,   /* prefill phase 3: per-chunk outputs */
    MIL_TRACE_ACCEPT = 7,        /* greedy commit: argmax per draft position, accepted lengths and copies in one launch */
    MIL_TRACE_PREFILL_SCAN = 8   /* prefill in one launch (chunk states, handoff and outputs) */
};

/* Which traceable kernels a mil_ssm_prefill of these sizes launches on this cache (with y
 * requested and 16-byte aligned x, B, C): a bit mask with bit k set for mil_trace_kernel
 * k.  Bf16 caches whose chunk is 256 and whose shapes the one-launch kernel covers get
 * (1 << MIL_TRACE_PREFILL_SCAN); other shapes get the three phases (STATE, PASS, OUT).
 * Returns 0 for a bad descriptor or sizes.  Host-side only. */
int mil_ssm_prefill_kernels(const mil_ssm_cache *cache, int32_t nseq, int32_t L, int32_t chunk);

/* Profiling hook: until changed, every launch of `kernel` made through this descriptor
 * is bracketed by hipEventRecord(ev_start) and hipEventRecord(ev_stop) on the call's
 * stream (both are hipEvent_t handles created by the caller).  MIL_TRACE_OFF (or NULL
 * events) turns it off.  Host-side only: nothing is enqueued by this call. */
int mil_ssm_cache_trace(mil_ssm_cache *cache, int32_t kernel, void *ev_start, void *ev_stop);

#ifdef __cplusplus
}
#endif

#endif /* MIL_SSM_H */
