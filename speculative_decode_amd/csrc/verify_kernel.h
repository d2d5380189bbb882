// Verify / fold kernel template (included by the per-dtype translation units).
// The speculative verify / fold kernel for the SSM layer of "The Mamba in the Llama".
//
// QbitAI article "Llama 3+Mamba 强强联手", speculative-decoding walkthrough: the Mamba
// layers take the K draft tokens in order, move the state only through accepted ones,
// keep no intermediate state, and on a rejection go back to the last accepted token.
// Here the cache keeps the state at the last fold point plus the accepted token rows
// since then ("pending"); one launch, per (slot, head, column tile):
//   1. reads each state row from HBM once,
//   2. folds the m pending rows in, token by token, with the one state step below,
//   3. writes the row back once (only when m > 0),
//   4. accumulates C_k . h over the row for every draft k,
// and then forms each draft's output from the folded state h0 in closed form
// (skycaiji.com summary, method paragraph: the discretised linear RNN), which is the
// recurrence unrolled over the K drafts:
//   y_k = alpha_k (C_k^T h0) + sum_{s<=k} beta_{k,s} dt_s (C_k . B_s) x_s + D x_k,
//   alpha_k = prod_{i<=k} abar_i,  beta_{k,s} = prod_{s<i<=k} abar_i,  abar_i = exp(dt_i A).
// No draft token ever touches the stored state; a later commit decides which ones count.
//
// Tree drafts (the pages name tree-organised candidates among speculative-decoding
// variants; skycaiji.com summary, related-work paragraph): with a parent array, draft k
// follows draft parent[k] (-1: the folded state h0) instead of draft k-1, and the same
// closed form runs over k's root path P(k) instead of 0..k:
//   y_k = alpha_k (C_k^T h0) + sum_{s in P(k)} beta_{k,s} dt_s (C_k . B_s) x_s + D x_k,
//   alpha_k = prod_{i in P(k)} abar_i,  beta_{k,s} = prod_{i in P(k), i > s} abar_i.
// Every branch starts from the one state read; products run in ascending node order, so a
// chain (parent[k] = k-1) is exactly the flat case and a node's output equals, bit for
// bit, a flat verify of its path's tokens.
//
// Work decomposition (gfx950, wave64): one workgroup per (slot, head, column tile of
// P/CS columns), S waves.  A lane owns 4 adjacent columns (16-byte loads) of ROWS
// consecutive state rows; P/(4 CS) lanes cover a row tile, so a wave reads 64 * 16
// bytes per load instruction.  Whole rows per workgroup (CS = 1) where the registers
// allow, so that each workgroup streams one contiguous block; splitting the columns keeps
// ROWS (and the registers a lane needs) small enough for several workgroups to share a CU
// where whole rows would not; the readout needs no exchange between tiles, since every
// output column sums over all N rows of its own column only.  State
// traffic is one read and at most one write per element; per-row work is in registers,
// partial C_k . h sums are combined across the row groups of a wave with shuffles and
// across waves through LDS, always in the same order.
#pragma once

#include "ssm_internal.h"

namespace mil {


// Stored element -> fp32 (bf16 widens exactly by a 16-bit shift).
__device__ __forceinline__ float ld(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t *p, size_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes at `base` (gfx9-family descriptor word 3); loads and
// stores through it take one per-lane offset plus a scalar offset, and accesses past
// `bytes` are dropped by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}
// The state is streamed: read once and written once per round, so its accesses carry
// the non-temporal cache policy (bit 1 of the cache-policy operand on gfx94x/gfx950);
// the write-back also sets sc1 (bit 4), which measured faster for the stores (batched
// round 20.8 -> 20.3 us; the loads showed no difference with it).
constexpr int kStreamPolicy = 2;
constexpr int kStreamStorePolicy = 2 | 16;
__device__ __forceinline__ float4 buf_load4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    const f32x4v t = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreamPolicy);
    return make_float4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void buf_store4(float4 v, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
    const f32x4v t = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(t, r, voff, soff, kStreamStorePolicy);
}

// A workgroup barrier for LDS traffic only: this wave's LDS accesses are complete
// (lgkmcnt(0)) when it arrives, while its global loads and stores stay in flight.
// __syncthreads() would also wait for those (vmcnt(0)), which here would hold the per-draft
// scalars behind the state loads.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The single state step that folds one accepted token into a stored state element:
//   h <- abar * h + B[n] * (dt * x[p]).
// Every path that writes a state through accepted tokens (verify's fold, commit's
// immediate fold, prefill's continuation fold) calls this, so they agree bit for bit.
__device__ __forceinline__ float state_step(float abar, float h, float bn, float u) {
    return __builtin_fmaf(abar, h, bn * u);
}

struct VerifyParams {
    float *state;
    int64_t head_stride;  // floats between consecutive (slot, head) blocks
    const void *pend_x, *pend_B, *pend_dt;
    const int32_t *pending;
    int32_t *append;  // [batch] where the next commit appends: 0 after a write-back, else pending
    const void *x, *B, *C, *dt;
    const float *A, *D;
    float *y;
    int H, P, N, G, K, k_max;
    int cs;   // column tiles per head
    int vec;  // draft x, B, C 16-byte aligned: token rows staged in 16-byte chunks
    const int32_t *parent;  // [batch][K] tree links (-1..k-1), or null for a chain
    int32_t *err;           // [batch] device error words (a bad parent link is reported)
};

// Launch shape: CS column tiles per head, S waves per workgroup, ROWS rows per lane.
struct Shape {
    int S, ROWS, CS;
};

// Threads a workgroup may have for a given ROWS (more rows need more registers per lane).
constexpr int max_threads(int rows) { return rows >= 16 ? 512 : 1024; }

// LDS floats of one workgroup covering Pc columns.
inline size_t verify_lds_floats(int N, int Pc, int K, int kmax, int S) {
    return (size_t)kmax * N + 2 * K * N + (size_t)kmax * Pc + K * Pc + 2 * kmax + 5 * K + K * K + (size_t)S * K * Pc;
}
constexpr size_t kVerifyLdsMax = 160 * 1024;

// General shape search (after the preference for <= 8 waves in shape_for).  Whole rows
// per workgroup (CS = 1) whenever LDS allows: each workgroup
// then streams one contiguous N x P block, which HBM serves better than the strided
// halves or quarters of rows that column tiles read.  Within that, the fewest waves with
// at most kRowsTarget rows per lane and at least kWavesTarget waves in the grid, else the
// most waves (fewest rows per lane).  Column tiles only where a whole-row workgroup's LDS
// (which grows with K, kmax and S) does not fit.
constexpr int kRowsTarget = 8;
constexpr int64_t kWavesTarget = 2048;

// Launch shape for K drafts with up to kmax pending rows; S = 0 when none fits.  First
// workgroups of at most 8 waves (16-wave workgroups measured slower: their cross-wave
// reduction and barriers cost more than the extra waves bring), whole rows preferred:
// the first shape with at most kRowsTarget rows per lane and kWavesTarget waves, else
// with a quarter of that (few sequences: a single sequence's 32 heads); then the general
// search below.
inline Shape shape_for(int batch, int H, int P, int N, int K, int kmax) {
    Shape best{0, 0, 0};
    if (P < 16 || P > 256 || (P & (P - 1)) || N < 16 || N > 256 || (N & (N - 1))) return best;
    // Whole rows in 8-wave workgroups with 9..16 rows per lane (N x P = 32768 floats per
    // head) where that grid still reaches the waves target, ahead of the column tiles the
    // loop below would take: at 32 slots, P = 128, N = 256 each workgroup then streams one
    // contiguous 128 KiB block, and verify took 38.3-38.7 us against 39.8-40.7 us with two
    // column tiles of 8 rows per lane (16-wave whole-row workgroups: 44.6 us).
    {
        const int rg = 8 * (256 / P);  // row groups of an 8-wave workgroup (P/4 lanes per row)
        const int rows = rg <= N ? N / rg : 0;
        if (rows > kRowsTarget && rows <= 16 && 8 * 64 <= max_threads(rows) &&
            verify_lds_floats(N, P, K, kmax, 8) * sizeof(float) <= kVerifyLdsMax &&
            (int64_t)batch * H * 8 >= kWavesTarget)
            return Shape{8, rows, 1};
    }
    for (int64_t target : {kWavesTarget, kWavesTarget / 4}) {
        for (int cs = 1; cs <= 4 && P / cs >= 16; cs *= 2) {
            const int Pc = P / cs, RGW = 256 / Pc;
            for (int S = 1; S <= 8; S *= 2) {
                const int rg = S * RGW;
                if (rg > N) break;
                const int rows = N / rg;
                if (rows > kRowsTarget || S * 64 > max_threads(rows)) continue;
                if (verify_lds_floats(N, Pc, K, kmax, S) * sizeof(float) > kVerifyLdsMax) continue;
                if ((int64_t)batch * H * cs * S >= target) return Shape{S, rows, cs};
            }
        }
    }
    for (int cs = 1; cs <= 4 && P / cs >= 16; cs *= 2) {
        const int Pc = P / cs;
        const int RGW = 256 / Pc;  // row groups per wave (Pc/4 lanes per row)
        for (int S = 1; S <= 16; S *= 2) {
            const int rg = S * RGW;
            if (rg > N) break;
            const int rows = N / rg;
            if (rows > 32 || S * 64 > max_threads(rows)) continue;
            if (verify_lds_floats(N, Pc, K, kmax, S) * sizeof(float) > kVerifyLdsMax) continue;
            best = {S, rows, cs};
            if (rows <= kRowsTarget && (int64_t)batch * H * cs * S >= kWavesTarget) return best;
        }
        if (best.S) return best;
    }
    return best;
}

hipError_t dispatch_verify_bf16(const VerifyParams &vp, int batch, hipStream_t s);
hipError_t dispatch_verify_f32(const VerifyParams &vp, int batch, hipStream_t s);

namespace {

// 16 stored bytes -> fp32 values in LDS (bf16 widens exactly by a 16-bit shift).
__device__ __forceinline__ void put16(float *dst, const uint4 v, const uint16_t *) {
    reinterpret_cast<float4 *>(dst)[0] = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                                                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
    reinterpret_cast<float4 *>(dst)[1] = make_float4(__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xffff0000u),
                                                     __uint_as_float(v.w << 16), __uint_as_float(v.w & 0xffff0000u));
}
__device__ __forceinline__ void put16(float *dst, const uint4 v, const float *) {
    *reinterpret_cast<uint4 *>(dst) = v;
}

// Draft k's root path as a bit mask (bit i: node i is on it), walking the parent links
// up from k.  A link outside -1..i-1 ends the walk (the node is taken as a child of the
// state) and is reported through *bad.
__device__ __forceinline__ uint32_t path_mask(const int *par, int k, bool &bad) {
    uint32_t m = 0;
    int a = k;
    while (a >= 0) {
        m |= 1u << a;
        const int q = par[a];
        if (q < -1 || q >= a) {
            bad = true;
            break;
        }
        a = q;
    }
    return m;
}

template <typename T, int ROWS>
__global__ __launch_bounds__(max_threads(ROWS)) void ssm_verify_kernel(const VerifyParams p) {
    extern __shared__ __align__(16) float lds[];
    const int N = p.N, P = p.P, H = p.H, G = p.G, K = p.K, kmax = p.k_max;
    const int Pc = P / p.cs;       // columns of this workgroup's tile
    const int LPR = Pc >> 2;       // lanes per state row
    const int RGW = 64 / LPR;      // row groups per wave
    const int NT = blockDim.x, S = NT >> 6;
    float *sRB = lds;              // [kmax][N]  pending rows' B
    float *sDB = sRB + kmax * N;   // [K][N]     drafts' B
    float *sDC = sDB + K * N;      // [K][N]     drafts' C
    float *sRX = sDC + K * N;      // [kmax][Pc] pending rows' x (own columns)
    float *sXd = sRX + kmax * Pc;  // [K][Pc]    drafts' x (own columns)
    float *sRA = sXd + K * Pc;     // [kmax]     pending rows' abar
    float *sRdt = sRA + kmax;      // [kmax]     pending rows' dt
    float *sDA = sRdt + kmax;      // [K]        drafts' abar
    float *sDdt = sDA + K;         // [K]        drafts' dt
    float *sAlpha = sDdt + K;      // [K]        alpha_k
    float *sW = sAlpha + K;        // [K][K]     beta_{k,s} dt_s (C_k . B_s)
    float *sRed = sW + K * K;      // [S][K][Pc] per-wave partial C_k . h0
    int *sPar = reinterpret_cast<int *>(sRed + S * K * Pc);  // [K] parent links

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c4 = lane % LPR, rsub = lane / LPR;
    const int n0 = (wave * RGW + rsub) * ROWS;
    const int h = blockIdx.x / p.cs, b = blockIdx.y;
    const int col0 = (blockIdx.x - h * p.cs) * Pc;
    const int g = h / (H / G);
    // The slot's pending count m: loaded here through the vector memory path (it returns in
    // order with the loads after it, so staging the token rows waits for it too) and used
    // only once every load is issued, so that no workgroup waits for it before asking for
    // its rows (a scalar load would be waited on with the kernel's other scalar loads).
    const int mraw = __hip_atomic_load(p.pending + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float Ah = p.A[h], Dh = p.D[h];

    const T *pX = static_cast<const T *>(p.pend_x);
    const T *pB = static_cast<const T *>(p.pend_B);
    const T *pDt = static_cast<const T *>(p.pend_dt);
    const T *dX = static_cast<const T *>(p.x);
    const T *dB = static_cast<const T *>(p.B);
    const T *dC = static_cast<const T *>(p.C);
    const T *dDt = static_cast<const T *>(p.dt);

    if (K == 0) {  // a fold alone: nothing to do for a slot without pending rows
        asm volatile("" ::: "memory");  // keeps this test (and its wait for m) off the K > 0 path
        if (min(max(__builtin_amdgcn_readfirstlane(mraw), 0), kmax) == 0) return;
    }

    // ---- staging.  The global loads go out in one batch and are waited on once: first
    // the token rows this workgroup needs as 16-byte chunks (pending B, draft B, draft C:
    // N wide; pending x, draft x: this tile's Pc columns), then the dt values, then the
    // state rows.  Loads return in issue order, so writing the token rows to LDS waits
    // for them alone while the state loads are still in flight.  All k_max pending rows
    // are loaded whatever m is (the area holds them; rows past m are staged and unused), so
    // no address waits for m. ----
    constexpr int E = 16 / sizeof(T);       // elements per chunk
    constexpr int CH = ROWS >= 32 ? 1 : 4;  // chunks per thread in the batch
    const int lgN = __builtin_ctz(N / E), lgP = __builtin_ctz(Pc / E);
    const int e0 = kmax << lgN, e1 = e0 + (K << lgN), e2 = e1 + (K << lgN);
    const int e3 = e2 + (kmax << lgP), e4 = e3 + (K << lgP);
    const bool batched = p.vec && e4 <= CH * NT;  // else: element loops after the state loads
    const int xoff = (int)(sRX - lds);
    uint4 v[CH];
    int dst[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) dst[j] = -1;
    if (batched) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = j * NT + tid;
            if (c < e4) {
                const T *src;
                if (c < e2) {
                    const int seg = c < e0 ? 0 : (c < e1 ? 1 : 2);
                    const int cc = c - (seg == 0 ? 0 : (seg == 1 ? e0 : e1));
                    const int r = cc >> lgN, q = (cc & ((1 << lgN) - 1)) * E;
                    const size_t row = seg == 0 ? (size_t)(b * kmax + r) : (size_t)(b * K + r);
                    src = (seg == 0 ? pB : (seg == 1 ? dB : dC)) + (row * G + g) * N + q;
                    dst[j] = (seg == 0 ? 0 : (seg == 1 ? kmax * N : (kmax + K) * N)) + r * N + q;
                } else {
                    const bool pend = c < e3;
                    const int cc = c - (pend ? e2 : e3);
                    const int r = cc >> lgP, q = (cc & ((1 << lgP) - 1)) * E;
                    const size_t row = pend ? (size_t)(b * kmax + r) : (size_t)(b * K + r);
                    src = (pend ? pX : dX) + (row * H + h) * P + col0 + q;
                    dst[j] = xoff + (pend ? 0 : kmax * Pc) + r * Pc + q;
                }
                v[j] = *reinterpret_cast<const uint4 *>(src);
            }
        }
    }
    // dt of pending row / draft `tid`, from rows that exist whatever m and K are
    const size_t prow = (size_t)(b * kmax + min(tid, kmax - 1)) * H + h;
    const T *dsrc = K > 0 ? dDt + (size_t)(b * K + max(min(tid, K - 1), 0)) * H + h : pDt + prow;
    const float pdt = ld(pDt, prow);
    const float ddt = ld(dsrc, 0);
    // draft tid's parent link, read before the state so that staging it waits for nothing
    // else.  The load is issued for a chain too (from the slot's pending count: any valid
    // word) and a chain's link tid - 1 is taken where it is staged.  With a branch around
    // the load the compiler guarded the link's register against the tree path's load in
    // flight, and the chain path waited for every load before issuing the state loads.
    const int *plink = p.parent ? p.parent + (size_t)b * K + max(min(tid, K - 1), 0) : p.pending + b;
    const int link = *plink;

    // the state rows: 16-byte buffer loads, one read per element
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(p.state + (size_t)(b * H + h) * p.head_stride, N * P * 4);
    const int voff = (n0 * P + col0 + 4 * c4) * 4;  // this lane's first row and columns
    float4 hv[ROWS];
#pragma unroll
    for (int i = 0; i < ROWS; ++i) hv[i] = buf_load4(srs, voff, i * P * 4);
    // uniform, so branches on m stay scalar; clamped to the pending area, so that no value in
    // the buffer can make the staging or the fold read or write outside it
    const int m = min(max(__builtin_amdgcn_readfirstlane(mraw), 0), kmax);

    if (batched) {
#pragma unroll
        for (int j = 0; j < CH; ++j)
            if (dst[j] >= 0) put16(lds + dst[j], v[j], static_cast<const T *>(nullptr));
    } else {
        for (int i = tid; i < m * N; i += NT) {
            const int s = i / N, n = i - s * N;
            sRB[i] = ld(pB, ((size_t)(b * kmax + s) * G + g) * N + n);
        }
        for (int i = tid; i < K * N; i += NT) {
            const int k = i / N, n = i - k * N;
            const size_t off = ((size_t)(b * K + k) * G + g) * N + n;
            sDB[i] = ld(dB, off);
            sDC[i] = ld(dC, off);
        }
        for (int i = tid; i < m * Pc; i += NT) {
            const int s = i / Pc, c = i - s * Pc;
            sRX[i] = ld(pX, ((size_t)(b * kmax + s) * H + h) * P + col0 + c);
        }
        for (int i = tid; i < K * Pc; i += NT) {
            const int k = i / Pc, c = i - k * Pc;
            sXd[i] = ld(dX, ((size_t)(b * K + k) * H + h) * P + col0 + c);
        }
    }
    if (tid < m) {
        sRdt[tid] = pdt;
        sRA[tid] = expf(pdt * Ah);
    }
    if (tid < K) {
        sDdt[tid] = ddt;
        sDA[tid] = expf(ddt * Ah);
        sPar[tid] = p.parent ? link : tid - 1;
    }

    lds_barrier();  // the staged rows are visible; the state loads may still be in flight

    // ---- per-draft scalars: alpha_k and w_{k,s}, eight lanes per (k, s) pair, over each
    // draft's root path (all of 0..k for a chain) ----
    // A chain's root path of draft k is 0..k: its mask is formed directly instead of by
    // walking k + 1 links through LDS, one dependent read after another (the same mask, so
    // the same products in the same order; at K = 8 the walks held the per-draft scalars
    // about 1 us: batched verify 17.0 -> 16.1 us).
    bool bad = false;
    const bool chain = p.parent == nullptr;
    if (tid < K) {
        const uint32_t pm = chain ? (2u << tid) - 1u : path_mask(sPar, tid, bad);
        float a = 1.f;
        for (int i = 0; i <= tid; ++i)
            if ((pm >> i) & 1u) a *= sDA[i];
        sAlpha[tid] = a;
    }
    // LP lanes per (k, s) pair (one pass for K <= 8 in a 512-thread workgroup), each taking
    // 4 consecutive n of every 4 LP (16-byte LDS reads) into four interleaved partial sums
    // (short rounding chains), then a butterfly over the LP lanes.  LP depends on N alone,
    // so a dot product is formed the same way whatever K is (a tree node's output stays
    // bit-identical to a flat verify of its path).
    const int LP = N >= 32 ? 8 : N / 4;
    const int lgLP = __builtin_ctz(LP);
    for (int base = 0; base < K * K * LP; base += NT) {
        const int i = base + tid;
        const int pair = i >> lgLP, part = i & (LP - 1);
        const int k = pair / max(K, 1), s = pair - k * K;
        const uint32_t pm = pair < K * K ? (chain ? (2u << k) - 1u : path_mask(sPar, k, bad)) : 0u;
        const bool live = pair < K * K && s <= k && ((pm >> s) & 1u);
        float d4[4] = {0.f, 0.f, 0.f, 0.f};
        if (live)
            for (int n = 4 * part, c = 0; n < N; n += 4 * LP, ++c) {
                const float4 cv = *reinterpret_cast<const float4 *>(sDC + k * N + n);
                const float4 bv = *reinterpret_cast<const float4 *>(sDB + s * N + n);
                float &a = d4[c & 3];
                a = __builtin_fmaf(cv.x, bv.x, a);
                a = __builtin_fmaf(cv.y, bv.y, a);
                a = __builtin_fmaf(cv.z, bv.z, a);
                a = __builtin_fmaf(cv.w, bv.w, a);
            }
        float dot = (d4[0] + d4[1]) + (d4[2] + d4[3]);
        for (int d = 1; d < LP; d <<= 1) dot += __shfl_xor(dot, d);
        if (part == 0 && pair < K * K) {
            float w = 0.f;
            if (live) {
                float beta = 1.f;
                for (int j = s + 1; j <= k; ++j)
                    if ((pm >> j) & 1u) beta *= sDA[j];
                w = beta * sDdt[s] * dot;
            }
            sW[k * K + s] = w;
        }
    }

    if (bad && p.err) atomicOr(p.err + b, MIL_DEVERR_TREE);

    // ---- fold the m pending rows, token by token: the lane's first half of the state rows
    // while the second half may still be arriving, then the second (each element takes the
    // same steps in the same order either way; batched shape 17.75 -> 17.5 us) ----
    constexpr int HALF = ROWS > 1 ? ROWS / 2 : 1;
#pragma unroll
    for (int i0 = 0; i0 < ROWS; i0 += HALF) {
        for (int s = 0; s < m; ++s) {
            const float a = sRA[s], d = sRdt[s];
            const float4 xr = *reinterpret_cast<const float4 *>(sRX + s * Pc + 4 * c4);
            const float4 u = make_float4(d * xr.x, d * xr.y, d * xr.z, d * xr.w);  // dt * x
            const float *bs = sRB + s * N + n0;
#pragma unroll
            for (int i = i0; i < i0 + HALF; ++i) {
                const float bn = bs[i];
                hv[i].x = state_step(a, hv[i].x, bn, u.x);
                hv[i].y = state_step(a, hv[i].y, bn, u.y);
                hv[i].z = state_step(a, hv[i].z, bn, u.z);
                hv[i].w = state_step(a, hv[i].w, bn, u.w);
            }
        }
    }
    // The folded state goes back to HBM only when the next commit could overflow the
    // pending area (m + K > k_max; always for a fold alone): otherwise the accepted rows stay
    // pending (the logical state is unchanged either way, and every later fold runs the
    // same steps in the same order, so the bits do not depend on when the write happens)
    // and the commit appends to them.  One thread per slot records where it appends.
    const bool write_back = m > 0 && (K == 0 || m + K > kmax);
    if (threadIdx.x == 0 && blockIdx.x == 0) p.append[b] = write_back || m == 0 ? 0 : m;
    if (K == 0) {  // fold only: no outputs
        if (write_back) {
#pragma unroll
            for (int i = 0; i < ROWS; ++i) buf_store4(hv[i], srs, voff, i * P * 4);
        }
        return;
    }

    // ---- C_k . h0 over this lane's rows, then over the wave's row groups, two drafts at a
    // time: independent sums, so that their shuffles overlap; each sum runs in the same order
    // as one draft at a time (a draft past K is clamped and computed but not stored).
    // Measured against one draft at a time: hybrid 37.7-38.0 -> 37.3 us, batched 16.0 us
    // either way; four at a time was no faster and needs 11 more registers at 16 rows. ----
    constexpr int KB = 2;
    for (int k0 = 0; k0 < K; k0 += KB) {
        float4 acc[KB];
#pragma unroll
        for (int u = 0; u < KB; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < ROWS; ++i) {
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                const float c = sDC[min(k0 + u, K - 1) * N + n0 + i];
                acc[u].x = __builtin_fmaf(c, hv[i].x, acc[u].x);
                acc[u].y = __builtin_fmaf(c, hv[i].y, acc[u].y);
                acc[u].z = __builtin_fmaf(c, hv[i].z, acc[u].z);
                acc[u].w = __builtin_fmaf(c, hv[i].w, acc[u].w);
            }
        }
        for (int d = LPR; d < 64; d <<= 1) {
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                acc[u].x += __shfl_xor(acc[u].x, d);
                acc[u].y += __shfl_xor(acc[u].y, d);
                acc[u].z += __shfl_xor(acc[u].z, d);
                acc[u].w += __shfl_xor(acc[u].w, d);
            }
        }
        if (rsub == 0) {
#pragma unroll
            for (int u = 0; u < KB; ++u)
                if (k0 + u < K) *reinterpret_cast<float4 *>(sRed + (wave * K + k0 + u) * Pc + 4 * c4) = acc[u];
        }
    }
    // the folded rows go back (once, when m > 0) after the C_k . h0 products have used them,
    // and the barrier waits for them to drain before the readout.  Measured against writing
    // them right after the fold (then draining under the products and the readout): the
    // same at 32 x 32 heads, N = 256, K = 4, and 1.5 us faster at 16 x 32 heads, N = 128,
    // K = 8, where every workgroup is resident at once and early stores compete with the
    // other workgroups' state loads.
    if (write_back) {
#pragma unroll
        for (int i = 0; i < ROWS; ++i) buf_store4(hv[i], srs, voff, i * P * 4);
    }
    __syncthreads();

    // ---- outputs: waves summed in order, then the closed-form draft terms ----
    for (int i = tid; i < K * LPR; i += NT) {
        const int k = i / LPR, q = i - k * LPR;
        float4 ch = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int w = 0; w < S; ++w) {
            const float4 v = *reinterpret_cast<const float4 *>(sRed + (w * K + k) * Pc + 4 * q);
            ch.x += v.x;
            ch.y += v.y;
            ch.z += v.z;
            ch.w += v.w;
        }
        const float al = sAlpha[k];
        float4 yv = make_float4(al * ch.x, al * ch.y, al * ch.z, al * ch.w);
        for (int s2 = 0; s2 <= k; ++s2) {
            const float wv = sW[k * K + s2];
            const float4 xs = *reinterpret_cast<const float4 *>(sXd + s2 * Pc + 4 * q);
            yv.x = __builtin_fmaf(wv, xs.x, yv.x);
            yv.y = __builtin_fmaf(wv, xs.y, yv.y);
            yv.z = __builtin_fmaf(wv, xs.z, yv.z);
            yv.w = __builtin_fmaf(wv, xs.w, yv.w);
        }
        const float4 xk = *reinterpret_cast<const float4 *>(sXd + k * Pc + 4 * q);
        yv.x = __builtin_fmaf(Dh, xk.x, yv.x);
        yv.y = __builtin_fmaf(Dh, xk.y, yv.y);
        yv.z = __builtin_fmaf(Dh, xk.z, yv.z);
        yv.w = __builtin_fmaf(Dh, xk.w, yv.w);
        *reinterpret_cast<float4 *>(p.y + ((size_t)(b * K + k) * H + h) * P + col0 + 4 * q) = yv;
    }
}

template <typename T, int ROWS>
hipError_t launch_one(const VerifyParams &vp, const Shape &sh, int batch, hipStream_t s) {
    const size_t lds = sizeof(float) * verify_lds_floats(vp.N, vp.P / sh.CS, vp.K, vp.k_max, sh.S);
    auto kern = ssm_verify_kernel<T, ROWS>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    VerifyParams q = vp;
    q.cs = sh.CS;
    hipLaunchKernelGGL(kern, dim3(vp.H * sh.CS, batch), dim3(sh.S * 64), lds, s, q);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_rows(const VerifyParams &vp, int batch, hipStream_t s) {
    const Shape sh = shape_for(batch, vp.H, vp.P, vp.N, vp.K, vp.k_max);
    switch (sh.ROWS) {
        case 1: return launch_one<T, 1>(vp, sh, batch, s);
        case 2: return launch_one<T, 2>(vp, sh, batch, s);
        case 4: return launch_one<T, 4>(vp, sh, batch, s);
        case 8: return launch_one<T, 8>(vp, sh, batch, s);
        case 16: return launch_one<T, 16>(vp, sh, batch, s);
        case 32: return launch_one<T, 32>(vp, sh, batch, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace mil
