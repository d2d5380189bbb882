// Chunked full-sequence scan of the SSM layer ("The Mamba in the Llama"; skycaiji.com
// summary, method paragraph: the layer is a discretised linear RNN whose state is
// expanded, evaluated through a hardware-aware decomposition).  The sequence is cut
// into chunks of Q tokens.  With abar_t = exp(dt_t A) and, for s <= t in one chunk,
// decay(s,t) = exp(A * sum_{r=s+1..t} dt_r):
//   phase 1  S_c   = sum_s decay(s, end) dt_s B_s x_s^T            (chunk's own state)
//   phase 2  h_in  : h_in(0) = h0,  h_in(c+1) = exp(A sum_c dt) h_in(c) + S_c
//   phase 3  y_t   = sum_{s<=t} decay(s,t) dt_s (C_t . B_s) x_s    (quadratic form)
//                  + exp(A sum_{r<=t} dt_r) C_t^T h_in(c) + D x_t
// which is the recurrence regrouped, so it agrees with the token-by-token scan up to
// rounding.
//
// Decay factors are never formed as a difference of two long prefix sums (whose
// rounding would grow with the chunk's total decay): every exponent is a sum over at
// most one 16-token tile, or a direct sum of whole-tile totals, so each factor's
// relative error is a few ulps of its own exponent.
//
// This file holds the fp32 vector-ALU form, used for fp32 inputs and for shapes the
// matrix-core form (prefill_mfma.hip, bf16 inputs) does not cover.
#include <algorithm>

#include "ssm_internal.h"

namespace mil {
namespace {

constexpr int kTile = 16;  // decay tile (tokens)

__device__ __forceinline__ float ld(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t *p, size_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

struct PrefillParams {
    const void *x, *B, *C, *dt;
    const float *A, *D;
    float *y;
    float *state;          // cache state, slot0 block
    int64_t head_stride;   // floats
    float *ws_state;       // [nseq][nch][H][N][P]
    float *ws_tot;         // [nseq][nch][H]
    int32_t *pos, *pending;  // cache counters (whole batch)
    int L, Q, nch, H, P, N, G;
    int slot0, nseq, batch;
    int cont;
};

// ---------------------------------------------------------------- phase 1
// grid (nch, H, nseq * slabs); each block owns `rows` state rows of one chunk-head.
template <typename T>
__global__ __launch_bounds__(256) void chunk_state_valu(const PrefillParams p, int rows, int slabs) {
    constexpr int EPT = 64;
    __shared__ float sDtA[256], sDt[256], sW[256];
    __shared__ float sBw[kTile][256];
    __shared__ float sX[kTile][256];
    const int c = blockIdx.x, h = blockIdx.y;
    const int seq = blockIdx.z / slabs, slab = blockIdx.z % slabs;
    const int tid = threadIdx.x;
    const int H = p.H, P = p.P, N = p.N, G = p.G;
    const int g = h / (H / G);
    const int c0 = c * p.Q;
    const int len = min(p.Q, p.L - c0);
    const float Ah = p.A[h];
    const T *X = static_cast<const T *>(p.x);
    const T *Bm = static_cast<const T *>(p.B);
    const T *Dt = static_cast<const T *>(p.dt);
    for (int s = tid; s < len; s += 256) {
        const float d = ld(Dt, ((size_t)seq * p.L + c0 + s) * H + h);
        sDt[s] = d;
        sDtA[s] = d * Ah;
    }
    __syncthreads();
    if (tid == 0) {
        // suffix sums sum_{r=s+1..len-1} dtA_r, accumulated from the end
        float suf = 0.f;
        for (int s = len - 1; s >= 0; --s) {
            sW[s] = expf(suf) * sDt[s];
            suf += sDtA[s];
        }
        if (slab == 0) p.ws_tot[((size_t)seq * p.nch + c) * H + h] = suf;
    }
    __syncthreads();
    const int n0 = slab * rows;
    const int nel = rows * P;
    float acc[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) acc[i] = 0.f;
    for (int t0 = 0; t0 < len; t0 += kTile) {
        const int tl = min(kTile, len - t0);
        for (int i = tid; i < kTile * rows; i += 256) {
            const int j = i / rows, n = i % rows;
            sBw[j][n] = j < tl ? sW[t0 + j] * ld(Bm, (((size_t)seq * p.L + c0 + t0 + j) * G + g) * N + n0 + n) : 0.f;
        }
        for (int i = tid; i < kTile * P; i += 256) {
            const int j = i / P, q = i % P;
            sX[j][q] = j < tl ? ld(X, (((size_t)seq * p.L + c0 + t0 + j) * H + h) * P + q) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = tid + 256 * i;
            if (e < nel) {
                const int n = e / P, q = e % P;
                float a = acc[i];
                for (int j = 0; j < kTile; ++j) a = __builtin_fmaf(sBw[j][n], sX[j][q], a);
                acc[i] = a;
            }
        }
        __syncthreads();
    }
    float *out = p.ws_state + (((size_t)seq * p.nch + c) * H + h) * (size_t)N * P + (size_t)n0 * P;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid + 256 * i;
        if (e < nel) out[e] = acc[i];
    }
}

// ---------------------------------------------------------------- phase 2
// grid (ceil(N*P/256), H, nseq): the short sequential pass across chunks, elementwise.
// Replaces each chunk state in the workspace by the state entering that chunk and
// writes the final state into the cache.
__global__ __launch_bounds__(256) void state_pass_kernel(const PrefillParams p) {
    const int h = blockIdx.y, seq = blockIdx.z;
    if (blockIdx.x == 0 && h == 0 && seq == 0) {
        // counters: the prefilled slots absorb L tokens; nothing is pending afterwards
        for (int i = threadIdx.x; i < p.batch; i += blockDim.x) {
            const bool mine = i >= p.slot0 && i < p.slot0 + p.nseq;
            if (mine) p.pos[i] = p.cont ? p.pos[i] + p.L : p.L;
            if (mine || p.cont) p.pending[i] = 0;
        }
    }
    const int64_t NP = (int64_t)p.N * p.P;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= NP) return;
    float *cache = p.state + (size_t)(seq * p.H + h) * p.head_stride + e;
    float hv = p.cont ? *cache : 0.f;
    for (int c = 0; c < p.nch; ++c) {
        const size_t ch = ((size_t)seq * p.nch + c) * p.H + h;
        float *slot = p.ws_state + ch * NP + e;
        const float sc = *slot;
        *slot = hv;
        hv = __builtin_fmaf(expf(p.ws_tot[ch]), hv, sc);
    }
    *cache = hv;
}

// ---------------------------------------------------------------- phase 3
// grid (ceil(Q/16), nch, H * nseq); each block produces one 16-token tile of y.
template <typename T>
__global__ __launch_bounds__(256) void chunk_out_valu(const PrefillParams p) {
    constexpr int OPT = 16;  // outputs per thread (16 rows x P <= 256 columns)
    __shared__ float sDtA[256], sDt[256], sR[256], sL[256];
    __shared__ float sTile[256 / kTile], sMid[256 / kTile];
    __shared__ float sC[kTile][256], sB[kTile][256], sX[kTile][256];
    __shared__ float sM[kTile][kTile];
    __shared__ float sEin[kTile];
    const int I = blockIdx.x, c = blockIdx.y;
    const int h = blockIdx.z % p.H, seq = blockIdx.z / p.H;
    const int tid = threadIdx.x;
    const int H = p.H, P = p.P, N = p.N, G = p.G;
    const int g = h / (H / G);
    const int c0 = c * p.Q;
    const int len = min(p.Q, p.L - c0);
    if (I * kTile >= len) return;
    const int ntile = (len + kTile - 1) / kTile;
    const int rl = min(kTile, len - I * kTile);  // rows in this tile
    const float Ah = p.A[h];
    const T *X = static_cast<const T *>(p.x);
    const T *Bm = static_cast<const T *>(p.B);
    const T *Cm = static_cast<const T *>(p.C);
    const T *Dt = static_cast<const T *>(p.dt);
    const size_t tok0 = (size_t)seq * p.L + c0;

    for (int s = tid; s < len; s += 256) {
        const float d = ld(Dt, (tok0 + s) * H + h);
        sDt[s] = d;
        sDtA[s] = d * Ah;
    }
    for (int i = tid; i < kTile * N; i += 256) {
        const int r = i / N, n = i % N;
        sC[r][n] = r < rl ? ld(Cm, ((tok0 + I * kTile + r) * G + g) * N + n) : 0.f;
    }
    __syncthreads();
    // tile-local inclusive prefix R_t and exclusive suffix L_s, by direct short sums
    for (int t = tid; t < len; t += 256) {
        const int ts = t / kTile * kTile, te = min(ts + kTile, len) - 1;
        float r = 0.f;
        for (int q = ts; q <= t; ++q) r += sDtA[q];
        float l = 0.f;
        for (int q = te; q > t; --q) l += sDtA[q];
        sR[t] = r;
        sL[t] = l;
    }
    __syncthreads();
    if (tid < ntile) sTile[tid] = sR[min(tid * kTile + kTile, len) - 1];
    __syncthreads();
    if (tid < I) {  // whole tiles strictly between column tile tid and row tile I
        float m = 0.f;
        for (int q = tid + 1; q < I; ++q) m += sTile[q];
        sMid[tid] = expf(m);
    }
    if (tid < rl) {  // decay from the chunk start to row t: whole tiles before I, then R_t
        float m = 0.f;
        for (int q = 0; q < I; ++q) m += sTile[q];
        sEin[tid] = expf(m + sR[I * kTile + tid]);
    }

    float acc[OPT];
#pragma unroll
    for (int i = 0; i < OPT; ++i) acc[i] = 0.f;
    const int nout = kTile * P;

    for (int J = 0; J <= I; ++J) {
        const int cl = min(kTile, len - J * kTile);
        __syncthreads();
        for (int i = tid; i < kTile * N; i += 256) {
            const int j = i / N, n = i % N;
            sB[j][n] = j < cl ? ld(Bm, ((tok0 + J * kTile + j) * G + g) * N + n) : 0.f;
        }
        for (int i = tid; i < kTile * P; i += 256) {
            const int j = i / P, q = i % P;
            sX[j][q] = j < cl ? ld(X, ((tok0 + J * kTile + j) * H + h) * P + q) : 0.f;
        }
        __syncthreads();
        {
            const int r = tid / kTile, j = tid % kTile;
            const int t = I * kTile + r, s = J * kTile + j;
            float mv = 0.f;
            if (r < rl && j < cl && s <= t) {
                float dot = 0.f;
                for (int n = 0; n < N; ++n) dot = __builtin_fmaf(sC[r][n], sB[j][n], dot);
                float dec;
                if (I == J) {
                    float e = 0.f;
                    for (int q = s + 1; q <= t; ++q) e += sDtA[q];
                    dec = expf(e);
                } else {
                    dec = expf(sL[s]) * sMid[J] * expf(sR[t]);
                }
                mv = dec * sDt[s] * dot;
            }
            sM[r][j] = mv;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < OPT; ++i) {
            const int o = tid + 256 * i;
            if (o < nout) {
                const int r = o / P, q = o % P;
                float a = acc[i];
                for (int j = 0; j < kTile; ++j) a = __builtin_fmaf(sM[r][j], sX[j][q], a);
                acc[i] = a;
            }
        }
    }
    // state carried in from earlier chunks, then the skip term
    const float *hin = p.ws_state + (((size_t)seq * p.nch + c) * H + h) * (size_t)N * P;
    const float Dh = p.D[h];
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
        const int o = tid + 256 * i;
        if (o < nout) {
            const int r = o / P, q = o % P;
            if (r < rl) {
                float ch = 0.f;
                for (int n = 0; n < N; ++n) ch = __builtin_fmaf(sC[r][n], hin[(size_t)n * P + q], ch);
                const size_t t = tok0 + I * kTile + r;
                const float yv = acc[i] + sEin[r] * ch + Dh * ld(X, (t * H + h) * P + q);
                p.y[(t * H + h) * P + q] = yv;
            }
        }
    }
}

}  // namespace

int64_t prefill_workspace_bytes(const mil_ssm_dims &d, int nseq, int L, int chunk) {
    const int64_t nch = (L + chunk - 1) / chunk;
    const int64_t states = (int64_t)nseq * nch * d.nheads * d.dstate * d.headdim * 4;
    const int64_t tots = (int64_t)nseq * nch * d.nheads * 4;
    // the single-launch form keeps one record per chunk of a launch (at most kScanChunks):
    // the chunk's own state and the state after it, plus its decay padded to 16 floats per
    // column slab (at most kScanSlabs slabs)
    const int64_t nchl = std::min<int64_t>(nch, kScanChunks);
    const int64_t chain = (int64_t)nseq * d.nheads * nchl * (2 * (int64_t)d.dstate * d.headdim + 16 * kScanSlabs) * 4;
    return std::max((states + 255) / 256 * 256 + (tots + 255) / 256 * 256, (chain + 255) / 256 * 256);
}

hipError_t launch_prefill(const CacheImpl &c, int slot0, int nseq, int L, int chunk, const void *x,
                          const void *B, const void *C, const void *dt, const float *A,
                          const float *D, float *y, void *ws, bool cont, hipStream_t s) {
    const auto a16 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    if (c.dtype == MIL_BF16 && prefill_mfma_supported(chunk, c.dims.dstate, c.dims.headdim) && a16(x) &&
        a16(B) && a16(C))
        return launch_prefill_mfma(c, slot0, nseq, L, chunk, x, B, C, dt, A, D, y, ws, cont, s);
    PrefillParams p;
    p.x = x;
    p.B = B;
    p.C = C;
    p.dt = dt;
    p.A = A;
    p.D = D;
    p.y = y;
    p.head_stride = c.lay.state_head_stride / 4;
    p.state = cache_state(c) + (size_t)slot0 * c.dims.nheads * p.head_stride;
    p.L = L;
    p.Q = chunk;
    p.nch = (L + chunk - 1) / chunk;
    p.H = c.dims.nheads;
    p.P = c.dims.headdim;
    p.N = c.dims.dstate;
    p.G = c.dims.ngroups;
    p.cont = cont ? 1 : 0;
    p.pos = cache_pos(c);
    p.pending = cache_pending(c);
    p.slot0 = slot0;
    p.nseq = nseq;
    p.batch = c.dims.batch;
    const int64_t states = (int64_t)nseq * p.nch * p.H * p.N * p.P * 4;
    p.ws_state = static_cast<float *>(ws);
    p.ws_tot = reinterpret_cast<float *>(static_cast<char *>(ws) + (states + 255) / 256 * 256);

    const int rows = min(p.N, 16384 / p.P);  // 64 state elements per thread
    const int slabs = p.N / rows;
    trace_begin(c, MIL_TRACE_PREFILL_STATE, s);
    if (c.dtype == MIL_BF16)
        hipLaunchKernelGGL(chunk_state_valu<uint16_t>, dim3(p.nch, p.H, nseq * slabs), dim3(256), 0, s, p, rows, slabs);
    else
        hipLaunchKernelGGL(chunk_state_valu<float>, dim3(p.nch, p.H, nseq * slabs), dim3(256), 0, s, p, rows, slabs);
    trace_end(c, MIL_TRACE_PREFILL_STATE, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t NP = (int64_t)p.N * p.P;
    trace_begin(c, MIL_TRACE_PREFILL_PASS, s);
    hipLaunchKernelGGL(state_pass_kernel, dim3((unsigned)((NP + 255) / 256), p.H, nseq), dim3(256), 0, s, p);
    trace_end(c, MIL_TRACE_PREFILL_PASS, s);
    e = hipGetLastError();
    if (e != hipSuccess || y == nullptr) return e;
    const dim3 g3((chunk + kTile - 1) / kTile, p.nch, p.H * nseq);
    trace_begin(c, MIL_TRACE_PREFILL_OUT, s);
    if (c.dtype == MIL_BF16)
        hipLaunchKernelGGL(chunk_out_valu<uint16_t>, g3, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(chunk_out_valu<float>, g3, dim3(256), 0, s, p);
    trace_end(c, MIL_TRACE_PREFILL_OUT, s);
    return hipGetLastError();
}

}  // namespace mil
