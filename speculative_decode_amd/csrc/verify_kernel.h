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
// Work decomposition (gfx950, wave64): a workgroup owns PT state columns of one
// (slot, head); each wave splits into 64/PT row groups of PT lanes, S waves per group,
// so each lane owns ROWS consecutive rows of one column.  State traffic is one coalesced
// fp32 read (and at most one write) per element; the per-row work is in registers and
// the cross-row-group sum goes through LDS once at the end, in a fixed order.
#pragma once

#include "ssm_internal.h"

namespace mil {


// Stored element -> fp32 (bf16 widens exactly by a 16-bit shift).
__device__ __forceinline__ float ld(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t *p, size_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

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
    const void *x, *B, *C, *dt;
    const float *A, *D;
    float *y;
    int H, P, N, G, K, k_max;
    int pt_log2;
};


// Launch shape for (P, N): PT columns per workgroup, S waves, ROWS rows per lane.
struct Shape {
    int PT, S, ROWS;
};

inline Shape shape_for(int P, int N) {
    const int PT = P < 64 ? P : 64;
    const int RGW = 64 / PT;
    int rows = N / RGW;  // with one wave
    int S = 1;
    while (rows > 32 && S < 8) {  // at most 32 rows per lane
        S *= 2;
        rows /= 2;
    }
    return {PT, S, rows};
}

inline int log2i(int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

inline bool shape_known(int P, int N) {
    const Shape sh = shape_for(P, N);
    const int RG = sh.S * (64 / sh.PT);
    return RG * sh.ROWS == N && P % sh.PT == 0 &&
           (sh.ROWS == 4 || sh.ROWS == 8 || sh.ROWS == 16 || sh.ROWS == 32);
}


hipError_t dispatch_verify_bf16(const VerifyParams &vp, int kt, int batch, hipStream_t s);
hipError_t dispatch_verify_f32(const VerifyParams &vp, int kt, int batch, hipStream_t s);

namespace {

template <typename T, int ROWS, int KT>
__global__ __launch_bounds__(512) void ssm_verify_kernel(const VerifyParams p) {
    // runtime shape: PT = 1 << p.pt_log2 columns per workgroup, S = blockDim.x / 64 waves
    extern __shared__ float lds[];
    const int PT = 1 << p.pt_log2;
    const int RGW = 64 >> p.pt_log2;     // row groups per wave
    const int NT = blockDim.x;
    const int RG = (NT >> 6) * RGW;      // row groups per workgroup
    const int N = p.N;                   // == RG * ROWS (checked by the launcher)
    float *sRB = lds;                    // [KT][N]  pending rows' B
    float *sDB = sRB + KT * N;           // [KT][N]  drafts' B
    float *sDC = sDB + KT * N;           // [KT][N]  drafts' C
    float *sRA = sDC + KT * N;           // [KT]     pending rows' abar
    float *sDA = sRA + KT;               // [KT]     drafts' abar
    float *sDdt = sDA + KT;              // [KT]     drafts' dt
    float *sAlpha = sDdt + KT;           // [KT]     alpha_k
    float *sW = sAlpha + KT;             // [KT][KT] beta_{k,s} dt_s (C_k . B_s)
    float *sXd = sW + KT * KT;           // [KT][PT] drafts' x on this column tile
    float *sRed = sXd + KT * PT;         // [RG][KT][PT] partial C_k . h0 per row group

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & (PT - 1);
    const int rg = wave * RGW + (lane >> p.pt_log2);
    const int b = blockIdx.z, h = blockIdx.y;
    const int H = p.H, P = p.P, G = p.G, K = p.K, kmax = p.k_max;
    const int g = h / (H / G);
    const int c0 = blockIdx.x * PT;
    const int pcol = c0 + col;
    const int m = p.pending[b];
    const float Ah = p.A[h];

    const T *pX = static_cast<const T *>(p.pend_x);
    const T *pB = static_cast<const T *>(p.pend_B);
    const T *pDt = static_cast<const T *>(p.pend_dt);
    const T *dX = static_cast<const T *>(p.x);
    const T *dB = static_cast<const T *>(p.B);
    const T *dC = static_cast<const T *>(p.C);
    const T *dDt = static_cast<const T *>(p.dt);

    // ---- small token loads first, so that waiting for them does not wait for the state ----
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
    for (int i = tid; i < K * PT; i += NT) {
        const int k = i >> p.pt_log2, c = i & (PT - 1);
        sXd[i] = ld(dX, ((size_t)(b * K + k) * H + h) * P + c0 + c);
    }
    float u[KT];  // dt_s * x_s[pcol] of the pending rows
#pragma unroll
    for (int s = 0; s < KT; ++s) {
        u[s] = 0.f;
        if (s < m) {
            const size_t row = (size_t)(b * kmax + s);
            u[s] = ld(pDt, row * H + h) * ld(pX, (row * H + h) * P + pcol);
        }
    }
    if (tid < m) sRA[tid] = expf(ld(pDt, (size_t)(b * kmax + tid) * H + h) * Ah);
    if (tid < K) {
        const float d = ld(dDt, (size_t)(b * K + tid) * H + h);
        sDdt[tid] = d;
        sDA[tid] = expf(d * Ah);
    }

    // ---- the state rows: one coalesced read per element ----
    float *st = p.state + (size_t)(b * H + h) * p.head_stride + pcol;
    const int n0 = rg * ROWS;
    float hr[ROWS];
#pragma unroll
    for (int i = 0; i < ROWS; ++i) hr[i] = st[(size_t)(n0 + i) * P];

    __syncthreads();

    // ---- per-draft scalars: alpha_k and w_{k,s} = beta_{k,s} dt_s (C_k . B_s) ----
    if (tid < K) {
        float a = 1.f;
        for (int i = 0; i <= tid; ++i) a *= sDA[i];
        sAlpha[tid] = a;
    }
    // eight lanes per (k, s) pair, each over every eighth n, then a fixed butterfly
    for (int base = 0; base < K * K * 8; base += NT) {
        const int i = base + tid;
        const int pair = i >> 3, part = i & 7;
        const int k = pair / max(K, 1), s = pair - k * K;
        const bool live = pair < K * K && s <= k;
        float dot = 0.f;
        if (live)
            for (int n = part; n < N; n += 8) dot = __builtin_fmaf(sDC[k * N + n], sDB[s * N + n], dot);
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        dot += __shfl_xor(dot, 4);
        if (part == 0 && pair < K * K) {
            float w = 0.f;
            if (live) {
                float beta = 1.f;
                for (int j = s + 1; j <= k; ++j) beta *= sDA[j];
                w = beta * sDdt[s] * dot;
            }
            sW[k * KT + s] = w;
        }
    }

    // ---- fold the pending rows, write back once, accumulate C_k . h0 ----
    float acc[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) acc[k] = 0.f;
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int n = n0 + i;
        float hv = hr[i];
#pragma unroll
        for (int s = 0; s < KT; ++s)
            if (s < m) hv = state_step(sRA[s], hv, sRB[s * N + n], u[s]);
        if (m > 0) st[(size_t)n * P] = hv;
#pragma unroll
        for (int k = 0; k < KT; ++k)
            if (k < K) acc[k] = __builtin_fmaf(sDC[k * N + n], hv, acc[k]);
    }
    if (K == 0) return;  // fold only
#pragma unroll
    for (int k = 0; k < KT; ++k)
        if (k < K) sRed[(rg * KT + k) * PT + col] = acc[k];
    __syncthreads();

    // ---- outputs: sum row groups in order, then the closed-form draft terms ----
    const float Dh = p.D[h];
    for (int i = tid; i < K * PT; i += NT) {
        const int k = i >> p.pt_log2, c = i & (PT - 1);
        float ch = 0.f;
        for (int r = 0; r < RG; ++r) ch += sRed[(r * KT + k) * PT + c];
        float yv = sAlpha[k] * ch;
        for (int s = 0; s <= k; ++s) yv = __builtin_fmaf(sW[k * KT + s], sXd[s * PT + c], yv);
        yv = __builtin_fmaf(Dh, sXd[k * PT + c], yv);
        p.y[((size_t)(b * K + k) * H + h) * P + c0 + c] = yv;
    }
}

size_t lds_bytes(int N, int KT, int PT, int S) {
    return sizeof(float) * (size_t)(3 * KT * N + 4 * KT + KT * KT + KT * PT + S * 64 * KT);
}

template <typename T, int ROWS, int KT>
hipError_t launch_one(VerifyParams vp, const Shape &sh, int batch, hipStream_t s) {
    vp.pt_log2 = log2i(sh.PT);
    const size_t lds = lds_bytes(vp.N, KT, sh.PT, sh.S);
    auto kern = ssm_verify_kernel<T, ROWS, KT>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    dim3 grid(vp.P / sh.PT, vp.H, batch);
    hipLaunchKernelGGL(kern, grid, dim3(sh.S * 64), lds, s, vp);
    return hipGetLastError();
}

template <typename T, int KT>
hipError_t dispatch_rows(const VerifyParams &vp, int batch, hipStream_t s) {
    const Shape sh = shape_for(vp.P, vp.N);
    switch (sh.ROWS) {
        case 4: return launch_one<T, 4, KT>(vp, sh, batch, s);
        case 8: return launch_one<T, 8, KT>(vp, sh, batch, s);
        case 16: return launch_one<T, 16, KT>(vp, sh, batch, s);
        case 32: return launch_one<T, 32, KT>(vp, sh, batch, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace mil
