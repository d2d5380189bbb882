// Input projections of the layer: x, B, C and the step size dt from the layer's input rows.
//
// "The Mamba in the Llama" builds the layer from an attention layer's own linear
// projection weights (arXiv abstract; skycaiji.com summary, method paragraph: the
// modified Mamba is initialised from the attention module).  Read here as
//   x = u W_V^T (per head),  B = u W_K^T,  C = u W_Q^T (per group),
//   dt = softplus(u W_dt^T + bias) (per head, so that dt > 0),
// one bf16 GEMM out[t][n] = sum_k u[t][k] W[n][k] over four weight blocks, with both
// operands K-contiguous (u [T][d], W [rows][d]) as v_mfma_f32_32x32x16_bf16 wants them,
// and fp32 accumulation.
//
// Work decomposition: a workgroup (4 waves) owns BM token rows x 128 output columns of one
// block (a column tile never straddles two blocks) and a slice of the d inputs.  Blocks of
// 64 inputs of the 128 weight rows and the BM u rows are loaded kDepth blocks ahead of the
// products, each wave reading whole 128-byte rows (eight rows per load instruction, so the
// vector memory path handles a quarter of the cache lines it would if each lane streamed
// its own weight row), and staged into one of two LDS buffers right before their
// products; wave w then takes the B operands of its 32 columns from LDS.  Each weight
// element is read once per row tile.  For few token rows (a decode round) the d inputs
// are split over S workgroups so that every CU streams weights; each writes fp32 partial
// sums and a second kernel adds the S partials in a fixed order, so the result does not
// depend on scheduling.
//
// MFMA operands: for input block kb, lane (l32, hf) takes inputs kb*64 + 32hf + [0, 32)
// of weight row l32 of its wave as four 8-element groups; step j (0..3) pairs group j of
// the weight row (B operand, column l32) with the same 8 inputs of token row l32 (A
// operand).  Any assignment of inputs to k-slots works as long as both operands use it.
#include <algorithm>

#include "ssm_internal.h"

namespace mil {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4v __attribute__((ext_vector_type(4)));

constexpr int kBN = 128;     // output columns per workgroup (4 waves x 32)
constexpr int kKB = 64;      // inputs per block
constexpr int kDepth = 4;    // weight blocks in flight per lane
constexpr int kUS = kKB + 8; // padded LDS row of u (elements)
constexpr int kWgTarget = 192;  // about one 4-wave workgroup per CU (more splits measured slower)

struct ProjParams {
    const uint16_t *u;           // [T][d] bf16
    const uint16_t *w[4];        // x, B, C, dt weight rows [cols[b]][d] bf16
    void *out[4];                // [T][cols[b]]
    const float *bias;           // [cols[3]] or null
    float *part;                 // [S][T][ncols] fp32 partial sums when S > 1
    int cols[4], colbase[4], tile0[5];
    int T, d, S, nkb, ncols, out_bf16;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}
// Weight loads use the default cache policy.  16-byte values are kept as ext_vector_type:
// arrays of them stay in registers.
__device__ __forceinline__ i32x4v wload(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(i32x4v v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float softplus(float z) { return z > 20.f ? z : log1pf(expf(z)); }

// Final value of output element (t, n) of block b, stored in the output type.
__device__ __forceinline__ void emit(const ProjParams &p, int b, int t, int n, float v) {
    if (b == 3) v = softplus(v + (p.bias ? p.bias[n] : 0.f));
    const size_t i = (size_t)t * p.cols[b] + n;
    if (p.out_bf16)
        static_cast<__bf16 *>(p.out[b])[i] = static_cast<__bf16>(v);
    else
        static_cast<float *>(p.out[b])[i] = v;
}

// EXACT: the block count is a multiple of kDepth, so the ring loop needs no guard.
template <int BM, bool EXACT>
__global__ __launch_bounds__(256) void project_gemm(const ProjParams p) {
    constexpr int MI = BM / 32;         // 32-row MFMA tiles per wave
    constexpr int UQ = BM * 8 / 256;    // 16-byte pieces of a u block per thread
    constexpr int WQ = kBN * 8 / 256;   // 16-byte pieces of a weight block per thread
    __shared__ __align__(16) __bf16 sU[2][BM][kUS];
    __shared__ __align__(16) __bf16 sW[2][kBN][kUS];

    const int ntiles = p.tile0[4];
    const int mt = blockIdx.x % ((p.T + BM - 1) / BM);
    const int rest = blockIdx.x / ((p.T + BM - 1) / BM);
    const int tile = rest % ntiles, split = rest / ntiles;
    const int b = tile >= p.tile0[3] ? 3 : tile >= p.tile0[2] ? 2 : tile >= p.tile0[1] ? 1 : 0;
    const int col0 = (tile - p.tile0[b]) * kBN;
    const int m0 = mt * BM;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5, l32 = lane & 31;
    const int d = p.d, nkb = p.nkb, k0 = split * nkb * kKB;

    // this lane's output column (columns past the block are never stored)
    const int n = col0 + wave * 32 + l32;
    const __amdgpu_buffer_rsrc_t wr = rsrc(p.w[b], (uint32_t)((size_t)p.cols[b] * d * 2));

    // weight and u pieces: row = piece / 8, 16-byte column = piece % 8, so the 64 lanes of
    // a wave read eight whole 128-byte rows of a block (weight rows past the block and u
    // rows past T clamped)
    int woff[WQ];
#pragma unroll
    for (int i = 0; i < WQ; ++i) {
        const int q = tid + 256 * i;
        const int r = min(col0 + q / 8, p.cols[b] - 1);
        woff[i] = (r * d + k0 + (q % 8) * 8) * 2;
    }
    size_t uoff[UQ];
#pragma unroll
    for (int i = 0; i < UQ; ++i) {
        const int q = tid + 256 * i;
        const int r = min(m0 + q / 8, p.T - 1);
        uoff[i] = (size_t)r * d + k0 + (q % 8) * 8;
    }

    // A ring of kDepth input blocks in flight: each slot holds this thread's weight and u
    // pieces of one block, loaded together.  Loads complete in issue order, so waiting for
    // the oldest slot leaves the other kDepth - 1 in flight.  Four named slots (constant
    // indices only, so they stay in registers).
    struct Slot {
        i32x4v w[WQ], u[UQ];
    };
    Slot s0, s1, s2, s3;
    // (the empty asm statements are compiler-only barriers that keep the blocks' loads in
    // this issue order, which the in-order completion above relies on)
    auto fetch = [&](Slot &sl, int kb) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < WQ; ++i) sl.w[i] = wload(wr, woff[i], kb * kKB * 2);
#pragma unroll
        for (int i = 0; i < UQ; ++i) sl.u[i] = *reinterpret_cast<const i32x4v *>(p.u + uoff[i] + kb * kKB);
        asm volatile("" ::: "memory");
    };
    fetch(s0, 0);
    fetch(s1, min(1, nkb - 1));
    fetch(s2, min(2, nkb - 1));
    fetch(s3, min(3, nkb - 1));

    f32x16 acc[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) acc[i] = f32x16{};

    // one input block: its weight and u pieces into LDS buffer kb & 1 (last read two blocks
    // ago, before the previous barrier), barrier, products, then the slot is refilled with
    // block kb + kDepth (clamped: a repeat read of the last block hits L2 and is never used)
    auto step = [&](Slot &sl, int kb) {
        const int buf = kb & 1;
#pragma unroll
        for (int i = 0; i < WQ; ++i) {
            const int q = tid + 256 * i;
            *reinterpret_cast<i32x4v *>(&sW[buf][q / 8][(q % 8) * 8]) = sl.w[i];
        }
#pragma unroll
        for (int i = 0; i < UQ; ++i) {
            const int q = tid + 256 * i;
            *reinterpret_cast<i32x4v *>(&sU[buf][q / 8][(q % 8) * 8]) = sl.u[i];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8 bw = *reinterpret_cast<const bf16x8 *>(&sW[buf][wave * 32 + l32][32 * hf + 8 * j]);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&sU[buf][32 * i + l32][32 * hf + 8 * j]);
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bw, acc[i], 0, 0, 0);
            }
        }
        fetch(sl, min(kb + kDepth, nkb - 1));
    };
    for (int kq = 0; kq < nkb; kq += kDepth) {
        // the guards are uniform over the workgroup
        step(s0, kq);
        if (EXACT || kq + 1 < nkb) step(s1, kq + 1);
        if (EXACT || kq + 2 < nkb) step(s2, kq + 2);
        if (EXACT || kq + 3 < nkb) step(s3, kq + 3);
    }

    // lane: column n; register r of tile i holds row m0 + 32i + 8(r/4) + 4hf + r%4
    if (n >= p.cols[b]) return;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = m0 + 32 * i + 8 * (r / 4) + 4 * hf + (r % 4);
            if (t >= p.T) continue;
            if (p.S == 1)
                emit(p, b, t, n, acc[i][r]);
            else
                p.part[((size_t)split * p.T + t) * p.ncols + p.colbase[b] + n] = acc[i][r];
        }
    }
}

// out = sum over the S partials in order 0..S-1, then the epilogue of the element's block.
__global__ __launch_bounds__(256) void project_reduce(const ProjParams p) {
    const int64_t total = (int64_t)p.T * p.ncols;
    for (int64_t e = blockIdx.x * (int64_t)256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int t = (int)(e / p.ncols), c = (int)(e % p.ncols);
        float v = 0.f;
        for (int s = 0; s < p.S; ++s) v += p.part[(size_t)s * total + e];
        const int b = c >= p.colbase[3] ? 3 : c >= p.colbase[2] ? 2 : c >= p.colbase[1] ? 1 : 0;
        emit(p, b, t, c - p.colbase[b], v);
    }
}

int block_m(int T) { return T > 128 ? 128 : T > 32 ? 64 : 32; }

struct Plan {
    int BM, S, nkb, ntiles, ncols;
    int cols[4], colbase[4], tile0[5];
};

Plan plan(const mil_ssm_dims &dm, int T, int d) {
    Plan pl;
    pl.cols[0] = dm.nheads * dm.headdim;
    pl.cols[1] = pl.cols[2] = dm.ngroups * dm.dstate;
    pl.cols[3] = dm.nheads;
    pl.ncols = 0;
    pl.tile0[0] = 0;
    for (int b = 0; b < 4; ++b) {
        pl.colbase[b] = pl.ncols;
        pl.ncols += pl.cols[b];
        pl.tile0[b + 1] = pl.tile0[b] + (pl.cols[b] + kBN - 1) / kBN;
    }
    pl.ntiles = pl.tile0[4];
    pl.BM = block_m(T);
    const int64_t base = (int64_t)((T + pl.BM - 1) / pl.BM) * pl.ntiles;
    const int blocks = d / kKB;
    pl.S = 1;
    while (pl.S < 16 && base * pl.S < kWgTarget && blocks % (2 * pl.S) == 0 && blocks / (2 * pl.S) >= kDepth)
        pl.S *= 2;
    pl.nkb = blocks / pl.S;
    return pl;
}

}  // namespace

bool project_supported(const mil_ssm_dims &dm, int T, int d) {
    if (T < 1 || d < kKB || d % kKB != 0) return false;
    const int64_t rows[4] = {(int64_t)dm.nheads * dm.headdim, (int64_t)dm.ngroups * dm.dstate,
                             (int64_t)dm.ngroups * dm.dstate, dm.nheads};
    for (int64_t r : rows)
        if (r * d * 2 > 0x7fffffffLL) return false;  // 32-bit buffer offsets
    return true;
}

int64_t project_workspace_bytes(const mil_ssm_dims &dm, int T, int d) {
    const Plan pl = plan(dm, T, d);
    if (pl.S == 1) return 0;
    return ((int64_t)pl.S * T * pl.ncols * 4 + 255) / 256 * 256;
}

hipError_t launch_project(const mil_ssm_dims &dm, int T, int d, const void *u, const void *const w[4],
                          const float *bias, bool out_bf16, void *const out[4], void *ws, hipStream_t s) {
    const Plan pl = plan(dm, T, d);
    ProjParams p;
    p.u = static_cast<const uint16_t *>(u);
    for (int b = 0; b < 4; ++b) {
        p.w[b] = static_cast<const uint16_t *>(w[b]);
        p.out[b] = out[b];
        p.cols[b] = pl.cols[b];
        p.colbase[b] = pl.colbase[b];
    }
    for (int b = 0; b < 5; ++b) p.tile0[b] = pl.tile0[b];
    p.bias = bias;
    p.part = static_cast<float *>(ws);
    p.T = T;
    p.d = d;
    p.S = pl.S;
    p.nkb = pl.nkb;
    p.ncols = pl.ncols;
    p.out_bf16 = out_bf16 ? 1 : 0;
    const int grid = ((T + pl.BM - 1) / pl.BM) * pl.ntiles * pl.S;
    const bool exact = pl.nkb % kDepth == 0;
#define MIL_PROJ_CASE(bm)                                                                   \
    if (pl.BM == bm) {                                                                      \
        if (exact)                                                                          \
            hipLaunchKernelGGL((project_gemm<bm, true>), dim3(grid), dim3(256), 0, s, p);  \
        else                                                                                \
            hipLaunchKernelGGL((project_gemm<bm, false>), dim3(grid), dim3(256), 0, s, p); \
    }
    MIL_PROJ_CASE(128)
    MIL_PROJ_CASE(64)
    MIL_PROJ_CASE(32)
#undef MIL_PROJ_CASE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || pl.S == 1) return e;
    const int64_t total = (int64_t)T * pl.ncols;
    const int rg = (int)std::min<int64_t>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(project_reduce, dim3(rg), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace mil
