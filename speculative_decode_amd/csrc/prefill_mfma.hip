// Matrix-core (MFMA) form of the chunked prefill for bf16 token inputs.
//
// Same three phases as the vector-ALU form (chunk states, a short sequential pass
// across chunks, chunk outputs), which is the layer of "The Mamba in the Llama"
// (skycaiji.com summary, method paragraph: discretised linear RNN, expanded state,
// hardware-aware decomposition) regrouped by chunk.  Within a chunk the dense parts
// run on v_mfma_f32_32x32x16_bf16 (bf16 operands, fp32 accumulation):
//   phase 1   S^T[p][n]  = sum_s X[s][p] * (w_s B[s][n]),       w_s = dt_s decay(s, end)
//   phase 3   Z = B_J C_I^T  (= G^T tile, G = C B^T),  M = mask(Z) * decay * dt,
//             Y_I += M X_J  (+ D on the diagonal),  Y_I = exp(a_t) C_I h_in + ...
// The token inputs are exact in bf16.  Operands derived in fp32 (w_s B, the masked M,
// the carried state h_in) are split into hi + lo bf16 parts and both products are
// accumulated, which keeps them to about 16 mantissa bits.
//
// Register layouts of the 32x32x16 instruction (lane l, half hf = l / 32):
//   A: row l%32, k-slots (hf, v);  B: column l%32, k-slots (hf, v);  A and B pair by (hf, v).
//   D: column l%32, register r holds row 8(r/4) + 4hf + r%4.
// Phase 3 computes Z with B_J as A and C_I as B, so each lane's D registers hold one
// output row t (= its column) and 16 source tokens s: exactly an A operand for M X
// once the k-slot (hf, v) <-> s correspondence is applied to how X is read from LDS.
#include <algorithm>

#include "ssm_internal.h"

namespace mil {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4v __attribute__((ext_vector_type(4)));  // 16 bytes that arrays keep in registers

constexpr int kT = 32;  // MFMA tile edge and decay tile (tokens)

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
__device__ __forceinline__ float bf2f(bf16 v) { return static_cast<float>(v); }
// Column i (0..7) of four rows of 8 bf16 each, as 4 consecutive bf16 (one row of the
// transpose): byte selects on register words, so nothing goes through memory.
__device__ __forceinline__ uint32_t word_of(const uint4 &v, int k) {
    return k == 0 ? v.x : (k == 1 ? v.y : (k == 2 ? v.z : v.w));
}
__device__ __forceinline__ uint2 column4(const uint4 &v0, const uint4 &v1, const uint4 &v2, const uint4 &v3, int i) {
    const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;  // high or low halves of each word
    uint2 w;
    w.x = __builtin_amdgcn_perm(word_of(v1, i >> 1), word_of(v0, i >> 1), sel);
    w.y = __builtin_amdgcn_perm(word_of(v3, i >> 1), word_of(v2, i >> 1), sel);
    return w;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// hi = nearest bf16 of each of a and b, lo = nearest bf16 of each remainder, each part as
// one packed word (a in the low half): one packed conversion per word, the remainders
// taken from the packed hi word's halves.
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
    const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xffff0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a - ha, b - hb}, bf16x2));
}
// A lane's 16 accumulator values (register r) split into the hi and lo A operands of two
// k-steps: register r goes to k-step r / 8, slot r % 8.
__device__ __forceinline__ void split16(const f32x16 &v, bf16x8 *ah, bf16x8 *al) {
    i32x4v h[2], l[2];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
        uint32_t hw, lw;
        split2(v[r], v[r + 1], hw, lw);
        h[r / 8][(r % 8) / 2] = (int)hw;
        l[r / 8][(r % 8) / 2] = (int)lw;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        ah[k] = __builtin_bit_cast(bf16x8, h[k]);
        al[k] = __builtin_bit_cast(bf16x8, l[k]);
    }
}

struct MParams {
    const uint16_t *x, *B, *C, *dt;  // bf16 bit patterns
    const float *A, *D;
    float *y;
    float *state;          // cache state of slot0
    int64_t head_stride;   // floats
    float *ws;             // [nseq][nch][H][P][N] fp32 chunk states, then h_in as hi/lo bf16
    float *ws_tot;         // [nseq][nch][H]
    int32_t *pos, *pending;
    int L, Q, nch, H, P, N, G;
    int slot0, nseq, batch, cont;
    int PS, nslab;         // phase 1: state rows p per workgroup, slabs per chunk-head
    // single-launch scan
    int32_t *scan;         // handoff words [batch][H][kScanSlabs][kScanRow]
    int t0;                // single launch: token index of this launch's first chunk
    int book;              // single launch: this launch sets pos / pending (the last launch of a prefill)
    int pos_add;           // single launch: the caller's continue flag (pos grows by L, every slot's pending is 0)
    int incl_every;        // single launch: chunks c > 0 with (c + 1) % incl_every == 0 publish their inclusive state
    int32_t *err;          // [batch] device error words
    float *chain;          // [nseq][H][P/PC][nch][N*PC + 16] published chunk states (register order), E_c
};

// Work-item order with consecutive items on one XCD: workgroups are dealt to the 8 XCDs
// round-robin, so item = xcd * (n/8) + k keeps the heads of one chunk (which share B and
// C rows) in one L2.
__device__ __forceinline__ int xcd_item(int n) {
    const int b = blockIdx.x;
    return (n % 8 == 0) ? (b % 8) * (n / 8) + b / 8 : b;
}

// Per-token decay factors of one chunk (32-token tiles; sums local to a tile or over
// whole-tile totals, so each exponent's rounding is relative to its own size).
//   R[t]    = sum_{tile start..t} dtA          (inclusive, within t's tile)
//   suf[s]  = sum_{s+1..tile end} dtA          (exclusive, within s's tile)
//   tot[i]  = sum over tile i
// One 32-lane half-wave per tile: a shuffle scan up for R, and a shuffle scan down over
// the shifted values for suf (a sum of later terms, not a difference).  dtA must be zero
// from len to the next multiple of 32.
__device__ void chunk_factors(const float *dtA, int len, float *R, float *suf, float *tot, int tid, int nt) {
    const int ntile = (len + kT - 1) / kT;
    for (int base = 0; base < ntile * kT; base += nt) {
        const int t = base + tid;
        const int l32 = tid & 31;
        const bool in = t < ntile * kT;
        float r = in ? dtA[t] : 0.f;
        float u = (in && l32 < 31) ? dtA[t + 1] : 0.f;
#pragma unroll
        for (int d = 1; d < 32; d <<= 1) {
            const float ru = __shfl_up(r, d, 32);
            const float ud = __shfl_down(u, d, 32);
            if (l32 >= d) r += ru;
            if (l32 + d < 32) u += ud;
        }
        if (in) {
            R[t] = r;
            suf[t] = u;
            if (l32 == 31) tot[t / kT] = r;
        }
    }
    __syncthreads();
}

// ------------------------------------------------------------------------- phase 1
// One workgroup (4 waves) per (seq, chunk, head, p-slab): S^T[p][n] for p in the slab.
// Tokens go through LDS in blocks of 64: X^T (bf16) and (w B)^T split hi/lo.
constexpr int kSB = 64;       // token block
constexpr int kSBS = kSB + 8; // padded LDS row (elements), 16-B aligned rows

template <int TPW>
__global__ __launch_bounds__(256) void chunk_state_mfma(const MParams p) {
    extern __shared__ __align__(16) char lds[];
    const int PS = p.PS, N = p.N, H = p.H, P = p.P, G = p.G;
    const int nitems = p.nseq * p.nch * H * p.nslab;
    const int item = xcd_item(nitems);
    const int slab = item % p.nslab;
    const int h = (item / p.nslab) % H;
    const int c = (item / p.nslab / H) % p.nch;
    const int seq = item / p.nslab / H / p.nch;
    const int g = h / (H / G);
    const int c0 = c * p.Q, len = min(p.Q, p.L - c0), p0 = slab * PS;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5, l32 = lane & 31;

    bf16 *sXT = reinterpret_cast<bf16 *>(lds);    // [PS][kSBS]
    bf16 *sWh = sXT + PS * kSBS;                   // [N][kSBS]
    bf16 *sWl = sWh + N * kSBS;                    // [N][kSBS]
    float *sDtA = reinterpret_cast<float *>(sWl + N * kSBS);  // [256]
    float *sW = sDtA + 256;                        // [256]
    float *sR = sW + 256, *sSuf = sR + 256, *sTot = sSuf + 256;  // [256],[256],[8]

    const size_t tok0 = (size_t)seq * p.L + c0;
    const float Ah = p.A[h];
    for (int s = tid; s < 256; s += 256) sDtA[s] = s < len ? bf2f(p.dt[(tok0 + s) * H + h]) * Ah : 0.f;
    __syncthreads();
    chunk_factors(sDtA, len, sR, sSuf, sTot, tid, 256);
    const int ntile = (len + kT - 1) / kT;
    for (int s = tid; s < len; s += 256) {
        // decay from s to the chunk end: rest of s's tile, then whole later tiles
        float e = sSuf[s];
        for (int q = s / kT + 1; q < ntile; ++q) e += sTot[q];
        sW[s] = __expf(e) * bf2f(p.dt[(tok0 + s) * H + h]);
    }
    if (tid == 0 && slab == 0) {
        float tt = 0.f;
        for (int q = 0; q < ntile; ++q) tt += sTot[q];
        p.ws_tot[((size_t)seq * p.nch + c) * H + h] = tt;
    }

    // output tiles of this wave: (pt, nt) pairs, TPW of them
    const int ntiles = N / kT;
    f32x16 acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) acc[i] = f32x16{};

    // token blocks of 64 go through LDS; the global loads of block b+1 are issued before
    // the matrix products of block b.  Items (4 tokens x 8 columns) per block: 2*PS of X and
    // 2*N of B, at most 512 each, so two per thread.
    const int xitems = (kSB / 4) * (PS / 8), witems = (kSB / 4) * (N / 8);
    uint4 vx[2][4], vw[2][4];
    float wv[2][4];
    auto fetch = [&](int sb) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int it = tid + j * 256;
            const int pg = it / (kSB / 4), sq = it % (kSB / 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = sb + sq * 4 + r;
                vx[j][r] = (it < xitems && s < len)
                               ? *reinterpret_cast<const uint4 *>(p.x + ((tok0 + s) * H + h) * P + p0 + pg * 8)
                               : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int it = tid + j * 256;
            const int ng = it / (kSB / 4), sq = it % (kSB / 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = sb + sq * 4 + r;
                const bool ok = it < witems && s < len;
                wv[j][r] = ok ? sW[s] : 0.f;
                vw[j][r] = ok ? *reinterpret_cast<const uint4 *>(p.B + ((tok0 + s) * G + g) * N + ng * 8)
                              : make_uint4(0, 0, 0, 0);
            }
        }
    };
    __syncthreads();  // sW visible
    fetch(0);
    for (int sb = 0; sb < len; sb += kSB) {
        __syncthreads();  // the previous block's products are done with LDS
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int it = tid + j * 256;
            if (it < xitems) {
                const int pg = it / (kSB / 4), sq = it % (kSB / 4);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    *reinterpret_cast<uint2 *>(sXT + (pg * 8 + i) * kSBS + sq * 4) =
                        column4(vx[j][0], vx[j][1], vx[j][2], vx[j][3], i);
            }
            if (it < witems) {
                const int ng = it / (kSB / 4), sq = it % (kSB / 4);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t wd = word_of(vw[j][r], i >> 1);
                        v[r] = wv[j][r] * __uint_as_float((i & 1) ? (wd & 0xffff0000u) : (wd << 16));
                    }
                    uint2 hi, lo;
                    split2(v[0], v[1], hi.x, lo.x);
                    split2(v[2], v[3], hi.y, lo.y);
                    *reinterpret_cast<uint2 *>(sWh + (ng * 8 + i) * kSBS + sq * 4) = hi;
                    *reinterpret_cast<uint2 *>(sWl + (ng * 8 + i) * kSBS + sq * 4) = lo;
                }
            }
        }
        if (sb + kSB < len) fetch(sb + kSB);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int tile = wave * TPW + i;
            const int pt = tile / ntiles, nt = tile % ntiles;
#pragma unroll
            for (int ks = 0; ks < kSB / 16; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sXT + (pt * kT + l32) * kSBS + ks * 16 + hf * 8);
                const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(sWh + (nt * kT + l32) * kSBS + ks * 16 + hf * 8);
                const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(sWl + (nt * kT + l32) * kSBS + ks * 16 + hf * 8);
                acc[i] = mfma(a, bh, acc[i]);
                acc[i] = mfma(a, bl, acc[i]);
            }
        }
    }
    // S^T tile -> workspace [p][n] (lane: column n, rows p)
    float *out = p.ws + (((size_t)seq * p.nch + c) * H + h) * (size_t)P * N;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int tile = wave * TPW + i;
        const int pt = tile / ntiles, nt = tile % ntiles;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int pr = p0 + pt * kT + 8 * (r / 4) + 4 * hf + (r % 4);
            out[(size_t)pr * N + nt * kT + l32] = acc[i][r];
        }
    }
}

// ------------------------------------------------------------------------- phase 2
// Sequential pass across chunks in the [p][n] layout, 8 consecutive n per thread.
// Each chunk's 32 bytes of fp32 S_c are replaced in place by the state entering that
// chunk as 8 hi bf16 followed by 8 lo bf16.  The final state goes to the cache in its
// [n][p] layout through an LDS transpose (and the starting state comes in the same way).
// grid (P/32 * N/64, H, nseq), 256 threads: 32 p x 8 groups of 8 n.
__global__ __launch_bounds__(256) void state_pass_pn(const MParams p) {
    __shared__ float sT[64][33];
    const int h = blockIdx.y, seq = blockIdx.z;
    const int N = p.N, P = p.P;
    const int ntl = N / 64;
    const int ptile = blockIdx.x / ntl, ntile = blockIdx.x % ntl;
    const int tid = threadIdx.x;
    const int pl = tid >> 3, ng = tid & 7;
    const int pcol = ptile * 32 + pl, n0 = ntile * 64 + ng * 8;
    if (blockIdx.x == 0 && h == 0 && seq == 0) {
        for (int i = tid; i < p.batch; i += blockDim.x) {
            const bool mine = i >= p.slot0 && i < p.slot0 + p.nseq;
            if (mine) p.pos[i] = p.cont ? p.pos[i] + p.L : p.L;
            if (mine || p.cont) p.pending[i] = 0;
        }
    }
    float *cache = p.state + (size_t)(seq * p.H + h) * p.head_stride;
    float hv[8];
    if (p.cont) {
        // coalesced rows n of the cache -> LDS -> this thread's 8 n of column pcol
        for (int i = tid; i < 64 * 32; i += 256) {
            const int n = i / 32, q = i % 32;
            sT[n][q] = cache[(size_t)(ntile * 64 + n) * P + ptile * 32 + q];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = sT[ng * 8 + i][pl];
        __syncthreads();
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = 0.f;
    }
    const size_t NP = (size_t)P * N;
    constexpr int U = 4;  // chunks whose states are loaded before any is rewritten
    for (int cb = 0; cb < p.nch; cb += U) {
        float4 s0[U], s1[U];
        float tt[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (cb + u < p.nch) {
                const size_t ch = ((size_t)seq * p.nch + cb + u) * p.H + h;
                const float *slot = p.ws + ch * NP + (size_t)pcol * N + n0;
                s0[u] = *reinterpret_cast<const float4 *>(slot);
                s1[u] = *reinterpret_cast<const float4 *>(slot + 4);
                tt[u] = p.ws_tot[ch];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (cb + u < p.nch) {
                const size_t ch = ((size_t)seq * p.nch + cb + u) * p.H + h;
                float *slot = p.ws + ch * NP + (size_t)pcol * N + n0;
                uint4 hi, lo;
                split2(hv[0], hv[1], hi.x, lo.x);
                split2(hv[2], hv[3], hi.y, lo.y);
                split2(hv[4], hv[5], hi.z, lo.z);
                split2(hv[6], hv[7], hi.w, lo.w);
                *reinterpret_cast<uint4 *>(slot) = hi;
                *reinterpret_cast<uint4 *>(slot + 4) = lo;
                const float e = __expf(tt[u]);
                const float sc[8] = {s0[u].x, s0[u].y, s0[u].z, s0[u].w, s1[u].x, s1[u].y, s1[u].z, s1[u].w};
#pragma unroll
                for (int i = 0; i < 8; ++i) hv[i] = __builtin_fmaf(e, hv[i], sc[i]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) sT[ng * 8 + i][pl] = hv[i];
    __syncthreads();
    for (int i = tid; i < 64 * 32; i += 256) {
        const int n = i / 32, q = i % 32;
        cache[(size_t)(ntile * 64 + n) * P + ptile * 32 + q] = sT[n][q];
    }
}

// Y += M X for one 32-column tile J: the A operands (hi, lo) hold M[t][s] with k-slot
// (hf, v) <-> s = 32J + 16ks + 8(v/4) + 4hf + v%4, so the B operand reads X^T row p at
// the same s: two groups of four consecutive tokens.  xr points at X^T[l32][32J + 4hf].
// One 32-token tile of B as the A operand of Z = B_J C_I^T: row l%32 of the tile, the NK
// k-steps of 16 state columns (lane half hf takes 8 of each).  Read all at once so that
// the reads' LDS latencies overlap instead of each waiting before its product.
template <int NK>
__device__ __forceinline__ void load_btile(bf16x8 *bq, const bf16 *sB, int J, int l32, int hf, int BS) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
        bq[kk] = *reinterpret_cast<const bf16x8 *>(sB + (J * kT + l32) * BS + kk * 16 + hf * 8);
}

// The B operands of Y += M X for one 32-token tile J (see accumulate_mx), read ahead.
template <int PT>
__device__ __forceinline__ void load_x(bf16x8 (*xv)[2], const bf16 *xr, int XS) {
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
        const bf16 *row = xr + pt * kT * XS;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x4 x0 = *reinterpret_cast<const bf16x4 *>(row + ks * 16);
            const bf16x4 x1 = *reinterpret_cast<const bf16x4 *>(row + ks * 16 + 8);
            xv[pt][ks] = bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        }
    }
}
template <int PT>
__device__ __forceinline__ void mx_products(f32x16 *acc, const bf16x8 *ah, const bf16x8 *al, bf16x8 (*xv)[2]) {
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            acc[pt] = mfma(ah[ks], xv[pt][ks], acc[pt]);
            acc[pt] = mfma(al[ks], xv[pt][ks], acc[pt]);
        }
}

template <int PT>
__device__ __forceinline__ void accumulate_mx(f32x16 *acc, const bf16x8 *ah, const bf16x8 *al, const bf16 *xr,
                                              int XS) {
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
        const bf16 *row = xr + pt * kT * XS;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x4 x0 = *reinterpret_cast<const bf16x4 *>(row + ks * 16);
            const bf16x4 x1 = *reinterpret_cast<const bf16x4 *>(row + ks * 16 + 8);
            const bf16x8 xv = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            acc[pt] = mfma(ah[ks], xv, acc[pt]);
            acc[pt] = mfma(al[ks], xv, acc[pt]);
        }
    }
}

// ------------------------------------------------------------------------- phase 3
// One workgroup per (seq, chunk, head, column slab of PC of the P columns); Q/32 waves,
// each owning one 32-row tile.  Waves w and w + 4 share a SIMD, so tiles are dealt as
// I = w (w < nw/2) and I = nw-1-(w-nw/2): a SIMD then holds tiles I and nw-1-I, whose
// causal parts (I+1 and nw-I column tiles) add up to the same work on every SIMD, and
// its two waves hide each other's latency.  Splitting the columns over P/PC workgroups
// (which recompute the same C B^T tiles) spreads short prompts over more compute units;
// the slabs of one (chunk, head) are consecutive items, so they share B and C in one L2.
template <int N, int PC>
__global__ __launch_bounds__(512) void chunk_out_mfma(const MParams p) {
    extern __shared__ __align__(16) char lds[];
    const int H = p.H, G = p.G, Q = p.Q, P = p.P;
    const int nps = P / PC;
    const int nitems = p.nseq * p.nch * H * nps;
    const int item = xcd_item(nitems);
    const int pc0 = (item % nps) * PC, hc = item / nps;
    const int h = hc % H, c = (hc / H) % p.nch, seq = hc / H / p.nch;
    const int g = h / (H / G);
    const int c0 = c * Q, len = min(Q, p.L - c0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5, l32 = lane & 31;
    const int NT = blockDim.x;
    const int BS = N + 8, XS = Q + 8;  // padded LDS rows (elements)
    constexpr int PT = PC / kT, NK = N / 16;
    constexpr int HS = N * 2 + 8;      // padded LDS row of the carried state (bf16 elements)

    // LDS: [B rows | X^T] during the intra-chunk products; the carried state (hi/lo)
    // reuses the same bytes afterwards; then the per-token factors.
    bf16 *sB = reinterpret_cast<bf16 *>(lds);      // [Q][BS]   B rows of the chunk
    bf16 *sXT = sB + Q * BS;                        // [PC][XS]  X^T of the chunk, this slab
    bf16 *sH = reinterpret_cast<bf16 *>(lds);       // [PC][HS]  carried state, later
    const size_t big = max((size_t)Q * BS + (size_t)PC * XS, (size_t)PC * HS) * 2;
    float *sDt = reinterpret_cast<float *>(lds + big);  // [Q]
    float *sDtA = sDt + Q, *sR = sDtA + Q, *sSuf = sR + Q, *sColf = sSuf + Q, *sEin = sColf + Q;
    float *sTot = sEin + Q;                         // [8]
    float *sMid = sTot + 8;                         // [8][8]

    const size_t tok0 = (size_t)seq * p.L + c0;
    const float Ah = p.A[h], Dh = p.D[h];
    const int nt = Q / kT;
    const int I = wave < nt / 2 ? wave : nt - 1 - (wave - nt / 2);  // this wave's 32-row tile
    const bool active = I * kT < len;
    const int t = I * kT + l32;  // this lane's output row as an A/B operand index

    // the carried state of this chunk ([p][n] groups of 8 hi + 8 lo bf16)
    const bool has_hin = p.cont || c > 0;
    const uint4 *hin = reinterpret_cast<const uint4 *>(p.ws + (((size_t)seq * p.nch + c) * H + h) * (size_t)P * N +
                                                       (size_t)pc0 * N);
    constexpr int HV = PC * N * 4 / 16;  // 16-byte pieces of this slab's rows
    constexpr int HPT = (HV + 511) / 512;
    constexpr bool kPrefetch = HPT <= 8;  // larger states are read at the LDS write instead
    // the light waves' registers cover the whole state only when NT * HPT pieces do (512 threads)
    const bool pre = kPrefetch && NT * HPT >= HV;

    // ---- staging.  Every load is unconditional (rows past the chunk end clamped, their
    // values zeroed after), so no branch makes the compiler wait for one load before the
    // next.  Issue order: dt, B and X, which the LDS writes below wait for, then the C rows
    // of this wave's tile (the B operand of Z and the A operand of C h_in), which are needed
    // only after the staging. ----
    const float dv0 = bf2f(p.dt[(tok0 + min(tid, len - 1)) * H + h]);  // NT = 2Q >= Q
    constexpr int BI = N / 16;  // B pieces per thread: Q*N/8 pieces over NT = 2Q threads
    uint4 vb[BI];
#pragma unroll
    for (int j = 0; j < BI; ++j) {
        const int it = tid + j * NT;
        const int sr = it / (N / 8), ng = it % (N / 8);
        vb[j] = *reinterpret_cast<const uint4 *>(p.B + ((tok0 + min(sr, len - 1)) * G + g) * N + ng * 8);
    }
    constexpr int XI = (PC + 63) / 64;  // X items (4 tokens x 8 columns) per thread
    uint4 vx[XI][4];
#pragma unroll
    for (int j = 0; j < XI; ++j) {
        const int it = tid + j * NT;
        const int pg = it / (Q / 4), sq = it % (Q / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int sr = sq * 4 + r;
            vx[j][r] = *reinterpret_cast<const uint4 *>(p.x + ((tok0 + min(sr, len - 1)) * H + h) * P + pc0 +
                                                         min(pg, PC / 8 - 1) * 8);
        }
    }
    asm volatile("" ::: "memory");  // the C rows and the carried state after the others
    bf16x8 cf[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
        cf[kk] = *reinterpret_cast<const bf16x8 *>(p.C + ((tok0 + min(t, len - 1)) * G + g) * N + kk * 16 + hf * 8);
    asm volatile("" ::: "memory");
    const float dv = tid < len ? dv0 : 0.f;
#pragma unroll
    for (int j = 0; j < BI; ++j) {
        const int sr = (tid + j * NT) / (N / 8);
        if (sr >= len) vb[j] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < XI; ++j) {
        const int sq = (tid + j * NT) % (Q / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (sq * 4 + r >= len) vx[j][r] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
        if (!(active && t < len)) cf[kk] = bf16x8{};
    if (tid < Q) {
        sDt[tid] = dv;
        sDtA[tid] = dv * Ah;  // zero past the chunk end
    }
#pragma unroll
    for (int j = 0; j < BI; ++j) {
        const int it = tid + j * NT;
        const int sr = it / (N / 8), ng = it % (N / 8);
        *reinterpret_cast<uint4 *>(sB + sr * BS + ng * 8) = vb[j];
    }
    // X^T (zero past the chunk end: those columns meet zero weights, but 0 * NaN is not 0);
    // token quads fastest, so neighbouring threads write neighbouring 8 bytes of a row
#pragma unroll
    for (int j = 0; j < XI; ++j) {
        const int it = tid + j * NT;
        if (it >= (Q / 4) * (PC / 8)) break;
        const int pg = it / (Q / 4), sq = it % (Q / 4);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<uint2 *>(sXT + (pg * 8 + i) * XS + sq * 4) =
                column4(vx[j][0], vx[j][1], vx[j][2], vx[j][3], i);
    }
    __syncthreads();
    chunk_factors(sDtA, len, sR, sSuf, sTot, tid, NT);
    const int ntile = (len + kT - 1) / kT;
    // the tile totals in registers (two LDS reads), summed in ascending tile order as a
    // sequential loop would; totals past the last tile are never selected
    const float4 tq0 = *reinterpret_cast<const float4 *>(sTot), tq1 = *reinterpret_cast<const float4 *>(sTot + 4);
    const float tv[8] = {tq0.x, tq0.y, tq0.z, tq0.w, tq1.x, tq1.y, tq1.z, tq1.w};
    for (int s = tid; s < len; s += NT) {
        sColf[s] = sDt[s] * __expf(sSuf[s]);  // dt_s * decay(s, end of s's tile)
        const int ti = s / kT;
        float m = sR[s];
#pragma unroll
        for (int q = 0; q < 8; ++q) m = q < ti ? m + tv[q] : m;
        sEin[s] = __expf(m);                  // decay from the chunk start through s
    }
    if (tid < 64) {
        const int Ii = tid / 8, J = tid % 8;
        float m = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) m = (q > J && q < Ii) ? m + tv[q] : m;
        sMid[tid] = (J < Ii && Ii < ntile) ? __expf(m) : 0.f;  // whole tiles strictly between J and Ii
    }
    __syncthreads();

    f32x16 acc[PT];
#pragma unroll
    for (int i = 0; i < PT; ++i) acc[i] = f32x16{};
    if (active) {
        // rows t >= len are computed but never stored (MFMA rows do not mix)
        const float et = __expf(sR[min(t, Q - 1)]);
        // off-diagonal tiles J < I: every s < t, so no mask; decay = colf(s) * mid(I,J) * e^{R_t}
        // software pipeline over the tiles J = 0..I: the matrix cores form tile J + 1's
        // Z (its B rows read from LDS a tile earlier still) while the vector units mask
        // tile J's, so neither waits for the other within the wave
        bf16x8 bq[NK];
        load_btile<NK>(bq, sB, 0, l32, hf, BS);
        f32x16 zn = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) zn = mfma(bq[kk], cf[kk], zn);
        load_btile<NK>(bq, sB, min(1, I), l32, hf, BS);
        for (int J = 0; J < I; ++J) {
            const f32x16 z = zn;
            zn = f32x16{};
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) zn = mfma(bq[kk], cf[kk], zn);
            load_btile<NK>(bq, sB, min(J + 2, I), l32, hf, BS);
            const float rowf = sMid[I * 8 + J] * et;
            f32x16 mv;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // registers 4q..4q+3 hold s = 32J + 8q + 4hf + (0..3)
                const float4 cf4 = *reinterpret_cast<const float4 *>(sColf + J * kT + 8 * q + 4 * hf);
                const float cv[4] = {cf4.x, cf4.y, cf4.z, cf4.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) mv[4 * q + u] = z[4 * q + u] * cv[u] * rowf;
            }
            bf16x8 ah[2], al[2];
            split16(mv, ah, al);
            accumulate_mx<PT>(acc, ah, al, sXT + l32 * XS + J * kT + 4 * hf, XS);
        }
        // diagonal tile J = I: causal mask, decay exp(R_t - R_s), dt_s, and D on s = t
        {
            const int J = I;
            const f32x16 z = zn;
            const float Rt = sR[min(t, Q - 1)];
            f32x16 mv;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 r4 = *reinterpret_cast<const float4 *>(sR + J * kT + 8 * q + 4 * hf);
                const float4 d4 = *reinterpret_cast<const float4 *>(sDt + J * kT + 8 * q + 4 * hf);
                const float rv[4] = {r4.x, r4.y, r4.z, r4.w}, dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int r = 4 * q + u;
                    const int sl = 8 * q + 4 * hf + u;  // s - 32J
                    float m = z[r] * dv[u] * __expf(Rt - rv[u]);
                    m = sl < l32 ? m : (sl == l32 ? m + Dh : 0.f);
                    mv[r] = m;
                }
            }
            bf16x8 ah[2], al[2];
            split16(mv, ah, al);
            accumulate_mx<PT>(acc, ah, al, sXT + l32 * XS + J * kT + 4 * hf, XS);
        }
    }
    // the light waves (the short causal rows, done first) fetch the carried state while
    // the others finish their rows, and park it in LDS once every wave is done with B and X^T
    constexpr int HPL = 2 * HPT;  // pieces per light thread
    const bool lightw = wave < nt / 2;
    i32x4v hpre[kPrefetch ? HPL : 1];
    if (kPrefetch && has_hin && lightw) {
#pragma unroll
        for (int i = 0; i < HPL; ++i)
            hpre[i] = *reinterpret_cast<const i32x4v *>(hin + min(tid + i * (NT / 2), HV - 1));
    }
    if (has_hin) {
        __syncthreads();  // every wave is done with B and X^T
        // N/4 pieces of 16 B per row p of the state
        if (pre) {
            if (lightw) {
#pragma unroll
                for (int i = 0; i < (kPrefetch ? HPL : 1); ++i) {
                    const int v = tid + i * (NT / 2);
                    if (v < HV) *reinterpret_cast<i32x4v *>(sH + (v / (N / 4)) * HS + (v % (N / 4)) * 8) = hpre[i];
                }
            }
        } else {
            for (int v = tid; v < HV; v += NT)
                *reinterpret_cast<uint4 *>(sH + (v / (N / 4)) * HS + (v % (N / 4)) * 8) = hin[v];
        }
        __syncthreads();
        if (active) {
            // acc += diag(exp(a_t)) C_I h_in, h_in as hi + lo
            f32x16 acc2[PT];
#pragma unroll
            for (int i = 0; i < PT; ++i) acc2[i] = f32x16{};
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const bf16 *row = sH + (pt * kT + l32) * HS;
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    const bf16 *grp = row + (kk * 2 + hf) * 16;  // 8 hi then 8 lo
                    const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(grp);
                    const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(grp + 8);
                    acc2[pt] = mfma(cf[kk], bh, acc2[pt]);
                    acc2[pt] = mfma(cf[kk], bl, acc2[pt]);
                }
            }
            float ein[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) ein[r] = sEin[min(I * kT + 8 * (r / 4) + 4 * hf + (r % 4), Q - 1)];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[pt][r] = __builtin_fmaf(ein[r], acc2[pt][r], acc[pt][r]);
            }
        }
    }
    if (!active) return;
    // y rows of this tile (lane: column p, rows t = 32I + 8(r/4) + 4hf + r%4), stored
    // non-temporally: nothing here reads them again
    float *yb = p.y + ((tok0 + I * kT) * H + h) * P + pc0 + l32;
    const int ystride = H * P;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int tl = 8 * (r / 4) + 4 * hf + (r % 4);
        if (I * kT + tl < len) {
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) __builtin_nontemporal_store(acc[pt][r], yb + tl * ystride + pt * kT);
        }
    }
}

// ------------------------------------------------------------------ single launch
// All three phases in one launch for up to kScanChunks chunks (longer prompts take several
// launches, each continuing from the state the one before wrote), one workgroup per
// (chunk, sequence, head, column slab), chunk-major; the slab is 64 columns or fewer, or the
// whole 128-column head for long prompts at N = 128.  The workgroup stages its chunk's B, C,
// X and dt once, forms the chunk's own state contribution S_c = sum_s (w_s B_s) x_s^T on the
// matrix cores and publishes it with the chunk's total decay E_c (the aggregate; chunk 0
// publishes its outgoing state E_0 h0 + S_0 instead, the inclusive state, so that it alone
// reads h0), forms the intra-chunk outputs, then finds the state entering its chunk by
// decoupled look-back: the nearest earlier chunk that has published its inclusive state,
// folded forward through the aggregates after it (h <- E_i h + S_i, in chunk order).  Every
// inclusive state is that same fold back to chunk 0, so the result does not depend on where
// a look-back ends, and no workgroup waits on a chain of others.  The last chunk of each
// dispatch round publishes its inclusive state for the rounds after it; the last chunk of
// the prompt writes the final state.  Flags hold a per-call value that comes from the
// device: each (slot, head, slab) row keeps the epoch its last call raised its flags to;
// every workgroup of this call reads it at its start and raises its flag to epoch + 1, and
// the last chunk stores epoch + 1 as the row's epoch once its wait is over, which is after
// every workgroup of the row has read the old value (each of them publishes before the
// last chunk's wait can end).  So no flag left by an earlier call, a graph replay or a byte
// copy of the cache equals this call's value, and nothing needs resetting.
//
// Ordering: workgroups start in chunk-major order and every one publishes before it
// waits, so the flags a workgroup waits for are always raised; the wait is bounded in time
// anyway (MIL_DEVERR_SCAN is reported and the kernel carries on), so nothing can hang.
// Flags, counters and published states use agent-coherent accesses (see shared_load).
constexpr long long kScanWaitTicks = 50000000;  // 0.5 s of the 100 MHz real-time counter

// Everything that crosses workgroups (the published states and decays, the flags, the
// counter) is read and written with agent-coherent accesses (relaxed agent-scope atomics:
// loads and stores that bypass the non-coherent cache levels), and each wave waits for
// its stores to complete (s_waitcnt vmcnt(0)) before the workgroup raises a flag.  So no
// access needs the whole-cache write-back or invalidation that release / acquire
// orderings would add (measured: they made the handoffs several times slower).
__device__ __forceinline__ int scan_load(const int32_t *f) {
    return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void scan_store(int32_t *f, int v) {
    __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Epochs run 1..2^30-1 (then again from 1); a flag is (epoch << 2) | kind.
constexpr int kFlagAggregate = 1;  // the chunk's own state S_c and decay E_c are published
constexpr int kFlagInclusive = 2;  // the state after the chunk (the next chunk's h_in) is published
__device__ __forceinline__ int scan_next_epoch(int e) {
    const int n = (e + 1) & 0x3fffffff;
    return n == 0 ? 1 : n;
}
__device__ __forceinline__ int scan_flag(int epoch, int kind) {
    return static_cast<int>((static_cast<uint32_t>(epoch) << 2) | static_cast<uint32_t>(kind));
}
__device__ __forceinline__ float shared_load(const float *q) {
    return __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void shared_store(float *q, float v) {
    __hip_atomic_store(q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr size_t kLdsMax = 160 * 1024;
constexpr int kScanQ = 256;  // the single-launch kernel's chunk length

// LDS of the single-launch kernel: the staged B rows and X^T, seven per-token float
// arrays, the tile totals, the 8 x 8 tile factors and a counter; then the carried state's
// hi / lo rows for C h_in.
constexpr size_t scan_base_lds(int Q, int N, int PC) {
    return ((size_t)Q * (N + 8) + (size_t)PC * (Q + 8)) * 2 + 7 * (size_t)Q * 4 + 8 * 4 + 64 * 4 + 16;
}
constexpr size_t scan_xchg_bytes(int N, int PC) { return (size_t)PC * (N * 2 + 8) * 2; }
// Slabs too wide for a separate carried-state area stage it in X^T's area instead, once
// every wave is done with X (one more barrier).
constexpr bool scan_wide(int N, int PC) { return scan_base_lds(kScanQ, N, PC) + scan_xchg_bytes(N, PC) > kLdsMax; }

// The published chunk states are moved 16 bytes per lane with the same cache bypass
// (sc1) that the relaxed agent-scope atomics above use, four registers at a time.  A tile's
// floats are laid out [register / 4][lane][register % 4].
constexpr int kCoherentPolicy = 16;  // sc1
__device__ __forceinline__ void shared_store4(__amdgpu_buffer_rsrc_t r, int boff, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4v, v), r, boff, 0, kCoherentPolicy);
}
__device__ __forceinline__ f32x4 shared_load4(__amdgpu_buffer_rsrc_t r, int boff) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, boff, 0, kCoherentPolicy));
}

template <int N, int PC>
__global__ __launch_bounds__(512) void chunk_scan_mfma(const MParams p) {
    extern __shared__ __align__(16) char lds[];
    const int H = p.H, G = p.G, Q = p.Q, P = p.P;
    const int nps = P / PC;
    const int per_chunk = p.nseq * H * nps;
    const int c = blockIdx.x / per_chunk;
    const int u = blockIdx.x - c * per_chunk;
    // within a chunk, consecutive items (heads of one B/C group, and their slabs) on one XCD
    const int sub = (per_chunk % 8 == 0) ? (u % 8) * (per_chunk / 8) + u / 8 : u;
    const int slab = sub % nps, hs = sub / nps;
    const int h = hs % H, seq = hs / H;
    const int pc0 = slab * PC;
    const int g = h / (H / G);
    const int c0 = p.t0 + c * Q, len = min(Q, p.L - c0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5, l32 = lane & 31;
    const int NT = blockDim.x, NW = NT >> 6;
    const int BS = N + 8, XS = Q + 8;
    constexpr int PT = PC / kT, NK = N / 16, HS = N * 2 + 8;
    constexpr int NTL = N / kT;                        // state row tiles
    constexpr int STILES = NTL * PT;                   // state tiles of this slab

    bf16 *sB = reinterpret_cast<bf16 *>(lds);
    bf16 *sXT = sB + Q * BS;
    const size_t big = ((size_t)Q * BS + (size_t)PC * XS) * 2;
    float *sDt = reinterpret_cast<float *>(lds + big);
    float *sDtA = sDt + Q, *sR = sDtA + Q, *sSuf = sR + Q, *sColf = sSuf + Q, *sEin = sColf + Q;
    float *sWst = sEin + Q;                         // [Q] dt_s * decay(s, chunk end)
    float *sTot = sWst + Q;                         // [8]
    float *sMid = sTot + 8;                         // [8][8]

    const size_t tok0 = (size_t)seq * p.L + c0;
    const float Ah = p.A[h], Dh = p.D[h];
    const int nt = Q / kT;
    const int I = wave < nt / 2 ? wave : nt - 1 - (wave - nt / 2);
    const bool active = I * kT < len;
    const int t = I * kT + l32;
    // this launch's epoch: the row's epoch + 1 (1..2^30-1, so no flag of it is ever zero),
    // read before anything else (the last chunk overwrites the row's epoch only after
    // every workgroup of the row has published)
    int32_t *flags = p.scan + (((size_t)(p.slot0 + seq) * H + h) * kScanSlabs + slab) * kScanRow;
    const int epoch = scan_next_epoch(__builtin_amdgcn_readfirstlane(scan_load(flags + kScanEpoch)));

    // ---- staging: B, X and dt first (the chunk state needs them), then the C rows (only
    // the outputs need them), so that writing B and X to LDS waits for them alone ----
    // every staging load is unconditional (rows past the chunk end clamped, their values
    // zeroed after), so no branch makes the compiler wait for one load before the next
    const float dv0 = bf2f(p.dt[(tok0 + min(tid, len - 1)) * H + h]);
    constexpr int BI = N / 16;
    uint4 vb[BI];
#pragma unroll
    for (int j = 0; j < BI; ++j) {
        const int it = tid + j * NT;
        const int sr = it / (N / 8), ng = it % (N / 8);
        vb[j] = *reinterpret_cast<const uint4 *>(p.B + ((tok0 + min(sr, len - 1)) * G + g) * N + ng * 8);
    }
    // X items: 4 tokens x 8 columns, the column group fastest, so that one load
    // instruction of a wave reads whole rows of the slab (8 tokens x PC / 8 groups)
    constexpr int XI = (PC + 63) / 64;
    uint4 vx[XI][4];
#pragma unroll
    for (int j = 0; j < XI; ++j) {
        const int it = tid + j * NT;
        const int pg = it % (PC / 8), sq = it / (PC / 8);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int sr = sq * 4 + r;
            vx[j][r] = *reinterpret_cast<const uint4 *>(p.x + ((tok0 + min(sr, len - 1)) * H + h) * P + pc0 + pg * 8);
        }
    }
    asm volatile("" ::: "memory");  // keep the C loads after the others in issue order
    bf16x8 cf[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
        cf[kk] = *reinterpret_cast<const bf16x8 *>(p.C + ((tok0 + min(t, len - 1)) * G + g) * N + kk * 16 + hf * 8);
    asm volatile("" ::: "memory");
    const float dv = tid < len ? dv0 : 0.f;
#pragma unroll
    for (int j = 0; j < BI; ++j) {
        const int sr = (tid + j * NT) / (N / 8);
        if (sr >= len) vb[j] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < XI; ++j) {
        const int sq = (tid + j * NT) / (PC / 8);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (sq * 4 + r >= len) vx[j][r] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
        if (!(active && t < len)) cf[kk] = bf16x8{};
    if (tid < Q) {
        sDt[tid] = dv;
        sDtA[tid] = dv * Ah;
    }
    if (tid < 2) reinterpret_cast<int *>(sMid + 64)[tid] = 0;  // the light and owning waves' counters
#pragma unroll
    for (int j = 0; j < BI; ++j) {
        const int it = tid + j * NT;
        const int sr = it / (N / 8), ng = it % (N / 8);
        *reinterpret_cast<uint4 *>(sB + sr * BS + ng * 8) = vb[j];
    }
#pragma unroll
    for (int j = 0; j < XI; ++j) {
        const int it = tid + j * NT;
        if (it >= (Q / 4) * (PC / 8)) break;
        const int pg = it % (PC / 8), sq = it / (PC / 8);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<uint2 *>(sXT + (pg * 8 + i) * XS + sq * 4) =
                column4(vx[j][0], vx[j][1], vx[j][2], vx[j][3], i);
    }
    __syncthreads();
    chunk_factors(sDtA, len, sR, sSuf, sTot, tid, NT);
    const int ntile = (len + kT - 1) / kT;
    // the tile totals in registers (two LDS reads), summed in ascending tile order as a
    // sequential loop would; totals past the last tile are never selected
    const float4 tq0 = *reinterpret_cast<const float4 *>(sTot), tq1 = *reinterpret_cast<const float4 *>(sTot + 4);
    const float tv[8] = {tq0.x, tq0.y, tq0.z, tq0.w, tq1.x, tq1.y, tq1.z, tq1.w};
    for (int s = tid; s < Q; s += NT) {
        if (s < len) {
            const int ti = s / kT;
            sColf[s] = sDt[s] * __expf(sSuf[s]);
            float m = sR[s];
#pragma unroll
            for (int q = 0; q < 8; ++q) m = q < ti ? m + tv[q] : m;
            sEin[s] = __expf(m);
            float e = sSuf[s];  // decay from s to the chunk end: rest of s's tile, then later tiles
#pragma unroll
            for (int q = 0; q < 8; ++q) e = (q > ti && q < ntile) ? e + tv[q] : e;
            sWst[s] = __expf(e) * sDt[s];
        } else {
            sWst[s] = 0.f;  // tokens past the chunk end carry no weight
        }
    }
    if (tid < 64) {
        const int Ii = tid / 8, J = tid % 8;
        float m = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) m = (q > J && q < Ii) ? m + tv[q] : m;
        sMid[tid] = (J < Ii && Ii < ntile) ? __expf(m) : 0.f;
    }
    float ttot = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) ttot = q < ntile ? ttot + tv[q] : ttot;
    const float Ec = __expf(ttot);
    __syncthreads();

    const int slot = p.slot0 + seq;
    const size_t REC = 2 * (size_t)N * PC + 16;  // floats per chunk record: S_c tiles, E_c (16), inclusive tiles
    const size_t INC = (size_t)N * PC + 16;      // offset of the inclusive tiles in a record
    float *recs = p.chain + (((size_t)seq * H + h) * nps + slab) * (size_t)p.nch * REC;
    const __amdgpu_buffer_rsrc_t agr = __builtin_amdgcn_make_buffer_rsrc(recs, (short)0,
                                                                         (int)(p.nch * REC * 4), 0x00020000);
    float *cache = p.state + (size_t)(seq * H + h) * p.head_stride;
    const bool has_hin = p.cont || c > 0;
    const bool last = c == p.nch - 1;
    // the state after the chunk is published by the last chunk of each dispatch round only:
    // the chunks of one round look back at the same time, so none finds another's, and a
    // later round's look-back ends at the nearest one (any chunk's inclusive state is the
    // same fold, so where a look-back ends changes no bit; chunk 0 always publishes)
    const bool pub_inc = !last && (c + 1) % p.incl_every == 0;

    // ---- the chunk's own state S[n][p] (this slab): S = sum_s (w_s B_s) x_s^T with
    // A operand (w B)^T and B operand X^T (as staged).  The rows n of B^T come off the
    // matrix cores: the product D = B_blk E with E the identity holds, per lane, one
    // column n of a 32-token block over 16 tokens (registers r: tokens 8(r/4) + 4hf + r%4),
    // which is the A-operand layout once scaled by w_s and split hi + lo.  The state tiles
    // belong to the four light waves (w < 4: the waves with the short causal rows of the
    // intra-chunk products): tile (row tile snt, column tile pt) to wave snt + NTL (pt % LW),
    // as its tile i = pt / LW.  Each owner forms its tiles over all the chunk's tokens in
    // token order, so the other four waves go straight to their longer rows and no partial
    // tiles cross waves.  They publish the tiles and raise the chunk's flag. ----
    constexpr int LW = 4 / NTL;                   // light waves per row tile
    constexpr int TPWL = PT >= LW ? PT / LW : 1;  // tiles per owning wave
    const int snt = wave % NTL;                   // this wave's row tile (light waves)
    const int jpart = wave / NTL;                 // light waves: first owned column tile
    const bool light = wave < 4;
    const bool owner = light && jpart < PT;
    constexpr bool kWide = scan_wide(N, PC);
    static_assert(!kWide || 2 * N + 8 <= kScanQ + 8, "the carried state's rows fit in X^T's");
    // the carried state's rows: their own area, or X^T's once the intra-chunk rows are done
    bf16 *sH = kWide ? sXT : reinterpret_cast<bf16 *>(lds + scan_base_lds(Q, N, PC));
    f32x16 sacc[TPWL];
#pragma unroll
    for (int i = 0; i < TPWL; ++i) sacc[i] = f32x16{};
    // The wide form forms its tiles two at a time (the identity products are repeated per
    // pair) and publishes each pair at once, so that fewer registers are in flight.
    constexpr int CSG = kWide ? 2 : TPWL;  // tiles formed together
    if (owner) {
        bf16x8 eye[2];  // identity: slot v of k-step kk is 1 where 16 kk + 8 hf + v = l32
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int v = 0; v < 8; ++v) eye[kk][v] = static_cast<bf16>(16 * kk + 8 * hf + v == l32 ? 1.f : 0.f);
#pragma unroll
        for (int g0 = 0; g0 < TPWL; g0 += CSG) {
            f32x16 pacc[CSG];
#pragma unroll
            for (int ii = 0; ii < CSG; ++ii) pacc[ii] = f32x16{};
            // every block of the chunk, unrolled and without a branch; blocks past a short
            // chunk's end add exact zeros (their B rows, X columns and weights were zeroed
            // when staged).  Software pipeline: a block's LDS operands are read two blocks
            // ahead and its identity products issued one block ahead, so that neither the LDS
            // latency nor the products' latency is waited for where the values are used.
            constexpr int NB = kScanQ / kT;
            struct Ops {
                bf16x8 bo[2];        // B rows of the block (A operand of the identity products)
                float4 wq[4];        // w_s of the lane's 16 tokens
                bf16x8 xv[CSG][2];   // X operands of the block's products, owned column tiles
            };
            auto fetch = [&](int b, Ops &o) {
                const int s0 = b * kT;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    o.bo[kk] = *reinterpret_cast<const bf16x8 *>(sB + (s0 + l32) * BS + snt * kT + kk * 16 + 8 * hf);
#pragma unroll
                for (int q = 0; q < 4; ++q) o.wq[q] = *reinterpret_cast<const float4 *>(sWst + s0 + 8 * q + 4 * hf);
#pragma unroll
                for (int ii = 0; ii < CSG; ++ii)
                    load_x<1>(&o.xv[ii], sXT + ((jpart + LW * (g0 + ii)) * kT + l32) * XS + s0 + 4 * hf, XS);
            };
            auto ident = [&](const Ops &o) {
                f32x16 tb = f32x16{};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) tb = mfma(o.bo[kk], eye[kk], tb);
                return tb;
            };
            Ops o0, o1;
            fetch(0, o0);
            fetch(1, o1);
            f32x16 tb = ident(o0);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const f32x16 tbn = b + 1 < NB ? ident(o1) : f32x16{};
                f32x16 mv;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float wv[4] = {o0.wq[q].x, o0.wq[q].y, o0.wq[q].z, o0.wq[q].w};
#pragma unroll
                    for (int u2 = 0; u2 < 4; ++u2) mv[4 * q + u2] = tb[4 * q + u2] * wv[u2];
                }
                bf16x8 ah[2], al[2];
                split16(mv, ah, al);
                mx_products<CSG>(pacc, ah, al, o0.xv);
                o0 = o1;
                if (b + 2 < NB) fetch(b + 2, o1);
                __builtin_amdgcn_sched_barrier(0);
                tb = tbn;
            }
            if constexpr (kWide) {
                // publish the pair.  Chunks c > 0: S_c in the record's aggregate area (read
                // back when needed).  Chunk 0: its inclusive state E_0 h0 + S_0 (also when it is
                // the last: it is then the final state), and h0 in the aggregate area, which no
                // look-back reads for chunk 0 (the cache itself may hold the final state by the
                // time chunk 0 needs h0 again).
#pragma unroll
                for (int ii = 0; ii < CSG; ++ii) {
                    const int pt = jpart + LW * (g0 + ii);
                    const int tl = snt + NTL * pt;
                    f32x16 h0 = f32x16{};
                    if (c == 0 && p.cont) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int n = snt * kT + 8 * (r / 4) + 4 * hf + (r % 4);
                            h0[r] = cache[(size_t)n * P + pc0 + pt * kT + l32];
                        }
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        f32x4 v, s4;
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            s4[u] = pacc[ii][4 * q + u];
                            v[u] = __builtin_fmaf(Ec, h0[4 * q + u], pacc[ii][4 * q + u]);
                        }
                        if (c == 0) {
                            const f32x4 h4 = {h0[4 * q], h0[4 * q + 1], h0[4 * q + 2], h0[4 * q + 3]};
                            if (p.cont)
                                shared_store4(agr, (int)(((size_t)tl * 1024 + (q * 64 + lane) * 4) * 4), h4);
                            shared_store4(agr, (int)((INC + (size_t)tl * 1024 + (q * 64 + lane) * 4) * 4), v);
                        } else {
                            shared_store4(agr, (int)(((size_t)c * REC + (size_t)tl * 1024 + (q * 64 + lane) * 4) * 4), s4);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int ii = 0; ii < CSG; ++ii) sacc[g0 + ii] = pacc[ii];
            }
        }
    }

    // ---- publish.  Each chunk's record holds its own contribution S_c with its decay E_c
    // (the aggregate) and, once known, the state after the chunk (inclusive).  Chunk 0 has
    // its inclusive state at once, E_0 h0 + S_0 (it alone reads h0); later chunks publish
    // their aggregate now and their inclusive state after the look-back below.  Each light
    // wave waits for its own stores, then counts itself in LDS; the fourth raises the flag.
    // The last chunk publishes nothing: nothing waits for it. ----
    int *sCnt = reinterpret_cast<int *>(sMid + 64);  // light waves past the first publication
    int *sCnt2 = sCnt + 1;                            // owning waves past the inclusive publication
    constexpr int NOWN = NTL * (PT < LW ? PT : LW);   // owning waves
    f32x16 hin[TPWL];
#pragma unroll
    for (int i = 0; i < TPWL; ++i) hin[i] = f32x16{};
    if (!kWide && c == 0 && p.cont && owner) {
#pragma unroll
        for (int i = 0; i < TPWL; ++i) {
            const int pt = jpart + LW * i;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n = snt * kT + 8 * (r / 4) + 4 * hf + (r % 4);
                hin[i][r] = cache[(size_t)n * P + pc0 + pt * kT + l32];
            }
        }
    }
    if (light) {
        // (the wide form stored its tiles as it formed them)
        if (!last || kWide) {
            const size_t base = (size_t)c * REC + (c == 0 ? INC : 0);
            if (!kWide && owner) {
#pragma unroll
                for (int i = 0; i < TPWL; ++i) {
                    const int tl = snt + NTL * (jpart + LW * i);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        f32x4 v;
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            v[u] = c == 0 ? __builtin_fmaf(Ec, hin[i][4 * q + u], sacc[i][4 * q + u]) : sacc[i][4 * q + u];
                        shared_store4(agr, (int)((base + (size_t)tl * 1024 + (q * 64 + lane) * 4) * 4), v);
                    }
                }
            }
            if (c > 0 && tid == 0) shared_store(recs + (size_t)c * REC + (size_t)N * PC, Ec);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are complete
        }
        if (lane == 0) {
            const int before = atomicAdd(sCnt, 1);
            if (!last && before == 3)
                scan_store(flags + c, scan_flag(epoch, c == 0 ? kFlagInclusive : kFlagAggregate));
        }
    }
    // ---- outputs: intra-chunk products, as in the output phase (only when y is wanted) ----
    const bool want_y = p.y != nullptr;
    f32x16 acc[PT];
#pragma unroll
    for (int i = 0; i < PT; ++i) acc[i] = f32x16{};
    if (active && want_y) {
        const float et = __expf(sR[min(t, Q - 1)]);
        // software pipeline over the tiles J = 0..I: the matrix cores form tile J + 1's
        // Z (its B rows read from LDS a tile earlier still) while the vector units mask
        // tile J's, so neither waits for the other within the wave
        bf16x8 bq[NK];
        load_btile<NK>(bq, sB, 0, l32, hf, BS);
        f32x16 zn = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) zn = mfma(bq[kk], cf[kk], zn);
        load_btile<NK>(bq, sB, min(1, I), l32, hf, BS);
        for (int J = 0; J < I; ++J) {
            const f32x16 z = zn;
            zn = f32x16{};
            const float rowf = sMid[I * 8 + J] * et;
            // tile J's column factors (registers 4q..4q+3 hold s = 32J + 8q + 4hf + (0..3))
            // and its X operands, read ahead
            float cv[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 cf4 = *reinterpret_cast<const float4 *>(sColf + J * kT + 8 * q + 4 * hf);
                cv[4 * q] = cf4.x, cv[4 * q + 1] = cf4.y, cv[4 * q + 2] = cf4.z, cv[4 * q + 3] = cf4.w;
            }
            bf16x8 xv[PT][2];
            load_x<PT>(xv, sXT + l32 * XS + J * kT + 4 * hf, XS);
            // the matrix cores form tile J + 1's Z one k-step at a time while the vector
            // units mask and split tile J's values, a few per k-step (the order is pinned,
            // so neither unit waits for the other's whole tile)
            i32x4v hw[2], lw[2];
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                zn = mfma(bq[kk], cf[kk], zn);
#pragma unroll
                for (int v = kk * 16 / NK; v < (kk + 1) * 16 / NK; v += 2) {
                    uint32_t hh, ll;
                    split2(z[v] * cv[v] * rowf, z[v + 1] * cv[v + 1] * rowf, hh, ll);
                    hw[v / 8][(v % 8) / 2] = (int)hh;
                    lw[v / 8][(v % 8) / 2] = (int)ll;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            load_btile<NK>(bq, sB, min(J + 2, I), l32, hf, BS);
            const bf16x8 ah[2] = {__builtin_bit_cast(bf16x8, hw[0]), __builtin_bit_cast(bf16x8, hw[1])};
            const bf16x8 al[2] = {__builtin_bit_cast(bf16x8, lw[0]), __builtin_bit_cast(bf16x8, lw[1])};
            mx_products<PT>(acc, ah, al, xv);
        }
        {
            const int J = I;
            const f32x16 z = zn;
            const float Rt = sR[min(t, Q - 1)];
            f32x16 mv;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 r4 = *reinterpret_cast<const float4 *>(sR + J * kT + 8 * q + 4 * hf);
                const float4 d4 = *reinterpret_cast<const float4 *>(sDt + J * kT + 8 * q + 4 * hf);
                const float rv[4] = {r4.x, r4.y, r4.z, r4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int u2 = 0; u2 < 4; ++u2) {
                    const int r = 4 * q + u2;
                    const int sl = 8 * q + 4 * hf + u2;
                    float m = z[r] * dv4[u2] * __expf(Rt - rv[u2]);
                    m = sl < l32 ? m : (sl == l32 ? m + Dh : 0.f);
                    mv[r] = m;
                }
            }
            bf16x8 ah[2], al[2];
            split16(mv, ah, al);
            accumulate_mx<PT>(acc, ah, al, sXT + l32 * XS + J * kT + 4 * hf, XS);
        }
    }
    // ---- the state entering this chunk (c > 0), by decoupled look-back.  Lane i of each
    // owning wave watches chunk c-1-i; the wave waits until some chunk j0 < c has published
    // the state after it (inclusive) and every chunk after j0 has published its own
    // contribution (aggregate), then reads j0's state and folds the contributions
    // j0+1..c-1 in order, h <- E_j h + S_j.  Every inclusive record is that same fold in
    // the same order, back to chunk 0's E_0 h0 + S_0, so h_in is bit for bit the state of
    // a sequential pass over the chunks, whichever j0 the wait ends at. ----
    // The whole-head form: after the rows all eight waves take part, each with two of the
    // head's sixteen state tiles (row tile snt, column tiles 2 jpart and 2 jpart + 1), so
    // that more of the records are in flight at once; each wave keeps several links of the
    // fold in flight (loads clamped to the last link, the fold of a link past the end a
    // select, so that no branch makes the compiler wait).
    constexpr int WT = 2;  // tiles per wave
    constexpr int LD = 2;  // links of the fold in flight
    f32x16 hinw[WT];
#pragma unroll
    for (int i = 0; i < WT; ++i) hinw[i] = f32x16{};
    if constexpr (kWide) {
        auto wtile = [&](int i) { return snt + NTL * (2 * jpart + i); };
        auto rec4 = [&](size_t off, int tl, int q) {
            return shared_load4(agr, (int)((off + (size_t)tl * 1024 + (q * 64 + lane) * 4) * 4));
        };
        // what the light waves published (S_c; chunk 0: h0 and its inclusive state) is
        // complete before any wave reads it back: they counted themselves after their stores
        if (lane == 0) {
            for (int spin = 0; spin < (1 << 20); ++spin) {
                if (__hip_atomic_load(sCnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= 4) break;
                __builtin_amdgcn_s_sleep(1);
            }
        }
        asm volatile("" ::: "memory");
        if (c == 0) {
            if (p.cont) {
#pragma unroll
                for (int i = 0; i < WT; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4 v = rec4(0, wtile(i), q);  // h0, parked in the aggregate area
#pragma unroll
                        for (int u = 0; u < 4; ++u) hinw[i][4 * q + u] = v[u];
                    }
            }
        } else {
            const long long tw0 = (long long)__builtin_amdgcn_s_memrealtime();
            int j0 = 0;
            while (true) {
                const int f = lane < c ? scan_load(flags + (c - 1 - lane)) : 0;
                const bool ready = lane < c && (static_cast<uint32_t>(f) >> 2) == static_cast<uint32_t>(epoch);
                const uint64_t mi = __ballot(ready && (f & 3) == kFlagInclusive);
                const uint64_t mr = __ballot(ready);
                if (mi) {
                    const int d = __builtin_ctzll(mi);
                    const uint64_t need = (1ull << d) - 1;
                    if ((mr & need) == need) {
                        j0 = c - 1 - d;
                        break;
                    }
                }
                __builtin_amdgcn_s_sleep(2);
                if ((long long)__builtin_amdgcn_s_memrealtime() - tw0 > kScanWaitTicks) {
                    if (lane == 0) atomicOr(p.err + slot, MIL_DEVERR_SCAN);
                    break;
                }
            }
            if (last && wave == 0 && lane == 0) scan_store(flags + kScanEpoch, epoch);
            asm volatile("" ::: "memory");  // the records are read after the flags
            f32x16 buf[LD][WT];
            float eb[LD];
#pragma unroll
            for (int i = 0; i < WT; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v = rec4((size_t)j0 * REC + INC, wtile(i), q);
#pragma unroll
                    for (int u = 0; u < 4; ++u) hinw[i][4 * q + u] = v[u];
                }
#pragma unroll
            for (int d = 0; d < LD; ++d) {
                const int jj = min(j0 + 1 + d, c - 1);
#pragma unroll
                for (int i = 0; i < WT; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4 v = rec4((size_t)jj * REC, wtile(i), q);
#pragma unroll
                        for (int u = 0; u < 4; ++u) buf[d][i][4 * q + u] = v[u];
                    }
                eb[d] = shared_load(recs + (size_t)jj * REC + (size_t)N * PC);
            }
            for (int j = j0 + 1; j < c; j += LD) {
#pragma unroll
                for (int d = 0; d < LD; ++d) {
                    const bool use = j + d < c;  // links past the end: loads clamped, fold skipped
                    const float e = eb[d];
#pragma unroll
                    for (int i = 0; i < WT; ++i)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float f = __builtin_fmaf(e, hinw[i][r], buf[d][i][r]);
                            hinw[i][r] = use ? f : hinw[i][r];
                        }
                    const int jj = min(j + d + LD, c - 1);
#pragma unroll
                    for (int i = 0; i < WT; ++i)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const f32x4 v = rec4((size_t)jj * REC, wtile(i), q);
#pragma unroll
                            for (int u = 0; u < 4; ++u) buf[d][i][4 * q + u] = v[u];
                        }
                    eb[d] = shared_load(recs + (size_t)jj * REC + (size_t)N * PC);
                }
            }
            // the state after this chunk, E_c h_in + S_c (S_c read back), for the chunks after it
            if (pub_inc) {
#pragma unroll
                for (int i = 0; i < WT; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4 s4 = rec4((size_t)c * REC, wtile(i), q);
                        f32x4 v;
#pragma unroll
                        for (int u = 0; u < 4; ++u) v[u] = __builtin_fmaf(Ec, hinw[i][4 * q + u], s4[u]);
                        shared_store4(agr, (int)(((size_t)c * REC + INC + (size_t)wtile(i) * 1024 + (q * 64 + lane) * 4) * 4), v);
                    }
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                // the aggregate count (four light waves) was seen above; the eighth wave past
                // its inclusive tiles raises the flag
                if (lane == 0 && atomicAdd(sCnt2, 1) == 7) scan_store(flags + c, scan_flag(epoch, kFlagInclusive));
            }
        }
        // the final state: chunk 0's inclusive record, or E_c h_in + S_c
        if (last) {
#pragma unroll
            for (int i = 0; i < WT; ++i) {
                const int pt = 2 * jpart + i;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v = rec4((size_t)c * REC + (c == 0 ? INC : 0), wtile(i), q);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int r = 4 * q + u;
                        const int n = snt * kT + 8 * (r / 4) + 4 * hf + (r % 4);
                        cache[(size_t)n * P + pc0 + pt * kT + l32] = c == 0 ? v[u] : __builtin_fmaf(Ec, hinw[i][r], v[u]);
                    }
                }
            }
        }
    } else {
        if (c > 0 && owner) {
            const long long tw0 = (long long)__builtin_amdgcn_s_memrealtime();
            int j0 = 0;
            while (true) {
                const int f = lane < c ? scan_load(flags + (c - 1 - lane)) : 0;
                const bool ready = lane < c && (static_cast<uint32_t>(f) >> 2) == static_cast<uint32_t>(epoch);
                const uint64_t mi = __ballot(ready && (f & 3) == kFlagInclusive);
                const uint64_t mr = __ballot(ready);
                if (mi) {
                    const int d = __builtin_ctzll(mi);            // nearest inclusive: chunk c-1-d
                    const uint64_t need = (1ull << d) - 1;        // chunks c-d..c-1: aggregates at least
                    if ((mr & need) == need) {
                        j0 = c - 1 - d;
                        break;
                    }
                }
                __builtin_amdgcn_s_sleep(2);
                if ((long long)__builtin_amdgcn_s_memrealtime() - tw0 > kScanWaitTicks) {
                    if (lane == 0) atomicOr(p.err + slot, MIL_DEVERR_SCAN);
                    break;
                }
            }
            // every earlier chunk of the row has published, so has read the old epoch: this
            // launch's epoch becomes the row's (also after a timeout, so that no flag of this
            // launch is ever above the row's epoch)
            if (last && wave == 0 && lane == 0) scan_store(flags + kScanEpoch, epoch);
            asm volatile("" ::: "memory");  // the records are read after the flags
            // j0's inclusive tiles, then the aggregates j0+1..c-1, the next one's loads (clamped
            // to the last, so that no branch makes the compiler wait for every load) in flight
            // while one is folded in
            constexpr int LBG = TPWL;  // tiles folded together
#pragma unroll
            for (int g0 = 0; g0 < TPWL; g0 += LBG) {
                f32x16 nx[LBG];
                float en = 0.f;
                const int ja = min(j0 + 1, c - 1);
#pragma unroll
                for (int ii = 0; ii < LBG; ++ii) {
                    const int tl = snt + NTL * (jpart + LW * (g0 + ii));
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int lo = (q * 64 + lane) * 4 + tl * 1024;
                        const f32x4 v = shared_load4(agr, (int)(((size_t)j0 * REC + INC + lo) * 4));
                        const f32x4 a = shared_load4(agr, (int)(((size_t)ja * REC + lo) * 4));
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            hin[g0 + ii][4 * q + u] = v[u];
                            nx[ii][4 * q + u] = a[u];
                        }
                    }
                }
                en = shared_load(recs + (size_t)ja * REC + (size_t)N * PC);
                for (int j = j0 + 1; j < c; ++j) {
                    f32x16 cur[LBG];
#pragma unroll
                    for (int ii = 0; ii < LBG; ++ii) cur[ii] = nx[ii];
                    const float e = en;
                    const int jn = min(j + 1, c - 1);
                    en = shared_load(recs + (size_t)jn * REC + (size_t)N * PC);
#pragma unroll
                    for (int ii = 0; ii < LBG; ++ii) {
                        const int tl = snt + NTL * (jpart + LW * (g0 + ii));
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const f32x4 v = shared_load4(agr, (int)(((size_t)jn * REC + (size_t)tl * 1024 + (q * 64 + lane) * 4) * 4));
#pragma unroll
                            for (int u = 0; u < 4; ++u) nx[ii][4 * q + u] = v[u];
                        }
                    }
#pragma unroll
                    for (int ii = 0; ii < LBG; ++ii)
#pragma unroll
                        for (int r = 0; r < 16; ++r) hin[g0 + ii][r] = __builtin_fmaf(e, hin[g0 + ii][r], cur[ii][r]);
                }
            }
            // the state after this chunk, E_c h_in + S_c, for the chunks after it
            if (pub_inc) {
#pragma unroll
                for (int i = 0; i < TPWL; ++i) {
                    const int tl = snt + NTL * (jpart + LW * i);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        f32x4 v;
                        const f32x4 s4 = {sacc[i][4 * q], sacc[i][4 * q + 1], sacc[i][4 * q + 2], sacc[i][4 * q + 3]};
#pragma unroll
                        for (int u = 0; u < 4; ++u) v[u] = __builtin_fmaf(Ec, hin[i][4 * q + u], s4[u]);
                        shared_store4(agr, (int)(((size_t)c * REC + INC + (size_t)tl * 1024 + (q * 64 + lane) * 4) * 4), v);
                    }
                }
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                if (lane == 0) {
                    // the aggregate flag (raised by the fourth light wave) goes up before this one
                    for (int spin = 0; spin < (1 << 20); ++spin) {
                        if (__hip_atomic_load(sCnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= 4) break;
                        __builtin_amdgcn_s_sleep(1);
                    }
                    if (atomicAdd(sCnt2, 1) == NOWN - 1) scan_store(flags + c, scan_flag(epoch, kFlagInclusive));
                }
            }
        }
        // ---- the final state, from the last chunk (nothing reads h0 after chunk 0 has) ----
        if (last && owner) {
#pragma unroll
            for (int i = 0; i < TPWL; ++i) {
                const int pt = jpart + LW * i;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int n = snt * kT + 8 * (r / 4) + 4 * hf + (r % 4);
                    cache[(size_t)n * P + pc0 + pt * kT + l32] = __builtin_fmaf(Ec, hin[i][r], sacc[i][r]);
                }
            }
        }
    }
    if (p.y == nullptr) {
        if (p.book && blockIdx.x == 0) {
            for (int i = tid; i < p.batch; i += NT) {
                const bool mine = i >= p.slot0 && i < p.slot0 + p.nseq;
                if (mine) p.pos[i] = p.pos_add ? p.pos[i] + p.L : p.L;
                if (mine || p.pos_add) p.pending[i] = 0;
            }
        }
        return;
    }
    if (has_hin) {
        // the carried state as [p][n] groups of 8 hi + 8 lo bf16
        if constexpr (kWide) {
            __syncthreads();  // every wave is done with X^T
#pragma unroll
            for (int i = 0; i < WT; ++i) {
                bf16 *row = sH + ((2 * jpart + i) * kT + l32) * HS;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int grp = snt * 4 + q;  // n group of 8: 8 hi then 8 lo
                    uint2 hi4, lo4;
                    split2(hinw[i][4 * q], hinw[i][4 * q + 1], hi4.x, lo4.x);
                    split2(hinw[i][4 * q + 2], hinw[i][4 * q + 3], hi4.y, lo4.y);
                    *reinterpret_cast<uint2 *>(row + grp * 16 + 4 * hf) = hi4;
                    *reinterpret_cast<uint2 *>(row + grp * 16 + 8 + 4 * hf) = lo4;
                }
            }
        } else if (owner) {
#pragma unroll
            for (int i = 0; i < TPWL; ++i) {
                const int pt = jpart + LW * i;
                bf16 *row = sH + (pt * kT + l32) * HS;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int grp = snt * 4 + q;  // n group of 8: 8 hi then 8 lo
                    uint2 hi4, lo4;
                    split2(hin[i][4 * q], hin[i][4 * q + 1], hi4.x, lo4.x);
                    split2(hin[i][4 * q + 2], hin[i][4 * q + 3], hi4.y, lo4.y);
                    *reinterpret_cast<uint2 *>(row + grp * 16 + 4 * hf) = hi4;
                    *reinterpret_cast<uint2 *>(row + grp * 16 + 8 + 4 * hf) = lo4;
                }
            }
        }
        __syncthreads();
        if (active) {
            f32x16 acc2[PT];
#pragma unroll
            for (int i = 0; i < PT; ++i) acc2[i] = f32x16{};
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const bf16 *row = sH + (pt * kT + l32) * HS;
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    const bf16 *grp = row + (kk * 2 + hf) * 16;
                    const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(grp);
                    const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(grp + 8);
                    acc2[pt] = mfma(cf[kk], bh, acc2[pt]);
                    acc2[pt] = mfma(cf[kk], bl, acc2[pt]);
                }
            }
            float ein[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) ein[r] = sEin[min(I * kT + 8 * (r / 4) + 4 * hf + (r % 4), Q - 1)];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[pt][r] = __builtin_fmaf(ein[r], acc2[pt][r], acc[pt][r]);
            }
        }
    }
    if (p.book && blockIdx.x == 0) {  // the slots' bookkeeping, off the start of the critical chunk
        for (int i = tid; i < p.batch; i += NT) {
            const bool mine = i >= p.slot0 && i < p.slot0 + p.nseq;
            if (mine) p.pos[i] = p.pos_add ? p.pos[i] + p.L : p.L;
            if (mine || p.pos_add) p.pending[i] = 0;
        }
    }
    if (!active) return;
    // y rows of this tile, stored non-temporally as in the output phase
    float *yb = p.y + ((tok0 + I * kT) * H + h) * P + pc0 + l32;
    const int ystride = H * P;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int tl = 8 * (r / 4) + 4 * hf + (r % 4);
        if (I * kT + tl < len) {
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) __builtin_nontemporal_store(acc[pt][r], yb + tl * ystride + pt * kT);
        }
    }
}

size_t scan_lds_bytes(int Q, int N, int P) {
    return scan_base_lds(Q, N, P) + (scan_wide(N, P) ? 0 : scan_xchg_bytes(N, P));
}

size_t out_lds_bytes(int Q, int N, int P) {
    const size_t big = std::max((size_t)Q * (N + 8) + (size_t)P * (Q + 8), (size_t)P * (N * 2 + 8)) * 2;
    return big + 6 * Q * 4 + 8 * 4 + 64 * 4;
}
size_t state_lds_bytes(int PS, int N) { return (size_t)(PS + 2 * N) * kSBS * 2 + (4 * 256 + 8) * 4; }

constexpr int64_t kOutItemsTarget = 256;  // output workgroups wanted (one per compute unit)

// Column slab width of the output work (and of the single launch): P split until the grid
// has a workgroup per compute unit.
// Compute units of the current device (cached per device; 256 if the query fails).
int compute_units() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

int slab_width(int nseq, int nch, int H, int P) {
    int pc = P;
    while (pc > kT && (int64_t)nseq * nch * H * (P / pc) < kOutItemsTarget) pc /= 2;
    return pc;
}

// Column slab width of the single launch: the output work's, at most 128 columns where
// N = 128 (the wide form: one workgroup forms each C B^T tile and its decay mask for all
// 128 columns, and the carried state reuses X^T's LDS) and 64 otherwise.
int scan_slab(int nseq, int nch, int H, int P, int N) {
    return std::min(slab_width(nseq, nch, H, P), N == 128 ? 128 : 64);
}

// The single-launch kernel for these sizes, or null (its LDS does not fit, or a chunk other
// than 256 tokens, which it is not built for).  One launch covers at most kScanChunks
// chunks; longer prompts take several launches, each continuing from the last.
const void *scan_kernel(int chunk, int N, int pc) {
    if (chunk != 256 || scan_lds_bytes(chunk, N, pc) > kLdsMax) return nullptr;
#define MIL_SCAN_CASE(n, pp) \
    if (N == n && pc == pp) return reinterpret_cast<const void *>(chunk_scan_mfma<n, pp>);
    MIL_SCAN_CASE(64, 32) MIL_SCAN_CASE(64, 64) MIL_SCAN_CASE(128, 32) MIL_SCAN_CASE(128, 64)
    MIL_SCAN_CASE(128, 128)
#undef MIL_SCAN_CASE
    return nullptr;
}

}  // namespace

bool prefill_single_launch(int nseq, int L, int chunk, int H, int P, int N) {
    if (!prefill_mfma_supported(chunk, N, P)) return false;
    const int nch = (L + chunk - 1) / chunk;
    return scan_kernel(chunk, N, scan_slab(nseq, std::min(nch, kScanChunks), H, P, N)) != nullptr;
}

// Shapes the matrix-core path covers: bf16 inputs, N and P multiples of 32 up to 256,
// a chunk the LDS can hold.
bool prefill_mfma_supported(int Q, int N, int P) {
    if (N % 32 != 0 || P % 32 != 0 || N > 256 || P > 256) return false;
    if (N % 64 != 0) return false;  // phase 2 works on 64-row tiles
    if (out_lds_bytes(Q, N, P) > kLdsMax) return false;
    const int PS = P < 32768 / N ? P : 32768 / N;
    // phase 1 deals (PS/32)*(N/32) output tiles to 4 waves, at most 8 each
    const int tiles = (PS / 32) * (N / 32);
    return PS % 32 == 0 && tiles % 4 == 0 && tiles >= 4 && tiles <= 32 && state_lds_bytes(PS, N) <= kLdsMax;
}

hipError_t launch_prefill_mfma(const CacheImpl &c, int slot0, int nseq, int L, int chunk, const void *x,
                               const void *B, const void *C, const void *dt, const float *A, const float *D,
                               float *y, void *ws, bool cont, hipStream_t s) {
    MParams p;
    p.x = static_cast<const uint16_t *>(x);
    p.B = static_cast<const uint16_t *>(B);
    p.C = static_cast<const uint16_t *>(C);
    p.dt = static_cast<const uint16_t *>(dt);
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
    p.pos = cache_pos(c);
    p.pending = cache_pending(c);
    p.slot0 = slot0;
    p.nseq = nseq;
    p.batch = c.dims.batch;
    p.cont = cont ? 1 : 0;
    p.t0 = 0;
    p.book = 1;
    p.pos_add = p.cont;
    p.incl_every = 1;
    p.scan = nullptr;
    p.err = nullptr;
    p.chain = nullptr;
    const int64_t states = (int64_t)nseq * p.nch * p.H * p.N * p.P * 4;
    p.ws = static_cast<float *>(ws);
    p.ws_tot = reinterpret_cast<float *>(static_cast<char *>(ws) + (states + 255) / 256 * 256);
    p.PS = p.P < 32768 / p.N ? p.P : 32768 / p.N;
    p.nslab = p.P / p.PS;

    const int pc = slab_width(nseq, p.nch, p.H, p.P);

    // one launch for all three phases where its LDS fits (chunks of 256, 8 waves), per run
    // of at most kScanChunks chunks: each later launch continues from the state the one
    // before it wrote to the cache, and the last one does the slots' bookkeeping
    if (scan_kernel(chunk, p.N, scan_slab(nseq, std::min(p.nch, kScanChunks), p.H, p.P, p.N))) {
        const int nch_all = p.nch;
        p.scan = cache_scan(c);
        p.err = cache_err(c);
        p.chain = static_cast<float *>(ws);
        p.pos_add = cont ? 1 : 0;
        const int cus = compute_units();
        for (int c0 = 0; c0 < nch_all; c0 += kScanChunks) {
            p.nch = std::min(kScanChunks, nch_all - c0);
            p.t0 = c0 * chunk;
            p.cont = (cont || c0 > 0) ? 1 : 0;
            p.book = c0 + p.nch == nch_all ? 1 : 0;
            const int spc = scan_slab(nseq, p.nch, p.H, p.P, p.N);
            // one workgroup per compute unit (its LDS): a dispatch round holds this many chunks
            p.incl_every = std::max(1, cus / (nseq * p.H * (p.P / spc)));
            const void *kf = scan_kernel(chunk, p.N, spc);
            if (!kf) return hipErrorInvalidValue;
            hipError_t e = hipFuncSetAttribute(kf, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
            if (e != hipSuccess) return e;
            void *args[] = {&p};
            trace_begin(c, MIL_TRACE_PREFILL_SCAN, s);
            e = hipLaunchKernel(kf, dim3(p.nch * nseq * p.H * (p.P / spc)), dim3(512), args,
                                scan_lds_bytes(chunk, p.N, spc), s);
            trace_end(c, MIL_TRACE_PREFILL_SCAN, s);
            if (e != hipSuccess) return e;
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const size_t l1 = state_lds_bytes(p.PS, p.N), l3 = out_lds_bytes(chunk, p.N, pc);
    const int tpw = (p.PS / kT) * (p.N / kT) / 4;
    const void *k1 = tpw == 1 ? reinterpret_cast<const void *>(chunk_state_mfma<1>)
                   : tpw == 2 ? reinterpret_cast<const void *>(chunk_state_mfma<2>)
                   : tpw == 4 ? reinterpret_cast<const void *>(chunk_state_mfma<4>)
                              : reinterpret_cast<const void *>(chunk_state_mfma<8>);
    const void *k3 = nullptr;
#define MIL_OUT_CASE(n, pp) \
    if (p.N == n && pc == pp) k3 = reinterpret_cast<const void *>(chunk_out_mfma<n, pp>);
    MIL_OUT_CASE(64, 32) MIL_OUT_CASE(64, 64) MIL_OUT_CASE(64, 128) MIL_OUT_CASE(64, 256)
    MIL_OUT_CASE(128, 32) MIL_OUT_CASE(128, 64) MIL_OUT_CASE(128, 128) MIL_OUT_CASE(128, 256)
    MIL_OUT_CASE(256, 32) MIL_OUT_CASE(256, 64) MIL_OUT_CASE(256, 128) MIL_OUT_CASE(256, 256)
#undef MIL_OUT_CASE
    if (!k3) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(k1, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
    if (e == hipSuccess) e = hipFuncSetAttribute(k3, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
    if (e != hipSuccess) return e;
    void *args[] = {&p};
    trace_begin(c, MIL_TRACE_PREFILL_STATE, s);
    e = hipLaunchKernel(k1, dim3(nseq * p.nch * p.H * p.nslab), dim3(256), args, l1, s);
    trace_end(c, MIL_TRACE_PREFILL_STATE, s);
    if (e != hipSuccess) return e;
    trace_begin(c, MIL_TRACE_PREFILL_PASS, s);
    hipLaunchKernelGGL(state_pass_pn, dim3((p.P / 32) * (p.N / 64), p.H, nseq), dim3(256), 0, s, p);
    trace_end(c, MIL_TRACE_PREFILL_PASS, s);
    e = hipGetLastError();
    if (e != hipSuccess || y == nullptr) return e;
    trace_begin(c, MIL_TRACE_PREFILL_OUT, s);
    e = hipLaunchKernel(k3, dim3(nseq * p.nch * p.H * (p.P / pc)), dim3(chunk / 32 * 64), args, l3, s);
    trace_end(c, MIL_TRACE_PREFILL_OUT, s);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace mil
