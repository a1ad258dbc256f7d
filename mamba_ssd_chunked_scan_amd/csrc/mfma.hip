// bf16 MFMA kernels (fp32 accumulation) for the two contraction stages of the
// chunked SSD scan: each chunk's own state, and the chunk output.  They cover
// headdim 64, d_state 64 or 128 and chunk 64, 128 or 256 with bf16 x/B/C; any
// other shape runs the generic kernels.
//
// Stage structure ("Compiler-First State Space Duality and Portable O(1)
// Autoregressive Caching for Inference", paperlayer summary, §3 Method,
// "Chunked recurrence", and the three contractions listed in B.5):
//   chunk state   S[p,n]  = sum_j x[j,p] w_j B[j,n],  w_j = dt_j exp(Acs_last - Acs_j)
//   chunk output  y[i,p]  = sum_{j<=i} (C_i.B_j) exp(Acs_i - Acs_j) dt_j x[j,p]
//                           + exp(Acs_i) (C_i . H[p]) + D x[i,p]
// The causal mask is the fixed lower triangle of the chunk ("Primitive-level
// implementation" in the same section): tiles above the diagonal are skipped
// outright and only the diagonal 32x32 tiles are masked element by element.
//
// gfx950 specifics used here:
//  * v_mfma_f32_32x32x16_bf16 (D[32x32] += A[32x16] B[16x32]).  Lane l
//    supplies row (A) or column (B) l%32 and the 8 k slots 8*(l/32)+e; the
//    accumulator holds column l%32 and rows 8*(r/4) + 4*(l/32) + r%4 in its
//    register r (r = 0..15).
//  * ds_read_b64_tr_b16, the LDS transpose read: within each group of 16
//    lanes, lane i receives element (i & 3) of the 8-byte reads of lanes
//    (i >> 2) + 4k, k = 0..3.  It turns a row-major [k][outer] tile into
//    k-contiguous MFMA operands, so every tile is staged in its natural layout
//    with plain 16-byte stores.
//  * v_cvt_pk_bf16_f32 for round-to-nearest-even packing.
//  * blocks are dealt to the 8 XCDs round-robin; the block index is remapped
//    so that the heads of one (batch, chunk) run on one XCD and share its L2
//    copy of the chunk's B and C rows.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "ssd.h"

namespace ssd {
namespace {

constexpr int kP = 64;   // headdim handled here
constexpr int kJT = 32;  // tokens per streamed stage (one 32-row tile)

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef short v4i16 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    return z;
}

__device__ __forceinline__ u32x4 masked(u32x4 v, bool keep) {
    const uint32_t m = keep ? 0xffffffffu : 0u;
    return u32x4{v[0] & m, v[1] & m, v[2] & m, v[3] & m};
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Splits two fp32 values into a packed bf16 pair hi = bf16(v) and the packed
// residual lo = bf16(v - hi): about 16 significant bits in two bf16 operands,
// with the full fp32 exponent range.
__device__ __forceinline__ uint32_t split2(float a, float b, uint32_t &lo) {
    const uint32_t h = pack_bf16x2(a, b);
    lo = pack_bf16x2(a - lo_bf16(h), b - hi_bf16(h));
    return h;
}

__device__ __forceinline__ void split8(const float m[8], u32x4 &hi, u32x4 &lo) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t l;
        hi[k] = split2(m[2 * k], m[2 * k + 1], l);
        lo[k] = l;
    }
}

// ds_read_b64_tr_b16 on a generic pointer into LDS.
__device__ __forceinline__ u32x2 ds_read_tr16(const bf16 *p) {
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)p);
    return __builtin_bit_cast(u32x2, v);
}

// MFMA operand from a row-major [k][outer] bf16 tile in LDS (row stride ld):
// this lane gets outer index outer0 + lane%32 and the k rows of its slots.
// kperm = false: slots e -> k0 + 8*(lane/32) + e (a plain 16-deep k step).
// kperm = true:  slots e -> k0 + 8*(e/4) + 4*(lane/32) + e%4, the row order
//                of a 32x32 accumulator, used when the other operand is built
//                from accumulator registers.
template <bool kperm>
__device__ __forceinline__ u32x4 tr_operand(const bf16 *tile, int ld, int k0, int outer0) {
    const int lane = threadIdx.x & 63, G = lane >> 4, s = lane & 15;
    const int kb = kperm ? k0 + 4 * (G >> 1) : k0 + 8 * (G >> 1);
    const bf16 *p = tile + (kb + (s >> 2)) * ld + outer0 + 16 * (G & 1) + 4 * (s & 3);
    const u32x2 a = ds_read_tr16(p);
    const u32x2 b = ds_read_tr16(p + (kperm ? 8 : 4) * ld);
    return u32x4{a[0], a[1], b[0], b[1]};
}

// Logical block index: block b runs on XCD b % 8, so XCD x receives logical
// blocks [x*per, (x+1)*per) with per = gridDim.x / 8 (the grid is padded to a
// multiple of 8).
__device__ __forceinline__ int64_t xcd_block() {
    const int64_t per = gridDim.x / 8;
    return (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
}

unsigned padded_grid(int64_t blocks) { return (unsigned)((blocks + 7) / 8 * 8); }

// Registers holding one 32-token stage between its global load and its LDS
// store: one 16-byte x segment and NBV 16-byte B segments per thread.  Two sets
// give a prefetch distance of two stages.
template <int NBV>
struct StageRegs {
    u32x4 x;
    u32x4 b[NBV];
};

using P0 = std::integral_constant<int, 0>;
using P1 = std::integral_constant<int, 1>;

// ------------------------------------------------------------ chunk state
// One block (4 waves) per (b, c, h).  S (64 x N fp32) = xw^T B, streamed over
// the chunk in 32-token stages (double-buffered; the next stage's global loads
// are in flight while the current one is multiplied).  xw = x * w is formed in
// fp32 and stored as a hi/lo bf16 pair, so its rounding stays near fp32
// level.  Both operands are read with the LDS transpose read.  Output tiles
// 32x32: wave w owns tiles w and w+4 of the (p-tile, n-tile) grid.
template <int Q, int N>
__global__ void __launch_bounds__(256, 2)
k_chunk_state_mfma(const bf16 *__restrict__ x, const bf16 *__restrict__ Bm,
                   const float *__restrict__ dt, const float *__restrict__ Acs,
                   float *__restrict__ states, int64_t L, int H, int G, int T, int64_t nblocks) {
    constexpr int LDX = kP + 16;              // x stage row stride (bf16)
    constexpr int LDB = N + 16;               // B stage row stride (bf16)
    constexpr int NST = Q / kJT;              // stages per chunk
    constexpr int BSEG = N / 8;               // 16-byte segments per B row
    constexpr int NBV = kJT * BSEG / 256;     // B segments per thread per stage
    __shared__ __attribute__((aligned(16))) bf16 xhi[2][kJT * LDX];
    __shared__ __attribute__((aligned(16))) bf16 xlo[2][kJT * LDX];
    __shared__ __attribute__((aligned(16))) bf16 bst[2][kJT * LDB];
    __shared__ float w[Q];
    const int64_t lb = xcd_block();
    if (lb >= nblocks) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = (int)(lb % H);
    const int64_t bc = lb / H;
    const int c = (int)(bc % T);
    const int64_t b = bc / T;
    const int g = h / (H / G);
    const int64_t t0 = (int64_t)c * Q;
    const int q = (int)min((int64_t)Q, L - t0);
    const bf16 *xbase = x + ((b * L + t0) * H + h) * kP;
    const bf16 *bbase = Bm + ((b * L + t0) * G + g) * N;
    // per-thread offsets are unsigned 32-bit from block-uniform bases (a
    // chunk spans < 2^31 elements of x, B, C and y), so loads and stores use
    // the scalar-base + 32-bit-offset address form and no 64-bit addresses
    // are kept in vector registers
    const unsigned xrs = H * kP, brs = G * N;
    const int xrow = tid >> 3, xseg = tid & 7;

    // weights first: every stage needs them
    {
        const float *acs = Acs + (b * H + h) * L + t0;
        const float last = acs[q - 1];
        for (int j = tid; j < Q; j += 256) {
            const int jj = min(j, q - 1);
            const float v = dt[(b * L + t0 + jj) * H + h] * ssd_exp(last - acs[jj]);
            w[j] = j < q ? v : 0.f;
        }
    }
    StageRegs<NBV> R[2];
    auto load_stage = [&](int st, StageRegs<NBV> &r) {
        const int j = st * kJT + xrow;
        r.x = *reinterpret_cast<const u32x4 *>(xbase + ((unsigned)min(j, q - 1) * xrs + xseg * 8u));
#pragma unroll
        for (int i = 0; i < NBV; ++i) {
            const int e = tid + 256 * i, rr = e / BSEG, sg = e % BSEG;
            r.b[i] = *reinterpret_cast<const u32x4 *>(bbase + ((unsigned)min(st * kJT + rr, q - 1) * brs + sg * 8u));
        }
    };
    auto store_stage = [&](int st, int buf, const StageRegs<NBV> &r) {
        const int j = st * kJT + xrow;
        const float wj = w[j];  // zero at and beyond q
        float v[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = lo_bf16(r.x[k]) * wj;
            v[2 * k + 1] = hi_bf16(r.x[k]) * wj;
        }
        u32x4 hi, lo;
        split8(v, hi, lo);
        *reinterpret_cast<u32x4 *>(&xhi[buf][xrow * LDX + xseg * 8]) = masked(hi, j < q);
        *reinterpret_cast<u32x4 *>(&xlo[buf][xrow * LDX + xseg * 8]) = masked(lo, j < q);
#pragma unroll
        for (int i = 0; i < NBV; ++i) {
            const int e = tid + 256 * i, rr = e / BSEG, sg = e % BSEG;
            *reinterpret_cast<u32x4 *>(&bst[buf][rr * LDB + sg * 8]) =
                masked(r.b[i], st * kJT + rr < q);
        }
    };

    // prefetch distance two: stage s+2's loads are issued while stage s is
    // multiplied and stage s+1 (already in registers) is written to LDS
    load_stage(0, R[0]);
    load_stage(1, R[1]);
    __syncthreads();  // w complete
    store_stage(0, 0, R[0]);
    __syncthreads();

    constexpr int NT = N / 32, TPW = (2 * NT) / 4;
    f32x16 acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t] = zero16();
    auto step = [&](int st, auto par) {
        constexpr int PAR = decltype(par)::value;  // st % 2, the LDS buffer
        if (st + 2 < NST) load_stage(st + 2, R[PAR]);
#pragma unroll
        for (int ks = 0; ks < kJT / 16; ++ks) {
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int tile = wave + 4 * t, pt = tile / NT, nt = tile % NT;
                const u32x4 ah = tr_operand<false>(xhi[PAR], LDX, 16 * ks, 32 * pt);
                const u32x4 al = tr_operand<false>(xlo[PAR], LDX, 16 * ks, 32 * pt);
                const u32x4 bb = tr_operand<false>(bst[PAR], LDB, 16 * ks, 32 * nt);
                acc[t] = mfma32(ah, bb, acc[t]);
                acc[t] = mfma32(al, bb, acc[t]);
            }
        }
        if (st + 1 < NST) store_stage(st + 1, PAR ^ 1, R[PAR ^ 1]);
        __syncthreads();
    };
    for (int st = 0; st < NST; st += 2) {  // NST is even
        step(st, P0{});
        step(st + 1, P1{});
    }
    float *out = states + ((b * T + c) * H + h) * (int64_t)(kP * N);
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int tile = wave + 4 * t, pt = tile / NT, nt = tile % NT;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int p = pt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            out[p * N + nt * 32 + (lane & 31)] = acc[t][r];
        }
    }
}

// ------------------------------------------------------------- chunk scan
// One block (4 waves) per (b, c, h); 32-row output tiles.  Wave w owns tiles
// {w, NI-1-w} when the chunk has 8 tiles (equal causal work), else tile w.
// Per owned tile the wave keeps Y^T (64 x 32, two accumulators over p) and
// the tile's C rows in registers; the two tiles share every operand read of
// a step, so their MFMA chains interleave.
//
//  prologue: the entering state H (hi/lo bf16) is staged in LDS and the state
//            term starts each accumulator: Y^T = exp(Acs_k) H C_i^T, k the
//            tile's first row;
//  j loop:   32-token stages of B (natural layout) and x (natural layout, read
//            transposed) stream through two LDS buffers, loaded two stages
//            ahead.  For each owned tile i >= j:  S^T = B_j C_i^T (MFMA);
//              off-diagonal: M^T = S^T * cf[j], cf[j] = exp(Acs_k - Acs_j) dt_j;
//              diagonal:     Y^T *= exp(Acs_i - Acs_k) first, then
//                            M^T[j][i] = S^T exp(Acs_i - Acs_j) dt_j for j <= i;
//            Y^T += X_j^T M^T (M as a hi/lo pair).
//  epilogue: one step after its diagonal (when the wave has no other work for
//            that tile) the tile's y = Y + D x is staged in LDS and written as
//            full 128-byte rows.
// The row factor exp(Acs_i - Acs_k) times exp(Acs_k) gives the state term its
// exp(Acs_i); every exponent used is <= 0.
template <int Q, int N>
__global__ void __launch_bounds__(256, 2)
k_chunk_scan_mfma(const bf16 *__restrict__ x, const float *__restrict__ dt,
                  const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm,
                  const float *__restrict__ D, const float *__restrict__ Acs,
                  const float *__restrict__ states, bf16 *__restrict__ y, int64_t L, int H, int G,
                  int T, int64_t nblocks) {
    constexpr int NI = Q / 32;
    constexpr int KS = N / 16;
    constexpr int LDH = N + 8;   // H rows, read as plain 16-byte operands
    constexpr int LDB = N + 8;   // B stage rows, read as plain 16-byte operands
    constexpr int LDX = kP + 16; // x stage rows, read transposed
    constexpr int LDY = kP + 8;  // bf16 y staging rows
    constexpr int H_BYTES = 2 * kP * LDH * 2;
    constexpr int Y_BYTES = 4 * 32 * LDY * 2;
    constexpr int HY_BYTES = H_BYTES > Y_BYTES ? H_BYTES : Y_BYTES;
    constexpr int BSEG = N / 8;
    constexpr int NBV = kJT * BSEG / 256;
    constexpr int NHV = kP * N / 4 / 256;
    __shared__ __attribute__((aligned(16))) char hy[HY_BYTES];
    __shared__ __attribute__((aligned(16))) bf16 bst[2][kJT * LDB];
    __shared__ __attribute__((aligned(16))) bf16 xst[2][kJT * LDX];
    __shared__ __attribute__((aligned(16))) float cf[NI][Q];
    __shared__ __attribute__((aligned(16))) float acs_s[Q];
    __shared__ __attribute__((aligned(16))) float dt_s[Q];
    const int64_t lb = xcd_block();
    if (lb >= nblocks) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int il = lane & 31, g2 = lane >> 5;
    const int h = (int)(lb % H);
    const int64_t bc = lb / H;
    const int c = (int)(bc % T);
    const int64_t b = bc / T;
    const int g = h / (H / G);
    const int64_t t0 = (int64_t)c * Q;
    const int q = (int)min((int64_t)Q, L - t0);
    const bf16 *xbase = x + ((b * L + t0) * H + h) * kP;
    const bf16 *bbase = Bm + ((b * L + t0) * G + g) * N;
    // per-thread offsets are unsigned 32-bit from block-uniform bases (a
    // chunk spans < 2^31 elements of x, B, C and y), so loads and stores use
    // the scalar-base + 32-bit-offset address form
    const unsigned xrs = H * kP, brs = G * N;
    const int xrow = tid >> 3, xseg = tid & 7;
    bf16 *Hh = reinterpret_cast<bf16 *>(hy);
    bf16 *Hl = Hh + kP * LDH;

    const int ntiles = NI == 8 ? 2 : (wave < NI ? 1 : 0);
    const int itile[2] = {wave, NI - 1 - wave};

    StageRegs<NBV> R[2];
    auto load_stage = [&](int st, StageRegs<NBV> &r) {
        const int j = st * kJT + xrow;
        r.x = *reinterpret_cast<const u32x4 *>(xbase + ((unsigned)min(j, q - 1) * xrs + xseg * 8u));
#pragma unroll
        for (int i = 0; i < NBV; ++i) {
            const int e = tid + 256 * i, rr = e / BSEG, sg = e % BSEG;
            r.b[i] = *reinterpret_cast<const u32x4 *>(
                bbase + ((unsigned)min(st * kJT + rr, q - 1) * brs + sg * 8u));
        }
    };
    auto store_stage = [&](int st, int buf, const StageRegs<NBV> &r) {
        *reinterpret_cast<u32x4 *>(&xst[buf][xrow * LDX + xseg * 8]) =
            masked(r.x, st * kJT + xrow < q);
#pragma unroll
        for (int i = 0; i < NBV; ++i) {
            const int e = tid + 256 * i, rr = e / BSEG, sg = e % BSEG;
            *reinterpret_cast<u32x4 *>(&bst[buf][rr * LDB + sg * 8]) =
                masked(r.b[i], st * kJT + rr < q);
        }
    };

    // ---- prologue: issue the global loads first
    float4 hv[NHV];
    {
        const float *Hc = states + ((b * T + c) * H + h) * (int64_t)(kP * N);
#pragma unroll
        for (int i = 0; i < NHV; ++i) hv[i] = *reinterpret_cast<const float4 *>(Hc + 4 * (tid + 256 * i));
    }
    load_stage(0, R[0]);
    load_stage(1, R[1]);  // NI >= 2
    {
        const float *acs = Acs + (b * H + h) * L + t0;
        const float last = acs[q - 1];
        for (int j = tid; j < Q; j += 256) {
            const int jj = min(j, q - 1);
            const float a = acs[jj], d = dt[(b * L + t0 + jj) * H + h];
            acs_s[j] = j < q ? a : last;
            dt_s[j] = j < q ? d : 0.f;
        }
    }
#pragma unroll
    for (int i = 0; i < NHV; ++i) {
        const int e = tid + 256 * i, p = e / (N / 4), n = (e % (N / 4)) * 4;
        u32x2 hh, hl;
        uint32_t l0, l1;
        hh[0] = split2(hv[i].x, hv[i].y, l0);
        hh[1] = split2(hv[i].z, hv[i].w, l1);
        hl[0] = l0;
        hl[1] = l1;
        *reinterpret_cast<u32x2 *>(Hh + p * LDH + n) = hh;
        *reinterpret_cast<u32x2 *>(Hl + p * LDH + n) = hl;
    }
    store_stage(0, 0, R[0]);
    // C rows of the owned tiles stay in registers for the whole kernel
    u32x4 creg[2][KS];
    {
        const bf16 *cbase = Cm + ((b * L + t0) * G + g) * N;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int i_loc = itile[t] * 32 + il;
            const unsigned coff = (unsigned)max(0, min(i_loc, q - 1)) * brs + 8u * g2;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                creg[t][s] = u32x4{0u, 0u, 0u, 0u};
                if (t < ntiles)
                    creg[t][s] = masked(*reinterpret_cast<const u32x4 *>(cbase + (coff + 16u * s)),
                                        i_loc < q);
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < NI * Q; e += 256) {
        const int kt = e / Q, j = e % Q;
        cf[kt][j] = j < 32 * kt ? ssd_exp(acs_s[32 * kt] - acs_s[j]) * dt_s[j] : 0.f;
    }
    // state term: Y^T = exp(Acs_k) H C_i^T, both tiles together (four chains)
    f32x16 yacc[2][2] = {{zero16(), zero16()}, {zero16(), zero16()}};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
            const int ho = (pt * 32 + il) * LDH + 16 * s + 8 * g2;
            const u32x4 ah = *reinterpret_cast<const u32x4 *>(Hh + ho);
            const u32x4 al = *reinterpret_cast<const u32x4 *>(Hl + ho);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                if (t < ntiles) {
                    yacc[t][pt] = mfma32(ah, creg[t][s], yacc[t][pt]);
                    yacc[t][pt] = mfma32(al, creg[t][s], yacc[t][pt]);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    float acs_i[2], ri[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int k = min(max(0, itile[t]), NI - 1) * 32;  // clamped for idle slots
        acs_i[t] = acs_s[k + il];
        ri[t] = ssd_exp(acs_i[t] - acs_s[k]);
        const float ek = ssd_exp(acs_s[k]);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
            for (int r = 0; r < 16; ++r) yacc[t][pt][r] *= ek;
    }
    __syncthreads();  // cf complete; H no longer read (its LDS becomes y staging)

    bf16 *ys = reinterpret_cast<bf16 *>(hy) + wave * 32 * LDY;
    bf16 *ybase = y + ((b * L + t0) * H + h) * kP;
    const float Dh = D ? D[h] : 0.f;

    // y tile t (D x already added) as bf16 via LDS, written as full rows
    auto epilogue = [&](int t, int jt) {
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int p0 = pt * 32 + 8 * rg + 4 * g2;
                u32x2 o;
                o[0] = pack_bf16x2(yacc[t][pt][4 * rg + 0], yacc[t][pt][4 * rg + 1]);
                o[1] = pack_bf16x2(yacc[t][pt][4 * rg + 2], yacc[t][pt][4 * rg + 3]);
                *reinterpret_cast<u32x2 *>(&ys[il * LDY + p0]) = o;
            }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int r = (lane >> 3) + 8 * kk, sg = lane & 7;
            const u32x4 o = *reinterpret_cast<const u32x4 *>(&ys[r * LDY + 8 * sg]);
            const int row = jt * 32 + r;  // formed in the loop: no hoisted 64-bit addresses
            if (row < q) *reinterpret_cast<u32x4 *>(ybase + ((unsigned)row * xrs + 8u * sg)) = o;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
    };

    auto jstep = [&](int jt, auto par) {
        constexpr int buf = decltype(par)::value;  // jt % 2, the LDS buffer
        if (jt + 2 < NI) load_stage(jt + 2, R[buf]);
        bool act[2], diag[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            act[t] = t < ntiles && itile[t] >= jt;
            diag[t] = act[t] && itile[t] == jt;
        }
        if (act[0] || act[1]) {
            f32x16 sacc[2] = {zero16(), zero16()};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 a =
                    *reinterpret_cast<const u32x4 *>(&bst[buf][il * LDB + 16 * ks + 8 * g2]);
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    if (act[t]) sacc[t] = mfma32(a, creg[t][ks], sacc[t]);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t)
                if (diag[t]) {
                    // rescale the state term to exp(Acs_i) and add D x (x rows
                    // of this tile are the current stage)
#pragma unroll
                    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
                        for (int rg = 0; rg < 4; ++rg) {
                            const int p0 = pt * 32 + 8 * rg + 4 * g2;
                            const u32x2 xr =
                                *reinterpret_cast<const u32x2 *>(&xst[buf][il * LDX + p0]);
                            const int r0 = 4 * rg;
                            yacc[t][pt][r0 + 0] = yacc[t][pt][r0 + 0] * ri[t] + Dh * lo_bf16(xr[0]);
                            yacc[t][pt][r0 + 1] = yacc[t][pt][r0 + 1] * ri[t] + Dh * hi_bf16(xr[0]);
                            yacc[t][pt][r0 + 2] = yacc[t][pt][r0 + 2] * ri[t] + Dh * lo_bf16(xr[1]);
                            yacc[t][pt][r0 + 3] = yacc[t][pt][r0 + 3] * ri[t] + Dh * hi_bf16(xr[1]);
                        }
                }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                // this lane's rows j of S^T in half u: j = jt*32 + 16u + 8(e/4) + 4 g2 + e%4
                u32x4 bop[2], bopl[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    if (!act[t]) continue;
                    float m[8];
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        const int jl = 16 * u + 8 * v + 4 * g2;
                        float4 fv;
                        if (!diag[t]) {
                            fv = *reinterpret_cast<const float4 *>(&cf[itile[t]][jt * 32 + jl]);
                        } else {
                            const float4 aj = *reinterpret_cast<const float4 *>(&acs_s[jt * 32 + jl]);
                            const float4 dj = *reinterpret_cast<const float4 *>(&dt_s[jt * 32 + jl]);
                            fv.x = jl + 0 <= il ? ssd_exp(acs_i[t] - aj.x) * dj.x : 0.f;
                            fv.y = jl + 1 <= il ? ssd_exp(acs_i[t] - aj.y) * dj.y : 0.f;
                            fv.z = jl + 2 <= il ? ssd_exp(acs_i[t] - aj.z) * dj.z : 0.f;
                            fv.w = jl + 3 <= il ? ssd_exp(acs_i[t] - aj.w) * dj.w : 0.f;
                        }
                        m[4 * v + 0] = sacc[t][8 * u + 4 * v + 0] * fv.x;
                        m[4 * v + 1] = sacc[t][8 * u + 4 * v + 1] * fv.y;
                        m[4 * v + 2] = sacc[t][8 * u + 4 * v + 2] * fv.z;
                        m[4 * v + 3] = sacc[t][8 * u + 4 * v + 3] * fv.w;
                    }
                    split8(m, bop[t], bopl[t]);
                }
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) {
                    const u32x4 xa = tr_operand<true>(xst[buf], LDX, 16 * u, 32 * pt);
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        if (act[t]) {
                            yacc[t][pt] = mfma32(xa, bop[t], yacc[t][pt]);
                            yacc[t][pt] = mfma32(xa, bopl[t], yacc[t][pt]);
                        }
                }
            }
        }
        // finished tiles are written one step later, off the diagonal step
#pragma unroll
        for (int t = 0; t < 2; ++t)
            if (t < ntiles && itile[t] == jt - 1) epilogue(t, jt - 1);
        if (jt + 1 < NI) store_stage(jt + 1, buf ^ 1, R[buf ^ 1]);
        __syncthreads();
    };
    for (int jt = 0; jt < NI; jt += 2) {  // NI is even
        jstep(jt, P0{});
        jstep(jt + 1, P1{});
    }
    // the last tile (NI-1) finished in the final step
#pragma unroll
    for (int t = 0; t < 2; ++t)
        if (t < ntiles && itile[t] == NI - 1) epilogue(t, NI - 1);
}

template <int Q, int N>
void launch_state_t(const ScanShape &s, const void *x, const void *Bm, const float *dt,
                    const float *Acs, float *states, hipStream_t st) {
    const int64_t nb = s.B * s.T * s.H;
    k_chunk_state_mfma<Q, N><<<padded_grid(nb), 256, 0, st>>>(
        (const bf16 *)x, (const bf16 *)Bm, dt, Acs, states, s.L, (int)s.H, (int)s.G, (int)s.T, nb);
}

template <int Q, int N>
void launch_scan_t(const ScanShape &s, const void *x, const float *dt, const void *Bm,
                   const void *Cm, const float *D, const float *Acs, const float *states, void *y,
                   hipStream_t st) {
    const int64_t nb = s.B * s.T * s.H;
    k_chunk_scan_mfma<Q, N><<<padded_grid(nb), 256, 0, st>>>(
        (const bf16 *)x, dt, (const bf16 *)Bm, (const bf16 *)Cm, D, Acs, states, (bf16 *)y, s.L,
        (int)s.H, (int)s.G, (int)s.T, nb);
}

}  // namespace

bool mfma_supported(const ScanShape &s) {
    return s.dtype == SSD_BF16 && s.P == kP && (s.N == 64 || s.N == 128) &&
           (s.Q == 64 || s.Q == 128 || s.Q == 256);
}

#define SSD_DISPATCH_QN(FN, ...)                                         \
    do {                                                                 \
        if (s.N == 128) {                                                \
            if (s.Q == 256) FN<256, 128>(__VA_ARGS__);                   \
            else if (s.Q == 128) FN<128, 128>(__VA_ARGS__);              \
            else FN<64, 128>(__VA_ARGS__);                               \
        } else {                                                         \
            if (s.Q == 256) FN<256, 64>(__VA_ARGS__);                    \
            else if (s.Q == 128) FN<128, 64>(__VA_ARGS__);               \
            else FN<64, 64>(__VA_ARGS__);                                \
        }                                                                \
    } while (0)

void launch_chunk_state_mfma(const ScanShape &s, const void *x, const void *Bm,
                             const float *dt, const float *Acs, float *states, hipStream_t st) {
    SSD_DISPATCH_QN(launch_state_t, s, x, Bm, dt, Acs, states, st);
}

void launch_chunk_scan_mfma(const ScanShape &s, const void *x, const float *dt,
                            const void *Bm, const void *Cm, const float *D, const float *Acs,
                            const float *states, void *y, hipStream_t st) {
    SSD_DISPATCH_QN(launch_scan_t, s, x, dt, Bm, Cm, D, Acs, states, y, st);
}

}  // namespace ssd
