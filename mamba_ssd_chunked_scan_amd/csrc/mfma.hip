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
// MFMA used: v_mfma_f32_32x32x16_bf16 (D[32x32] += A[32x16] B[16x32]).  Lane l
// supplies row (A) or column (B) l%32 and 8 consecutive k slots 8*(l/32)+e.
// The accumulator holds column l%32 and rows 8*(r/4) + 4*(l/32) + r%4 in its
// register r (r = 0..15).
#include "common.hpp"
#include "launch.hpp"
#include "ssd.h"

namespace ssd {
namespace {

constexpr int kP = 64;  // headdim handled here

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// element e (0..7) of 8 packed bf16
__device__ __forceinline__ float elem8(u32x4 v, int e) {
    const uint32_t w = v[e >> 1];
    return (e & 1) ? hi_bf16(w) : lo_bf16(w);
}

// 16-bit half e&1 of word e>>1 of two rows, packed as (row0, row1)
__device__ __forceinline__ uint32_t pair16(u32x4 r0, u32x4 r1, int e) {
    const uint32_t a = r0[e >> 1], b = r1[e >> 1];
    return (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

__device__ __forceinline__ u32x4 pack8(const float m[8]) {
    u32x4 v;
    v[0] = pack_bf16x2(m[0], m[1]);
    v[1] = pack_bf16x2(m[2], m[3]);
    v[2] = pack_bf16x2(m[4], m[5]);
    v[3] = pack_bf16x2(m[6], m[7]);
    return v;
}

// m = hi + lo with hi = bf16(m) and lo = bf16(m - hi): about 16 significant
// bits in two bf16 operands, with the full fp32 exponent range.
__device__ __forceinline__ void pack8_split(const float m[8], u32x4 &hi, u32x4 &lo) {
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = m[e] - bf16_to_f32(f32_to_bf16(m[e]));
    hi = pack8(m);
    lo = pack8(r);
}

__device__ __forceinline__ uint32_t split_pair(float a, float b, uint32_t &lo) {
    const bf16 ha = f32_to_bf16(a), hb = f32_to_bf16(b);
    lo = pack_bf16x2(a - bf16_to_f32(ha), b - bf16_to_f32(hb));
    return (uint32_t)ha | ((uint32_t)hb << 16);
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

// Loads rows [0, Q) of one head's x chunk (64 bf16 per row) into registers:
// thread (seg = tid%8, rp = tid/8) takes the 16-byte segment seg of rows
// 2rp + 64i and 2rp + 64i + 1.  Row addresses are clamped to q-1 so every load
// is in bounds; rows at or beyond q are zeroed afterwards.  All loads are
// issued before any is consumed.
template <int Q>
__device__ __forceinline__ void load_x_rows(u32x4 (&r)[Q / 32], const bf16 *xrow0,
                                            int64_t rstride, int q) {
    const int seg = threadIdx.x & 7, rp = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < Q / 32; ++i) {
        const int j = 2 * rp + 64 * (i >> 1) + (i & 1);
        r[i] = *reinterpret_cast<const u32x4 *>(xrow0 + min(j, q - 1) * rstride + seg * 8);
    }
#pragma unroll
    for (int i = 0; i < Q / 32; ++i) r[i] = masked(r[i], 2 * rp + 64 * (i >> 1) + (i & 1) < q);
}

// Writes the rows loaded by load_x_rows transposed, xT[p*LD + j], two rows per
// 32-bit store.  With a weight array the values are scaled by w[j] in fp32 and
// stored as a hi/lo bf16 pair (xT and xTlo).
template <int Q, int LD>
__device__ __forceinline__ void store_x_transposed(const u32x4 (&r)[Q / 32], bf16 *xT,
                                                   const float *w, bf16 *xTlo) {
    const int seg = threadIdx.x & 7, rp = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < Q / 64; ++i) {
        const int j = 2 * rp + 64 * i;
        const u32x4 r0 = r[2 * i], r1 = r[2 * i + 1];
        uint32_t *dst = reinterpret_cast<uint32_t *>(xT + seg * 8 * LD + j);
        if (w) {
            uint32_t *dlo = reinterpret_cast<uint32_t *>(xTlo + seg * 8 * LD + j);
            const float w0 = w[j], w1 = w[j + 1];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint32_t lo;
                dst[e * (LD / 2)] = split_pair(elem8(r0, e) * w0, elem8(r1, e) * w1, lo);
                dlo[e * (LD / 2)] = lo;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[e * (LD / 2)] = pair16(r0, r1, e);
        }
    }
}

// ------------------------------------------------------------ chunk state
// One block (4 waves) per (b, c, h).  S (64 x N fp32) = xw^T B with both
// operands staged transposed in LDS (the contraction runs over tokens, which
// are the rows in memory).  xw = x * w is formed in fp32 and carried as a
// hi/lo bf16 pair, so its rounding stays near fp32 level.  Output tiles
// 32x32: wave w owns tiles w and w+4 of the (p-tile, n-tile) grid.
template <int Q, int N>
__global__ void __launch_bounds__(256)
k_chunk_state_mfma(const bf16 *__restrict__ x, const bf16 *__restrict__ Bm,
                   const float *__restrict__ dt, const float *__restrict__ Acs,
                   float *__restrict__ states, int64_t L, int H, int G, int T) {
    constexpr int LD = Q + 8;
    __shared__ __attribute__((aligned(16))) bf16 xT[kP * LD];
    __shared__ __attribute__((aligned(16))) bf16 xTlo[kP * LD];
    __shared__ __attribute__((aligned(16))) bf16 BT[N * LD];
    __shared__ float w[Q];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.x % H;
    const int64_t bc = blockIdx.x / H;
    const int c = (int)(bc % T);
    const int64_t b = bc / T;
    const int g = h / (H / G);
    const int64_t t0 = (int64_t)c * Q;
    const int q = (int)min((int64_t)Q, L - t0);
    // issue every global load of the block first
    u32x4 xr[Q / 32];
    load_x_rows<Q>(xr, x + ((b * L + t0) * H + h) * kP, (int64_t)H * kP, q);
    constexpr int SEGS = N / 8, RP = 256 / SEGS, NB = Q / RP;  // NB rows per thread
    const int bseg = tid % SEGS, brp = tid / SEGS;
    const bf16 *brow0 = Bm + ((b * L + t0) * G + g) * N + bseg * 8;
    const int64_t brs = (int64_t)G * N;
    u32x4 br[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int j = 2 * brp + 2 * RP * (i >> 1) + (i & 1);
        br[i] = *reinterpret_cast<const u32x4 *>(brow0 + min(j, q - 1) * brs);
    }
    const float *acs = Acs + (b * H + h) * L + t0;
    const float last = acs[q - 1];
    for (int j = tid; j < Q; j += 256) {
        const int jj = min(j, q - 1);
        const float v = dt[(b * L + t0 + jj) * H + h] * ssd_exp(last - acs[jj]);
        w[j] = j < q ? v : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i)
        br[i] = masked(br[i], 2 * brp + 2 * RP * (i >> 1) + (i & 1) < q);
#pragma unroll
    for (int i = 0; i < NB / 2; ++i) {
        const int j = 2 * brp + 2 * RP * i;
        uint32_t *dst = reinterpret_cast<uint32_t *>(BT + bseg * 8 * LD + j);
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e * (LD / 2)] = pair16(br[2 * i], br[2 * i + 1], e);
    }
    __syncthreads();  // w complete
    store_x_transposed<Q, LD>(xr, xT, w, xTlo);
    __syncthreads();
    constexpr int NT = N / 32, TPW = (2 * NT) / 4;
    const int row = lane & 31, kh = (lane >> 5) * 8;
    f32x16 acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t] = zero16();
#pragma unroll 4
    for (int k0 = 0; k0 < Q; k0 += 16) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int tile = wave + 4 * t, pt = tile / NT, nt = tile % NT;
            const int ao = (pt * 32 + row) * LD + k0 + kh;
            const u32x4 a = *reinterpret_cast<const u32x4 *>(xT + ao);
            const u32x4 al = *reinterpret_cast<const u32x4 *>(xTlo + ao);
            const u32x4 bb = *reinterpret_cast<const u32x4 *>(BT + (nt * 32 + row) * LD + k0 + kh);
            acc[t] = mfma32(a, bb, acc[t]);
            acc[t] = mfma32(al, bb, acc[t]);
        }
    }
    float *out = states + ((b * T + c) * H + h) * (int64_t)(kP * N);
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int tile = wave + 4 * t, pt = tile / NT, nt = tile % NT;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int p = pt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            out[p * N + nt * 32 + row] = acc[t][r];
        }
    }
}

// ------------------------------------------------------------- chunk scan
// One block (4 waves) per (b, c, h); 32-row output tiles i, wave w owns tiles
// {w, NI-1-w} when the chunk has 8 tiles (equal causal work) and tile w
// otherwise.  Per output tile the wave computes Y^T (64 x 32, two
// accumulators over p):
//   off-diagonal j-tiles:  S^T = B_j C_i^T (MFMA), scaled per column j by
//       cf[j] = exp(Acs_k - Acs_j) dt_j with k the tile's first row, then
//       Y^T += X_j^T M^T;  afterwards Y^T *= exp(Acs_i - Acs_k) per row i;
//   state term:            Y^T += exp(Acs_i) H C_i^T;
//   diagonal j-tile:       M^T[j][i] = S^T exp(Acs_i - Acs_j) dt_j for j <= i;
//   epilogue:              y = Y + D x, rounded to bf16.
// Both exponent splits keep every exponent <= 0, so nothing overflows.  The
// operands formed inside the kernel (M and the entering state H) are carried
// as hi/lo bf16 pairs (two MFMAs each), so only x, B and C, which arrive in
// bf16, are single bf16 operands.
template <int Q, int N>
__global__ void __launch_bounds__(256)
k_chunk_scan_mfma(const bf16 *__restrict__ x, const float *__restrict__ dt,
                  const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm,
                  const float *__restrict__ D, const float *__restrict__ Acs,
                  const float *__restrict__ states, bf16 *__restrict__ y, int64_t L, int H, int G,
                  int T) {
    constexpr int NI = Q / 32;
    constexpr int LDX = Q + 8;
    constexpr int LDB = N + 8;
    constexpr int KS = N / 16;
    __shared__ __attribute__((aligned(16))) bf16 xT[kP * LDX];
    __shared__ __attribute__((aligned(16))) bf16 Bs[Q * LDB];
    __shared__ __attribute__((aligned(16))) bf16 Hs[kP * LDB];
    __shared__ __attribute__((aligned(16))) bf16 Hlo[kP * LDB];
    __shared__ __attribute__((aligned(16))) float acs_s[Q];
    __shared__ __attribute__((aligned(16))) float dt_s[Q];
    __shared__ __attribute__((aligned(16))) float cf[NI][Q];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.x % H;
    const int64_t bc = blockIdx.x / H;
    const int c = (int)(bc % T);
    const int64_t b = bc / T;
    const int g = h / (H / G);
    const int64_t t0 = (int64_t)c * Q;
    const int q = (int)min((int64_t)Q, L - t0);
    // issue every global load of the block first: x rows, B rows, entering state
    u32x4 xr[Q / 32];
    load_x_rows<Q>(xr, x + ((b * L + t0) * H + h) * kP, (int64_t)H * kP, q);
    constexpr int SEGS = N / 8, NB = Q * SEGS / 256, NH = kP * N / 4 / 256;
    const bf16 *brow0 = Bm + ((b * L + t0) * G + g) * N;
    const int64_t brs = (int64_t)G * N;
    u32x4 br[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int e = tid + 256 * i, j = e / SEGS, seg = e % SEGS;
        br[i] = *reinterpret_cast<const u32x4 *>(brow0 + min(j, q - 1) * brs + seg * 8);
    }
    const float *Hc = states + ((b * T + c) * H + h) * (int64_t)(kP * N);
    float4 hr[NH];
#pragma unroll
    for (int i = 0; i < NH; ++i) hr[i] = *reinterpret_cast<const float4 *>(Hc + 4 * (tid + 256 * i));
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
    store_x_transposed<Q, LDX>(xr, xT, nullptr, nullptr);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int e = tid + 256 * i, j = e / SEGS, seg = e % SEGS;
        *reinterpret_cast<u32x4 *>(Bs + j * LDB + seg * 8) = masked(br[i], j < q);
    }
#pragma unroll
    for (int i = 0; i < NH; ++i) {
        const int e = tid + 256 * i, p = e / (N / 4), n = (e % (N / 4)) * 4;
        uint32_t l0, l1;
        u32x2 pk, pl;
        pk[0] = split_pair(hr[i].x, hr[i].y, l0);
        pk[1] = split_pair(hr[i].z, hr[i].w, l1);
        pl[0] = l0;
        pl[1] = l1;
        *reinterpret_cast<u32x2 *>(Hs + p * LDB + n) = pk;
        *reinterpret_cast<u32x2 *>(Hlo + p * LDB + n) = pl;
    }
    __syncthreads();
    for (int e = tid; e < NI * Q; e += 256) {
        const int kt = e / Q, j = e % Q;
        cf[kt][j] = j < 32 * kt ? ssd_exp(acs_s[32 * kt] - acs_s[j]) * dt_s[j] : 0.f;
    }
    __syncthreads();

    const float Dh = D ? D[h] : 0.f;
    const int il = lane & 31, g2 = lane >> 5;
    const int ntiles = NI == 8 ? 2 : (wave < NI ? 1 : 0);
    for (int ti = 0; ti < ntiles; ++ti) {
        const int it = ti == 0 ? wave : NI - 1 - wave;
        const int i_loc = it * 32 + il;
        const int64_t tok = b * L + t0 + i_loc;
        u32x4 creg[KS];
        const int64_t ctok = b * L + t0 + min(i_loc, q - 1);
#pragma unroll
        for (int s = 0; s < KS; ++s)
            creg[s] = *reinterpret_cast<const u32x4 *>(Cm + (ctok * G + g) * N + 16 * s + 8 * g2);
#pragma unroll
        for (int s = 0; s < KS; ++s) creg[s] = masked(creg[s], i_loc < q);
        const float acs_i = acs_s[i_loc];
        const int k = it * 32;
        f32x16 yacc[2] = {zero16(), zero16()};
        // off-diagonal j-tiles (all j < k <= i)
        for (int jt = 0; jt < it; ++jt) {
            f32x16 s = zero16();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 a =
                    *reinterpret_cast<const u32x4 *>(Bs + (jt * 32 + il) * LDB + 16 * ks + 8 * g2);
                s = mfma32(a, creg[ks], s);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int jb = jt * 32 + 16 * u + 4 * g2;
                const float4 c0 = *reinterpret_cast<const float4 *>(&cf[it][jb]);
                const float4 c1 = *reinterpret_cast<const float4 *>(&cf[it][jb + 8]);
                float m[8] = {s[8 * u + 0] * c0.x, s[8 * u + 1] * c0.y, s[8 * u + 2] * c0.z,
                              s[8 * u + 3] * c0.w, s[8 * u + 4] * c1.x, s[8 * u + 5] * c1.y,
                              s[8 * u + 6] * c1.z, s[8 * u + 7] * c1.w};
                u32x4 bop, bopl;
                pack8_split(m, bop, bopl);
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) {
                    const bf16 *xr = xT + (pt * 32 + il) * LDX + jb;
                    const u32x2 lo = *reinterpret_cast<const u32x2 *>(xr);
                    const u32x2 hi = *reinterpret_cast<const u32x2 *>(xr + 8);
                    const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
                    yacc[pt] = mfma32(a, bop, yacc[pt]);
                    yacc[pt] = mfma32(a, bopl, yacc[pt]);
                }
            }
        }
        // state term
        f32x16 z[2] = {zero16(), zero16()};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                const int ho = (pt * 32 + il) * LDB + 16 * ks + 8 * g2;
                const u32x4 a = *reinterpret_cast<const u32x4 *>(Hs + ho);
                const u32x4 al = *reinterpret_cast<const u32x4 *>(Hlo + ho);
                z[pt] = mfma32(a, creg[ks], z[pt]);
                z[pt] = mfma32(al, creg[ks], z[pt]);
            }
        }
        const float ri = ssd_exp(acs_i - acs_s[k]);
        const float ei = ssd_exp(acs_i);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
            for (int r = 0; r < 16; ++r) yacc[pt][r] = yacc[pt][r] * ri + z[pt][r] * ei;
        // diagonal tile
        {
            f32x16 s = zero16();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 a =
                    *reinterpret_cast<const u32x4 *>(Bs + (k + il) * LDB + 16 * ks + 8 * g2);
                s = mfma32(a, creg[ks], s);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                float m[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int jl = 16 * u + 8 * (e >> 2) + 4 * g2 + (e & 3);
                    const int j = k + jl;
                    m[e] = jl <= il ? s[8 * u + e] * ssd_exp(acs_i - acs_s[j]) * dt_s[j] : 0.f;
                }
                u32x4 bop, bopl;
                pack8_split(m, bop, bopl);
                const int jb = k + 16 * u + 4 * g2;
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) {
                    const bf16 *xr = xT + (pt * 32 + il) * LDX + jb;
                    const u32x2 lo = *reinterpret_cast<const u32x2 *>(xr);
                    const u32x2 hi = *reinterpret_cast<const u32x2 *>(xr + 8);
                    const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
                    yacc[pt] = mfma32(a, bop, yacc[pt]);
                    yacc[pt] = mfma32(a, bopl, yacc[pt]);
                }
            }
        }
        // epilogue: lane holds row i_loc and p = pt*32 + 8*(r/4) + 4*g2 + r%4
        if (i_loc < q) {
            bf16 *yr = y + (tok * H + h) * kP;
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int p0 = pt * 32 + 8 * rg + 4 * g2;
                    float v[4];
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        const float xv = __uint_as_float((uint32_t)xT[(p0 + kk) * LDX + i_loc] << 16);
                        v[kk] = yacc[pt][4 * rg + kk] + Dh * xv;
                    }
                    u32x2 pk;
                    pk[0] = pack_bf16x2(v[0], v[1]);
                    pk[1] = pack_bf16x2(v[2], v[3]);
                    *reinterpret_cast<u32x2 *>(yr + p0) = pk;
                }
            }
        }
    }
}

template <int Q, int N>
void launch_state_t(const ScanShape &s, const void *x, const void *Bm, const float *dt,
                    const float *Acs, float *states, hipStream_t st) {
    k_chunk_state_mfma<Q, N><<<(unsigned)(s.B * s.T * s.H), 256, 0, st>>>(
        (const bf16 *)x, (const bf16 *)Bm, dt, Acs, states, s.L, (int)s.H, (int)s.G, (int)s.T);
}

template <int Q, int N>
void launch_scan_t(const ScanShape &s, const void *x, const float *dt, const void *Bm,
                   const void *Cm, const float *D, const float *Acs, const float *states, void *y,
                   hipStream_t st) {
    k_chunk_scan_mfma<Q, N><<<(unsigned)(s.B * s.T * s.H), 256, 0, st>>>(
        (const bf16 *)x, dt, (const bf16 *)Bm, (const bf16 *)Cm, D, Acs, states, (bf16 *)y, s.L,
        (int)s.H, (int)s.G, (int)s.T);
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
