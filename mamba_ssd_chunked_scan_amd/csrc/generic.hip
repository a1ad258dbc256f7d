// Generic kernels of the chunked SSD scan and the decode step.
//
// These handle every supported shape and both storage dtypes with fp32 VALU
// arithmetic.  They are the fp32 path and the fallback for shapes the MFMA
// kernels do not tile; the chunk-cumsum and state-passing kernels here serve
// every path.  The stages follow the chunked algorithm of "Compiler-First
// State Space Duality and Portable O(1) Autoregressive Caching for Inference"
// (paperlayer summary, §3 Method, "Chunked recurrence"; contractions of B.5):
// a within-chunk cumulative log-decay, each chunk's own state, a sequential
// pass of states across chunks, and the chunk output from its diagonal block
// plus the entering state.
#include <algorithm>

#include <type_traits>

#include "common.hpp"
#include "stages.hpp"
#include "launch.hpp"
#include "ssd.h"

namespace ssd {
namespace {

// ---------------------------------------------------------------- cumsum
// Acs[b,h,t] = within-chunk inclusive cumsum of dt*A.  One block per
// (batch, chunk) and 4 heads, one wave per head: each lane holds Q/64
// consecutive tokens (summed sequentially), and the lane totals are combined
// with a wave prefix scan.  All products and sums are fp32.  With an active
// dt activation the activated dt is used and, when dt_out is given, written
// there (same layout as dt) for the later stages.
__global__ void __launch_bounds__(256)
k_chunk_cumsum(const float *__restrict__ dt, const float *__restrict__ A,
               float *__restrict__ Acs, int64_t L, int H, int Q, int T, DtAct act,
               float *__restrict__ dt_out, const int2 *__restrict__ ctab) {
    const int64_t b = blockIdx.x / T;
    const int c = blockIdx.x % T;
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
    if (h >= H) return;  // wave-uniform
    const ChunkPos cp = chunk_pos(ctab, c, Q, L);
    const int64_t t0 = cp.t0;
    const int q = cp.q;
    if (q <= 0) return;
    const int E = Q >= 64 ? Q / 64 : 1;  // tokens per lane (<= 4)
    const float a = A[h];
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = lane * E + k;
        v[k] = 0.f;
        if (k < E && i < q) {
            const int64_t di = (b * L + t0 + i) * H + h;
            const float d = act_dt(act, dt[di], h);
            if (dt_out) dt_out[di] = d;
            v[k] = d * a;
        }
    }
    float run = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        run += v[k];
        v[k] = run;
    }
    const float incl = wave_inclusive_scan(run, lane);
    float excl = __shfl_up(incl, 1, kWave);
    if (lane == 0) excl = 0.f;
    float *out = Acs + (b * H + h) * L + t0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = lane * E + k;
        if (k < E && i < q) out[i] = v[k] + excl;
    }
}

// ---------------------------------------------------------- chunk state
// states[b,c,h,p,n] = sum_j x[j,p] * w_j * B[j,n],  w_j = dt_j exp(Acs_last - Acs_j).
// kAdjoint (the gradient's chunk term, with x = dy and B = C): w_j = exp(Acs_j),
// the decay from the chunk's entering state to token j.
// One block per (b, c, h) and PB = min(P, 4096/N) rows of p; each thread
// owns a 4 x 4 (p, n) tile.  The chunk streams through LDS 32 tokens at a
// time (x rows restricted to the block's p range, whole B rows, both fp32),
// so each token costs a thread two 16-byte LDS reads for 16 FMAs.
constexpr int kStateJT = 32;

template <typename Tin, bool kAdjoint = false, typename TX = Tin>
__global__ void __launch_bounds__(256)
k_chunk_state_generic(const TX *__restrict__ x, const Tin *__restrict__ Bm,
                      const float *__restrict__ dt, const float *__restrict__ Acs,
                      float *__restrict__ states, int64_t L, int H, int P, int N, int G, int Q,
                      int T, const int2 *__restrict__ ctab) {
    __shared__ float w[256];
    extern __shared__ __attribute__((aligned(16))) float st_sm[];
    const int h = blockIdx.x % H;
    const int64_t bc = blockIdx.x / H;
    const int c = (int)(bc % T);
    const int64_t b = bc / T;
    const int g = h / (H / G);
    const ChunkPos cp = chunk_pos(ctab, c, Q, L);
    const int64_t t0 = cp.t0;
    const int q = cp.q;
    if (q <= 0) return;
    const int PB = min(P, 4096 / N);          // rows of p in this block
    const int p0 = blockIdx.y * PB;
    const int pb = min(PB, P - p0);
    const int PBS = (PB + 3) & ~3;            // LDS row stride of x (16-byte rows)
    float *xs = st_sm;                        // [JT][PBS]
    float *bs = xs + kStateJT * PBS;          // [JT][N]
    const float *acs = Acs + (b * H + h) * L + t0;
    const float last = acs[q - 1];
    for (int j = threadIdx.x; j < q; j += 256)
        w[j] = kAdjoint ? ssd_exp(acs[j]) : dt[(b * L + t0 + j) * H + h] * ssd_exp(last - acs[j]);
    const int nq = N / 4;
    const int ni = threadIdx.x % nq, pi = threadIdx.x / nq;
    const bool active = 4 * pi < pb;
    float acc[4][4] = {};
    const int64_t xrow = (int64_t)H * P, brow = (int64_t)G * N;
    const TX *xb = x + ((b * L + t0) * H + h) * P + p0;
    const Tin *bb = Bm + ((b * L + t0) * G + g) * N;
    for (int j0 = 0; j0 < q; j0 += kStateJT) {
        const int jn = min(kStateJT, q - j0);
        __syncthreads();  // w ready / the previous tile no longer read
        for (int e = threadIdx.x; e < jn * PBS; e += 256) {
            const int j = e / PBS, pl = e - j * PBS;
            xs[e] = pl < pb ? Elem<TX>::ld(xb, (j0 + j) * xrow + pl) : 0.f;
        }
        for (int e = threadIdx.x; e < jn * N; e += 256) {
            const int j = e / N, n = e - j * N;
            bs[e] = Elem<Tin>::ld(bb, (j0 + j) * brow + n);
        }
        __syncthreads();
        if (active) {
            for (int j = 0; j < jn; ++j) {
                const float wj = w[j0 + j];
                const float4 xv = *reinterpret_cast<const float4 *>(&xs[j * PBS + 4 * pi]);
                const float4 bv = *reinterpret_cast<const float4 *>(&bs[j * N + 4 * ni]);
                const float xw[4] = {xv.x * wj, xv.y * wj, xv.z * wj, xv.w * wj};
                const float bb4[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int k = 0; k < 4; ++k) acc[a][k] = fmaf(xw[a], bb4[k], acc[a][k]);
            }
        }
    }
    if (!active) return;
    float *out = states + (((b * T + c) * H + h) * (int64_t)P + p0 + 4 * pi) * N + 4 * ni;
#pragma unroll
    for (int a = 0; a < 4; ++a)
        if (4 * pi + a < pb)
            *reinterpret_cast<float4 *>(out + (int64_t)a * N) =
                make_float4(acc[a][0], acc[a][1], acc[a][2], acc[a][3]);
}

// LDS bytes and grid of k_chunk_state_generic.
size_t state_generic_lds(const ScanShape &s) {
    const int64_t PB = std::min<int64_t>(s.P, 4096 / s.N);
    return (size_t)kStateJT * (((PB + 3) & ~3LL) + s.N) * 4;
}
dim3 state_generic_grid(const ScanShape &s) {
    const int64_t PB = std::min<int64_t>(s.P, 4096 / s.N);
    return dim3((unsigned)(s.B * s.T * s.H), (unsigned)((s.P + PB - 1) / PB));
}

// -------------------------------------------------------- state passing
// One thread per 4 consecutive state elements of one (b, h).
__global__ void __launch_bounds__(256)
k_state_passing(float *__restrict__ states, const float *__restrict__ Acs,
                const float *init, float *fin, int64_t L, int H, int64_t PN, int Q, int T,
                const int2 *__restrict__ ctab, const int2 *__restrict__ sch) {
    const int64_t e = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 4;
    if (e >= PN) return;
    state_passing_body(states, Acs, init, fin, blockIdx.x, e, L, H, PN, Q, T, ctab, sch);
}

// Reverse pass of the gradient's chunk terms: per (b, h) and 4 consecutive
// state elements, from the last chunk to the first, E <- dfinal (or 0); slot
// c receives E, the derivative with respect to the state at the end of chunk
// c, then E <- exp(Acs at the end of chunk c) E + dS_c (the derivative with
// respect to the state entering chunk c).  What is left is the derivative
// with respect to the initial state.  Loads run kPassAhead chunks ahead.
__global__ void __launch_bounds__(256)
k_state_passing_rev(float *__restrict__ ds, const float *__restrict__ Acs,
                    const float *__restrict__ dfin, float *__restrict__ dinit, int64_t L, int H,
                    int64_t PN, int Q, int T, const int2 *__restrict__ ctab,
                    const int2 *__restrict__ sch) {
    const int64_t e = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 4;
    if (e >= PN) return;
    // a row: a batch row (slots b T .. b T + T - 1) or a sequence of a
    // variable-length batch (its slots from sch, chunk ends from ctab)
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / H;
    const int h = (int)(bh % H);
    int64_t k0;
    int n;
    const float *acs;
    if (sch) {
        const int2 r = sch[b];
        k0 = r.x;
        n = r.y;
        acs = Acs + (int64_t)h * L;
    } else {
        k0 = b * T;
        n = T;
        acs = Acs + bh * L;
    }
    float4 E = make_float4(0.f, 0.f, 0.f, 0.f);
    if (dfin) E = *reinterpret_cast<const float4 *>(dfin + bh * PN + e);
    const int64_t cstride = (int64_t)H * PN;
    float *base = ds + (k0 * H + h) * PN + e;
    for (int c0 = n - 1; c0 >= 0; c0 -= kPassAhead) {
        float4 sv[kPassAhead];
        float r[kPassAhead];
#pragma unroll
        for (int k = 0; k < kPassAhead; ++k) {
            const int c = c0 - k;
            if (c >= 0) {
                sv[k] = *reinterpret_cast<const float4 *>(base + c * cstride);
                int64_t last;
                if (ctab) {
                    const int2 cp = ctab[k0 + c];
                    last = (int64_t)cp.x + cp.y - 1;
                } else {
                    last = min(L, (int64_t)(c + 1) * Q) - 1;
                }
                r[k] = ssd_exp(acs[last]);
            }
        }
#pragma unroll
        for (int k = 0; k < kPassAhead; ++k) {
            const int c = c0 - k;
            if (c >= 0) {
                *reinterpret_cast<float4 *>(base + c * cstride) = E;
                E.x = r[k] * E.x + sv[k].x;
                E.y = r[k] * E.y + sv[k].y;
                E.z = r[k] * E.z + sv[k].z;
                E.w = r[k] * E.w + sv[k].w;
            }
        }
    }
    if (dinit) *reinterpret_cast<float4 *>(dinit + bh * PN + e) = E;
}

// ----------------------------------------------------------- chunk scan
constexpr int kScanRows = 16;

// CB[i][j] = C_i . B_j in fp32 for one (b, c, g) and a tile of 16 rows i, every
// column j <= i, into the lower triangle of the chunk stored row after row
// (row i at i(i+1)/2, Q(Q+1)/2 values per (b, c, g)).  It does not involve
// the head, so it is formed once here and read by every head of the group.  C rows of the tile and 16 B rows at a
// time are staged in LDS; each thread forms one (i, j) dot product in the
// order n = 0..N-1.
template <typename Tin>
__global__ void __launch_bounds__(256)
k_chunk_cb_generic(const Tin *__restrict__ Bm, const Tin *__restrict__ Cm, float *__restrict__ cb,
                   int64_t L, int N, int G, int Q, int T, const int2 *__restrict__ ctab) {
    __shared__ float Cs[kScanRows][257];
    __shared__ float Bs[kScanRows][257];
    const int64_t bcg = blockIdx.x;
    const int g = (int)(bcg % G);
    const int64_t bc = bcg / G;
    const int c = (int)(bc % T);
    const int64_t b = bc / T;
    const ChunkPos cp = chunk_pos(ctab, c, Q, L);
    const int64_t t0 = cp.t0;
    const int q = cp.q;
    const int i0 = blockIdx.y * kScanRows;
    if (i0 >= q) return;
    const int rows = min(kScanRows, q - i0);
    for (int e = threadIdx.x; e < kScanRows * N; e += 256) {
        const int ii = e / N, n = e % N;
        Cs[ii][n] = ii < rows ? Elem<Tin>::ld(Cm, ((b * L + t0 + i0 + ii) * G + g) * N + n) : 0.f;
    }
    const int ii = threadIdx.x / kScanRows, jj = threadIdx.x % kScanRows;
    const int64_t irow = i0 + ii;
    float *out = cb + bcg * ((int64_t)Q * (Q + 1) / 2) + irow * (irow + 1) / 2;
    const int jend = i0 + rows;  // columns j < jend can be needed
    for (int j0 = 0; j0 < jend; j0 += kScanRows) {
        __syncthreads();  // Cs staged; the previous B rows no longer read
        for (int e = threadIdx.x; e < kScanRows * N; e += 256) {
            const int r = e / N, n = e % N;
            Bs[r][n] = j0 + r < jend ? Elem<Tin>::ld(Bm, ((b * L + t0 + j0 + r) * G + g) * N + n)
                                     : 0.f;
        }
        __syncthreads();
        const int j = j0 + jj;
        if (ii < rows && j <= i0 + ii) {
            float dot = 0.f;
            for (int n = 0; n < N; ++n) dot += Cs[ii][n] * Bs[jj][n];
            out[j] = dot;
        }
    }
}

// One block per (b, c, h) and 16 output rows.  M[i][j] = CB[i][j] exp(Acs_i -
// Acs_j) dt_j for j <= i is built in LDS from the group's C.B buffer, then
// each output (i, p) is sum_j M[i][j] x[j,p] + exp(Acs_i) (C_i . H_c[p]) +
// D x[i,p].

template <typename Tin>
__global__ void __launch_bounds__(256)
k_chunk_scan_generic(const Tin *__restrict__ x, const float *__restrict__ dt,
                     const Tin *__restrict__ Bm, const Tin *__restrict__ Cm,
                     const float *__restrict__ D, const float *__restrict__ Acs,
                     const float *__restrict__ states, const float *__restrict__ cbuf,
                     Tin *__restrict__ y, const Tin *__restrict__ z, int64_t L, int H, int P,
                     int N, int G, int Q, int T, const int2 *__restrict__ ctab) {
    __shared__ float Ms[kScanRows][257];
    __shared__ float Cs[kScanRows][257];
    __shared__ float acs_s[256];
    __shared__ float dt_s[256];
    const int h = blockIdx.x % H;
    const int64_t bc = blockIdx.x / H;
    const int c = (int)(bc % T);
    const int64_t b = bc / T;
    const int g = h / (H / G);
    const ChunkPos cp = chunk_pos(ctab, c, Q, L);
    const int64_t t0 = cp.t0;
    const int q = cp.q;
    const int i0 = blockIdx.y * kScanRows;
    if (i0 >= q) return;
    const int rows = min(kScanRows, q - i0);
    for (int j = threadIdx.x; j < q; j += 256) {
        acs_s[j] = Acs[(b * H + h) * L + t0 + j];
        dt_s[j] = dt[(b * L + t0 + j) * H + h];
    }
    for (int e = threadIdx.x; e < kScanRows * N; e += 256) {
        const int ii = e / N, n = e % N;
        Cs[ii][n] = ii < rows ? Elem<Tin>::ld(Cm, ((b * L + t0 + i0 + ii) * G + g) * N + n) : 0.f;
    }
    __syncthreads();
    const int jmax = i0 + rows;  // columns j < jmax can be non-zero
    const float *cbr = cbuf + ((b * T + c) * G + g) * ((int64_t)Q * (Q + 1) / 2);
    (void)Bm;  // B enters through the group's C.B buffer
    for (int e = threadIdx.x; e < kScanRows * jmax; e += 256) {
        const int ii = e / jmax, j = e % jmax;
        const int i = i0 + ii;
        float m = 0.f;
        if (ii < rows && j <= i) m = cbr[(int64_t)i * (i + 1) / 2 + j] * ssd_exp(acs_s[i] - acs_s[j]) * dt_s[j];
        Ms[ii][j] = m;
    }
    __syncthreads();
    const float Dh = D ? D[h] : 0.f;
    const float *Hc = states + ((b * T + c) * H + h) * (int64_t)P * N;
    // each work item is one channel p and four rows ii0..ii0+3: every x and H
    // value it loads feeds four rows.  Row i sums j = 0..i only (a later
    // token's x never enters an earlier output, even through a 0 weight),
    // in the order j = 0.., n = 0..; C rows past the chunk are 0.
    constexpr int kRq = 4;
    for (int e = threadIdx.x; e < (kScanRows / kRq) * P; e += 256) {
        const int p = e % P, ii0 = (e / P) * kRq;
        if (ii0 >= rows) continue;
        float acc[kRq] = {0.f, 0.f, 0.f, 0.f}, off[kRq] = {0.f, 0.f, 0.f, 0.f};
        const int ifirst = i0 + ii0;  // the first row of the item: j <= ifirst serves all four
        for (int j = 0; j <= ifirst; ++j) {
            const float xv = Elem<Tin>::ld(x, ((b * L + t0 + j) * H + h) * P + p);
#pragma unroll
            for (int r = 0; r < kRq; ++r) acc[r] += Ms[ii0 + r][j] * xv;
        }
        for (int j = ifirst + 1; j < min(jmax, ifirst + kRq); ++j) {
            const float xv = Elem<Tin>::ld(x, ((b * L + t0 + j) * H + h) * P + p);
#pragma unroll
            for (int r = 1; r < kRq; ++r)
                if (j <= ifirst + r) acc[r] += Ms[ii0 + r][j] * xv;
        }
        const float *hr = Hc + (int64_t)p * N;
        for (int n = 0; n < N; ++n) {
            const float hv = hr[n];
#pragma unroll
            for (int r = 0; r < kRq; ++r) off[r] += Cs[ii0 + r][n] * hv;
        }
#pragma unroll
        for (int r = 0; r < kRq; ++r) {
            const int ii = ii0 + r, i = i0 + ii;
            if (ii >= rows) break;
            const int64_t xi = ((b * L + t0 + i) * H + h) * P + p;
            float yv = acc[r] + ssd_exp(acs_s[i]) * off[r] + Dh * Elem<Tin>::ld(x, xi);
            if (z) yv *= silu_f(Elem<Tin>::ld(z, xi));
            Elem<Tin>::st(y, xi, yv);
        }
    }
}

// ------------------------------------------------- variable-length batches
// Chunk table of a packed batch of NS sequences from cu[0..NS] (the token
// offsets of the sequences).  Sequence s covers tokens [cu[s], cu[s+1]) and
// is cut into ceil(len/Q) chunks from its own first token, so no chunk spans
// two sequences and every sequence starts from its own state.  Its chunks
// take consecutive slots in sequence order: ctab[slot] = {first token,
// length}, sch[s] = {first slot, slots}; slots past the last chunk get
// length 0.  Offsets are clamped into [0, total] and slots past the end of
// the table are dropped, so no offsets can lead a later kernel outside the
// packed arrays (results for offsets that are not non-decreasing from 0 to
// total are unspecified).  One block: each thread takes a contiguous range
// of sequences, and a block prefix sum of the per-thread chunk counts places
// them.
__global__ void __launch_bounds__(1024)
k_varlen_table(const int32_t *__restrict__ cu, int NS, int total, int Q, int slots,
               int2 *__restrict__ ctab, int2 *__restrict__ sch, int2 *__restrict__ spos) {
    __shared__ int64_t wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (NS + 1023) / 1024;
    const int s0 = min(NS, tid * per), s1 = min(NS, s0 + per);
    auto start = [&](int s) { return min(max(cu[s], 0), total); };
    auto length = [&](int s) { return max(0, min(cu[s + 1], total) - start(s)); };
    // counts are 64-bit: offsets that overlap can add up to more than 2^31
    int64_t cnt = 0;
    for (int s = s0; s < s1; ++s) cnt += (length(s) + Q - 1) / Q;
    int64_t v = cnt;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int64_t o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int64_t first = v - cnt, nall = 0;
    for (int w = 0; w < 16; ++w) {
        if (w < wave) first += wsum[w];
        nall += wsum[w];
    }
    for (int s = s0; s < s1; ++s) {
        const int t0 = start(s), len = length(s), nk = (len + Q - 1) / Q;
        const int64_t room = max((int64_t)0, (int64_t)slots - first);
        sch[s] = make_int2((int)min(first, (int64_t)slots), (int)min((int64_t)nk, room));
        for (int j = 0; j < nk && j < room; ++j) {
            ctab[first + j] = make_int2(t0 + j * Q, min(Q, len - j * Q));
            if (spos) spos[first + j] = make_int2(s, j);
        }
        first += nk;
    }
    for (int64_t k = nall + tid; k < slots; k += 1024) {
        ctab[k] = make_int2(0, 0);
        if (spos) spos[k] = make_int2(-1, 0);
    }
}

// ----------------------------------------------------------- misc
// Final states of the sequences of a variable-length batch that have no
// tokens (no chunk slot): their init state passes through (zeros without
// one).  Grid-stride over (sequence, 4 state values).
__global__ void k_empty_finals(const int2 *__restrict__ sch, int64_t NS, const float *init,
                               float *fin, int64_t per) {
    const int64_t n4 = NS * (per / 4);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t s = i / (per / 4);
        if (sch[s].y != 0) continue;
        const int64_t e = i * 4;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (init) v = *reinterpret_cast<const float4 *>(init + e);
        *reinterpret_cast<float4 *>(fin + e) = v;
    }
}

__global__ void k_copy_or_zero(float *dst, const float *src, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

// ---------------------------------------------------------- decode step
// Each thread owns 4 consecutive state elements of one (b,h,p) row; the N/4
// lanes of a row are adjacent in the wave and reduce C.s with xor shuffles.
template <typename Tin>
__device__ __forceinline__ void ld4(const Tin *p, int64_t i, float v[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = Elem<Tin>::ld(p, i + k);
}

// One token on this thread's 4 state elements: s <- r s + u B, returns the
// partial C.s.  Written with explicit fused multiply-adds so that every
// kernel using it performs the same operations in the same order.
__device__ __forceinline__ float step_update(float4 &s, float r, float u, const float bv[4],
                                             const float cv[4]) {
    s.x = fmaf(r, s.x, u * bv[0]);
    s.y = fmaf(r, s.y, u * bv[1]);
    s.z = fmaf(r, s.z, u * bv[2]);
    s.w = fmaf(r, s.w, u * bv[3]);
    return fmaf(cv[3], s.w, fmaf(cv[2], s.z, fmaf(cv[1], s.y, cv[0] * s.x)));
}

template <typename Tin>
__global__ void __launch_bounds__(256)
k_step(float *__restrict__ state, const Tin *__restrict__ x, const float *__restrict__ dt,
       const float *__restrict__ A, const Tin *__restrict__ Bm, const Tin *__restrict__ Cm,
       const float *__restrict__ D, Tin *__restrict__ y, int64_t rows, int H, int P, int N,
       int G, int lpr_log2, DtAct act, const Tin *__restrict__ z) {
    const int lpr = 1 << lpr_log2;
    const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gt >> lpr_log2;
    const int sub = (int)(gt & (lpr - 1));
    const bool active = row < rows;
    float part = 0.f, xv = 0.f;
    int h = 0;
    if (active) {
        const int64_t bh = row / P;
        h = (int)(bh % H);
        const int64_t b = bh / H;
        const int g = h / (H / G);
        const float d = act_dt(act, dt[b * H + h], h);
        const float r = ssd_exp(d * A[h]);
        xv = Elem<Tin>::ld(x, row);
        const float u = d * xv;
        float4 *sp = reinterpret_cast<float4 *>(state + row * N) + sub;
        float4 s = *sp;
        float bv[4], cv[4];
        ld4(Bm, (b * G + g) * N + sub * 4, bv);
        ld4(Cm, (b * G + g) * N + sub * 4, cv);
        part = step_update(s, r, u, bv, cv);
        *sp = s;
    }
    for (int off = lpr >> 1; off > 0; off >>= 1) part += __shfl_xor(part, off, kWave);
    if (active && sub == 0) {
        float yv = fmaf(D ? D[h] : 0.f, xv, part);
        if (z) yv *= silu_f(Elem<Tin>::ld(z, row));
        Elem<Tin>::st(y, row, yv);
    }
}

// One token with 16 state values per lane: the float4 groups sub, sub+L,
// sub+2L and sub+3L of a row's N/4 groups, L = N/16 lanes per row.  Four
// 16-byte state loads per lane are in flight at once (k_step has one), which
// is what the state stream needs to approach the HBM rate when it is not in a
// cache.  The lane adds its four partials as (g0 + g2) + (g1 + g3) and then
// butterflies over its L lanes: exactly the pairing of k_step's butterfly
// over N/4 lanes (its first two levels pair g with g ^ 2L and then with
// g ^ L), so y and the state are bit for bit those of k_step.  N >= 16.
template <typename Tin>
__global__ void __launch_bounds__(256)
k_step_wide(float *__restrict__ state, const Tin *__restrict__ x, const float *__restrict__ dt,
            const float *__restrict__ A, const Tin *__restrict__ Bm, const Tin *__restrict__ Cm,
            const float *__restrict__ D, Tin *__restrict__ y, int64_t rows, int H, int P, int N,
            int G, int l_log2, DtAct act, const Tin *__restrict__ z) {
    const int L = 1 << l_log2;
    const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gt >> l_log2;
    const int sub = (int)(gt & (L - 1));
    const bool active = row < rows;
    float part = 0.f, xv = 0.f;
    int h = 0;
    if (active) {
        const int64_t bh = row / P;
        h = (int)(bh % H);
        const int64_t b = bh / H;
        const int g = h / (H / G);
        const float d = act_dt(act, dt[b * H + h], h);
        const float r = ssd_exp(d * A[h]);
        xv = Elem<Tin>::ld(x, row);
        const float u = d * xv;
        float4 *sp = reinterpret_cast<float4 *>(state + row * N) + sub;
        float4 sv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) sv[k] = sp[k * L];
        const int64_t bc = (b * G + g) * N + sub * 4;
        float pk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float bv[4], cv[4];
            ld4(Bm, bc + (int64_t)k * L * 4, bv);
            ld4(Cm, bc + (int64_t)k * L * 4, cv);
            pk[k] = step_update(sv[k], r, u, bv, cv);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) sp[k * L] = sv[k];
        part = (pk[0] + pk[2]) + (pk[1] + pk[3]);
    }
    for (int off = L >> 1; off > 0; off >>= 1) part += __shfl_xor(part, off, kWave);
    if (active && sub == 0) {
        float yv = fmaf(D ? D[h] : 0.f, xv, part);
        if (z) yv *= silu_f(Elem<Tin>::ld(z, row));
        Elem<Tin>::st(y, row, yv);
    }
}


// nsteps consecutive decode tokens in one launch.  Same thread layout and
// per-token arithmetic as k_step (so the result equals nsteps chained steps
// bit for bit), but the thread's 4 state elements stay in registers across
// the tokens: the state is read and written once per launch instead of once
// per token.  Inputs are in the prefill layout ([B, nsteps, ...]); the next
// token's inputs are loaded while the current one is applied.
template <typename Tin>
__global__ void __launch_bounds__(256)
k_step_multi(float *__restrict__ state, const Tin *__restrict__ x, const float *__restrict__ dt,
             const float *__restrict__ A, const Tin *__restrict__ Bm, const Tin *__restrict__ Cm,
             const float *__restrict__ D, Tin *__restrict__ y, int64_t rows, int64_t nsteps,
             int H, int P, int N, int G, int lpr_log2, DtAct act, const Tin *__restrict__ z) {
    const int lpr = 1 << lpr_log2;
    const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gt >> lpr_log2;
    const int sub = (int)(gt & (lpr - 1));
    const bool active = row < rows;
    // inactive lanes follow row 0's addresses so that every lane takes part
    // in the row reductions; they load but never store
    const int64_t rr = active ? row : 0;
    const int64_t bh = rr / P;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const int p = (int)(rr % P);
    const int g = h / (H / G);
    const float a = A[h];
    const float Dh = D ? D[h] : 0.f;
    // per-token strides in the [B, nsteps, ...] layouts
    const int64_t xs = (int64_t)H * P, ds = H, bs = (int64_t)G * N;
    const Tin *xp = x + (b * nsteps * H + h) * P + p;
    const float *dp = dt + b * nsteps * H + h;
    const Tin *bp = Bm + (b * nsteps * G + g) * N + sub * 4;
    const Tin *cp = Cm + (b * nsteps * G + g) * N + sub * 4;
    Tin *yp = y + (b * nsteps * H + h) * P + p;
    const Tin *zp = z ? z + (b * nsteps * H + h) * P + p : nullptr;
    float4 *sp = reinterpret_cast<float4 *>(state + rr * N) + sub;
    float4 s = *sp;
    float xv = 0.f, d = 0.f, bv[4], cv[4];
    if (nsteps > 0) {
        xv = Elem<Tin>::ld(xp, 0);
        d = act_dt(act, dp[0], h);
        ld4(bp, 0, bv);
        ld4(cp, 0, cv);
    }
    for (int64_t t = 0; t < nsteps; ++t) {
        // next token's inputs (clamped to the last token: loaded, not used)
        const int64_t tn = t + 1 < nsteps ? t + 1 : t;
        const float xn = Elem<Tin>::ld(xp, tn * xs), dn = act_dt(act, dp[tn * ds], h);
        float bn[4], cn[4];
        ld4(bp, tn * bs, bn);
        ld4(cp, tn * bs, cn);
        const float r = ssd_exp(d * a);
        const float u = d * xv;
        float part = step_update(s, r, u, bv, cv);
        for (int off = lpr >> 1; off > 0; off >>= 1) part += __shfl_xor(part, off, kWave);
        if (active && sub == 0) {
            float yv = fmaf(Dh, xv, part);
            if (z) yv *= silu_f(Elem<Tin>::ld(zp, t * xs));
            Elem<Tin>::st(yp, t * xs, yv);
        }
        xv = xn;
        d = dn;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            bv[k] = bn[k];
            cv[k] = cn[k];
        }
    }
    if (active) *sp = s;
}

// k_step_multi for blocks whose rows all belong to one (b, h).  A lane keeps
// 16 state elements of its row (L = N/16 lanes per row): the float4 groups
// sub, sub+L, sub+2L, sub+3L of the N/4 groups that k_step spreads over N/4
// lanes.  Adding those four partials as (g0 + g2) + (g1 + g3) and then
// butterflying over the L lanes pairs the same values in the same order as
// k_step's butterfly over N/4 lanes, so every token's y and the final state
// are bit for bit those of chained k_step calls.  Per group of KC tokens the
// block stages B and C of its group, x of its rows, the decay exp(dt*A) and
// dt*x in LDS with one burst of loads, keeps y in LDS and writes it out
// coalesced: the token loop makes no global memory access.
template <typename Tin, int KC, int L>
__global__ void __launch_bounds__(256)
k_step_multi_lds(float *__restrict__ state, const Tin *__restrict__ x,
                 const float *__restrict__ dt, const float *__restrict__ A,
                 const Tin *__restrict__ Bm, const Tin *__restrict__ Cm,
                 const float *__restrict__ D, Tin *__restrict__ y, int64_t nsteps, int H, int P,
                 int G, DtAct act, const Tin *__restrict__ z) {
    constexpr int N = 16 * L;
    constexpr int RPB = 256 / L < 64 ? 256 / L : 64;  // rows per block
    __shared__ float4 bs_[KC][N / 4], cs_[KC][N / 4];
    __shared__ float xs_[KC][RPB], us_[KC][RPB], ys_[KC][RPB];
    __shared__ float rs_[KC];
    const int tid = threadIdx.x;
    const int sub = tid % L, rl = tid / L;
    const int64_t row0 = (int64_t)blockIdx.x * RPB;  // all RPB rows share (b, h)
    const int64_t bh = row0 / P;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const int p0 = (int)(row0 % P);
    const int g = h / (H / G);
    const float a = A[h];
    const float Dh = D ? D[h] : 0.f;
    const int64_t xst = (int64_t)H * P, bst = (int64_t)G * N;
    const Tin *xb = x + (b * nsteps * H + h) * P + p0;
    const float *db = dt + b * nsteps * H + h;
    const Tin *bb = Bm + (b * nsteps * G + g) * N;
    const Tin *cb = Cm + (b * nsteps * G + g) * N;
    Tin *yb = y + (b * nsteps * H + h) * P + p0;
    const Tin *zb = z ? z + (b * nsteps * H + h) * P + p0 : nullptr;
    float4 *sp = reinterpret_cast<float4 *>(state + (row0 + rl) * N) + sub;
    float4 s[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] = sp[j * L];
    for (int64_t t0 = 0; t0 < nsteps; t0 += KC) {
        const int kc = (int)min((int64_t)KC, nsteps - t0);
        __syncthreads();  // the previous group's y has been written out
        float *bsf = reinterpret_cast<float *>(bs_), *csf = reinterpret_cast<float *>(cs_);
        for (int e = tid; e < kc * N; e += RPB * L) {
            const int t = e / N, n = e - t * N;
            bsf[e] = Elem<Tin>::ld(bb, (t0 + t) * bst + n);
            csf[e] = Elem<Tin>::ld(cb, (t0 + t) * bst + n);
        }
        for (int e = tid; e < kc * RPB; e += RPB * L) {
            const int t = e / RPB, r = e - t * RPB;
            const float xv = Elem<Tin>::ld(xb, (t0 + t) * xst + r);
            xs_[t][r] = xv;
            us_[t][r] = act_dt(act, db[(t0 + t) * H], h) * xv;
        }
        if (tid < kc) rs_[tid] = ssd_exp(act_dt(act, db[(t0 + tid) * H], h) * a);
        __syncthreads();
        for (int t = 0; t < kc; ++t) {
            const float r = rs_[t], u = us_[t][rl];
            float q[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 b4 = bs_[t][sub + j * L], c4 = cs_[t][sub + j * L];
                const float bv[4] = {b4.x, b4.y, b4.z, b4.w}, cv[4] = {c4.x, c4.y, c4.z, c4.w};
                q[j] = step_update(s[j], r, u, bv, cv);
            }
            float part = (q[0] + q[2]) + (q[1] + q[3]);
#pragma unroll
            for (int off = L >> 1; off > 0; off >>= 1) part += __shfl_xor(part, off, kWave);
            if (sub == 0) ys_[t][rl] = fmaf(Dh, xs_[t][rl], part);
        }
        __syncthreads();
        for (int e = tid; e < kc * RPB; e += RPB * L) {
            const int t = e / RPB, r = e - t * RPB;
            float yv = ys_[t][r];
            if (z) yv *= silu_f(Elem<Tin>::ld(zb, (t0 + t) * xst + r));
            Elem<Tin>::st(yb, (t0 + t) * xst + r, yv);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) sp[j * L] = s[j];
}

template <typename Tin, int L>
void launch_multi_lds(const StepShape &s, int64_t nsteps, float *state, const void *x,
                      const float *dt, const float *A, const void *Bm, const void *Cm,
                      const float *D, void *y, const DtAct &act, const void *z, hipStream_t st) {
    constexpr int RPB = 256 / L < 64 ? 256 / L : 64;
    const unsigned blocks = (unsigned)(s.B * s.H * s.P / RPB);
    k_step_multi_lds<Tin, 16, L><<<blocks, RPB * L, 0, st>>>(
        state, (const Tin *)x, dt, A, (const Tin *)Bm, (const Tin *)Cm, D, (Tin *)y, nsteps,
        (int)s.H, (int)s.P, (int)s.G, act, (const Tin *)z);
}

// Rows per block of k_step_multi_lds for a state size (0: not handled there).
int multi_lds_rows(int64_t N) {
    switch (N) {
    case 16: case 32: case 64: return 64;
    case 128: return 32;
    case 256: return 16;
    default: return 0;
    }
}

template <typename Tin>
void launch_multi_lds_n(const StepShape &s, int64_t nsteps, float *state, const void *x,
                        const float *dt, const float *A, const void *Bm, const void *Cm,
                        const float *D, void *y, const DtAct &act, const void *z,
                        hipStream_t st) {
#define SSD_MULTI_L(LL) \
    launch_multi_lds<Tin, LL>(s, nsteps, state, x, dt, A, Bm, Cm, D, y, act, z, st)
    switch (s.N) {
    case 16: SSD_MULTI_L(1); break;
    case 32: SSD_MULTI_L(2); break;
    case 64: SSD_MULTI_L(4); break;
    case 128: SSD_MULTI_L(8); break;
    default: SSD_MULTI_L(16); break;
    }
#undef SSD_MULTI_L
}

template <typename Tin>
void launch_step_t(const StepShape &s, int64_t nsteps, float *state, const void *x,
                   const float *dt, const float *A, const void *Bm, const void *Cm,
                   const float *D, void *y, const DtAct &act, const void *z, hipStream_t st) {
    const int64_t rows = s.B * s.H * s.P;
    int lpr_log2 = 0;
    while ((4LL << lpr_log2) < s.N) ++lpr_log2;  // lanes per row = N / 4
    const unsigned blocks = (unsigned)(((rows << lpr_log2) + 255) / 256);
    if (nsteps < 0 && s.N >= 16) {  // a single step, 16 state values per lane
        const int l_log2 = lpr_log2 - 2;
        const unsigned wblocks = (unsigned)(((rows << l_log2) + 255) / 256);
        k_step_wide<Tin><<<wblocks, 256, 0, st>>>(state, (const Tin *)x, dt, A,
                                                  (const Tin *)Bm, (const Tin *)Cm, D, (Tin *)y,
                                                  rows, (int)s.H, (int)s.P, (int)s.N, (int)s.G,
                                                  l_log2, act, (const Tin *)z);
        return;
    }
    if (nsteps < 0) {  // a single step, [B, ...] layouts
        k_step<Tin><<<blocks, 256, 0, st>>>(state, (const Tin *)x, dt, A, (const Tin *)Bm,
                                            (const Tin *)Cm, D, (Tin *)y, rows, (int)s.H,
                                            (int)s.P, (int)s.N, (int)s.G, lpr_log2, act,
                                            (const Tin *)z);
        return;
    }
    const int rpb = multi_lds_rows(s.N);
    if (rpb > 0 && s.P % rpb == 0) {  // each block's rows share one (b, h): stage in LDS
        launch_multi_lds_n<Tin>(s, nsteps, state, x, dt, A, Bm, Cm, D, y, act, z, st);
        return;
    }
    k_step_multi<Tin><<<blocks, 256, 0, st>>>(state, (const Tin *)x, dt, A, (const Tin *)Bm,
                                              (const Tin *)Cm, D, (Tin *)y, rows, nsteps,
                                              (int)s.H, (int)s.P, (int)s.N, (int)s.G, lpr_log2,
                                              act, (const Tin *)z);
}

// ------------------------------------------------------------- gated norm
// One block per (token, norm group) pair (grid-stride over the pairs), a
// fixed reduction order (lanes, then the four waves in turn), no workspace:
// the call repeats bit for bit.  kVec: the group's CG channels (a multiple of
// 8, at most 8 * 256 * kVecK) are read once as 8-element vectors into
// registers, summed, scaled and written back; otherwise they are read twice
// element by element.
constexpr int kVecK = 4;

template <typename T, bool kVec>
__global__ void __launch_bounds__(256)
k_gated_norm(T *__restrict__ y, const float *__restrict__ w, float eps, int64_t pairs,
             int64_t HP, int CG, int NG) {
    __shared__ float part[4];
    const int tid = threadIdx.x;
    for (int64_t pr = blockIdx.x; pr < pairs; pr += gridDim.x) {
        const int64_t tok = pr / NG;
        const int k = (int)(pr - tok * NG);
        T *row = y + tok * HP + (int64_t)k * CG;
        const float *wr = w + (int64_t)k * CG;
        float ss = 0.f;
        float v[kVec ? kVecK : 1][8];
        if constexpr (kVec) {
#pragma unroll
            for (int u = 0; u < kVecK; ++u) {
                const int c = 8 * (tid + 256 * u);
                if (c < CG) {
                    ld8(row + c, v[u]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) ss = fmaf(v[u][e], v[u][e], ss);
                }
            }
        } else {
            for (int c = tid; c < CG; c += 256) {
                const float x = Elem<T>::ld(row, c);
                ss = fmaf(x, x, ss);
            }
        }
        ss = wave_sum_dpp(ss);
        if ((tid & 63) == 0) part[tid >> 6] = ss;
        __syncthreads();
        const float tot = ((part[0] + part[1]) + part[2]) + part[3];
        const float r = 1.f / sqrtf(tot / (float)CG + eps);
        if constexpr (kVec) {
#pragma unroll
            for (int u = 0; u < kVecK; ++u) {
                const int c = 8 * (tid + 256 * u);
                if (c < CG) {
                    const float4 wa = *reinterpret_cast<const float4 *>(wr + c);
                    const float4 wb = *reinterpret_cast<const float4 *>(wr + c + 4);
                    const float ww[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[u][e] = v[u][e] * r * ww[e];
                    st8(row + c, v[u]);
                }
            }
        } else {
            for (int c = tid; c < CG; c += 256) Elem<T>::st(row, c, Elem<T>::ld(row, c) * r * wr[c]);
        }
        __syncthreads();  // part[] is reused by the next pair
    }
}

}  // namespace

// ------------------------------------------------------------ launchers
void launch_chunk_cumsum(const ScanShape &s, const float *dt, const float *A, float *Acs,
                         hipStream_t st, const DtAct &act, float *dt_out) {
    dim3 grid((unsigned)(s.B * s.T), (unsigned)((s.H + 3) / 4));
    k_chunk_cumsum<<<grid, 256, 0, st>>>(dt, A, Acs, s.L, (int)s.H, (int)s.Q, (int)s.T, act,
                                         dt_out, s.ctab);
}

void launch_chunk_state(const ScanShape &s, const void *x, const void *Bm, const float *dt,
                        const float *Acs, float *states, hipStream_t st) {
    if (mfma_supported(s)) {
        launch_chunk_state_mfma(s, x, Bm, dt, Acs, states, st);
        return;
    }
    const dim3 grid = state_generic_grid(s);
    const size_t lds = state_generic_lds(s);
    if (s.dtype == SSD_BF16)
        k_chunk_state_generic<bf16><<<grid, 256, lds, st>>>(
            (const bf16 *)x, (const bf16 *)Bm, dt, Acs, states, s.L, (int)s.H, (int)s.P,
            (int)s.N, (int)s.G, (int)s.Q, (int)s.T, s.ctab);
    else
        k_chunk_state_generic<float><<<grid, 256, lds, st>>>(
            (const float *)x, (const float *)Bm, dt, Acs, states, s.L, (int)s.H, (int)s.P,
            (int)s.N, (int)s.G, (int)s.Q, (int)s.T, s.ctab);
}

void launch_chunk_dstate(const ScanShape &s, const void *dy, const void *Cm, const float *Acs,
                         float *dstates, hipStream_t st, bool dy_f32) {
    const dim3 grid = state_generic_grid(s);
    const size_t lds = state_generic_lds(s);
    if (s.dtype == SSD_BF16 && dy_f32)
        k_chunk_state_generic<bf16, true, float><<<grid, 256, lds, st>>>(
            (const float *)dy, (const bf16 *)Cm, nullptr, Acs, dstates, s.L, (int)s.H, (int)s.P,
            (int)s.N, (int)s.G, (int)s.Q, (int)s.T, s.ctab);
    else if (s.dtype == SSD_BF16)
        k_chunk_state_generic<bf16, true><<<grid, 256, lds, st>>>(
            (const bf16 *)dy, (const bf16 *)Cm, nullptr, Acs, dstates, s.L, (int)s.H, (int)s.P,
            (int)s.N, (int)s.G, (int)s.Q, (int)s.T, s.ctab);
    else
        k_chunk_state_generic<float, true><<<grid, 256, lds, st>>>(
            (const float *)dy, (const float *)Cm, nullptr, Acs, dstates, s.L, (int)s.H, (int)s.P,
            (int)s.N, (int)s.G, (int)s.Q, (int)s.T, s.ctab);
}

void launch_state_passing_rev(const ScanShape &s, float *dstates, const float *Acs,
                              const float *dfin, float *dinit, hipStream_t st) {
    const int64_t PN = s.P * s.N;
    const int64_t rows = s.sch ? s.NS : s.B;  // batch rows, or sequences
    if (rows == 0) return;
    dim3 grid((unsigned)(rows * s.H), (unsigned)((PN / 4 + 255) / 256));
    k_state_passing_rev<<<grid, 256, 0, st>>>(dstates, Acs, dfin, dinit, s.L, (int)s.H, PN,
                                               (int)s.Q, (int)s.T, s.ctab, s.sch);
}

void launch_state_passing(const ScanShape &s, float *states, const float *Acs,
                          const float *init, float *fin, hipStream_t st) {
    const int64_t PN = s.P * s.N;
    const int64_t rows = s.sch ? s.NS : s.B;  // batch rows, or sequences
    if (rows == 0) return;
    dim3 grid((unsigned)(rows * s.H), (unsigned)((PN / 4 + 255) / 256));
    k_state_passing<<<grid, 256, 0, st>>>(states, Acs, init, fin, s.L, (int)s.H, PN,
                                           (int)s.Q, (int)s.T, s.ctab, s.sch);
}

size_t chunk_scan_ws_bytes(const ScanShape &s) {
    // the MFMA kernels' tiles, or the lower triangle of a Q x Q fp32 C.B
    // matrix per (b, c, g)
    return mfma_supported(s) ? chunk_cb_bytes(s)
                             : (size_t)(s.B * s.T * s.G) * (size_t)(s.Q * (s.Q + 1) / 2) * 4;
}

void launch_chunk_cb(const ScanShape &s, const void *Bm, const void *Cm, void *ws, hipStream_t st) {
    if (mfma_supported(s)) {
        launch_chunk_cb_mfma(s, Bm, Cm, ws, st);
        return;
    }
    if (s.B * s.T * s.G == 0) return;
    dim3 grid((unsigned)(s.B * s.T * s.G), (unsigned)((s.Q + kScanRows - 1) / kScanRows));
    if (s.dtype == SSD_BF16)
        k_chunk_cb_generic<bf16><<<grid, 256, 0, st>>>((const bf16 *)Bm, (const bf16 *)Cm,
                                                        (float *)ws, s.L, (int)s.N, (int)s.G,
                                                        (int)s.Q, (int)s.T, s.ctab);
    else
        k_chunk_cb_generic<float><<<grid, 256, 0, st>>>((const float *)Bm, (const float *)Cm,
                                                         (float *)ws, s.L, (int)s.N, (int)s.G,
                                                         (int)s.Q, (int)s.T, s.ctab);
}

void launch_chunk_scan(const ScanShape &s, const void *x, const float *dt, const void *Bm,
                       const void *Cm, const float *D, const float *Acs, const float *states,
                       const void *ws, void *y, hipStream_t st, const void *z) {
    if (mfma_supported(s)) {
        launch_chunk_scan_mfma(s, x, dt, Cm, D, Acs, states, ws, y, st, z);
        return;
    }
    dim3 grid((unsigned)(s.B * s.T * s.H), (unsigned)((s.Q + kScanRows - 1) / kScanRows));
    if (s.dtype == SSD_BF16)
        k_chunk_scan_generic<bf16><<<grid, 256, 0, st>>>(
            (const bf16 *)x, dt, (const bf16 *)Bm, (const bf16 *)Cm, D, Acs, states,
            (const float *)ws, (bf16 *)y, (const bf16 *)z, s.L, (int)s.H, (int)s.P, (int)s.N,
            (int)s.G, (int)s.Q, (int)s.T, s.ctab);
    else
        k_chunk_scan_generic<float><<<grid, 256, 0, st>>>(
            (const float *)x, dt, (const float *)Bm, (const float *)Cm, D, Acs, states,
            (const float *)ws, (float *)y, (const float *)z, s.L, (int)s.H, (int)s.P, (int)s.N,
            (int)s.G, (int)s.Q, (int)s.T, s.ctab);
}

void launch_varlen_table(const int32_t *cu, int64_t NS, int64_t total, int64_t Q, int64_t slots,
                         int2 *ctab, int2 *sch, int2 *spos, hipStream_t st) {
    k_varlen_table<<<1, 1024, 0, st>>>(cu, (int)NS, (int)total, (int)Q, (int)slots, ctab, sch,
                                       spos);
}

void launch_gated_norm(void *y, const float *w, float eps, int64_t ntok, int64_t H, int64_t P,
                       int64_t NG, int dtype, hipStream_t st) {
    const int64_t pairs = ntok * NG;
    if (pairs <= 0) return;
    const unsigned blocks = (unsigned)(pairs < 16384 ? pairs : 16384);
    const int CG = (int)(H / NG * P);
    // vectors: groups of whole 8-channel runs (P % 8 == 0 keeps every group
    // and row start 16-byte aligned, y and w being so) that fit the registers
    const bool vec = P % 8 == 0 && CG <= 8 * 256 * kVecK;
#define SSD_NORM(T_, V_)                                                                     \
    k_gated_norm<T_, V_><<<blocks, 256, 0, st>>>(static_cast<T_ *>(y), w, eps, pairs, H * P, \
                                                 CG, (int)NG)
    if (dtype == SSD_BF16) {
        if (vec) SSD_NORM(bf16, true);
        else SSD_NORM(bf16, false);
    } else {
        if (vec) SSD_NORM(float, true);
        else SSD_NORM(float, false);
    }
#undef SSD_NORM
}

void launch_empty_finals(const int2 *sch, int64_t NS, const float *init, float *fin,
                         int64_t per, hipStream_t st) {
    if (!fin || NS <= 0) return;
    const int64_t n4 = NS * (per / 4);
    const unsigned blocks = (unsigned)(n4 / 256 + 1 < 4096 ? n4 / 256 + 1 : 4096);
    k_empty_finals<<<blocks, 256, 0, st>>>(sch, NS, init, fin, per);
}

// Zero up to four fp32 buffers in one launch (null pointers are skipped).
struct ZeroSet {
    float *p[4];
    int64_t n[4];
};

__global__ void k_zero_set(ZeroSet z) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int k = 0; k < 4; ++k) {
        if (!z.p[k]) continue;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < z.n[k]; i += stride)
            z.p[k][i] = 0.f;
    }
}

void launch_zero4(float *a, int64_t na, float *b, int64_t nb, float *c, int64_t nc, float *d,
                  int64_t nd, hipStream_t st) {
    ZeroSet z{{a, b, c, d}, {a ? na : 0, b ? nb : 0, c ? nc : 0, d ? nd : 0}};
    int64_t m = 0;
    for (int k = 0; k < 4; ++k) m = z.n[k] > m ? z.n[k] : m;
    if (m == 0) return;
    const int64_t blocks = (m + 255) / 256;
    k_zero_set<<<(unsigned)(blocks < 4096 ? blocks : 4096), 256, 0, st>>>(z);
}

void launch_copy_or_zero(float *dst, const float *src, int64_t n, hipStream_t st) {
    if (n <= 0 || dst == src) return;
    k_copy_or_zero<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(dst, src, n);
}

void launch_step(const StepShape &s, int64_t nsteps, float *state, const void *x,
                 const float *dt, const float *A, const void *Bm, const void *Cm, const float *D,
                 void *y, const DtAct &act, const void *z, hipStream_t st) {
    if (s.dtype == SSD_BF16)
        launch_step_t<bf16>(s, nsteps, state, x, dt, A, Bm, Cm, D, y, act, z, st);
    else
        launch_step_t<float>(s, nsteps, state, x, dt, A, Bm, Cm, D, y, act, z, st);
}

}  // namespace ssd
