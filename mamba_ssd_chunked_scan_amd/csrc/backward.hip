// Gradient of the chunked SSD scan: the per-chunk kernel.
//
// The forward pass is the chunked form of "Compiler-First State Space
// Duality and Portable O(1) Autoregressive Caching for Inference" (paperlayer
// summary, §3 Method, "Chunked recurrence"; the training comparison of §4
// runs forward and backward).  Inside chunk c, with Acs the within-chunk
// cumulative log-decay, L[i][j] = exp(Acs_i - Acs_j) for j <= i, CB[i][j] =
// C_i.B_j, H the state entering the chunk and E the derivative of the loss
// with respect to the state at its end:
//
//   y_i    = sum_{j<=i} CB[i][j] L[i][j] dt_j x_j + exp(Acs_i) H C_i + D x_i
//   H_next = exp(Acs_last) H + sum_j exp(Acs_last - Acs_j) dt_j x_j B_j^T
//
// Its derivatives, with K[i][j] = dy_i.x_j and GD[i][j] = CB[i][j] L[i][j] K[i][j]:
//
//   dx_j   = dt_j (sum_{i>=j} CB[i][j] L[i][j] dy_i + exp(Acs_last - Acs_j) E B_j) + D dy_j
//   dB_j  += dt_j (sum_{i>=j} L[i][j] K[i][j] C_i + exp(Acs_last - Acs_j) x_j^T E)
//   dC_i  += sum_{j<=i} L[i][j] K[i][j] dt_j B_j + exp(Acs_i) dy_i^T H
//   dAcs_t = sum_j GD[t][j] dt_j - dt_t sum_i GD[i][t]          (intra-chunk)
//          + exp(Acs_t) dy_t^T H C_t                              (state to output)
//          - s3_t + [t = last] (sum_j s3_j + exp(Acs_last) <E, H>) (chunk end state)
//   with s3_j = exp(Acs_last - Acs_j) dt_j x_j^T E B_j;
//   ddt_k  = A sum_{t>=k} dAcs_t + sum_i GD[i][k] + s3_j / dt_j at j = k
//   dA    += sum_t dAcs_t sum_{k<=t} dt_k,        dD += sum_i dy_i.x_i
//
// (Acs_t = A sum_{k<=t} dt_k, and dt also enters directly as the input
// weight).  H and E of every chunk come from the forward state pass and its
// reverse, run by the caller; the derivative with respect to H itself is
// carried by that reverse pass.
#include "common.hpp"
#include "launch.hpp"
#include "ssd.h"

namespace ssd {
namespace {

constexpr int kBQ = 32;         // tokens per gradient chunk
constexpr int kBThreads = 256;
constexpr int kMaxItems = 8;    // (row, 4 state elements) items per thread: 32 * 256 / 4 / 256

// LDS layout (floats): x, dy [Q][P+1]; B, C [Q][N+1]; CB L, K L, GD [Q][Q+1]
// (odd row strides: the 32 rows of a column fall in 32 different banks);
// 6 vectors of Q; 8 scratch; then the E / H slice buffer (at least 8N floats:
// it also holds the (N/4) x Q partial sums of two per-token reductions).
__host__ __device__ inline int64_t bwd_fixed_floats(int P, int N) {
    return 2LL * kBQ * (P + 1) + 2LL * kBQ * (N + 1) + 3LL * kBQ * (kBQ + 1) + 6 * kBQ + 8;
}

template <typename Tin>
__global__ void __launch_bounds__(kBThreads)
k_chunk_bwd(const Tin *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
            const Tin *__restrict__ Bm, const Tin *__restrict__ Cm, const float *__restrict__ D,
            const float *__restrict__ Acs, const float *__restrict__ Hs,
            const float *__restrict__ Es, const Tin *__restrict__ dy, Tin *__restrict__ dx,
            float *__restrict__ ddt, float *__restrict__ dB, float *__restrict__ dC,
            float *__restrict__ dA, float *__restrict__ dD, int64_t L, int H, int P, int N, int G,
            int T, int slice_rows) {
    constexpr int Q = kBQ, LQ = kBQ + 1;
    extern __shared__ __attribute__((aligned(16))) float sm[];
    const int PS = P + 1, NS = N + 1;
    float *bs = sm;                 // [Q][NS]
    float *cs = bs + Q * NS;        // [Q][NS]
    float *xs = cs + Q * NS;        // [Q][PS]
    float *ys = xs + Q * PS;        // dy [Q][PS]
    float *CBL = ys + Q * PS;       // [Q][LQ]
    float *KL = CBL + Q * LQ;       // [Q][LQ]
    float *GD = KL + Q * LQ;        // [Q][LQ]
    float *acs_s = GD + Q * LQ;     // [Q]
    float *dt_s = acs_s + Q;        // [Q]
    float *cdt_s = dt_s + Q;        // [Q] sum_{k<=t} dt_k
    float *s3d = cdt_s + Q;         // [Q] exp(Acs_last - Acs_j) x_j^T E B_j
    float *hq = s3d + Q;            // [Q] exp(Acs_i) dy_i^T H C_i
    float *rowg = hq + Q;           // [Q] sum_j GD[t][j] dt_j, then dAcs
    float *red = rowg + Q;          // [8]
    float *slab = sm + ((bwd_fixed_floats(P, N) + 3) & ~3LL);  // E or H rows, 16-byte aligned

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.x % H;
    const int64_t bc = blockIdx.x / H;
    const int c = (int)(bc % T);
    const int64_t b = bc / T;
    const int g = h / (H / G);
    const int64_t t0 = (int64_t)c * Q;
    const int q = (int)min((int64_t)Q, L - t0);
    const float a = A[h];
    const float Dh = D ? D[h] : 0.f;
    const int64_t xrow = (int64_t)H * P, brow = (int64_t)G * N, PN = (int64_t)P * N;
    const int64_t xo = ((b * L + t0) * H + h) * P;
    const int64_t bo = ((b * L + t0) * G + g) * N;
    const float *Hc = Hs + ((b * T + c) * H + h) * PN;
    const float *Ec = Es + ((b * T + c) * H + h) * PN;

    // ---- stage the chunk's rows (zeros past q) and its per-token scalars
    for (int e = tid; e < Q * P; e += kBThreads) {
        const int j = e / P, p = e - j * P;
        const bool ok = j < q;
        xs[j * PS + p] = ok ? Elem<Tin>::ld(x, xo + j * xrow + p) : 0.f;
        ys[j * PS + p] = ok ? Elem<Tin>::ld(dy, xo + j * xrow + p) : 0.f;
    }
    for (int e = tid; e < Q * N; e += kBThreads) {
        const int j = e / N, n = e - j * N;
        const bool ok = j < q;
        bs[j * NS + n] = ok ? Elem<Tin>::ld(Bm, bo + j * brow + n) : 0.f;
        cs[j * NS + n] = ok ? Elem<Tin>::ld(Cm, bo + j * brow + n) : 0.f;
    }
    if (wave == 0) {
        const float d = lane < q ? dt[(b * L + t0 + lane) * H + h] : 0.f;
        const float cd = wave_inclusive_scan(d, lane);
        if (lane < Q) {
            dt_s[lane] = d;
            cdt_s[lane] = cd;
            acs_s[lane] = lane < q ? Acs[(b * H + h) * L + t0 + lane] : 0.f;
            s3d[lane] = 0.f;
            hq[lane] = 0.f;
        }
    }
    __syncthreads();
    const float alast = acs_s[q - 1];

    // ---- the three masked Q x Q matrices
    for (int e = tid; e < Q * Q; e += kBThreads) {
        const int i = e / Q, j = e - i * Q;
        float cbl = 0.f, kl = 0.f, gd = 0.f;
        if (j <= i && i < q) {
            float cb = 0.f, k = 0.f;
            for (int n = 0; n < N; ++n) cb = fmaf(cs[i * NS + n], bs[j * NS + n], cb);
            for (int p = 0; p < P; ++p) k = fmaf(ys[i * PS + p], xs[j * PS + p], k);
            const float l = ssd_exp(acs_s[i] - acs_s[j]);
            cbl = cb * l;
            kl = k * l;
            gd = cb * kl;
        }
        CBL[i * LQ + j] = cbl;
        KL[i * LQ + j] = kl;
        GD[i * LQ + j] = gd;
    }
    __syncthreads();
    if (tid < Q) {  // row sums of GD dt (intra-chunk dAcs, + side)
        float r = 0.f;
        for (int j = 0; j <= tid; ++j) r = fmaf(GD[tid * LQ + j], dt_s[j], r);
        rowg[tid] = r;
    }

    // ---- E slices: dx, and x_j^T E for dB
    const int nq = N / 4;
    const int nitems = Q * nq;  // (row, 4 state elements)
    float4 acc4[kMaxItems];
#pragma unroll
    for (int k = 0; k < kMaxItems; ++k) acc4[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p0 = 0; p0 < P; p0 += slice_rows) {
        const int pr = min(slice_rows, P - p0);
        __syncthreads();  // the previous slice is no longer read
        for (int e = tid; e < pr * nq; e += kBThreads)
            reinterpret_cast<float4 *>(slab)[e] = reinterpret_cast<const float4 *>(Ec + p0 * N)[e];
        __syncthreads();
        // dx_j[p] for p in the slice
        for (int e = tid; e < Q * pr; e += kBThreads) {
            const int j = e % Q, pl = e / Q, p = p0 + pl;
            if (j >= q) continue;
            float intra = 0.f;
            for (int i = j; i < q; ++i) intra = fmaf(CBL[i * LQ + j], ys[i * PS + p], intra);
            float eb = 0.f;
            for (int n = 0; n < N; ++n) eb = fmaf(slab[pl * N + n], bs[j * NS + n], eb);
            const float v = dt_s[j] * (intra + ssd_exp(alast - acs_s[j]) * eb) + Dh * ys[j * PS + p];
            Elem<Tin>::st(dx, xo + j * xrow + p, v);
        }
        // x_j^T E, items (j, n4)
#pragma unroll
        for (int k = 0; k < kMaxItems; ++k) {
            const int e = tid + k * kBThreads;
            if (e < nitems) {
                const int j = e % Q, n4 = e / Q;
                float4 s = acc4[k];
                for (int pl = 0; pl < pr; ++pl) {
                    const float xv = xs[j * PS + p0 + pl];
                    const float4 ev = reinterpret_cast<const float4 *>(slab + pl * N)[n4];
                    s.x = fmaf(xv, ev.x, s.x);
                    s.y = fmaf(xv, ev.y, s.y);
                    s.z = fmaf(xv, ev.z, s.z);
                    s.w = fmaf(xv, ev.w, s.w);
                }
                acc4[k] = s;
            }
        }
    }
    // dB, and s3 (x_j^T E B_j); the slice buffer takes the s3 partials, so
    // every thread must be done with the last E slice first
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxItems; ++k) {
        const int e = tid + k * kBThreads;
        if (e < nitems) {
            const int j = e % Q, n4 = e / Q;
            if (j < q) {
                float4 intra = make_float4(0.f, 0.f, 0.f, 0.f);
                for (int i = j; i < q; ++i) {
                    const float kl = KL[i * LQ + j];
                    const float *cr = cs + i * NS + 4 * n4;
                    const float4 cv = make_float4(cr[0], cr[1], cr[2], cr[3]);
                    intra.x = fmaf(kl, cv.x, intra.x);
                    intra.y = fmaf(kl, cv.y, intra.y);
                    intra.z = fmaf(kl, cv.z, intra.z);
                    intra.w = fmaf(kl, cv.w, intra.w);
                }
                const float dtj = dt_s[j], f = ssd_exp(alast - acs_s[j]);
                const float4 xe = acc4[k];
                float *o = dB + bo + j * brow + 4 * n4;
                atomicAdd(o + 0, dtj * (intra.x + f * xe.x));
                atomicAdd(o + 1, dtj * (intra.y + f * xe.y));
                atomicAdd(o + 2, dtj * (intra.z + f * xe.z));
                atomicAdd(o + 3, dtj * (intra.w + f * xe.w));
                const float *br = bs + j * NS + 4 * n4;
                const float4 bv = make_float4(br[0], br[1], br[2], br[3]);
                slab[n4 * Q + j] = f * (xe.x * bv.x + xe.y * bv.y + xe.z * bv.z + xe.w * bv.w);
            }
        }
        acc4[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // s3 / dt_j per token: the partials summed in a fixed order (so ddt is the
    // same on every run)
    __syncthreads();
    if (tid < q) {
        float v = 0.f;
        for (int n4 = 0; n4 < nq; ++n4) v += slab[n4 * Q + tid];
        s3d[tid] = v;
    }

    // ---- H slices: dy_i^T H for dC
    for (int p0 = 0; p0 < P; p0 += slice_rows) {
        const int pr = min(slice_rows, P - p0);
        __syncthreads();
        for (int e = tid; e < pr * nq; e += kBThreads)
            reinterpret_cast<float4 *>(slab)[e] = reinterpret_cast<const float4 *>(Hc + p0 * N)[e];
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kMaxItems; ++k) {
            const int e = tid + k * kBThreads;
            if (e < nitems) {
                const int i = e % Q, n4 = e / Q;
                float4 s = acc4[k];
                for (int pl = 0; pl < pr; ++pl) {
                    const float yv = ys[i * PS + p0 + pl];
                    const float4 hv = reinterpret_cast<const float4 *>(slab + pl * N)[n4];
                    s.x = fmaf(yv, hv.x, s.x);
                    s.y = fmaf(yv, hv.y, s.y);
                    s.z = fmaf(yv, hv.z, s.z);
                    s.w = fmaf(yv, hv.w, s.w);
                }
                acc4[k] = s;
            }
        }
    }
    // dC, and the state-to-output term of dAcs (partials into the slice buffer
    // once every thread is done with the last H slice)
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxItems; ++k) {
        const int e = tid + k * kBThreads;
        if (e < nitems) {
            const int i = e % Q, n4 = e / Q;
            if (i < q) {
                float4 intra = make_float4(0.f, 0.f, 0.f, 0.f);
                for (int j = 0; j <= i; ++j) {
                    const float w = KL[i * LQ + j] * dt_s[j];
                    const float *br = bs + j * NS + 4 * n4;
                    const float4 bv = make_float4(br[0], br[1], br[2], br[3]);
                    intra.x = fmaf(w, bv.x, intra.x);
                    intra.y = fmaf(w, bv.y, intra.y);
                    intra.z = fmaf(w, bv.z, intra.z);
                    intra.w = fmaf(w, bv.w, intra.w);
                }
                const float ei = ssd_exp(acs_s[i]);
                const float4 yh = acc4[k];
                float *o = dC + bo + i * brow + 4 * n4;
                atomicAdd(o + 0, intra.x + ei * yh.x);
                atomicAdd(o + 1, intra.y + ei * yh.y);
                atomicAdd(o + 2, intra.z + ei * yh.z);
                atomicAdd(o + 3, intra.w + ei * yh.w);
                const float *cr = cs + i * NS + 4 * n4;
                const float4 cv = make_float4(cr[0], cr[1], cr[2], cr[3]);
                slab[n4 * Q + i] = ei * (yh.x * cv.x + yh.y * cv.y + yh.z * cv.z + yh.w * cv.w);
            }
        }
    }
    __syncthreads();  // the partials written
    if (tid < q) {
        float v = 0.f;
        for (int n4 = 0; n4 < nq; ++n4) v += slab[n4 * Q + tid];
        hq[tid] = v;
    }

    // ---- <E, H>
    float eh = 0.f;
    for (int64_t e = tid; e < PN / 4; e += kBThreads) {
        const float4 ev = reinterpret_cast<const float4 *>(Ec)[e];
        const float4 hv = reinterpret_cast<const float4 *>(Hc)[e];
        eh += ev.x * hv.x + ev.y * hv.y + ev.z * hv.z + ev.w * hv.w;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) eh += __shfl_xor(eh, off, kWave);
    if (lane == 0) red[wave] = eh;
    __syncthreads();

    // ---- per-token scalars: dAcs, ddt, dA, dD (wave 0, lane t = token)
    if (wave == 0) {
        const float EH = red[0] + red[1] + red[2] + red[3];
        const int t = lane;
        const bool in = t < q;
        float colgd = 0.f, s3 = 0.f, dacs = 0.f, kdiag = 0.f;
        if (in) {
            for (int i = t; i < q; ++i) colgd += GD[i * LQ + t];
            s3 = s3d[t] * dt_s[t];
            dacs = rowg[t] - dt_s[t] * colgd + hq[t] - s3;
            kdiag = KL[t * LQ + t];
        }
        // sum_j s3_j goes to the last token, with exp(Acs_last) <E, H>
        float s3sum = s3;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) s3sum += __shfl_xor(s3sum, off, kWave);
        if (t == q - 1) dacs += s3sum + ssd_exp(alast) * EH;
        // suffix sums of dAcs over the chunk (lanes >= q hold 0)
        float suf = dacs;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const float o = __shfl_down(suf, d, kWave);
            if (t + d < kWave) suf += o;
        }
        if (in) ddt[(b * L + t0 + t) * H + h] = a * suf + colgd + (in ? s3d[t] : 0.f);
        float da = in ? dacs * cdt_s[t] : 0.f;
        float dd = kdiag;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            da += __shfl_xor(da, off, kWave);
            dd += __shfl_xor(dd, off, kWave);
        }
        if (lane == 0) {
            atomicAdd(&dA[h], da);
            if (dD) atomicAdd(&dD[h], dd);
        }
    }
}

// Rows of E / H per slice so that the whole block fits the 160 KB of LDS
// (at most 16 KB of slice, at least one row).
int bwd_slice_rows(int P, int N, size_t *lds_bytes) {
    const int64_t fixed = (bwd_fixed_floats(P, N) + 3) & ~3LL;
    int64_t budget = (160 * 1024) / 4 - fixed;
    int64_t rows = min((int64_t)P, min((int64_t)(4096 / N), budget / N));
    if (rows < 1) rows = 1;
    *lds_bytes = (size_t)(fixed + max(rows, (int64_t)8) * N) * 4;
    return (int)rows;
}

template <typename Tin>
void launch_bwd_t(const ScanShape &s, const void *x, const float *dt, const float *A,
                  const void *Bm, const void *Cm, const float *D, const float *Acs,
                  const float *Hs, const float *Es, const void *dy, void *dx, float *ddt,
                  float *dB, float *dC, float *dA, float *dD, hipStream_t st) {
    size_t lds = 0;
    const int rows = bwd_slice_rows((int)s.P, (int)s.N, &lds);
    static bool attr_set = false;  // once per instantiation (per process)
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_chunk_bwd<Tin>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        attr_set = true;
    }
    k_chunk_bwd<Tin><<<(unsigned)(s.B * s.T * s.H), kBThreads, lds, st>>>(
        (const Tin *)x, dt, A, (const Tin *)Bm, (const Tin *)Cm, D, Acs, Hs, Es,
        (const Tin *)dy, (Tin *)dx, ddt, dB, dC, dA, dD, s.L, (int)s.H, (int)s.P, (int)s.N,
        (int)s.G, (int)s.T, rows);
}

}  // namespace

void launch_chunk_bwd(const ScanShape &s, const void *x, const float *dt, const float *A,
                      const void *Bm, const void *Cm, const float *D, const float *Acs,
                      const float *Hs, const float *Es, const void *dy, void *dx, float *ddt,
                      float *dB, float *dC, float *dA, float *dD, hipStream_t st) {
    if (s.dtype == SSD_BF16)
        launch_bwd_t<bf16>(s, x, dt, A, Bm, Cm, D, Acs, Hs, Es, dy, dx, ddt, dB, dC, dA, dD, st);
    else
        launch_bwd_t<float>(s, x, dt, A, Bm, Cm, D, Acs, Hs, Es, dy, dx, ddt, dB, dC, dA, dD, st);
}

}  // namespace ssd
