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
constexpr int kHeadsPerBlock = 4;

// LDS layout (floats), rows padded to multiples of 4 plus 4 (16-byte rows,
// staggered banks): B, C [Q][NS]; x, dy [Q][PS]; CB, CB L, K L, GD [Q][LQ];
// 6 vectors of Q; 2 x 4 x Q cross-wave partials; 8 scratch; then the E / H
// slice buffer.
__host__ __device__ inline int bwd_ps(int P) { return ((P + 3) & ~3) + 4; }
__host__ __device__ inline int bwd_ns(int N) { return N + 4; }
constexpr int kLQ = kBQ + 4;
__host__ __device__ inline int64_t bwd_fixed_floats(int P, int N) {
    return 2LL * kBQ * bwd_ns(N) + 2LL * kBQ * bwd_ps(P) + 4LL * kBQ * kLQ + 6 * kBQ +
           8 * kBQ + 8;
}

__device__ __forceinline__ float4 f4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ void fma4(float4 &acc, float a, const float4 &b) {
    acc.x = fmaf(a, b.x, acc.x);
    acc.y = fmaf(a, b.y, acc.y);
    acc.z = fmaf(a, b.z, acc.z);
    acc.w = fmaf(a, b.w, acc.w);
}
__device__ __forceinline__ float dot4(const float4 &a, const float4 &b) {
    return fmaf(a.x, b.x, fmaf(a.y, b.y, fmaf(a.z, b.z, a.w * b.w)));
}

// One block per (b, c, group, slice of kHeadsPerBlock heads of the group).
// KI = ceil(N / 32): (token, 4 state elements) items per thread.
template <typename Tin, int KI>
__global__ void __launch_bounds__(kBThreads)
k_chunk_bwd(const Tin *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
            const Tin *__restrict__ Bm, const Tin *__restrict__ Cm, const float *__restrict__ D,
            const float *__restrict__ Acs, const float *__restrict__ Hs,
            const float *__restrict__ Es, const Tin *__restrict__ dy, Tin *__restrict__ dx,
            float *__restrict__ ddt, float *__restrict__ dB, float *__restrict__ dC,
            float *__restrict__ dA, float *__restrict__ dD, int64_t L, int H, int P, int N, int G,
            int T, int slice_rows) {
    constexpr int Q = kBQ, LQ = kLQ;
    extern __shared__ __attribute__((aligned(16))) float sm[];
    const int PS = bwd_ps(P), NS = bwd_ns(N);
    float *bs = sm;                  // [Q][NS]
    float *cs = bs + Q * NS;         // [Q][NS]
    float *xs = cs + Q * NS;         // [Q][PS]
    float *ys = xs + Q * PS;         // dy [Q][PS]
    float *CB = ys + Q * PS;         // [Q][LQ]  C_i.B_j (all i, j)
    float *CBL = CB + Q * LQ;        // [Q][LQ]  CB L, j <= i < q
    float *KL = CBL + Q * LQ;        // [Q][LQ]  (dy_i.x_j) L
    float *GD = KL + Q * LQ;         // [Q][LQ]  CB KL
    float *acs_s = GD + Q * LQ;      // [Q]
    float *dt_s = acs_s + Q;         // [Q]
    float *cdt_s = dt_s + Q;         // [Q] sum_{k<=t} dt_k
    float *rowg = cdt_s + Q;         // [Q] sum_j GD[t][j] dt_j
    float *colg = rowg + Q;          // [Q] sum_i GD[i][t]
    float *s3h = colg + Q;           // [Q] exp(Acs_last - Acs_j) x_j^T E B_j, then exp(Acs_i) dy_i^T H C_i
    float *part = s3h + Q;           // [2][4][Q] cross-wave partials
    float *red = part + 8 * Q;       // [8]
    float *slab = sm + ((bwd_fixed_floats(P, N) + 3) & ~3LL);  // E or H rows [slice][N]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = H / G, nslices = (R + kHeadsPerBlock - 1) / kHeadsPerBlock;
    int64_t rest = blockIdx.x;
    const int hsl = (int)(rest % nslices);
    rest /= nslices;
    const int g = (int)(rest % G);
    rest /= G;
    const int c = (int)(rest % T);
    const int64_t b = rest / T;
    const int h0 = g * R + hsl * kHeadsPerBlock;
    const int nh = min(kHeadsPerBlock, g * R + R - h0);
    const int64_t t0 = (int64_t)c * Q;
    const int q = (int)min((int64_t)Q, L - t0);
    const int64_t xrow = (int64_t)H * P, brow = (int64_t)G * N, PN = (int64_t)P * N;
    const int64_t bo = ((b * L + t0) * G + g) * N;
    const int nq = N / 4;
    const int nitems = Q * nq;
    // item k of this thread: token j = tid % Q, state elements 4 (tid / Q + 8 k) ..
    const int jt = tid % Q, nq0 = tid / Q;
    // E / H slices move through registers: the next slice's loads are issued
    // before the current slice is used (a slice is at most 2048 floats, two
    // float4 per thread)
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    auto load_slice = [&](const float *src, int p0, float4 (&pf)[2]) __attribute__((always_inline)) {
        const int n = min(slice_rows, P - p0) * nq;
        const float4 *s4 = reinterpret_cast<const float4 *>(src + (int64_t)p0 * N);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = tid + k * kBThreads;
            pf[k] = e < n ? s4[e] : z4;
        }
    };
    auto store_slice = [&](const float4 (&pf)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 2; ++k) reinterpret_cast<float4 *>(slab)[tid + k * kBThreads] = pf[k];
    };

    // ---- B and C of the chunk (shared by the block's heads) and C.B
    for (int e = tid; e < Q * NS; e += kBThreads) {
        const int j = e / NS, n = e - j * NS;
        const bool ok = j < q && n < N;
        bs[e] = ok ? Elem<Tin>::ld(Bm, bo + j * brow + n) : 0.f;
        cs[e] = ok ? Elem<Tin>::ld(Cm, bo + j * brow + n) : 0.f;
    }
    __syncthreads();
    {  // 1 x 4 tile per thread: row i, columns 4 jq ..
        const int i = tid >> 3, j0 = 4 * (tid & 7);
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int n = 0; n < N; n += 4) {
            const float4 cv = f4(cs + i * NS + n);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += dot4(cv, f4(bs + (j0 + r) * NS + n));
        }
        *reinterpret_cast<float4 *>(CB + i * LQ + j0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }

    float4 dbacc[KI], dcacc[KI];
#pragma unroll
    for (int k = 0; k < KI; ++k) {
        dbacc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        dcacc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    for (int hh = 0; hh < nh; ++hh) {
        const int h = h0 + hh;
        const float a = A[h];
        const float Dh = D ? D[h] : 0.f;
        const int64_t xo = ((b * L + t0) * H + h) * P;
        const float *Hc = Hs + ((b * T + c) * H + h) * PN;
        const float *Ec = Es + ((b * T + c) * H + h) * PN;
        __syncthreads();  // the previous head's rows and scalars are no longer read
        // ---- this head's x, dy and per-token scalars
        for (int e = tid; e < Q * PS; e += kBThreads) {
            const int j = e / PS, p = e - j * PS;
            const bool ok = j < q && p < P;
            xs[e] = ok ? Elem<Tin>::ld(x, xo + j * xrow + p) : 0.f;
            ys[e] = ok ? Elem<Tin>::ld(dy, xo + j * xrow + p) : 0.f;
        }
        if (wave == 0) {
            const float d = lane < q ? dt[(b * L + t0 + lane) * H + h] : 0.f;
            const float cd = wave_inclusive_scan(d, lane);
            if (lane < Q) {
                dt_s[lane] = d;
                cdt_s[lane] = cd;
                acs_s[lane] = lane < q ? Acs[(b * H + h) * L + t0 + lane] : 0.f;
            }
        }
        // the first E slice is in flight while K and the masked matrices form
        float4 pf[2];
        load_slice(Ec, 0, pf);
        __syncthreads();
        const float alast = acs_s[q - 1];
        // ---- K = dy.x^T (1 x 4 tile), then the masked CB L, K L and GD, with
        // the row sums of GD dt and the column sums of GD
        {
            const int i = tid >> 3, j0 = 4 * (tid & 7);
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
            for (int p = 0; p < PS; p += 4) {
                const float4 yv = f4(ys + i * PS + p);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] += dot4(yv, f4(xs + (j0 + r) * PS + p));
            }
            const float4 cb4 = f4(CB + i * LQ + j0);
            const float cbv[4] = {cb4.x, cb4.y, cb4.z, cb4.w};
            float cbl[4], kl[4], gd[4], rs = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = j0 + r;
                const bool m = j <= i && i < q;
                const float l = m ? ssd_exp(acs_s[i] - acs_s[j]) : 0.f;
                cbl[r] = cbv[r] * l;
                kl[r] = acc[r] * l;
                gd[r] = cbv[r] * kl[r];
                rs = fmaf(gd[r], dt_s[j], rs);
            }
            *reinterpret_cast<float4 *>(CBL + i * LQ + j0) = make_float4(cbl[0], cbl[1], cbl[2], cbl[3]);
            *reinterpret_cast<float4 *>(KL + i * LQ + j0) = make_float4(kl[0], kl[1], kl[2], kl[3]);
            *reinterpret_cast<float4 *>(GD + i * LQ + j0) = make_float4(gd[0], gd[1], gd[2], gd[3]);
            // row i: the 8 lanes of this row (lanes 8m .. 8m+7)
            rs += __shfl_xor(rs, 1, kWave);
            rs += __shfl_xor(rs, 2, kWave);
            rs += __shfl_xor(rs, 4, kWave);
            if ((tid & 7) == 0) rowg[i] = rs;
            // columns j0..j0+3: lanes with the same tid & 7 hold rows 8 wave .. 8 wave + 7
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float cv = gd[r];
                cv += __shfl_xor(cv, 8, kWave);
                cv += __shfl_xor(cv, 16, kWave);
                cv += __shfl_xor(cv, 32, kWave);
                if (lane < 8) part[wave * Q + j0 + r] = cv;
            }
        }
        __syncthreads();
        if (tid < Q) colg[tid] = ((part[tid] + part[Q + tid]) + part[2 * Q + tid]) + part[3 * Q + tid];

        // ---- E slices: dx, and x_j^T E for dB
        float4 acc4[KI];
#pragma unroll
        for (int k = 0; k < KI; ++k) acc4[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int p0 = 0; p0 < P; p0 += slice_rows) {
            const int pr = min(slice_rows, P - p0);
            __syncthreads();  // the previous slice (or colg's partials) no longer read
            store_slice(pf);
            __syncthreads();
            if (p0 + slice_rows < P) load_slice(Ec, p0 + slice_rows, pf);
            else load_slice(Hc, 0, pf);  // the first H slice
            // dx_j[p, p+1]: item (j, p pair), all threads busy
            const int ppn = (pr + 1) / 2;
            for (int e = tid; e < Q * ppn; e += kBThreads) {
                const int j = e % Q, pl = 2 * (e / Q), p = p0 + pl;
                if (j >= q) continue;
                const bool two = pl + 1 < pr;
                float in0 = 0.f, in1 = 0.f;
                for (int i = j; i < q; ++i) {
                    const float w = CBL[i * LQ + j];
                    in0 = fmaf(w, ys[i * PS + p], in0);
                    in1 = fmaf(w, ys[i * PS + p + 1], in1);
                }
                float eb0 = 0.f, eb1 = 0.f;
                const float *e0 = slab + pl * N, *e1 = slab + (two ? pl + 1 : pl) * N;
                for (int n = 0; n < N; n += 4) {
                    const float4 bv = f4(bs + j * NS + n);
                    eb0 += dot4(bv, f4(e0 + n));
                    eb1 += dot4(bv, f4(e1 + n));
                }
                const float dtj = dt_s[j], f = ssd_exp(alast - acs_s[j]);
                Elem<Tin>::st(dx, xo + j * xrow + p, dtj * (in0 + f * eb0) + Dh * ys[j * PS + p]);
                if (two)
                    Elem<Tin>::st(dx, xo + j * xrow + p + 1,
                                  dtj * (in1 + f * eb1) + Dh * ys[j * PS + p + 1]);
            }
            // x_j^T E over the slice: items (jt, nq0 + 8k)
            for (int pl = 0; pl < pr; ++pl) {
                const float xv = xs[jt * PS + p0 + pl];
                const float *er = slab + pl * N;
#pragma unroll
                for (int k = 0; k < KI; ++k) {
                    const int n4 = nq0 + 8 * k;
                    if (n4 < nq) fma4(acc4[k], xv, f4(er + 4 * n4));
                }
            }
        }
        // dB (accumulated over the block's heads) and s3
        {
            float s3 = 0.f;
            const float dtj = dt_s[jt], f = ssd_exp(alast - acs_s[jt]);
            const bool in = jt < q;
#pragma unroll
            for (int k = 0; k < KI; ++k) {
                const int n4 = nq0 + 8 * k;
                if (n4 < nq && in) {
                    float4 intra = make_float4(0.f, 0.f, 0.f, 0.f);
                    for (int i = jt; i < q; ++i) fma4(intra, KL[i * LQ + jt], f4(cs + i * NS + 4 * n4));
                    const float4 xe = acc4[k];
                    dbacc[k].x += dtj * (intra.x + f * xe.x);
                    dbacc[k].y += dtj * (intra.y + f * xe.y);
                    dbacc[k].z += dtj * (intra.z + f * xe.z);
                    dbacc[k].w += dtj * (intra.w + f * xe.w);
                    s3 += f * dot4(xe, f4(bs + jt * NS + 4 * n4));
                }
                acc4[k] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            // token jt's partials: lanes jt and jt + 32 of every wave
            s3 += __shfl_xor(s3, 32, kWave);
            if (lane < 32) part[4 * Q + wave * Q + jt] = s3;
        }

        // ---- H slices: dy_i^T H for dC; <E, H> from the H rows as they pass
        // and the same E rows (read again, from L2)
        float eh = 0.f;
        for (int p0 = 0; p0 < P; p0 += slice_rows) {
            const int pr = min(slice_rows, P - p0);
            __syncthreads();
            store_slice(pf);
            {
                float4 pe[2];
                load_slice(Ec, p0, pe);
                eh += dot4(pe[0], pf[0]) + dot4(pe[1], pf[1]);
            }
            __syncthreads();
            if (p0 + slice_rows < P) load_slice(Hc, p0 + slice_rows, pf);
            for (int pl = 0; pl < pr; ++pl) {
                const float yv = ys[jt * PS + p0 + pl];
                const float *hr = slab + pl * N;
#pragma unroll
                for (int k = 0; k < KI; ++k) {
                    const int n4 = nq0 + 8 * k;
                    if (n4 < nq) fma4(acc4[k], yv, f4(hr + 4 * n4));
                }
            }
        }
        // dC (accumulated over the block's heads) and the state-to-output term
        {
            float hq = 0.f;
            const int i = jt;
            const float ei = ssd_exp(acs_s[i]);
            const bool in = i < q;
#pragma unroll
            for (int k = 0; k < KI; ++k) {
                const int n4 = nq0 + 8 * k;
                if (n4 < nq && in) {
                    float4 intra = make_float4(0.f, 0.f, 0.f, 0.f);
                    for (int j = 0; j <= i; ++j)
                        fma4(intra, KL[i * LQ + j] * dt_s[j], f4(bs + j * NS + 4 * n4));
                    const float4 yh = acc4[k];
                    dcacc[k].x += intra.x + ei * yh.x;
                    dcacc[k].y += intra.y + ei * yh.y;
                    dcacc[k].z += intra.z + ei * yh.z;
                    dcacc[k].w += intra.w + ei * yh.w;
                    hq += ei * dot4(yh, f4(cs + i * NS + 4 * n4));
                }
            }
            hq += __shfl_xor(hq, 32, kWave);
            if (lane < 32) part[wave * Q + i] = hq;
        }
        // ---- <E, H>
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) eh += __shfl_xor(eh, off, kWave);
        if (lane == 0) red[wave] = eh;
        __syncthreads();

        // ---- per-token scalars: dAcs, ddt, dA, dD (wave 0, lane t = token)
        if (wave == 0) {
            const float EH = ((red[0] + red[1]) + red[2]) + red[3];
            const int t = lane;
            const bool in = t < q;
            float s3d = 0.f, dacs = 0.f, kdiag = 0.f, colgd = 0.f;
            if (in) {
                s3d = ((part[4 * Q + t] + part[5 * Q + t]) + part[6 * Q + t]) + part[7 * Q + t];
                const float hqt = ((part[t] + part[Q + t]) + part[2 * Q + t]) + part[3 * Q + t];
                colgd = colg[t];
                dacs = rowg[t] - dt_s[t] * colgd + hqt - s3d * dt_s[t];
                kdiag = KL[t * LQ + t];
            }
            float s3sum = in ? s3d * dt_s[t] : 0.f;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) s3sum += __shfl_xor(s3sum, off, kWave);
            if (t == q - 1) dacs += s3sum + ssd_exp(alast) * EH;
            float suf = dacs;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const float o = __shfl_down(suf, d, kWave);
                if (t + d < kWave) suf += o;
            }
            if (in) ddt[(b * L + t0 + t) * H + h] = a * suf + colgd + s3d;
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
    // ---- dB, dC of the block's heads: one atomic per element
#pragma unroll
    for (int k = 0; k < KI; ++k) {
        const int n4 = nq0 + 8 * k;
        if (n4 < nq && jt < q) {
            float *ob = dB + bo + jt * brow + 4 * n4;
            float *oc = dC + bo + jt * brow + 4 * n4;
            atomicAdd(ob + 0, dbacc[k].x);
            atomicAdd(ob + 1, dbacc[k].y);
            atomicAdd(ob + 2, dbacc[k].z);
            atomicAdd(ob + 3, dbacc[k].w);
            atomicAdd(oc + 0, dcacc[k].x);
            atomicAdd(oc + 1, dcacc[k].y);
            atomicAdd(oc + 2, dcacc[k].z);
            atomicAdd(oc + 3, dcacc[k].w);
        }
    }
}

// Rows of E / H per slice so that the whole block fits the 160 KB of LDS
// (at most 8 KB of slice, so two float4 per thread carry it; at least one row).
int bwd_slice_rows(int P, int N, size_t *lds_bytes) {
    const int64_t fixed = (bwd_fixed_floats(P, N) + 3) & ~3LL;
    const int64_t budget = (160 * 1024) / 4 - fixed;
    int64_t rows = min((int64_t)P, min((int64_t)(2048 / N), budget / N));
    if (rows < 1) rows = 1;
    // the buffer is always 2048 floats: every thread stores its two float4
    *lds_bytes = (size_t)(fixed + 2048) * 4;
    return (int)rows;
}

template <typename Tin, int KI>
void launch_bwd_t(const ScanShape &s, const void *x, const float *dt, const float *A,
                  const void *Bm, const void *Cm, const float *D, const float *Acs,
                  const float *Hs, const float *Es, const void *dy, void *dx, float *ddt,
                  float *dB, float *dC, float *dA, float *dD, hipStream_t st) {
    size_t lds = 0;
    const int rows = bwd_slice_rows((int)s.P, (int)s.N, &lds);
    static bool attr_set = false;  // once per instantiation (per process)
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&k_chunk_bwd<Tin, KI>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        attr_set = true;
    }
    const int64_t R = s.H / s.G;
    const int64_t nslices = (R + kHeadsPerBlock - 1) / kHeadsPerBlock;
    k_chunk_bwd<Tin, KI><<<(unsigned)(s.B * s.T * s.G * nslices), kBThreads, lds, st>>>(
        (const Tin *)x, dt, A, (const Tin *)Bm, (const Tin *)Cm, D, Acs, Hs, Es,
        (const Tin *)dy, (Tin *)dx, ddt, dB, dC, dA, dD, s.L, (int)s.H, (int)s.P, (int)s.N,
        (int)s.G, (int)s.T, rows);
}

}  // namespace

void launch_chunk_bwd(const ScanShape &s, const void *x, const float *dt, const float *A,
                      const void *Bm, const void *Cm, const float *D, const float *Acs,
                      const float *Hs, const float *Es, const void *dy, void *dx, float *ddt,
                      float *dB, float *dC, float *dA, float *dD, hipStream_t st) {
#define SSD_BWD(T_, KI_) \
    launch_bwd_t<T_, KI_>(s, x, dt, A, Bm, Cm, D, Acs, Hs, Es, dy, dx, ddt, dB, dC, dA, dD, st)
#define SSD_BWD_KI(T_)                                 \
    do {                                               \
        if (s.N <= 32) SSD_BWD(T_, 1);                 \
        else if (s.N == 64) SSD_BWD(T_, 2);            \
        else if (s.N == 128) SSD_BWD(T_, 4);           \
        else SSD_BWD(T_, 8);                           \
    } while (0)
    if (s.dtype == SSD_BF16)
        SSD_BWD_KI(bf16);
    else
        SSD_BWD_KI(float);
#undef SSD_BWD_KI
#undef SSD_BWD
}

}  // namespace ssd
