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
#include <atomic>

#include "common.hpp"
#include "launch.hpp"
#include "mfma_ops.hpp"
#include "ssd.h"

namespace ssd {
namespace {

using namespace mx;

constexpr int kBQ = 32;         // tokens per gradient chunk
constexpr int kBThreads = 256;
constexpr int kHeadsPerBlock = 4;  // of the generic (VALU) kernel

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
            int T, int slice_rows, const int2 *__restrict__ ctab) {
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
    const ChunkPos cp = chunk_pos(ctab, c, Q, L);
    const int64_t t0 = cp.t0;
    const int q = cp.q;
    if (q <= 0) return;  // an unused slot of a variable-length batch
    const int64_t xrow = (int64_t)H * P, brow = (int64_t)G * N, PN = (int64_t)P * N;
    const int64_t bo = ((b * L + t0) * G + g) * N;
    const int nq = N / 4;
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

// ---------------------------------------------------------------- matrix cores
// The same per-chunk gradient for bf16 x/B/C/dy, headdim 64 and d_state 64 or
// 128, with every contraction on v_mfma_f32_32x32x16_bf16 (fp32 accumulation),
// for chunks of Q = 32 QT tokens (QT row tiles of 32).  bf16 inputs enter the
// products exactly; fp32 factors (the masked matrices CB L dt and K L dt, and
// the states E and H) enter as hi/lo bf16 pairs.  One block (4 QT waves) per
// (b, c, g, slice of 4 heads); wave w works on row tile rt = w / 4 (tokens
// 32 rt ..) with role w % 4.  Per head:
//   K = dy x^T tiles (ti, rt), ti >= rt, then K L, CB L and GD element by
//   element in the accumulator layout (lane: column j; registers: rows i);
//   dx  (rt, p-tile)  = sum_ti (dt CB L)^T dy + dt f B E^T + D dy;
//   dB  (rt, n-tile) += sum_ti (dt K L)^T C + dt f x E      (summed over heads);
//   dC  (rt, n-tile) += sum_tj (K L dt) B + exp(Acs) dy H   (summed over heads);
// with f_j = exp(Acs_last - Acs_j).  E and H pass through LDS in two slices
// of 32 headdim rows, the next slice in registers while the current one is
// multiplied; <E, H> is formed from those registers in fp32.  The row sums
// that the per-token scalars need (s3, the state-to-output term, GD dt) are
// reduced across the lanes of the accumulator layout with ds_swizzle.
template <int N, int QT>
struct BwdLds {
    static constexpr int Q = 32 * QT;
    static constexpr int NCB = QT * (QT + 1) / 2;  // causal 32x32 tiles of C.B
    static constexpr int LDN = N + 16;  // bf16 row stride: B, C and the E / H slices
    static constexpr int LDP = 64 + 16; // bf16 row stride: x, dy
    static constexpr int LDK = Q + 16;  // bf16 row stride: (K L dt)^T
    static constexpr int LDC = 40;      // fp32 row stride: C.B tiles
    static constexpr int B_ = 0;
    static constexpr int C_ = B_ + Q * LDN * 2;
    static constexpr int X_ = C_ + Q * LDN * 2;
    static constexpr int Y_ = X_ + Q * LDP * 2;
    static constexpr int KH_ = Y_ + Q * LDP * 2;
    static constexpr int KL_ = KH_ + Q * LDK * 2;
    static constexpr int CB_ = KL_ + Q * LDK * 2;
    static constexpr int S_ = CB_ + NCB * 32 * LDC * 4;  // E hi, E lo, H hi, H lo [32][LDN]
    static constexpr int V_ = S_ + 4 * 32 * LDN * 2;
    // floats from V_: [2 head parities][6][Q] vectors, [QT][Q] partial row sums
    // of GD dt, [Q] column sums of GD, [2 slices][Q] s3 partials, [2][Q]
    // state-to-output partials, [4 QT] <E,H> partials, [4] diagonals of K
    static constexpr int NV = 12 * Q + QT * Q + Q + 2 * Q + 2 * Q + 4 * QT + 4;
    static constexpr int BYTES = V_ + NV * 4;
};
static_assert(BwdLds<128, 2>::BYTES <= 160 * 1024, "LDS budget");

template <int M>
__device__ __forceinline__ float swz_xor(float v) {  // lane l <- lane l ^ M within 32
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (M << 10) | 0x1f));
}

// Row of accumulator register r in this lane (column = lane % 32).
__device__ __forceinline__ int acc_row(int r, int lane) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Sums each accumulator register over the 32 lanes of its half wave (the 32
// columns of its row).  Lane l returns the total of register (l % 32) / 2,
// i.e. of row acc_row((l % 32) / 2, l); lanes 2k and 2k+1 agree.
__device__ __forceinline__ float rowsum32(const f32x16 &v) {
    const int l = threadIdx.x & 31;
    float u[16], a[8];
    // the empty asm keeps each register a separate value: otherwise the
    // selects below fold into a lane-variable vector index (a 16-way chain
    // of compares and selects)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        u[r] = v[r];
        asm("" : "+v"(u[r]));
    }
    const bool b4 = l & 16, b3 = l & 8, b2 = l & 4, b1 = l & 2;
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = (b4 ? u[k + 8] : u[k]) + swz_xor<16>(b4 ? u[k] : u[k + 8]);
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = (b3 ? a[k + 4] : a[k]) + swz_xor<8>(b3 ? a[k] : a[k + 4]);
#pragma unroll
    for (int k = 0; k < 2; ++k) a[k] = (b2 ? a[k + 2] : a[k]) + swz_xor<4>(b2 ? a[k] : a[k + 2]);
    a[0] = (b1 ? a[1] : a[0]) + swz_xor<2>(b1 ? a[0] : a[1]);
    return a[0] + swz_xor<1>(a[0]);
}

// MFMA A operand from 8 consecutive bf16 values at p (LDS) times w, in fp32,
// split into a hi / lo bf16 pair.
__device__ __forceinline__ void scaled_operand(const bf16 *p, float w, u32x4 &hi, u32x4 &lo) {
    const u32x4 raw = *reinterpret_cast<const u32x4 *>(p);
    float m[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        m[2 * k] = lo_bf16(raw[k]) * w;
        m[2 * k + 1] = hi_bf16(raw[k]) * w;
    }
    split8(m, hi, lo);
}

template <int N, int QT>
__global__ void __launch_bounds__(256 * QT, QT == 1 ? 2 : 1)
k_chunk_bwd_mfma(const bf16 *__restrict__ x, const float *__restrict__ dt,
                 const float *__restrict__ A, const bf16 *__restrict__ Bm,
                 const bf16 *__restrict__ Cm, const float *__restrict__ D,
                 const float *__restrict__ Acs, const float *__restrict__ Hs,
                 const float *__restrict__ Es, const bf16 *__restrict__ dy, bf16 *__restrict__ dx,
                 float *__restrict__ ddt, float *__restrict__ dB, float *__restrict__ dC,
                 float *__restrict__ dA, float *__restrict__ dD, int64_t L, int H, int G, int T,
                 int hpb, int nslices, int64_t nblocks, const int2 *__restrict__ ctab) {
    using Ly = BwdLds<N, QT>;
    constexpr int Q = Ly::Q, P = 64, NT = N / 32, NTH = 256 * QT, W = 4 * QT;
    constexpr int LDN = Ly::LDN, LDP = Ly::LDP, LDK = Ly::LDK, LDC = Ly::LDC;
    constexpr int NF = 8 * N / NTH;  // float4 of E (and of H) per thread per slice
    constexpr int BSEG = N / 8;      // 16-byte segments per B or C row
    extern __shared__ __attribute__((aligned(16))) char smem[];
    bf16 *bs = reinterpret_cast<bf16 *>(smem + Ly::B_);
    bf16 *cs = reinterpret_cast<bf16 *>(smem + Ly::C_);
    bf16 *xs = reinterpret_cast<bf16 *>(smem + Ly::X_);
    bf16 *ys = reinterpret_cast<bf16 *>(smem + Ly::Y_);
    bf16 *klh = reinterpret_cast<bf16 *>(smem + Ly::KH_);
    bf16 *kll = reinterpret_cast<bf16 *>(smem + Ly::KL_);
    float *cbm = reinterpret_cast<float *>(smem + Ly::CB_);
    bf16 *seh = reinterpret_cast<bf16 *>(smem + Ly::S_);
    bf16 *sel = seh + 32 * LDN, *shh = sel + 32 * LDN, *shl = shh + 32 * LDN;
    float *vec = reinterpret_cast<float *>(smem + Ly::V_);  // [2][6][Q]
    float *rowgp = vec + 2 * 6 * Q, *colg = rowgp + QT * Q, *s3p = colg + Q, *hqp = s3p + 2 * Q;
    float *red = hqp + 2 * Q, *scal = red + 4 * QT;

    const uint32_t lb = xcd_block();
    if (lb >= nblocks) return;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int R = H / G;
    uint32_t rest = lb;
    const int hsl = (int)(rest % (uint32_t)nslices);
    rest /= (uint32_t)nslices;
    const int g = (int)(rest % (uint32_t)G);
    rest /= (uint32_t)G;
    const int c = (int)(rest % (uint32_t)T);
    const int64_t b = rest / (uint32_t)T;
    const int h0 = g * R + hsl * hpb;
    const int nh = min(hpb, g * R + R - h0);
    const ChunkPos cp = chunk_pos(ctab, c, Q, L);
    const int64_t t0 = cp.t0;
    const int q = cp.q;
    if (q <= 0) return;  // an unused slot of a variable-length batch
    // block-uniform 64-bit bases, per-lane 32-bit offsets (a chunk spans fewer
    // than 2^31 elements of every tensor)
    const unsigned brs = (unsigned)G * N, xrs = (unsigned)H * P;
    const bf16 *bbase = Bm + ((b * L + t0) * G + g) * N;
    const bf16 *cbase = Cm + ((b * L + t0) * G + g) * N;
    const int64_t xb = (b * L + t0) * H;  // token row base of x, dy, dx (times H)
    const int64_t PN = (int64_t)P * N;

    // wave roles within the row tile rt: n-tiles of dB and dC, the dx p-tile
    // (= the slice it is formed in), and the writer of the tile's shared terms
    const int rt = wave >> 2, wk = wave & 3;
    const bool doB = NT == 4 || wk < 2;
    const int tB = wk;
    const bool doC = NT == 4 || wk >= 2;
    const int tC = NT == 4 ? wk : wk - 2;
    const bool doX = NT == 4 ? wk >= 2 : wk < 2;
    const int tX = NT == 4 ? wk - 2 : wk;
    const bool writer = wk == 0;
    // the wave's 32x32 product per E / H slice sX: B E^T (dx and s3) on the
    // dx waves, C H^T (the state-to-output term) on the others
    const int sX = doX ? tX : (NT == 4 ? wk : wk - 2);

    // ---- staging helpers
    const int xr = tid >> 3, xseg = tid & 7;  // one 16-byte segment of x and of dy
    const u32x4 z4 = u32x4{0u, 0u, 0u, 0u};
    auto load_xy = [&](int h, u32x4 &xv, u32x4 &yv) __attribute__((always_inline)) {
        const int64_t base = (xb + h) * P;
        const unsigned o = (unsigned)xr * xrs + 8u * xseg;
        xv = xr < q ? *reinterpret_cast<const u32x4 *>(x + base + o) : z4;
        yv = xr < q ? *reinterpret_cast<const u32x4 *>(dy + base + o) : z4;
    };
    auto store_xy = [&](const u32x4 &xv, const u32x4 &yv) __attribute__((always_inline)) {
        *reinterpret_cast<u32x4 *>(xs + xr * LDP + 8 * xseg) = xv;
        *reinterpret_cast<u32x4 *>(ys + xr * LDP + 8 * xseg) = yv;
    };
    // per-token vectors of head h (wave 0, lane t = token): dt and Acs
    auto load_vec = [&](int h, float &d, float &a) __attribute__((always_inline)) {
        const int lane = tid & 63;
        const float *dtb = dt + (b * L + t0) * H + h;
        const float *ab = Acs + (b * H + h) * L + t0;
        d = lane < q ? dtb[(unsigned)lane * H] : 0.f;
        a = lane < q ? ab[lane] : 0.f;
    };
    // vectors [parity]: 0 Acs, 1 dt, 2 cumulative dt, 3 f, 4 dt f, 5 exp(Acs)
    auto store_vec = [&](int par, float d, float a) __attribute__((always_inline)) {
        const int lane = tid & 63;
        const float cd = wave_scan_dpp(d);
        const float alast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), q - 1));
        if (lane < Q) {
            float *v = vec + par * 6 * Q;
            const bool in = lane < q;
            const float f = in ? ssd_exp(alast - a) : 0.f;
            v[lane] = a;
            v[Q + lane] = d;
            v[2 * Q + lane] = cd;
            v[3 * Q + lane] = f;
            v[4 * Q + lane] = d * f;
            v[5 * Q + lane] = in ? ssd_exp(a) : 0.f;
        }
    };
    struct SliceRegs {
        float4 e[NF], h[NF];
    };
    auto load_slice = [&](int h, int s, SliceRegs &r) __attribute__((always_inline)) {
        const int64_t o = ((b * T + c) * H + h) * PN + (int64_t)s * 32 * N;
        const float4 *e4 = reinterpret_cast<const float4 *>(Es + o);
        const float4 *h4 = reinterpret_cast<const float4 *>(Hs + o);
#pragma unroll
        for (int k = 0; k < NF; ++k) {
            r.e[k] = e4[tid + NTH * k];
            r.h[k] = h4[tid + NTH * k];
        }
    };
    auto store_slice = [&](const SliceRegs &r, float &eh) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < NF; ++k) {
            const int e = tid + NTH * k, pl = e / (N / 4), n = 4 * (e % (N / 4));
            uint32_t l0, l1;
            const uint32_t h0e = split2(r.e[k].x, r.e[k].y, l0), h1e = split2(r.e[k].z, r.e[k].w, l1);
            *reinterpret_cast<u32x2 *>(seh + pl * LDN + n) = u32x2{h0e, h1e};
            *reinterpret_cast<u32x2 *>(sel + pl * LDN + n) = u32x2{l0, l1};
            const uint32_t h0h = split2(r.h[k].x, r.h[k].y, l0), h1h = split2(r.h[k].z, r.h[k].w, l1);
            *reinterpret_cast<u32x2 *>(shh + pl * LDN + n) = u32x2{h0h, h1h};
            *reinterpret_cast<u32x2 *>(shl + pl * LDN + n) = u32x2{l0, l1};
            eh = fmaf(r.e[k].x, r.h[k].x, eh);
            eh = fmaf(r.e[k].y, r.h[k].y, eh);
            eh = fmaf(r.e[k].z, r.h[k].z, eh);
            eh = fmaf(r.e[k].w, r.h[k].w, eh);
        }
    };

    // ---- B and C rows of the chunk (shared by the block's heads), then C.B
    for (int e = tid; e < Q * BSEG; e += NTH) {
        const int r = e / BSEG, sg = e % BSEG;
        const unsigned o = (unsigned)r * brs + 8u * sg;
        const bool in = r < q;
        *reinterpret_cast<u32x4 *>(bs + r * LDN + 8 * sg) =
            in ? *reinterpret_cast<const u32x4 *>(bbase + o) : z4;
        *reinterpret_cast<u32x4 *>(cs + r * LDN + 8 * sg) =
            in ? *reinterpret_cast<const u32x4 *>(cbase + o) : z4;
    }
    u32x4 nx, ny;
    float nd = 0.f, na = 0.f;
    // E / H slices in registers: sr[s] holds slice s of the next head whose
    // slice s is not yet in LDS (two slices, one head, ahead)
    SliceRegs sr[2];
    load_xy(h0, nx, ny);
    if (wave == 0) load_vec(h0, nd, na);
    load_slice(h0, 0, sr[0]);
    load_slice(h0, 1, sr[1]);
    __syncthreads();
    if (wave < Ly::NCB) {  // C.B tile (ti, tj): A = C rows of ti, B = B rows of tj
        const int lane = tid & 63, il = lane & 31, hw = lane >> 5;
        const int ti = wave == 0 ? 0 : 1, tj = wave - ti * (ti + 1) / 2;
        f32x16 acc = zero16();
#pragma unroll
        for (int ks = 0; ks < N / 16; ++ks)
            acc = mfma32(*reinterpret_cast<const u32x4 *>(cs + (32 * ti + il) * LDN + 16 * ks + 8 * hw),
                         *reinterpret_cast<const u32x4 *>(bs + (32 * tj + il) * LDN + 16 * ks + 8 * hw),
                         acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) cbm[(wave * 32 + acc_row(r, lane)) * LDC + il] = acc[r];
    }
    float eh = 0.f;
    store_xy(nx, ny);
    if (wave == 0) store_vec(0, nd, na);
    store_slice(sr[0], eh);
    if (nh > 1) load_slice(h0 + 1, 0, sr[0]);
    __syncthreads();

    f32x16 dBt = zero16(), dCt = zero16();
    for (int hh = 0; hh < nh; ++hh) {
        const int h = h0 + hh, par = hh & 1;
        // the lane index is re-derived opaquely each head, so that the many
        // per-lane LDS addresses and masks below are formed where they are
        // used instead of being hoisted out of the loop (and spilled)
        int lane = tid & 63;
        asm volatile("" : "+v"(lane));
        const int il = lane & 31, hw = lane >> 5;
        const int jg = 32 * rt + il;  // this lane's token in row tile rt
        const float *v = vec + par * 6 * Q;
        const float *vacs = v, *vdt = v + Q, *vcd = v + 2 * Q, *vf = v + 3 * Q, *vwdf = v + 4 * Q,
                    *vei = v + 5 * Q;
        // ---- K tiles (ti, rt) = dy x^T; K L dt, CB L dt (and GD) in the
        // accumulator layout; the intra-chunk dB and dx products from registers
        f32x16 accX = zero16();
        {
            const float acs_j = vacs[jg], dt_j = vdt[jg];
            float cg = 0.f, kd = 0.f;
#pragma unroll
            for (int ti = 0; ti < QT; ++ti) {
                if (ti < rt) continue;
                f32x16 K = zero16();
#pragma unroll
                for (int ks = 0; ks < P / 16; ++ks)
                    K = mfma32(*reinterpret_cast<const u32x4 *>(ys + (32 * ti + il) * LDP + 16 * ks + 8 * hw),
                               *reinterpret_cast<const u32x4 *>(xs + jg * LDP + 16 * ks + 8 * hw), K);
                const float *cbt = cbm + (ti * (ti + 1) / 2 + rt) * 32 * LDC;
                f32x16 kl, cbl, gdt;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = 32 * ti + acc_row(r, lane);
                    // exp for every element, then the causal / length mask as a
                    // select (a branch per element otherwise)
                    const float e = ssd_exp(vacs[i] - acs_j);
                    const float lv = (jg <= i && i < q) ? e : 0.f;
                    const float cb = cbt[acc_row(r, lane) * LDC + il];
                    kl[r] = K[r] * lv * dt_j;   // (K L)[i][j] dt_j
                    cbl[r] = cb * lv * dt_j;    // (CB L)[i][j] dt_j
                    const float gd = cb * K[r] * lv;
                    if (writer) {
                        gdt[r] = gd * dt_j;
                        cg += gd;
                        kd += i == jg ? K[r] : 0.f;
                    }
                }
                if (writer) {
                    // row sums of GD dt (partial over this column tile)
                    const float rs = rowsum32(gdt);
                    if ((lane & 1) == 0) rowgp[rt * Q + 32 * ti + acc_row(il >> 1, lane)] = rs;
                    // (K L dt)^T as hi / lo bf16 rows j, for the dC product
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        uint32_t l0, l1;
                        const uint32_t a0 = split2(kl[4 * gq], kl[4 * gq + 1], l0);
                        const uint32_t a1 = split2(kl[4 * gq + 2], kl[4 * gq + 3], l1);
                        const int o = jg * LDK + 32 * ti + 8 * gq + 4 * hw;
                        *reinterpret_cast<u32x2 *>(klh + o) = u32x2{a0, a1};
                        *reinterpret_cast<u32x2 *>(kll + o) = u32x2{l0, l1};
                    }
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    float m[8];
                    u32x4 hi, lo;
                    if (doB) {  // dB[j][n] += sum_i (K L dt)[i][j] C[i][n]
#pragma unroll
                        for (int e = 0; e < 8; ++e) m[e] = kl[8 * ks + e];
                        split8(m, hi, lo);
                        const u32x4 bo = tr_operand<true>(cs + 32 * ti * LDN, LDN, 16 * ks, 32 * tB);
                        dBt = mfma32(hi, bo, dBt);
                        dBt = mfma32(lo, bo, dBt);
                    }
                    if (doX) {  // dx[j][p] = sum_i (CB L dt)[i][j] dy[i][p]
#pragma unroll
                        for (int e = 0; e < 8; ++e) m[e] = cbl[8 * ks + e];
                        split8(m, hi, lo);
                        const u32x4 bo = tr_operand<true>(ys + 32 * ti * LDP, LDP, 16 * ks, 32 * tX);
                        accX = mfma32(hi, bo, accX);
                        accX = mfma32(lo, bo, accX);
                    }
                }
                // one K tile at a time: keeps the temporaries of the two tiles
                // from being live together
                __builtin_amdgcn_sched_barrier(0);
            }
            if (writer) {
                // column sums of GD and the diagonal of K for this column tile
                cg += __shfl_xor(cg, 32, kWave);
                if (lane < 32) colg[jg] = cg;
                kd = wave_sum_dpp(kd);
                if (lane == 0) scal[rt] = kd;
            }
        }
        // ---- one 32-row slice of E and H (in LDS).  The per-row scales of the
        // state terms (dt f for x E, exp(Acs) for dy H) go into the A operand,
        // formed in fp32 and split hi / lo, so both products accumulate
        // straight into dB and dC
        auto slice = [&](int s) __attribute__((always_inline)) {
            const float wB = vwdf[jg], wC = vei[jg];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int pc = 32 * s + 16 * ks + 8 * hw;
                u32x4 hi, lo;
                if (doB) {  // dB[j][n] += dt_j f_j sum_p x[j][p] E[p][n]
                    scaled_operand(xs + jg * LDP + pc, wB, hi, lo);
                    const u32x4 bh = tr_operand<false>(seh, LDN, 16 * ks, 32 * tB);
                    dBt = mfma32(hi, bh, dBt);
                    dBt = mfma32(hi, tr_operand<false>(sel, LDN, 16 * ks, 32 * tB), dBt);
                    dBt = mfma32(lo, bh, dBt);
                }
                if (doC) {  // dC[i][n] += exp(Acs_i) sum_p dy[i][p] H[p][n]
                    scaled_operand(ys + jg * LDP + pc, wC, hi, lo);
                    const u32x4 bh = tr_operand<false>(shh, LDN, 16 * ks, 32 * tC);
                    dCt = mfma32(hi, bh, dCt);
                    dCt = mfma32(hi, tr_operand<false>(shl, LDN, 16 * ks, 32 * tC), dCt);
                    dCt = mfma32(lo, bh, dCt);
                }
            }
            if (sX == s) {
                // B E^T (rows j, columns p of this slice) on the dx waves,
                // C H^T (rows i) on the others: A = B or C rows, B = E or H rows
                const bf16 *ar = (doX ? bs : cs) + jg * LDN + 8 * hw;
                const bf16 *sh = (doX ? seh : shh) + il * LDN + 8 * hw;
                const bf16 *sl = (doX ? sel : shl) + il * LDN + 8 * hw;
                f32x16 acc = zero16();
#pragma unroll
                for (int ks = 0; ks < N / 16; ++ks) {
                    const u32x4 a = *reinterpret_cast<const u32x4 *>(ar + 16 * ks);
                    acc = mfma32(a, *reinterpret_cast<const u32x4 *>(sh + 16 * ks), acc);
                    acc = mfma32(a, *reinterpret_cast<const u32x4 *>(sl + 16 * ks), acc);
                }
                const int p = 32 * s + il;
                f32x16 sv;
                if (doX) {  // dx of tile (rt, s); s3_j = f_j sum_p x[j][p] (B E^T)[j][p]
                    const float Dh = D ? D[h] : 0.f;
                    bf16 *dxh = dx + (xb + h) * P;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = 32 * rt + acc_row(r, lane);
                        const float yv = bf16_to_f32(ys[j * LDP + p]);
                        if (j < q) {
                            const float o = fmaf(Dh, yv, fmaf(vwdf[j], acc[r], accX[r]));
                            dxh[(unsigned)j * xrs + p] = f32_to_bf16(o);
                        }
                        sv[r] = vf[j] * bf16_to_f32(xs[j * LDP + p]) * acc[r];
                    }
                } else {  // exp(Acs_i) sum_p dy[i][p] (C H^T)[i][p]
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int i = 32 * rt + acc_row(r, lane);
                        sv[r] = vei[i] * bf16_to_f32(ys[i * LDP + p]) * acc[r];
                    }
                }
                const float sum = rowsum32(sv);
                if ((lane & 1) == 0) (doX ? s3p : hqp)[s * Q + 32 * rt + acc_row(il >> 1, lane)] = sum;
            }
        };
        slice(0);
        __syncthreads();  // slice 0 and (K L dt)^T: done / visible
        if (doC) {        // dC[i][n] += sum_{j <= i} (K L dt)[i][j] B[j][n]
#pragma unroll
            for (int tj = 0; tj < QT; ++tj) {
                if (tj > rt) continue;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int k0 = 32 * tj + 16 * ks;
                    const u32x4 bo = tr_operand<false>(bs, LDN, k0, 32 * tC);
                    dCt = mfma32(tr_operand<false>(klh, LDK, k0, 32 * rt), bo, dCt);
                    dCt = mfma32(tr_operand<false>(kll, LDK, k0, 32 * rt), bo, dCt);
                }
            }
        }
        store_slice(sr[1], eh);
        const bool more = hh + 1 < nh;
        if (more) {
            load_slice(h + 1, 1, sr[1]);
            load_xy(h + 1, nx, ny);
            if (wave == 0) load_vec(h + 1, nd, na);
        }
        __syncthreads();  // slice 1 visible
        slice(1);
        eh = wave_sum_dpp(eh);
        if (lane == 0) red[wave] = eh;
        eh = 0.f;
        __syncthreads();  // partials visible; x, dy and the slice buffer free
        // ---- per-token scalars: dAcs, ddt, dA, dD (wave 0, lane t = token)
        if (wave == 0) {
            const int t = lane;
            const bool in = t < q;
            float EH = 0.f, KD = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) EH += red[w];
#pragma unroll
            for (int k = 0; k < QT; ++k) KD += scal[k];
            const float alast = vacs[q - 1];
            float s3d = 0.f, dacs = 0.f, colgd = 0.f, dtt = 0.f;
            if (in) {
                float hqt = 0.f, rg = 0.f;
#pragma unroll
                for (int k = 0; k < 2; ++k) {  // the two E / H slices
                    s3d += s3p[k * Q + t];
                    hqt += hqp[k * Q + t];
                }
#pragma unroll
                for (int k = 0; k < QT; ++k)
                    if (32 * k <= t) rg += rowgp[k * Q + t];  // column tiles at or left of t's
                dtt = vdt[t];
                colgd = colg[t];
                dacs = rg - dtt * colgd + hqt - s3d * dtt;
            }
            const float s3sum = wave_sum_dpp(s3d * dtt);
            if (t == q - 1) dacs += s3sum + ssd_exp(alast) * EH;
            // suffix sums: a prefix scan of the lane-reversed values
            const float rsum = wave_scan_dpp(__shfl(dacs, 63 - t, kWave));
            const float suf = __shfl(rsum, 63 - t, kWave);
            if (in) ddt[((b * L + t0) * H + h) + (unsigned)t * H] = A[h] * suf + colgd + s3d;
            const float da = wave_sum_dpp(in ? dacs * vcd[t] : 0.f);
            if (lane == 0) {
                atomicAdd(&dA[h], da);
                if (dD) atomicAdd(&dD[h], KD);
            }
        }
        if (more) {  // the next head's rows, vectors and first slice
            store_xy(nx, ny);
            if (wave == 0) store_vec(par ^ 1, nd, na);
            store_slice(sr[0], eh);
            if (hh + 2 < nh) load_slice(h + 2, 0, sr[0]);
        }
        __syncthreads();
    }
    // ---- dB, dC of the block's heads: one atomic per element
    const int lane = tid & 63, il = lane & 31;
    float *dBb = dB + ((b * L + t0) * G + g) * N + 32 * tB;
    float *dCb = dC + ((b * L + t0) * G + g) * N + 32 * tC;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int j = 32 * rt + acc_row(r, lane);
        if (j < q) {
            const unsigned o = (unsigned)j * brs + il;
            if (doB) atomicAdd(dBb + o, dBt[r]);
            if (doC) atomicAdd(dCb + o, dCt[r]);
        }
    }
}

// Raises a kernel's dynamic-LDS limit on the current device, once per device
// (the attribute belongs to each device's copy of the kernel).  A failure
// shows up as the launch's own error.
template <auto *Kernel>
void allow_dynamic_lds(int bytes) {
    static std::atomic<bool> done[64];  // host threads may launch concurrently
    int dev = 0;
    const bool known = hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64;
    if (known && done[dev].load(std::memory_order_relaxed)) return;
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(Kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess &&
        known)
        done[dev].store(true, std::memory_order_relaxed);
}

// Heads per block of the per-chunk gradient.  One block fits a CU (its LDS),
// so the grid of groups * ceil(R / hpb) blocks runs in rounds of one block
// per CU, and a block takes about hpb + 0.5 head-times (the heads one after
// another, plus the staging of B, C and C.B and the dB / dC atomics it does
// once).  The choice minimises rounds * (hpb + 0.5), the larger hpb on a tie
// (fewer atomics).  Measured at the 2.7B workload (64 chunk groups, 80
// heads): hpb 20 (one round of 256 blocks) 472-481 us per gradient call, 10
// 490-496, 5 498-499, 4 501-517, 8 527-531, 2 533-545, 16 (1.25 rounds) 612,
// 40 (half the CUs idle) 688-690.
int bwd_heads_per_block(int64_t groups, int64_t R, int cus) {
    int best = 1;
    double best_cost = 0.0;
    for (int hpb = 1; hpb <= R; ++hpb) {
        const int64_t nb = groups * ((R + hpb - 1) / hpb);
        const int64_t rounds = (nb + cus - 1) / cus;
        const double cost = (double)rounds * (hpb + 0.5);
        if (hpb == 1 || cost <= best_cost) {
            best = hpb;
            best_cost = cost;
        }
    }
    return best;
}

template <int N, int QT>
void launch_bwd_mfma_t(const ScanShape &s, const void *x, const float *dt, const float *A,
                       const void *Bm, const void *Cm, const float *D, const float *Acs,
                       const float *Hs, const float *Es, const void *dy, void *dx, float *ddt,
                       float *dB, float *dC, float *dA, float *dD, hipStream_t st) {
    allow_dynamic_lds<&k_chunk_bwd_mfma<N, QT>>(BwdLds<N, QT>::BYTES);
    const int64_t R = s.H / s.G;
    const int hpb = bwd_heads_per_block(s.B * s.T * s.G, R, device_cus());
    const int64_t nslices = (R + hpb - 1) / hpb;
    const int64_t nblocks = s.B * s.T * s.G * nslices;
    k_chunk_bwd_mfma<N, QT><<<padded_grid(nblocks), 256 * QT, BwdLds<N, QT>::BYTES, st>>>(
        (const bf16 *)x, dt, A, (const bf16 *)Bm, (const bf16 *)Cm, D, Acs, Hs, Es,
        (const bf16 *)dy, (bf16 *)dx, ddt, dB, dC, dA, dD, s.L, (int)s.H, (int)s.G, (int)s.T,
        hpb, (int)nslices, nblocks, s.ctab);
}

// ------------------------------------------------------- edges, backward
// The output gate y_out = y * silu(z): dys = dy * z s and dz = dy * y * s
// (1 + z (1 - s)) with s = sigmoid(z), 8 values per thread per step.
template <typename T>
__global__ void __launch_bounds__(256)
k_gate_bwd(const T *__restrict__ dy, const T *__restrict__ y, const T *__restrict__ z,
           T *__restrict__ dys, T *__restrict__ dz, float *__restrict__ dys32, int64_t n) {
    const int64_t n8 = n / 8;
    if (blockIdx.x == 0 && threadIdx.x < n - 8 * n8) {  // the last n % 8 values
        const int64_t i = 8 * n8 + threadIdx.x;
        const float g = Elem<T>::ld(dy, i), zz = Elem<T>::ld(z, i);
        const float sg = sigmoid_f(zz);
        Elem<T>::st(dys, i, g * (zz * sg));
        if (dys32) dys32[i] = g * (zz * sg);
        Elem<T>::st(dz, i, g * Elem<T>::ld(y, i) * (sg * (1.f + zz * (1.f - sg))));
    }
    for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
        float g[8], yy[8], zz[8], a[8], b[8];
        ld8(dy + 8 * i, g);
        ld8(y + 8 * i, yy);
        ld8(z + 8 * i, zz);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float sg = sigmoid_f(zz[e]);
            a[e] = g[e] * (zz[e] * sg);
            b[e] = g[e] * yy[e] * (sg * (1.f + zz[e] * (1.f - sg)));
        }
        st8(dys + 8 * i, a);
        if (dys32) st8(dys32 + 8 * i, a);
        st8(dz + 8 * i, b);
    }
}

// The dt activation: block (h, y) turns rows [y R, (y+1) R) of head h's
// ddt column into the raw-dt gradient (the activation's derivative: sigmoid
// of the biased value under softplus, 1 without, 0 where the clamp holds a
// bound it was pushed past) and writes its sum to part[h][y].
constexpr int kDtRows = 4096;
__global__ void __launch_bounds__(256)
k_dt_act_bwd(float *__restrict__ ddt, const float *__restrict__ dt_raw, DtAct act,
             float *__restrict__ part, int64_t rows, int H) {
    __shared__ float red[4];
    const int h = blockIdx.x, tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.y * kDtRows;
    const int64_t r1 = r0 + kDtRows < rows ? r0 + kDtRows : rows;
    const float bias = act.bias ? act.bias[h] : 0.f;
    float acc = 0.f;
    for (int64_t r = r0 + tid; r < r1; r += 256) {
        const int64_t i = r * H + h;
        const float u = dt_raw[i] + bias;
        float d = 1.f, pre = u;
        if (act.softplus) {
            d = sigmoid_f(u);
            pre = softplus_f(u);
        }
        if (act.limit && (pre < act.lo || pre > act.hi)) d = 0.f;
        const float v = ddt[i] * d;
        ddt[i] = v;
        acc += v;
    }
    if (part) {
        acc = wave_sum_dpp(acc);
        if ((tid & 63) == 0) red[tid >> 6] = acc;
        __syncthreads();
        if (tid == 0) part[(int64_t)h * gridDim.y + blockIdx.y] = ((red[0] + red[1]) + red[2]) + red[3];
    }
}

// The gated RMSNorm with the gate under it, backward.  Block (range, k)
// takes tokens [range tr, +tr) of norm group k: CG channels as
// 8-value vectors, vector u of thread t at channel 8 (t + 256 u).  Per token,
// with v the gated output (v = y without a gate), r = 1 / sqrt(mean(v^2) +
// eps) and S = sum(dout w v) (two block sums, fixed order):
//   dv = r (w dout - v r^2 S / CG),  dys = dv silu(z),  dz = dv y silu'(z);
// the thread's sum over its tokens of dout v r goes to part[range][k CG + c].
constexpr int kNormVec = 4;  // vectors per thread: CG <= 8 * 256 * kNormVec

template <typename T>
__global__ void __launch_bounds__(256)
k_norm_gate_bwd(const T *__restrict__ dout, const T *__restrict__ y, const T *__restrict__ z,
                const float *__restrict__ w, float eps, T *__restrict__ dys, T *__restrict__ dz,
                float *__restrict__ part, int64_t ntok, int64_t HP, int CG,
                float *__restrict__ dys32, int tr) {
    __shared__ float red[2][4];
    const int tid = threadIdx.x, k = blockIdx.y;
    const int64_t t0 = (int64_t)blockIdx.x * tr;
    const int64_t t1 = t0 + tr < ntok ? t0 + tr : ntok;
    float dw[kNormVec][8];
#pragma unroll
    for (int u = 0; u < kNormVec; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) dw[u][e] = 0.f;
    // v = y silu(z) (or y) of vector u at offset o
    auto gated = [&](int64_t o, float yv[8], float zv[8], float v[8]) __attribute__((always_inline)) {
        ld8(y + o, yv);
        if (z) {
            ld8(z + o, zv);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = yv[e] * (zv[e] * sigmoid_f(zv[e]));
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = yv[e];
        }
    };
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t base = t * HP + (int64_t)k * CG;
        float ss = 0.f, sd = 0.f;
#pragma unroll
        for (int u = 0; u < kNormVec; ++u) {
            const int c = 8 * (tid + 256 * u);
            if (c < CG) {
                float yv[8], zv[8], v[8], g[8], ww[8];
                gated(base + c, yv, zv, v);
                ld8(dout + base + c, g);
                ld8(w + (int64_t)k * CG + c, ww);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ss = fmaf(v[e], v[e], ss);
                    sd = fmaf(g[e] * ww[e], v[e], sd);
                }
            }
        }
        ss = wave_sum_dpp(ss);
        sd = wave_sum_dpp(sd);
        if ((tid & 63) == 0) {
            red[0][tid >> 6] = ss;
            red[1][tid >> 6] = sd;
        }
        __syncthreads();
        const float sst = ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3];
        const float sdt = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
        const float r = 1.f / sqrtf(sst / (float)CG + eps);
        const float a = r * r * sdt / (float)CG;
#pragma unroll
        for (int u = 0; u < kNormVec; ++u) {
            const int c = 8 * (tid + 256 * u);
            if (c < CG) {
                float yv[8], zv[8], v[8], g[8], ww[8], o1[8], o2[8];
                gated(base + c, yv, zv, v);
                ld8(dout + base + c, g);
                ld8(w + (int64_t)k * CG + c, ww);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float dv = r * (ww[e] * g[e] - v[e] * a);
                    dw[u][e] = fmaf(g[e] * v[e], r, dw[u][e]);
                    if (z) {
                        const float sg = sigmoid_f(zv[e]);
                        o1[e] = dv * (zv[e] * sg);
                        o2[e] = dv * yv[e] * (sg * (1.f + zv[e] * (1.f - sg)));
                    } else {
                        o1[e] = dv;
                    }
                }
                st8(dys + base + c, o1);
                if (dys32) st8(dys32 + base + c, o1);
                if (z) st8(dz + base + c, o2);
            }
        }
        __syncthreads();  // red[] is reused by the next token
    }
    float *pr = part + (int64_t)blockIdx.x * HP + (int64_t)k * CG;
#pragma unroll
    for (int u = 0; u < kNormVec; ++u) {
        const int c = 8 * (tid + 256 * u);
        if (c < CG) {
            *reinterpret_cast<float4 *>(pr + c) = make_float4(dw[u][0], dw[u][1], dw[u][2], dw[u][3]);
            *reinterpret_cast<float4 *>(pr + c + 4) = make_float4(dw[u][4], dw[u][5], dw[u][6], dw[u][7]);
        }
    }
}

// out[y][c] = rows [y R, (y+1) R) of part [rows][n] summed in order: one
// thread per column, block (column block, y).
constexpr int kSumRows = 64;
__global__ void __launch_bounds__(256)
k_sum_cols(const float *__restrict__ part, int64_t rows, int64_t n, int64_t R,
           float *__restrict__ out) {
    const int64_t c = blockIdx.x * 256LL + threadIdx.x;
    if (c >= n) return;
    const int64_t r0 = (int64_t)blockIdx.y * R;
    const int64_t r1 = r0 + R < rows ? r0 + R : rows;
    float s = 0.f;
#pragma unroll 8
    for (int64_t r = r0; r < r1; ++r) s += part[r * n + c];
    out[(int64_t)blockIdx.y * n + c] = s;
}

// dbias[h] = the parts of head h summed in order.
__global__ void k_sum_parts(const float *__restrict__ part, int64_t nparts,
                            float *__restrict__ dbias, int H) {
    const int h = blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= H) return;
    float s = 0.f;
    for (int64_t k = 0; k < nparts; ++k) s += part[h * nparts + k];
    dbias[h] = s;
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
    allow_dynamic_lds<&k_chunk_bwd<Tin, KI>>(160 * 1024);
    const int64_t R = s.H / s.G;
    const int64_t nslices = (R + kHeadsPerBlock - 1) / kHeadsPerBlock;
    k_chunk_bwd<Tin, KI><<<(unsigned)(s.B * s.T * s.G * nslices), kBThreads, lds, st>>>(
        (const Tin *)x, dt, A, (const Tin *)Bm, (const Tin *)Cm, D, Acs, Hs, Es,
        (const Tin *)dy, (Tin *)dx, ddt, dB, dC, dA, dD, s.L, (int)s.H, (int)s.P, (int)s.N,
        (int)s.G, (int)s.T, rows, s.ctab);
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
    if (bwd_states_mfma_ok(s)) {  // 64-token chunks (two row tiles)
#define SSD_BWDM(N_, QT_) \
    launch_bwd_mfma_t<N_, QT_>(s, x, dt, A, Bm, Cm, D, Acs, Hs, Es, dy, dx, ddt, dB, dC, dA, dD, st)
        if (s.N == 64) SSD_BWDM(64, 2);
        else SSD_BWDM(128, 2);
#undef SSD_BWDM
    } else if (s.dtype == SSD_BF16)
        SSD_BWD_KI(bf16);
    else
        SSD_BWD_KI(float);
#undef SSD_BWD_KI
#undef SSD_BWD
}

void launch_gate_bwd(const void *dy, const void *y, const void *z, void *dys, void *dz,
                     int64_t n, int dtype, hipStream_t st, float *dys32) {
    if (n <= 0) return;
    const int64_t want = (n / 8 + 255) / 256;
    const unsigned blocks = (unsigned)(want < 1 ? 1 : (want < 65536 ? want : 65536));
    if (dtype == SSD_BF16)
        k_gate_bwd<bf16><<<blocks, 256, 0, st>>>((const bf16 *)dy, (const bf16 *)y, (const bf16 *)z,
                                                 (bf16 *)dys, (bf16 *)dz, dys32, n);
    else
        k_gate_bwd<float><<<blocks, 256, 0, st>>>((const float *)dy, (const float *)y,
                                                  (const float *)z, (float *)dys, (float *)dz,
                                                  dys32, n);
}

int64_t dt_bias_parts(int64_t rows) { return (rows + kDtRows - 1) / kDtRows; }

void launch_dt_act_bwd(float *ddt, const float *dt_raw, const DtAct &act, int64_t rows,
                       int64_t H, float *part, float *dbias, hipStream_t st) {
    const int64_t np = dt_bias_parts(rows);
    if (np <= 0) return;
    k_dt_act_bwd<<<dim3((unsigned)H, (unsigned)np), 256, 0, st>>>(ddt, dt_raw, act,
                                                                  dbias ? part : nullptr, rows,
                                                                  (int)H);
    if (dbias) k_sum_parts<<<(unsigned)((H + 63) / 64), 64, 0, st>>>(part, np, dbias, (int)H);
}

bool norm_bwd_ok(int64_t H, int64_t P, int64_t NG) {
    return P % 8 == 0 && (H / NG) * P <= 8 * 256 * kNormVec;
}

// Tokens per block of the norm's gradient: about 2048 blocks over the
// (token, group) pairs, 1 to 64 tokens each (more tokens per block, fewer
// partial sums of the weight's gradient to add up).
int64_t norm_bwd_rows(int64_t ntok, int64_t NG) {
    const int64_t tr = (ntok * NG + 2047) / 2048;
    return tr < 1 ? 1 : (tr > 64 ? 64 : tr);
}

// Rows of partial sums of the weight's gradient: one per block range, then
// one per kSumRows of those (the first level of their sum).
int64_t norm_bwd_parts(int64_t ntok, int64_t NG) {
    const int64_t tr = norm_bwd_rows(ntok, NG);
    const int64_t nr = (ntok + tr - 1) / tr;
    return nr + (nr + kSumRows - 1) / kSumRows;
}

void launch_norm_gate_bwd(const void *dout, const void *y, const void *z, const float *w,
                          float eps, int64_t ntok, int64_t H, int64_t P, int64_t NG, void *dys,
                          void *dz, float *part, float *dw, int dtype, hipStream_t st,
                          float *dys32) {
    const int tr = (int)norm_bwd_rows(ntok, NG);
    const int64_t nr = (ntok + tr - 1) / tr;
    if (nr <= 0) return;
    const int CG = (int)((H / NG) * P);
    const dim3 grid((unsigned)nr, (unsigned)NG);
    if (dtype == SSD_BF16)
        k_norm_gate_bwd<bf16><<<grid, 256, 0, st>>>((const bf16 *)dout, (const bf16 *)y,
                                                    (const bf16 *)z, w, eps, (bf16 *)dys,
                                                    (bf16 *)dz, part, ntok, H * P, CG, dys32,
                                                    tr);
    else
        k_norm_gate_bwd<float><<<grid, 256, 0, st>>>((const float *)dout, (const float *)y,
                                                     (const float *)z, w, eps, (float *)dys,
                                                     (float *)dz, part, ntok, H * P, CG,
                                                     dys32, tr);
    if (dw) {  // two levels: kSumRows rows at a time, then those sums
        const int64_t n2 = (nr + kSumRows - 1) / kSumRows;
        float *part2 = part + nr * H * P;
        const unsigned cb = (unsigned)((H * P + 255) / 256);
        k_sum_cols<<<dim3(cb, (unsigned)n2), 256, 0, st>>>(part, nr, H * P, kSumRows, part2);
        k_sum_cols<<<dim3(cb, 1), 256, 0, st>>>(part2, n2, H * P, n2, dw);
    }
}

}  // namespace ssd
