// Device bodies shared by more than one kernel of libssd.
#pragma once

#include "common.hpp"

namespace ssd {

// Chunks whose loads the state passes issue ahead of the dependent updates.
constexpr int kPassAhead = 8;

// Inter-chunk state pass ("Compiler-First State Space Duality and Portable
// O(1) Autoregressive Caching for Inference", paperlayer summary, §3 Method,
// "Chunked recurrence"): per (row, h) and 4 consecutive state elements at
// element offset e, sequential over the row's chunks: states[c] <- H_c,
// H_{c+1} = exp(Acs at the end of chunk c) H_c + S_c, H_0 = init (or 0).
// A row is a batch row (fixed chunking: slots b*T .. b*T+T-1) or, with
// sch/ctab, a sequence of a variable-length batch (its slots from sch, chunk
// ends from ctab; Acs is [H, L] with L all packed tokens).  Loads run
// kPassAhead chunks ahead of the dependent update so that several are in flight.
__device__ __forceinline__ void state_passing_body(float *__restrict__ states,
                                                   const float *__restrict__ Acs,
                                                   const float *init, float *fin, int64_t bh,
                                                   int64_t e, int64_t L, int H, int64_t PN, int Q,
                                                   int T, const int2 *ctab, const int2 *sch) {
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
    float4 hv = make_float4(0.f, 0.f, 0.f, 0.f);
    if (init) hv = *reinterpret_cast<const float4 *>(init + bh * PN + e);
    const int64_t cstride = (int64_t)H * PN;
    float *base = states + (k0 * H + h) * PN + e;
    for (int c0 = 0; c0 < n; c0 += kPassAhead) {
        float4 s[kPassAhead];
        float r[kPassAhead];
#pragma unroll
        for (int k = 0; k < kPassAhead; ++k) {
            const int c = c0 + k;
            if (c < n) {
                s[k] = *reinterpret_cast<const float4 *>(base + c * cstride);
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
            const int c = c0 + k;
            if (c < n) {
                *reinterpret_cast<float4 *>(base + c * cstride) = hv;
                hv.x = r[k] * hv.x + s[k].x;
                hv.y = r[k] * hv.y + s[k].y;
                hv.z = r[k] * hv.z + s[k].z;
                hv.w = r[k] * hv.w + s[k].w;
            }
        }
    }
    if (fin) *reinterpret_cast<float4 *>(fin + bh * PN + e) = hv;
}

}  // namespace ssd
