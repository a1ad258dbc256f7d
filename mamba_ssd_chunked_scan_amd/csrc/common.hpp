// Device helpers shared by the libssd kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace ssd {

constexpr int kWave = 64;

// bf16 is carried as its 16-bit pattern; arithmetic is always fp32.
using bf16 = uint16_t;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

typedef __bf16 bf16x2_t __attribute__((__vector_size__(2 * sizeof(__bf16))));

// fp32 -> bf16, round to nearest even, by the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32); NaN stays NaN.
__device__ __forceinline__ bf16 f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16, (__bf16)f);
}

// Two fp32 values -> packed bf16x2 (low half = a), one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Storage-type traits: load a value as fp32 / store an fp32 value.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float ld(const float *p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void st(float *p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16> {
    static __device__ __forceinline__ float ld(const bf16 *p, int64_t i) {
        return bf16_to_f32(p[i]);
    }
    static __device__ __forceinline__ void st(bf16 *p, int64_t i, float v) {
        p[i] = f32_to_bf16(v);
    }
};

// exp(v) through the hardware base-2 exponential.  Arguments here are
// differences of cumulative log-decays, so v <= 0 in valid use; results below
// the fp32 range flush to 0, which is the correct limit.
__device__ __forceinline__ float ssd_exp(float v) {
    return __builtin_amdgcn_exp2f(v * 1.4426950408889634f);
}

// log(1 + e^v).  Above 20, e^-v is below half an ulp of v, so v itself is the
// correctly rounded value (and e^v would overflow near 88).
__device__ __forceinline__ float softplus_f(float v) {
    return v > 20.f ? v : log1pf(expf(v));
}

// The dt activation (DtAct, launch.hpp); all fields zero does no arithmetic.
__device__ __forceinline__ float act_dt(const DtAct &a, float d, int h) {
    if (a.bias) d += a.bias[h];
    if (a.softplus) d = softplus_f(d);
    if (a.limit) d = fminf(fmaxf(d, a.lo), a.hi);
    return d;
}

// The output gate silu(z) = z / (1 + e^-z), with the hardware base-2
// exponential and reciprocal (each within ~1 ulp; the gate's error is a few
// fp32 ulps, far below the output's rounding).  For z -> -inf, e^-z
// overflows to inf and the reciprocal to 0: the correct limit -0.
__device__ __forceinline__ float silu_f(float z) {
    return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// sigmoid(z) = 1 / (1 + e^-z) with the same base-2 exponential and
// reciprocal as silu_f (the gate's derivative pairs with the gate itself).
__device__ __forceinline__ float sigmoid_f(float z) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// 8 consecutive values of a storage type as fp32 (16 bytes of bf16 or 32 of
// fp32; the address aligned to that) and back.
template <typename T>
__device__ __forceinline__ void ld8(const T *p, float v[8]) {
    if constexpr (sizeof(T) == 2) {
        const uint4 u = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(w[k] << 16);
            v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    } else {
        const float4 a = *reinterpret_cast<const float4 *>(p);
        const float4 b = *reinterpret_cast<const float4 *>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}
template <typename T>
__device__ __forceinline__ void st8(T *p, const float v[8]) {
    if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint4 *>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                   pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    } else {
        *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// First token (within its batch row) and length of chunk slot c.  Fixed
// chunking: t0 = c*Q, q = min(Q, L - t0).  Variable-length batches: the slot's
// entry of the chunk table (q = 0 for an unused slot).
struct ChunkPos {
    int64_t t0;
    int q;
};
__device__ __forceinline__ ChunkPos chunk_pos(const int2 *ctab, int64_t c, int Q, int64_t L) {
    if (ctab) {
        const int2 e = ctab[c];
        return ChunkPos{e.x, e.y};
    }
    const int64_t t0 = c * Q;
    return ChunkPos{t0, (int)min((int64_t)Q, L - t0)};
}

// v from lane (this lane's position under DPP control CTRL); lanes whose
// source is outside the row, or whose row is not in ROW_MASK, get 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes of a wave on the DPP network: shifts
// by 1, 2, 4 and 8 lanes within each row of 16, then each row's total carried
// into the later rows with row_bcast:15 (into rows 1 and 3) and row_bcast:31
// (into rows 2 and 3).  Six dependent VALU steps, no LDS.
__device__ __forceinline__ float wave_scan_dpp(float v) {
    v += dpp_f<0x111>(v);       // row_shr:1
    v += dpp_f<0x112>(v);       // row_shr:2
    v += dpp_f<0x114>(v);       // row_shr:4
    v += dpp_f<0x118>(v);       // row_shr:8
    v += dpp_f<0x142, 0xa>(v);  // row_bcast:15
    v += dpp_f<0x143, 0xc>(v);  // row_bcast:31
    return v;
}

// Sum over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ float wave_sum_dpp(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_scan_dpp(v)), 63));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_inclusive_scan(float v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        float o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

}  // namespace ssd
