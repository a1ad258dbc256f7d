// Matrix-core building blocks shared by the bf16 MFMA kernels (gfx950):
// the v_mfma_f32_32x32x16_bf16 wrapper, hi/lo bf16 splitting of fp32
// values, LDS transpose-read operands, the XCD-aware block order and raw
// buffer resources.
//
//  * v_mfma_f32_32x32x16_bf16 (D[32x32] += A[32x16] B[16x32]).  Lane l
//    supplies row (A) or column (B) l%32 and the 8 k slots 8*(l/32)+e; the
//    accumulator holds column l%32 and rows 8*(r/4) + 4*(l/32) + r%4 in its
//    register r (r = 0..15).
//  * ds_read_b64_tr_b16, the LDS transpose read: within each group of 16
//    lanes, lane i receives element (i & 3) of the 8-byte reads of lanes
//    (i >> 2) + 4k, k = 0..3.  It turns a row-major [k][outer] tile into
//    k-contiguous MFMA operands.
#pragma once

#include "common.hpp"

namespace ssd {
namespace mx {

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
__device__ __forceinline__ uint32_t xcd_block() {
    const uint32_t per = gridDim.x / 8;
    return (blockIdx.x % 8) * per + blockIdx.x / 8;
}

// (b, c, h) of logical block lb over a [B][T][H] grid: 32-bit scalar
// arithmetic (a grid has fewer than 2^32 blocks).
struct BCH {
    uint32_t b, c, h;
};
__device__ __forceinline__ BCH split_bch(uint32_t lb, uint32_t H, uint32_t T) {
    const uint32_t bc = lb / H;
    return BCH{bc / T, bc % T, lb - bc * H};
}

inline unsigned padded_grid(int64_t blocks) { return (unsigned)((blocks + 7) / 8 * 8); }

// Raw buffer resource over [base, base + bytes): 16-byte loads at or past the
// end return zeros and stores there are dropped, and the per-lane offset is a
// 32-bit register beside a scalar base.  Dword 3 is the gfx9 raw-buffer format.
using rsrc_t = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
// The same range starting `off` bytes in (wave-uniform): the resource's own
// base and size move, so the range check covers the shift and the per-lane
// offset stays a small register.
__device__ __forceinline__ rsrc_t buffer_rsrc_at(const void *base, uint32_t bytes, uint32_t off) {
    off = __builtin_amdgcn_readfirstlane(off);
    // every field in scalar registers: a resource in vector registers would
    // need a loop over lanes at each access
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes > off ? bytes - off : 0u);
    return buffer_rsrc(static_cast<const char *>(base) + off, n);
}
__device__ __forceinline__ u32x4 buffer_load16(rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
__device__ __forceinline__ void buffer_store16(u32x4 v, rsrc_t r, uint32_t voff) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, 0);
}
// The same with the nontemporal cache policy (nt), for data not read again
// soon.
__device__ __forceinline__ void buffer_store16_nt(u32x4 v, rsrc_t r, uint32_t voff) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, 2);
}

}  // namespace mx
}  // namespace ssd
