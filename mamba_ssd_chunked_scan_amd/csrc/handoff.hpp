// Block-to-block hand-off of chunk states within one kernel: device-scope
// (sc1) stores and loads of the state data, and a 64-bit flag per published
// piece (bit 0 set, the chunk's decay in the high word).
//
// Visibility across XCDs.  A device-wide release or acquire fence writes back
// or invalidates a whole L2, so the hand-off avoids them: the data and the
// flags are written and read with device-scope (sc1) accesses, which bypass
// the non-coherent caches; a wave's stores are complete (s_waitcnt vmcnt(0))
// before it writes the flag that publishes them, and a reader issues its data
// loads only after its flag load has returned.
//
// Every wait is bounded: one that runs out sets bit 0 of the error word and
// goes on as if the flag were set (a zero decay word), so a broken hand-off
// shows up as a flagged wrong result instead of a hang.
#pragma once

#include "mfma_ops.hpp"

namespace ssd {
namespace mx {

constexpr uint32_t kSpinLimit = 1u << 20;  // flag polls before a wait gives up

// Device-scope stores and loads (cache policy sc1) at byte offset voff of a
// wave-uniform buffer resource: 16 bytes, or 4.
__device__ __forceinline__ void st16_dev(rsrc_t r, uint32_t voff, float a, float b, float c, float d) {
    const u32x4 v{__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, 16);
}
__device__ __forceinline__ u32x4 ld16_dev(rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 16));
}
__device__ __forceinline__ void st4_dev(rsrc_t r, uint32_t voff, float a) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), r, voff, 0, 16);
}
__device__ __forceinline__ float ld4_dev(rsrc_t r, uint32_t voff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 16));
}

// Wait (bounded) until the flag at f is set; returns its decay word.  The
// caller's loads that follow are issued after the flag load returned.
__device__ __forceinline__ float wait_flag(const unsigned long long *f, unsigned *err) {
    unsigned long long v = 0;
    uint32_t n = 0;
    while (true) {
        v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (v & 1ull) break;
        if (++n >= kSpinLimit) {
            __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            v = 1ull;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return __uint_as_float((uint32_t)(v >> 32));
}

// Publish: the wave's stores are complete before the flag is written.
__device__ __forceinline__ void set_flag(unsigned long long *f, float r) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __hip_atomic_store(f, ((unsigned long long)__float_as_uint(r) << 32) | 1ull, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace mx
}  // namespace ssd
