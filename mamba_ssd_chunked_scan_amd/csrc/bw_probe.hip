// Plain device copy, read and write kernels of known size: the practical HBM
// ceiling the benchmark quotes beside the MI355X spec peak, and the kernels
// whose hardware byte counters calibrate the traffic figures.  Built as a
// separate library for the benchmark; libssd does not contain or call it.
//
// One 16-byte access per thread and 256 threads a block (4 KB a block): on
// this part many short blocks reach a higher rate than fewer blocks with
// several accesses per thread (measured: copy 6.3 against 5.5-5.7 TB/s, read
// 6.7 against 6.3-6.4, write 6.9 against 6.1).  The copy uses nontemporal
// loads and stores (6.7 TB/s).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) k_copy(v4f *__restrict__ dst, const v4f *__restrict__ src,
                                              int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Reads n 16-byte words.  The store depends on the words read, so they are
// kept, but it is taken only when their sum equals `never` (the host passes a
// NaN, which no sum equals): the kernel moves no bytes but the reads.
__global__ void __launch_bounds__(256) k_read(float *__restrict__ out, const v4f *__restrict__ src,
                                              int64_t n, float never) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        const v4f a = src[i];
        const float v = (a.x + a.y) + (a.z + a.w);
        if (v == never) out[blockIdx.x] = v;
    }
}

__global__ void __launch_bounds__(256) k_write(v4f *__restrict__ dst, float value, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = v4f{value, value, value, value};
}

}  // namespace

extern "C" {

// kind 0: copy bytes from src to dst; 1: read bytes of src (dst must hold one
// float per 4 KB of src; nothing is written to it); 2: write bytes of dst.
// bytes must be a multiple of 16, pointers 16-byte aligned.  Returns 0, or -1
// for invalid arguments, or 1 if the launch failed.
int ssd_bw_run(int kind, void *dst, const void *src, size_t bytes, void *stream) {
    if (bytes % 16 || !dst || (kind != 2 && !src) || kind < 0 || kind > 2) return -1;
    if (((uintptr_t)dst | (uintptr_t)src) & 15) return -1;
    const int64_t n = (int64_t)(bytes / 16);
    if (n == 0) return 0;
    const int64_t nb = (n + 255) / 256;
    if (nb > INT32_MAX) return -1;
    const unsigned blocks = (unsigned)nb;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (kind == 0)
        k_copy<<<blocks, 256, 0, st>>>((v4f *)dst, (const v4f *)src, n);
    else if (kind == 1)
        k_read<<<blocks, 256, 0, st>>>((float *)dst, (const v4f *)src, n, __builtin_nanf(""));
    else
        k_write<<<blocks, 256, 0, st>>>((v4f *)dst, 1.0f, n);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
