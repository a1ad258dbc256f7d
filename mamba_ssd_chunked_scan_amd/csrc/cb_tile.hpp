// The C.B tiles of the chunk output, shared by the kernels that form them.
#pragma once

#include "common.hpp"
#include "mfma_ops.hpp"

namespace ssd {
namespace mx {

// ------------------------------------------------------------- C.B tiles
// CB[i][j] = C_i . B_j for the causal 32x32 tiles (row tile ti >= column tile
// jt) of one (b, c, g).  The product does not involve the head, so it is formed
// once here and read by every head of group g.  One wave per tile: the tile is
// S^T = B_jt C_ti^T (rows j, columns i), stored as 4 KB in the register layout
// of that 32x32 accumulator (lane l: column i = l%32; register r: row
// j = 8(r/4) + 4(l/32) + r%4), fp32, so the chunk scan reads it with one
// 16-byte load per lane per unit: unit v (16 bytes at v*1024 + 16 lane) holds
// registers 4v..4v+3.  The scan applies the per-head weights (and on the
// diagonal the mask) before it rounds the tile into MFMA operands.
// Tiles of (b, c, g) are consecutive, tile (ti, jt) at ti(ti+1)/2 + jt.
// The wave of each diagonal tile also stores the row tile's C rows as the
// MFMA operands the chunk scan's state term uses (lane l: row 32 ti + l%32,
// 8 values from column 16 s + 8 (l/32)), at cfr[((b,c,g) NI + ti) KS + s][lane],
// so that the scan reads them as contiguous 1 KB wave loads.
// Tile w (flat over (b, c, g) and the NT causal tiles) by one wave.
template <int Q, int N>
__device__ __forceinline__ void cb_tile(const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm,
                                        u32x4 *__restrict__ cb, u32x4 *__restrict__ cfr,
                                        int64_t L, int G, int T, int64_t w,
                                        const int2 *__restrict__ ctab) {
    constexpr int NI = Q / 32, NT = NI * (NI + 1) / 2, KS = N / 16;
    const int lane = threadIdx.x & 63, il = lane & 31, g2 = lane >> 5;
    const int tile = (int)(w % NT);
    const int64_t bcg = w / NT;
    int ti = 0;
    while ((ti + 1) * (ti + 2) / 2 <= tile) ++ti;
    const int jt = tile - ti * (ti + 1) / 2;
    const int g = (int)(bcg % G);
    const int64_t bc = bcg / G;
    const int c = (int)(bc % T);
    const int64_t b = bc / T;
    const ChunkPos cp = chunk_pos(ctab, c, Q, L);
    const int64_t t0 = cp.t0;
    const int q = cp.q;
    if (q <= 0) return;  // an unused slot of a variable-length batch
    const unsigned rs = G * N;
    const bf16 *bbase = Bm + ((b * L + t0) * G + g) * N;
    const bf16 *cbase = Cm + ((b * L + t0) * G + g) * N;
    // rows past the end of a short chunk are clamped to its last row: finite
    // values that the scan multiplies by zero (x and dt are zero there)
    const unsigned co = (unsigned)min(32 * ti + il, q - 1) * rs + 8u * g2;
    const unsigned bo = (unsigned)min(32 * jt + il, q - 1) * rs + 8u * g2;
    u32x4 crow[KS], brow[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        crow[s] = *reinterpret_cast<const u32x4 *>(cbase + (co + 16u * s));
        brow[s] = *reinterpret_cast<const u32x4 *>(bbase + (bo + 16u * s));
    }
    f32x16 acc = zero16();
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = mfma32(brow[s], crow[s], acc);
    u32x4 *o = cb + (bcg * NT + tile) * 256;
#pragma unroll
    for (int v = 0; v < 4; ++v)
        o[v * 64 + lane] = u32x4{__float_as_uint(acc[4 * v]), __float_as_uint(acc[4 * v + 1]),
                                 __float_as_uint(acc[4 * v + 2]), __float_as_uint(acc[4 * v + 3])};
    if (jt == ti) {
        u32x4 *cf = cfr + (bcg * NI + ti) * KS * 64 + lane;
#pragma unroll
        for (int s = 0; s < KS; ++s) cf[s * 64] = crow[s];
    }
}

}  // namespace mx
}  // namespace ssd
