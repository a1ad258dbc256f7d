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
    // an unused slot of a variable-length batch, or a row tile wholly past
    // the end of a short chunk: the chunk output has no rows there
    if (32 * ti >= q) return;
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

// The same tiles and C fragments, a block at a time: 256 threads form every
// causal tile of 8 / NI consecutive (b, c, g) (one for chunk 256, two for
// 128, four for 64).  The block first stages the B rows of its (b, c, g)s in
// LDS with whole-row (coalesced) loads; each wave then holds the C rows of
// one row tile in registers at a time and forms the tiles of that row from
// the staged B rows.  Wave w of a (b, c, g) takes row tiles p and NI-1-p
// (p = w mod NI/2), NI+1 tiles in all, so the waves are evenly loaded.  The
// C rows of a row tile are loaded once for all its tiles (cb_tile loads them
// per tile).  Rows past the end of a short chunk are clamped to its last row,
// as in cb_tile, and row tiles wholly past it are skipped.  `bs` is the
// block's LDS: 256 rows of N + 8 bf16.
template <int Q, int N>
__device__ __forceinline__ void cb_block(const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm,
                                         u32x4 *__restrict__ cb, u32x4 *__restrict__ cfr,
                                         int64_t L, int G, int T, int64_t blk, int64_t ncg,
                                         const int2 *__restrict__ ctab, bf16 *bs) {
    constexpr int NI = Q / 32, NT = NI * (NI + 1) / 2, KS = N / 16;
    constexpr int BPB = 8 / NI;          // (b, c, g)s per block
    constexpr int LDB = N + 8;
    constexpr int SEG = N / 8;           // 16-byte segments per row
    const int tid = threadIdx.x, lane = tid & 63, il = lane & 31, g2 = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const unsigned rs = G * N;
    // stage: row r of the block's 256 is row r % Q of (b, c, g) number r / Q
#pragma unroll
    for (int i = 0; i < 256 * SEG / 256; ++i) {
        const int e = tid + 256 * i, r = e / SEG, sg = e % SEG;
        const int64_t bcg = blk * BPB + r / Q;
        u32x4 v{0u, 0u, 0u, 0u};
        if (bcg < ncg) {
            const int g = (int)(bcg % G);
            const int64_t bc = bcg / G;
            const int c = (int)(bc % T);
            const int64_t b = bc / T;
            const ChunkPos cp = chunk_pos(ctab, c, Q, L);
            if (cp.q > 0) {
                const bf16 *bbase = Bm + ((b * L + cp.t0) * G + g) * N;
                v = *reinterpret_cast<const u32x4 *>(bbase + (unsigned)min(r % Q, cp.q - 1) * rs + 8u * sg);
            }
        }
        *reinterpret_cast<u32x4 *>(bs + r * LDB + 8 * sg) = v;
    }
    __syncthreads();
    const int64_t bcg = blk * BPB + wave / (NI / 2);
    if (bcg >= ncg) return;
    const int g = (int)(bcg % G);
    const int64_t bc = bcg / G;
    const int c = (int)(bc % T);
    const int64_t b = bc / T;
    const ChunkPos cp = chunk_pos(ctab, c, Q, L);
    const int q = cp.q;
    if (q <= 0) return;  // an unused slot of a variable-length batch
    const bf16 *cbase = Cm + ((b * L + cp.t0) * G + g) * N;
    const bf16 *bsg = bs + (wave / (NI / 2)) * Q * LDB;
    const int p = wave % (NI / 2);
#pragma unroll 1
    for (int side = 0; side < 2; ++side) {
        const int ti = side == 0 ? p : NI - 1 - p;
        if (32 * ti >= q) continue;  // wholly past the end of a short chunk
        const unsigned co = (unsigned)min(32 * ti + il, q - 1) * rs + 8u * g2;
        u32x4 crow[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) crow[s] = *reinterpret_cast<const u32x4 *>(cbase + (co + 16u * s));
#pragma unroll 1
        for (int jt = 0; jt <= ti; ++jt) {
            f32x16 acc = zero16();
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u32x4 bb = *reinterpret_cast<const u32x4 *>(bsg + (32 * jt + il) * LDB + 16 * s + 8 * g2);
                acc = mfma32(bb, crow[s], acc);
            }
            u32x4 *o = cb + (bcg * NT + ti * (ti + 1) / 2 + jt) * 256;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                o[v * 64 + lane] = u32x4{__float_as_uint(acc[4 * v]), __float_as_uint(acc[4 * v + 1]),
                                         __float_as_uint(acc[4 * v + 2]), __float_as_uint(acc[4 * v + 3])};
        }
        u32x4 *cf = cfr + (bcg * NI + ti) * KS * 64 + lane;
#pragma unroll
        for (int s = 0; s < KS; ++s) cf[s * 64] = crow[s];
    }
}

}  // namespace mx
}  // namespace ssd
