// bf16 MFMA kernels (fp32 accumulation) for the two contraction stages of the
// chunked SSD scan: each chunk's own state, and the chunk output.  They cover
// headdim 64, d_state 64 or 128 and chunk 64, 128 or 256 with bf16 x/B/C; any
// other shape runs the generic kernels.
//
// Stage structure ("Compiler-First State Space Duality and Portable O(1)
// Autoregressive Caching for Inference", paperlayer summary, §3 Method,
// "Chunked recurrence", and the three contractions listed in B.5):
//   chunk state   S[p,n]  = sum_j x[j,p] w_j B[j,n],  w_j = dt_j exp(Acs_last - Acs_j)
//   chunk output  y[i,p]  = sum_{j<=i} (C_i.B_j) exp(Acs_i - Acs_j) dt_j x[j,p]
//                           + exp(Acs_i) (C_i . H[p]) + D x[i,p]
// The causal mask is the fixed lower triangle of the chunk ("Primitive-level
// implementation" in the same section): tiles above the diagonal are skipped
// outright and only the diagonal 32x32 tiles are masked element by element.
//
// gfx950 specifics used here:
//  * the MFMA lane layout and the LDS transpose read (mfma_ops.hpp);
//  * v_cvt_pk_bf16_f32 for round-to-nearest-even packing.
//  * blocks are dealt to the 8 XCDs round-robin; the block index is remapped
//    so that the heads of one (batch, chunk) run on one XCD and share its L2
//    copy of the chunk's B and C rows.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "mfma_ops.hpp"
#include "stages.hpp"
#include "cb_tile.hpp"
#include "handoff.hpp"
#include "ssd.h"

namespace ssd {
namespace {

constexpr int kP = 64;   // headdim handled here
constexpr int kChainCtlWords = 64;  // control words before the hand-off flags
constexpr int kChainQueues = 8;     // work queues of the chained state pass, one per XCD
constexpr int kJT = 32;  // tokens per streamed stage (one 32-row tile)

using namespace mx;

// Registers holding one 32-token stage between its global load and its LDS
// store: one 8-value x segment (XW 16-byte words: 1 for bf16 x, 2 for fp32)
// and NBV 16-byte B segments per thread.  Two sets give a prefetch distance
// of two stages.
template <int NBV, int XW>
struct StageRegs {
    u32x4 x[XW];
    u32x4 b[NBV];
};

using P0 = std::integral_constant<int, 0>;
using P1 = std::integral_constant<int, 1>;

// ------------------------------------------------------------ chunk state
// One block (4 waves) per (b, c, h).  S (64 x N fp32) = xw^T B, streamed over
// the chunk in 32-token stages (double-buffered; the next stage's global loads
// are in flight while the current one is multiplied).  xw = x * w is formed in
// fp32 and stored as a hi/lo bf16 pair, so its rounding stays near fp32
// level.  Both operands are read with the LDS transpose read.  Output tiles
// 32x32: wave w owns tiles w and w+4 of the (p-tile, n-tile) grid.
//
// kCumsum: the block also forms its chunk's cumulative log-decay (an in-block
// prefix sum of dt*A over the chunk's tokens) and writes it to Acs for the
// later stages, instead of reading it.  It then also applies the dt
// activation `act` and, when dt_out is given, writes the activated dt there.
// kAdjoint (the gradient's chunk term, with x = dy and B = C): the weight is
// exp(Acs_j), the decay from the chunk's entering state to token j.  TX: x's
// type; fp32 x (the gradient's dy behind a gate, kept unrounded) is weighted
// and split like bf16 x.
//
// kChain: the block also passes the state on ("Chunked recurrence": the state
// entering chunk c+1 is the one entering chunk c decayed over the chunk plus
// the chunk's own state), so the chunk states never take a separate pass.
// Blocks take their items by atomic tickets from eight work queues, one per
// XCD, each holding a contiguous range of heads (for 8 groups of 10 heads,
// queue q is group q), in chunk-major order within the queue (every batch row
// and head of the range for chunk c before chunk c+1; chunk slots in order for
// a variable-length batch).  A block draws from the queue of the XCD it runs
// on (the XCC_ID hardware register), so the heads that share B rows share that
// XCD's L2 copy, and from the others in turn once its own is empty.  A block
// waits only for its predecessor chunk of the same (sequence, head), which
// sits in the same queue under a smaller ticket: it was taken by a block that
// is already running and waits only for smaller tickets itself, so progress
// never depends on the order in which blocks are dispatched or on which XCD
// runs what.  There are as many blocks as items and each takes exactly one, so
// every item is taken.  Each
// wave waits for and publishes its own two 32x32 tiles of the 64 x N state
// (one flag per (chunk, head, wave)), through the sc1 hand-off of
// handoff.hpp: it reads the state entering its chunk from the `states` slot
// of the chunk (written there by the predecessor; the initial state or zero
// for a sequence's first chunk, which the block stores there itself for the
// output stage) and stores the state entering the next chunk into the next
// slot, or the final state after a sequence's last chunk.
struct ChainArgs {
    const float *init;            // [sequences][H][P][N] or null (zero)
    float *fin;                   // [sequences][H][P][N] or null
    unsigned long long *flags;    // [slots][H][4]: the state entering slot+1 is stored
    unsigned *ctl;                // [1] error word, [8 + q] ticket of queue q; zeroed before the launch
    const int2 *sch;              // variable-length batch: sequence -> (first slot, slots)
    const int2 *spos;             // slot -> (sequence, position in it)
    int64_t B;                    // batch rows (fixed-length batch)
};

template <int Q, int N, bool kCumsum, bool kAdjoint = false, typename TX = bf16,
          bool kChain = false>
__global__ void __launch_bounds__(256, 2)
k_chunk_state_mfma(const TX *__restrict__ x, const bf16 *__restrict__ Bm,
                   const float *__restrict__ dt, const float *__restrict__ A,
                   float *__restrict__ Acs, float *__restrict__ states, int64_t L, int H, int G,
                   int T, int64_t nblocks, DtAct act, float *__restrict__ dt_out,
                   const int2 *__restrict__ ctab, const ChainArgs ca = ChainArgs{}) {
    static_assert(!kChain || (kCumsum && !kAdjoint), "the chain runs with the in-block cumsum");
    constexpr int LDX = kP + 16;              // x stage row stride (bf16)
    constexpr int LDB = N + 16;               // B stage row stride (bf16)
    constexpr int NST = Q / kJT;              // stages per chunk
    constexpr int BSEG = N / 8;               // 16-byte segments per B row
    constexpr int NBV = kJT * BSEG / 256;     // B segments per thread per stage
    __shared__ __attribute__((aligned(16))) bf16 xhi[2][kJT * LDX];
    __shared__ __attribute__((aligned(16))) bf16 xlo[2][kJT * LDX];
    __shared__ __attribute__((aligned(16))) bf16 bst[2][kJT * LDB];
    __shared__ float w[Q];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int h, c;
    int64_t b;
    if constexpr (kChain) {
        __shared__ int item_s[3];
        if (tid == 0) {
            const uint32_t rows = ctab ? 1u : (uint32_t)ca.B;
            const int home = (int)(__builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & 7);
            int hh = -1, cc = 0, bb = 0;
            for (int k = 0; k < kChainQueues && hh < 0; ++k) {
                const int qu = (home + k) % kChainQueues;
                const int h0 = (int)(((int64_t)qu * H) / kChainQueues);
                const int h1 = (int)(((int64_t)(qu + 1) * H) / kChainQueues);
                const uint32_t nh = (uint32_t)(h1 - h0);
                if (nh == 0) continue;
                const uint32_t tk = __hip_atomic_fetch_add(ca.ctl + 8 + qu, 1u, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
                if (tk >= rows * (uint32_t)T * nh) continue;
                // chunk-major within the queue: ticket = (c * rows + b) * nh + (h - h0)
                const uint32_t cb_ = tk / nh;
                hh = h0 + (int)(tk - cb_ * nh);
                cc = (int)(cb_ / rows);
                bb = (int)(cb_ - (uint32_t)cc * rows);
            }
            item_s[0] = hh;
            item_s[1] = cc;
            item_s[2] = bb;
        }
        __syncthreads();
        h = __builtin_amdgcn_readfirstlane(item_s[0]);
        if (h < 0) return;  // not reached: there are as many blocks as items
        c = __builtin_amdgcn_readfirstlane(item_s[1]);
        b = __builtin_amdgcn_readfirstlane(item_s[2]);
    } else {
        const uint32_t lb = xcd_block();
        if (lb >= nblocks) return;
        const BCH ix = split_bch(lb, H, T);
        h = ix.h;
        c = ix.c;
        b = ix.b;
    }
    const int g = h / (H / G);
    const ChunkPos cp = chunk_pos(ctab, c, Q, L);
    const int64_t t0 = cp.t0;
    const int q = cp.q;
    if (q <= 0) return;  // an unused slot of a variable-length batch
    const TX *xbase = x + ((b * L + t0) * H + h) * kP;
    const bf16 *bbase = Bm + ((b * L + t0) * G + g) * N;
    // per-thread offsets are unsigned 32-bit from block-uniform bases (a
    // chunk spans < 2^31 elements of x, B, C and y), so loads and stores use
    // the scalar-base + 32-bit-offset address form and no 64-bit addresses
    // are kept in vector registers
    const unsigned xrs = H * kP, brs = G * N;
    const int xrow = tid >> 3, xseg = tid & 7;

    // weights first: every stage needs them (Q <= 256: one token per thread)
    float total = 0.f;  // Acs at the chunk's last token: its whole log-decay
    if constexpr (kCumsum) {
        __shared__ float wsum[4];
        __shared__ float last_s;
        float d = 0.f;
        if (tid < q) {
            const int64_t di = (b * L + t0 + tid) * H + h;
            d = act_dt(act, dt[di], h);
            if (dt_out) dt_out[di] = d;
        }
        const float v = wave_inclusive_scan(d * A[h], lane);
        if (lane == 63) wsum[wave] = v;
        __syncthreads();
        float acs = v;
        for (int k = 0; k < wave; ++k) acs += wsum[k];
        if (tid < q) Acs[(b * H + h) * L + t0 + tid] = acs;
        if (tid == q - 1) last_s = acs;
        __syncthreads();
        total = last_s;
        if (tid < Q) w[tid] = tid < q ? d * ssd_exp(total - acs) : 0.f;
    } else {
        const float *acs = Acs + (b * H + h) * L + t0;
        const float last = acs[q - 1];
        if (tid < Q) {
            const int jj = min(tid, q - 1);
            const float v = kAdjoint ? ssd_exp(acs[jj])
                                     : dt[(b * L + t0 + jj) * H + h] * ssd_exp(last - acs[jj]);
            w[tid] = tid < q ? v : 0.f;
        }
    }
    constexpr int XW = sizeof(TX) / 2;
    StageRegs<NBV, XW> R[2];
    auto load_stage = [&](int st, StageRegs<NBV, XW> &r) {
        const int j = st * kJT + xrow;
        const TX *xp = xbase + ((unsigned)min(j, q - 1) * xrs + xseg * 8u);
#pragma unroll
        for (int k = 0; k < XW; ++k) r.x[k] = *reinterpret_cast<const u32x4 *>(xp + k * (8 / XW));
#pragma unroll
        for (int i = 0; i < NBV; ++i) {
            const int e = tid + 256 * i, rr = e / BSEG, sg = e % BSEG;
            r.b[i] = *reinterpret_cast<const u32x4 *>(bbase + ((unsigned)min(st * kJT + rr, q - 1) * brs + sg * 8u));
        }
    };
    auto store_stage = [&](int st, int buf, const StageRegs<NBV, XW> &r) {
        const int j = st * kJT + xrow;
        const float wj = w[j];  // zero at and beyond q
        float v[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if constexpr (XW == 1) {
                v[2 * k] = lo_bf16(r.x[0][k]) * wj;
                v[2 * k + 1] = hi_bf16(r.x[0][k]) * wj;
            } else {
                v[2 * k] = __uint_as_float(r.x[(2 * k) / 4][(2 * k) % 4]) * wj;
                v[2 * k + 1] = __uint_as_float(r.x[(2 * k + 1) / 4][(2 * k + 1) % 4]) * wj;
            }
        }
        u32x4 hi, lo;
        split8(v, hi, lo);
        *reinterpret_cast<u32x4 *>(&xhi[buf][xrow * LDX + xseg * 8]) = masked(hi, j < q);
        *reinterpret_cast<u32x4 *>(&xlo[buf][xrow * LDX + xseg * 8]) = masked(lo, j < q);
#pragma unroll
        for (int i = 0; i < NBV; ++i) {
            const int e = tid + 256 * i, rr = e / BSEG, sg = e % BSEG;
            *reinterpret_cast<u32x4 *>(&bst[buf][rr * LDB + sg * 8]) =
                masked(r.b[i], st * kJT + rr < q);
        }
    };

    // stages that hold tokens of this chunk: a short chunk (the last of a
    // sequence) skips the stages after them, rounded up to the pair the loop
    // below takes at a time (their x and B rows are masked to zero, so they
    // would add exact zeros)
    const int nst = NST == 1 ? 1
                              : __builtin_amdgcn_readfirstlane(
                                    min(NST, 2 * ((q + 2 * kJT - 1) / (2 * kJT))));

    // prefetch distance two: stage s+2's loads are issued while stage s is
    // multiplied and stage s+1 (already in registers) is written to LDS
    load_stage(0, R[0]);
    if (NST > 1) load_stage(1, R[1]);
    __syncthreads();  // w complete
    store_stage(0, 0, R[0]);
    __syncthreads();

    constexpr int NT = N / 32, TPW = (2 * NT) / 4;
    f32x16 acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t] = zero16();
    // lim: the stages run (nst, or the constant NST for a whole chunk)
    auto step = [&](int st, int lim, auto par) {
        constexpr int PAR = decltype(par)::value;  // st % 2, the LDS buffer
        if (st + 2 < lim) load_stage(st + 2, R[PAR]);
#pragma unroll
        for (int ks = 0; ks < kJT / 16; ++ks) {
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int tile = wave + 4 * t, pt = tile / NT, nt = tile % NT;
                const u32x4 ah = tr_operand<false>(xhi[PAR], LDX, 16 * ks, 32 * pt);
                const u32x4 al = tr_operand<false>(xlo[PAR], LDX, 16 * ks, 32 * pt);
                const u32x4 bb = tr_operand<false>(bst[PAR], LDB, 16 * ks, 32 * nt);
                acc[t] = mfma32(ah, bb, acc[t]);
                acc[t] = mfma32(al, bb, acc[t]);
            }
        }
        if (st + 1 < lim) store_stage(st + 1, PAR ^ 1, R[PAR ^ 1]);
        __syncthreads();
    };
    if constexpr (NST == 1) {  // a 32-token chunk: one stage
        step(0, 1, P0{});
    } else if (nst == NST) {  // a whole chunk: the loop unrolled at compile time
        for (int st = 0; st < NST; st += 2) {  // NST is even
            step(st, NST, P0{});
            step(st + 1, NST, P1{});
        }
    } else {  // a short chunk
#pragma unroll 1
        for (int st = 0; st < nst; st += 2) {  // nst is even
            step(st, nst, P0{});
            step(st + 1, nst, P1{});
        }
    }
    // this lane's element r of tile t: row p, column n of the 64 x N state
    auto eoff = [&](int t, int r) {
        const int tile = wave + 4 * t, pt = tile / NT, nt = tile % NT;
        const int p = pt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        return (uint32_t)(p * N + nt * 32 + (lane & 31));
    };
    constexpr int64_t PN = (int64_t)kP * N;
    const int64_t here = ((b * T + c) * H + h);  // this chunk's state slot
    if constexpr (!kChain) {
        float *out = states + here * PN;
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) out[eoff(t, r)] = acc[t][r];
    } else {
        int64_t seq = b;
        int pos = c, npos = T;
        if (ctab) {
            const int2 sp = ca.spos[c];
            seq = sp.x;
            pos = sp.y;
            npos = ca.sch[seq].y;
        }
        unsigned long long *flag = ca.flags + here * 4 + wave;
        float hin[TPW][16];
        if (pos == 0) {
            // the initial state (read before anything of this sequence is
            // published: the final state may overwrite it), also stored as
            // the state entering this chunk for the output stage
            const float *ip = ca.init ? ca.init + (seq * H + h) * PN : nullptr;
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) hin[t][r] = ip ? ip[eoff(t, r)] : 0.f;
            float *out = states + here * PN;
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) out[eoff(t, r)] = hin[t][r];
        } else {
            wait_flag(flag - 4 * H, ca.ctl + 1);  // the previous chunk, same head and wave
            const rsrc_t rs = buffer_rsrc(states + here * PN, (uint32_t)(PN * 4));
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) hin[t][r] = ld4_dev(rs, eoff(t, r) * 4u);
        }
        const float rc = ssd_exp(total);
        if (pos == npos - 1) {
            if (ca.fin) {
                float *fp = ca.fin + (seq * H + h) * PN;
#pragma unroll
                for (int t = 0; t < TPW; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) fp[eoff(t, r)] = fmaf(rc, hin[t][r], acc[t][r]);
            }
        } else {
            const rsrc_t rs = buffer_rsrc(states + (here + H) * PN, (uint32_t)(PN * 4));
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    st4_dev(rs, eoff(t, r) * 4u, fmaf(rc, hin[t][r], acc[t][r]));
            set_flag(flag, rc);
        }
    }
}

template <int Q, int N>
__global__ void __launch_bounds__(256)
k_chunk_cb_mfma(const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm, u32x4 *__restrict__ cb,
                int64_t L, int G, int T, int64_t ntiles, const int2 *__restrict__ ctab) {
    const int64_t w = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= ntiles) return;
    cb_tile<Q, N>(Bm, Cm, cb, cb + ntiles * 256, L, G, T, w, ctab);
}

// Before the chained chunk-state launch: the first nzb blocks clear its
// hand-off flags and control words (a kernel, not a memset, so that the call
// can be captured in a graph), the rest form the C.B tiles: a block per
// 8 / NI (b, c, g)s (cb_block) when there are many of them (kBlock), else a
// wave per tile (cb_tile), whose short waves finish sooner when the few
// blocks of a small grid cannot fill the chip.
template <int Q, int N, bool kBlock>
__global__ void __launch_bounds__(256)
k_chain_prep(const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm, u32x4 *__restrict__ cb,
             int64_t L, int G, int T, int64_t ntiles, const int2 *__restrict__ ctab,
             unsigned long long *__restrict__ flags, int64_t nflags, unsigned *__restrict__ ctl,
             int64_t nzb, int64_t ncg) {
    __shared__ __attribute__((aligned(16))) bf16 bs[kBlock ? 256 * (N + 8) : 8];
    const int64_t blk = blockIdx.x;
    if (blk < nzb) {
        const int64_t i = blk * 256 + threadIdx.x;
        if (i < nflags) flags[i] = 0ull;
        if (blk == 0 && threadIdx.x < kChainCtlWords) ctl[threadIdx.x] = 0u;
        return;
    }
    if constexpr (kBlock) {
        cb_block<Q, N>(Bm, Cm, cb, cb + ntiles * 256, L, G, T, blk - nzb, ncg, ctab, bs);
    } else {
        const int64_t w = (blk - nzb) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        if (w >= ntiles) return;
        cb_tile<Q, N>(Bm, Cm, cb, cb + ntiles * 256, L, G, T, w, ctab);
    }
}

// (b, c, g)s from which the C.B tiles are formed a block at a time: below,
// the blocks of cb_block would be too few to fill the chip (measured on
// MI355X: 16 (b, c, g)s of chunk 256 take 23 us that way against 6 us a wave
// per tile; 4096 take 321 us against 579 us).
constexpr int64_t kCbBlockMin = 512;

// The inter-chunk state pass and the C.B tiles in one launch: the first
// nsp blocks pass states (memory-bound), the rest form C.B tiles on the
// otherwise idle matrix cores.  Both only read what the chunk-state stage
// and the inputs provide, and both feed the chunk-output stage.
template <int Q, int N>
__global__ void __launch_bounds__(256)
k_state_passing_cb(float *__restrict__ states, const float *__restrict__ Acs, const float *init,
                   float *fin, int64_t L, int H, int64_t PN, int T, int64_t nsp, int ny,
                   const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm,
                   u32x4 *__restrict__ cb, int G, int64_t ntiles, const int2 *__restrict__ ctab,
                   const int2 *__restrict__ sch) {
    const int64_t blk = blockIdx.x;
    if (blk < nsp) {
        const int64_t e = ((blk % ny) * 256 + threadIdx.x) * 4;
        if (e >= PN) return;
        state_passing_body(states, Acs, init, fin, blk / ny, e, L, H, PN, Q, T, ctab, sch);
        return;
    }
    const int64_t w = (blk - nsp) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= ntiles) return;
    cb_tile<Q, N>(Bm, Cm, cb, cb + ntiles * 256, L, G, T, w, ctab);
}

// ------------------------------------------------------------- chunk scan
// One block per (b, c, h) with one wave per 32-row output tile (NI = Q/32
// waves).  Wave w owns tile w for w < NI/2 and tile 3NI/2-1-w otherwise, so
// the two waves that share a SIMD (w and w + NI/2 when waves are dealt to the
// 4 SIMDs in turn) together make NI+1 causal tile visits.  The wave keeps
// Z = Y^T of its tile (64 x 32 fp32, two accumulators over p).  With
// e(t) = 32t + 31 the last row of tile t, Acs_{e(-1)} = 0 and ae =
// Acs_{e(ti-1)}, the output row i of tile ti is
//   y_i = exp(Acs_i - ae) Z_i + diagonal-tile part + D x_i,
//   Z   = exp(ae) C_i.H + sum_{jt < ti} sum_{j in jt} CB[i][j] F_jt w_j x_j,
//         w_j = exp(Acs_{e(jt)} - Acs_j) dt_j,  F_jt = exp(ae - Acs_{e(jt)}),
// which is the chunk output of the reference form regrouped by 32-row tiles:
// every exponent is <= 0, so nothing overflows, and an underflow drops only
// terms that are at least as small in the exact result.  The off-diagonal
// visits are independent accumulations into Z.
//
// The block stages the entering state H and the chunk's raw x (bf16, exact)
// in LDS once: H first, for the state term, while x is still arriving, and x
// after it.  After those two block barriers each wave runs its own visits
// with no further barrier, so the waves on a SIMD interleave freely and none
// waits for another's tile; the waves with longer chains of visits run at a
// higher wave priority.  The off-diagonal weight F_jt w_j (w_j one value per
// token, formed once per block) goes onto the fp32 C.B tile: the wave forms
// CBw[i][j] = CB[i][j] F_jt w_j in registers as a hi/lo bf16 pair, and the
// product with exact x takes two MFMAs.  The diagonal tile applies
// exp(Acs_i - Acs_j) dt_j under the causal mask element by element (hi/lo
// too), and the state term takes H as a hi/lo pair against the exact C
// operand fragments from the C.B kernel.  The next visit's C.B tile is loaded
// while the current one is multiplied.
//
// Every global access is a whole-line wave access: x rows, H, the C operand
// fragments and C.B tiles (1 KB each) from the C.B kernel, and y rows, which
// go out through the wave's own LDS rows as full 128-byte rows.  Loops and
// branches depend on wave-uniform values only.
//
// kGate: every y value is multiplied by silu(z) (z in y's layout) in fp32
// before its rounding to bf16.
template <int Q, int N, bool kGate>
__global__ void __launch_bounds__(Q * 2) __attribute__((amdgpu_waves_per_eu(Q == 256 ? 4 : 2)))
k_chunk_scan_mfma(const bf16 *__restrict__ x, const float *__restrict__ dt,
                  const float *__restrict__ D, const float *__restrict__ Acs,
                  const float *__restrict__ states, const u32x4 *__restrict__ cb,
                  const u32x4 *__restrict__ cfr, bf16 *__restrict__ y,
                  const bf16 *__restrict__ z, int64_t L, int H, int G, int T, int64_t nblocks,
                  const int2 *__restrict__ ctab) {
    constexpr int NI = Q / 32, NT = NI * (NI + 1) / 2, KS = N / 16;
    constexpr int TH = Q * 2;             // threads: NI waves
    constexpr int LDH = N + 8;            // H rows, read as plain 16-byte operands
    constexpr int LDX = kP + 8;           // x rows, read transposed
    constexpr int LDY = kP + 8;           // bf16 y staging rows
    constexpr int H_BYTES = 2 * kP * LDH * 2;
    constexpr int Y_BYTES = NI * 32 * LDY * 2;
    constexpr int U_BYTES = H_BYTES > Y_BYTES ? H_BYTES : Y_BYTES;
    constexpr int NXV = Q * kP / 8 / TH;  // 16-byte x segments per thread
    constexpr int NHV = kP * N / 4 / TH;  // float4 of H per thread
    static_assert(NXV * TH * 8 == Q * kP && NHV * TH * 4 == kP * N, "staging split");
    // H (until the state term is done), then the per-wave y staging rows
    __shared__ __attribute__((aligned(16))) char hu[U_BYTES];
    __shared__ __attribute__((aligned(16))) bf16 xs[Q * LDX];
    __shared__ __attribute__((aligned(16))) float acs_s[Q];
    __shared__ __attribute__((aligned(16))) float dt_s[Q];
    __shared__ __attribute__((aligned(16))) float w_s[Q];
    const uint32_t lb = xcd_block();
    if (lb >= nblocks) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int il = lane & 31, g2 = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ti = wave < NI / 2 ? wave : 3 * NI / 2 - 1 - wave;
    const BCH ix = split_bch(lb, H, T);
    const int h = ix.h, c = ix.c;
    const int64_t b = ix.b;
    const int g = h / (H / G);
    const ChunkPos cp = chunk_pos(ctab, c, Q, L);
    const int64_t t0 = cp.t0;
    const int q = cp.q;
    if (q <= 0) return;  // an unused slot of a variable-length batch
    const bf16 *xbase = x + ((b * L + t0) * H + h) * kP;
    // per-thread offsets are unsigned 32-bit from block-uniform bases (a
    // chunk spans < 2^31 bytes of x and y), so loads and stores use the
    // scalar-base + 32-bit-offset address form
    const unsigned xrs = H * kP;
    const int64_t bcg = (b * T + c) * G + g;
    const u32x4 *cbg = cb + bcg * NT * 256;

    // x rows of this chunk and head: bytes up to the end of row q-1, so rows
    // past a short chunk's end read as zeros; y rows likewise (stores dropped)
    const uint32_t xy_bytes = ((unsigned)(q - 1) * xrs + kP) * 2u;
    // the fp32 C.B tile (ti, jt <= ti) as four 16-byte operands of this lane
    const uint32_t cbvoff = lane * 16u;
    auto load_cb = [&](int jt, u32x4 (&o)[4]) __attribute__((always_inline)) {
        const int tile = ti * (ti + 1) / 2 + jt;
        const rsrc_t r = buffer_rsrc_at(cbg, (tile + 1) * 4096u, tile * 4096u);
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = buffer_load16(r, cbvoff + k * 1024u);
    };

    // ---- prologue: global loads in the order they are needed
    float acs_v = 0.f, dt_v = 0.f;
    if (tid < Q) {
        const float *acs = Acs + (b * H + h) * L + t0;
        const int jj = min(tid, q - 1);
        acs_v = acs[jj];
        dt_v = dt[(b * L + t0 + jj) * H + h];
        if (tid >= q) {
            acs_v = acs[q - 1];
            dt_v = 0.f;
        }
    }
    const float *Hc = states + ((b * T + c) * H + h) * (int64_t)(kP * N);
    float4 hv[NHV];
#pragma unroll
    for (int i = 0; i < NHV; ++i) hv[i] = *reinterpret_cast<const float4 *>(Hc + 4 * (tid + TH * i));
    u32x4 cf[KS];
    {
        const u32x4 *f = cfr + (bcg * NI + ti) * KS * 64 + lane;
#pragma unroll
        for (int s = 0; s < KS; ++s) cf[s] = f[s * 64];
    }
    // x after what the state term needs (loads complete in issue order)
    u32x4 xv[NXV];
    {
        const rsrc_t xr = buffer_rsrc_at(xbase, xy_bytes, 0u);
#pragma unroll
        for (int i = 0; i < NXV; ++i) {
            const int e = tid + TH * i;
            xv[i] = buffer_load16(xr, ((unsigned)(e >> 3) * xrs + 8u * (e & 7)) * 2u);
        }
    }
    u32x4 cbr[4];  // the C.B tile of the wave's next visit
    load_cb(0, cbr);
    if (tid < Q) {
        // w_j needs Acs at its tile's last row, held by lane 31 of its half-wave
        const float ae = __shfl(acs_v, lane | 31);
        acs_s[tid] = acs_v;
        dt_s[tid] = dt_v;
        w_s[tid] = ssd_exp(ae - acs_v) * dt_v;  // 0 past q
    }
    bf16 *Hh = reinterpret_cast<bf16 *>(hu);
    bf16 *Hl = Hh + kP * LDH;
#pragma unroll
    for (int i = 0; i < NHV; ++i) {
        const int e = tid + TH * i, p = e / (N / 4), n = (e % (N / 4)) * 4;
        u32x2 hh, hl;
        uint32_t l0, l1;
        hh[0] = split2(hv[i].x, hv[i].y, l0);
        hh[1] = split2(hv[i].z, hv[i].w, l1);
        hl[0] = l0;
        hl[1] = l1;
        *reinterpret_cast<u32x2 *>(Hh + p * LDH + n) = hh;
        *reinterpret_cast<u32x2 *>(Hl + p * LDH + n) = hl;
    }
    __syncthreads();  // acs_s, dt_s, w_s, H (x is still arriving)

    // state term Z = H C_i^T
    f32x16 Z[2] = {zero16(), zero16()};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
            const int ho = (pt * 32 + il) * LDH + 16 * s + 8 * g2;
            const u32x4 ah = *reinterpret_cast<const u32x4 *>(Hh + ho);
            const u32x4 al = *reinterpret_cast<const u32x4 *>(Hl + ho);
            Z[pt] = mfma32(ah, cf[s], Z[pt]);
            Z[pt] = mfma32(al, cf[s], Z[pt]);
        }
    }
#pragma unroll
    for (int i = 0; i < NXV; ++i) {
        const int e = tid + TH * i;
        *reinterpret_cast<u32x4 *>(&xs[(e >> 3) * LDX + 8 * (e & 7)]) = xv[i];
    }
    __syncthreads();  // x staged; H no longer read: its LDS becomes the y staging rows
    // a wave whose 32 rows all lie past the end of a short chunk (the last of
    // a sequence) has no output: it leaves here (no block barrier follows)
    if (ti * 32 >= q) return;

    bf16 *ys = reinterpret_cast<bf16 *>(hu) + wave * 32 * LDY;
    const bf16 *ybase = y + ((b * L + t0) * H + h) * kP;
    if constexpr (kGate) {
        // the wave's z tile (32 rows x 128 bytes) copied straight into its
        // staging rows, unpadded, four 1 KB buffer-to-LDS loads (lane i's 16
        // bytes land at 16 i; rows past a short chunk's end arrive as zeros);
        // the rows are not used for y until this wave's epilogue
        static_assert(32 * kP * 2 <= 32 * LDY * 2, "z tile fits the staging rows");
        const bf16 *zbase = z + ((b * L + t0) * H + h) * kP;
        const rsrc_t zr = buffer_rsrc_at(zbase, xy_bytes, (unsigned)(ti * 32) * xrs * 2u);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                zr, (__attribute__((address_space(3))) void *)(ys + kk * 512), 16,
                ((unsigned)((lane >> 3) + 8 * kk) * xrs + 8u * (lane & 7)) * 2u, 0, 0, 0);
    }
    const float Dh = D ? D[h] : 0.f;

    // off-diagonal visits.  With ae = Acs_{e(ti-1)}, the state term and every
    // off-diagonal term reach row i through the diagonal's exp(Acs_i - ae), so
    // Z is scaled by exp(ae) once and tile jt enters with the weight
    // exp(ae - Acs_j) dt_j = F_jt w_j, F_jt = exp(ae - Acs_{e(jt)}): the visits
    // are independent accumulations, and none waits on another's result.
    // CBw = CB F_jt w_j (hi/lo) multiplies the exact x rows of tile jt; the
    // next visit's C.B tile is loaded once this one is weighted.
    // the waves with the longest chains of visits issue first when several
    // are ready: a block ends with its slowest wave
    if (ti >= 6) __builtin_amdgcn_s_setprio(3);
    else if (ti >= 4) __builtin_amdgcn_s_setprio(2);
    else if (ti >= 2) __builtin_amdgcn_s_setprio(1);
    const float ae = ti > 0 ? acs_s[ti * 32 - 1] : 0.f;
    {
        const float fs = ssd_exp(ae);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
            for (int r = 0; r < 16; ++r) Z[pt][r] *= fs;
    }
#pragma unroll 1
    for (int jt = 0; jt < ti; ++jt) {
        const float F = ssd_exp(ae - acs_s[jt * 32 + 31]);
        u32x4 wh[2], wl[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float m[8];
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const float4 wj = *reinterpret_cast<const float4 *>(&w_s[jt * 32 + 16 * u + 8 * v + 4 * g2]);
                const u32x4 cv = cbr[2 * u + v];
                m[4 * v + 0] = __uint_as_float(cv[0]) * (wj.x * F);
                m[4 * v + 1] = __uint_as_float(cv[1]) * (wj.y * F);
                m[4 * v + 2] = __uint_as_float(cv[2]) * (wj.z * F);
                m[4 * v + 3] = __uint_as_float(cv[3]) * (wj.w * F);
            }
            split8(m, wh[u], wl[u]);
        }
        load_cb(jt + 1, cbr);  // the next visit's tile (the diagonal one last)
        const bf16 *xt = xs + jt * 32 * LDX;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                const u32x4 xa = tr_operand<true>(xt, LDX, 16 * u, 32 * pt);
                Z[pt] = mfma32(xa, wh[u], Z[pt]);
                Z[pt] = mfma32(xa, wl[u], Z[pt]);
            }
    }

    // diagonal visit: M[i][j] = CB[i][j] exp(Acs_i - Acs_j) dt_j for j <= i
    // (registers 8u+4v..+3 of this lane hold rows jl..jl+3, jl = 16u + 8v +
    // 4(l/32)), as hi/lo pairs in mo[2u], mo[2u+1].  Masked elements are
    // computed anyway and replaced by 0 with a select (their exponent may be
    // positive and their product not finite; the select discards it).
    {
        const float ai = acs_s[ti * 32 + il];
        u32x4 mo[4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float m[8];
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const int jl = 16 * u + 8 * v + 4 * g2;
                const float4 aj = *reinterpret_cast<const float4 *>(&acs_s[ti * 32 + jl]);
                const float4 dj = *reinterpret_cast<const float4 *>(&dt_s[ti * 32 + jl]);
                const u32x4 cv = cbr[2 * u + v];
                const float e0 = __uint_as_float(cv[0]) * ssd_exp(ai - aj.x) * dj.x;
                const float e1 = __uint_as_float(cv[1]) * ssd_exp(ai - aj.y) * dj.y;
                const float e2 = __uint_as_float(cv[2]) * ssd_exp(ai - aj.z) * dj.z;
                const float e3 = __uint_as_float(cv[3]) * ssd_exp(ai - aj.w) * dj.w;
                m[4 * v + 0] = jl + 0 <= il ? e0 : 0.f;
                m[4 * v + 1] = jl + 1 <= il ? e1 : 0.f;
                m[4 * v + 2] = jl + 2 <= il ? e2 : 0.f;
                m[4 * v + 3] = jl + 3 <= il ? e3 : 0.f;
            }
            split8(m, mo[2 * u], mo[2 * u + 1]);
        }
        const bf16 *xt = xs + ti * 32 * LDX;
        // rescale to exp(Acs_i) and add D x (x rows of this tile)
        const float rf = ssd_exp(ai - ae);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int p0 = pt * 32 + 8 * rg + 4 * g2;
                const u32x2 xr = *reinterpret_cast<const u32x2 *>(&xt[il * LDX + p0]);
                const int r0 = 4 * rg;
                Z[pt][r0 + 0] = Z[pt][r0 + 0] * rf + Dh * lo_bf16(xr[0]);
                Z[pt][r0 + 1] = Z[pt][r0 + 1] * rf + Dh * hi_bf16(xr[0]);
                Z[pt][r0 + 2] = Z[pt][r0 + 2] * rf + Dh * lo_bf16(xr[1]);
                Z[pt][r0 + 3] = Z[pt][r0 + 3] * rf + Dh * hi_bf16(xr[1]);
            }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                const u32x4 xa = tr_operand<true>(xt, LDX, 16 * u, 32 * pt);
                Z[pt] = mfma32(xa, mo[2 * u], Z[pt]);
                Z[pt] = mfma32(xa, mo[2 * u + 1], Z[pt]);
            }
    }

    // y rows of the tile as bf16 via this wave's LDS rows, written as full
    // 128-byte rows (8 lanes per row, 8 rows per store)
    if constexpr (kGate) {
        // z of this lane's accumulator elements (token il, channels
        // p0..p0+3), from the copy the wave prefetched into its staging
        // rows; the multiply is in fp32, before the single rounding below
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the z copy has landed
        const bf16 *zl = ys;
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int p0 = pt * 32 + 8 * rg + 4 * g2;
                const u32x2 zz = *reinterpret_cast<const u32x2 *>(&zl[il * kP + p0]);
                Z[pt][4 * rg + 0] *= silu_f(lo_bf16(zz[0]));
                Z[pt][4 * rg + 1] *= silu_f(hi_bf16(zz[0]));
                Z[pt][4 * rg + 2] *= silu_f(lo_bf16(zz[1]));
                Z[pt][4 * rg + 3] *= silu_f(hi_bf16(zz[1]));
            }
        // the z reads above feed the products the stores below write, so
        // they have completed before the staging rows are overwritten
    }
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int p0 = pt * 32 + 8 * rg + 4 * g2;
            u32x2 o;
            o[0] = pack_bf16x2(Z[pt][4 * rg + 0], Z[pt][4 * rg + 1]);
            o[1] = pack_bf16x2(Z[pt][4 * rg + 2], Z[pt][4 * rg + 3]);
            *reinterpret_cast<u32x2 *>(&ys[il * LDY + p0]) = o;
        }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
    // nontemporal (y is not read again here; measured 1 us less per call at
    // the 2.7B shape than plain stores, bit for bit the same)
    const uint32_t yvoff = ((unsigned)(lane >> 3) * xrs + 8u * (lane & 7)) * 2u;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int r = (lane >> 3) + 8 * kk, sg = lane & 7;
        const u32x4 o = *reinterpret_cast<const u32x4 *>(&ys[r * LDY + 8 * sg]);
        buffer_store16_nt(o, buffer_rsrc_at(ybase, xy_bytes, (unsigned)(ti * 32 + 8 * kk) * xrs * 2u),
                          yvoff);
    }
}

template <int Q, int N>
void launch_state_t(const ScanShape &s, const void *x, const void *Bm, const float *dt,
                    const float *Acs, float *states, hipStream_t st) {
    const int64_t nb = s.B * s.T * s.H;
    k_chunk_state_mfma<Q, N, false><<<padded_grid(nb), 256, 0, st>>>(
        (const bf16 *)x, (const bf16 *)Bm, dt, nullptr, const_cast<float *>(Acs), states, s.L,
        (int)s.H, (int)s.G, (int)s.T, nb, DtAct{}, nullptr, s.ctab);
}


template <int Q, int N>
void launch_cb_t(const ScanShape &s, const void *Bm, const void *Cm, void *cb, hipStream_t st) {
    constexpr int NI = Q / 32;
    const int64_t ntiles = s.B * s.T * s.G * (NI * (NI + 1) / 2);
    k_chunk_cb_mfma<Q, N><<<(unsigned)((ntiles + 3) / 4), 256, 0, st>>>(
        (const bf16 *)Bm, (const bf16 *)Cm, (u32x4 *)cb, s.L, (int)s.G, (int)s.T, ntiles, s.ctab);
}

template <int Q, int N>
void launch_scan_t(const ScanShape &s, const void *x, const float *dt, const void *Cm,
                   const float *D, const float *Acs, const float *states, const void *cb, void *y,
                   hipStream_t st, const void *z) {
    const int64_t nb = s.B * s.T * s.H;
    constexpr int NI = Q / 32;
    const int64_t ntiles = s.B * s.T * s.G * (NI * (NI + 1) / 2);
    (void)Cm;  // C enters through the operand fragments the C.B kernel stored
    const u32x4 *cbt = (const u32x4 *)cb, *cfr = cbt + ntiles * 256;
    if (z)
        k_chunk_scan_mfma<Q, N, true><<<padded_grid(nb), Q * 2, 0, st>>>(
            (const bf16 *)x, dt, D, Acs, states, cbt, cfr, (bf16 *)y, (const bf16 *)z, s.L,
            (int)s.H, (int)s.G, (int)s.T, nb, s.ctab);
    else
        k_chunk_scan_mfma<Q, N, false><<<padded_grid(nb), Q * 2, 0, st>>>(
            (const bf16 *)x, dt, D, Acs, states, cbt, cfr, (bf16 *)y, nullptr, s.L, (int)s.H,
            (int)s.G, (int)s.T, nb, s.ctab);
}

// The whole chunked scan in three launches: the C.B tiles (with the hand-off
// flags cleared), the chunk states with the in-block cumsum and the chained
// state pass, the chunk output.
template <int Q, int N>
void launch_fused_t(const ScanShape &s, const void *x, const float *dt, const float *A,
                    const void *Bm, const void *Cm, const float *D, const float *init, void *y,
                    float *fin, float *Acs, float *states, void *cb, void *chain, hipStream_t st,
                    const DtAct &act, float *dt_out, const void *z) {
    constexpr int NI = Q / 32;
    const int64_t nb = s.B * s.T * s.H;
    const int64_t ntiles = s.B * s.T * s.G * (NI * (NI + 1) / 2);
    unsigned *ctl = static_cast<unsigned *>(chain);
    unsigned long long *flags =
        reinterpret_cast<unsigned long long *>(static_cast<char *>(chain) + kChainCtlWords * 4);
    const int64_t nflags = nb * 4, nzb = (nflags + 255) / 256;
    const int64_t ncg = s.B * s.T * s.G;
    if (ncg >= kCbBlockMin)
        k_chain_prep<Q, N, true><<<(unsigned)(nzb + (ncg + 8 / NI - 1) / (8 / NI)), 256, 0, st>>>(
            (const bf16 *)Bm, (const bf16 *)Cm, (u32x4 *)cb, s.L, (int)s.G, (int)s.T, ntiles,
            s.ctab, flags, nflags, ctl, nzb, ncg);
    else
        k_chain_prep<Q, N, false><<<(unsigned)(nzb + (ntiles + 3) / 4), 256, 0, st>>>(
            (const bf16 *)Bm, (const bf16 *)Cm, (u32x4 *)cb, s.L, (int)s.G, (int)s.T, ntiles,
            s.ctab, flags, nflags, ctl, nzb, ncg);
    ChainArgs ca;
    ca.init = init;
    ca.fin = fin;
    ca.flags = flags;
    ca.ctl = ctl;
    ca.sch = s.sch;
    ca.spos = s.spos;
    ca.B = s.B;
    k_chunk_state_mfma<Q, N, true, false, bf16, true><<<(unsigned)nb, 256, 0, st>>>(
        (const bf16 *)x, (const bf16 *)Bm, dt, A, Acs, states, s.L, (int)s.H, (int)s.G, (int)s.T,
        nb, act, dt_out, s.ctab, ca);
    launch_scan_t<Q, N>(s, x, dt_out ? dt_out : dt, Cm, D, Acs, states, cb, y, st, z);
}

// The earlier arrangement, kept for comparison: chunk states, then the state
// pass and the C.B tiles in one launch, then the chunk output.
template <int Q, int N>
void launch_staged3_t(const ScanShape &s, const void *x, const float *dt, const float *A,
                      const void *Bm, const void *Cm, const float *D, const float *init, void *y,
                      float *fin, float *Acs, float *states, void *cb, hipStream_t st,
                      const DtAct &act, float *dt_out, const void *z) {
    constexpr int NI = Q / 32;
    const int64_t nb = s.B * s.T * s.H;
    k_chunk_state_mfma<Q, N, true><<<padded_grid(nb), 256, 0, st>>>(
        (const bf16 *)x, (const bf16 *)Bm, dt, A, Acs, states, s.L, (int)s.H, (int)s.G, (int)s.T,
        nb, act, dt_out, s.ctab);
    const int64_t PN = s.P * s.N;
    const int ny = (int)((PN / 4 + 255) / 256);
    const int64_t nsp = (s.sch ? s.NS : s.B) * s.H * ny;  // batch rows, or sequences
    const int64_t ntiles = s.B * s.T * s.G * (NI * (NI + 1) / 2);
    k_state_passing_cb<Q, N><<<(unsigned)(nsp + (ntiles + 3) / 4), 256, 0, st>>>(
        states, Acs, init, fin, s.L, (int)s.H, PN, (int)s.T, nsp, ny, (const bf16 *)Bm,
        (const bf16 *)Cm, (u32x4 *)cb, (int)s.G, ntiles, s.ctab, s.sch);
    launch_scan_t<Q, N>(s, x, dt_out ? dt_out : dt, Cm, D, Acs, states, cb, y, st, z);
}

}  // namespace

bool mfma_supported(const ScanShape &s) {
    // the kernels form byte offsets within one chunk (up to two stages past
    // its end) in 32 bits: (Q + 64) rows of x/y, or of B/C, must stay below 2^31
    const bool offsets32 = (s.Q + 64) * s.H * s.P * 2 < (int64_t(1) << 31) &&
                           (s.Q + 64) * s.G * s.N * 2 < (int64_t(1) << 31);
    return s.dtype == SSD_BF16 && s.P == kP && (s.N == 64 || s.N == 128) &&
           (s.Q == 64 || s.Q == 128 || s.Q == 256) && offsets32;
}

#define SSD_DISPATCH_QN(FN, ...)                                         \
    do {                                                                 \
        if (s.N == 128) {                                                \
            if (s.Q == 256) FN<256, 128>(__VA_ARGS__);                   \
            else if (s.Q == 128) FN<128, 128>(__VA_ARGS__);              \
            else FN<64, 128>(__VA_ARGS__);                               \
        } else {                                                         \
            if (s.Q == 256) FN<256, 64>(__VA_ARGS__);                    \
            else if (s.Q == 128) FN<128, 64>(__VA_ARGS__);               \
            else FN<64, 64>(__VA_ARGS__);                                \
        }                                                                \
    } while (0)

bool bwd_mfma_ok(const ScanShape &s) {
    // offsets within one 64-token chunk (plus two stages) stay below 2^31
    const int64_t q = 64;
    const bool offsets32 = (q + 64) * s.H * s.P * 2 < (int64_t(1) << 31) &&
                           (q + 64) * s.G * s.N * 2 < (int64_t(1) << 31);
    return s.dtype == SSD_BF16 && s.P == kP && (s.N == 64 || s.N == 128) && offsets32;
}

bool bwd_states_mfma_ok(const ScanShape &s) { return bwd_mfma_ok(s) && s.Q == 64; }

template <int Q, int N, bool kAdj, typename TX = bf16>
void launch_bwd_states_t(const ScanShape &s, const void *xin, const void *bin, const float *dt,
                         const float *Acs, float *out, hipStream_t st) {
    const int64_t nb = s.B * s.T * s.H;
    k_chunk_state_mfma<Q, N, false, kAdj, TX><<<padded_grid(nb), 256, 0, st>>>(
        (const TX *)xin, (const bf16 *)bin, dt, nullptr, const_cast<float *>(Acs), out, s.L,
        (int)s.H, (int)s.G, (int)s.T, nb, DtAct{}, nullptr, s.ctab);
}

void launch_bwd_states_mfma(const ScanShape &s, const void *xin, const void *bin,
                            const float *dt, const float *Acs, float *out, bool adjoint,
                            hipStream_t st, bool x_f32) {
#define SSD_BWDS(Q_, N_)                                                                   \
    do {                                                                                   \
        if (adjoint && x_f32)                                                              \
            launch_bwd_states_t<Q_, N_, true, float>(s, xin, bin, dt, Acs, out, st);      \
        else if (adjoint) launch_bwd_states_t<Q_, N_, true>(s, xin, bin, dt, Acs, out, st); \
        else launch_bwd_states_t<Q_, N_, false>(s, xin, bin, dt, Acs, out, st);           \
    } while (0)
    if (s.N == 128) SSD_BWDS(64, 128);
    else SSD_BWDS(64, 64);
#undef SSD_BWDS
}

void launch_bwd_states_cumsum_mfma(const ScanShape &s, const void *x, const void *Bm,
                                   const float *dt, const float *A, float *Acs, float *out,
                                   const DtAct &act, float *dt_out, hipStream_t st) {
    const int64_t nb = s.B * s.T * s.H;
    if (s.N == 128)
        k_chunk_state_mfma<64, 128, true><<<padded_grid(nb), 256, 0, st>>>(
            (const bf16 *)x, (const bf16 *)Bm, dt, A, Acs, out, s.L, (int)s.H, (int)s.G, (int)s.T,
            nb, act, dt_out, s.ctab);
    else
        k_chunk_state_mfma<64, 64, true><<<padded_grid(nb), 256, 0, st>>>(
            (const bf16 *)x, (const bf16 *)Bm, dt, A, Acs, out, s.L, (int)s.H, (int)s.G, (int)s.T,
            nb, act, dt_out, s.ctab);
}

void launch_chunk_state_mfma(const ScanShape &s, const void *x, const void *Bm,
                             const float *dt, const float *Acs, float *states, hipStream_t st) {
    SSD_DISPATCH_QN(launch_state_t, s, x, Bm, dt, Acs, states, st);
}

size_t chunk_cb_bytes(const ScanShape &s) {
    // C.B tiles, then the C operand fragments (Q x N bf16 per (b, c, g))
    const int64_t ni = s.Q / 32;
    return (size_t)(s.B * s.T * s.G) * ((size_t)(ni * (ni + 1) / 2) * 4096 + (size_t)(s.Q * s.N * 2));
}

void launch_chunk_cb_mfma(const ScanShape &s, const void *Bm, const void *Cm, void *cb,
                          hipStream_t st) {
    SSD_DISPATCH_QN(launch_cb_t, s, Bm, Cm, cb, st);
}

size_t chain_ws_bytes(const ScanShape &s) {
    return kChainCtlWords * 4 + (size_t)(s.B * s.T * s.H) * 4 * 8;
}

void launch_scan_fused_mfma(const ScanShape &s, const void *x, const float *dt, const float *A,
                            const void *Bm, const void *Cm, const float *D, const float *init,
                            void *y, float *fin, float *Acs, float *states, void *cb, void *chain,
                            hipStream_t st, const DtAct &act, float *dt_out, const void *z) {
    if (chain)
        SSD_DISPATCH_QN(launch_fused_t, s, x, dt, A, Bm, Cm, D, init, y, fin, Acs, states, cb,
                        chain, st, act, dt_out, z);
    else
        SSD_DISPATCH_QN(launch_staged3_t, s, x, dt, A, Bm, Cm, D, init, y, fin, Acs, states, cb,
                        st, act, dt_out, z);
}

void launch_chunk_scan_mfma(const ScanShape &s, const void *x, const float *dt, const void *Cm,
                            const float *D, const float *Acs, const float *states, const void *cb,
                            void *y, hipStream_t st, const void *z) {
    SSD_DISPATCH_QN(launch_scan_t, s, x, dt, Cm, D, Acs, states, cb, y, st, z);
}

}  // namespace ssd
