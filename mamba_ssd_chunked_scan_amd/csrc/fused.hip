// The whole chunked prefill in one kernel per chunk of 256 tokens ("Compiler-
// First State Space Duality and Portable O(1) Autoregressive Caching for
// Inference", paperlayer summary, §3 Method, "Chunked recurrence", and the
// three contractions of B.5): one block per (batch row, chunk, head) forms the
// chunk's cumulative log-decay, its own state, takes the state entering the
// chunk from its predecessor and hands the next one on, and writes the chunk's
// output.  x is read from HBM once and kept in LDS from the state product
// through the output; the chunk states never make a round trip through a
// separate pass.
//
//   Acs_i   = sum_{k<=i} dt_k A                       (within the chunk)
//   S^T     = sum_j B_j^T (w_j x_j),  w_j = dt_j exp(Acs_last - Acs_j)
//   H_{c+1} = exp(Acs_last) H_c + S_c                 (H_0 = init state)
//   y_i     = sum_{j<=i} (C_i.B_j) exp(Acs_i - Acs_j) dt_j x_j
//             + exp(Acs_i) C_i.H_c + D x_i
//
// The hand-off between chunks.  Entering states are passed from block to
// block through a workspace slot per (chunk, head), with a flag per 32x32
// tile of the state (each wave publishes and consumes its own tile, so no
// block barrier sits on the chain).  Chunks are grouped by `grp` along each
// sequence: every chunk but the last of its group publishes its own state S_c
// (with its decay) as soon as it has formed it, and the last chunk of a group
// publishes the state entering the next group.  A chunk then needs only the
// state entering its group and the states of the group's earlier chunks, so
// the serial chain has one link per group, not one per chunk.
//
// Block order and progress.  The heads are split into 8 contiguous ranges,
// one work queue per range, and a block takes items from the queue of the XCD
// it runs on (the XCC_ID hardware register) while that queue lasts, then from
// the others in turn.  The heads of one range share their B/C group as far as
// the head split allows, so the group's C.B tiles are fetched into that XCD's
// L2 once and read there by the range's heads.  Within a queue, items are
// numbered by an atomic ticket in chunk-major order (all batch rows and heads
// of the range for chunk c before chunk c+1).  A chunk only waits for earlier
// chunks of its own (sequence, head), which sit in the same queue under
// smaller tickets: they were taken by blocks that are already running and only
// wait for smaller tickets themselves, so progress never depends on which
// XCD runs what.  Blocks are persistent (a grid of at most two per CU): each
// takes its next ticket while it works on the current one.  Every wait is
// bounded; one that runs out sets the error word in the workspace and goes on
// with a zero state, so a broken hand-off shows up as a flagged wrong result
// instead of a hang.
//
// Visibility across XCDs: the sc1 hand-off of handoff.hpp.
#include "cb_tile.hpp"
#include "common.hpp"
#include "handoff.hpp"
#include "launch.hpp"
#include "mfma_ops.hpp"
#include "ssd.h"

namespace ssd {
namespace {

using namespace mx;

constexpr int kP = 64;     // headdim
constexpr int kQ = 256;    // tokens per chunk
constexpr int kNI = kQ / 32;  // 32-row output tiles per chunk = waves per block
constexpr int kTH = kNI * 64;  // threads per block
constexpr int kJS = 32;    // tokens per streamed stage of the state product
constexpr int kNST = kQ / kJS;

struct FusedArgs {
    const bf16 *x;
    const float *dt;
    const float *A;
    const bf16 *Bm;
    const float *D;
    const float *init;
    float *fin;
    bf16 *y;
    const bf16 *z;
    const u32x4 *cb;
    const u32x4 *cfr;
    float *hand;                  // [slots][H][P][N] fp32 hand-off states
    unsigned long long *flags;    // [slots][H][tiles]: bit 0 set, decay in the high word
    unsigned *ctl;                // [1] error word, [8 + q] ticket of queue q
    const int2 *ctab;             // variable-length chunk table (null: fixed chunking)
    const int2 *sch;              // sequences: first slot, slots
    const int2 *spos;             // slot -> (sequence, position in it)
    int64_t B, L;
    int H, G, T;
    int grp;
    int nq;                       // work queues: 1, or one per XCD (8)
    DtAct act;
};

constexpr int kQueues = 8;

// Heads [h0, h1) of queue q of nq: contiguous ranges of H/nq or H/nq + 1 heads.
__device__ __forceinline__ void queue_heads(int q, int nq, int H, int &h0, int &h1) {
    h0 = (int)(((int64_t)q * H) / nq);
    h1 = (int)(((int64_t)(q + 1) * H) / nq);
}

template <int N, bool kGate>
__global__ void __launch_bounds__(kTH) __attribute__((amdgpu_waves_per_eu(4)))
k_ssd_fused(const FusedArgs a0) {
    constexpr int NTN = N / 32;           // n tiles of the state
    constexpr int NTILE = 2 * NTN;        // 32x32 tiles of the 64 x N state
    constexpr int NT = kNI * (kNI + 1) / 2, KS = N / 16;
    constexpr int LDX = kP + 16;          // exact x rows
    constexpr int LDW = kP + 8;           // weighted x stage rows
    constexpr int LDB = N + 16;           // B stage rows
    constexpr int LDH = N + 8;            // entering-state rows
    constexpr int LDY = kP + 8;           // y staging rows
    constexpr int W_BYTES = 2 * 2 * kJS * LDW * 2;  // two stages, hi and lo
    constexpr int B_BYTES = 2 * kJS * LDB * 2;      // two stages
    constexpr int A_BYTES = W_BYTES + B_BYTES;
    constexpr int H_BYTES = 2 * kP * LDH * 2;
    constexpr int Y_BYTES = kNI * 32 * LDY * 2;
    constexpr int U_BYTES = (A_BYTES > H_BYTES ? (A_BYTES > Y_BYTES ? A_BYTES : Y_BYTES)
                                               : (H_BYTES > Y_BYTES ? H_BYTES : Y_BYTES));
    constexpr int NXV = kQ * kP / 8 / kTH;  // 16-byte x segments per thread
    constexpr int BSEG = N / 8;             // 16-byte segments per B row
    constexpr int NBV = kQ * BSEG / kTH;    // 16-byte B segments per thread
    static_assert(NXV == 4 && kJS * BSEG <= kTH && kTH % (kJS * BSEG) == 0, "staging split");
    // phase-A stages, then the entering state (hi/lo), then the y staging rows
    __shared__ __attribute__((aligned(16))) char un[U_BYTES];
    __shared__ __attribute__((aligned(16))) bf16 xs[kQ * LDX];
    __shared__ __attribute__((aligned(16))) float acs_s[kQ];
    __shared__ __attribute__((aligned(16))) float dt_s[kQ];
    __shared__ __attribute__((aligned(16))) float w_s[kQ];
    __shared__ float wsum[kNI];
    __shared__ float last_s;
    __shared__ unsigned tk_s;

    bf16 *const xwh = reinterpret_cast<bf16 *>(un);            // [2][kJS*LDW]
    bf16 *const xwl = xwh + 2 * kJS * LDW;                     // [2][kJS*LDW]
    bf16 *const bst = xwl + 2 * kJS * LDW;                     // [2][kJS*LDB]
    bf16 *const Hh = reinterpret_cast<bf16 *>(un);
    bf16 *const Hl = Hh + kP * LDH;

    const int64_t PN = (int64_t)kP * N;
    // the block's queue: the XCD it runs on, then the others in turn
    const int nq = a0.nq;
    const int q_home = (int)(__builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & (kQueues - 1)) % nq;
    const int64_t rows = a0.ctab ? 1 : a0.B;
    // queue index, its ticket, and the queue's item count
    auto draw = [&](int &qi, unsigned &tk) {
        while (qi < nq) {
            const int q = (q_home + qi) % nq;
            int h0, h1;
            queue_heads(q, nq, a0.H, h0, h1);
            const int64_t n = rows * a0.T * (h1 - h0);
            if (n > 0) {
                tk = __hip_atomic_fetch_add(a0.ctl + 8 + q, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (tk < n) return;
            }
            ++qi;
        }
    };
    __shared__ int qi_s;
    if (threadIdx.x == 0) {
        int qi = 0;
        unsigned tk = 0;
        draw(qi, tk);
        qi_s = qi;
        tk_s = tk;
    }
    __syncthreads();
    int qi = __builtin_amdgcn_readfirstlane(qi_s);
    unsigned tk = __builtin_amdgcn_readfirstlane(tk_s);
#pragma unroll 1
    while (qi < nq) {
        // the arguments are read afresh from the argument segment for every
        // item (through an opaque copy of their address) rather than held in
        // scalar registers across the loop
        typedef const __attribute__((address_space(4))) FusedArgs *kargs_t;
        kargs_t ap = (kargs_t)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(ap));
        const __attribute__((address_space(4))) FusedArgs &a = *ap;
        // lane-dependent values are formed afresh for every item (an opaque
        // copy of the thread index): kept live across the whole loop they
        // would not fit the 128 registers of four waves per SIMD
        int tid;
        asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
        const int lane = tid & 63;
        const int il = lane & 31, g2 = lane >> 5;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int ti = wave < kNI / 2 ? wave : 3 * kNI / 2 - 1 - wave;
        const unsigned xrs = a.H * kP, brs = a.G * N;
        const int qu = (q_home + qi) % nq;
        // the next item, taken now so that its ticket is in hand when this one ends
        int qn = qi;
        unsigned next = 0;
        if (tid == 0) draw(qn, next);

        // ---- the work item: chunk-major order
        int64_t slot, b, seq;
        int h, pos, npos;
        {
            int h0, h1;
            queue_heads(qu, nq, a.H, h0, h1);
            const unsigned nh = (unsigned)(h1 - h0);
            const unsigned per = (unsigned)(a.ctab ? 1 : a.B) * nh;
            const unsigned cc = tk / per, rem = tk - cc * per;
            h = h0 + (int)(rem % nh);
            b = a.ctab ? 0 : rem / nh;
            if (a.ctab) {
                slot = cc;
                const int2 sp = a.spos[slot];
                seq = sp.x;
                pos = sp.y;
                npos = seq >= 0 ? a.sch[seq].y : 0;
            } else {
                slot = b * a.T + cc;
                seq = b;
                pos = (int)cc;
                npos = a.T;
            }
        }
        const ChunkPos cp = chunk_pos(a.ctab, a.ctab ? slot : pos, kQ, a.L);
        const int64_t t0 = cp.t0;
        const int q = cp.q;
        if (q > 0 && seq >= 0) {
            const int g = h / (a.H / a.G);
            const bf16 *xbase = a.x + ((b * a.L + t0) * a.H + h) * kP;
            const bf16 *bbase = a.Bm + ((b * a.L + t0) * a.G + g) * N;
            const uint32_t xy_bytes = ((unsigned)(q - 1) * xrs + kP) * 2u;
            const uint32_t b_bytes = ((unsigned)(q - 1) * brs + N) * 2u;
            const rsrc_t xr = buffer_rsrc_at(xbase, xy_bytes, 0u);
            const rsrc_t br = buffer_rsrc_at(bbase, b_bytes, 0u);

            // ---- prologue: every global load of the chunk's own inputs at
            // once (dt, x, all of B), so that their latency is paid once
            float d = 0.f;
            if (tid < q) {
                DtAct act;
                act.bias = a.act.bias;
                act.lo = a.act.lo;
                act.hi = a.act.hi;
                act.softplus = a.act.softplus;
                act.limit = a.act.limit;
                d = act_dt(act, a.dt[(b * a.L + t0 + tid) * a.H + h], h);
            }
            u32x4 xv[NXV];
#pragma unroll
            for (int i = 0; i < NXV; ++i) {
                const int e = tid + kTH * i;
                xv[i] = buffer_load16(xr, ((unsigned)(e >> 3) * xrs + 8u * (e & 7)) * 2u);
            }
            // B segment e = tid + kTH i: row e / BSEG, 16-byte column e % BSEG
            u32x4 bv[NBV];
#pragma unroll
            for (int i = 0; i < NBV; ++i) {
                const int e = tid + kTH * i;
                bv[i] = buffer_load16(br, ((unsigned)(e / BSEG) * brs + 8u * (e % BSEG)) * 2u);
            }

            // ---- chunk cumsum of dt*A (one token per thread of waves 0..3)
            const float v = wave_scan_dpp(d * a.A[h]);
            if (lane == 63) wsum[wave] = v;
            __syncthreads();
            float acs = v;
            for (int k = 0; k < wave; ++k) acs += wsum[k];
            // off-diagonal weight: decay from token j to the end of its 32-row tile
            const float ae_t = __shfl(acs, lane | 31);
            if (tid < kQ) {
                acs_s[tid] = acs;
                dt_s[tid] = d;
                w_s[tid] = ssd_exp(ae_t - acs) * d;  // 0 past q
            }
            if (tid == kQ - 1) last_s = acs;  // flat past q: the chunk's total
#pragma unroll
            for (int i = 0; i < NXV; ++i) {
                const int e = tid + kTH * i;
                *reinterpret_cast<u32x4 *>(&xs[(e >> 3) * LDX + 8 * (e & 7)]) = xv[i];
            }
            __syncthreads();
            const float last = last_s;

            // ---- phase A: the chunk's own state S^T (N x 64) on the matrix
            // cores, streamed through LDS in 32-token stages from registers.
            // Stage st: the weighted x rows (hi/lo) from the 256 threads that
            // hold them, and the B rows of the stage.
            auto store_stage = [&](int st, int buf) {
                if ((tid >> 8) == (st & 1)) {
                    const int row = (tid >> 3) & 31;
                    const float f = ssd_exp(last - acs_s[st * kJS + kJS - 1]);
                    const float wj = f * w_s[st * kJS + row];
                    const u32x4 r = xv[st >> 1];
                    float m[8];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        m[2 * k] = lo_bf16(r[k]) * wj;
                        m[2 * k + 1] = hi_bf16(r[k]) * wj;
                    }
                    u32x4 hi, lo;
                    split8(m, hi, lo);
                    *reinterpret_cast<u32x4 *>(&xwh[buf * kJS * LDW + row * LDW + 8 * (tid & 7)]) = hi;
                    *reinterpret_cast<u32x4 *>(&xwl[buf * kJS * LDW + row * LDW + 8 * (tid & 7)]) = lo;
                }
                // the stage's kJS * BSEG segments: register st / SPR of the
                // threads whose segment index falls in the stage
                constexpr int SPR = kTH / (kJS * BSEG);  // stages per register
                if (SPR == 1 || (tid / (kJS * BSEG)) == st % SPR) {
                    const int e = tid % (kJS * BSEG);
                    *reinterpret_cast<u32x4 *>(&bst[buf * kJS * LDB + (e / BSEG) * LDB + 8 * (e % BSEG)]) =
                        bv[st / SPR];
                }
            };
            store_stage(0, 0);
            __syncthreads();

            const bool owner = wave < NTILE;  // this wave owns state tile `wave`
            const int snt = wave % NTN, spt = wave / NTN;
            f32x16 sacc = zero16();
#pragma unroll
            for (int st = 0; st < kNST; ++st) {
                const int buf = st & 1;
                if (owner) {
#pragma unroll
                    for (int ks = 0; ks < kJS / 16; ++ks) {
                        const u32x4 ab = tr_operand<false>(bst + buf * kJS * LDB, LDB, 16 * ks, 32 * snt);
                        const u32x4 xh = tr_operand<false>(xwh + buf * kJS * LDW, LDW, 16 * ks, 32 * spt);
                        const u32x4 xl = tr_operand<false>(xwl + buf * kJS * LDW, LDW, 16 * ks, 32 * spt);
                        sacc = mfma32(ab, xh, sacc);
                        sacc = mfma32(ab, xl, sacc);
                    }
                }
                if (st + 1 < kNST) store_stage(st + 1, buf ^ 1);
                __syncthreads();
            }

            const float rc = ssd_exp(last);
            const int j = pos % a.grp;
            const bool lastg = j == a.grp - 1 || pos == npos - 1;
            const int m0 = pos - j;  // position of the group's first chunk
            // this lane's 4 runs of 4 state elements: p = 32 spt + il,
            // n = 32 snt + 8 k + 4 g2 (the accumulator's registers 4k..4k+3)
            const uint32_t eoff = (uint32_t)((32 * spt + il) * N + 32 * snt + 4 * g2);
            const int64_t fl_h = (int64_t)a.H * NTILE;
            auto hand_at = [&](int64_t sl) {
                return buffer_rsrc(a.hand + (sl * a.H + h) * PN, (uint32_t)(PN * 4));
            };
            auto flag_at = [&](int64_t sl) { return a.flags + (sl * fl_h + (int64_t)h * NTILE + wave); };


            // ---- phase B: the state entering this chunk, and the hand-off
            bool pub = false;  // this wave has a flag to set once its stores are done
            if (owner) {
                float hs[16];
                if (m0 == 0) {
                    // the initial state, read before anything of this sequence
                    // is published (the final state may overwrite it)
                    if (a.init) {
                        const float *ip = a.init + ((int64_t)seq * a.H + h) * PN + eoff;
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const float4 t = *reinterpret_cast<const float4 *>(ip + 8 * k);
                            hs[4 * k] = t.x; hs[4 * k + 1] = t.y; hs[4 * k + 2] = t.z; hs[4 * k + 3] = t.w;
                        }
                    } else {
#pragma unroll
                        for (int k = 0; k < 16; ++k) hs[k] = 0.f;
                    }
                }
                if (!lastg) {  // publish this chunk's own state for the rest of its group
                    const rsrc_t o = hand_at(slot);
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        st16_dev(o, (eoff + 8 * k) * 4u, sacc[4 * k], sacc[4 * k + 1], sacc[4 * k + 2],
                                 sacc[4 * k + 3]);
                    set_flag(flag_at(slot), rc);
                }
                if (m0 > 0) {
                    const int64_t sl = slot - j - 1;  // last chunk of the previous group
                    wait_flag(flag_at(sl), a.ctl + 1);
                    const rsrc_t p = hand_at(sl);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const u32x4 t = ld16_dev(p, (eoff + 8 * k) * 4u);
#pragma unroll
                        for (int e = 0; e < 4; ++e) hs[4 * k + e] = __uint_as_float(t[e]);
                    }
                }
                // the group's earlier chunks, oldest first
#pragma unroll 1
                for (int i = 0; i < j; ++i) {
                    const int64_t sl = slot - j + i;
                    const float r = wait_flag(flag_at(sl), a.ctl + 1);
                    const rsrc_t p = hand_at(sl);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const u32x4 t = ld16_dev(p, (eoff + 8 * k) * 4u);
#pragma unroll
                        for (int e = 0; e < 4; ++e) hs[4 * k + e] = r * hs[4 * k + e] + __uint_as_float(t[e]);
                    }
                }
                if (lastg) {  // the state after this chunk: the next group's, or the final one
                    float hn[16];
#pragma unroll
                    for (int k = 0; k < 16; ++k) hn[k] = rc * hs[k] + sacc[k];
                    if (pos == npos - 1) {
                        if (a.fin) {
                            float *fp = a.fin + ((int64_t)seq * a.H + h) * PN + eoff;
#pragma unroll
                            for (int k = 0; k < 4; ++k)
                                *reinterpret_cast<float4 *>(fp + 8 * k) =
                                    make_float4(hn[4 * k], hn[4 * k + 1], hn[4 * k + 2], hn[4 * k + 3]);
                        }
                    } else {
                        const rsrc_t o = hand_at(slot);
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            st16_dev(o, (eoff + 8 * k) * 4u, hn[4 * k], hn[4 * k + 1], hn[4 * k + 2],
                                     hn[4 * k + 3]);
                        pub = true;  // its flag follows once the stores are complete
                    }
                }
                // the entering state as hi/lo MFMA operands, rows p, columns n
                const int p = 32 * spt + il;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int n = 32 * snt + 8 * k + 4 * g2;
                    u32x2 hh, hl;
                    uint32_t l0, l1;
                    hh[0] = split2(hs[4 * k], hs[4 * k + 1], l0);
                    hh[1] = split2(hs[4 * k + 2], hs[4 * k + 3], l1);
                    hl[0] = l0;
                    hl[1] = l1;
                    *reinterpret_cast<u32x2 *>(Hh + p * LDH + n) = hh;
                    *reinterpret_cast<u32x2 *>(Hl + p * LDH + n) = hl;
                }
            }
            // the C operand fragments of the state term
            const int64_t bcg = ((a.ctab ? 0 : b) * a.T + (a.ctab ? slot : pos)) * a.G + g;
            const u32x4 *cbg = a.cb + bcg * NT * 256;
            u32x4 cf[KS];
            {
                const u32x4 *f = a.cfr + (bcg * kNI + ti) * KS * 64 + lane;
#pragma unroll
                for (int s = 0; s < KS; ++s) cf[s] = f[s * 64];
            }
            __syncthreads();  // the entering state is in LDS

            // ---- phase C: the chunk output (state term, off-diagonal and
            // diagonal tiles, D x), as one wave per 32-row tile
            const uint32_t cbvoff = lane * 16u;
            auto load_cb = [&](int jt, u32x4 (&o)[4]) __attribute__((always_inline)) {
                const int tile = ti * (ti + 1) / 2 + jt;
                const rsrc_t r = buffer_rsrc_at(cbg, (tile + 1) * 4096u, tile * 4096u);
#pragma unroll
                for (int k = 0; k < 4; ++k) o[k] = buffer_load16(r, cbvoff + k * 1024u);
            };
            u32x4 cbr[4];  // the C.B tile of the wave's next visit
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
            // the hand-off's stores are complete by now in all likelihood:
            // publish them (set_flag waits for them)
            if (pub) set_flag(flag_at(slot), rc);
            load_cb(0, cbr);
            __syncthreads();  // H no longer read: its LDS becomes the y staging rows

            bf16 *ys = reinterpret_cast<bf16 *>(un) + wave * 32 * LDY;
            bf16 *ybase = a.y + ((b * a.L + t0) * a.H + h) * kP;
            if constexpr (kGate) {
                // the wave's z tile (32 rows x 128 bytes) copied straight into
                // its staging rows (lane i's 16 bytes land at 16 i; rows past a
                // short chunk arrive as zeros), used before y is staged there
                static_assert(32 * kP * 2 <= 32 * LDY * 2, "z tile fits the staging rows");
                const bf16 *zbase = a.z + ((b * a.L + t0) * a.H + h) * kP;
                const rsrc_t zr = buffer_rsrc_at(zbase, xy_bytes, (unsigned)(ti * 32) * xrs * 2u);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        zr, (__attribute__((address_space(3))) void *)(ys + kk * 512), 16,
                        ((unsigned)((lane >> 3) + 8 * kk) * xrs + 8u * (lane & 7)) * 2u, 0, 0, 0);
            }
            const float Dh = a.D ? a.D[h] : 0.f;
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
                    for (int v2 = 0; v2 < 2; ++v2) {
                        const float4 wj = *reinterpret_cast<const float4 *>(&w_s[jt * 32 + 16 * u + 8 * v2 + 4 * g2]);
                        const u32x4 cv = cbr[2 * u + v2];
                        m[4 * v2 + 0] = __uint_as_float(cv[0]) * (wj.x * F);
                        m[4 * v2 + 1] = __uint_as_float(cv[1]) * (wj.y * F);
                        m[4 * v2 + 2] = __uint_as_float(cv[2]) * (wj.z * F);
                        m[4 * v2 + 3] = __uint_as_float(cv[3]) * (wj.w * F);
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
            {
                const float ai = acs_s[ti * 32 + il];
                u32x4 mo[4];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    float m[8];
#pragma unroll
                    for (int v2 = 0; v2 < 2; ++v2) {
                        const int jl = 16 * u + 8 * v2 + 4 * g2;
                        const float4 aj = *reinterpret_cast<const float4 *>(&acs_s[ti * 32 + jl]);
                        const float4 dj = *reinterpret_cast<const float4 *>(&dt_s[ti * 32 + jl]);
                        const u32x4 cv = cbr[2 * u + v2];
                        const float e0 = __uint_as_float(cv[0]) * ssd_exp(ai - aj.x) * dj.x;
                        const float e1 = __uint_as_float(cv[1]) * ssd_exp(ai - aj.y) * dj.y;
                        const float e2 = __uint_as_float(cv[2]) * ssd_exp(ai - aj.z) * dj.z;
                        const float e3 = __uint_as_float(cv[3]) * ssd_exp(ai - aj.w) * dj.w;
                        m[4 * v2 + 0] = jl + 0 <= il ? e0 : 0.f;
                        m[4 * v2 + 1] = jl + 1 <= il ? e1 : 0.f;
                        m[4 * v2 + 2] = jl + 2 <= il ? e2 : 0.f;
                        m[4 * v2 + 3] = jl + 3 <= il ? e3 : 0.f;
                    }
                    split8(m, mo[2 * u], mo[2 * u + 1]);
                }
                const bf16 *xt = xs + ti * 32 * LDX;
                const float rf = ssd_exp(ai - ae);
#pragma unroll
                for (int pt = 0; pt < 2; ++pt)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const int p0 = pt * 32 + 8 * rg + 4 * g2;
                        const u32x2 xr2 = *reinterpret_cast<const u32x2 *>(&xt[il * LDX + p0]);
                        const int r0 = 4 * rg;
                        Z[pt][r0 + 0] = Z[pt][r0 + 0] * rf + Dh * lo_bf16(xr2[0]);
                        Z[pt][r0 + 1] = Z[pt][r0 + 1] * rf + Dh * hi_bf16(xr2[0]);
                        Z[pt][r0 + 2] = Z[pt][r0 + 2] * rf + Dh * lo_bf16(xr2[1]);
                        Z[pt][r0 + 3] = Z[pt][r0 + 3] * rf + Dh * hi_bf16(xr2[1]);
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
            if constexpr (kGate) {
                __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the z copy has landed
#pragma unroll
                for (int pt = 0; pt < 2; ++pt)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const int p0 = pt * 32 + 8 * rg + 4 * g2;
                        const u32x2 zz = *reinterpret_cast<const u32x2 *>(&ys[il * kP + p0]);
                        Z[pt][4 * rg + 0] *= silu_f(lo_bf16(zz[0]));
                        Z[pt][4 * rg + 1] *= silu_f(hi_bf16(zz[0]));
                        Z[pt][4 * rg + 2] *= silu_f(lo_bf16(zz[1]));
                        Z[pt][4 * rg + 3] *= silu_f(hi_bf16(zz[1]));
                    }
                // the z reads above feed the products stored below, so they
                // have completed before the staging rows are overwritten
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
            const uint32_t yvoff = ((unsigned)(lane >> 3) * xrs + 8u * (lane & 7)) * 2u;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int r = (lane >> 3) + 8 * kk, sg = lane & 7;
                const u32x4 o = *reinterpret_cast<const u32x4 *>(&ys[r * LDY + 8 * sg]);
                buffer_store16(o, buffer_rsrc_at(ybase, xy_bytes, (unsigned)(ti * 32 + 8 * kk) * xrs * 2u),
                               yvoff);
            }
        }
        __syncthreads();  // every LDS read of this item is done
        if (tid == 0) {
            tk_s = next;
            qi_s = qn;
        }
        __syncthreads();
        tk = __builtin_amdgcn_readfirstlane(tk_s);
        qi = __builtin_amdgcn_readfirstlane(qi_s);
    }
}

// The C.B tiles and C operand fragments of every (b, c, g), and a clean
// hand-off state (flags, ticket, error word) for the fused kernel.
template <int Q, int N>
__global__ void __launch_bounds__(256)
k_fused_prep(const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm, u32x4 *__restrict__ cb,
             int64_t L, int G, int T, int64_t ntiles, int64_t cb_blocks,
             unsigned long long *__restrict__ flags, int64_t nflags, unsigned *__restrict__ ctl,
             const int2 *__restrict__ ctab) {
    const int64_t blk = blockIdx.x;
    if (blk < cb_blocks) {
        const int64_t w = blk * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        if (w >= ntiles) return;
        cb_tile<Q, N>(Bm, Cm, cb, cb + ntiles * 256, L, G, T, w, ctab);
        return;
    }
    const int64_t i = (blk - cb_blocks) * 256 + threadIdx.x;
    if (i < nflags) flags[i] = 0ull;
    if (i < 16) ctl[i] = 0u;
}

template <int N>
void launch_fused_t(const ScanShape &s, const FusedWs &w, const void *x, const float *dt,
                    const float *A, const void *Bm, const void *Cm, const float *D,
                    const float *init, void *y, float *fin, hipStream_t st, const DtAct &act,
                    const void *z, int grp, int nq, int max_blocks) {
    constexpr int NI = kQ / 32;
    const int64_t ntiles = s.B * s.T * s.G * (NI * (NI + 1) / 2);
    const int64_t cbb = (ntiles + 3) / 4;
    const int64_t nflags = s.B * s.T * s.H * (2 * N / 32);
    k_fused_prep<kQ, N><<<(unsigned)(cbb + (nflags + 255) / 256), 256, 0, st>>>(
        (const bf16 *)Bm, (const bf16 *)Cm, (u32x4 *)w.cb, s.L, (int)s.G, (int)s.T, ntiles, cbb,
        w.flags, nflags, w.ctl, s.ctab);
    FusedArgs a;
    a.x = (const bf16 *)x;
    a.dt = dt;
    a.A = A;
    a.Bm = (const bf16 *)Bm;
    a.D = D;
    a.init = init;
    a.fin = fin;
    a.y = (bf16 *)y;
    a.z = (const bf16 *)z;
    a.cb = (const u32x4 *)w.cb;
    a.cfr = a.cb + ntiles * 256;
    a.hand = w.hand;
    a.flags = w.flags;
    a.ctl = w.ctl;
    a.ctab = s.ctab;
    a.sch = s.sch;
    a.spos = s.spos;
    a.B = s.B;
    a.L = s.L;
    a.H = (int)s.H;
    a.G = (int)s.G;
    a.T = (int)s.T;
    a.grp = grp;
    a.nq = nq;
    a.act = act;
    const int64_t nitems = s.B * s.T * s.H;
    const int64_t grid = nitems < max_blocks ? nitems : max_blocks;
    if (z) k_ssd_fused<N, true><<<(unsigned)grid, kTH, 0, st>>>(a);
    else k_ssd_fused<N, false><<<(unsigned)grid, kTH, 0, st>>>(a);
}

}  // namespace

bool fused_supported(const ScanShape &s) { return mfma_supported(s) && s.Q == kQ; }

size_t fused_ws_bytes(const ScanShape &s) {
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t slots = (size_t)(s.B * s.T);
    return 256 + up(slots * s.H * (2 * s.N / 32) * 8) + up(chunk_cb_bytes(s)) +
           up(slots * s.H * (size_t)(s.P * s.N) * 4);
}

FusedWs fused_ws_carve(const ScanShape &s, void *ws) {
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    char *p = static_cast<char *>(ws);
    FusedWs w;
    w.ctl = reinterpret_cast<unsigned *>(p);
    p += 256;
    const size_t slots = (size_t)(s.B * s.T);
    w.flags = reinterpret_cast<unsigned long long *>(p);
    p += up(slots * s.H * (2 * s.N / 32) * 8);
    w.cb = p;
    p += up(chunk_cb_bytes(s));
    w.hand = reinterpret_cast<float *>(p);
    return w;
}

void launch_scan_fused_chain(const ScanShape &s, const FusedWs &w, const void *x, const float *dt,
                             const float *A, const void *Bm, const void *Cm, const float *D,
                             const float *init, void *y, float *fin, hipStream_t st,
                             const DtAct &act, const void *z, int grp, int nq, int max_blocks) {
    if (s.N == 128)
        launch_fused_t<128>(s, w, x, dt, A, Bm, Cm, D, init, y, fin, st, act, z, grp, nq, max_blocks);
    else
        launch_fused_t<64>(s, w, x, dt, A, Bm, Cm, D, init, y, fin, st, act, z, grp, nq, max_blocks);
}

}  // namespace ssd
