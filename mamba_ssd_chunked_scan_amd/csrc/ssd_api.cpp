// C-ABI layer of libssd: argument validation, workspace carving and the
// launch sequence.  Every check happens before the first HIP call; the only
// HIP calls made here are kernel launches (through the launchers),
// hipGetLastError and, once per device, the query of its compute units.
#include <cstring>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>

#include "launch.hpp"
#include "ssd.h"

using ssd::ScanShape;
using ssd::StepShape;

namespace ssd {

// Compute units of the current device, looked up once per device.
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
        v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

}  // namespace ssd

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// Largest grid dimension the launchers use is batch*T*nheads blocks.
constexpr int64_t kMaxBlocks = 0x7fffffffLL;

ssd_status check_common(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                        int64_t ngroups, int32_t dtype, int32_t reserved) {
    if (batch < 0 || nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1 ||
        nheads % ngroups != 0)
        return SSD_ERR_SHAPE;
    if (dtype != SSD_F32 && dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (reserved != 0) return SSD_ERR_UNSUPPORTED;
    if (headdim > 256 || dstate < 4 || dstate > 256 || !pow2(dstate)) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

ssd_status check_scan(const ssd_scan_desc *d, ScanShape *s) {
    if (!d) return SSD_ERR_NULL_PTR;
    if (d->seqlen < 0) return SSD_ERR_SHAPE;
    ssd_status st = check_common(d->batch, d->nheads, d->headdim, d->dstate, d->ngroups,
                                 d->dtype, d->reserved);
    if (st != SSD_OK) return st;
    if (d->chunk < 16 || d->chunk > 256 || !pow2(d->chunk)) return SSD_ERR_UNSUPPORTED;
    s->B = d->batch;
    s->L = d->seqlen;
    s->H = d->nheads;
    s->P = d->headdim;
    s->N = d->dstate;
    s->G = d->ngroups;
    s->Q = d->chunk;
    s->T = (d->seqlen + d->chunk - 1) / d->chunk;
    s->dtype = d->dtype;
    // grid-size limit (also guards the products below against overflow)
    if (s->T > 0 && s->B > kMaxBlocks / s->T / s->H) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

ssd_status check_ptrs(std::initializer_list<const void *> required,
                      std::initializer_list<const void *> optional) {
    for (const void *p : required)
        if (!p) return SSD_ERR_NULL_PTR;
    for (const void *p : required)
        if (!aligned16(p)) return SSD_ERR_ALIGN;
    for (const void *p : optional)
        if (p && !aligned16(p)) return SSD_ERR_ALIGN;
    return SSD_OK;
}

size_t acs_bytes(const ScanShape &s) { return round_up((size_t)(s.B * s.H * s.L) * 4); }

size_t states_bytes(const ScanShape &s) {
    return round_up((size_t)(s.B * s.T * s.H) * (size_t)(s.P * s.N) * 4);
}

size_t scan_ws_bytes(const ScanShape &s) {
    if (s.B == 0 || s.L == 0) return 0;
    return round_up(ssd::chunk_scan_ws_bytes(s));
}

// the activated dt of ssd_scan_fwd_ex, [B, L, H] fp32
size_t dt_eff_bytes(const ScanShape &s) { return round_up((size_t)(s.B * s.L * s.H) * 4); }

// the chained state pass's flags and control words (MFMA shapes)
size_t chain_bytes(const ScanShape &s) {
    return ssd::mfma_supported(s) ? round_up(ssd::chain_ws_bytes(s)) : 0;
}

size_t chain_offset(const ScanShape &s) {
    return acs_bytes(s) + states_bytes(s) + scan_ws_bytes(s) + dt_eff_bytes(s);
}

size_t staged_ws_bytes(const ScanShape &s) { return chain_offset(s) + chain_bytes(s); }

// Either path's workspace fits (the single-kernel path's, where it applies, or
// the separate stages').
size_t workspace_bytes(const ScanShape &s) {
    if (s.B == 0 || s.L == 0) return 0;
    const size_t st = staged_ws_bytes(s);
    if (!ssd::fused_supported(s)) return st;
    const size_t fu = round_up(ssd::fused_ws_bytes(s));
    return fu > st ? fu : st;
}

// Blocks the single-kernel prefill keeps resident: two per compute unit of
// the current device.
int resident_blocks() { return 2 * ssd::device_cus(); }

// The single-kernel prefill is opt-in (SSD_PREFILL_PATH=fused): measured side
// by side it is slower than the separate stage kernels on every workload
// shape so far.  The workspace fits either path.
bool staged_forced() {
    const char *e = getenv("SSD_PREFILL_PATH");
    return !(e && e[0] == 'f');
}

// The MFMA stage kernels pass the state on either inside the chunk-state
// launch (a chain of hand-offs between its blocks) or in a launch of its own.
// A hand-off costs about 2.4 us (a device-scope load, the store's
// acknowledgement and a flag poll, in series), so a chain of T chunks is
// hidden only while the chunk-state grid spans several rounds of resident
// blocks; the separate pass instead moves the chunk states through HBM twice
// more.  Measured (MI355X, chunk 256, 4 chunk-state blocks resident per CU):
// 1280 blocks (T = 16) 105.7 us chained against 82.8 us separate; 40960
// blocks (T = 64) 2.73 ms against 3.06 ms.  The chain is taken from four
// rounds of resident blocks on; SSD_PREFILL_PATH=chained or =separate forces
// either.
bool chain_state_pass(const ScanShape &s) {
    const char *e = getenv("SSD_PREFILL_PATH");
    if (e && strcmp(e, "chained") == 0) return true;
    if (e && strcmp(e, "separate") == 0) return false;
    const int64_t blocks = s.B * s.T * s.H;
    return blocks >= 4 * (int64_t)(2 * resident_blocks());
}

// Work queues of the single-kernel prefill: one per XCD (heads split into 8
// ranges), or one for all (SSD_CHAIN_QUEUES=1).
int work_queues() {
    const char *e = getenv("SSD_CHAIN_QUEUES");
    return (e && atoi(e) == 1) ? 1 : 8;
}

// Chunks per hand-off group of the single-kernel prefill.  A chain of chunks
// per (sequence, head) is handed on link by link; when there are fewer chains
// than resident blocks, consecutive chunks of a chain run at the same time
// and each link's latency is exposed, so the chain is cut into groups whose
// chunks share one link.  SSD_CHAIN_GROUP (1, 2, 4 or 8) overrides the choice.
int chain_group(int64_t chains, int resident) {
    const char *e = getenv("SSD_CHAIN_GROUP");
    const int forced = e ? atoi(e) : 0;
    if (forced == 1 || forced == 2 || forced == 4 || forced == 8) return forced;
    if (chains >= resident) return 1;
    if (2 * chains >= resident) return 2;
    return 4;
}

// ssd_edges -> the kernels' dt activation and gate pointer (NULL: neither).
ssd_status read_edges(const ssd_edges *e, ssd::DtAct *act, const void **z) {
    *act = ssd::DtAct{};
    *z = nullptr;
    if (!e) return SSD_OK;
    if (e->dt_limit && !(e->dt_min <= e->dt_max)) return SSD_ERR_UNSUPPORTED;
    act->bias = e->dt_bias;
    act->softplus = e->dt_softplus ? 1 : 0;
    act->limit = e->dt_limit ? 1 : 0;
    act->lo = e->dt_min;
    act->hi = e->dt_max;
    *z = e->z;
    return SSD_OK;
}

bool act_active(const ssd::DtAct &a) { return a.bias || a.softplus || a.limit; }

// ssd_edges' gated RMSNorm for nheads H and ngroups G (w NULL: no norm).
struct NormEdge {
    const float *w = nullptr;
    float eps = 0.f;
    int64_t groups = 0;
};
ssd_status read_norm(const ssd_edges *e, int64_t H, int64_t G, NormEdge *n) {
    *n = NormEdge{};
    if (!e || !e->norm_weight) return SSD_OK;
    if (!(e->norm_eps >= 0.f)) return SSD_ERR_UNSUPPORTED;  // negative or NaN
    const int64_t ng = e->norm_groups ? e->norm_groups : G;
    if (ng < 1 || H % ng) return SSD_ERR_SHAPE;
    n->w = e->norm_weight;
    n->eps = e->norm_eps;
    n->groups = ng;
    return SSD_OK;
}

// The gradient's own chunking: 64 tokens on the matrix-core path (half the
// state traffic of 32), 32 on the generic one.
ScanShape bwd_shape(const ScanShape &s) {
    ScanShape b = s;
    b.ctab = nullptr;
    b.Q = ssd::bwd_mfma_ok(b) ? 64 : 32;
    b.T = (s.L + b.Q - 1) / b.Q;
    b.sch = nullptr;
    return b;
}

// The same for a variable-length batch (s from check_varlen): slots of the
// gradient's chunk for its sequences (total / Q + nseq covers every
// sequence's chunks); the caller sets the chunk table.
ScanShape bwd_varlen_shape(const ScanShape &s) {
    ScanShape b = s;
    b.ctab = nullptr;
    b.sch = nullptr;
    b.Q = ssd::bwd_mfma_ok(b) ? 64 : 32;
    b.T = s.L / b.Q + s.NS;
    return b;
}

// Chunk table, sequence table and slot positions of a variable-length batch,
// after the rest.
size_t varlen_table_bytes(const ScanShape &s) {
    return 2 * round_up((size_t)s.T * 8) + round_up((size_t)s.NS * 8);
}

ssd_status check_varlen(const ssd_varlen_desc *d, ScanShape *s) {
    if (!d) return SSD_ERR_NULL_PTR;
    if (d->nseq < 0 || d->total < 0) return SSD_ERR_SHAPE;
    ssd_status st = check_common(1, d->nheads, d->headdim, d->dstate, d->ngroups, d->dtype,
                                 d->reserved);
    if (st != SSD_OK) return st;
    if (d->chunk < 16 || d->chunk > 256 || !pow2(d->chunk)) return SSD_ERR_UNSUPPORTED;
    // token offsets and chunk slots are 32-bit in the chunk table
    const int64_t lim = (int64_t(1) << 31) - 512;
    if (d->total > lim || d->nseq > lim) return SSD_ERR_UNSUPPORTED;
    const int64_t slots = d->total / d->chunk + d->nseq;  // >= sum of ceil(len / chunk)
    if (slots > lim || (slots > 0 && d->nheads > kMaxBlocks / slots)) return SSD_ERR_UNSUPPORTED;
    s->B = 1;
    s->L = d->total;
    s->H = d->nheads;
    s->P = d->headdim;
    s->N = d->dstate;
    s->G = d->ngroups;
    s->Q = d->chunk;
    s->T = slots;
    s->dtype = d->dtype;
    s->NS = d->nseq;
    return SSD_OK;
}

// The scan after argument checks: workspace = Acs | states | C.B tiles |
// activated dt | hand-off flags of the chained state pass (layout of
// staged_ws_bytes; the single-kernel path carves its own).
void run_scan(const ScanShape &s, const ssd::DtAct &act, const void *z, const void *x,
              const float *dt, const float *A, const void *B, const void *C, const float *D,
              const float *init_state, void *y, float *final_state, char *ws, hipStream_t hs) {
    float *Acs = reinterpret_cast<float *>(ws);
    float *states = reinterpret_cast<float *>(ws + acs_bytes(s));
    void *scan_ws = ws + acs_bytes(s) + states_bytes(s);
    float *dt_eff = act_active(act)
                        ? reinterpret_cast<float *>(ws + acs_bytes(s) + states_bytes(s) +
                                                    scan_ws_bytes(s))
                        : nullptr;
    if (ssd::fused_supported(s) && !staged_forced()) {
        const int res = resident_blocks();
        const int64_t chains = (s.sch ? s.NS : s.B) * s.H;
        ssd::launch_scan_fused_chain(s, ssd::fused_ws_carve(s, ws), x, dt, A, B, C, D, init_state,
                                     y, final_state, hs, act, z, chain_group(chains, res),
                                     work_queues(), res);
        // a sequence without tokens has no block: its final state is its init
        if (s.sch) ssd::launch_empty_finals(s.sch, s.NS, init_state, final_state, s.H * s.P * s.N, hs);
    } else if (ssd::mfma_supported(s)) {
        void *chain = chain_state_pass(s) ? ws + chain_offset(s) : nullptr;
        ssd::launch_scan_fused_mfma(s, x, dt, A, B, C, D, init_state, y, final_state, Acs, states,
                                    scan_ws, chain, hs, act, dt_eff, z);
        // a sequence without tokens has no block: its final state is its init
        if (chain && s.sch)
            ssd::launch_empty_finals(s.sch, s.NS, init_state, final_state, s.H * s.P * s.N, hs);
    } else {
        ssd::launch_chunk_cumsum(s, dt, A, Acs, hs, act, dt_eff);
        const float *dts = dt_eff ? dt_eff : dt;
        ssd::launch_chunk_state(s, x, B, dts, Acs, states, hs);
        ssd::launch_state_passing(s, states, Acs, init_state, final_state, hs);
        ssd::launch_chunk_cb(s, B, C, scan_ws, hs);
        ssd::launch_chunk_scan(s, x, dts, B, C, D, Acs, states, scan_ws, y, hs, z);
    }
}

ssd_status after_launch() {
    return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}

hipStream_t as_stream(void *stream) { return reinterpret_cast<hipStream_t>(stream); }

// Where the path a call takes keeps its hand-off error word, if it has one.
ssd_status error_word_at(const ScanShape &s, bool empty, size_t *offset) {
    if (empty) return SSD_ERR_UNSUPPORTED;
    if (ssd::fused_supported(s) && !staged_forced()) {
        *offset = 4;
        return SSD_OK;
    }
    if (ssd::mfma_supported(s) && chain_state_pass(s)) {
        *offset = chain_offset(s) + 4;
        return SSD_OK;
    }
    return SSD_ERR_UNSUPPORTED;
}

}  // namespace

extern "C" {

const char *ssd_status_string(int status) {
    switch (status) {
    case SSD_OK: return "ok";
    case SSD_ERR_NULL_PTR: return "a required pointer is NULL";
    case SSD_ERR_SHAPE: return "invalid shape (negative or zero dimension, or nheads % ngroups != 0)";
    case SSD_ERR_UNSUPPORTED:
        return "unsupported argument (chunk, headdim, dstate, dtype, reserved field, or "
               "dt_limit with dt_min > dt_max)";
    case SSD_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case SSD_ERR_WORKSPACE: return "workspace is smaller than the size its query function reports";
    case SSD_ERR_HIP: return "the HIP runtime reported an error at launch";
    case SSD_ERR_SCRATCH:
        return "the call needs more device scratch than the library's built-in "
               "SSD_NOALLOC_SCRATCH_BYTES (use ssd_scan_fwd with a workspace)";
    default: return "unknown status";
    }
}

int ssd_abi_version(void) { return 12; }

ssd_status ssd_scan_error_word(const ssd_scan_desc *d, size_t *offset) {
    if (!offset) return SSD_ERR_NULL_PTR;
    ScanShape s;
    ssd_status st = check_scan(d, &s);
    if (st != SSD_OK) return st;
    return error_word_at(s, s.B == 0 || s.L == 0, offset);
}

ssd_status ssd_varlen_error_word(const ssd_varlen_desc *d, size_t *offset) {
    if (!offset) return SSD_ERR_NULL_PTR;
    ScanShape s;
    ssd_status st = check_varlen(d, &s);
    if (st != SSD_OK) return st;
    return error_word_at(s, s.NS == 0 || s.L == 0, offset);
}

ssd_status ssd_scan_workspace_size(const ssd_scan_desc *d, size_t *bytes) {
    if (!bytes) return SSD_ERR_NULL_PTR;
    ScanShape s;
    ssd_status st = check_scan(d, &s);
    if (st != SSD_OK) return st;
    *bytes = workspace_bytes(s);
    return SSD_OK;
}

ssd_status ssd_scan_fwd_ex(const ssd_scan_desc *d, const ssd_edges *edges, const void *x,
                           const float *dt, const float *A, const void *B, const void *C,
                           const float *D, const float *init_state, void *y,
                           float *final_state, void *workspace, size_t ws_bytes, void *stream) {
    ScanShape s;
    ssd_status st = check_scan(d, &s);
    if (st != SSD_OK) return st;
    ssd::DtAct act;
    const void *z;
    st = read_edges(edges, &act, &z);
    if (st != SSD_OK) return st;
    NormEdge nm;
    st = read_norm(edges, s.H, s.G, &nm);
    if (st != SSD_OK) return st;
    if (s.B == 0) return SSD_OK;
    if (s.L == 0) {
        st = check_ptrs({}, {init_state, final_state});
        if (st != SSD_OK) return st;
        if (final_state)
            ssd::launch_copy_or_zero(final_state, init_state, s.B * s.H * s.P * s.N,
                                     as_stream(stream));
        return after_launch();
    }
    st = check_ptrs({x, dt, A, B, C, y},
                    {D, init_state, final_state, workspace, z, act.bias, nm.w});
    if (st != SSD_OK) return st;
    const size_t need = workspace_bytes(s);
    if (ws_bytes < need) return SSD_ERR_WORKSPACE;
    if (!workspace) return SSD_ERR_NULL_PTR;
    hipStream_t hs = as_stream(stream);
    run_scan(s, act, z, x, dt, A, B, C, D, init_state, y, final_state,
             static_cast<char *>(workspace), hs);
    if (nm.w) ssd::launch_gated_norm(y, nm.w, nm.eps, s.B * s.L, s.H, s.P, nm.groups, s.dtype, hs);
    return after_launch();
}

// The gradient's grid is batch x (seqlen / 32) x nheads blocks at most.
ssd_status check_bwd(const ssd_scan_desc *d, ScanShape *s) {
    ssd_status st = check_scan(d, s);
    if (st != SSD_OK) return st;
    const int64_t T32 = (s->L + 31) / 32;
    if (T32 > 0 && s->B > kMaxBlocks / T32 / s->H) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// Workspace of a gradient beyond its core (Acs, entering states, end-state
// derivatives at the gradient's chunking b): the activated dt (dt activation
// on); the partial sums of dnorm_weight (norm on); the ungated output, the dy
// reaching the scan and the chunk-output stage's workspace (gate or norm
// on); the partial sums of ddt_bias (any edges).
size_t bwd_core_bytes(const ScanShape &b) { return acs_bytes(b) + 2 * states_bytes(b); }

size_t bwd_edges_bytes(const ScanShape &s, const ScanShape &b, bool act, bool gate, bool dbias,
                       int64_t norm_groups) {
    const bool norm = norm_groups > 0;
    size_t n = 0;
    if (act) n += dt_eff_bytes(s);
    if (norm)
        n += round_up((size_t)(ssd::norm_bwd_parts(s.B * s.L, norm_groups) * s.H * s.P) * 4);
    if (gate || norm) {
        const size_t elem = s.dtype == SSD_BF16 ? 2 : 4;
        const size_t nel = (size_t)(s.B * s.L * s.H * s.P);
        n += 2 * round_up(nel * elem) + round_up(ssd::chunk_scan_ws_bytes(b));
        if (s.dtype == SSD_BF16) n += round_up(nel * 4);  // the gated dy unrounded
    }
    if (dbias) n += round_up((size_t)(s.H * ssd::dt_bias_parts(s.B * s.L)) * 4);
    return n;
}

// The edges of a gradient call: as for the forward, and the norm's gradient
// only for the shapes its kernel tiles.
ssd_status read_bwd_edges(const ssd_edges *edges, const ScanShape &s, ssd::DtAct *act,
                          const void **z, NormEdge *nm) {
    ssd_status st = read_edges(edges, act, z);
    if (st != SSD_OK) return st;
    st = read_norm(edges, s.H, s.G, nm);
    if (st != SSD_OK) return st;
    if (nm->w && !ssd::norm_bwd_ok(s.H, s.P, nm->groups)) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// Inputs and outputs of a gradient call.
struct BwdIn {
    const void *x;
    const float *dt, *A;
    const void *B, *C;
    const float *D, *init;
    const void *dy;
    const float *dfinal;
};
struct BwdOut {
    void *dx;
    float *ddt, *dA, *dB, *dC, *dD, *dinit;
    void *dz;
    float *ddt_bias, *dnorm_weight;
};

// Nothing to differentiate (no tokens): dA = dD = ddt_bias = dnorm_weight = 0
// and dinit = dfinal for every row (rows states).
ssd_status bwd_empty(const ScanShape &s, int64_t rows, const BwdIn &in, const BwdOut &o,
                     hipStream_t hs) {
    ssd_status st = check_ptrs({o.dA}, {o.dD, o.dinit, in.dfinal, o.ddt_bias, o.dnorm_weight});
    if (st != SSD_OK) return st;
    ssd::launch_copy_or_zero(o.dA, nullptr, s.H, hs);
    if (o.dD) ssd::launch_copy_or_zero(o.dD, nullptr, s.H, hs);
    if (o.ddt_bias) ssd::launch_copy_or_zero(o.ddt_bias, nullptr, s.H, hs);
    if (o.dnorm_weight) ssd::launch_copy_or_zero(o.dnorm_weight, nullptr, s.H * s.P, hs);
    if (o.dinit) ssd::launch_copy_or_zero(o.dinit, in.dfinal, rows * s.H * s.P * s.N, hs);
    return after_launch();
}

// The gradient after the argument checks: s the call's shape, b the
// gradient's chunking (with the chunk table of a variable-length batch), ws
// at least bwd_core_bytes(b) + bwd_edges_bytes(...) bytes.
void run_bwd(const ScanShape &s, const ScanShape &b, const ssd::DtAct &act, const void *z,
             const NormEdge &nm, bool edges_given, const BwdIn &in, const BwdOut &o, char *ws,
             hipStream_t hs) {
    const bool gate = z != nullptr, actv = act_active(act), norm = nm.w != nullptr;
    float *Acs = reinterpret_cast<float *>(ws);
    float *Hst = reinterpret_cast<float *>(ws + acs_bytes(b));
    float *Est = reinterpret_cast<float *>(ws + acs_bytes(b) + states_bytes(b));
    char *extra = ws + bwd_core_bytes(b);
    float *dt_eff = nullptr;
    if (actv) {
        dt_eff = reinterpret_cast<float *>(extra);
        extra += dt_eff_bytes(s);
    }
    float *npart = nullptr;
    if (norm) {
        npart = reinterpret_cast<float *>(extra);
        extra += round_up((size_t)(ssd::norm_bwd_parts(s.B * s.L, nm.groups) * s.H * s.P) * 4);
    }
    void *yun = nullptr, *dys = nullptr, *cbws = nullptr;
    float *dys32 = nullptr;  // bf16 calls: the gated dy in fp32 for the state derivatives
    const int64_t nel = s.B * s.L * s.H * s.P;
    if (gate || norm) {
        const size_t eb = round_up((size_t)nel * (s.dtype == SSD_BF16 ? 2 : 4));
        yun = extra;
        dys = extra + eb;
        cbws = extra + 2 * eb;
        extra += 2 * eb + round_up(ssd::chunk_scan_ws_bytes(b));
        if (s.dtype == SSD_BF16) {
            dys32 = reinterpret_cast<float *>(extra);
            extra += round_up((size_t)nel * 4);
        }
    }
    float *part = (edges_given && o.ddt_bias) ? reinterpret_cast<float *>(extra) : nullptr;
    // outputs accumulated with atomics start from zero (a fill kernel, so the
    // call can be captured in a HIP graph)
    const int64_t bcn = s.B * s.L * s.G * s.N;
    ssd::launch_zero4(o.dB, bcn, o.dC, bcn, o.dA, s.H, o.dD, s.H, hs);
    // the forward's Acs (and the activated dt) and entering states at the
    // gradient's chunks (on the matrix cores, the cumsum in the same launch)
    const bool mm = ssd::bwd_states_mfma_ok(b);
    const float *dtu = dt_eff ? dt_eff : in.dt;
    if (mm) {
        ssd::launch_bwd_states_cumsum_mfma(b, in.x, in.B, in.dt, in.A, Acs, Hst, act, dt_eff, hs);
    } else {
        ssd::launch_chunk_cumsum(b, in.dt, in.A, Acs, hs, act, dt_eff);
        ssd::launch_chunk_state(b, in.x, in.B, dtu, Acs, Hst, hs);
    }
    ssd::launch_state_passing(b, Hst, Acs, in.init, nullptr, hs);
    // gate / norm: the ungated output from the chunk-output stage on those
    // states, then the gradient reaching the scan output, dz and dnorm_weight
    const void *dyu = in.dy;
    if (gate || norm) {
        ssd::launch_chunk_cb(b, in.B, in.C, cbws, hs);
        ssd::launch_chunk_scan(b, in.x, dtu, in.B, in.C, in.D, Acs, Hst, cbws, yun, hs);
        if (norm)
            ssd::launch_norm_gate_bwd(in.dy, yun, z, nm.w, nm.eps, s.B * s.L, s.H, s.P, nm.groups,
                                      dys, o.dz, npart, o.dnorm_weight, s.dtype, hs, dys32);
        else
            ssd::launch_gate_bwd(in.dy, yun, z, dys, o.dz, nel, s.dtype, hs, dys32);
        dyu = dys;
    }
    // derivatives with respect to every chunk's end state, and the initial
    // state's: from the unrounded gated dy when there is one (the bf16 copy
    // would put one more rounding into sums that can cancel)
    if (mm) {
        if (dys32) ssd::launch_bwd_states_mfma(b, dys32, in.C, nullptr, Acs, Est, true, hs, true);
        else ssd::launch_bwd_states_mfma(b, dyu, in.C, nullptr, Acs, Est, true, hs);
    } else {
        ssd::launch_chunk_dstate(b, dys32 ? static_cast<const void *>(dys32) : dyu, in.C, Acs,
                                 Est, hs, dys32 != nullptr);
    }
    ssd::launch_state_passing_rev(b, Est, Acs, in.dfinal, o.dinit, hs);
    // per-chunk gradients
    ssd::launch_chunk_bwd(b, in.x, dtu, in.A, in.B, in.C, in.D, Acs, Hst, Est, dyu, o.dx, o.ddt,
                          o.dB, o.dC, o.dA, o.dD, hs);
    // through the dt activation, and the bias's gradient
    if (actv || part)
        ssd::launch_dt_act_bwd(o.ddt, in.dt, act, s.B * s.L, s.H, part, part ? o.ddt_bias : nullptr,
                               hs);
}

ssd_status ssd_scan_bwd_workspace_size(const ssd_scan_desc *d, size_t *bytes) {
    return ssd_scan_bwd_ex_workspace_size(d, nullptr, bytes);
}

ssd_status ssd_scan_bwd_ex_workspace_size(const ssd_scan_desc *d, const ssd_edges *edges,
                                          size_t *bytes) {
    if (!bytes) return SSD_ERR_NULL_PTR;
    ScanShape s;
    ssd_status st = check_bwd(d, &s);
    if (st != SSD_OK) return st;
    ssd::DtAct act;
    const void *z;
    NormEdge nm;
    st = read_bwd_edges(edges, s, &act, &z, &nm);
    if (st != SSD_OK) return st;
    if (s.B == 0 || s.L == 0) {
        *bytes = 0;
        return SSD_OK;
    }
    const ScanShape b = bwd_shape(s);
    *bytes = bwd_core_bytes(b) + bwd_edges_bytes(s, b, act_active(act), z != nullptr,
                                                 edges != nullptr, nm.w ? nm.groups : 0);
    return SSD_OK;
}

ssd_status ssd_scan_bwd(const ssd_scan_desc *d, const void *x, const float *dt, const float *A,
                        const void *B, const void *C, const float *D, const float *init_state,
                        const void *dy, const float *dfinal, void *dx, float *ddt, float *dA,
                        float *dB, float *dC, float *dD, float *dinit, void *workspace,
                        size_t ws_bytes, void *stream) {
    return ssd_scan_bwd_ex(d, nullptr, x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt, dA,
                           dB, dC, dD, dinit, nullptr, nullptr, nullptr, workspace, ws_bytes,
                           stream);
}

ssd_status ssd_scan_bwd_ex(const ssd_scan_desc *d, const ssd_edges *edges, const void *x,
                           const float *dt, const float *A, const void *B, const void *C,
                           const float *D, const float *init_state, const void *dy,
                           const float *dfinal, void *dx, float *ddt, float *dA, float *dB,
                           float *dC, float *dD, float *dinit, void *dz, float *ddt_bias,
                           float *dnorm_weight, void *workspace, size_t ws_bytes,
                           void *stream) {
    ScanShape s;
    ssd_status st = check_bwd(d, &s);
    if (st != SSD_OK) return st;
    ssd::DtAct act;
    const void *z;
    NormEdge nm;
    st = read_bwd_edges(edges, s, &act, &z, &nm);
    if (st != SSD_OK) return st;
    const BwdIn in{x, dt, A, B, C, D, init_state, dy, dfinal};
    const BwdOut o{dx, ddt, dA, dB, dC, dD, dinit, z ? dz : nullptr,
                   edges ? ddt_bias : nullptr, nm.w ? dnorm_weight : nullptr};
    hipStream_t hs = as_stream(stream);
    if (s.B == 0 || s.L == 0) return bwd_empty(s, s.B, in, o, hs);
    if (z && !dz) return SSD_ERR_NULL_PTR;
    st = check_ptrs({x, dt, A, B, C, dy, dx, ddt, dA, dB, dC},
                    {D, init_state, dfinal, dD, dinit, workspace, z, o.dz, act.bias, o.ddt_bias,
                     nm.w, o.dnorm_weight});
    if (st != SSD_OK) return st;
    const ScanShape b = bwd_shape(s);
    const size_t need = bwd_core_bytes(b) + bwd_edges_bytes(s, b, act_active(act), z != nullptr,
                                                            edges != nullptr, nm.w ? nm.groups : 0);
    if (ws_bytes < need) return SSD_ERR_WORKSPACE;
    if (!workspace) return SSD_ERR_NULL_PTR;
    run_bwd(s, b, act, z, nm, edges != nullptr, in, o, static_cast<char *>(workspace), hs);
    return after_launch();
}

ssd_status ssd_varlen_workspace_size(const ssd_varlen_desc *d, size_t *bytes) {
    if (!bytes) return SSD_ERR_NULL_PTR;
    ScanShape s;
    ssd_status st = check_varlen(d, &s);
    if (st != SSD_OK) return st;
    *bytes = (s.NS == 0 || s.L == 0) ? 0 : workspace_bytes(s) + varlen_table_bytes(s);
    return SSD_OK;
}

ssd_status ssd_scan_fwd_varlen(const ssd_varlen_desc *d, const ssd_edges *edges,
                               const int32_t *cu_seqlens, const void *x, const float *dt,
                               const float *A, const void *B, const void *C, const float *D,
                               const float *init_states, void *y, float *final_states,
                               void *workspace, size_t ws_bytes, void *stream) {
    ScanShape s;
    ssd_status st = check_varlen(d, &s);
    if (st != SSD_OK) return st;
    ssd::DtAct act;
    const void *z;
    st = read_edges(edges, &act, &z);
    if (st != SSD_OK) return st;
    NormEdge nm;
    st = read_norm(edges, s.H, s.G, &nm);
    if (st != SSD_OK) return st;
    if (s.NS == 0) return SSD_OK;
    if (s.L == 0) {  // every sequence is empty
        st = check_ptrs({}, {init_states, final_states});
        if (st != SSD_OK) return st;
        if (final_states)
            ssd::launch_copy_or_zero(final_states, init_states, s.NS * s.H * s.P * s.N,
                                     as_stream(stream));
        return after_launch();
    }
    st = check_ptrs({cu_seqlens, x, dt, A, B, C, y},
                    {D, init_states, final_states, workspace, z, act.bias, nm.w});
    if (st != SSD_OK) return st;
    const size_t base = workspace_bytes(s);
    if (ws_bytes < base + varlen_table_bytes(s)) return SSD_ERR_WORKSPACE;
    if (!workspace) return SSD_ERR_NULL_PTR;
    char *ws = static_cast<char *>(workspace);
    int2 *ctab = reinterpret_cast<int2 *>(ws + base);
    int2 *sch = reinterpret_cast<int2 *>(ws + base + round_up((size_t)s.T * 8));
    int2 *spos = reinterpret_cast<int2 *>(ws + base + round_up((size_t)s.T * 8) +
                                          round_up((size_t)s.NS * 8));
    hipStream_t hs = as_stream(stream);
    ssd::launch_varlen_table(cu_seqlens, s.NS, s.L, s.Q, s.T, ctab, sch, spos, hs);
    s.ctab = ctab;
    s.sch = sch;
    s.spos = spos;
    run_scan(s, act, z, x, dt, A, B, C, D, init_states, y, final_states, ws, hs);
    if (nm.w) ssd::launch_gated_norm(y, nm.w, nm.eps, s.L, s.H, s.P, nm.groups, s.dtype, hs);
    return after_launch();
}

// The gradient of a ragged batch: checks of ssd_scan_fwd_varlen, the
// gradient's own chunking with its chunk table.
ssd_status check_bwd_varlen(const ssd_varlen_desc *d, ScanShape *s, ScanShape *b) {
    ssd_status st = check_varlen(d, s);
    if (st != SSD_OK) return st;
    *b = bwd_varlen_shape(*s);
    if (b->T > kMaxBlocks || (b->T > 0 && s->H > kMaxBlocks / b->T)) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

ssd_status ssd_scan_bwd_varlen_workspace_size(const ssd_varlen_desc *d, const ssd_edges *edges,
                                              size_t *bytes) {
    if (!bytes) return SSD_ERR_NULL_PTR;
    ScanShape s, b;
    ssd_status st = check_bwd_varlen(d, &s, &b);
    if (st != SSD_OK) return st;
    ssd::DtAct act;
    const void *z;
    NormEdge nm;
    st = read_bwd_edges(edges, s, &act, &z, &nm);
    if (st != SSD_OK) return st;
    if (s.NS == 0 || s.L == 0) {
        *bytes = 0;
        return SSD_OK;
    }
    *bytes = bwd_core_bytes(b) +
             bwd_edges_bytes(s, b, act_active(act), z != nullptr, edges != nullptr,
                             nm.w ? nm.groups : 0) +
             varlen_table_bytes(b);
    return SSD_OK;
}

ssd_status ssd_scan_bwd_varlen(const ssd_varlen_desc *d, const ssd_edges *edges,
                               const int32_t *cu_seqlens, const void *x, const float *dt,
                               const float *A, const void *B, const void *C, const float *D,
                               const float *init_states, const void *dy,
                               const float *dfinal_states, void *dx, float *ddt, float *dA,
                               float *dB, float *dC, float *dD, float *dinit_states, void *dz,
                               float *ddt_bias, float *dnorm_weight, void *workspace,
                               size_t ws_bytes, void *stream) {
    ScanShape s, b;
    ssd_status st = check_bwd_varlen(d, &s, &b);
    if (st != SSD_OK) return st;
    ssd::DtAct act;
    const void *z;
    NormEdge nm;
    st = read_bwd_edges(edges, s, &act, &z, &nm);
    if (st != SSD_OK) return st;
    const BwdIn in{x, dt, A, B, C, D, init_states, dy, dfinal_states};
    const BwdOut o{dx, ddt, dA, dB, dC, dD, dinit_states, z ? dz : nullptr,
                   edges ? ddt_bias : nullptr, nm.w ? dnorm_weight : nullptr};
    hipStream_t hs = as_stream(stream);
    if (s.NS == 0 || s.L == 0) return bwd_empty(s, s.NS, in, o, hs);
    if (z && !dz) return SSD_ERR_NULL_PTR;
    st = check_ptrs({cu_seqlens, x, dt, A, B, C, dy, dx, ddt, dA, dB, dC},
                    {D, init_states, dfinal_states, dD, dinit_states, workspace, z, o.dz,
                     act.bias, o.ddt_bias, nm.w, o.dnorm_weight});
    if (st != SSD_OK) return st;
    const size_t base = bwd_core_bytes(b) + bwd_edges_bytes(s, b, act_active(act), z != nullptr,
                                                            edges != nullptr, nm.w ? nm.groups : 0);
    if (ws_bytes < base + varlen_table_bytes(b)) return SSD_ERR_WORKSPACE;
    if (!workspace) return SSD_ERR_NULL_PTR;
    char *ws = static_cast<char *>(workspace);
    int2 *ctab = reinterpret_cast<int2 *>(ws + base);
    int2 *sch = reinterpret_cast<int2 *>(ws + base + round_up((size_t)b.T * 8));
    ssd::launch_varlen_table(cu_seqlens, s.NS, s.L, b.Q, b.T, ctab, sch, nullptr, hs);
    b.ctab = ctab;
    b.sch = sch;
    run_bwd(s, b, act, z, nm, edges != nullptr, in, o, ws, hs);
    return after_launch();
}

ssd_status ssd_scan_fwd(const ssd_scan_desc *d, const void *x, const float *dt, const float *A,
                        const void *B, const void *C, const float *D, const float *init_state,
                        void *y, float *final_state, void *workspace, size_t ws_bytes,
                        void *stream) {
    return ssd_scan_fwd_ex(d, nullptr, x, dt, A, B, C, D, init_state, y, final_state, workspace,
                           ws_bytes, stream);
}

ssd_status ssd_scan_fwd_noalloc(const ssd_scan_desc *d, const void *x, const float *dt,
                                const float *A, const void *B, const void *C, const float *D,
                                const float *init_state, void *y, float *final_state,
                                void *stream) {
    ScanShape s;
    ssd_status st = check_scan(d, &s);
    if (st != SSD_OK) return st;
    if (s.B == 0) return SSD_OK;
    if (s.L == 0) {
        st = check_ptrs({}, {init_state, final_state});
        if (st != SSD_OK) return st;
        if (final_state)
            ssd::launch_copy_or_zero(final_state, init_state, s.B * s.H * s.P * s.N,
                                     as_stream(stream));
        return after_launch();
    }
    st = check_ptrs({x, dt, A, B, C, y}, {D, init_state, final_state});
    if (st != SSD_OK) return st;
    const size_t need = workspace_bytes(s);
    if (need > SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_SCRATCH;
    void *ws = nullptr;
    if (ssd::scratch_ptr(&ws) != hipSuccess || !ws) return SSD_ERR_HIP;
    run_scan(s, ssd::DtAct{}, nullptr, x, dt, A, B, C, D, init_state, y, final_state,
             static_cast<char *>(ws), as_stream(stream));
    return after_launch();
}

ssd_status ssd_step_multi_ex(const ssd_step_desc *d, const ssd_edges *edges, int64_t nsteps,
                             float *state, const void *x, const float *dt, const float *A,
                             const void *B, const void *C, const float *D, void *y,
                             void *stream) {
    if (!d) return SSD_ERR_NULL_PTR;
    ssd_status st = check_common(d->batch, d->nheads, d->headdim, d->dstate, d->ngroups,
                                 d->dtype, d->reserved);
    if (st != SSD_OK) return st;
    if (nsteps < 0) return SSD_ERR_SHAPE;
    ssd::DtAct act;
    const void *z;
    st = read_edges(edges, &act, &z);
    if (st != SSD_OK) return st;
    NormEdge nm;
    st = read_norm(edges, d->nheads, d->ngroups, &nm);
    if (st != SSD_OK) return st;
    if (d->batch == 0 || nsteps == 0) return SSD_OK;
    if (d->batch > kMaxBlocks / d->nheads / d->headdim) return SSD_ERR_UNSUPPORTED;
    st = check_ptrs({state, x, dt, A, B, C, y}, {D, z, act.bias, nm.w});
    if (st != SSD_OK) return st;
    StepShape s{d->batch, d->nheads, d->headdim, d->dstate, d->ngroups, d->dtype};
    hipStream_t hs = as_stream(stream);
    ssd::launch_step(s, nsteps, state, x, dt, A, B, C, D, y, act, z, hs);
    if (nm.w)
        ssd::launch_gated_norm(y, nm.w, nm.eps, d->batch * nsteps, d->nheads, d->headdim,
                               nm.groups, d->dtype, hs);
    return after_launch();
}

ssd_status ssd_step_ex(const ssd_step_desc *d, const ssd_edges *edges, float *state,
                       const void *x, const float *dt, const float *A, const void *B,
                       const void *C, const float *D, void *y, void *stream) {
    if (!d) return SSD_ERR_NULL_PTR;
    ssd_status st = check_common(d->batch, d->nheads, d->headdim, d->dstate, d->ngroups,
                                 d->dtype, d->reserved);
    if (st != SSD_OK) return st;
    ssd::DtAct act;
    const void *z;
    st = read_edges(edges, &act, &z);
    if (st != SSD_OK) return st;
    NormEdge nm;
    st = read_norm(edges, d->nheads, d->ngroups, &nm);
    if (st != SSD_OK) return st;
    if (d->batch == 0) return SSD_OK;
    if (d->batch > kMaxBlocks / d->nheads / d->headdim) return SSD_ERR_UNSUPPORTED;
    st = check_ptrs({state, x, dt, A, B, C, y}, {D, z, act.bias, nm.w});
    if (st != SSD_OK) return st;
    StepShape s{d->batch, d->nheads, d->headdim, d->dstate, d->ngroups, d->dtype};
    hipStream_t hs = as_stream(stream);
    ssd::launch_step(s, -1, state, x, dt, A, B, C, D, y, act, z, hs);
    if (nm.w)
        ssd::launch_gated_norm(y, nm.w, nm.eps, d->batch, d->nheads, d->headdim, nm.groups,
                               d->dtype, hs);
    return after_launch();
}

ssd_status ssd_step(const ssd_step_desc *d, float *state, const void *x, const float *dt,
                    const float *A, const void *B, const void *C, const float *D, void *y,
                    void *stream) {
    return ssd_step_ex(d, nullptr, state, x, dt, A, B, C, D, y, stream);
}

ssd_status ssd_step_multi(const ssd_step_desc *d, int64_t nsteps, float *state, const void *x,
                          const float *dt, const float *A, const void *B, const void *C,
                          const float *D, void *y, void *stream) {
    return ssd_step_multi_ex(d, nullptr, nsteps, state, x, dt, A, B, C, D, y, stream);
}

ssd_status ssd_chunk_cumsum(const ssd_scan_desc *d, const float *dt, const float *A,
                            float *Acs, void *stream) {
    ScanShape s;
    ssd_status st = check_scan(d, &s);
    if (st != SSD_OK) return st;
    if (s.B == 0 || s.L == 0) return SSD_OK;
    st = check_ptrs({dt, A, Acs}, {});
    if (st != SSD_OK) return st;
    ssd::launch_chunk_cumsum(s, dt, A, Acs, as_stream(stream));
    return after_launch();
}

ssd_status ssd_chunk_state(const ssd_scan_desc *d, const void *x, const void *B,
                           const float *dt, const float *Acs, float *states, void *stream) {
    ScanShape s;
    ssd_status st = check_scan(d, &s);
    if (st != SSD_OK) return st;
    if (s.B == 0 || s.L == 0) return SSD_OK;
    st = check_ptrs({x, B, dt, Acs, states}, {});
    if (st != SSD_OK) return st;
    ssd::launch_chunk_state(s, x, B, dt, Acs, states, as_stream(stream));
    return after_launch();
}

ssd_status ssd_state_passing(const ssd_scan_desc *d, float *states, const float *Acs,
                             const float *init_state, float *final_state, void *stream) {
    ScanShape s;
    ssd_status st = check_scan(d, &s);
    if (st != SSD_OK) return st;
    if (s.B == 0) return SSD_OK;
    if (s.L == 0) {
        st = check_ptrs({}, {init_state, final_state});
        if (st != SSD_OK) return st;
        if (final_state)
            ssd::launch_copy_or_zero(final_state, init_state, s.B * s.H * s.P * s.N,
                                     as_stream(stream));
        return after_launch();
    }
    st = check_ptrs({states, Acs}, {init_state, final_state});
    if (st != SSD_OK) return st;
    ssd::launch_state_passing(s, states, Acs, init_state, final_state, as_stream(stream));
    return after_launch();
}

ssd_status ssd_chunk_scan_workspace_size(const ssd_scan_desc *d, size_t *bytes) {
    if (!bytes) return SSD_ERR_NULL_PTR;
    ScanShape s;
    ssd_status st = check_scan(d, &s);
    if (st != SSD_OK) return st;
    *bytes = scan_ws_bytes(s);
    return SSD_OK;
}

ssd_status ssd_chunk_cb(const ssd_scan_desc *d, const void *B, const void *C, void *workspace,
                        size_t ws_bytes, void *stream) {
    ScanShape s;
    ssd_status st = check_scan(d, &s);
    if (st != SSD_OK) return st;
    const size_t need = scan_ws_bytes(s);
    if (need == 0) return SSD_OK;
    st = check_ptrs({B, C, workspace}, {});
    if (st != SSD_OK) return st;
    if (ws_bytes < need) return SSD_ERR_WORKSPACE;
    ssd::launch_chunk_cb(s, B, C, workspace, as_stream(stream));
    return after_launch();
}

ssd_status ssd_chunk_scan(const ssd_scan_desc *d, const void *x, const float *dt,
                          const void *B, const void *C, const float *D, const float *Acs,
                          const float *states, void *y, const void *workspace, size_t ws_bytes,
                          void *stream) {
    ScanShape s;
    ssd_status st = check_scan(d, &s);
    if (st != SSD_OK) return st;
    if (s.B == 0 || s.L == 0) return SSD_OK;
    st = check_ptrs({x, dt, B, C, Acs, states, y}, {D, workspace});
    if (st != SSD_OK) return st;
    const size_t need = scan_ws_bytes(s);
    if (ws_bytes < need) return SSD_ERR_WORKSPACE;
    if (need && !workspace) return SSD_ERR_NULL_PTR;
    ssd::launch_chunk_scan(s, x, dt, B, C, D, Acs, states, workspace, y, as_stream(stream));
    return after_launch();
}

}  // extern "C"
