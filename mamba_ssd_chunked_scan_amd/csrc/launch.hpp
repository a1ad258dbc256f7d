// Internal launch interface between the C-ABI layer (ssd_api.cpp) and the
// kernels.  Shapes arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

struct ScanShape {
    int64_t B, L, H, P, N, G, Q, T;  // T = ceil(L / Q)
    int dtype;                        // SSD_F32 or SSD_BF16
    // Variable-length batches (null otherwise): B = 1, L = all tokens packed,
    // T = chunk slots; ctab[T] = {first token, length} of every slot (length
    // 0: unused), sch[NS] = {first slot, slots} of every sequence.
    const int2 *ctab = nullptr;
    const int2 *sch = nullptr;
    int64_t NS = 0;
    // slot -> {sequence, position within it} (sequence -1: unused slot)
    const int2 *spos = nullptr;
};

struct StepShape {
    int64_t B, H, P, N, G;
    int dtype;
};

// Activation of the raw step size fused into the first kernel that reads dt:
// d <- d + bias[h] (bias non-null), softplus(d) (softplus != 0), clamp to
// [lo, hi] (limit != 0).  Zero-initialised it is the identity.
struct DtAct {
    const float *bias;
    float lo, hi;
    int softplus, limit;
};

// Stage kernels of the chunked scan (layouts as in include/ssd.h).
// With an active act, the activated dt is used and written to dt_out (when
// non-null) in dt's layout for the later stages.
void launch_chunk_cumsum(const ScanShape &s, const float *dt, const float *A, float *Acs,
                         hipStream_t st, const DtAct &act = DtAct{}, float *dt_out = nullptr);
void launch_chunk_state(const ScanShape &s, const void *x, const void *Bm, const float *dt,
                        const float *Acs, float *states, hipStream_t st);
void launch_state_passing(const ScanShape &s, float *states, const float *Acs,
                          const float *init, float *fin, hipStream_t st);
// Device workspace of the chunk-output stage (0 when its kernel needs none).
size_t chunk_scan_ws_bytes(const ScanShape &s);
// C.B tiles into the chunk-output workspace (no-op when it needs none).
void launch_chunk_cb(const ScanShape &s, const void *Bm, const void *Cm, void *ws, hipStream_t st);
void launch_chunk_scan(const ScanShape &s, const void *x, const float *dt, const void *Bm,
                       const void *Cm, const float *D, const float *Acs, const float *states,
                       const void *ws, void *y, hipStream_t st, const void *z = nullptr);

// Chunk table of a variable-length batch (ScanShape::ctab / sch / spos) from
// the sequences' token offsets cu[0..NS]; slots >= the number of chunks.
// spos may be null.
void launch_varlen_table(const int32_t *cu, int64_t NS, int64_t total, int64_t Q, int64_t slots,
                         int2 *ctab, int2 *sch, int2 *spos, hipStream_t st);

// Gated RMSNorm of finished outputs, in place: y is ntok rows of H*P values
// (heads outer), each split into NG groups of whole heads; every group is
// scaled by 1 / sqrt(mean square + eps) and then by w (per channel).
void launch_gated_norm(void *y, const float *w, float eps, int64_t ntok, int64_t H, int64_t P,
                       int64_t NG, int dtype, hipStream_t st);

// Final states of a variable-length batch's empty sequences (sch[s].y == 0):
// init (or zeros) copied to fin; per = state values per sequence (H P N, a
// multiple of 4).  No-op when fin is null.
void launch_empty_finals(const int2 *sch, int64_t NS, const float *init, float *fin,
                         int64_t per, hipStream_t st);

// The current device's address of the built-in scratch of
// ssd_scan_fwd_noalloc (SSD_NOALLOC_SCRATCH_BYTES), looked up once per device.
hipError_t scratch_ptr(void **out);

// dst[i] = src ? src[i] : 0 for i < n (no-op when dst == src).
void launch_copy_or_zero(float *dst, const float *src, int64_t n, hipStream_t st);
// Zero up to four fp32 buffers of the given element counts in one launch
// (null pointers are skipped).
void launch_zero4(float *a, int64_t na, float *b, int64_t nb, float *c, int64_t nc, float *d,
                  int64_t nd, hipStream_t st);

// Decode: nsteps < 0 is one token with [B, ...] inputs; nsteps >= 1 tokens
// in one launch with inputs in the prefill layout [B, nsteps, ...].  z (the
// output gate, x's layout) may be null.
void launch_step(const StepShape &s, int64_t nsteps, float *state, const void *x,
                 const float *dt, const float *A, const void *Bm, const void *Cm, const float *D,
                 void *y, const DtAct &act, const void *z, hipStream_t st);

// Gradient (fixed chunking, generic kernels):
// dS_c = sum_s exp(Acs_s) dy_s C_s^T per chunk (states layout) ...
void launch_chunk_dstate(const ScanShape &s, const void *dy, const void *Cm, const float *Acs,
                         float *dstates, hipStream_t st, bool dy_f32 = false);
// ... turned in place, last chunk first, into the derivative with respect to
// each chunk's end state; dinit (may be null) gets the initial state's.
void launch_state_passing_rev(const ScanShape &s, float *dstates, const float *Acs,
                              const float *dfin, float *dinit, hipStream_t st);
// Per-chunk gradients from the entering states H and the end-state
// derivatives E: dx and ddt written; dB, dC (fp32), dA, dD (may be null)
// accumulated with atomics into zeroed buffers.  s.Q is 32, or 64 on the
// matrix-core path.
void launch_chunk_bwd(const ScanShape &s, const void *x, const float *dt, const float *A,
                      const void *Bm, const void *Cm, const float *D, const float *Acs,
                      const float *Hs, const float *Es, const void *dy, void *dx, float *ddt,
                      float *dB, float *dC, float *dA, float *dD, hipStream_t st);

// Whether the gradient takes the matrix-core path (bf16, headdim 64, d_state
// 64 or 128, fixed length); it then runs at 64-token chunks, else at 32.
bool bwd_mfma_ok(const ScanShape &s);
// Gradient through the output gate y_out = y * silu(z), elementwise over n
// values of x's layout: dys = dy * silu(z), dz = dy * y * silu'(z).
// dys32 (may be null): the same dys in fp32, unrounded.
void launch_gate_bwd(const void *dy, const void *y, const void *z, void *dys, void *dz,
                     int64_t n, int dtype, hipStream_t st, float *dys32 = nullptr);
// Gradient through the dt activation, in place: ddt [rows][H] with respect
// to the activated dt becomes the gradient with respect to the raw dt; when
// dbias is non-null it gets the per-head sums over the rows (fixed order,
// through part: H * dt_bias_parts(rows) floats of workspace).
int64_t dt_bias_parts(int64_t rows);
void launch_dt_act_bwd(float *ddt, const float *dt_raw, const DtAct &act, int64_t rows,
                       int64_t H, float *part, float *dbias, hipStream_t st);

// Gradient through the gated RMSNorm (and the gate under it when z is
// non-null): dys gets the gradient reaching the scan output, dz the gate's,
// dw (may be null) the weight's, through part (norm_bwd_parts(ntok, NG) x
// H*P floats).  Shapes norm_bwd_ok accepts: headdim a multiple of 8, groups
// of at most 8192 channels.
bool norm_bwd_ok(int64_t H, int64_t P, int64_t NG);
int64_t norm_bwd_parts(int64_t ntok, int64_t NG);
void launch_norm_gate_bwd(const void *dout, const void *y, const void *z, const float *w,
                          float eps, int64_t ntok, int64_t H, int64_t P, int64_t NG, void *dys,
                          void *dz, float *part, float *dw, int dtype, hipStream_t st,
                          float *dys32 = nullptr);

// The gradient's 64-token chunk states (and their adjoint, with x = dy and
// B = C) on the matrix cores, for bwd_mfma_ok shapes.
bool bwd_states_mfma_ok(const ScanShape &s);
// x_f32: xin is fp32 (adjoint only), not the call's dtype.
void launch_bwd_states_mfma(const ScanShape &s, const void *xin, const void *bin,
                            const float *dt, const float *Acs, float *out, bool adjoint,
                            hipStream_t st, bool x_f32 = false);
// The gradient's forward chunk states with the chunk cumsum formed in the same
// launch (written to Acs; with an active act, the activated dt to dt_out).
void launch_bwd_states_cumsum_mfma(const ScanShape &s, const void *x, const void *Bm,
                                   const float *dt, const float *A, float *Acs, float *out,
                                   const DtAct &act, float *dt_out, hipStream_t st);

// Compute units of the current device (looked up once per device).
int device_cus();

// Whether the MFMA kernels handle this shape (otherwise the generic ones run).
bool mfma_supported(const ScanShape &s);
void launch_chunk_state_mfma(const ScanShape &s, const void *x, const void *Bm,
                             const float *dt, const float *Acs, float *states, hipStream_t st);
// C.B tiles of every (b, c, g), shared by the heads of a group (chunk_cb_bytes).
size_t chunk_cb_bytes(const ScanShape &s);
void launch_chunk_cb_mfma(const ScanShape &s, const void *Bm, const void *Cm, void *cb,
                          hipStream_t st);
// Workspace of the chained state pass: control words (the error word at byte
// 4, the tickets of the eight per-XCD work queues at words 8..15) and one
// 64-bit flag per (chunk slot, head, wave).
size_t chain_ws_bytes(const ScanShape &s);
// ssd_scan_fwd on the MFMA path, three launches.  With `chain` (a region of
// chain_ws_bytes): the C.B tiles, the chunk states with the in-block cumsum
// and the chained state pass, the chunk output.  Without: the chunk states,
// the separate state pass with the C.B tiles, the chunk output.  With an
// active act, the chunk-state kernel writes the activated dt to dt_out, which
// the chunk-output kernel then reads; z may be null.
void launch_scan_fused_mfma(const ScanShape &s, const void *x, const float *dt, const float *A,
                            const void *Bm, const void *Cm, const float *D, const float *init,
                            void *y, float *fin, float *Acs, float *states, void *cb, void *chain,
                            hipStream_t st, const DtAct &act = DtAct{},
                            float *dt_out = nullptr, const void *z = nullptr);
void launch_chunk_scan_mfma(const ScanShape &s, const void *x, const float *dt, const void *Cm,
                            const float *D, const float *Acs, const float *states, const void *cb,
                            void *y, hipStream_t st, const void *z = nullptr);

// The single-kernel prefill (chunk 256, MFMA shapes): chunk states handed on
// from block to block.  Workspace: a 256-byte control block (ticket, error
// word at byte 4), the hand-off flags, the C.B tiles and fragments, the
// hand-off states.
struct FusedWs {
    unsigned *ctl;
    unsigned long long *flags;
    void *cb;
    float *hand;
};
bool fused_supported(const ScanShape &s);
size_t fused_ws_bytes(const ScanShape &s);
FusedWs fused_ws_carve(const ScanShape &s, void *ws);
// grp: chunks per hand-off group (>= 1); nq: work queues (1, or 8: one per
// XCD); max_blocks: the persistent grid.
void launch_scan_fused_chain(const ScanShape &s, const FusedWs &w, const void *x, const float *dt,
                             const float *A, const void *Bm, const void *Cm, const float *D,
                             const float *init, void *y, float *fin, hipStream_t st,
                             const DtAct &act, const void *z, int grp, int nq, int max_blocks);

}  // namespace ssd
