/*
 * ssd.h - C ABI of libssd, the MI355X (gfx950) Mamba-2 SSD selective scan.
 *
 * The operation.  Per batch row b, head h (group g = h / (nheads/ngroups)) and
 * channel p, with a = A[h] and the state s[n] carried over tokens t:
 *
 *     s[n]        = exp(dt[b,t,h] * a) * s[n] + dt[b,t,h] * x[b,t,h,p] * B[b,t,g,n]
 *     y[b,t,h,p]  = sum_n C[b,t,g,n] * s[n] + D[h] * x[b,t,h,p]
 *
 * starting from init_state (zero when NULL) and ending in final_state.  A is
 * one scalar per head, which is what reduces the transition to a scalar
 * exponential ("Compiler-First State Space Duality and Portable O(1)
 * Autoregressive Caching for Inference", paperlayer summary, §3 Method,
 * "State-space duality").  ssd_scan_fwd evaluates it with the chunked
 * algorithm of the same section ("Chunked recurrence"): a matrix form inside
 * each chunk of `chunk` tokens and a sequential pass of one summary state per
 * chunk; results do not depend on the chunk size beyond rounding.  ssd_step is
 * one token of the recurrence on a caller-owned, fixed-size state (§3,
 * "Autoregressive cache"), updated in place as the block-level step method of
 * the pyshine "Mamba" repository tour describes.
 *
 * Conventions for every entry point.
 *  - Pointers are DEVICE pointers, 16-byte aligned, to contiguous row-major
 *    arrays with the layouts given below.  The caller owns every buffer,
 *    including the workspace; the library never allocates or frees memory,
 *    never synchronises, and keeps no state between calls (reentrant).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns at once.  Asynchronous faults surface at the caller's
 *    next synchronisation.
 *  - Every argument check runs before the first HIP call; on error nothing is
 *    enqueued.  After enqueueing, a launch failure reported by
 *    hipGetLastError is returned as SSD_ERR_HIP.  No C++ exception crosses
 *    this interface.
 *  - Values are not checked: NaN/Inf propagate.  dt >= 0 and A <= 0 are
 *    preconditions (decays must not exceed 1); they are not verified.
 *  - dtype (SSD_F32 or SSD_BF16) applies to x, B, C and y.  dt, A, D and all
 *    states are always fp32.  bf16 results are rounded to nearest even from
 *    fp32 accumulators.
 *  - Index arithmetic is 64-bit; any size that fits device memory is accepted.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssd_status {
    SSD_OK = 0,
    SSD_ERR_NULL_PTR = 1,    /* a required pointer is NULL                       */
    SSD_ERR_SHAPE = 2,       /* negative/zero dimension, nheads % ngroups != 0   */
    SSD_ERR_UNSUPPORTED = 3, /* chunk, headdim or dstate outside the limits below,
                                unknown dtype, or dt_limit with dt_min > dt_max  */
    SSD_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                 */
    SSD_ERR_WORKSPACE = 5,   /* workspace smaller than its *_workspace_size      */
    SSD_ERR_HIP = 6,         /* the HIP runtime reported an error at launch      */
    SSD_ERR_SCRATCH = 7      /* the call needs more than SSD_NOALLOC_SCRATCH_BYTES
                                of built-in scratch (ssd_scan_fwd_noalloc only)   */
} ssd_status;

typedef enum ssd_dtype { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

/* Shape of a prefill call.  batch >= 0, seqlen >= 0, nheads >= 1,
 * 1 <= ngroups, nheads % ngroups == 0.
 * chunk: 16, 32, 64, 128 or 256.  headdim: 1..256.  dstate: 4..256, a power of
 * two.  seqlen need not be a multiple of chunk (the last chunk is short). */
typedef struct ssd_scan_desc {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
    int32_t dtype; /* ssd_dtype */
    int32_t reserved; /* must be 0 */
} ssd_scan_desc;

/* Shape of a variable-length (ragged) prefill: nseq sequences packed back to
 * back along one token axis of `total` tokens.  nseq >= 0, total >= 0, both
 * below 2^31 - 512; other fields as in ssd_scan_desc. */
typedef struct ssd_varlen_desc {
    int64_t nseq, total, nheads, headdim, dstate, ngroups, chunk;
    int32_t dtype; /* ssd_dtype */
    int32_t reserved; /* must be 0 */
} ssd_varlen_desc;

/* Shape of a decode step: as above without seqlen and chunk. */
typedef struct ssd_step_desc {
    int64_t batch, nheads, headdim, dstate, ngroups;
    int32_t dtype; /* ssd_dtype */
    int32_t reserved; /* must be 0 */
} ssd_step_desc;

/* Static English text for a status code (never NULL). */
const char *ssd_status_string(int status);

/* ABI version of this header: 12. */
int ssd_abi_version(void);

/* ---------------------------------------------------------------- prefill */

/* Bytes of device workspace ssd_scan_fwd needs for shape *d (0 is possible). */
ssd_status ssd_scan_workspace_size(const ssd_scan_desc *d, size_t *bytes);

/* Chunked SSD scan over a whole sequence ("Compiler-First ...", §3,
 * "Chunked recurrence"; the contractions of B.5).
 *   x           [batch, seqlen, nheads, headdim]      dtype
 *   dt          [batch, seqlen, nheads]               fp32, final step sizes
 *                                                    (no bias/softplus applied here)
 *   A           [nheads]                              fp32
 *   B, C        [batch, seqlen, ngroups, dstate]      dtype
 *   D           [nheads] fp32, or NULL (no skip term)
 *   init_state  [batch, nheads, headdim, dstate] fp32, or NULL (zero state)
 *   y           [batch, seqlen, nheads, headdim]      dtype, written
 *   final_state [batch, nheads, headdim, dstate] fp32, or NULL (not written);
 *               may equal init_state (in-place continuation); no other aliasing.
 *   workspace   device buffer of at least ssd_scan_workspace_size bytes
 *               (may be NULL when that size is 0).  Its contents need no
 *               initialisation and are scratch after the call, except the
 *               error word described at ssd_scan_error_word.
 * seqlen == 0 writes final_state = init_state (or zeros); batch == 0 is a no-op.
 *
 * The chunked stages run as separate kernels.  On the matrix-core shapes
 * (bf16 x/B/C, headdim 64, dstate 64 or 128, chunk 64, 128 or 256) the pass
 * of the state between chunks ("a lightweight scan" of summary states, §3
 * "Chunked recurrence") runs either in a launch of its own or, when the
 * chunk-state grid spans at least four rounds of resident blocks, inside
 * the chunk-state launch: each (batch row, chunk, head) block then hands the
 * state entering the next chunk on to that chunk's block through the
 * workspace.  SSD_PREFILL_PATH=separate or =chained forces either.  For
 * chunk 256 with bf16 x/B/C, headdim 64 and dstate 64 or 128,
 * SSD_PREFILL_PATH=fused selects instead a single kernel for all stages
 * (after a small one that forms the C.B products shared by the heads of a
 * group), with the same hand-off.  The hand-off's waits between blocks are
 * bounded; see ssd_scan_error_word.  Every arrangement gives the operation's
 * result within the same tolerance; they differ in speed. */
ssd_status ssd_scan_fwd(const ssd_scan_desc *d, const void *x, const float *dt,
                        const float *A, const void *B, const void *C, const float *D,
                        const float *init_state, void *y, float *final_state,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device scratch built into the library for ssd_scan_fwd_noalloc:
 * 64 MiB on each device the library is loaded on (the 2.7B head shape at
 * 4096 tokens needs about 48 MB). */
#define SSD_NOALLOC_SCRATCH_BYTES (64u << 20)

/* ssd_scan_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the workspace ssd_scan_workspace_size
 * reports for *d is taken from SSD_NOALLOC_SCRATCH_BYTES of scratch that the
 * library holds on each device (a static device array, not an allocation).
 * The call allocates nothing and frees nothing; its results are those of
 * ssd_scan_fwd on the same arguments.  A shape that needs more than the
 * scratch holds returns SSD_ERR_SCRATCH before anything is enqueued.  Every
 * call on one device shares that device's scratch: two calls that may
 * overlap on one device (different streams, or threads) race and must not be
 * made.  The first call on a device looks up the scratch's device address
 * (hipGetSymbolAddress); a failure there returns SSD_ERR_HIP.  A call that
 * takes the chained state pass (see ssd_scan_fwd) keeps its error word in
 * the scratch too, where the caller cannot read it; a caller that must check
 * it uses ssd_scan_fwd with a workspace, or SSD_PREFILL_PATH=separate. */
ssd_status ssd_scan_fwd_noalloc(const ssd_scan_desc *d, const void *x, const float *dt,
                                const float *A, const void *B, const void *C, const float *D,
                                const float *init_state, void *y, float *final_state,
                                void *stream);

/* Byte offset, within the workspace of an ssd_scan_fwd(_ex) call of shape *d,
 * of a 32-bit error word that the call sets to 0 before its hand-off kernel
 * runs and to a nonzero value if one of that kernel's bounded waits for the
 * state of an earlier chunk ran out (the results of such a call are not
 * valid).  The caller may read it after the call completes.
 * SSD_ERR_UNSUPPORTED when the call of shape *d hands no state between
 * blocks (the separate state pass, or an empty call: there is no such wait
 * then); the answer follows SSD_PREFILL_PATH and the shape as ssd_scan_fwd
 * reads them. */
ssd_status ssd_scan_error_word(const ssd_scan_desc *d, size_t *offset);

/* ---------------------------------------------------------------- gradient */

typedef struct ssd_edges ssd_edges; /* the fused edges, defined below */

/* Bytes of device workspace ssd_scan_bwd needs for shape *d. */
ssd_status ssd_scan_bwd_workspace_size(const ssd_scan_desc *d, size_t *bytes);

/* Gradient of ssd_scan_fwd, for training ("Compiler-First ...", B.5 times
 * forward plus backward): for the scalar
 *     J = sum(dy * y) + sum(dfinal * final_state)
 * (dy and dfinal the derivatives arriving from above), the derivatives of J
 * with respect to every input of the forward call.  Inputs are the forward
 * call's (same layouts; the forward outputs are not needed: the chunk states
 * are recomputed) plus
 *   dy      [batch, seqlen, nheads, headdim]  dtype
 *   dfinal  [batch, nheads, headdim, dstate]  fp32, or NULL (no final-state term)
 * Outputs (all overwritten):
 *   dx      [batch, seqlen, nheads, headdim]  dtype
 *   ddt     [batch, seqlen, nheads]           fp32
 *   dA      [nheads]                          fp32
 *   dB, dC  [batch, seqlen, ngroups, dstate]  fp32 (summed over the heads of a group)
 *   dD      [nheads] fp32, or NULL (not computed)
 *   dinit   [batch, nheads, headdim, dstate]  fp32, or NULL (not computed)
 * dt is the activated step size (the edges of ssd_scan_fwd_ex are not
 * differentiated here).  The kernels choose their own chunking whatever
 * d->chunk is (64 tokens for bf16 with headdim 64 and dstate 64 or 128, else
 * 32); like the forward, the result does not depend on the chunk beyond
 * rounding.
 * dB, dC, dA and dD are accumulated with floating-point atomics, so their
 * last bits may differ between runs.  seqlen == 0 or batch == 0: dA = dD = 0
 * and dinit = dfinal (or 0). */
ssd_status ssd_scan_bwd(const ssd_scan_desc *d, const void *x, const float *dt, const float *A,
                        const void *B, const void *C, const float *D, const float *init_state,
                        const void *dy, const float *dfinal, void *dx, float *ddt, float *dA,
                        float *dB, float *dC, float *dD, float *dinit, void *workspace,
                        size_t workspace_bytes, void *stream);

/* The gradient of ssd_scan_fwd_ex: the same J with y the edged output, with
 * respect to every input of that call.  dt is the raw step size and ddt its
 * gradient: the scan's step-size gradient times the activation's derivative
 * (sigmoid(dt + bias) under softplus, 1 without, 0 where the clamp holds the
 * value at a bound it was pushed past).  Further outputs:
 *   dz        [batch, seqlen, nheads, headdim] dtype: the gate's gradient
 *             dy * y * silu'(z), y the ungated output; required when
 *             edges->z is set, else ignored
 *   ddt_bias  [nheads] fp32, or NULL: the gradient of dt_bias, ddt summed
 *             over batch and tokens in a fixed order
 *   dnorm_weight [nheads * headdim] fp32, or NULL: the gradient of the gated
 *             RMSNorm's weight (edges->norm_weight set), summed over tokens
 *             in a fixed order; the norm's gradient also flows into dz and
 *             everything before it.  It needs headdim a multiple of 8 and
 *             norm groups of at most 8192 channels (SSD_ERR_UNSUPPORTED
 *             otherwise).
 * The ungated output comes from the chunk-output stage run on the entering
 * states the gradient forms anyway (no second forward pass).
 * edges == NULL is ssd_scan_bwd.  Workspace: ssd_scan_bwd_ex_workspace_size
 * bytes for the same edges. */
ssd_status ssd_scan_bwd_ex_workspace_size(const ssd_scan_desc *d, const ssd_edges *edges,
                                          size_t *bytes);
ssd_status ssd_scan_bwd_ex(const ssd_scan_desc *d, const ssd_edges *edges, const void *x,
                           const float *dt, const float *A, const void *B, const void *C,
                           const float *D, const float *init_state, const void *dy,
                           const float *dfinal, void *dx, float *ddt, float *dA, float *dB,
                           float *dC, float *dD, float *dinit, void *dz, float *ddt_bias,
                           float *dnorm_weight, void *workspace, size_t workspace_bytes,
                           void *stream);

/* ------------------------------------------------------- fused scan edges */

/* The elementwise steps that surround the scan in a Mamba block, fused into
 * the scan's own kernels (the pyshine "Mamba" repository tour, "Why You Need
 * This": the block feeds the scan softplus(dt + dt_bias), with the bias set so
 * that the result starts between dt_min and dt_max, and the scan kernels
 * optionally gate their output with z).
 *   dt_bias     [nheads] fp32, added to every dt before the activation, or NULL
 *   dt_softplus 1: dt <- softplus(dt + bias) = log(1 + exp(dt + bias));
 *               0: dt <- dt + bias
 *   dt_limit    1: the activated dt is then clamped to [dt_min, dt_max]
 *               (dt_min <= dt_max required); 0: no clamp
 *   z           gate with the layout and dtype of x, or NULL: every output is
 *               multiplied by silu(z) = z / (1 + exp(-z)) in fp32 before its
 *               single rounding to the output dtype
 *   norm_weight [nheads * headdim] fp32, or NULL (no norm): the gated
 *               RMSNorm that the same tour's Mamba2 block applies to the scan
 *               output (its layernorm_gated module).  Each token's channels
 *               (head-major, headdim inner) split into norm_groups groups of
 *               whole heads; within a group, after the gate,
 *                   out = v / sqrt(mean(v^2) + norm_eps) * norm_weight
 *               computed in fp32 from the stored gated output (one more
 *               rounding to the output dtype).  It runs as a separate pass
 *               over y after the scan, since a group spans heads that the scan
 *               kernels write in different blocks.
 *   norm_eps    >= 0 (with 0, an all-zero group gives NaN)
 *   norm_groups groups per token, dividing nheads; 0 means ngroups (the B/C
 *               groups: the heads that share B and C share a norm)
 * The step size the recurrence uses is the activated dt, everywhere dt enters
 * (decay and input weight).  A NULL ssd_edges pointer, or one with every field
 * zero / NULL, is the plain operation. */
struct ssd_edges {
    const float *dt_bias;
    const void *z;
    float dt_min, dt_max;
    int32_t dt_softplus;
    int32_t dt_limit;
    const float *norm_weight;
    float norm_eps;
    int32_t norm_groups;
};

/* ssd_scan_fwd with the edges above (edges may be NULL).  dt here is the raw
 * pre-activation value; the first kernel to read it writes the activated dt
 * into the workspace for the later ones.  Workspace as for ssd_scan_fwd. */
ssd_status ssd_scan_fwd_ex(const ssd_scan_desc *d, const ssd_edges *edges, const void *x,
                           const float *dt, const float *A, const void *B, const void *C,
                           const float *D, const float *init_state, void *y,
                           float *final_state, void *workspace, size_t workspace_bytes,
                           void *stream);

/* ------------------------------------------------ variable-length prefill */

/* Bytes of device workspace ssd_scan_fwd_varlen needs for shape *d. */
ssd_status ssd_varlen_workspace_size(const ssd_varlen_desc *d, size_t *bytes);

/* A ragged batch in one call, for serving requests of different lengths
 * together ("Bringing blazing fast state space models to the Modular MAX
 * framework", "What We Built": variable-length selective-scan kernels for
 * batched serving; the pyshine "Mamba" repository tour: the CUDA core's
 * variable-length strands): sequence s covers tokens
 * [cu_seqlens[s], cu_seqlens[s+1]) of the packed arrays, starts from its own
 * init state, ends in its own final state, and never sees another
 * sequence's tokens.  The result for each sequence is that of ssd_scan_fwd_ex
 * on it alone (batch 1, same chunk size): each sequence is cut into chunks
 * from its own first token, its last chunk may be short, and an empty
 * sequence passes its init state through.
 *   cu_seqlens   [nseq + 1] int32, device: 0 = cu[0] <= cu[1] <= ... <=
 *                cu[nseq] = total.  Offsets outside that contract give
 *                unspecified results but no access outside the arrays below
 *                (they are clamped into [0, total] on the device).
 *   x, y         [total, nheads, headdim]     dtype
 *   dt           [total, nheads]              fp32 (raw when edges activate it)
 *   B, C         [total, ngroups, dstate]     dtype
 *   A, D         [nheads] fp32 (D may be NULL)
 *   init_states  [nseq, nheads, headdim, dstate] fp32, or NULL (zero states)
 *   final_states [nseq, nheads, headdim, dstate] fp32, or NULL; may equal
 *                init_states
 *   edges        as for ssd_scan_fwd_ex, or NULL (z in x's layout)
 *   workspace    at least ssd_varlen_workspace_size bytes.
 * nseq == 0 is a no-op; total == 0 writes final = init for every sequence.
 * The chunk table is built on the device from cu_seqlens, so the call needs
 * no host copy of the lengths and can be captured in a HIP graph.  Shapes of
 * the single-kernel path of ssd_scan_fwd take it here too, with one
 * hand-off chain per (sequence, head). */
ssd_status ssd_scan_fwd_varlen(const ssd_varlen_desc *d, const ssd_edges *edges,
                               const int32_t *cu_seqlens, const void *x, const float *dt,
                               const float *A, const void *B, const void *C, const float *D,
                               const float *init_states, void *y, float *final_states,
                               void *workspace, size_t workspace_bytes, void *stream);

/* As ssd_scan_error_word, for ssd_scan_fwd_varlen of shape *d. */
ssd_status ssd_varlen_error_word(const ssd_varlen_desc *d, size_t *offset);

/* The gradient of ssd_scan_fwd_varlen (its edges as for ssd_scan_bwd_ex):
 * every sequence's gradient on its own tokens, as ssd_scan_bwd_ex would give
 * for it alone (batch 1), with the sequences' layouts of
 * ssd_scan_fwd_varlen.
 *   dy             [total, nheads, headdim]                 dtype
 *   dfinal_states  [nseq, nheads, headdim, dstate] fp32, or NULL
 *   dx, ddt, dB, dC, dz   per packed token (layouts of x, dt, B, C, x)
 *   dA, dD, ddt_bias, dnorm_weight   summed over all sequences
 *   dinit_states   [nseq, nheads, headdim, dstate] fp32, or NULL; an empty
 *                  sequence gets its dfinal (or zeros)
 *   workspace      ssd_scan_bwd_varlen_workspace_size bytes for the same
 *                  edges.
 * The gradient cuts each sequence into chunks of its own size from its first
 * token (64 or 32 tokens, as for ssd_scan_bwd_ex), with a chunk table built
 * on the device: no host copy of the lengths, graph-capturable. */
ssd_status ssd_scan_bwd_varlen_workspace_size(const ssd_varlen_desc *d, const ssd_edges *edges,
                                              size_t *bytes);
ssd_status ssd_scan_bwd_varlen(const ssd_varlen_desc *d, const ssd_edges *edges,
                               const int32_t *cu_seqlens, const void *x, const float *dt,
                               const float *A, const void *B, const void *C, const float *D,
                               const float *init_states, const void *dy,
                               const float *dfinal_states, void *dx, float *ddt, float *dA,
                               float *dB, float *dC, float *dD, float *dinit_states, void *dz,
                               float *ddt_bias, float *dnorm_weight, void *workspace,
                               size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------- decode step */

/* One cached decode token ("Compiler-First ...", §3 "Autoregressive cache"):
 *   state [batch, nheads, headdim, dstate] fp32, read and updated in place
 *   x     [batch, nheads, headdim]  dtype      dt [batch, nheads] fp32
 *   A     [nheads] fp32             B, C [batch, ngroups, dstate] dtype
 *   D     [nheads] fp32 or NULL     y [batch, nheads, headdim] dtype, written
 * y uses the state after this token's update. */
ssd_status ssd_step(const ssd_step_desc *d, float *state, const void *x, const float *dt,
                    const float *A, const void *B, const void *C, const float *D, void *y,
                    void *stream);

/* nsteps consecutive decode tokens in one launch, for inputs that are all
 * known up front (a short continuation of a cached sequence, draft tokens to
 * verify): the same result as nsteps calls of ssd_step on the same stream,
 * bit for bit, but the state is read and written once instead of once per
 * token ("Compiler-First ...", §3 "Autoregressive cache", with the loop
 * over tokens kept on the device).  Inputs use the prefill layout:
 *   state [batch, nheads, headdim, dstate] fp32, read and updated in place
 *   x     [batch, nsteps, nheads, headdim]  dtype
 *   dt    [batch, nsteps, nheads]           fp32
 *   A     [nheads] fp32                     D [nheads] fp32 or NULL
 *   B, C  [batch, nsteps, ngroups, dstate]  dtype
 *   y     [batch, nsteps, nheads, headdim]  dtype, written
 * nsteps == 0 and batch == 0 are no-ops; nsteps < 0 is SSD_ERR_SHAPE. */
ssd_status ssd_step_multi(const ssd_step_desc *d, int64_t nsteps, float *state, const void *x,
                          const float *dt, const float *A, const void *B, const void *C,
                          const float *D, void *y, void *stream);

/* ssd_step and ssd_step_multi with the fused edges (edges may be NULL); z has
 * the layout of x.  ssd_step_multi_ex equals nsteps calls of ssd_step_ex bit
 * for bit, as without edges. */
ssd_status ssd_step_ex(const ssd_step_desc *d, const ssd_edges *edges, float *state,
                       const void *x, const float *dt, const float *A, const void *B,
                       const void *C, const float *D, void *y, void *stream);
ssd_status ssd_step_multi_ex(const ssd_step_desc *d, const ssd_edges *edges, int64_t nsteps,
                             float *state, const void *x, const float *dt, const float *A,
                             const void *B, const void *C, const float *D, void *y,
                             void *stream);

/* ------------------------------------------------- stages of the prefill scan
 * The four steps of ssd_scan_fwd, callable one at a time for stage checks.
 * Shapes as for ssd_scan_fwd; T = ceil(seqlen / chunk); chunk c covers tokens
 * [c*chunk, min(seqlen, (c+1)*chunk)).  Intermediate layouts:
 *   Acs    [batch, nheads, seqlen] fp32   within-chunk inclusive cumsum of dt*A
 *   states [batch, T, nheads, headdim, dstate] fp32
 */

/* Acs[b,h,t] = sum over tokens k of t's chunk with k <= t of dt[b,k,h]*A[h]. */
ssd_status ssd_chunk_cumsum(const ssd_scan_desc *d, const float *dt, const float *A,
                            float *Acs, void *stream);

/* states[b,c,h,p,n] = sum_{j in chunk c} x[b,j,h,p] * dt[b,j,h]
 *                       * exp(Acs[b,h,last(c)] - Acs[b,h,j]) * B[b,j,g,n]
 * (the state chunk c alone contributes, starting from zero). */
ssd_status ssd_chunk_state(const ssd_scan_desc *d, const void *x, const void *B,
                           const float *dt, const float *Acs, float *states, void *stream);

/* In place over chunks, per (b,h): H_0 = init_state (or 0);
 *   H_{c+1} = exp(Acs[b,h,last(c)]) * H_c + states[c];  states[c] <- H_c.
 * On return states[c] holds the state ENTERING chunk c and final_state (if not
 * NULL) holds H_T.  final_state may equal init_state. */
ssd_status ssd_state_passing(const ssd_scan_desc *d, float *states, const float *Acs,
                             const float *init_state, float *final_state, void *stream);

/* Bytes of device workspace that ssd_chunk_cb fills and ssd_chunk_scan reads
 * for shape *d (0 is possible: then both ignore the workspace). */
ssd_status ssd_chunk_scan_workspace_size(const ssd_scan_desc *d, size_t *bytes);

/* The within-chunk products CB[i][j] = C_i . B_j (j <= i, same chunk and
 * group).  They do not involve the head, so they are formed once per
 * (batch, chunk, group) and shared by the nheads/ngroups heads of the group
 * ("Compiler-First ...", §3, "Primitive-level implementation" and the
 * intra-chunk contraction of B.5).  The workspace layout is internal to the
 * library; it is written here and read by ssd_chunk_scan for the same d, B
 * and C.  workspace: at least ssd_chunk_scan_workspace_size bytes (may be NULL
 * when that size is 0, in which case nothing is launched). */
ssd_status ssd_chunk_cb(const ssd_scan_desc *d, const void *B, const void *C, void *workspace,
                        size_t workspace_bytes, void *stream);

/* y for every chunk from the chunk-entry states:
 *   y[t] = sum_{j <= t in chunk} (C_t . B_j) exp(Acs_t - Acs_j) dt_j x_j
 *          + exp(Acs_t) (C_t . H_c) + D x_t
 * with H_c = states[c] as left by ssd_state_passing and C_t . B_j as left in
 * the workspace by ssd_chunk_cb ("Compiler-First ...", §3, the intra-chunk
 * output contraction of B.5).  workspace: the buffer ssd_chunk_cb filled for
 * the same d, B and C (may be NULL when ssd_chunk_scan_workspace_size is 0);
 * it must not overlap any other argument. */
ssd_status ssd_chunk_scan(const ssd_scan_desc *d, const void *x, const float *dt,
                          const void *B, const void *C, const float *D, const float *Acs,
                          const float *states, void *y, const void *workspace,
                          size_t workspace_bytes, void *stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* SSD_H */
