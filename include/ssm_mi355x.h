/*
 * ssm_mi355x.h -- C ABI of the MI355X (gfx950) selective state-space scan library.
 *
 * The library computes the core of Mamba's selective SSM layer (S6) and its
 * Mamba-2 SSD form.  Sources, cited by page title and section:
 *   [guide]  "Mamba / State Space Models complete guide" (youngju.dev),
 *            sec. 2 (continuous SSM, ZOH discretization, convolution kernel),
 *            sec. 5 (selective scan listing, Mamba block), sec. 6 (Mamba 2).
 *   [expl]   "Paper explainer: Mamba (2312.00752)" (0h-n0.github.io),
 *            "Technical details": ZOH, selection mechanism, hardware-aware scan.
 *   [ssm]    "SSM & Mamba" (disassemble-channel.com): "Discretization / ZOH",
 *            "Equivalence with convolution", "Mamba: selective SSM".
 *   [ssd]    "Mamba-2 / Structured State Space Duality" (abeam guide):
 *            "Basic idea", "Linear and quadratic forms", block design.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensors are dense, contiguous, row-major, in the order written next
 *    to each argument.  Every pointer is a DEVICE pointer on the current HIP
 *    device, aligned to its element size.  The caller owns every buffer; the
 *    library keeps no pointer after the call returns and never frees one.
 *  - "act" tensors (x, B, C, z, y) use the dtype `act_dtype`; dt/delta uses
 *    `delta_dtype`.  A, Dskip, biases, h0 and h_final are always fp32.  The
 *    recurrent state is always fp32.  bf16 outputs are rounded to nearest even.
 *  - Optional pointers may be NULL (stated per argument).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    null stream).  Results are valid once the stream has synchronised.
 *  - Argument errors are detected on the host before anything is enqueued
 *    and reported through the return value (an ssm_status); nothing is
 *    launched then.  A HIP runtime failure returns SSM_ERR_HIP.  A message
 *    with detail for the last failure of the calling thread is available from
 *    ssm_last_error().
 *  - Outputs must not alias inputs, except that h_final may equal h0 (the
 *    state is read before it is overwritten, which gives an in-place
 *    single-token decode step when seqlen == 1).
 *  - workspace: device scratch of at least the size the matching
 *    *_workspace_bytes() query returns for the same shapes, or NULL, in which
 *    case the library takes stream-ordered memory (hipMallocAsync) for the
 *    duration of the call.  Calls that share a workspace must be ordered on
 *    one stream.
 */
#ifndef SSM_MI355X_H
#define SSM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types of act / delta tensors */
enum ssm_dtype { SSM_F32 = 0, SSM_BF16 = 1 };

/* return codes */
enum ssm_status {
  SSM_OK = 0,
  SSM_ERR_NULL = 1,         /* a required pointer is NULL */
  SSM_ERR_SHAPE = 2,        /* a size is negative, inconsistent or overflows 64-bit indexing */
  SSM_ERR_DTYPE = 3,        /* unknown dtype code */
  SSM_ERR_UNSUPPORTED = 4,  /* valid but not implemented here (e.g. scan dstate > 256) */
  SSM_ERR_WORKSPACE = 5,    /* workspace given but smaller than required */
  SSM_ERR_HIP = 6,          /* a HIP runtime call failed (see ssm_last_error) */
  SSM_ERR_ALIGNMENT = 7     /* a pointer is not aligned to its element size */
};

/*
 * Selective scan forward (S6).  For every batch b and channel d, with state
 * h (dstate entries, fp32) starting at h0[b,d,:] (zeros if h0 == NULL):
 *
 *   v    = delta[b,t,d] + (delta_bias ? delta_bias[d] : 0)
 *   dt   = delta_softplus ? log(1 + e^v) : v              ([expl] selection mechanism)
 *   h_n  = exp(dt*A[d,n]) * h_n + (exp(dt*A[d,n]) - 1)/A[d,n] * B[b,t,n] * x[b,t,d]
 *                                                         ([ssm] ZOH for diagonal A;
 *                                                          the gain is dt when A[d,n] == 0)
 *   y[b,t,d] = (sum_n C[b,t,n]*h_n + Dskip[d]*x[b,t,d]) * silu(z[b,t,d])
 *                                                         ([guide] sec. 5: skip, then gate)
 * for t = 0..seqlen-1, so y at token t includes token t's own input
 * ([guide] sec. 2: y[0] = C Bbar u[0]).  h_final[b,d,:] = state after the
 * last token.
 *
 *   x, delta, z, y : (batch, seqlen, dim)      act / delta / act / act dtype
 *   A              : (dim, dstate) fp32        real diagonal entries (normally < 0)
 *   B, C           : (batch, seqlen, dstate)   act dtype, shared by all channels
 *   Dskip          : (dim) fp32 or NULL (no skip term)
 *   z              : NULL for no gate
 *   delta_bias     : (dim) fp32 or NULL
 *   delta_softplus : 0 or 1
 *   h0             : (batch, dim, dstate) fp32 or NULL (zeros)
 *   y              : required output
 *   h_final        : (batch, dim, dstate) fp32 output or NULL
 *   dstate         : 1..256 (129..256 run 8 rows of 32 states per wave)
 * Long sequences with few (batch, channel) slices need time parallelism.
 * With 16 states, whole groups of 8 channels, 16-byte aligned x, delta, z, y,
 * B and C, and at least one such group per compute unit, the lanes of a wave
 * split the time axis and combine their partial states in registers (one
 * pass, no workspace).  Otherwise the sequence is split into time chunks whose
 * states are computed in a first pass and combined on the device (workspace).
 */
int ssm_scan_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                 const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                 const float* h0, void* y, float* h_final,
                 int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                 int act_dtype, int delta_dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * ssm_scan_fwd that allocates nothing, for callers that cannot allocate
 * device memory while they run: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Arguments, layouts, ownership and
 * errors are those of ssm_scan_fwd without the workspace: the caller still
 * passes every input and output, and the time-split chunk states live in a
 * fixed device array of ssm_scan_fwd_noalloc_max_workspace_bytes() bytes
 * (32 MiB) that the library holds on each GPU it runs on until the process
 * ends.  Shapes whose workspace (ssm_scan_workspace_bytes()) exceeds it
 * return SSM_ERR_WORKSPACE before anything is enqueued.  The call makes no
 * hipMalloc, hipFree or other allocating call (its first call on a device
 * looks the array's address up once).  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller; calls on one stream are
 * ordered by the stream.  Nothing in the array needs to start at zero.
 */
int ssm_scan_fwd_noalloc(const void* x, const void* delta, const float* A, const void* B, const void* C,
                         const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                         const float* h0, void* y, float* h_final,
                         int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                         int act_dtype, int delta_dtype, void* stream);

/* Size of ssm_scan_fwd_noalloc's fixed per-GPU workspace in bytes. */
size_t ssm_scan_fwd_noalloc_max_workspace_bytes(void);

/* flag bits of ssm_scan_fwd_ex */
enum ssm_scan_flag {
  SSM_SCAN_REVERSE = 1,         /* run the recurrence from the last token to the first */
  SSM_SCAN_EULER = 2,           /* Euler input discretization: gain dt instead of ZOH */
  SSM_SCAN_DELTA_PER_TOKEN = 4  /* delta is (batch, seqlen): one dt per token for all channels */
};

/*
 * Variants of ssm_scan_fwd selected by flags (any combination; 0 is
 * ssm_scan_fwd itself).  Arguments, layouts, ownership and errors are those
 * of ssm_scan_fwd, plus:
 *   SSM_SCAN_REVERSE : the scan of the time-reversed sequence, i.e.
 *       flip_t(scan(flip_t(inputs))) with flip_t reversing the token axis of
 *       x, delta, B, C and z.  y[b,t,d] then depends on tokens t..seqlen-1,
 *       h0 is the state entering at token seqlen-1 and h_final the state
 *       after token 0.  This is the backward branch of a bidirectional or
 *       multi-direction scan ([guide] sec. 9, VMamba: an image's patch sequence
 *       scanned in four orders, each a flip or transpose of the same S6
 *       scan); layouts stay in natural token order, nothing is copied.
 *   SSM_SCAN_EULER : Bbar = dt * B, i.e. h_n = exp(dt*A[d,n]) h_n +
 *       dt * B[b,t,n] * x[b,t,d], the simplified discretization of the
 *       code listings ([guide] sec. 5 naive selective scan; [ssm] the numpy
 *       selective SSM implementation) in place of exact ZOH.
 *   SSM_SCAN_DELTA_PER_TOKEN : delta holds batch * seqlen values (row-major
 *       (batch, seqlen), delta dtype); every channel of token t reads
 *       delta[b,t] (plus its own delta_bias[d] when given), as in [ssm]'s numpy
 *       selective SSM, which projects one step size per token.
 * Unknown bits return SSM_ERR_UNSUPPORTED.
 */
int ssm_scan_fwd_ex(const void* x, const void* delta, const float* A, const void* B, const void* C,
                    const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                    const float* h0, void* y, float* h_final,
                    int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                    int act_dtype, int delta_dtype, int flags,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Training forward: ssm_scan_fwd_ex (same arguments, layouts, ownership,
 * flags and errors) that also writes the recurrent state entering every 16th
 * token, for ssm_scan_bwd_train.  [expl] "hardware-aware scan": the states
 * are not kept per token; the backward pass recomputes them inside each
 * 16-token tile from the state stored at the tile's start, so only one
 * state in 16 leaves the chip.
 *   states : fp32, (ceil(seqlen / 16), batch, dim, dstate), required when
 *            batch, seqlen and dim are all > 0.  states[k, b, d, n] is the
 *            state h[b, d, n] before the token at position 16k in processing
 *            order (token 16k forward, token seqlen-1-16k with
 *            SSM_SCAN_REVERSE); states[0] is h0 (zeros without h0).  Size:
 *            ssm_scan_train_states_bytes().  Every element is written.
 * Workspace: ssm_scan_workspace_bytes() for the same shapes, or NULL.
 */
int ssm_scan_fwd_train(const void* x, const void* delta, const float* A, const void* B, const void* C,
                       const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                       const float* h0, void* y, float* h_final,
                       int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                       int act_dtype, int delta_dtype, int flags, float* states,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of ssm_scan_fwd_train's states: ceil(seqlen/16) * batch * dim *
 * dstate * 4.  0 for empty or unsupported sizes (dstate > 256). */
size_t ssm_scan_train_states_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

/*
 * Final state only: the same recurrence as ssm_scan_fwd, writing h_final
 * (required) and no y; C, Dskip and z are not needed.  ([guide] sec. 2/4:
 * recurrent inference keeps only the fixed-size state.)
 */
int ssm_scan_final_state(const void* x, const void* delta, const float* A, const void* B,
                         const float* delta_bias, int delta_softplus, const float* h0,
                         float* h_final,
                         int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                         int act_dtype, int delta_dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Workspace enough for ssm_scan_fwd / ssm_scan_final_state (and their
 * variants) on these shapes: 0 when no time split is planned.  It does not
 * depend on dtypes, flags or alignment, so it is an upper bound: a call whose
 * arguments take the one-pass long-sequence kernel needs none.  Depends on
 * the current device. */
size_t ssm_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

/*
 * Mamba-2 SSD forward ([ssd] "Basic idea" and "Linear and quadratic forms";
 * [guide] sec. 6: one scalar A per head, dt per head, B/C of width dstate
 * shared by the heads of a group).  For batch b, head h (group
 * g = h / (nheads/ngroups)), head channel p and state n, with state
 * S[p][n] starting at h0[b,h,p,n] (zeros if NULL):
 *
 *   dt      = softplus?(dt[b,t,h] + dt_bias[h])
 *   S[p][n] = exp(dt*A[h]) S[p][n] + (exp(dt*A[h]) - 1)/A[h] * B[b,t,g,n] * x[b,t,h,p]
 *   y[b,t,h,p] = (sum_n C[b,t,g,n] S[p][n] + Dskip[h] x[b,t,h,p]) * silu(z[b,t,h,p])
 *
 * With bf16 activations, headdim 64 or 128 and dstate 64 or 128 it is
 * computed blockwise ([ssd] block decomposition): within a block of 64
 * tokens as a causal, decayed matrix product on the matrix cores, across
 * blocks by passing the state.  The block is 64 tokens whatever `chunk_size`
 * is: any block length gives the same map (the state entering a block is the
 * decayed sum of everything before it), so `chunk_size` (64, 128 or 256, the
 * chunk lengths of the pages' chunked form) is validated and otherwise does
 * not change the computation; results are identical for every accepted value.
 * Every other call (fp32 activations, or other head or state sizes) runs the
 * same map as its recurrence over tokens ([ssd] the SSM side of the duality),
 * one token after another per (batch, head), with no workspace: slower on
 * long sequences with few heads, and exact to fp32 rounding.
 *
 *   x, z, y : (batch, seqlen, nheads, headdim)  act dtype (z NULL for no gate)
 *   dt      : (batch, seqlen, nheads)           delta dtype
 *   A       : (nheads) fp32, must be finite
 *   B, C    : (batch, seqlen, ngroups, dstate)  act dtype
 *   Dskip, dt_bias : (nheads) fp32 or NULL
 *   h0, h_final    : (batch, nheads, headdim, dstate) fp32 or NULL
 * Supported: act_dtype SSM_F32 or SSM_BF16, any headdim, dstate 1 .. 256,
 * chunk_size in {64, 128, 256}, nheads % ngroups == 0.  dstate above 256
 * returns SSM_ERR_UNSUPPORTED.
 */
int ssd_chunk_scan_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                       const float* Dskip, const void* z, const float* dt_bias, int dt_softplus,
                       const float* h0, void* y, float* h_final,
                       int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t ngroups, int64_t dstate, int64_t chunk_size,
                       int act_dtype, int dt_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Workspace needed by ssd_chunk_scan_fwd for these shapes: for the blocked
 * form (headdim 64 or 128, dstate 64 or 128), the C_t . B_s products of every
 * 64-token block and group (10 causal 16x16 fp32 tiles, formed once and
 * shared by the group's heads), plus, when the (batch, head) pairs are too
 * few to fill the device and the sequence is split into time chunks, the
 * chunk states carried on the device; zero for other shapes and for seqlen 0.
 * It does not depend on the dtypes, so it is an upper bound: fp32
 * activations need none.  chunk_size does not change it.  Depends on the
 * current device. */
size_t ssd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                           int64_t ngroups, int64_t dstate, int64_t chunk_size);

/*
 * Single-token state update (recurrent inference, [guide] sec. 2 recurrent
 * view and sec. 4 inference; [ssd] inference: the past lives in a fixed-size
 * state).  Advances every (batch, channel) state by one token, in place, and
 * writes that token's output:
 *
 *   dt  = softplus?(delta[b,d] + delta_bias[d])
 *   state[b,d,n] = exp(dt*A[d,n]) state[b,d,n] + (exp(dt*A[d,n]) - 1)/A[d,n] * B[b,n] * x[b,d]
 *   y[b,d]  = (sum_n C[b,n] state[b,d,n] + Dskip[d] x[b,d]) * silu(z[b,d])
 *
 * i.e. ssm_scan_fwd with seqlen == 1 and h_final == h0 == state.
 *
 *   x, delta, z, y : (batch, dim)          act / delta / act / act dtype
 *   A              : (dim, dstate) fp32
 *   B, C           : (batch, dstate)       act dtype
 *   Dskip, delta_bias : (dim) fp32 or NULL; z NULL for no gate
 *   state          : (batch, dim, dstate) fp32, read and overwritten (required)
 *   y              : required output; must not alias state
 *   dstate         : 1..256
 * No workspace.  Enqueued on `stream`.
 */
int ssm_state_update(const void* x, const void* delta, const float* A, const void* B, const void* C,
                     const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                     float* state, void* y,
                     int64_t batch, int64_t dim, int64_t dstate,
                     int act_dtype, int delta_dtype, void* stream);

/*
 * Mamba-2 single-token state update ([ssd] inference; the recurrent form of
 * ssd_chunk_scan_fwd).  For head h (group g = h / (nheads/ngroups)) and head
 * channel p:
 *
 *   dt  = softplus?(dt[b,h] + dt_bias[h])
 *   state[b,h,p,n] = exp(dt*A[h]) state[b,h,p,n] + (exp(dt*A[h]) - 1)/A[h] * B[b,g,n] * x[b,h,p]
 *   y[b,h,p] = (sum_n C[b,g,n] state[b,h,p,n] + Dskip[h] x[b,h,p]) * silu(z[b,h,p])
 *
 *   x, z, y : (batch, nheads, headdim)   act dtype (z NULL for no gate)
 *   dt      : (batch, nheads)            dt dtype
 *   A       : (nheads) fp32
 *   B, C    : (batch, ngroups, dstate)   act dtype
 *   Dskip, dt_bias : (nheads) fp32 or NULL
 *   state   : (batch, nheads, headdim, dstate) fp32, read and overwritten (required)
 *   dstate 1..256, any headdim >= 1, nheads % ngroups == 0.  No workspace.
 */
int ssd_state_update(const void* x, const void* dt, const float* A, const void* B, const void* C,
                     const float* Dskip, const void* z, const float* dt_bias, int dt_softplus,
                     float* state, void* y,
                     int64_t batch, int64_t nheads, int64_t headdim, int64_t ngroups, int64_t dstate,
                     int act_dtype, int dt_dtype, void* stream);

/*
 * Causal depthwise 1-D convolution + SiLU, the step of the Mamba block that
 * produces the scan's input ([guide] sec. 5, the Mamba block: Conv1d with one
 * group per channel, padding width-1, output trimmed to seqlen, then silu):
 *
 *   out[b,t,d] = silu( bias[d] + sum_{k<width} weight[d,k] * xx[b, t-(width-1)+k, d] )
 *
 * where xx[b,i,d] = x[b,i,d] for i >= 0 and, for i < 0, the inputs carried in
 * from a previous segment, state_in[b, d, (width-1)+i] (oldest first; zeros
 * when state_in is NULL, i.e. the block's zero padding).  state_out receives
 * the last width-1 inputs of that extended sequence, so a later segment, or
 * a single decode token (seqlen 1), continues the same convolution.
 *
 *   x, out              : (batch, seqlen, dim)  act dtype; out must not overlap x
 *   weight              : (dim, width) fp32;  bias : (dim) fp32 or NULL
 *   state_in, state_out : (batch, dim, width-1) act dtype or NULL; state_out
 *                         may be the same buffer as state_in (in-place update)
 *   silu                : 1 applies silu, 0 returns the convolution alone
 *   width               : 1..8
 * No workspace.  Enqueued on `stream`.
 */
int ssm_causal_conv1d_fwd(const void* x, const float* weight, const float* bias, const void* state_in,
                          int silu, void* out, void* state_out,
                          int64_t batch, int64_t seqlen, int64_t dim, int64_t width,
                          int act_dtype, void* stream);

/*
 * Backward pass of ssm_scan_fwd (training).  Given dout = dloss/dy and
 * optionally dh_final = dloss/dh_final, computes the gradients of
 *   loss = sum dout * y + sum dh_final * h_final
 * with respect to every input of ssm_scan_fwd.  The pages give no backward
 * pass; this is the exact adjoint of the forward recurrence (reverse-time
 * scan of lam = dloss/dh with the same ZOH factors).
 *
 *   inputs as ssm_scan_fwd (x, delta, A, B, C, Dskip, z, delta_bias,
 *   delta_softplus, h0), plus
 *   dout        : (batch, seqlen, dim) act dtype (required)
 *   dh_final    : (batch, dim, dstate) fp32 or NULL (zeros)
 * outputs (all overwritten):
 *   dx          : (batch, seqlen, dim) act dtype (required)
 *   ddelta      : (batch, seqlen, dim) delta dtype (required): gradient with
 *                 respect to the delta input, through bias and softplus
 *   dA          : (dim, dstate) fp32 (required)
 *   dB, dC      : (batch, seqlen, dstate) fp32 (required; summed over channels)
 *   dDskip      : (dim) fp32, required when Dskip is given, else ignored
 *   dz          : (batch, seqlen, dim) act dtype, required when z is given
 *   ddelta_bias : (dim) fp32, required when delta_bias is given
 *   dh0         : (batch, dim, dstate) fp32 or NULL
 * dstate 1..256 (one pass over the sequence per 16 states).  dB and dC are
 * summed over channels in a fixed order (per
 * 16-channel group, then over the groups), so they are deterministic; the
 * sums over channels and batch of dA, and over batch of dDskip and
 * ddelta_bias, use fp32 atomics, so their last bits vary from run to run.
 * Workspace: ssm_scan_bwd_workspace_bytes() (the states of a block of 16 at
 * every 16-token tile start, the dB/dC partials of every 16-channel group,
 * and for dstate > 16 three fp32 accumulators of batch x seqlen x dim), or
 * NULL for stream-ordered scratch.
 */
int ssm_scan_bwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                 const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                 const float* h0, const void* dout, const float* dh_final,
                 void* dx, void* ddelta, float* dA, float* dB, float* dC, float* dDskip, void* dz,
                 float* ddelta_bias, float* dh0,
                 int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                 int act_dtype, int delta_dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass of ssm_scan_fwd_ex: the same arguments, layouts, ownership and
 * errors as ssm_scan_bwd, for the forward variant selected by `flags` (any
 * combination of SSM_SCAN_REVERSE, SSM_SCAN_EULER, SSM_SCAN_DELTA_PER_TOKEN;
 * 0 is ssm_scan_bwd).  With SSM_SCAN_REVERSE the gradients are those of the
 * reversed scan (h0 enters at the last token, dh_final applies to the state
 * after token 0); with SSM_SCAN_EULER those of the gain dt (dgain/ddt = 1, no
 * dependence on A).  With SSM_SCAN_DELTA_PER_TOKEN, delta and ddelta are
 * (batch, seqlen) in the delta dtype: one step size per token shared by every
 * channel, so ddelta is the per-channel gradient summed over the channels (in
 * a fixed order: deterministic); ddelta_bias stays per channel.  Workspace:
 * ssm_scan_bwd_ex_workspace_bytes() for these flags, or NULL.  Unknown bits
 * return SSM_ERR_UNSUPPORTED.
 */
int ssm_scan_bwd_ex(const void* x, const void* delta, const float* A, const void* B, const void* C,
                    const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                    const float* h0, const void* dout, const float* dh_final,
                    void* dx, void* ddelta, float* dA, float* dB, float* dC, float* dDskip, void* dz,
                    float* ddelta_bias, float* dh0,
                    int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                    int act_dtype, int delta_dtype, int flags,
                    void* workspace, size_t workspace_bytes, void* stream);

size_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

/* Workspace of ssm_scan_bwd_ex with these flags: ssm_scan_bwd's, plus, with
 * SSM_SCAN_DELTA_PER_TOKEN, an fp32 batch x seqlen x dim buffer of the
 * per-channel ddelta.  0 for unsupported sizes or flags. */
size_t ssm_scan_bwd_ex_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int flags);

/*
 * Training backward: ssm_scan_bwd_ex (same arguments, layouts, ownership,
 * flags and errors) taking the states that ssm_scan_fwd_train wrote for the
 * same inputs, h0 and flags, in place of its own forward pass over the
 * sequence (the pass that stores a state every 16 tokens).  The results
 * equal ssm_scan_bwd_ex's.  `states` is read only and required when batch,
 * seqlen and dim are all > 0; states from other inputs give meaningless
 * gradients (no check is possible).  Workspace:
 * ssm_scan_bwd_train_workspace_bytes() for these flags (ssm_scan_bwd_ex's
 * less the stored states), or NULL.
 */
int ssm_scan_bwd_train(const void* x, const void* delta, const float* A, const void* B, const void* C,
                       const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                       const float* h0, const void* dout, const float* dh_final,
                       void* dx, void* ddelta, float* dA, float* dB, float* dC, float* dDskip, void* dz,
                       float* ddelta_bias, float* dh0,
                       int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                       int act_dtype, int delta_dtype, int flags, const float* states,
                       void* workspace, size_t workspace_bytes, void* stream);

size_t ssm_scan_bwd_train_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int flags);

/* Static text for a status code (never NULL). */
const char* ssm_status_string(int status);

/* Detail for the calling thread's most recent failure ("" if none). */
const char* ssm_last_error(void);

/* SHA-256, as 64 lowercase hex digits, of the sources the library was built
 * from (every file of its csrc/ directory and every header of include/).  A
 * loader compares it with the sources beside the library and refuses a build
 * made from other sources.  Static storage; never NULL. */
const char* ssm_source_digest(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_MI355X_H */
