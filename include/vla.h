/*
 * vla.h -- C ABI of the MI355X (gfx950) Variational Linear Attention forward library.
 *
 * Method: "Variational Linear Attention: Stable Associative Memory for Long-Context
 * Transformers" (Pandey & Singh), as summarised on gist.science ("VLA summary" below).
 * For every independent (batch, head) stream and every token t the library computes
 *
 *   khat_t = k_t / ||k_t||                                    (VLA summary §2.1, §2.3)
 *   z_t    = A_{t-1} u_t
 *   A_t    = A_{t-1} - z_t z_t^T / (1 + u_t^T z_t)            (§2.3 step 1, Sherman-Morrison)
 *   ahat_t = A_t khat_t / ||A_t khat_t||                      (§2.3 step 2)
 *   S_t    = S_{t-1} + (v_t - S_{t-1} khat_t) ahat_t^T        (§2.3 step 3)
 *   n_t    = n_{t-1} + phi(k_t),  phi(x) = x + 1 (x > 0), e^x (x <= 0)   (ELU+1, §2.3)
 *   o_t    = S_t phi(q_t) / (n_t^T phi(q_t) + eps)            (ratio readout, §2.3)
 *
 * from the initial state A_0 = I / lambda0, S_0 = 0, n_0 = 0 (vla_forward) or a carried
 * state (vla_forward_state).  Readings of what the
 * pages leave open: z_t = A_{t-1} u_t with u_t a per-token input used as given; a zero
 * key gives khat = 0 and a zero A_t khat gives ahat = 0 (no memory write; A still
 * downdates).
 *
 * Arithmetic: inputs are widened exactly to fp32; state and accumulation are fp32; `out`
 * is rounded once (round to nearest even) to the input dtype.  Results are deterministic:
 * the same inputs, shape and path give bitwise-identical outputs (no atomics).
 */
#ifndef RLS_VLA_H
#define RLS_VLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t is `struct ihipStream_t *`; NULL means the default (null) stream. */
struct ihipStream_t;

typedef enum {
  VLA_SUCCESS = 0,
  VLA_ERROR_INVALID_VALUE = 1, /* NULL required pointer, size < 1, lambda0 <= 0 or not
                                  finite, eps < 0 or not finite, unknown dtype, path or
                                  gain, workspace smaller than vla_workspace_size(), an
                                  output overlapping an input, another output or the
                                  workspace                                             */
  VLA_ERROR_NOT_SUPPORTED = 2, /* d not in {32, 64, 96, 128}; a pointer not 16-byte
                                  aligned; a forced path, chunk or gain the shape
                                  cannot use                                            */
  VLA_ERROR_OUT_OF_MEMORY = 3, /* internal workspace allocation failed                */
  VLA_ERROR_LAUNCH = 4,        /* a HIP launch or runtime call failed                 */
  VLA_ERROR_NO_DEVICE = 5      /* no usable gfx950 device is current                  */
} vla_status_t;

typedef enum { VLA_DTYPE_F32 = 0, VLA_DTYPE_BF16 = 1 } vla_dtype_t;

typedef enum {
  VLA_PATH_AUTO = 0,  /* library chooses from (B*H, T, d)                              */
  VLA_PATH_SEQ = 1,   /* one workgroup per stream, token by token, state on chip       */
  VLA_PATH_CHUNK = 2, /* chunked (Woodbury / WY) form; parallel over time segments     */
  VLA_PATH_DECODE = 3 /* T = 1 only: one workgroup per stream with its state in
                         registers (chosen by AUTO whenever T = 1)                      */
} vla_path_t;

/* Gain of the S update.  UNIT is the method: ahat = A_t khat / ||A_t khat|| (VLA summary
 * §2.3 step 2).  RAW uses A_t khat without the normalisation: the ablation that §3.1
 * (Prop. 2) contrasts with the unit gain, whose state-transition products can grow without
 * bound.  RAW runs on the sequential and decode paths only (AUTO picks them; a forced
 * chunked path is VLA_ERROR_NOT_SUPPORTED). */
typedef enum { VLA_GAIN_UNIT = 0, VLA_GAIN_RAW = 1 } vla_gain_t;

typedef struct {
  int64_t B, H, T, d;       /* q, k, v, u, out are [B, H, T, d], row-major, d fastest   */
  int32_t dtype;            /* vla_dtype_t of q, k, v, u and out                        */
  int32_t path;             /* vla_path_t                                               */
  float eps;                /* readout denominator offset, >= 0 (1e-6 in all workloads) */
  int32_t chunk;            /* chunk length of the chunked path; 0 = library default    */
  void *workspace;          /* device scratch owned by the caller, or NULL              */
  size_t workspace_bytes;   /* its size in bytes; ignored when workspace is NULL        */
  int32_t gain;             /* vla_gain_t; 0 (UNIT) is the method                       */
} vla_desc_t;

/*
 * vla_forward -- the recurrence above over all B*H streams, enqueued on `stream`.
 *
 * q, k, v, u  device pointers, [B, H, T, d] in desc->dtype, read only, 16-byte aligned.
 * lambda0     initial penalty scale (M_0 = lambda0 I, A_0 = I / lambda0); > 0, finite.
 * out         device pointer, [B, H, T, d] in desc->dtype, fully overwritten; must not
 *             alias any input.
 * S_final     device pointer to [B, H, d, d] fp32 (S[i][j], i = value index, j = key
 *             index) receiving S_T, or NULL if not wanted.
 * A_final     device pointer to [B, H, d, d] fp32 receiving A_T (symmetric), or NULL.
 * desc        shapes, dtype, eps, path and workspace; read during the call only.
 * stream      HIP stream (NULL = null stream); the call is asynchronous.
 *
 * Ownership: the caller owns every buffer; the library keeps no pointer after the call
 * returns.  Outputs (out, S_final, A_final) must overlap neither one another nor any input,
 * and a caller's workspace must overlap none of them: an overlap returns
 * VLA_ERROR_INVALID_VALUE before any device work.  Workspace: the chunked path needs
 * vla_workspace_size() bytes of device scratch.  If desc->workspace is NULL the library uses
 * a cache of its own, one buffer per (device, stream), grown on demand: that call may
 * allocate, and a growing call first waits for the earlier work of its stream (so time
 * steady-state calls, or pass a workspace).  On a stream under graph capture a cache that
 * would have to grow gives VLA_ERROR_NOT_SUPPORTED: capture with a workspace.  Calls that
 * share a caller's workspace must be ordered on one stream.  Errors: a status code is
 * returned and nothing is enqueued on an argument error; the call never aborts or throws.
 * Kernel faults surface at the caller's next synchronisation.  NaN and Inf in the inputs
 * propagate and are not checked.
 * Streams: a chunked-path call of at least 2^20 tokens (B*H*T) on two or more streams, not
 * under graph capture, runs half of its (batch, head) streams on a second HIP stream of the
 * device that the library creates on first use and keeps (default priority, non-blocking),
 * forked from `stream` and joined back into it with events: the call stays ordered on
 * `stream` like any other, and its results are those of one launch over all streams.
 */
vla_status_t vla_forward(const void *q, const void *k, const void *v, const void *u,
                         float lambda0, void *out, float *S_final, float *A_final,
                         const vla_desc_t *desc, struct ihipStream_t *stream);

/*
 * vla_forward_state -- vla_forward continuing from a carried state: the streaming use of
 * the recurrence (VLA summary §5, practical scope: a fixed-size state for streaming
 * inference without a KV cache), where a long stream is fed in
 * pieces (or one token at a time, T = 1: decoding) and each call starts from the state the
 * previous one ended in.
 *
 * S0          device pointer to [B, H, d, d] fp32: S before the first token, or NULL for 0.
 * A0          device pointer to [B, H, d, d] fp32: A before the first token (the inverse
 *             penalty; symmetric positive definite, e.g. a previous call's A_final), or NULL
 *             for I / lambda0.  It is used as (A0 + A0^T) / 2.
 * n0          device pointer to [B, H, d] fp32: the readout normaliser n before the first
 *             token (a previous call's n_final), or NULL for 0.
 * lambda0     as in vla_forward; only read when A0 is NULL.
 * S_final, A_final   as in vla_forward.
 * n_final     device pointer to [B, H, d] fp32 receiving n_T, or NULL.
 *             S_final, A_final and n_final must not overlap S0, A0 or n0 (no in-place
 *             update: feed a decode loop from two sets of state buffers in turn), nor one
 *             another, out or q, k, v, u; an overlap returns VLA_ERROR_INVALID_VALUE.
 * The other arguments, ownership, workspace and error behaviour are those of vla_forward
 * (state pointers must be 16-byte aligned, else VLA_ERROR_NOT_SUPPORTED).  Splitting a
 * sequence into two calls, the second starting from the first's (S_final, A_final,
 * n_final), gives the single call's result up to rounding.  vla_forward is this call with
 * S0 = A0 = n0 = NULL and n_final = NULL.
 */
vla_status_t vla_forward_state(const void *q, const void *k, const void *v, const void *u,
                               float lambda0, const float *S0, const float *A0, const float *n0,
                               void *out, float *S_final, float *A_final, float *n_final,
                               const vla_desc_t *desc, struct ihipStream_t *stream);

/*
 * vla_forward_state_noalloc -- vla_forward_state for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It runs the same kernels as vla_forward_state on the same arguments, and the
 * chunked path's scratch (vla_workspace_size() bytes) lives in one static device array per
 * GPU of VLA_NOALLOC_SCRATCH_BYTES bytes, held by the library until the process ends; the
 * call allocates nothing, creates no timing events (vla_profile_enable is ignored) and never
 * runs streams on the library's second HIP stream.
 *
 * desc->workspace must be NULL (VLA_ERROR_INVALID_VALUE otherwise).  A descriptor whose
 * chunked path needs more than VLA_NOALLOC_SCRATCH_BYTES of scratch returns
 * VLA_ERROR_NOT_SUPPORTED before any device work (the sequential and decode paths need
 * none).  Every allocation-free call on one GPU shares that GPU's array: such calls must be
 * ordered (one stream, or streams joined by events); calls that overlap on one GPU race and
 * give wrong results.  Nothing in the array needs to start at any value (every byte a call
 * reads it has written first).  Everything else is as for vla_forward_state.
 */
#define VLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
vla_status_t vla_forward_state_noalloc(const void *q, const void *k, const void *v, const void *u,
                                       float lambda0, const float *S0, const float *A0,
                                       const float *n0, void *out, float *S_final, float *A_final,
                                       float *n_final, const vla_desc_t *desc,
                                       struct ihipStream_t *stream);

/*
 * vla_linear_attention -- the baseline the VLA update is measured against: standard linear
 * attention with the same ELU+1 feature map and ratio readout (VLA summary §2.1, the
 * unconditional accumulation VLA replaces; §2.3, the readout; §2.4 prices the VLA update at
 * about five times its operations), per (batch, head) stream from S_0 = 0, n_0 = 0:
 *
 *   S_t = S_{t-1} + v_t phi(k_t)^T,  n_t = n_{t-1} + phi(k_t),
 *   o_t = S_t phi(q_t) / (n_t^T phi(q_t) + eps)
 *
 * q, k, v     device pointers, [B, H, T, d] in desc->dtype, read only, 16-byte aligned.
 * out         device pointer, [B, H, T, d] in desc->dtype, fully overwritten; out, S_final,
 *             n_final and a caller's workspace overlap neither one another nor q, k, v, else
 *             VLA_ERROR_INVALID_VALUE.
 * S_final     device pointer to [B, H, d, d] fp32 (S[i][j], i = value, j = key) receiving
 *             S_T, or NULL.
 * n_final     device pointer to [B, H, d] fp32 receiving n_T, or NULL.
 * desc        as for vla_forward, with path VLA_PATH_AUTO, chunk 0 (or 64, the only chunk
 *             length) and gain VLA_GAIN_UNIT, else VLA_ERROR_NOT_SUPPORTED.  Chunked, time-segment parallel;
 *             workspace as for vla_forward, sized by vla_la_workspace_size().
 * Ownership, asynchrony and error behaviour are those of vla_forward.
 */
vla_status_t vla_linear_attention(const void *q, const void *k, const void *v, void *out,
                                  float *S_final, float *n_final, const vla_desc_t *desc,
                                  struct ihipStream_t *stream);

/* Bytes of device workspace vla_linear_attention needs for this descriptor. */
vla_status_t vla_la_workspace_size(const vla_desc_t *desc, size_t *bytes);

/*
 * vla_backward -- gradients of the recurrence of vla_forward (fixed start S_0 = 0,
 * A_0 = I / lambda0, n_0 = 0) for the scalar loss
 *   L = <d_out, out> + <dS_T, S_T> + <dA_T, A_T> + <dn_T, n_T>,
 * i.e. the reverse pass of training through the layer (VLA summary §3.1 argues the unit gain
 * keeps these gradients stable; §4 trains the models).
 *
 * q, k, v, u, lambda0  the forward's inputs, as for vla_forward (device, [B, H, T, d],
 *             desc->dtype, 16-byte aligned).
 * d_out       device pointer, [B, H, T, d] in desc->dtype: the cotangent of out.
 * dS_T, dA_T  device pointers to [B, H, d, d] fp32 cotangents of S_T and A_T, or NULL (0).
 * dn_T        device pointer to [B, H, d] fp32 cotangent of n_T, or NULL (0).
 * dq, dk, dv, du  device pointers, [B, H, T, d] fp32, fully overwritten.
 * dlambda0    device pointer to [B * H] fp32 receiving each stream's share of dL/dlambda0
 *             (their sum is the derivative; every stream starts from I / lambda0), or NULL.
 * desc        gain VLA_GAIN_UNIT, else VLA_ERROR_NOT_SUPPORTED.  path VLA_PATH_SEQ: one segment
 *             per stream (a replay of the forward token by token, then the reverse sweep).
 *             VLA_PATH_CHUNK: time split into the chunked forward's segments (desc->chunk, 0 =
 *             default; unsupported chunk or d: VLA_ERROR_NOT_SUPPORTED), all segments run in
 *             parallel: the chunked forward's passes give the state at every segment start,
 *             the cotangent of S crosses segments through per-segment affine maps (the reverse
 *             of the forward's segment maps) and the cotangents of n and of the penalty through
 *             suffix sums.  VLA_PATH_AUTO: CHUNK when that gives at least two segments per
 *             stream (at d = 128 only for at most 128 streams), else SEQ.
 *             VLA_PATH_DECODE: NOT_SUPPORTED.
 *             The workspace holds vla_backward_workspace_size() bytes (per stream T x (4 d + 8)
 *             floats of per-token vectors, the state at every 64th token and the cotangent of S
 *             at every 32nd token; with time segments
 *             the chunked forward's workspace and an fp64 d x d matrix per segment on top), else
 *             the per-device cache is used as for vla_forward.
 * At ||k_t|| = 0 or ||A_t khat_t|| = 0 the normalisation has no derivative; the
 * gradient through it is taken as 0.  The gradients (and a caller's workspace) must overlap
 * neither one another nor any input, else VLA_ERROR_INVALID_VALUE.  Ownership, asynchrony and
 * error behaviour are those of vla_forward.
 */
vla_status_t vla_backward(const void *q, const void *k, const void *v, const void *u,
                          float lambda0, const void *d_out, const float *dS_T, const float *dA_T,
                          const float *dn_T, float *dq, float *dk, float *dv, float *du,
                          float *dlambda0, const vla_desc_t *desc, struct ihipStream_t *stream);

/* Bytes of device workspace vla_backward needs for this descriptor. */
vla_status_t vla_backward_workspace_size(const vla_desc_t *desc, size_t *bytes);

/* Bytes of device workspace vla_forward needs for this descriptor (0 for the
 * sequential path).  Same argument checks as vla_forward; no device work. */
vla_status_t vla_workspace_size(const vla_desc_t *desc, size_t *bytes);

/* The path vla_forward would run for this descriptor (resolves VLA_PATH_AUTO). */
vla_status_t vla_resolve_path(const vla_desc_t *desc, int32_t *path);

/* Static, human-readable name of a status code. */
const char *vla_status_string(vla_status_t status);

/*
 * Optional per-kernel timing, for benchmarks.  While enabled, every kernel the library
 * launches is bracketed by a HIP event pair recorded on the launch stream; the pairs are
 * resolved (waiting for them) by vla_profile_count / vla_profile_get and accumulated per
 * kernel name.  Enabling creates events (host allocations); timing adds a few microseconds
 * of event records per launch.  Not thread-safe against concurrent vla_forward calls.
 */
vla_status_t vla_profile_enable(int32_t enable);   /* 1 = record, 0 = stop recording     */
vla_status_t vla_profile_reset(void);               /* drop all recorded timings          */
int32_t vla_profile_count(void);                    /* kernels with timings (waits on GPU) */
/* Name (NUL-terminated, truncated to name_cap), summed milliseconds and launch count of
 * the index-th timed kernel; VLA_ERROR_INVALID_VALUE for an index out of range. */
vla_status_t vla_profile_get(int32_t index, char *name, size_t name_cap, double *total_ms,
                             int64_t *launches);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int32_t vla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RLS_VLA_H */
