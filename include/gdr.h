/*
 * gdr.h -- C ABI of libgdr: the chunkwise-parallel forward pass of the
 * generalized gated delta rule, and its single-token decode step, on AMD
 * Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [QD]   "Q-Delta: Beyond Key-Value Associative State Evolution"
 *   [GDN2] "Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention"
 *   [KDA]  "You could have come up with Kimi Delta Attention"
 *   [CH11] "Chapter 11  Gated DeltaNet: understanding the recurrence from a
 *          matrix state"
 *
 * The operation.  For each (batch b, head h) an independent state
 * S in R^{dk x dv} (rows = key channels, [GDN2] key design 1, [CH11] 11.1)
 * evolves over tokens t = 0..T-1 as
 *
 *     S_bar = Diag(exp(g_t)) S          forget    ([KDA] 3-4)
 *     r     = S_bar^T e_t               predict along the erase direction
 *     S     = S_bar + k_t (z_t - r)^T   write along the key
 *     o_t   = S^T q_t                   read the post-update state ([CH11] 11.2)
 *
 * with the erase direction e_t and written value z_t chosen by the gate kinds:
 *     erase BETA:    e = beta_t * k_t    (qmix: e = beta_t * (k_t + lambda q_t), [QD] key design 3,
 *                                         lambda fixed per head or time-varying, key design 2)
 *     erase CHANNEL: e = b_t (.) k_t     ([GDN2] key design 1; b is not clamped)
 *     write BETA:    z = beta_t * v_t
 *     write CHANNEL: z = w_t (.) v_t     ([GDN2] key design 1)
 *     erase = write = VALUE: one beta per value channel gates the prediction
 *                    error ([CH11] 11.3): S = S_bar + k_t (beta_t (.) (v_t - S_bar^T k_t))^T,
 *                    i.e. every column of S follows its own scalar-beta rule.
 * DeltaNet = (NONE, BETA, BETA); Gated DeltaNet = (SCALAR, BETA, BETA);
 * KDA = (CHANNEL, BETA, BETA); Q-Delta = (SCALAR, BETA, BETA, qmix);
 * Gated DeltaNet-2 = (CHANNEL, CHANNEL, CHANNEL).
 *
 * gdr_chunk_fwd evaluates this with the chunk WY algorithm of [GDN2] key
 * design 2 (chunks of C = 64 tokens; intra-chunk matrices plus an
 * inter-chunk state recurrence), which reaches the token recurrence's result
 * up to rounding.  gdr_recurrent_step applies one token; gdr_recurrent_fwd
 * runs the token loop itself over any T (the fully recurrent form that [QD]
 * key design 3 pairs with the chunked one), for short sequences.
 *
 * Optional output epilogue ([CH11] 11.3; [GDN2] method flowchart): with
 * out_gate set, every entry point writes, instead of the readout o_t,
 *     y_t = o_t / sqrt(mean(o_t^2) + eps) (.) norm_weight (.) silu(gate_t)
 * per (batch, token, head) over the dv channels, silu(x) = x / (1 + e^-x).
 *
 * Caller-side preparation ([GDN2] training strategy, [CH11] 11.3): q and k
 * arrive already L2-normalised (q scaled as the model wants); gates are fp32
 * activations; g = log(alpha) <= 0 is finite.  The library never rescales.
 *
 * Conventions for every entry point:
 *  - Ownership: the caller owns every buffer, the optional workspace
 *    included.  The library allocates nothing, frees nothing and keeps no
 *    pointer after the call returns.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    with no host synchronisation.  Pointers are device pointers.
 *  - Inputs are read-only.  `o` must not overlap any input.  `state_out` may
 *    be exactly `state_in` (in-place update) but must not partially overlap it.
 *  - Errors: GDR_OK (0) or a non-zero gdr_status.  On a validation error
 *    nothing is launched and no output is written; gdr_last_error() gives a
 *    thread-local message.  GDR_E_HIP reports a HIP launch error.
 *  - Reentrant: no global mutable state besides the thread-local message
 *    (and the per-device scratch of gdr_chunk_fwd_noalloc, see there).
 *  - Deterministic: no atomics; the same inputs give bitwise-identical output.
 */
#ifndef GDR_H
#define GDR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 3
#define GDR_CHUNK 64

typedef enum gdr_status {
  GDR_OK = 0,
  GDR_E_NULL = 1,        /* a required pointer (or the args struct) is NULL      */
  GDR_E_SHAPE = 2,       /* B, T, H, dk, dv, chunk out of range                  */
  GDR_E_DTYPE = 3,       /* unknown io dtype                                      */
  GDR_E_ALIGN = 4,       /* a pointer is not aligned as documented                */
  GDR_E_UNSUPPORTED = 5, /* a valid combination the library does not implement   */
  GDR_E_HIP = 6,         /* the HIP runtime reported an error                     */
  GDR_E_ARGS = 7         /* inconsistent arguments (kinds, aliasing, struct size) */
} gdr_status;

typedef enum gdr_dtype { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;
typedef enum gdr_decay { GDR_DECAY_NONE = 0, GDR_DECAY_SCALAR = 1, GDR_DECAY_CHANNEL = 2 } gdr_decay;
typedef enum gdr_gate { GDR_GATE_BETA = 0, GDR_GATE_CHANNEL = 1, GDR_GATE_VALUE = 2 } gdr_gate;

/*
 * Arguments.  Every per-token tensor is [B, T, H, ...], contiguous, row-major
 * (the last index fastest).
 *
 *   q, k     [B,T,H,dk]   io dtype                         16-byte aligned
 *   v        [B,T,H,dv]   io dtype                         16-byte aligned
 *   o        [B,T,H,dv]   io dtype, written                16-byte aligned
 *   g        decay SCALAR: [B,T,H] fp32; CHANNEL: [B,T,H,dk] fp32 (16-byte
 *            aligned); NONE: must be NULL.  Log of the retention gate.
 *   beta     [B,T,H] fp32; required iff erase or write is BETA (or qmix);
 *            [B,T,H,dv] fp32 when erase = write = VALUE
 *   b        [B,T,H,dk] fp32, 16-byte aligned; required iff erase CHANNEL
 *   w        [B,T,H,dv] fp32, 16-byte aligned; required iff write CHANNEL
 *   lambda   qmix 1: [H] fp32 (one lambda per head); qmix 2: [B,T,H] fp32
 *            (time-varying lambda_t); required iff qmix (then erase must be BETA)
 *   state_in [B,H,dk,dv] fp32, 16-byte aligned, or NULL for a zero state
 *   state_out[B,H,dk,dv] fp32, 16-byte aligned, or NULL (not written)
 *   out_gate [B,T,H,dv] io dtype, 16-byte aligned, or NULL (no epilogue)
 *   norm_weight [dv] fp32; required iff out_gate
 *   norm_eps  RMSNorm epsilon; <= 0 selects 1e-6
 *
 * Fields set to zero select defaults; set struct_size = sizeof(gdr_args).
 * Older structs are accepted: ABI version 1 (ending at `o`, struct_size =
 * offsetof(gdr_args, workspace)) runs without a workspace, version 2 (ending
 * at workspace_bytes) without the epilogue.
 * dv_split: 0 lets the library choose how many workgroups share one head's
 * value columns; otherwise the column-slice width (16, 32 or 64, dividing dv).
 * When T == 0, q/k/v/o/gates may be NULL and state_out receives state_in
 * (or zeros).
 *
 * workspace, workspace_bytes: optional device scratch, 256-byte aligned, for
 * the two-pass form of the bf16, dk = 128 forward under a per-channel decay,
 * or under no or a scalar decay with the beta erase gate.  When a head's
 * value columns are split into slices of 16 or 32 (few heads: B * H * dv / 64
 * < 256), the single-pass kernels repeat every chunk's state-independent work
 * (decay factors, Gram tiles, inverse) in each slice; with a workspace of at
 * least gdr_workspace_size() bytes that work runs once per chunk, in a
 * separate parallel pass that writes one record per (batch, head, chunk) to
 * the workspace (58.5 KiB under a per-channel decay, 11.5 KiB otherwise), and
 * a second pass applies the records to the state.  NULL (or too small) keeps
 * the single pass.  The workspace must not overlap any
 * other argument; its contents are undefined after the call, and concurrent
 * calls need separate workspaces.
 */
typedef struct gdr_args {
  uint32_t struct_size;
  int32_t B, T, H, dk, dv;
  int32_t chunk;     /* must be 64 (0 = 64) */
  int32_t io;        /* gdr_dtype of q, k, v, o */
  int32_t decay;     /* gdr_decay */
  int32_t erase;     /* gdr_gate */
  int32_t write;     /* gdr_gate */
  int32_t qmix;      /* 0 none, 1 lambda per head, 2 lambda per token */
  int32_t dv_split;  /* 0 = auto */
  const void *q, *k, *v;
  const float *g, *beta, *b, *w, *lambda;
  const float *state_in;
  float *state_out;
  void *o;
  void *workspace;          /* optional, see above; NULL = none */
  uint64_t workspace_bytes; /* bytes available at workspace */
  const void *out_gate;     /* ABI version 3: output epilogue gate, NULL = none */
  const float *norm_weight;
  float norm_eps;
} gdr_args;

/* What a call would launch (filled by gdr_plan). */
typedef struct gdr_plan_info {
  int32_t grid;        /* workgroups */
  int32_t block;       /* threads per workgroup */
  int32_t dv_slice;    /* value columns per workgroup */
  int32_t lds_bytes;   /* LDS per workgroup */
  int32_t n_chunks;    /* chunks per sequence */
  int32_t passes;      /* 1, or 2 for the workspace form (grid, block and
                          lds_bytes then describe the second pass) */
} gdr_plan_info;

/*
 * Chunkwise forward over any T >= 0 ([GDN2] key design 2, C = 64).
 * Supported: io BF16 or F32 with dk in {64, 128}; dv a multiple of 16,
 * 16..256, divisible by the slice width.  fp32 I/O keeps fp32 accuracy (the
 * tighter fp32 tolerance): fp32 products, or at dk 128 in the two-pass form
 * split-precision products (each operand as two bf16 halves, fp32
 * accumulation); the per-value-channel beta and a time-varying lambda run on
 * the plain kernels (fp32 arithmetic or split precision).  Other
 * valid combinations return GDR_E_UNSUPPORTED.  The epilogue (out_gate)
 * needs dv in {64, 128, 256}; it runs as a second kernel over o in place,
 * because the chunk kernels split a head's value columns over workgroups.
 */
gdr_status gdr_chunk_fwd(const gdr_args *a, void *stream);

/*
 * The chunkwise forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and support matrix as gdr_chunk_fwd
 * with a workspace of gdr_workspace_size() bytes; the two-pass records are
 * written to a scratch array inside the library instead of a caller
 * workspace (a->workspace and a->workspace_bytes are ignored).
 *  - Limit: the scratch holds GDR_NOALLOC_SCRATCH_BYTES (64 MiB) per device;
 *    a call whose records need more (gdr_workspace_size) returns GDR_E_SHAPE
 *    before any launch.  Shapes without a two-pass form run the single pass
 *    and touch no scratch.
 *  - The call allocates nothing (no hipMalloc, no library allocation).  Each
 *    GPU the library runs on holds its own copy of the scratch until the
 *    process ends; its device address is looked up once per device, on the
 *    first call made with that device current.
 *  - Every call on one GPU shares that GPU's scratch: calls that overlap in
 *    time on one GPU (concurrent streams, or several host threads) race and
 *    must be serialised by the caller.  The records are rewritten in full by
 *    each call; nothing in the scratch needs clearing.
 */
#define GDR_NOALLOC_SCRATCH_BYTES (64ull << 20)
gdr_status gdr_chunk_fwd_noalloc(const gdr_args *a, void *stream);

/*
 * One decode step ([CH11] 11.3: the streaming caller passes the previous
 * final state back in).  Requires T == 1.  io BF16 or F32, dk and dv in
 * {64, 128}.  state_out may equal state_in for an in-place update.  The
 * epilogue is fused.
 */
gdr_status gdr_recurrent_step(const gdr_args *a, void *stream);

/*
 * The fully recurrent form over any T >= 0 ([QD] key design 3 provides it
 * beside the chunked kernel; [CH11] 11.3's streaming caller): the token loop
 * in one kernel, one workgroup per (batch, head), the state in registers for
 * the whole call.  For short sequences (prefill of a few tokens, speculative
 * decode); the chunk form is the one for long ones.  Every gate kind and
 * qmix; io BF16 or F32; dk and dv in {64, 128}.  state_out may equal
 * state_in.  The epilogue is fused.
 */
gdr_status gdr_recurrent_fwd(const gdr_args *a, void *stream);

/*
 * The output epilogue on its own ([CH11] 11.3): y = o / sqrt(mean(o^2) +
 * eps) (.) weight (.) silu(gate) over each row of dv values.  o, gate and y
 * are [rows][dv] in the io dtype, 16-byte aligned; y may be exactly o (in
 * place) but must not partially overlap o, gate or weight.  dv in {64, 128,
 * 256}; eps <= 0 selects 1e-6.
 */
typedef struct gdr_norm_args {
  uint32_t struct_size; /* sizeof(gdr_norm_args) */
  int32_t dv;
  int32_t io;           /* gdr_dtype */
  float eps;
  int64_t rows;         /* >= 0, e.g. B * T * H */
  const void *o;
  const void *gate;
  const float *weight;  /* [dv] fp32 */
  void *y;
} gdr_norm_args;
gdr_status gdr_output_norm_gate(const gdr_norm_args *a, void *stream);

/*
 * Backward of the chunkwise forward ([GDN2] key design 3: the chunk form's
 * backward, with dT = -tril(A^T dA A^T, -1) and the gate weights inside the
 * dA products): for a loss L with dL/do = d_o and dL/dS_final = d_state,
 * the gradients of every input of the forward call `fwd`.
 *
 *   fwd       the forward's arguments (q, k, v, gates, kinds, state_in);
 *             its o, state_out, workspace and epilogue fields are not read
 *             (the gradient is the one of the readout o, before any epilogue)
 *   d_o       [B,T,H,dv] io dtype, 16-byte aligned
 *   d_state   [B,H,dk,dv] fp32, or NULL (zero)
 *   dq, dk    [B,T,H,dk] fp32, written        dv  [B,T,H,dv] fp32, written
 *   dg        like g (SCALAR [B,T,H], CHANNEL [B,T,H,dk]); iff a decay
 *   dbeta     [B,T,H]; iff beta is used       db  [B,T,H,dk]; iff erase CHANNEL
 *   dw        [B,T,H,dv]; iff write CHANNEL   dlam [H] (qmix 1) or [B,T,H] (qmix 2)
 *   dstate    [B,H,dk,dv] fp32 or NULL: the gradient of state_in
 *   workspace >= gdr_bwd_workspace_size() bytes, 256-byte aligned (required
 *             when T > 0): the per-chunk states and factors the reverse
 *             passes read back (about 320 KiB per (batch, head, chunk) at
 *             dk = dv = 128)
 * Outputs are fp32 and must overlap neither the inputs nor each other.
 * Supported: io BF16 or F32, dk and dv in {64, 128}, every decay, the BETA
 * and CHANNEL gates and qmix; the per-value-channel beta returns
 * GDR_E_UNSUPPORTED.  fp32 accumulation throughout; products in fp32 or in
 * split precision (each operand as two bf16 halves; bf16 inputs multiplied
 * exactly), within 2.1e-5 of the float64 adjoint on the test set.
 * Deterministic (no atomics).
 */
typedef struct gdr_bwd_args {
  uint32_t struct_size;     /* sizeof(gdr_bwd_args) */
  const gdr_args *fwd;
  const void *d_o;
  const float *d_state;
  float *dq, *dk, *dv, *dg, *dbeta, *db, *dw, *dlam, *dstate;
  void *workspace;
  uint64_t workspace_bytes;
} gdr_bwd_args;
gdr_status gdr_chunk_bwd(const gdr_bwd_args *a, void *stream);

/* Host-only: the workspace bytes gdr_chunk_bwd needs for `a`. */
gdr_status gdr_bwd_workspace_size(const gdr_bwd_args *a, uint64_t *bytes);

/* Host-only: the workspace bytes that gdr_chunk_fwd can use for `a` (0 when
 * the shape takes no workspace).  Checks `a` like gdr_plan. */
gdr_status gdr_workspace_size(const gdr_args *a, uint64_t *bytes);

/* Host-only validation of `a` for op 0 (chunk), 1 (step) or 2 (recurrent);
 * launches nothing and touches no device memory, so it runs without a GPU. */
gdr_status gdr_validate(const gdr_args *a, int op);

/* Host-only launch plan for op 0 / 1 / 2.  Checks shapes, kinds and the support
 * matrix like gdr_validate but not the pointers (they may be NULL). */
gdr_status gdr_plan(const gdr_args *a, int op, gdr_plan_info *out);

const char *gdr_status_str(gdr_status s);
const char *gdr_last_error(void);
int gdr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
