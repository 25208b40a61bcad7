/*
 * swimba.h -- C ABI of libswimba.so: the Swimba (Switch Mamba)
 * parameter-space mixture-of-experts selective scan on MI355X (gfx950).
 *
 * Pages cited by title and section:
 *   [SW] "Swimba: Switch Mamba Model Scales State Space Models" (gist.science
 *        summaries; Dutch "Kernmechanisme van Swimba": router weights per token,
 *        parameters of the active experts mixed, one recurrence; Spanish
 *        "Distinción de Diseños" / French "Distinction des deux designs": the
 *        separate design with one state trajectory per expert; French
 *        "Fondements Théoriques": Theorems 1-4).
 *   [MB] "Mamba y las SSMs: el retorno del estado persistente" (section "SSMs":
 *        h_t = A h_{t-1} + B x_t, y_t = C h_t + D x_t; section "Mamba":
 *        selective B_t, C_t and transition exp(Delta_t A); Figure 2: the state
 *        kept on chip, inputs and outputs streamed from HBM).
 *
 * What the library computes, per sequence b and channel d (N = 16 states):
 *   router:  l_e = sum_d x_d Wr[d,e]; top k by (logit desc, expert asc);
 *            gates = softmax over the k selected logits.
 *   mixed:   Abar = sum_j g_j A[e_j,d,:], beta = sum_j g_j dt_bias[e_j,d],
 *            delta = sum_j g_j Dskip[e_j,d]; Delta = softplus(dt_raw + beta);
 *            h <- exp(Delta Abar) * h + Delta * B_t * x;  y = C_t . h + delta x
 *            (y reads the updated state).  Options: A one scalar per channel
 *            (a_form), zero-order-hold input term (disc).
 *   separate: each expert keeps its own state; at token t each selected
 *            expert e_j advances with its own A, bias, Dskip and emits y_j;
 *            y = sum_j g_j y_j; unselected experts' states do not change.
 *   slots:   each routing slot j keeps its own state, which advances at every
 *            token with the parameters of the expert in slot j (unmixed) and
 *            keeps its value when that expert changes; y = sum_j g_j y_j.
 *   all experts: each expert keeps its own state and advances it at every
 *            token with its own parameters, selected or not; the routing
 *            only picks whose outputs y = sum_j g_j y_{e_j} mixes.
 *   streams: A shared by the experts; each selected expert's B, C and X
 *            streams arrive per routing slot; the injection
 *            Delta sum_j g_j B_j X_j and the readout vector sum_j g_j C_j
 *            are mixed ([SW] "Kernmechanisme van Swimba").
 *
 * Conventions (all entry points):
 *   - Every tensor argument is a DEVICE pointer owned by the caller, dense and
 *     row-major (last index fastest), and must stay valid until the work
 *     enqueued on `stream` has finished.  The library allocates no memory,
 *     keeps no state beyond a per-device cache of the compute-unit count (and
 *     the fixed buffer of swimba_scan_noalloc), and never synchronises the
 *     stream; calls on different streams may run concurrently (except
 *     swimba_scan_noalloc calls on one device).
 *   - Work is enqueued on `stream` (NULL = the null stream).  A return of
 *     SWIMBA_OK means the kernels were launched; execution errors surface in
 *     later HIP calls on that stream.
 *   - Arguments are validated on the host before anything is launched; on a
 *     negative return nothing was enqueued.  Values are not inspected:
 *     NaN/Inf propagate.  The scans assume A < 0 and gates >= 0 (contractive
 *     transitions, [SW] Theorem 3); when the kernels see otherwise they fall
 *     back to an exact but slower carry between chunks.
 *   - bf16 tensors hold raw bfloat16 bits (uint16).  Arithmetic is fp32.
 */
#ifndef SWIMBA_H
#define SWIMBA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SWIMBA_F32 = 0, SWIMBA_BF16 = 1 } swimba_dtype;

enum {
  SWIMBA_OK = 0,
  SWIMBA_EINVAL = -1,       /* a null pointer, a negative size, k > E, ...   */
  SWIMBA_EUNSUPPORTED = -2, /* valid but not built: N != 16, E > 64, ...     */
  SWIMBA_EWORKSPACE = -3,   /* workspace smaller than the query, or unaligned */
  SWIMBA_EHIP = -4,         /* a kernel launch failed                         */
  SWIMBA_ESCRATCH = -5      /* swimba_scan_noalloc: the chunk workspace would
                               exceed SWIMBA_NOALLOC_SCRATCH_BYTES           */
};

/* Largest expert count and the only state size the library supports. */
#define SWIMBA_MAX_EXPERTS 64
#define SWIMBA_STATE_N 16

/*
 * swimba_route -- router logits, top-k and gates for T tokens ([SW] Dutch
 * summary "Kernmechanisme van Swimba": per-token weights pi_t over the
 * active experts, top-1 or top-k).
 *   x      [T, D]  token features, dtype x_dtype
 *   Wr     [D, E]  fp32 router weights
 *   idx    [T, k]  out, int32: selected experts, largest logit first; equal
 *                  logits are taken in ascending expert order
 *   gate   [T, k]  out, fp32: softmax over the selected logits (top-1: 1.0)
 * Logits are fp32 sums; a token whose logits tie to within fp32 rounding may
 * order those experts either way.  Constraints: T >= 0, D >= 1,
 * 1 <= k <= E <= SWIMBA_MAX_EXPERTS.  T == 0 launches nothing.
 */
int swimba_route(const void* x, swimba_dtype x_dtype, const float* Wr, int64_t T, int D, int E,
                 int k, int32_t* idx, float* gate, hipStream_t stream);

/* How the scans join chunks of one sequence. */
typedef enum {
  SWIMBA_CARRY_AUTO = 0,   /* library's choice (the decay-bounded fix-up)    */
  SWIMBA_CARRY_REWALK = 1, /* recompute every chunk from its carried state   */
  SWIMBA_CARRY_FIXUP = 2   /* recompute only until the carried state has
                              decayed below fp32 resolution (needs A < 0)    */
} swimba_carry;

/*
 * Shape of the transition A.  DIAGONAL: one entry per state, A[..., D, N].
 * SCALAR: one entry per channel shared by its N states, A[..., D] -- the
 * Mamba-2 form A_t = a_t I that Swimba is built on ([SW] Spanish summary
 * "Arquitectura de Swimba", French "Architecture de Swimba": Mamba-2 and its
 * SSD operator); one exponential per (token, channel) instead of N.
 */
typedef enum { SWIMBA_A_DIAGONAL = 0, SWIMBA_A_SCALAR = 1 } swimba_a_form;

/*
 * Discretisation of the input term.  EULER: Delta B_t x.  ZOH: zero-order
 * hold, B_bar = A^{-1}(exp(Delta A) - I) B_t ([MB] "Mamba": the discretised
 * state equations), i.e. the coefficient (exp(Delta Abar) - 1)/Abar per state
 * entry in place of Delta.
 */
typedef enum { SWIMBA_DISC_EULER = 0, SWIMBA_DISC_ZOH = 1 } swimba_disc;

typedef struct {
  int B, L, D, N, E, k;         /* batch, length, channels, states (16), experts, active */
  swimba_dtype in_dtype;        /* dtype of x, dt_raw, Bm, Cm                            */
  swimba_dtype y_dtype;         /* dtype of y                                            */
  const void* x;                /* [B, L, D]                                             */
  const void* dt_raw;           /* [B, L, D]  step size before bias and softplus          */
  const void* Bm;               /* [B, L, N]  selective input vector B_t (16-byte aligned)  */
  const void* Cm;               /* [B, L, N]  selective output vector C_t (16-byte aligned) */
  const int32_t* idx;           /* [B, L, k]  routing, 0 <= idx < E (values outside are
                                   not reported: the kernels clamp them to 0 or E-1)    */
  const float* gate;            /* [B, L, k]  routing weights                             */
  const float* A;               /* [E, D, N]  per-expert diagonal transition (< 0);
                                   [E, D] with a_form SCALAR                            */
  const float* dt_bias;         /* [E, D]                                                 */
  const float* Dskip;           /* [E, D]     per-expert feed-through D                   */
  const float* h0;              /* NULL = zeros; [B, D, N] (separate and all experts:
                                   [B, E, D, N]; slots: [B, k, D, N])                    */
  void* y;                      /* [B, L, D]  out                                         */
  float* h_final;               /* NULL = not written; [B, D, N] (separate and all
                                   experts: [B, E, D, N]; slots: [B, k, D, N])           */
  int chunk;                    /* tokens per chunk; 0 = library's choice                 */
  swimba_carry carry;           /* chunk join method                                      */
  hipEvent_t* phase_events;     /* NULL, or 6 timing events: start and end of the chunk
                                   pass, of the carry pass and of the fix-up pass, in
                                   that order, stamped by each pass's kernel dispatch
                                   (no extra packets on `stream`); a pass that does not
                                   run has both events recorded where it would run      */
  swimba_a_form a_form;         /* A is [E, D, N] (DIAGONAL, 0) or [E, D] (SCALAR)        */
  swimba_disc disc;             /* input term: EULER (0) or ZOH                          */
} swimba_scan_args;

/* Which scan a workspace or plan query is for. */
enum {
  SWIMBA_DESIGN_MIXED = 0,    /* swimba_scan          */
  SWIMBA_DESIGN_SEPARATE = 1, /* swimba_scan_separate */
  SWIMBA_DESIGN_SLOTS = 2,    /* swimba_scan_slots    */
  SWIMBA_DESIGN_ALL_EXPERTS = 3 /* swimba_scan_all_experts */
};

/*
 * swimba_scan_workspace_size -- bytes of device workspace the scan named by
 * `design` (SWIMBA_DESIGN_*) needs for these arguments (0 when the sequence
 * is one chunk).  Returns 0 as well for invalid arguments or an unknown
 * design; the scan call itself reports those.  The library's chunking
 * depends on the device's compute-unit count: this query (and
 * swimba_scan_plan) plans for the current device, a scan call for the device
 * of its stream.
 */
size_t swimba_scan_workspace_size(const swimba_scan_args* a, int design);

/*
 * swimba_scan_plan -- the chunking the scan named by `design` will use for these arguments:
 * tokens per chunk and number of chunks (both 0 when B or L is 0).  Reads
 * sizes and options only; returns the status the scan's size validation
 * would return.
 */
int swimba_scan_plan(const swimba_scan_args* a, int design, int* chunk, int* nchunks);

/*
 * swimba_scan -- the parameter-space-mixed selective scan: one state
 * trajectory per (b, d), the selected experts' A, dt_bias and Dskip mixed by
 * the gates at every token ([SW] "Kernmechanisme van Swimba"; Theorem 1; [MB]
 * "Mamba": exp(Delta A) transition, Figure 2 on-chip state).
 *   ws, ws_bytes: device workspace of at least swimba_scan_workspace_size(a,0)
 *   bytes, 256-byte aligned; its contents on entry do not matter.
 * Constraints: B, L >= 0; D >= 1; N == 16; 1 <= k <= E <= 64; chunk >= 0;
 * with E > 16, E * D * 64 < 2^31 (SWIMBA_EUNSUPPORTED otherwise).  Up to 16
 * experts the expert tables are staged in LDS; from 17 to 32 experts with a
 * diagonal A only the A rows are (dt_bias and Dskip are read from memory per
 * token); beyond, each token's selected expert rows are read from memory
 * (slower per token).  L == 0 writes h_final = h0 (or zeros).
 */
int swimba_scan(const swimba_scan_args* a, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * swimba_scan_noalloc -- swimba_scan for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same computation, kernels, constraints and outputs as
 * swimba_scan; the chunk workspace lives in a buffer the library owns
 * instead of a caller's `ws`.
 *   - The buffer is a fixed device array of SWIMBA_NOALLOC_SCRATCH_BYTES
 *     (64 MiB), one per device, which each device the library runs on holds
 *     until the process ends.  The call makes no hipMalloc, hipFree
 *     or other allocating call; its first chunked call on a device looks the
 *     buffer's address up (hipGetSymbolAddress).
 *   - A call whose swimba_scan_workspace_size(a, SWIMBA_DESIGN_MIXED) would
 *     exceed the buffer returns SWIMBA_ESCRATCH and enqueues nothing (a
 *     larger chunk, or swimba_scan with a caller workspace, avoids it).
 *     The size is planned for the device of `stream`.
 *   - Every call on one device shares that device's buffer, which keeps the
 *     last call's contents: calls that overlap on one GPU (on different
 *     streams, or from different host threads without ordering) race and
 *     give wrong results.  Order them on one stream.  Nothing in the buffer
 *     needs to start at zero: each call writes every entry it reads.
 */
#define SWIMBA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int swimba_scan_noalloc(const swimba_scan_args* a, hipStream_t stream);

/*
 * swimba_scan_separate -- the separate design ([SW] "MoE of separate SSMs"):
 * one state per expert (h0/h_final [B, E, D, N]); each selected expert
 * advances with its own parameters; y = sum_j g_j y_j.  An expert listed
 * twice for one token advances twice.  Same constraints as swimba_scan.  Up
 * to 16 experts one wave keeps one expert's states and row in registers;
 * with more, each wave keeps the states of two (E <= 32) or four experts and
 * reloads their rows once per staged round (slower per token).  Chunks are
 * joined by a fix-up that stops once every expert's carried state has
 * decayed below fp32 resolution of its state (A < 0; SWIMBA_CARRY_REWALK or
 * a non-negative A re-walk whole chunks); the library's chunking gives this
 * design a few long chunks.
 */
int swimba_scan_separate(const swimba_scan_args* a, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * swimba_scan_slots -- separate trajectories per routing slot, the other
 * reading of the separate design ([SW] Spanish "Distinción de Diseños",
 * French "Distinction des deux designs"): h0/h_final [B, k, D, N]; slot j's
 * state advances at every token with the A, dt_bias and Dskip of expert
 * idx[t, j] (not mixed) and carries over when that expert changes; y adds
 * the slots' outputs C_t . h_j + Dskip x weighted by the gates, which never
 * enter a state.  Where every slot keeps one expert for the whole sequence
 * this equals swimba_scan_separate.  Workspace: swimba_scan_workspace_size
 * with SWIMBA_DESIGN_SLOTS.  Same constraints as swimba_scan, plus k <= 4
 * (the k x N states of a channel are held in registers); with more than 16
 * experts the rows are read from memory every token and k <= 2
 * (SWIMBA_EUNSUPPORTED otherwise).
 */
int swimba_scan_slots(const swimba_scan_args* a, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * swimba_scan_all_experts -- the third reading of the separate design ([SW]
 * Spanish "Distinción de Diseños", French "Distinction des deux designs":
 * separate SSMs, one per expert): h0/h_final [B, E, D, N]; every expert's
 * state advances at every token with its own A, dt_bias and Dskip, whether
 * or not the token selected it, so each trajectory is a plain selective scan
 * and does not depend on the routing; y = sum_j g_j (C_t . h_{e_j} +
 * Dskip[e_j] x).  E state updates per token instead of k.  With k = E and
 * every expert selected at every token this equals swimba_scan_separate.
 * Workspace: swimba_scan_workspace_size with SWIMBA_DESIGN_ALL_EXPERTS.
 * Same constraints as swimba_scan_separate.
 */
int swimba_scan_all_experts(const swimba_scan_args* a, void* ws, size_t ws_bytes,
                            hipStream_t stream);

typedef struct {
  swimba_scan_args fwd;         /* the forward call's arguments; its y, h_final,
                                   chunk and phase_events are not used            */
  const void* dy;               /* [B, L, D]  dL/dy, dtype dy_dtype               */
  swimba_dtype dy_dtype;
  const float* dh_final;        /* [B, D, N]  dL/dh_final, or NULL for zero        */
  float* dx;                    /* [B, L, D]  out                                  */
  float* ddt_raw;               /* [B, L, D]  out                                  */
  float* dBm;                   /* [B, L, N]  out, summed over channels            */
  float* dCm;                   /* [B, L, N]  out, summed over channels            */
  float* dgate;                 /* [B, L, k]  out, summed over channels            */
  float* dA;                    /* [E, D, N]  out, summed over batch and tokens    */
  float* ddt_bias;              /* [E, D]     out                                  */
  float* dDskip;                /* [E, D]     out                                  */
  float* dh0;                   /* [B, D, N]  out, or NULL                         */
} swimba_scan_grad_args;

/*
 * swimba_scan_backward -- gradients of swimba_scan for training ([SW] French
 * summary "Résultats Expérimentaux": the Swimba layers are trained; [MB]
 * "Mamba": the selective recurrence).  With lam_t = dL/dh_t obeying
 * lam_t = C_t dy_t + a_{t+1} lam_{t+1} (lam_{L-1} from dh_final), returns
 * dL/d of x, dt_raw, B_t, C_t, the gates (as free inputs: the router's own
 * backward is not part of this call), A, dt_bias, Dskip and h0, all fp32.
 * The forward is recomputed inside from the same arguments (same chunking
 * as swimba_scan).
 *   ws, ws_bytes: device workspace of at least
 *   swimba_scan_backward_workspace_size(g) bytes, 256-byte aligned (the
 *   forward's disc must be EULER; ZOH returns SWIMBA_EUNSUPPORTED).  No
 *   state is kept per token: the gradient pass rebuilds each 8-token block's
 *   states from a checkpoint, so the workspace holds the per-chunk records
 *   (decays, states, adjoints, parameter-gradient partials), the block
 *   checkpoints (16 bytes per token and channel) and per-tile sums over
 *   channels (about 0.5 bytes per token and channel).
 * Constraints: those of swimba_scan with E <= 16 and a_form DIAGONAL (SCALAR
 * returns SWIMBA_EUNSUPPORTED).  B == 0 or L == 0 writes zero parameter gradients
 * and dh0 = dh_final (or zeros).  Every output is deterministic.
 */
size_t swimba_scan_backward_workspace_size(const swimba_scan_grad_args* g);
int swimba_scan_backward(const swimba_scan_grad_args* g, void* ws, size_t ws_bytes,
                         hipStream_t stream);

typedef struct {
  int B, D, N, E, k;
  swimba_dtype in_dtype, y_dtype;
  const void* x;                /* [B, D]                                        */
  const void* dt_raw;           /* [B, D]                                        */
  const void* Bm;               /* [B, N]                                        */
  const void* Cm;               /* [B, N]                                        */
  const float* Wr;              /* [D, E]: route this token when idx == NULL     */
  const int32_t* idx;           /* NULL, or forced routing [B, k], 0 <= idx < E
                                   (values outside are clamped to 0 or E-1)      */
  const float* gate;            /* [B, k] with idx                               */
  int32_t* idx_out;             /* NULL, or [B, k]: routing used                 */
  float* gate_out;              /* NULL, or [B, k]                               */
  const float* A;               /* [E, D, N], or [E, D] with a_form SCALAR       */
  const float* dt_bias;         /* [E, D]                                        */
  const float* Dskip;           /* [E, D]                                        */
  float* state;                 /* [B, D, N] fp32, read and updated in place     */
  void* y;                      /* [B, D] out                                    */
  swimba_a_form a_form;         /* A is [E, D, N] (DIAGONAL, 0) or [E, D] (SCALAR) */
  swimba_disc disc;             /* input term: EULER (0) or ZOH                  */
} swimba_step_args;

/*
 * swimba_step -- one decoding step of the mixed scan on a persistent state
 * ([MB] Figure 2: the state persists and is updated once per token): route
 * (unless forced), mix, discretise, update `state` in place and emit y.
 * Equal to swimba_scan over a length-1 sequence with h0 = h_final = state.
 * Constraints: B >= 0, D >= 1, N == 16, 1 <= k <= E <= 64; Wr or idx/gate.
 */
int swimba_step(const swimba_step_args* a, hipStream_t stream);

typedef struct {
  int B, L, D, N, k;            /* batch, length, channels, states (16), routing slots    */
  swimba_dtype in_dtype;        /* dtype of X, dt_raw, Bs, Cs                            */
  swimba_dtype y_dtype;         /* dtype of y                                            */
  const void* X;                /* [B, L, k, D]  input stream of each slot's expert      */
  const void* dt_raw;           /* [B, L, D]     shared step size before bias, softplus  */
  const void* Bs;               /* [B, L, k, N]  each slot's B stream                    */
  const void* Cs;               /* [B, L, k, N]  each slot's C stream                    */
  const float* gate;            /* [B, L, k]     router weight of each slot              */
  const float* A;               /* [D, N]        shared diagonal transition (< 0),
                                                 16-byte aligned                         */
  const float* dt_bias;         /* [D]                                                   */
  const float* h0;              /* NULL = zeros; [B, D, N]                               */
  void* y;                      /* [B, L, D]     out                                     */
  float* h_final;               /* NULL = not written; [B, D, N]                         */
  int chunk;                    /* tokens per chunk; 0 = library's choice                */
  swimba_carry carry;           /* chunk join method                                     */
  hipEvent_t* phase_events;     /* NULL, or 6 timing events, as in swimba_scan_args      */
} swimba_stream_args;

/*
 * swimba_scan_streams_workspace_size -- device workspace bytes for
 * swimba_scan_streams (0 when the sequence is one chunk or the arguments are
 * invalid).  swimba_scan_streams_plan -- its chunking (tokens per chunk,
 * number of chunks); returns the status the size validation would return.
 */
size_t swimba_scan_streams_workspace_size(const swimba_stream_args* a);
int swimba_scan_streams_plan(const swimba_stream_args* a, int* chunk, int* nchunks);

/*
 * swimba_scan_streams -- the stream-mixed form of the layer ([SW] Dutch
 * summary "Kernmechanisme van Swimba", French "Architecture de Swimba"): every
 * expert emits B, C and X streams, the transition A is shared, and one
 * recurrence runs over the mixed injection and readout.  Slot j of token t
 * holds the streams of the token's j-th selected expert with weight
 * gate[t, j].  Per (b, d), with Delta = softplus(dt_raw + dt_bias[d]):
 *   h[n] <- exp(Delta A[d,n]) h[n] + Delta sum_j gate_j Bs_j[n] X_j[d]
 *   y     = sum_n (sum_j gate_j Cs_j[n]) h[n]          (after the update)
 * The step size is shared (it is not one of the experts' streams) and the
 * readout has no feed-through term, as printed on the page.
 *   ws, ws_bytes: device workspace of at least
 *   swimba_scan_streams_workspace_size(a) bytes, 256-byte aligned.
 * Constraints: B, L >= 0; D >= 1; N == 16; 1 <= k <= 4 (EUNSUPPORTED above);
 * chunk >= 0; Bs and Cs aligned to two elements.  L == 0 writes
 * h_final = h0 (or zeros).  Chunks are joined exactly when A < 0; otherwise
 * every chunk is recomputed from its carried state.
 */
int swimba_scan_streams(const swimba_stream_args* a, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Static string for a status code. */
const char* swimba_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SWIMBA_H */
