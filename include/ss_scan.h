/*
 * ss_scan.h -- C ABI of the MI355X (gfx950) Mamba-1 S6 selective scan.
 *
 * The method (nnterp "selective_scan" page, class docstring; TransformerLens
 * "ssm_mixer" page, compute_ssm_state): per batch row b and channel c, with a
 * state h of state_dim numbers,
 *
 *   dt_t = softplus(dt_t + dt_bias[c])        (dt_softplus != 0)
 *        = dt_t + dt_bias[c]                  (dt_softplus == 0)
 *   h_t  = exp(dt_t * A[c,:]) * h_{t-1} + dt_t * B[b,:,t] * x_t
 *   y_t  = (C[b,:,t] . h_t + D[c] * x_t) * silu(z_t)    (gate when z != NULL)
 *
 * computed in fp32 with the state held in fp32. The calls mirror the two
 * kernel calls the nnterp page names: the prompt scan
 * (x, dt, A, B, C, D=, z=, delta_bias=) and the single-token state update
 * (state, x, dt, A, B, C, D, z=, dt_bias=), and take the kernel's
 * channel-first layouts from the same page. Those two calls (and the scan
 * that also returns states) take their tensors in an argument struct
 * (ss_scan_args, ss_update_args) plus a stream; the other calls take flat
 * argument lists.
 *
 * Conventions shared by every call:
 *  - All tensor pointers are DEVICE pointers to contiguous C-order arrays;
 *    the caller owns every buffer. The library allocates nothing and keeps no
 *    state between calls; calls are thread-safe.
 *  - io_dtype (ss_dtype) is the element type of x, dt, z, B, C and y.
 *    A, D, dt_bias, h0, h_last and state are always float32.
 *  - The call enqueues its kernel on `stream` (a hipStream_t; NULL = the
 *    default stream) and returns without synchronising, so it can be
 *    recorded by stream capture into a HIP graph and replayed.
 *  - Arguments are validated before anything is enqueued; a validation
 *    error returns its ss_status with no side effect. A failed launch returns
 *    SS_ERR_HIP.
 *  - Inputs are never modified (the decode state excepted). Outputs must not
 *    overlap inputs, except h_last == h0 (same pointer) in the scan and the
 *    in-place state of the decode step.
 *  - state_dim must be in [1, 64]; anything else is SS_ERR_UNSUPPORTED (the
 *    scan and the decode step).
 *  - Non-finite inputs are outside the contract.
 *  - Results are bitwise identical run to run for the same inputs.
 */
#ifndef SS_SCAN_H
#define SS_SCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SS_ABI_VERSION 9
#define SS_MAX_STATE_DIM 64
#define SS_MAX_GATED_DK 256
#define SS_MAX_CONV_WIDTH 8

typedef enum {
  SS_OK = 0,
  SS_ERR_NULL = 1,        /* a required pointer is NULL */
  SS_ERR_SHAPE = 2,       /* a size is negative or an index would overflow */
  SS_ERR_DTYPE = 3,       /* io_dtype is not an ss_dtype */
  SS_ERR_UNSUPPORTED = 4, /* state_dim outside [1, SS_MAX_STATE_DIM]; gated scan: dk, dv; conv width; rank */
  SS_ERR_ALIAS = 5,       /* an output overlaps an input it may not overlap */
  SS_ERR_HIP = 6,         /* the HIP runtime failed to launch the kernel */
  SS_ERR_ALIGN = 7        /* a pointer is not aligned to its element size */
} ss_status;

typedef enum { SS_F32 = 0, SS_BF16 = 1 } ss_dtype;

/*
 * Prompt / prefill scan over seqlen tokens: the arguments of ss_scan_fwd.
 *
 *   x, dt, z, y : [batch, channels, seqlen]   io_dtype
 *   B, C        : [batch, state_dim, seqlen]  io_dtype (one group: shared by
 *                                             every channel of a batch row)
 *   A           : [channels, state_dim]       float32 (negative rates)
 *   D, dt_bias  : [channels]                  float32, NULL reads as zeros
 *   z           : NULL = no gate
 *   h0          : [batch, channels, state_dim] float32, NULL = zero state
 *                 (a prompt's scan starts from zeros; nnterp page, attributes)
 *   reset       : [batch, seqlen] uint8 or NULL. reset[b,t] != 0 marks the
 *                 first token of a packed document: the state is zeroed
 *                 before that token, i.e. its decay exp(dt_t*A) is replaced
 *                 by 0 ("s6_reset" post, Enforced Boundary Resetting).
 *   dt_softplus : nonzero: dt <- softplus(dt + dt_bias); zero: dt + dt_bias
 *   y           : output [batch, channels, seqlen] io_dtype
 *   h_last      : output [batch, channels, state_dim] float32, the state
 *                 after the last token (what the next call or decode step
 *                 starts from; nnterp page, state_output), or NULL. It may
 *                 be the same pointer as h0. With seqlen == 0 it receives
 *                 the initial state.
 *
 * io_dtype holds an ss_dtype value (an int32_t field, so that a caller can
 * pass any integer and get SS_ERR_DTYPE back for a bad one).
 */
typedef struct {
  int64_t batch, channels, state_dim, seqlen;
  int32_t io_dtype;
  const void *x, *dt;
  const void* z;
  const void *B, *C;
  const float* A;
  const float* D;
  const float* dt_bias;
  const float* h0;
  const uint8_t* reset;
  int32_t dt_softplus;
  void* y;
  float* h_last;
} ss_scan_args;

/*
 * The single-token decode update's arguments (ss_state_update).
 *
 *   state       : [batch, channels, state_dim] float32, read and written
 *   x, dt, z, y : [batch, channels]           io_dtype (z NULL = no gate)
 *   B, C        : [batch, state_dim]          io_dtype
 *   A           : [channels, state_dim]       float32
 *   D, dt_bias  : [channels]                  float32, NULL reads as zeros
 *   dt_softplus : as in ss_scan_args
 */
typedef struct {
  int64_t batch, channels, state_dim;
  int32_t io_dtype;
  float* state;
  const void *x, *dt, *z;
  const void *B, *C;
  const float *A, *D, *dt_bias;
  int32_t dt_softplus;
  void* y;
} ss_update_args;

/*
 * Prompt scan (nnterp "selective_scan" page: the scan call
 * (x, dt, A, B, C, D=, z=, delta_bias=) with its channel-first layouts).
 * args must not be NULL (SS_ERR_NULL). batch == 0 or channels == 0 is a
 * no-op returning SS_OK.
 */
ss_status ss_scan_fwd(const ss_scan_args* args, void* stream);

/*
 * The prompt scan of ss_scan_fwd that also returns states of the recurrence
 * (nnterp "selective_scan" page: the `states` attribute, the state after
 * every token of a scan; TransformerLens "ssm_mixer" page: compute_ssm_state,
 * every step or one selected time_step). Every other argument, output and
 * convention is that of ss_scan_fwd, and y and h_last are bitwise those of
 * ss_scan_fwd for the same inputs.
 *
 *   states      : output float32, never NULL:
 *                   time_step < 0: [batch, channels, state_dim, seqlen], the
 *                     state h_t after every token t, seq fastest like x and
 *                     y (element [b, c, n, t] is h_t[n] of row (b, c));
 *                   0 <= time_step < seqlen: [batch, channels, state_dim],
 *                     the state after token time_step.
 *                 It must not overlap any input or y / h_last.
 *   time_step   : see states; time_step >= seqlen is SS_ERR_SHAPE.
 *
 * Writing every state moves 4 * state_dim bytes per channel-token to HBM (the
 * states are 2 * state_dim times the size of a bf16 y), so that form is bound
 * by HBM bandwidth; the single-step form costs about what ss_scan_fwd does.
 */
ss_status ss_scan_fwd_states(const ss_scan_args* args, float* states, int64_t time_step, void* stream);

/*
 * The prompt scan with its input-side producer fused in (nnterp
 * "selective_scan" page, class docstring: the scan's x is the causal conv1d
 * output after SiLU; TransformerLens "ssm_mixer" page: x is the post-conv
 * SiLU input). Here args->x holds x_pre, the conv input, [batch, channels,
 * seqlen] in io_dtype; the kernel forms
 *
 *   x[b, c, t] = silu(conv_b[c] + sum_{k<width} conv_w[c, k] * x_pre[b, c, t - (width-1) + k])
 *
 * in fp32 (not rounded to io_dtype, never written to memory) and scans it,
 * as ss_conv1d_silu followed by ss_scan_fwd would, except that x keeps fp32
 * precision. A tap before position 0 reads 0, and with args->reset so does a
 * tap before the first token of the current document (as ss_conv1d_silu).
 *
 *   conv_w      : [channels, width] float32; width in [1, SS_MAX_CONV_WIDTH]
 *                 (else SS_ERR_UNSUPPORTED)
 *   conv_b      : [channels] float32, or NULL (= 0)
 *
 * Everything else is ss_scan_fwd's: arguments, outputs (conv_w and conv_b
 * must not overlap y or h_last), conventions and errors.
 */
ss_status ss_scan_fwd_conv(const ss_scan_args* args, const float* conv_w, const float* conv_b, int64_t width,
                           void* stream);

/*
 * Single-token decode update of a cached state, in place (nnterp
 * "selective_scan" page: the state-update call
 * (state, x, dt, A, B, C, D, z=, dt_bias=) on one token; the updated state
 * is what the cache receives and y reads it). args must not be NULL
 * (SS_ERR_NULL). batch == 0 or channels == 0 is a no-op returning SS_OK.
 */
ss_status ss_state_update(const ss_update_args* args, void* stream);

/*
 * For measurement: ss_scan_fwd and ss_state_update with a pair of events
 * that the kernel's own dispatch records, start_event when the kernel starts
 * and stop_event when it ends, so that hipEventElapsedTime(start, stop) is
 * the kernel's duration (what a kernel trace reports). An event pair recorded
 * around the call instead also counts the dispatch gap before the kernel
 * (about 1.5 to 3 us on MI355X).
 *
 *   start_event, stop_event : hipEvent_t created by the caller (with timing
 *                 enabled), or NULL (then not recorded); owned by the caller.
 *
 * Everything else is the untimed call's: arguments, outputs, conventions and
 * errors. A call that launches nothing (a zero size) records the events on
 * the stream; a call that returns an error records neither. They are meant
 * for eager timing: stream capture into a HIP graph is supported for the
 * untimed calls only. The events are set for the calling thread during the
 * call, so concurrent timed calls from different threads do not mix.
 */
ss_status ss_scan_fwd_timed(const ss_scan_args* args, void* stream, void* start_event, void* stop_event);
ss_status ss_state_update_timed(const ss_update_args* args, void* stream, void* start_event, void* stop_event);

/*
 * Scalar-gated state scan ("Mamba 2 Gated State Scan" problem page,
 * statement and requirements): per batch item a state S of dk x dv numbers,
 *
 *   S_t = gamma_t * S_{t-1} + k_t v_t^T,     y_t = q_t^T S_t
 *
 * (the output reads the updated state), computed in fp32 with the state in
 * fp32, starting from s0 (zeros when s0 is NULL, as the page starts every
 * batch state).
 *
 *   q, k        : [batch, seqlen, dk]   io_dtype
 *   v           : [batch, seqlen, dv]   io_dtype
 *   gamma       : [batch, seqlen]       float32, each in [0, 1]
 *   s0          : [batch, dk, dv]       state_dtype, or NULL (zeros)
 *   y           : output [batch, seqlen, dv] io_dtype (rounded to nearest even
 *                 for bf16)
 *   final_state : output [batch, dk, dv] state_dtype, the state after the
 *                 last token (s0, or zeros, when seqlen == 0), or NULL. It
 *                 may be the same pointer as s0.
 *
 * The page returns the final state in the dtype of q: state_dtype ==
 * io_dtype gives that; state_dtype == SS_F32 with bf16 I/O keeps the state
 * unrounded, so that a sequence cut into calls (final_state passed back as
 * s0) gives what one call over the whole sequence gives, up to fp32
 * rounding order.
 *
 * dk must be in [1, SS_MAX_GATED_DK] and dv >= 1 (else SS_ERR_UNSUPPORTED).
 * Tensors are contiguous; callers with strided tensors copy them first.
 * batch == 0 is a no-op returning SS_OK. Conventions of the other calls hold
 * (device pointers, asynchronous on `stream`, validation before any launch,
 * inputs untouched, bitwise reproducible).
 */
int ss_gated_scan(int64_t batch, int64_t seqlen, int64_t dk, int64_t dv, int io_dtype, int state_dtype,
                  const void* q, const void* k, const void* v, const float* gamma, const void* s0, void* y,
                  void* final_state, void* stream);

/*
 * Effective attention of the selective scan (TransformerLens "ssm_mixer"
 * page, compute_effective_attention): per batch item b and channel c,
 *
 *   M[b, c, i, j] = sum_n C[b, n, i] * prod_{k=j+1..i} exp(A[c, n] * dt[b, c, k]) * B[b, n, j]
 *
 * for j <= i (the empty product at j == i is 1) and 0 for j > i, in fp32.
 * dt is the scan's step size: softplus(dt + dt_bias) when dt_softplus is
 * nonzero, else dt + dt_bias (dt_bias NULL = 0), as in ss_scan_fwd.
 * include_dt_scaling nonzero multiplies column j by dt[b, c, j], the page's
 * reconstruction form (sum_j M[b, c, i, j] x[b, c, j] + D[c] x[b, c, i] is
 * ss_scan_fwd's output before the gate, from a zero state, without resets).
 * per_state_coord nonzero keeps the terms per state coordinate n instead of
 * summing them.
 *
 *   dt          : [batch, channels, seqlen]       io_dtype
 *   A           : [channels, state_dim]           float32
 *   B, C        : [batch, state_dim, seqlen]      io_dtype
 *   dt_bias     : [channels] float32, or NULL
 *   M           : output float32, [batch, channels, seqlen, seqlen], or
 *                 [batch, channels, state_dim, seqlen, seqlen] with
 *                 per_state_coord; every element is written (zeros above
 *                 the diagonal)
 *
 * The output grows as seqlen^2 (the page meant it for short sequences); its
 * size must fit in int64 bytes (else SS_ERR_SHAPE). state_dim must be in
 * [1, SS_MAX_STATE_DIM]. batch, channels or seqlen == 0 is a no-op returning
 * SS_OK. M must not overlap any input (SS_ERR_ALIAS). Conventions of the
 * other calls hold (device pointers, asynchronous on `stream`, validation
 * before any launch, inputs untouched, bitwise reproducible).
 */
int ss_effective_attention(int64_t batch, int64_t channels, int64_t state_dim, int64_t seqlen, int io_dtype,
                           const void* dt, const float* A, const void* B, const void* C, const float* dt_bias,
                           int dt_softplus, int include_dt_scaling, int per_state_coord, float* M, void* stream);

/*
 * Input side of the scan (nnterp "selective_scan" page, class docstring: the
 * scan's x is the causal conv1d output after SiLU and its dt the dt_proj
 * output; TransformerLens "ssm_mixer" page: x is the post-conv SiLU input).
 *
 * ss_conv1d_silu: depthwise causal convolution of width W over the sequence,
 * then SiLU, in fp32:
 *
 *   x[b, c, t] = silu(conv_b[c] + sum_{k<W} conv_w[c, k] * x_pre[b, c, t - (W-1) + k])
 *
 * A tap before position 0 reads 0, and with a reset mask so does a tap
 * before the first token of the current document (reset[b, s] != 0 marks a
 * document's first token, as in ss_scan_fwd): documents packed in one row do
 * not see each other.
 *
 *   x_pre, x    : [batch, channels, seqlen]  io_dtype (x rounded to nearest
 *                 even for bf16)
 *   conv_w      : [channels, width] float32; width in [1, SS_MAX_CONV_WIDTH]
 *   conv_b      : [channels] float32, or NULL (= 0)
 *   reset       : [batch, seqlen] uint8, or NULL
 */
int ss_conv1d_silu(int64_t batch, int64_t channels, int64_t seqlen, int64_t width, int io_dtype,
                   const void* x_pre, const float* conv_w, const float* conv_b, const uint8_t* reset,
                   void* x, void* stream);

/*
 * ss_dt_proj: the step sizes from the low-rank projection, fp32 accumulation
 * on the matrix cores:
 *
 *   dt[b, c, t] = sum_{k<rank} w_dt[c, k] * delta[b, t, k]
 *
 * and with apply_softplus nonzero dt <- softplus(dt + dt_bias[c]) (dt_bias
 * NULL = 0), the step size ss_scan_fwd would otherwise form (then call the
 * scan with dt_softplus = 0 and no dt_bias).
 *
 *   w_dt        : [channels, rank]          io_dtype
 *   delta       : [batch, seqlen, rank]     io_dtype (token-major, as the
 *                 projection of the tokens produces it)
 *   dt_bias     : [channels] float32, or NULL
 *   dt          : output [batch, channels, seqlen] io_dtype
 *
 * For both calls: rank >= 1 (else SS_ERR_UNSUPPORTED); batch, channels or
 * seqlen == 0 is a no-op returning SS_OK; outputs must not overlap inputs
 * (SS_ERR_ALIAS). Conventions of the other calls hold (device pointers,
 * asynchronous on `stream`, validation before any launch, inputs untouched,
 * bitwise reproducible).
 */
int ss_dt_proj(int64_t batch, int64_t channels, int64_t seqlen, int64_t rank, int io_dtype,
               const void* w_dt, const void* delta, const float* dt_bias, int apply_softplus,
               void* dt, void* stream);

/* Static, NUL-terminated name of a status code (unknown codes included). */
const char* ss_status_str(int status);

/* SS_ABI_VERSION of the built library. */
int ss_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SS_SCAN_H */
