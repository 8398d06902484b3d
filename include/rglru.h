/*
 * rglru.h - C ABI of the MI355X (gfx950) RG-LRU temporal-branch library (librglru.so).
 *
 * The temporal branch of the Griffin/Hawk recurrent block: a causal depthwise Conv1D of
 * temporal width 4 followed by the RG-LRU layer.  Definitions (the Griffin
 * model-architecture page, sections "Recurrent block" and "Real-Gated Linear Recurrent
 * Unit (RG-LRU)", Eq. (1)-(4)), with x_t in the equations read as the conv output u_t:
 *
 *   u_t = conv_b + sum_{k=0..3} conv_w[k] * x_{t-k}          (rounded to the I/O dtype)
 *   r_t = sigma(W_a u_t + b_a)                                (recurrence gate, Eq. 1)
 *   i_t = sigma(W_x u_t + b_x)                                (input gate, Eq. 2)
 *   log a_t = c * r_t * log sigma(Lambda)                     (Eq. 3, in log space)
 *   h_t = a_t * h_{t-1} + sqrt(1 - a_t^2) * (i_t * u_t)       (Eq. 4, diagonal)
 *   y_t = h_t                                                 (rounded to the I/O dtype)
 *
 * Conventions shared by every entry point:
 *   - Row-major, contiguous tensors, last dimension fastest.  B = batch, T = time,
 *     D = D_RNN channels.  x, y, dy are [B,T,D]; W_a, W_x are [D,D] stored [out,in]
 *     (z = W u); conv_w is [4,D] and tap k multiplies x_{t-k}; conv state tensors are
 *     [B,3,D] holding (x_{t-3}, x_{t-2}, x_{t-1}); vectors b_a, b_x, lambda, conv_b are [D].
 *   - The I/O dtype `io` applies to x, conv_w, W_a, W_x, y, the conv state and dy.
 *     Always fp32: b_a, b_x, lambda, conv_b, h0, h_T, the decode state h and every
 *     gradient output.
 *   - Shapes: B >= 1, T >= 1, D >= 64 with D % 64 == 0, B*T*D < 2^31.
 *   - Every pointer is a device pointer, 16-byte aligned, owned by the caller.  The
 *     library never allocates or frees device memory and keeps no state between calls.
 *     Scratch memory is passed in as `ws` of at least the size the matching
 *     *_workspace_bytes query returns.
 *   - No output may alias an input, except the declared in/out state of the decode step.
 *   - Every call is asynchronous on `stream` (0 = the null stream).  Arguments are
 *     validated before any HIP call; invalid arguments return a negative status and
 *     launch nothing.  A launch failure returns RGLRU_EHIP.  Device faults surface at
 *     the caller's next synchronisation.  No C++ exception crosses this interface.
 *   - Calls that share a workspace must not overlap in time.
 *   - Every call runs with the same fixed settings: nothing set by an earlier call changes
 *     a later one.
 */
#ifndef RGLRU_H
#define RGLRU_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RGLRU_OK = 0,
  RGLRU_EINVAL = -1,     /* null required pointer, B/T/D <= 0, misaligned pointer */
  RGLRU_ESHAPE = -2,     /* D % 64 != 0 or B*T*D too large */
  RGLRU_EDTYPE = -3,     /* unknown I/O dtype */
  RGLRU_EWORKSPACE = -4, /* ws null or smaller than the query returns */
  RGLRU_EHIP = -5,       /* a kernel launch or HIP runtime call failed */
  RGLRU_EINTERNAL = -6,
  RGLRU_ESTALL = -7,     /* rglru_workspace_status: a chained-scan wait gave up */
  RGLRU_ESCRATCH = -8    /* allocation-free call: the shape needs more than the fixed scratch */
} rglru_status;

typedef enum { RGLRU_F32 = 0, RGLRU_BF16 = 1 } rglru_dtype;

/* Human-readable name of a status code; never NULL. */
const char* rglru_status_string(int status);

/*
 * Causal depthwise Conv1D, temporal width 4 (the "Recurrent block" section of the
 * Griffin model-architecture page: a small separable Conv1D with 4*D parameters).
 *   u[b,t,d] = RNE_io( b[d] + w[0,d] x[b,t,d] + w[1,d] x[b,t-1,d] + w[2,d] x[b,t-2,d]
 *                      + w[3,d] x[b,t-3,d] ),
 * with x[b,t,d] for t < 0 taken from state_in[b,3+t,d] (zeros when state_in is NULL).
 * The sum is taken in fp64 (bias, then taps 0..3; every product is exact there) and
 * rounded once to the I/O dtype.
 *   x [B,T,D] io; w [4,D] io; b [D] fp32 or NULL (zero); state_in [B,3,D] io or NULL;
 *   u [B,T,D] io (output); state_out [B,3,D] io or NULL: the last three time rows of
 *   [state_in || x].
 */
int conv1d_causal4(int B, int T, int D, rglru_dtype io, const void* x, const void* w,
                   const float* b, const void* state_in, void* u, void* state_out,
                   hipStream_t stream);

/* Workspace bytes rglru_fwd needs for this shape (0 for invalid arguments). */
size_t rglru_fwd_workspace_bytes(int B, int T, int D, rglru_dtype io);

/*
 * Forward of the temporal branch: conv (skipped when conv_w is NULL, then x is already
 * the RG-LRU input), Eq. (1)-(4), y_t = h_t.
 *   c: the scalar constant of Eq. (3) (8 on the pages; any value >= 0 accepted).
 *   conv_b, conv_state_in: as in conv1d_causal4 (nullable).
 *   W_a, W_x [D,D] io ([out,in]); b_a, b_x, lambda [D] fp32.
 *   h0 [B,D] fp32, the state before the first token, or NULL (zeros).
 *   y [B,T,D] io (output).  h_T [B,D] fp32 (output, nullable): the unrounded final
 *   state.  conv_state_out [B,3,D] io (nullable): conv history after the last token
 *   (conv_state_in and conv_state_out are ignored when conv_w is NULL).
 *   Results are bitwise reproducible run to run.
 */
int rglru_fwd(int B, int T, int D, rglru_dtype io, float c, const void* x,
              const void* conv_w, const float* conv_b, const void* conv_state_in,
              const void* W_a, const void* W_x, const float* b_a, const float* b_x,
              const float* lambda, const float* h0, void* y, float* h_T,
              void* conv_state_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes rglru_lru needs (0 for invalid arguments). */
size_t rglru_lru_workspace_bytes(int B, int T, int D, rglru_dtype io);

/*
 * The RG-LRU layer alone (Eq. (1)-(4) of the RG-LRU section) on an input u that is
 * already the conv output: rglru_fwd is conv1d_causal4 followed by rglru_lru on the same
 * stream, and equals rglru_lru when conv_w is NULL.  For bf16 I/O one fused kernel runs
 * the gate GEMM on the matrix cores and the chunked scan in its epilogue (a_t and beta_t
 * never reach HBM), except at shapes whose tiles would fill their last round of compute
 * units poorly, where the gate GEMM and the scan run as two launches (a pure function of
 * B, T, D).  For fp32 I/O both projections run as one GEMM launch and the scan forms
 * a_t and beta_t from them in fp64; scans of fewer than 256 workgroups get them from a
 * launch of their own instead (formed in fp64, rounded once to fp32).
 *   u [B,T,D] io; W_a, W_x [D,D] io; b_a, b_x, lambda [D] fp32; h0 [B,D] fp32 or NULL;
 *   y [B,T,D] io (output); h_T [B,D] fp32 (output, nullable).  Bitwise reproducible.
 */
int rglru_lru(int B, int T, int D, rglru_dtype io, float c, const void* u, const void* W_a,
              const void* W_x, const float* b_a, const float* b_x, const float* lambda,
              const float* h0, void* y, float* h_T, void* ws, size_t ws_bytes,
              hipStream_t stream);

/*
 * The unfused halves of the RG-LRU layer, for callers that produce or consume the gates
 * themselves (together they evaluate what rglru_lru does, to the bar of the I/O dtype).
 *
 * rglru_gates: Eq. (1)-(3) and the input scale of Eq. (4) for every (batch, time) row:
 *   r = sigma(W_a u + b_a), i = sigma(W_x u + b_x), a = exp(c r log sigma(Lambda)),
 *   beta = sqrt(1 - a^2) i.
 *   u [B,T,D] io (the RG-LRU input, i.e. the conv output); W_a, W_x [D,D] io; b_a, b_x,
 *   lambda [D] fp32; a, beta [B,T,D] fp32 (outputs).  No workspace.
 */
int rglru_gates(int B, int T, int D, rglru_dtype io, float c, const void* u, const void* W_a,
                const void* W_x, const float* b_a, const float* b_x, const float* lambda,
                float* a, float* beta, hipStream_t stream);

/* Workspace bytes rglru_scan needs (0 for invalid arguments). */
size_t rglru_scan_workspace_bytes(int B, int T, int D, rglru_dtype io);

/*
 * rglru_scan: the conv (recomputed from x when conv_w is not NULL, as in conv1d_causal4)
 * fused with the diagonal recurrence of Eq. (4): h_t = a_t h_{t-1} + beta_t u_t, y_t = h_t
 * (rounded to io), evaluated as a chunked parallel scan (the blog page "Griffin's
 * Compromise", "Term explanation: Parallel scan").
 *   x [B,T,D] io; conv_w, conv_b, conv_state_in as in rglru_fwd (nullable); a, beta
 *   [B,T,D] fp32 as written by rglru_gates; h0 [B,D] fp32 or NULL; y [B,T,D] io (output);
 *   h_T [B,D] fp32 (output, nullable).  The state is fp32 for bf16 I/O and fp64 for fp32
 *   I/O.  Results are bitwise reproducible run to run.
 */
int rglru_scan(int B, int T, int D, rglru_dtype io, const void* x, const void* conv_w,
               const float* conv_b, const void* conv_state_in, const float* a,
               const float* beta, const float* h0, void* y, float* h_T, void* ws,
               size_t ws_bytes, hipStream_t stream);

/* Workspace bytes rglru_decode_step needs (0 for invalid arguments): the conv output of
 * the step and, for bf16 I/O, the fp32 partial sums of the split gate projection. */
size_t rglru_decode_workspace_bytes(int B, int D, rglru_dtype io);

/*
 * One generation step with the fixed-size state (the blog page "Griffin's Compromise",
 * section "Hawk": generation reads and writes only the current token and a fixed-size
 * state).  Computes rglru_fwd on a length-1 sequence with carried state (the same value
 * up to the fp32 summation order of the gate projection, which is fixed, so repeated
 * calls give identical bits).
 *   x_t [B,D] io; conv_state [B,3,D] io, in/out (shifted in place; ignored when conv_w
 *   is NULL); h [B,D] fp32, in/out (the recurrent state, updated in place);
 *   y_t [B,D] io (output).  Other arguments as in rglru_fwd.
 */
int rglru_decode_step(int B, int D, rglru_dtype io, float c, const void* x_t,
                      const void* conv_w, const float* conv_b, void* conv_state,
                      const void* W_a, const void* W_x, const float* b_a,
                      const float* b_x, const float* lambda, float* h, void* y_t,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * rglru_decode_step for callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The same
 * step and the same results; the scratch the step needs (rglru_decode_workspace_bytes(B, D,
 * io) bytes: the step's conv output, plus the fp32 gate pre-activations for fp32 I/O) lives in
 * a fixed device array of RGLRU_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on until the process ends.  A shape that needs more returns RGLRU_ESCRATCH and
 * launches nothing.  Nothing in the scratch carries over between calls, but every call on
 * one GPU uses the same array: calls that overlap in time on one GPU (two streams, two
 * threads) race and must be serialised by the caller.
 */
#define RGLRU_NOALLOC_SCRATCH_BYTES (32u << 20)
int rglru_decode_step_noalloc(int B, int D, rglru_dtype io, float c, const void* x_t,
                              const void* conv_w, const float* conv_b, void* conv_state,
                              const void* W_a, const void* W_x, const float* b_a,
                              const float* b_x, const float* lambda, float* h, void* y_t,
                              hipStream_t stream);

/* Workspace bytes rglru_bwd needs for this shape (0 for invalid arguments). */
size_t rglru_bwd_workspace_bytes(int B, int T, int D, rglru_dtype io);

/*
 * Backward of rglru_fwd (the pages give no backward; it is the chain rule through the
 * definitions above, with both I/O roundings treated as identity).  The forward is
 * recomputed internally from the same inputs, so nothing is saved between calls.
 *   dy [B,T,D] io: gradient of y.  dh_T [B,D] fp32 or NULL (zero): gradient of h_T.
 *   Outputs, all fp32, all overwritten: dx [B,T,D]; dconv_w [4,D]; dconv_b [D];
 *   dW_a, dW_x [D,D]; db_a, db_x, dlambda [D]; dh0 [B,D] or NULL.
 *   When conv_w is NULL, dx is the gradient of the RG-LRU input and dconv_w, dconv_b
 *   may be NULL (they are not written).
 *   Where sqrt(1 - a_t^2) = 0 its contribution to d(log a_t) is taken as 0.
 *   Reductions over batch and time run in a fixed order: results are bitwise
 *   reproducible run to run.
 */
int rglru_bwd(int B, int T, int D, rglru_dtype io, float c, const void* x,
              const void* conv_w, const float* conv_b, const void* conv_state_in,
              const void* W_a, const void* W_x, const float* b_a, const float* b_x,
              const float* lambda, const float* h0, const void* dy, const float* dh_T,
              float* dx, float* dconv_w, float* dconv_b, float* dW_a, float* dW_x,
              float* db_a, float* db_x, float* dlambda, float* dh0, void* ws,
              size_t ws_bytes, hipStream_t stream);

/*
 * Training forward: rglru_fwd that also keeps what the backward reads (the chain rule
 * through Eq. (1)-(4) needs u_t, r_t, i_t and h_{t-1}), so that rglru_bwd_saved does not
 * evaluate the forward again.  The same launches as the first part of rglru_bwd: u = the
 * conv output, r and i from the gate projection, then the forward scan from (r, i) writing
 * y, h_T and every state h_t.  y matches the oracle to the same tolerance as rglru_fwd's;
 * the two differ in the last bits where rglru_fwd evaluates the gates in another order.
 *   saved: caller-owned device buffer of rglru_train_saved_bytes(B, T, D, io) bytes,
 *   16-byte aligned, written in full (its layout is private to the library: pass it only to
 *   rglru_bwd_saved with the same shape, dtype and inputs).  At 4 x 2048 x 5376 bf16 that
 *   is 0.62 GB: u (io), r and i (fp32), h_t (fp32; fp64 for fp32 I/O).
 *   ws: rglru_fwd_train_workspace_bytes(B, T, D, io) bytes of scratch.
 *   Other arguments as in rglru_fwd; y must not be NULL.
 */
size_t rglru_train_saved_bytes(int B, int T, int D, rglru_dtype io);
size_t rglru_fwd_train_workspace_bytes(int B, int T, int D, rglru_dtype io);
int rglru_fwd_train(int B, int T, int D, rglru_dtype io, float c, const void* x,
                    const void* conv_w, const float* conv_b, const void* conv_state_in,
                    const void* W_a, const void* W_x, const float* b_a, const float* b_x,
                    const float* lambda, const float* h0, void* y, float* h_T,
                    void* conv_state_out, void* saved, size_t saved_bytes, void* ws,
                    size_t ws_bytes, hipStream_t stream);

/*
 * rglru_bwd from the activations rglru_fwd_train kept in `saved` (same shape, dtype and
 * inputs x, conv_w, conv_b, conv_state_in, W_a, W_x, lambda, h0 and c): the forward is not
 * evaluated again, so b_a and b_x are not needed.  The gradients equal rglru_bwd's bit for
 * bit (rglru_bwd evaluates the forward with the same kernels in the same order).
 *   ws: rglru_bwd_saved_workspace_bytes(B, T, D, io) bytes.  saved_bytes smaller than
 *   rglru_train_saved_bytes or saved NULL: RGLRU_EINVAL.  Other arguments as in rglru_bwd.
 */
size_t rglru_bwd_saved_workspace_bytes(int B, int T, int D, rglru_dtype io);
int rglru_bwd_saved(int B, int T, int D, rglru_dtype io, float c, const void* x,
                    const void* conv_w, const float* conv_b, const void* conv_state_in,
                    const void* W_a, const void* W_x, const float* lambda, const float* h0,
                    const void* dy, const float* dh_T, float* dx, float* dconv_w,
                    float* dconv_b, float* dW_a, float* dW_x, float* db_a, float* db_x,
                    float* dlambda, float* dh0, const void* saved, size_t saved_bytes, void* ws,
                    size_t ws_bytes, hipStream_t stream);

/* Workspace bytes rglru_block_fwd needs (0 for invalid arguments). */
size_t rglru_block_fwd_workspace_bytes(int B, int T, int D, int R, rglru_dtype io);

/*
 * Forward of the whole recurrent block around the temporal branch (the Griffin
 * model-architecture page, section "Recurrent block", Fig. 2(c)): the model-width input x
 * goes through two linear layers D -> R (R = D_RNN) in parallel; the first feeds the
 * temporal branch (rglru_fwd), GeLU is applied to the second, the two are multiplied
 * elementwise, and a linear layer R -> D gives the output:
 *   p = RNE_io(x W_in[0:R]^T),  g = RNE_io(GeLU(x W_in[R:2R]^T)),  GeLU(q) = q Phi(q) (exact)
 *   (y, h_T, conv_state_out) = rglru_fwd(p, ...)  with y kept unrounded,
 *   out = RNE_io(RNE_io(y g) W_out^T).
 * The linears have no bias.  For bf16 I/O the products accumulate in fp32 on the matrix
 * cores; for fp32 I/O they accumulate in fp64.
 *   x [B,T,D] io; W_in [2R,D] io ([out,in], the branch rows first, then the GeLU rows);
 *   conv_w [4,R] io or NULL (no conv), conv_b [R] fp32 or NULL, conv_state_in [B,3,R] io
 *   or NULL; W_a, W_x [R,R] io; b_a, b_x, lambda [R] fp32; h0 [B,R] fp32 or NULL;
 *   W_out [D,R] io; out [B,T,D] io (output); h_T [B,R] fp32 (output, nullable);
 *   conv_state_out [B,3,R] io (output, nullable).
 *   Shapes: D % 64 == 0 and R % 64 == 0, B*T*max(D,R) < 2^31; otherwise RGLRU_ESHAPE.
 *   Results are bitwise reproducible run to run.
 */
int rglru_block_fwd(int B, int T, int D, int R, rglru_dtype io, float c, const void* x,
                    const void* W_in, const void* conv_w, const float* conv_b,
                    const void* conv_state_in, const void* W_a, const void* W_x,
                    const float* b_a, const float* b_x, const float* lambda, const float* h0,
                    const void* W_out, void* out, float* h_T, void* conv_state_out, void* ws,
                    size_t ws_bytes, hipStream_t stream);

/* Workspace bytes rglru_block_decode_step needs (0 for invalid arguments). */
size_t rglru_block_decode_workspace_bytes(int B, int D, int R, rglru_dtype io);

/*
 * One generation step of the whole recurrent block (rglru_block_fwd on a length-1 sequence
 * with the carried state; the blog page "Griffin's Compromise", section "Hawk": generation
 * reads and writes only the current token and a fixed-size state): the input linears on
 * x_t, the branch's decode step (rglru_decode_step) on p with the state updated in place,
 * z = RNE_io(h g), out_t = RNE_io(z W_out^T).  Run over the tokens after an
 * rglru_block_fwd prefill whose h_T and conv_state_out seed (h, conv_state), it continues
 * that forward (to fp32 summation order).
 *   x_t [B,D] io; conv_state [B,3,R] io in/out (ignored when conv_w is NULL); h [B,R] fp32
 *   in/out; out_t [B,D] io (output); the weights as in rglru_block_fwd.
 *   Repeated calls give identical bits.
 */
int rglru_block_decode_step(int B, int D, int R, rglru_dtype io, float c, const void* x_t,
                            const void* W_in, const void* conv_w, const float* conv_b,
                            void* conv_state, const void* W_a, const void* W_x, const float* b_a,
                            const float* b_x, const float* lambda, float* h, const void* W_out,
                            void* out_t, void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes gated_mlp_fwd needs (0 for invalid arguments). */
size_t gated_mlp_fwd_workspace_bytes(int B, int T, int D, int MD, rglru_dtype io);

/*
 * Forward of the gated MLP block (the Griffin model-architecture page, section "MLP block",
 * Fig. 2(b)): two linear layers D -> MD on the same input (MD = M*D, expansion M = 3 on
 * the pages), GeLU on the first branch, an elementwise product, and a linear layer MD -> D:
 *   h = RNE_io( GeLU(x W_1^T) * (x W_2^T) ),  GeLU(q) = q Phi(q) (exact),
 *   out = RNE_io( h W_3^T ).
 * No biases.  The two branch outputs are not rounded on their own (for bf16 I/O they stay in
 * the fp32 accumulators of one matrix-core GEMM whose epilogue forms h).
 *   x [B,T,D] io; W_1, W_2 [MD,D] io ([out,in]); W_3 [D,MD] io; out [B,T,D] io (output).
 *   Shapes: D % 64 == 0, MD % 64 == 0, B*T*max(D,MD) < 2^31; otherwise RGLRU_ESHAPE.
 *   Results are bitwise reproducible run to run.
 */
int gated_mlp_fwd(int B, int T, int D, int MD, rglru_dtype io, const void* x, const void* W_1,
                  const void* W_2, const void* W_3, void* out, void* ws, size_t ws_bytes,
                  hipStream_t stream);

/* Workspace bytes local_mqa_fwd needs (0 for invalid arguments). */
size_t local_mqa_fwd_workspace_bytes(int B, int T, int D, rglru_dtype io);

/*
 * Forward of the local (sliding-window) multi-query attention block (the Griffin
 * model-architecture page, sections "Global multi-query attention" and "Local sliding-window
 * attention"; window 1024 on the blog page "Griffin's Compromise", section "Griffin:
 * Attention for Recent Memory"): H = D / 128 query heads of width 128 share one key head
 * and one value head; RoPE (no absolute position embedding); query t attends to the keys at
 * the `window` most recent positions up to and including its own:
 *   [q k v] = x [W_q; W_k; W_v]^T,  q [.., H, 128] and k rotated by RoPE at the absolute
 *   position pos0 + t (pair (2i, 2i+1) by the angle pos * 10000^(-2i/128)), rounded to io;
 *   a_t = sum_{s in (t - window, t]} softmax_s(q_t . k_s / sqrt(128)) v_s, per head,
 *   rounded to io;  out = RNE_io(a W_o^T).
 * No biases.  For bf16 I/O the projections and both attention products run on the matrix
 * cores with fp32 accumulation and an online softmax in fp32; for fp32 I/O the projections
 * accumulate in fp64 and the attention is evaluated in fp64.
 *   x [B,T,D] io; W_qkv [D + 256, D] io ([out,in]: the D rows of W_q, then the 128 rows of
 *   W_k, then the 128 rows of W_v); W_o [D,D] io; out [B,T,D] io (output);
 *   k_out, v_out [B,T,128] io (outputs, nullable): the rotated keys and the values, i.e.
 *   the key/value cache content of these positions.
 *   window >= 1; pos0 >= 0 is the absolute position of the first token (RoPE only: the
 *   attention sees the T tokens of this call).
 *   Shapes: D % 128 == 0, B*T*(D+256) < 2^31; otherwise RGLRU_ESHAPE.
 *   Results are bitwise reproducible run to run.
 */
int local_mqa_fwd(int B, int T, int D, rglru_dtype io, int window, int pos0, const void* x,
                  const void* W_qkv, const void* W_o, void* out, void* k_out, void* v_out,
                  void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes local_mqa_decode_step needs (0 for invalid arguments). */
size_t local_mqa_decode_workspace_bytes(int B, int D, rglru_dtype io);

/*
 * One generation step of the local-MQA block with a bounded key/value cache (the Griffin
 * model-architecture page, section "Local sliding-window attention": the cache is limited
 * to the window).  Each sequence b has a cache of `window` slots; slot j holds the rotated
 * key and the value of the most recent position p <= pos[b] with p % window == j.  The step
 * computes q, k, v of the token x_t[b] at absolute position pos[b] exactly as local_mqa_fwd
 * does, writes k and v into slot pos[b] % window, attends over the cached positions
 * (pos[b] - window, pos[b]] (slots 0 .. min(pos[b], window - 1)) and applies W_o.  Run over
 * positions 0, 1, 2, ... from an empty cache it reproduces local_mqa_fwd (to fp32
 * summation order); a prefill hands over by writing local_mqa_fwd's k_out/v_out rows of the
 * last `window` positions into their slots.
 *   pos [B] int32, device memory, read by the kernels (a negative position is taken as 0);
 *   x_t [B,D] io; W_qkv [D + 256, D] and W_o [D,D] io as in local_mqa_fwd;
 *   k_cache, v_cache [B, window, 128] io, in/out (one slot written per sequence);
 *   out [B,D] io (output).
 *   Shapes: D % 128 == 0, B*window*128 < 2^31.  Repeated calls give identical bits.
 */
int local_mqa_decode_step(int B, int D, rglru_dtype io, int window, const int* pos, const void* x_t,
                          const void* W_qkv, const void* W_o, void* k_cache, void* v_cache,
                          void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Status of the chained scans of the last call that ran on the workspace `ws` (a workspace
 * of rglru_fwd, rglru_lru, rglru_scan, rglru_bwd or rglru_block_fwd, which all start with
 * the same counter words).  Chunks of a chained scan (the blog page "Griffin's Compromise",
 * "Term explanation: Parallel scan") wait for the summary of their predecessor chunk; that
 * wait is bounded, and one that gives up writes NaN where the carry was needed instead of
 * hanging.  Returns RGLRU_ESTALL if any wait of that call gave up, RGLRU_OK otherwise.
 * Synchronous: copies one word to the host on `stream` and waits for the stream.
 */
int rglru_workspace_status(const void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RGLRU_H */
