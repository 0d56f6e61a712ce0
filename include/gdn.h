/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet token-mixer library.
 *
 * The operation is the GDN layer of "The Key to Going Linear: Analysis-Driven
 * Transformer Linearization" (Kuzina, Whatmough, Ehteshami Bejnordi):
 *   section 3.1.2:  S_t = (I - beta_t k_t k_t^T) G_t S_{t-1} + beta_t k_t v_t^T,
 *                   y_t = q_t^T S_t,
 * with a scalar gate G_t = alpha_t I per (token, head), a key-major fp32 state
 * S in R^{Dk x Dv}, and the read-out taken after token t is written:
 *   out_t = scale * S_t^T q_t.
 * Section 4 adds a disjoint softmax path over sink tokens and a sliding window
 * ("Adding Sliding Window Attention") and causal short convolutions on q, k, v
 * ("Adapting Q/K/V").
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees or synchronises; every call is enqueued on `stream`
 *     (a hipStream_t; NULL = the default stream) and returns immediately.
 *   - Tensors are dense row-major.  Token tensors are [B, T, H, D] (the
 *     natural output of a [B, T, H*D] projection); states are [B, H, Dk, Dv]
 *     float32; gates alpha/beta are [B, T, H] float32.
 *   - `dtype` (gdn_dtype) is the element type of the token inputs (q, k, v,
 *     x, KV caches): GDN_BF16 (bfloat16) or GDN_F32.  `out_dtype` is the
 *     element type of `out` / `y`: the input dtype, or GDN_F32 with bf16
 *     inputs (f32 results of bf16 inputs; a bf16 output is exactly that f32
 *     result rounded once to nearest-even).  Gates, states and taps are
 *     always f32.  In bf16 mode all arithmetic accumulates in f32 and the
 *     matrix products take 16-bit operands (bf16, or f16: bf16 values convert
 *     to f16 exactly when their magnitude lies in f16's normal range,
 *     2^-14 .. 65504, intermediates are rounded to f16); in f32 mode every
 *     product is f32.
 *   - Token/state pointers must be 16-byte aligned.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     failed check returns GDN_ERR_INVALID_ARG or GDN_ERR_UNSUPPORTED and
 *     enqueues nothing; a launch failure returns GDN_ERR_HIP.  The message of
 *     the last failure on the calling thread is gdn_last_error().  Faults
 *     inside a kernel surface at the caller's next synchronisation.
 *   - Data-dependent preconditions are documented, not checked: alpha in
 *     (0, 1], beta in [0, 1], q and k of moderate norm (the workloads
 *     L2-normalise them per token).  In bf16 mode the prefills' products
 *     take f16 operands, so v, the state and the chunk intermediates must
 *     stay below 65504 in magnitude: a value beyond it becomes +-inf in its
 *     operand and the outputs are not finite (q and k convert rounding
 *     toward zero and clip at +-65504 instead); magnitudes below 2^-14 keep
 *     fewer bits.  With unit-norm keys and beta in [0, 1] the erase keeps
 *     every state entry within the sum of the |beta v| written into it.  The
 *     decode steps and the f32 mode have no such limit.
 *   - Calls are thread-safe; there is no mutable global state besides the
 *     per-thread error message, and the static scratch of
 *     gdn_prefill_chunked_noalloc (with its per-device address, set once).
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1, /* NULL pointer, bad size, misalignment, too small */
  GDN_ERR_UNSUPPORTED = 2, /* valid request outside the supported shapes     */
  GDN_ERR_HIP = 3          /* a HIP runtime call failed                       */
} gdn_status;

typedef enum { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

/* ABI version of this header (incremented on any signature change). */
#define GDN_ABI_VERSION 1
int gdn_abi_version(void);

/* Message of the last failed call on this thread ("" if none). */
const char* gdn_last_error(void);

/*
 * Workspace (bytes) that gdn_prefill_chunked needs for these sizes.
 *   - bf16 inputs, Dk = Dv = 128, chunk = 64: 0 when one pass per head fills
 *     the GPU; with few (batch, head) pairs and long sequences the sequence
 *     is split into P segments, and the workspace holds, per head, the f32
 *     128 x 128 state maps of the first P - 1 segments and their initial
 *     states (3 (P - 1) x 64 KiB).
 *   - otherwise: per chunk of `chunk` tokens, the chunk's triangular-solve
 *     matrix, its decay-masked query-key products and its cumulative log
 *     gates.
 * Also 0 if the sizes are invalid.
 */
size_t gdn_prefill_workspace_bytes(int B, int T, int H, int Dk, int Dv,
                                   int chunk, int dtype);

/*
 * Chunk-parallel GDN prefill (section 3.1.2 recurrence, computed exactly up
 * to rounding by a chunked WY/UT rewrite).  Equivalent to running the
 * recurrence token by token over t = 0..T-1 for every (b, h):
 *   q, k      [B, T, H, Dk]  dtype      alpha, beta [B, T, H]  f32
 *   v         [B, T, H, Dv]  dtype      out         [B, T, H, Dv] out_dtype
 *   state_in  [B, H, Dk, Dv] f32, or NULL for a zero initial state
 *   state_out [B, H, Dk, Dv] f32, or NULL; may alias state_in (resume)
 *   scale     multiplies every read-out (1.0 for the page's y_t = q_t^T S_t)
 *   chunk     16, 32 or 64 tokens per chunk (a tuning choice: the result is
 *             the same recurrence for any chunk, up to rounding)
 *   workspace device scratch of at least gdn_prefill_workspace_bytes(...)
 *             bytes, 256-byte aligned; may be NULL when that size is 0
 * Limits: B >= 0, T >= 0, H >= 1, Dk and Dv in {16, 32, 64, 128}.  T = 0
 * copies state_in (or zeros) to state_out.  alpha must be > 0 (the kernels
 * work with log alpha).
 */
gdn_status gdn_prefill_chunked(const void* q, const void* k, const void* v,
                               const float* alpha, const float* beta,
                               const float* state_in, float* state_out, void* out,
                               int B, int T, int H, int Dk, int Dv, int chunk,
                               int dtype, int out_dtype, float scale, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * gdn_prefill_chunked without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments (minus workspace and
 * workspace_bytes), same results (the same kernels run): the scratch they
 * need comes from a static device array of GDN_NOALLOC_SCRATCH_BYTES in the
 * library, one copy per GPU, held until the process ends.  The call itself
 * allocates nothing; its first call on a device, with that device current,
 * looks up the array's device address (hipGetSymbolAddress) and keeps it.
 *   - Sizes whose gdn_prefill_workspace_bytes(...) exceeds
 *     GDN_NOALLOC_SCRATCH_BYTES return GDN_ERR_UNSUPPORTED and enqueue
 *     nothing (use gdn_prefill_chunked with a workspace).
 *   - `stream` must belong to the current device.
 *   - Every call on one GPU shares that GPU's scratch and leaves its contents
 *     behind (nothing in it needs to start at zero): calls that can run at
 *     the same time on one GPU (other streams, other threads) race and give
 *     wrong results; order them on one stream.
 */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)
gdn_status gdn_prefill_chunked_noalloc(const void* q, const void* k, const void* v,
                                       const float* alpha, const float* beta,
                                       const float* state_in, float* state_out,
                                       void* out, int B, int T, int H, int Dk, int Dv,
                                       int chunk, int dtype, int out_dtype, float scale,
                                       void* stream);

/*
 * gdn_prefill_chunked on the raw q, k, v projections, with the projection
 * adaptation of section 4 ("Adapting Q/K/V") done inside the prefill's tile
 * loads: per head and channel c, with x the raw projection and K = 4,
 *   q_t = n(SiLU(sum_j taps_q[c][j] * xq_{t-3+j}[c])),  likewise k with taps_k
 *   v_t =   SiLU(sum_j taps_v[c][j] * xv_{t-3+j}[c])
 *   x_{<0} = 0 (every sequence starts with an empty convolution history),
 *   n(y) = y / (||y||_2 + conv_eps) over the head's Dk channels (the key
 *   normalisation of appendix B.1, "Metric 1"), then the recurrence exactly
 *   as gdn_prefill_chunked on those q, k, v.  The convolution, SiLU and
 *   norm run in f32 and their results go to the MFMA operands in f16 once:
 *   they are never rounded to bf16 nor written to memory.
 *   xq, xk, xv [B, T, H, 128] bf16 (the projections, channels of a head
 *              consecutive: the [B, T, H * 128] layout of gdn_short_conv_silu)
 *   taps_q, taps_k, taps_v [H * 128, conv_kernel] f32; taps[c][3] multiplies
 *              the current token
 *   conv_eps   >= 0 (0 gives NaN for an all-zero convolution output)
 *   everything else as gdn_prefill_chunked (same workspace size).
 * Limits: dtype GDN_BF16, Dk = Dv = 128, chunk = 64, conv_kernel = 4
 * (otherwise GDN_ERR_UNSUPPORTED).  The SiLU outputs of q and k are
 * normalised, so the f16 operand range holds for them; v's SiLU output must
 * stay below 65504 in magnitude, as gdn_prefill_chunked's v.
 */
gdn_status gdn_prefill_chunked_conv(const void* xq, const void* xk, const void* xv,
                                    const float* taps_q, const float* taps_k,
                                    const float* taps_v, int conv_kernel,
                                    float conv_eps, const float* alpha,
                                    const float* beta, const float* state_in,
                                    float* state_out, void* out, int B, int T, int H,
                                    int Dk, int Dv, int chunk, int dtype,
                                    int out_dtype, float scale, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * One recurrence step for a batch of sequences (section 3.1.2 at a single
 * token; the recurrent form used for generation):
 *   q, k [B, H, Dk] dtype;  v [B, H, Dv] dtype;  alpha, beta [B, H] f32
 *   state_in, state_out [B, H, Dk, Dv] f32 (may alias: in-place update)
 *   out [B, H, Dv] out_dtype:   out = scale * S'^T q
 * Each state is read once and written once.  Limits as for the prefill.
 */
gdn_status gdn_decode_step(const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta,
                           const float* state_in, float* state_out, void* out, int B,
                           int H, int Dk, int Dv, int dtype, int out_dtype,
                           float scale, void* stream);

/*
 * Causal depthwise short convolution + SiLU on one projection output
 * (section 4, "Adapting Q/K/V"), optionally followed by an L2 normalisation
 * of every group of `l2norm_group` consecutive channels (one head), as the
 * key normalisation k / (||k||_2 + eps) of appendix B.1:
 *   x [B, T, Ch] dtype, y [B, T, Ch] out_dtype;  taps [Ch, K] f32,
 *   taps[c][K-1] multiplies x_t
 *   y_t[c] = SiLU(sum_j taps[c][j] * x_{t-K+1+j}[c]),  x_{<0} = 0
 * Limits: K in 1..8; Ch a multiple of 8; l2norm_group 0 (off) or a power of
 * two in 8..512 dividing Ch.  y must not overlap x.
 */
gdn_status gdn_short_conv_silu(const void* x, const float* taps, void* y, int B,
                               int T, int Ch, int K, int l2norm_group, float eps,
                               int dtype, int out_dtype, void* stream);

/*
 * One decode step of the same short convolution (section 4, "Adapting
 * Q/K/V": the causal convolution evaluated at one new token), for callers
 * that generate token by token.  For every sequence b and channel c:
 *   a = sum_{j<K-1} taps[c][j] * conv_state[b][j][c] + taps[c][K-1] * x[b][c]
 *   y[b][c] = SiLU(a)  (then the optional group L2 normalisation)
 * and conv_state[b] becomes rows 1 .. K-2 of itself followed by x[b].
 *   x          [B, Ch] dtype: the new token's projection output
 *   taps       [Ch, K] f32, as in gdn_short_conv_silu
 *   conv_state [B, K-1, Ch] dtype, caller-owned, updated in place: the
 *              previous K-1 inputs, oldest first (zeros before the first
 *              token).  After gdn_short_conv_silu over tokens 0 .. T-1 the
 *              matching state is x_{T-K+1} .. x_{T-1} (rows before token 0
 *              are zero).  May be NULL when K = 1.
 *   y          [B, Ch] out_dtype
 * Limits as gdn_short_conv_silu.  x, y and conv_state must not overlap.
 */
gdn_status gdn_short_conv_step(const void* x, const float* taps, void* conv_state,
                               void* y, int B, int Ch, int K, int l2norm_group,
                               float eps, int dtype, int out_dtype, void* stream);

/*
 * Softmax decode step over sink tokens and a sliding window (section 4,
 * "Adding Sliding Window Attention": I = sinks + window, logits scaled by
 * softmax_scale, normally 1/sqrt(D)).
 *   q        [B, H, D] dtype: the current token's softmax-path query
 *   k_cache, v_cache [B, H, n_sink + window, D] dtype.  Slot i < n_sink holds
 *            the token at 0-based position i; the token at position p >=
 *            n_sink lives in slot n_sink + (p - n_sink) % window.
 *   n_tokens [B] int32 (device): tokens seen including the current one, so
 *            the current token is at position n_tokens[b] - 1 (>= 0 required,
 *            n_tokens[b] >= 1).  The attended set is positions
 *            {0..min(n_sink, t)-1} and {max(n_sink, t-window)..t-1}, t =
 *            n_tokens[b]; each position at most once.
 *   k_new, v_new [B, H, D] dtype or both NULL: when given, the current
 *            token's key/value are first stored into its cache slot (this
 *            overwrites the token leaving the window) and attended from there.
 *   accumulate 0: out = y_swa; 1: out += y_swa (adds to the linear path's
 *            read-out written earlier on the same stream).
 *   out      [B, H, D] out_dtype.
 * Limits: D in {64, 128}; n_sink >= 0; window >= 1.
 */
gdn_status gdn_swa_sink_decode(const void* q, const void* k_new, const void* v_new,
                               void* k_cache, void* v_cache, const int* n_tokens,
                               int B, int H, int D, int n_sink, int window,
                               float softmax_scale, int accumulate, void* out,
                               int dtype, int out_dtype, void* stream);

/*
 * Softmax over sink tokens and a sliding window at every position of a
 * sequence (section 4, "Adding Sliding Window Attention", in prefill form):
 * position t (0-based) attends to I_t = {0 .. n_sink-1} u {t-window+1 .. t},
 * each position at most once, with logits softmax_scale * q_t . k_i.
 *   q, k, v  [B, T, H, D] dtype: the softmax path's own projections
 *   out      [B, T, H, D] out_dtype.  Rows t >= accumulate_from add the
 *            result (out += y), rows below it are overwritten: pass T (or
 *            more) for a plain write, 0 to add to every row.
 * Limits: dtype GDN_BF16 and D = 128 (else GDN_ERR_UNSUPPORTED); n_sink >= 0;
 * window >= 1; softmax_scale > 0 and finite.  out must not overlap q, k or v.
 */
gdn_status gdn_swa_sink_prefill(const void* q, const void* k, const void* v, void* out, int B,
                                int T, int H, int D, int n_sink, int window, float softmax_scale,
                                int accumulate_from, int dtype, int out_dtype, void* stream);

/*
 * Fill the decode-time KV cache of gdn_swa_sink_decode from a sequence's
 * keys and values (section 4: the cache keeps the sinks and the window):
 *   k, v     [B, T, H, D] dtype
 *   k_cache, v_cache [B, H, n_sink + window, D] dtype, caller-owned.  Slot
 *            i < n_sink gets position i (i < T); position p >= n_sink, for the
 *            last `window` such positions before T, goes to slot
 *            n_sink + (p - n_sink) % window.  Other slots are left untouched.
 * After it, gdn_swa_sink_decode with n_tokens = T + 1 attends the right set.
 * Limits: D in {64, 128}; n_sink >= 0; window >= 1.
 */
gdn_status gdn_swa_cache_fill(const void* k, const void* v, void* k_cache, void* v_cache, int B,
                              int T, int H, int D, int n_sink, int window, int dtype, void* stream);

/*
 * Workspace (bytes) that gdn_hybrid_prefill needs for these sizes (0 = none;
 * reusable across calls on one stream).  0 for unsupported sizes.
 */
size_t gdn_hybrid_prefill_workspace_bytes(int B, int T, int H, int D, int n_sink, int window);

/*
 * The whole hybrid layer over a sequence (section 4, "Adding Sliding Window
 * Attention": the linear state holds exactly the tokens in neither the sinks
 * nor the window, and the two read-outs are added without weights):
 *   out_t = lin_scale * S_lin(t)^T q_lin_t + y^swa_t,
 * where S_lin(t) is the section 3.1.2 state over tokens n_sink .. t-window
 * (0-based; S = 0 when that set is empty) and y^swa is gdn_swa_sink_prefill.
 *   q_lin, k_lin, v_lin [B, T, H, D] dtype and alpha, beta [B, T, H] f32: the
 *            linear path's inputs (token j enters the state with its own
 *            alpha_j, beta_j, k_j, v_j when it leaves the window)
 *   q_swa, k_swa, v_swa [B, T, H, D] dtype: the softmax path's inputs
 *   state_out [B, H, D, D] f32 or NULL: the linear state after the sequence
 *            (tokens n_sink .. T-1-window), the state the next decode step
 *            starts from (that step inserts token T - window with
 *            gdn_decode_step before reading it)
 *   out      [B, T, H, D] out_dtype
 *   k_cache, v_cache [B, H, n_sink + window, D] dtype, or both NULL: filled
 *            as by gdn_swa_cache_fill for the decode steps that follow
 *   workspace: gdn_hybrid_prefill_workspace_bytes(...) bytes, 256-byte
 *            aligned (NULL allowed when that is 0)
 * Enqueues the linear path (one chunked prefill over all sequences, reading
 * them as strided views), then the softmax path adding into out, then the
 * cache fill.  softmax_scale > 0 and finite.  With a bf16 out, the
 * linear read-out is stored as bf16 first and the sum is rounded once more
 * (as in the decode pair gdn_decode_step + gdn_swa_sink_decode with
 * accumulate = 1); an f32 out rounds neither.  Limits: dtype
 * GDN_BF16 and D = 128 (else GDN_ERR_UNSUPPORTED).  No output may overlap
 * an input.
 */
gdn_status gdn_hybrid_prefill(const void* q_lin, const void* k_lin, const void* v_lin,
                              const float* alpha, const float* beta, const void* q_swa,
                              const void* k_swa, const void* v_swa, float* state_out, void* out,
                              void* k_cache, void* v_cache, int B, int T, int H, int D, int n_sink,
                              int window, float lin_scale, float softmax_scale, int dtype,
                              int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Channel-wise gate (section 3.2's diagonal gates prod_j diag(alpha_j) in
 * the section 3.1.2 update): G_t = diag(alpha_t) with alpha_t in R^{Dk} per
 * (token, head), applied to the rows of the key-major state BEFORE the erase,
 * in the page's order (for a diagonal gate the order matters):
 *   S_t = (I - beta_t k_t k_t^T) diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *   out_t = scale * S_t^T q_t.
 * gdn_prefill_chunked_chgate: the same call as gdn_prefill_chunked with
 *   alpha [B, T, H, Dk] f32 (every entry in (0, 1]; the prefill works with
 *   log alpha; 16-byte aligned), chunks of 32 tokens.  f32 inputs: f32
 *   arithmetic throughout.  bf16 inputs: the per-chunk pass in f32, the
 *   recurrence's products with f16 operands and f32 accumulation (state f32).
 *   workspace: gdn_prefill_chgate_workspace_bytes(B, T, H) bytes, 256-byte
 *   aligned.  state_out may alias state_in.  Limits: Dk and
 *   Dv in {32, 64, 128}.
 * gdn_decode_step_chgate: the same call as gdn_decode_step with alpha
 *   [B, H, Dk] f32.  Limits as gdn_decode_step.
 */
size_t gdn_prefill_chgate_workspace_bytes(int B, int T, int H);
gdn_status gdn_prefill_chunked_chgate(const void* q, const void* k, const void* v,
                                      const float* alpha, const float* beta, const float* state_in,
                                      float* state_out, void* out, int B, int T, int H, int Dk, int Dv,
                                      int dtype, int out_dtype, float scale, void* workspace,
                                      size_t workspace_bytes, void* stream);
gdn_status gdn_decode_step_chgate(const void* q, const void* k, const void* v, const float* alpha,
                                  const float* beta, const float* state_in, float* state_out,
                                  void* out, int B, int H, int Dk, int Dv, int dtype, int out_dtype,
                                  float scale, void* stream);

/*
 * Gated linear attention with a key-dependent gate (kGLA, section 3.2.2,
 * "Gated Linear Attention with Key-Dependent Gate"):
 *   y_t = sum_{i<=t} ( q_t^T [prod_{j=i+1}^{t} diag(alpha_j)
 *                               (I - beta_j Diag(k_j o k_j))] k_i ) v_i,
 * i.e. the state update S_t = diag(alpha_t o (1 - beta_t k_t o k_t)) S_{t-1}
 * + k_t v_t^T with out_t = scale * S_t^T q_t read after the write.  The
 * diagonal erase Diag(k o k) stands in for the delta rule's rank-1 k k^T; the
 * write carries no step size (the printed sum has none).  Arguments, layouts,
 * limits and workspace (gdn_prefill_chgate_workspace_bytes) as for
 * gdn_prefill_chunked_chgate: alpha [B, T, H, Dk] f32, beta [B, T, H] f32.
 * Precondition (documented, not checked): alpha in (0, 1], beta in [0, 1]
 * and beta k[c]^2 < 1 for every channel (the kernels work with the log of
 * the gate, which must be positive).
 */
gdn_status gdn_prefill_chunked_kgla(const void* q, const void* k, const void* v,
                                    const float* alpha, const float* beta,
                                    const float* state_in, float* state_out, void* out,
                                    int B, int T, int H, int Dk, int Dv, int dtype,
                                    int out_dtype, float scale, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * One kGLA step per (b, h) (section 3.2.2 at a single token):
 *   S' = diag(alpha o (1 - beta k o k)) S + k v^T,   out = scale * S'^T q;
 * q, k, alpha [B, H, Dk]; v [B, H, Dv]; beta [B, H]; states as for
 * gdn_decode_step_chgate (may alias).  No precondition on the gate's sign:
 * the step multiplies by it directly.
 */
gdn_status gdn_decode_step_kgla(const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, const float* state_in, float* state_out,
                                void* out, int B, int H, int Dk, int Dv, int dtype, int out_dtype,
                                float scale, void* stream);

/*
 * Backward pass of gdn_prefill_chunked (scalar gate; section 3.1.2 update,
 * trained through as in section 3.3): for an output gradient dout and an
 * optional gradient dstate_out of the final state, the gradients of the
 * inputs by the adjoint of the token loop,
 *   G_t = scale q_t dout_t^T + A_{t+1} G_{t+1},  A_t = alpha_t (I - beta_t k_t k_t^T),
 *   dq_t = scale S_t dout_t, dv_t = beta_t G_t^T k_t,
 *   dk_t = -alpha_t beta_t (G_t p_t + S_{t-1} G_t^T k_t) + beta_t G_t v_t,
 *   dalpha_t = <G_t, S_{t-1}> - beta_t (G_t^T k_t).p_t,
 *   dbeta_t = (G_t^T k_t).(v_t - alpha_t p_t),  p_t = S_{t-1}^T k_t,
 *   dstate_in = A_0 G_0.
 *   q, k [B,T,H,Dk], v [B,T,H,Dv] dtype; alpha, beta [B,T,H] f32;
 *   state_in [B,H,Dk,Dv] f32 or NULL (zeros); dout [B,T,H,Dv] f32;
 *   dstate_out [B,H,Dk,Dv] f32 or NULL (zeros).
 *   Outputs (f32, caller-owned): dq, dk [B,T,H,Dk], dv [B,T,H,Dv],
 *   dalpha, dbeta [B,T,H], dstate_in [B,H,Dk,Dv].
 *   workspace: gdn_prefill_backward_workspace_bytes(B, T, H, Dk, Dv) bytes,
 *   256-byte aligned; its contents are scratch (overwritten by every call).
 * Dk = Dv = 128 takes the chunked reverse mode (chunks of 64 tokens, every
 * product on f32 MFMA): a per-chunk pass (gates, Gram matrices, triangular
 * inverse), a forward pass over the chunks storing the state entering each,
 * a reverse pass carrying the state gradient, and a per-chunk pass forming
 * dq, dk, dalpha, dbeta; the workspace holds ~304 KiB per (b, h, chunk).
 * Other head sizes take the token loop above directly: one work-group per
 * (b, h, slice of 32 state columns) with the state every 4 tokens in the
 * workspace and per-slice partials summed by a second kernel.  Both forms
 * are f32 throughout and sum in a fixed order (deterministic results).
 * Limits: Dk and Dv in {16, 32, 64, 128}.
 */
size_t gdn_prefill_backward_workspace_bytes(int B, int T, int H, int Dk, int Dv);
gdn_status gdn_prefill_backward(const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, const float* state_in, const float* dout,
                                const float* dstate_out, float* dq, float* dk, float* dv,
                                float* dalpha, float* dbeta, float* dstate_in, int B, int T, int H,
                                int Dk, int Dv, int dtype, float scale, void* workspace,
                                size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
