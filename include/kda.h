/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) library.
 *
 * What is computed (definitions from the pages):
 *  - "Kimi K3: Bounded Decay and Delta Memory" (PaperLeet), section "Formula
 *    and conventions": the bounded per-channel gate
 *        g = g_min * sigmoid(e^A * z),   alpha = e^g   (alpha in [e^g_min, 1]),
 *    and the per-token recurrence
 *        Sbar_t = Diag(alpha_t) S_{t-1}
 *        S_t    = Sbar_t + beta_t k_t (v_t - k_t^T Sbar_t)^T
 *        o_t    = scale * S_t^T q_t          (scale = 1 leaves q unscaled, as the contract has it).
 *  - KDA cheat sheet, "Chunkwise parallel form": the same recurrence evaluated
 *    chunk by chunk (serial from one chunk to the next, parallel inside a chunk); and the
 *    gate table: g >= -5 bounds the cumulative log-decay of a 16-token tile by
 *    -80, which keeps every rescale factor of the chunk kernel finite.
 *  - "Kept memory" page: the per-head state is kept between calls and a decode
 *    call updates it with one new token.
 *
 * Conventions for every entry point:
 *  - Every pointer argument is a DEVICE pointer, except where stated.  The caller
 *    owns every buffer; the library never allocates, never synchronises and never
 *    prints.  Work is enqueued on `stream` (NULL = the default stream) and the
 *    call returns as soon as it is enqueued.
 *  - Tensors are dense, row-major, innermost dimension last.  Token tensors are
 *    [B, T, H, D] (q, k, gate: D = K; v, out: D = V); beta is [B, T, H]; states
 *    are [N, H, K, V] (key rows, value columns: the pages' key-by-value
 *    orientation).  Element types are given by the kda_dtype arguments; gate,
 *    beta and states are always float32.
 *  - Inputs are never written.  Outputs must not overlap any input (checked for
 *    the obvious cases: equal base pointers -> KDA_ERR_ALIAS).
 *  - Errors are returned synchronously from host-side validation, before anything
 *    is enqueued; KDA_ERR_HIP means the launch itself failed.  Faults inside a
 *    kernel surface, as usual for HIP, at the caller's next synchronisation.
 *  - Preconditions not checked on the device: finite inputs.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 1: gate, chunk and step entry points; 2: adds the fused-gate variants and the
 * token-recurrent prefill; 3: adds the backward (kda_chunk_bwd, kda_bounded_decay_bwd) */
#define KDA_ABI_VERSION 4

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
    KDA_ERR_BAD_SHAPE = 2,    /* a size is negative/zero where it must be positive */
    KDA_ERR_BAD_DTYPE = 3,    /* unknown dtype or gate kind */
    KDA_ERR_UNSUPPORTED = 4,  /* sizes outside the compiled set (see each call) */
    KDA_ERR_BAD_ARGUMENT = 5, /* e.g. lower_bound >= 0, cu_seqlens with B != 1 */
    KDA_ERR_ALIAS = 6,        /* an output buffer is also an input buffer */
    KDA_ERR_HIP = 7           /* the kernel launch failed */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* How a gate tensor is given: retention factors alpha in [0, 1], or their natural
 * logarithm g = ln(alpha) <= 0. */
typedef enum { KDA_GATE_ALPHA = 0, KDA_GATE_LOG = 1 } kda_gate_kind;

/* Input preparation the *_fused_gate entry points can do inside the kernels (the model
 * excerpt on the Kept-memory page asks its kernels for all three; PaperLeet's contract
 * expects prepared inputs, which is what the plain entry points take).  Bits of `flags`:
 *   KDA_QK_L2NORM    q and k are divided by their L2 norm over K, x / max(|x|, 1e-6)
 *                    (the KDARecurrent page's unit normalisation of q and k)
 *   KDA_BETA_LOGITS  beta holds the write-strength logits; the kernel applies the sigmoid
 *   KDA_STATE_VK     every state argument is [.., V, K] (K contiguous) instead of
 *                    [.., K, V] (the transposed storage some model code keeps)
 * Any other bit set returns KDA_ERR_BAD_ARGUMENT. */
#define KDA_QK_L2NORM 1u
#define KDA_BETA_LOGITS 2u
#define KDA_STATE_VK 4u

/*
 * kda_bounded_decay -- the bounded per-channel decay gate (PaperLeet "Formula and
 * conventions", operator bounded_decay; cheat sheet gate table, Kimi K3 column).
 *
 *   out[r,h,c] = alpha   = exp(g)                     if out_kind == KDA_GATE_ALPHA
 *              = g       = lower_bound * sigmoid(exp(log_scale[h]) * (logits[r,h,c] + bias[h*K+c]))
 *                                                     if out_kind == KDA_GATE_LOG
 *   logits    [rows, H, K] in logits_dtype (rows = B*T)
 *   log_scale [H] float32 (the per-head A; the applied scale is e^A)
 *   bias      [H*K] float32 or NULL (a featurewise offset added before the scale)
 *   lower_bound  g_min, must be < 0 (the pages use -5)
 *   out       [rows, H, K] float32
 * Arithmetic is float32 with a sign-split sigmoid that never overflows.
 * rows == 0 enqueues nothing.  Any H, K >= 1 is supported.
 */
kda_status kda_bounded_decay(const void *logits, kda_dtype logits_dtype, const float *log_scale,
                             const float *bias, float lower_bound, int64_t rows, int H, int K,
                             kda_gate_kind out_kind, float *out, hipStream_t stream);

/*
 * kda_chunk_fwd -- chunkwise-parallel prefill of the recurrence (cheat sheet
 * "Chunkwise parallel form"; PaperLeet recurrent_kda contract for shapes, the
 * read-after-write output and the empty-sequence rule).
 *
 *   q, k   [B, T, H, K] in in_dtype;  v [B, T, H, V] in in_dtype
 *   gate   [B, T, H, K] float32, retention (KDA_GATE_ALPHA) or log-retention (KDA_GATE_LOG)
 *   beta   [B, T, H] float32 write strengths
 *   initial_state [N, H, K, V] float32, or NULL for zeros
 *   final_state   [N, H, K, V] float32, or NULL (not written).  It may equal
 *                 initial_state (in-place resume); no other overlap is allowed.
 *   cu_seqlens    NULL: N = B sequences of length T (one per batch row).
 *                 Otherwise int32 [num_seqs + 1] device array of packed offsets
 *                 (B must be 1, cu_seqlens[0] = 0, cu_seqlens[num_seqs] = T,
 *                 non-decreasing; zero-length sequences are allowed and get
 *                 final = initial).  N = num_seqs; the state restarts at every
 *                 sequence.  The offsets are read only on the device.
 *   chunk_size    16, 32 or 64: tokens per chunk (results differ only by rounding)
 *   scale         multiplies every output (1.0 leaves q unscaled)
 *   out    [B, T, H, V] in out_dtype
 * Supported: K, V in {16, 32, 64, 128} and chunk sizes whose per-workgroup LDS
 * layout fits 160 KB.  Without a workspace (one kernel), kda_chunk_fwd_supported() tells
 * which: chunk size 16 and 32 for every K, V on the bf16 path and up to K = 64 on the
 * float32 path, 64 only for small widths.  With a workspace (two kernels),
 * kda_chunk_fwd_workspace_size() > 0 tells which: chunk size 16 and 32 for every K, V on
 * both paths, 64 for every K, V on the bf16 path and at K <= 32 on the float32 path.
 * Anything else returns
 * KDA_ERR_UNSUPPORTED.  in_dtype KDA_F32 computes in float32 (matrix cores in fp32);
 * KDA_BF16 uses bf16/fp16 matrix-core operands with float32 accumulation and a
 * float32 master state.
 * Preconditions: every log-decay ln(alpha) >= -5 (the K3 bound; it is what keeps
 * the chunk's rescale factors inside float range; alpha = 0 is not allowed here);
 * on the bf16 path q and k at unit scale (each row's L2 norm at most about 1, as the
 * KDA layer normalises them: the decayed key and query operands pass through fp16
 * matrix-core operands).  Values and states may have any finite magnitude: the state,
 * the pseudo-values and their products go through 16-bit operands with an exact
 * power-of-two scale chosen per chunk from their largest magnitude.
 * T == 0 (or B == 0): nothing is launched for the scan; final_state is set to
 * initial_state (copied unless the pointers are equal) or zeros.
 *   workspace, workspace_bytes
 *          NULL: one kernel per (sequence, head, value block) does all of a chunk's work.
 *          Otherwise a device buffer, 16-byte aligned, of at least
 *          kda_chunk_fwd_workspace_size() bytes, owned by the caller and overlapping no
 *          other argument: a pre-pass over all (chunk, head) pairs at once forms each
 *          chunk's state-independent products (the decayed query and key operands, T and
 *          A_qk of the chunkwise form) into it, and a second kernel runs the serial part
 *          from them (same results up to rounding order).  Its contents are scratch: they
 *          are undefined after the call, and calls that share one workspace must not
 *          overlap in time.  A shape the two-kernel form does not support (workspace size
 *          0) returns KDA_ERR_UNSUPPORTED; a workspace too small or misaligned returns
 *          KDA_ERR_BAD_ARGUMENT.
 * `out` must be 8-byte aligned for bf16 output and 16-byte aligned for float32 output
 * (KDA_ERR_BAD_ARGUMENT otherwise): each store writes four value columns of a token.
 */
kda_status kda_chunk_fwd(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                         const float *gate, kda_gate_kind gate_kind, const float *beta,
                         const float *initial_state, float *final_state,
                         const int32_t *cu_seqlens, int num_seqs, int B, int64_t T, int H, int K,
                         int V, int chunk_size, float scale, void *out, kda_dtype out_dtype,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_fwd_workspace_size -- host-only query: bytes of workspace the two-kernel form
 * of kda_chunk_fwd / kda_chunk_fwd_fused_gate needs for this shape (varlen != 0: packed
 * sequences, B == 1, T the total length, num_seqs sequences), or 0 if that form does not
 * support it.  The size grows with the number of chunks: about 3 C K + 2 C^2 matrix
 * operands (2 bytes each on the bf16 path, 4 on the float32 path) per (chunk, head).
 */
size_t kda_chunk_fwd_workspace_size(kda_dtype in_dtype, int B, int64_t T, int num_seqs, int varlen, int H,
                                    int K, int V, int chunk_size);

/*
 * kda_chunk_fwd_fused_gate -- kda_chunk_fwd with the gate applied inside the kernel
 * (PaperLeet "Formula and conventions", operator bounded_decay; the KDARecurrent page
 * passes the raw gate logits, the per-head scale A, the featurewise bias and the lower
 * bound to its kernels rather than a precomputed retention):
 *
 *   alpha[t,h,c] = exp(lower_bound * sigmoid(exp(log_scale[h]) * (logits[t,h,c] + bias[h*K+c])))
 *
 *   logits    [B, T, H, K] in in_dtype (the dtype of q, k and v)
 *   log_scale [H] float32;  bias [H*K] float32 or NULL
 *   lower_bound  in [-5, 0): the bound itself is the chunk path's precondition
 *                (every log-decay >= -5), so it is checked here (KDA_ERR_BAD_ARGUMENT)
 *   flags     KDA_QK_L2NORM | KDA_BETA_LOGITS | KDA_STATE_VK or 0 (see above)
 * Every other argument, the supported set and the empty-sequence rule are those of
 * kda_chunk_fwd.  The gate is evaluated in float32 on the hardware exp2/reciprocal
 * (a few ulp from kda_bounded_decay's value), never written to memory, and needs no
 * float32 gate tensor: the HBM stream drops from 4 to 2 bytes per gate element with
 * bf16 logits.
 */
kda_status kda_chunk_fwd_fused_gate(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                                    const void *logits, const float *log_scale, const float *bias,
                                    float lower_bound, unsigned flags, const float *beta, const float *initial_state,
                                    float *final_state, const int32_t *cu_seqlens, int num_seqs, int B,
                                    int64_t T, int H, int K, int V, int chunk_size, float scale, void *out,
                                    kda_dtype out_dtype, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * kda_recurrent_fwd -- the same operation as kda_chunk_fwd (same arguments, layouts,
 * state rules, varlen and empty-sequence behaviour; the states must be 16-byte aligned
 * and out 16-byte aligned, 8-byte for bf16 output, else KDA_ERR_BAD_ARGUMENT)
 * evaluated token by token with the state held in registers (PaperLeet "Formula and conventions"; the model excerpt on the
 * Kept-memory page runs a token-recurrent kernel beside the chunked one for any length).
 * Meant for short sequences (speculative decoding, short prompts), where the chunked
 * form's per-chunk work does not pay off.  No chunk size; any alpha in [0, 1] is
 * allowed (no log-decay bound); all arithmetic is float32 on the vector units.
 * Supported: K, V in {16, 32, 64, 128}.
 */
kda_status kda_recurrent_fwd(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                             const float *gate, kda_gate_kind gate_kind, const float *beta,
                             const float *initial_state, float *final_state, const int32_t *cu_seqlens,
                             int num_seqs, int B, int64_t T, int H, int K, int V, float scale, void *out,
                             kda_dtype out_dtype, hipStream_t stream);

/*
 * kda_recurrent_fwd_fused_gate -- kda_recurrent_fwd with the gate evaluated inside the
 * kernel from logits [B, T, H, K] (in in_dtype), log_scale [H], bias [H*K] or NULL and
 * any lower_bound < 0 (the formula of kda_chunk_fwd_fused_gate); `flags` as there.
 */
kda_status kda_recurrent_fwd_fused_gate(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                                        const void *logits, const float *log_scale, const float *bias,
                                        float lower_bound, unsigned flags, const float *beta,
                                        const float *initial_state,
                                        float *final_state, const int32_t *cu_seqlens, int num_seqs, int B,
                                        int64_t T, int H, int K, int V, float scale, void *out,
                                        kda_dtype out_dtype, hipStream_t stream);

/*
 * kda_recurrent_step -- one decode token over a kept state, updated IN PLACE
 * (Kept-memory page: a decode call advances the kept per-head state by one token and
 * leaves the result for the next call; PaperLeet recurrence with T = 1).
 *
 *   q, k  [B, H, K] in in_dtype;  v [B, H, V] in in_dtype
 *   gate  [B, H, K] float32 (alpha or ln alpha, per gate_kind; any alpha in [0, 1])
 *   beta  [B, H] float32
 *   state [B, H, K, V] float32, read and overwritten with S_t
 *   out   [B, H, V] in out_dtype: o = scale * S_t^T q
 * Supported: K, V in {16, 32, 64, 128}.  All arithmetic is float32.  B == 0
 * enqueues nothing.
 */
kda_status kda_recurrent_step(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                              const float *gate, kda_gate_kind gate_kind, const float *beta,
                              float *state, int B, int H, int K, int V, float scale, void *out,
                              kda_dtype out_dtype, hipStream_t stream);

/*
 * kda_recurrent_step_fused_gate -- kda_recurrent_step with the gate applied inside the
 * kernel from logits [B, H, K] (in in_dtype), log_scale [H], bias [H*K] or NULL and
 * lower_bound < 0 (any value: the step accepts every alpha in [0, 1]); the formula and
 * `flags` are those of kda_chunk_fwd_fused_gate (with KDA_STATE_VK the state is
 * [B, H, V, K]).  The state is updated in place as in
 * kda_recurrent_step.
 */
kda_status kda_recurrent_step_fused_gate(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                                         const void *logits, const float *log_scale, const float *bias,
                                         float lower_bound, unsigned flags, const float *beta, float *state, int B,
                                         int H,
                                         int K, int V, float scale, void *out, kda_dtype out_dtype,
                                         hipStream_t stream);

/*
 * kda_chunk_fwd_supported -- host-only query (no device work): the number of value
 * columns one workgroup of kda_chunk_fwd handles for this shape (16, 32 or 64), or 0
 * if kda_chunk_fwd would return KDA_ERR_UNSUPPORTED for it.
 */
int kda_chunk_fwd_supported(kda_dtype in_dtype, int K, int V, int chunk_size);

/*
 * kda_chunk_bwd -- gradients of kda_chunk_fwd (PaperLeet "Return requirements": the scan
 * passes gradients to q, k, v, alpha, beta and the initial state; "Formula and
 * conventions": the operations are differentiable).  For the loss
 *     L = <d_out, out> + <d_final_state, final_state>
 * of the forward call with the same inputs it writes
 *   dq, dk [B, T, H, K] and dv [B, T, H, V] in grad_dtype,
 *   dgate  [B, T, H, K] float32: dL/dalpha (KDA_GATE_ALPHA) or dL/d ln alpha (KDA_GATE_LOG),
 *          matching how `gate` is given,
 *   dbeta  [B, T, H] float32,
 *   d_initial_state [N, H, K, V] float32, or NULL (not wanted).  With initial_state NULL
 *          the forward started from zeros and this is the gradient at the zero state.
 * Inputs: q, k, v, gate, gate_kind, beta, initial_state, cu_seqlens, num_seqs, B, T, H,
 * K, V and scale exactly as given to the forward; d_out [B, T, H, V] in dout_dtype;
 * d_final_state [N, H, K, V] float32 or NULL (zeros).
 * The forward is recomputed chunk by chunk (64 tokens) from the inputs; its intermediates
 * (chunk start states, their gradients, the per-chunk matrices) live in `workspace`, a
 * device buffer of at least kda_chunk_bwd_workspace_size(...) bytes that the caller owns
 * (about 0.55 MB per 64-token chunk and head at K = V = 128); its contents on entry do not
 * matter and on return are unspecified.  KDA_ERR_BAD_ARGUMENT if it is too small.
 * All arithmetic is float32 (matrix cores for the products).  Supported: K, V in
 * {16, 32, 64, 128}, N and H up to 65535, and (64-token chunk slots) x H below 2^31 (else
 * KDA_ERR_UNSUPPORTED).  Preconditions as kda_chunk_fwd: every log-decay
 * >= -5 (alpha > 0).  No output may overlap an input or another output.
 * T == 0 (or B == 0): no token gradients; d_initial_state = d_final_state (or zeros).
 */
size_t kda_chunk_bwd_workspace_size(int B, int64_t T, int H, int K, int V, int num_seqs, int varlen);
kda_status kda_chunk_bwd(const void *q, const void *k, const void *v, kda_dtype in_dtype, const float *gate,
                         kda_gate_kind gate_kind, const float *beta, const float *initial_state,
                         const int32_t *cu_seqlens, int num_seqs, int B, int64_t T, int H, int K, int V,
                         float scale, const void *d_out, kda_dtype dout_dtype, const float *d_final_state,
                         void *dq, void *dk, void *dv, kda_dtype grad_dtype, float *dgate, float *dbeta,
                         float *d_initial_state, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_bounded_decay_bwd -- gradients of kda_bounded_decay (PaperLeet "Return
 * requirements": bounded_decay passes gradients to the logits and the log-scale).
 *   grad        [rows, H, K] float32: dL/dalpha (grad_kind KDA_GATE_ALPHA) or dL/dg
 *               (KDA_GATE_LOG), for the gate evaluated from logits, log_scale, bias and
 *               lower_bound as in kda_bounded_decay
 *   d_logits    [rows, H, K] in dlogits_dtype
 *   d_log_scale [H] float32 or NULL;  d_bias [H*K] float32 or NULL (the gradient a
 *               featurewise bias receives; valid whether or not `bias` is given)
 * The sums over rows are done in a fixed order (bit-reproducible); float32 throughout.
 * rows == 0 writes zeros to d_log_scale and d_bias.
 */
kda_status kda_bounded_decay_bwd(const void *logits, kda_dtype logits_dtype, const float *log_scale,
                                 const float *bias, float lower_bound, int64_t rows, int H, int K,
                                 const float *grad, kda_gate_kind grad_kind, void *d_logits,
                                 kda_dtype dlogits_dtype, float *d_log_scale, float *d_bias, hipStream_t stream);

/*
 * kda_chunk_fwd_fused_gate_noalloc -- kda_chunk_fwd_fused_gate in its two-kernel form with
 * no workspace argument: the pre-pass packages and the carried state live in a fixed device
 * array of the library (KDA_NOALLOC_SCRATCH_BYTES, 64 MiB on every GPU the library runs on,
 * held until the process ends).  For callers that cannot allocate device memory: code under
 * graph capture, tight serving loops, harnesses that forbid allocation.  Nothing is
 * allocated or freed by the call.  Arguments, layouts, results and errors are those of
 * kda_chunk_fwd_fused_gate (same kernels); a shape whose workspace
 * (kda_chunk_fwd_workspace_size) exceeds the array, or that has no two-kernel form, returns
 * KDA_ERR_UNSUPPORTED -- at H = 96, K = V = 128 and chunk size 32 about 600 tokens fit.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time on the same
 * GPU (other streams, other threads) race and must be serialised by the caller.  The
 * array's contents are scratch: nothing in it needs clearing between calls.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)
kda_status kda_chunk_fwd_fused_gate_noalloc(const void *q, const void *k, const void *v, kda_dtype in_dtype,
                                            const void *logits, const float *log_scale, const float *bias,
                                            float lower_bound, unsigned flags, const float *beta,
                                            const float *initial_state, float *final_state,
                                            const int32_t *cu_seqlens, int num_seqs, int B, int64_t T, int H,
                                            int K, int V, int chunk_size, float scale, void *out,
                                            kda_dtype out_dtype, hipStream_t stream);
/* bytes of that device array (KDA_NOALLOC_SCRATCH_BYTES) */
size_t kda_noalloc_scratch_bytes(void);

/* A static, human-readable name for a status code. */
const char *kda_status_string(kda_status s);

/* KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

/* Text of the last HIP launch error seen by this thread (empty if none). */
const char *kda_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
