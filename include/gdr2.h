/*
 * gdr2.h -- C ABI of libgdr2, the Gated Delta Rule-2 operator for AMD
 * Instinct MI355X (gfx950).
 *
 * The operator (Gated DeltaNet-2 pages, "The Gated Delta Rule-2 State
 * Update", Eq. 10 and Steps 1-5): per head, with a dk x dv state S,
 *
 *     S_t = (I - k_t (b_t * k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t * v_t)^T
 *     o_t = S_t^T q_t,            alpha_t = exp(log_alpha_t)   (Eq. 12)
 *
 * alpha_t (dk) is a channel-wise decay on the key axis, b_t (dk) a
 * channel-wise erase gate on the key axis and w_t (dv) a channel-wise write
 * gate on the value axis.  The output reads the updated state and there is no
 * query scaling.  The gates are not clamped: b may lie in [0, 2] (the pages'
 * negative-eigenvalue variant, gate parameterisation after Eq. 11).
 *
 * Conventions shared by every entry point
 *   - All tensor arguments are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or retains them.
 *   - Token tensors are contiguous [B, T, H, D] (D fastest); the state is
 *     contiguous fp32 [N, H, dk, dv] (row i = key channel, dv fastest).
 *   - Every base pointer must be 16-byte aligned (else GDR2_E_ALIGN).
 *   - dk and dv must each be 32, 64 or 128 (else GDR2_E_UNSUPPORTED).
 *   - in_dtype (GDR2_F32 or GDR2_BF16) is the storage type of q, k, v, b, w
 *     and o; log_alpha has its own storage type.  The decay is always summed
 *     in fp32 (pages, Appendix D.1).
 *   - Calls are stream ordered and asynchronous: they enqueue kernels on
 *     `stream` (a hipStream_t; NULL is the null stream) and return without
 *     synchronising.  They are reentrant: the only global mutable state is a
 *     thread-local error string, per kernel and device an atomic flag
 *     recording that its LDS limit has been raised (setting it twice is
 *     harmless), and the static scratch of gdr2_chunk_fwd_noalloc.
 *   - Every argument error is detected on the host before any device call:
 *     nothing is written, the status is returned and gdr2_last_error()
 *     describes it.  A failed launch returns GDR2_E_LAUNCH.
 *   - Device-side contract violations are undefined results, not errors:
 *     cu_seqlens that is not non-decreasing from 0 to T, NaN/Inf inputs,
 *     o aliasing an input.  Out-of-range cu_seqlens entries are clamped to
 *     [0, T] so that no access leaves the caller's buffers.
 */
#ifndef GDR2_H
#define GDR2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Both enumerations are int-sized in C and C++ alike.  C++ gets the int
 * underlying type spelled out so that every int a C caller passes (an unknown
 * dtype code, say, which the entry points reject) is a valid value of the
 * parameter's type rather than undefined behaviour. */
#ifdef __cplusplus
#define GDR2_ENUM_BASE : int
#else
#define GDR2_ENUM_BASE
#endif

typedef enum GDR2_ENUM_BASE { GDR2_F32 = 0, GDR2_BF16 = 1 } gdr2_dtype;

typedef enum GDR2_ENUM_BASE {
    GDR2_OK = 0,
    GDR2_E_NULL = 1,        /* a required pointer is NULL */
    GDR2_E_SHAPE = 2,       /* a size is negative, zero where it must not be, or inconsistent */
    GDR2_E_DTYPE = 3,       /* unknown dtype code */
    GDR2_E_ALIGN = 4,       /* a base pointer is not 16-byte aligned */
    GDR2_E_UNSUPPORTED = 5, /* dk or dv outside {32, 64, 128} */
    GDR2_E_WORKSPACE = 6,   /* workspace missing or smaller than required */
    GDR2_E_LAUNCH = 7       /* the HIP runtime refused a launch */
} gdr2_status;

/*
 * Bytes of device workspace gdr2_chunk_fwd needs for these sizes (0 means the
 * workspace pointer may be NULL).  num_seqs is the value passed to
 * gdr2_chunk_fwd: the number of packed sequences with cu_seqlens, 0 without.
 * Returns 0 for arguments gdr2_chunk_fwd would reject.
 *
 * With in_dtype = GDR2_BF16 the forward runs in two passes and the workspace
 * holds one record per (64-token chunk, head) of the intra-chunk results the
 * state pass consumes: 2*4*(dk/32) KiB + 2*(dk/16) KiB + 6 KiB + (dv/16)*2 KiB
 * + 4*dk bytes each (70.5 KiB at dk = dv = 128), for B*ceil(T/64) chunks, or
 * ceil(T/64) + num_seqs chunks with packed sequences plus small tables.
 * Without cu_seqlens, when B*H is below 64 and dk == dv, each sequence's
 * chunks are split into P segments (a power of two, at most 16, with
 * B*H*P <= 256 and at least 16 chunks per segment; then P is reduced to
 * ceil(ceil(T/64) / ceil(ceil(T/64) / P))), and the workspace adds, from the
 * next 256-byte boundary after the records, B*P*H*dk*(dk + dv) fp32 values
 * for the segments' transfer matrices and end states.  With cu_seqlens, dk ==
 * dv and more than 32 chunks in all (ceil(T/64) > 32), long sequences may be
 * split too, as a plan built on the device from cu_seqlens decides: the
 * tables gain the plan (16 bytes per segment and 8 per sequence, each from a
 * 256-byte boundary, then 256 bytes), for at most nsmax = num_seqs +
 * (ceil(T/64) + num_seqs) / 32 segments, and the records are followed, from
 * the next 256-byte boundary, by nsmax*H*dk*(dk + dv) fp32 values.  Last, from
 * the next 256-byte boundary, comes one int32 per record (its chunk took the
 * exact strong-decay path).  With GDR2_F32 the
 * forward runs on the fp32 blocks of the backward's front pass and needs
 * exactly gdr2_chunk_bwd_workspace_bytes(B, T, H, dk, dv, num_seqs) bytes.
 * The workspace is scratch: its contents on entry do not matter and are not
 * meaningful on return.
 */
size_t gdr2_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int num_seqs,
                                      gdr2_dtype in_dtype);

/*
 * Chunkwise forward over whole sequences (pages, "Chunkwise Parallel Training
 * via WY Representation": Step 1 decay normalisation, Step 2 WY form, Step 3
 * state and output equations, Eqs. 20-24; packed variable-length batches per
 * Appendix C.6).  The chunk size is internal; the result does not depend on
 * it beyond rounding.
 *
 *   q, k, log_alpha, b : [B, T, H, dk]      v, w : [B, T, H, dv]
 *   S0  : fp32 [N, H, dk, dv] initial state per sequence, or NULL for zeros.
 *   o   : [B, T, H, dv] in in_dtype (written for every token of every sequence;
 *         with cu_seqlens, tokens outside [cu[0], cu[N]) are not written).
 *   S_T : fp32 [N, H, dk, dv] state after each sequence's last token, or NULL.
 *         S_T may alias S0 exactly (each state is read before it is written).
 *   cu_seqlens : NULL, in which case N = B and every batch row is one sequence
 *         of T tokens; or device int32 [num_seqs + 1] token offsets of packed
 *         sequences inside the single row (requires B == 1, N = num_seqs).
 *         A zero-length sequence gets S_T = S0.
 *   workspace : device scratch of at least gdr2_chunk_fwd_workspace_bytes().
 *
 * Execution: with GDR2_BF16, an intra-chunk kernel handles every (chunk,
 * head) in parallel (decay scan, chunk matrix, WY inverse and its products)
 * and writes a record per chunk to the workspace; a state kernel then walks
 * each sequence's chunks in order.  When the chains are split into segments
 * (see gdr2_chunk_fwd_workspace_bytes), a transfer pass first gives every
 * segment its affine map of the entry state (Eq. 23 composed over its
 * chunks), an fp32 scan chains the maps, and the state pass then walks all
 * segments at once from their true entry states.  Packed sequences are
 * planned one by one on the device: a sequence of nc chunks gets ceil(nc / L)
 * segments of balanced length, where L is the largest of 32 chunks, the
 * chunks times heads per compute unit, and sqrt(2 x the longest sequence's
 * chunks), so a long sequence among short ones no longer sets the call's
 * length.  With GDR2_F32 a front
 * kernel forms every (chunk, head)'s decay, chunk matrices, WY inverse and its
 * products in fp32 (the first pass of gdr2_chunk_bwd), and a sequential
 * kernel per (sequence, head, 32 value channels) forms o and S_T from them.
 *
 * Precision: the cumulative log-decay, the WY solve's diagonal blocks, every
 * accumulation and the state are fp32.  With in_dtype = GDR2_F32 every
 * matrix product takes fp32 operands.  With GDR2_BF16 the products take
 * 16-bit operands: bf16 for the decay-normalised chunk matrix, a bf16 hi/lo
 * pair for the causal score matrix, and fp16 for the state-pass operands
 * (stored in that form in the workspace records): the state, the chunk's
 * write targets U = A (w * v) and residuals R, and the decay-scaled q, k, b k,
 * which are at most |q|, |k|, |b k|.  The state-pass values must therefore
 * stay inside the fp16 range (|S|, |U|, |R| < 65504; with unit-norm keys and
 * b, w in [0, 2] that is |v| and |S0| below about 1e4); beyond it they become
 * +-inf and o and S_T come out non-finite.  The fp32 path has no such bound.
 *
 * Decay: any log_alpha <= 0 is computed as given.  The 16-bit products use
 * decay factors normalised on one row per chunk, or per 16-token block when
 * the chunk's decay is stronger; a chunk whose decay even those factors
 * cannot carry (a factor beyond 2^112) is flagged and formed again, entry by
 * entry with the exact decay, by the same kernel after its other chunks (about
 * three times the cost of an ordinary chunk).  The fp32 path uses one row per
 * chunk and the same exact path beyond e^80.
 */
gdr2_status gdr2_chunk_fwd(const void *q, const void *k, const void *v,
                           const void *log_alpha, const void *b, const void *w,
                           const float *S0, void *o, float *S_T,
                           const int32_t *cu_seqlens, int num_seqs,
                           int B, int T, int H, int dk, int dv,
                           gdr2_dtype in_dtype, gdr2_dtype log_alpha_dtype,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdr2_chunk_fwd with the output o stored in fp32 whatever in_dtype (the same
 * passage and the same arithmetic; with in_dtype = GDR2_F32 it is exactly
 * gdr2_chunk_fwd).  o : fp32 [B, T, H, dv].  For 16-bit inputs this keeps the
 * output's fp32 accumulation instead of rounding it to bf16: a bf16 store of
 * an exact value is off by up to 2^-8 of its magnitude, which for outputs
 * many times the RMS exceeds an error bound taken relative to the RMS.  Every
 * other argument, the workspace and the errors are those of gdr2_chunk_fwd.
 */
gdr2_status gdr2_chunk_fwd_f32_out(const void *q, const void *k, const void *v,
                                   const void *log_alpha, const void *b, const void *w,
                                   const float *S0, float *o, float *S_T,
                                   const int32_t *cu_seqlens, int num_seqs,
                                   int B, int T, int H, int dk, int dv,
                                   gdr2_dtype in_dtype, gdr2_dtype log_alpha_dtype,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdr2_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments without a workspace, and the same results.  The
 * workspace is a static device array of GDR2_NOALLOC_SCRATCH_BYTES inside the
 * library, one per device it runs on, held until the process ends; the call
 * allocates nothing (no hipMalloc, no library allocation).  Sizes whose
 * workspace (gdr2_chunk_fwd_workspace_bytes) exceeds that array give
 * GDR2_E_WORKSPACE: at dk = dv = 128 with bf16 inputs, about 3,600
 * (64-token chunk, head) items, e.g. B = 3, T = 4096, H = 16.  Every call on
 * one device shares its array, so calls that overlap on one device (other
 * streams, other threads) race and give undefined results; calls in stream
 * order on one stream do not.
 */
#define GDR2_NOALLOC_SCRATCH_BYTES (256u << 20)
gdr2_status gdr2_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                   const void *log_alpha, const void *b, const void *w,
                                   const float *S0, void *o, float *S_T,
                                   const int32_t *cu_seqlens, int num_seqs,
                                   int B, int T, int H, int dk, int dv,
                                   gdr2_dtype in_dtype, gdr2_dtype log_alpha_dtype, void *stream);

/*
 * Bytes of device workspace gdr2_chunk_bwd needs for these sizes (num_seqs as
 * for gdr2_chunk_fwd).  Returns 0 for sizes gdr2_chunk_bwd would reject.  The
 * backward keeps the intermediates its passes hand on, per (64-token chunk,
 * head), in fp32: (4 * 64 * dk + 3 * 64 * dv + 2 * 64 * 64 + 2 * dk * dv + dk)
 * * 4 bytes, rounded up to 256, per item (0.39 MB at dk = dv = 128), for
 * B * ceil(T/64) chunks (ceil(T/64) + num_seqs with packed sequences) times H,
 * then from the next 256-byte boundary one int per item, which records whether
 * its chunk's decay needs the exact-decay path.
 */
size_t gdr2_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int num_seqs);

/*
 * Backward of gdr2_chunk_fwd (Gated DeltaNet-2 pages, "Gate-Aware Backward
 * Pass", Appendix B): gradients of L with respect to every input, given dL/do
 * and dL/dS_T.  The forward quantities are recomputed from the inputs; the
 * state pass runs again to obtain the state entering every chunk, then the
 * state gradient runs over the chunks in reverse (the output and state
 * paths), and every chunk forms the gate-aware WY gradients (dA with the
 * write gate inside dU (w*v)^T and the erase gate inside dY (gamma*b*k)^T,
 * Eqs. 64-65; dT = -tril(A^T dA A^T, -1)) and the gate and decay gradients,
 * with dlog_alpha the reverse cumulative sum of dgamma * gamma inside each
 * chunk.  Everything is stored and accumulated in fp32.  Most products run
 * as three bf16 MFMA products on a hi/lo split of each fp32 operand (about
 * 2^-16 of each term); the WY inverse runs in fp32 (forward substitution and
 * fp32 MFMA).  The gradients meet a max error of 1e-4 relative to each
 * tensor's largest value (measured 3e-6 to 1.3e-5 at B4 T4096 H16 d128, at
 * most 1.6e-5 over the tested inputs).
 *
 *   q, k, log_alpha, b, v, w, S0, cu_seqlens, num_seqs, B, T, H, dk, dv and
 *       the dtypes: exactly as passed to gdr2_chunk_fwd.
 *   dO   : dL/do, [B, T, H, dv] in in_dtype.
 *   dS_T : dL/dS_T, fp32 [N, H, dk, dv], or NULL for zero.
 *   dq, dk, dlog_alpha, db : fp32 [B, T, H, dk];  dv, dw : fp32 [B, T, H, dv];
 *   dS0  : fp32 [N, H, dk, dv], or NULL (not computed).  With cu_seqlens,
 *       gradient rows outside [cu[0], cu[N]) are not written.
 *   workspace : at least gdr2_chunk_bwd_workspace_bytes() bytes of scratch.
 * With T == 0 the token tensors may be NULL and dS0 = dS_T (zeros without it).
 * Any log_alpha <= 0 is handled: the decay-weighted chunk products use factors
 * normalised on a chunk's row 31, and a chunk where some channel's decay moves
 * more than 80 nats from that row forms them entry by entry with the exact
 * decay instead.  The decay gradient sums each of its terms once (no term is
 * added and taken away again), so it keeps its relative precision when the
 * decay is strong and the gradient itself is small.
 */
gdr2_status gdr2_chunk_bwd(const void *q, const void *k, const void *v, const void *log_alpha,
                           const void *b, const void *w, const float *S0, const void *dO,
                           const float *dS_T, float *dq, float *dk, float *dv, float *dlog_alpha,
                           float *db, float *dw, float *dS0, const int32_t *cu_seqlens,
                           int num_seqs, int B, int T, int H, int dk_, int dv_,
                           gdr2_dtype in_dtype, gdr2_dtype log_alpha_dtype, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Gate prologue flags of gdr2_chunk_fwd_block (Gated DeltaNet-2 pages, "Gate
 * Parameterization", Eqs. 11-12, and the block's per-head q/k L2 norm).
 */
#define GDR2_PRO_QK_L2NORM 1u /* q, k <- x / sqrt(sum over dk of x^2 + qk_eps)              */
#define GDR2_PRO_DECAY 2u     /* f is W_f x: log_alpha = -exp(a) * softplus(f + delta)      */
#define GDR2_PRO_GATES 4u     /* b, w are W_b x, W_w x: b <- b_scale * sigmoid(b), w <- sigmoid(w) */

/*
 * The chunkwise forward from the block's projections, with grouped value heads
 * (Gated DeltaNet-2 pages: "Gate Parameterization", Eq. 12 log-decay
 * g = -exp(a) * softplus(W_f x + delta) and Eq. 11 gates b = sigmoid(W_b x),
 * with the factor 2 of the negative-eigenvalue variant, and w = sigmoid(W_w x);
 * q and k L2-normalised per head ("Big-Picture Architecture" item 1); with
 * H_v > H value heads, the key-side q, k, g and b are repeated across each
 * value-head group).  The selected activations run inside the intra-chunk
 * pass on the loaded values, in fp32, so the activated tensors never reach
 * HBM; the operator is then exactly gdr2_chunk_fwd on them.
 *
 *   q, k : bf16 [B, T, H, dk]          (raw when GDR2_PRO_QK_L2NORM)
 *   f    : [B, T, H, dk] in f_dtype    (W_f x with GDR2_PRO_DECAY, else log_alpha)
 *   b    : bf16 [B, T, H, dk]          (W_b x with GDR2_PRO_GATES, else the erase gate)
 *   v, w : bf16 [B, T, Hv, dv]         (w is W_w x with GDR2_PRO_GATES)
 *   decay_a, decay_bias : fp32 [H, dk], a and delta of Eq. 12 per key head
 *         and channel (required with GDR2_PRO_DECAY, else ignored).
 *   b_scale : 1 for the sigmoid erase gate, 2 for the negative-eigenvalue
 *         variant (GDR2_PRO_GATES; must be finite).
 *   qk_eps : >= 0 (GDR2_PRO_QK_L2NORM; a zero row gives NaN when it is 0).
 *   H, Hv : key heads and value heads; Hv must be a multiple of H, and value
 *         head h reads key head h / (Hv / H) (the group's value heads are
 *         consecutive).
 *   S0, S_T : fp32 [N, Hv, dk, dv] (NULL as in gdr2_chunk_fwd); o : bf16
 *         [B, T, Hv, dv]; cu_seqlens, num_seqs as in gdr2_chunk_fwd.
 *   workspace : at least gdr2_chunk_fwd_workspace_bytes(B, T, Hv, dk, dv,
 *         num_seqs, GDR2_BF16) bytes.
 * Unknown flag bits give GDR2_E_UNSUPPORTED; Hv not a multiple of H gives
 * GDR2_E_SHAPE.  flags = 0 with Hv = H is gdr2_chunk_fwd with bf16 inputs.
 * Precision and the handling of strong decay are those of gdr2_chunk_fwd
 * with GDR2_BF16, applied to the activated values.
 */
gdr2_status gdr2_chunk_fwd_block(const void *q, const void *k, const void *v, const void *f,
                                 const void *b, const void *w, const float *decay_a,
                                 const float *decay_bias, unsigned flags, float b_scale,
                                 float qk_eps, const float *S0, void *o, float *S_T,
                                 const int32_t *cu_seqlens, int num_seqs, int B, int T, int H,
                                 int Hv, int dk, int dv, gdr2_dtype f_dtype, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * One recurrent decode step for N independent sequences (pages, Appendix C.5:
 * forward-only recurrent kernel with an fp32 state, Eq. 10 applied to one
 * token).  The state is read once and written once.
 *
 *   q, k, log_alpha, b : [N, H, dk]      v, w : [N, H, dv]
 *   S : fp32 [N, H, dk, dv], updated in place.
 *   o : [N, H, dv] in in_dtype; must not alias S or an input.
 */
gdr2_status gdr2_decode_step(const void *q, const void *k, const void *v,
                             const void *log_alpha, const void *b, const void *w,
                             float *S, void *o, int N, int H, int dk, int dv,
                             gdr2_dtype in_dtype, gdr2_dtype log_alpha_dtype, void *stream);

/*
 * Output epilogue of the Gated DeltaNet-2 block (pages, "Big-Picture
 * Architecture" item 6 and "Gated DeltaNet-2 token mixer block" item 5: the
 * recurrent output is RMS-normalised, then gated channel by channel by a
 * SiLU-activated output gate):
 *
 *     y = o / sqrt(mean(o^2) + eps) * weight * silu(z),   silu(z) = z * sigmoid(z)
 *
 * with the mean over each group of `group` consecutive channels of a row.
 * Normalising each head on its own is o viewed as [B*T*H, dv] with group = dv
 * (weight [dv], shared by the heads), or as [B*T, H*dv] with group = dv and a
 * per-head weight [H*dv]; group = d normalises a whole row.
 *
 *   o, z, y : [rows, d] contiguous in dtype (z is the gate's pre-activation).
 *             y may alias o or z exactly (each element is read before its
 *             output is written); partial overlaps are undefined.
 *   weight  : fp32 [d], or NULL for ones.
 *   group   : a multiple of 8, at most GDR2_NORM_GATE_MAX_GROUP, dividing d.
 *   eps     : finite, >= 0.  With eps = 0 an all-zero group gives NaN.
 * rows = 0 is a no-op (the pointers may then be NULL).  Errors as for every entry point (GDR2_E_SHAPE for a
 * bad group or eps).  Arithmetic is fp32; y is rounded once to dtype.
 */
#define GDR2_NORM_GATE_MAX_GROUP 8192
gdr2_status gdr2_norm_gate(const void *o, const void *z, const float *weight, void *y,
                           long long rows, int d, int group, float eps, gdr2_dtype dtype,
                           void *stream);

/*
 * gdr2_decode_step with the output epilogue fused into its store: the same
 * state update (S is updated in place exactly as gdr2_decode_step does), but
 * instead of o it writes
 *
 *     y = o / sqrt(mean(o^2) + eps) * norm_weight * silu(z)
 *
 * per (sequence, head) over the dv channels (the block's output RMSNorm and
 * SiLU gate, pages "Big-Picture Architecture" item 6).  The workgroup that
 * owns a head already holds its whole output row, so the epilogue costs one
 * read of z and no extra pass.
 *
 *   z : [N, H, dv] in in_dtype; y : [N, H, dv] in in_dtype.  y may alias z
 *       exactly; it must not alias S or another input.
 *   norm_weight : fp32 [dv] shared by all heads, or NULL for ones.
 *   eps : finite, >= 0 (else GDR2_E_SHAPE).
 */
gdr2_status gdr2_decode_step_norm_gate(const void *q, const void *k, const void *v,
                                       const void *log_alpha, const void *b, const void *w,
                                       float *S, const void *z, const float *norm_weight,
                                       float eps, void *y, int N, int H, int dk, int dv,
                                       gdr2_dtype in_dtype, gdr2_dtype log_alpha_dtype,
                                       void *stream);

/* Static description of a status code. */
const char *gdr2_status_string(gdr2_status s);

/* Thread-local detail of the last non-OK status returned on this thread. */
const char *gdr2_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int gdr2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR2_H */
