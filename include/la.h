/*
 * la.h -- C ABI of the causal linear attention library (phi = elu + 1) for
 * AMD Instinct MI355X (gfx950).
 *
 * The method: "Transformers are RNNs: Fast Autoregressive Transformers with
 * Linear Attention -- part 2/3".  With phi(x) = elu(x) + 1 (eq. 7, alpha = 1),
 *   S_i = sum_{j<=i} phi(K_j) V_j^T,   Z_i = sum_{j<=i} phi(K_j)   (eq. 10-11)
 *   O_i = phi(Q_i)^T S_i / phi(Q_i)^T Z_i                           (eq. 12)
 * i.e. the causal masked attention of eq. 8 with sim(q,k) = phi(q).phi(k).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are device pointers owned by the caller, contiguous, row-major:
 *      Q, K      [B, H, N, D]      V, O, dO  [B, H, N, M]
 *      den       [B, H, N]   float32
 *      S         [B, H, D, M] float32, S[d][m] = sum_j phi(K_j)[d] V_j[m]
 *      Z         [B, H, D]    float32
 *    Q, K, V, O, dO, dQ, dK, dV (and decode q, k, v, y) share one storage
 *    type `dtype` (LA_F32 or LA_BF16); states, den and checkpoints are float32.
 *    Arithmetic is float32 throughout (bf16 values are widened exactly).
 *  - Heads are independent; B*H is a batch axis (Transformer Family v2,
 *    multi-head attention).
 *  - Supported sizes: B, H >= 1; N >= 0 (N = 0 is a no-op returning LA_OK);
 *    D, M in {32, 64}, or wide feature vectors (below) of D = 64 ns features
 *    up to 4096.  Every pointer must be 16-byte aligned.
 *  - Wide feature vectors ("Linear Attention/zh", feature maps: the degree-2
 *    polynomial map, whose feature count is about the square of the head
 *    size, or a few hundred positive random features; "Transformers are RNNs
 *    -- part 2/3", section 3.2.1): D > 64, a multiple of 64, with feature =
 *    LA_FEATURE_IDENTITY and no decay, in la_forward_causal,
 *    la_backward_causal, la_forward_noncausal, la_backward_noncausal and
 *    la_decode_step.  Q, K, dQ, dK are then stored feature-sliced:
 *    [B, H, D/64, N, 64], slice s holding features 64 s .. 64 s + 63 of every
 *    token (the layout la_feature_random and la_feature_poly2 write for C >
 *    64).  S [B, H, D, M], Z [B, H, D] and decode's q, k [B, H, D] keep their
 *    layouts.  Sums over all D features (O's numerator and denominator, dV)
 *    are formed per slice and added in a fixed order.
 *  - Outputs must not overlap inputs (decode's S and Z are updated in place
 *    by design).  Overlaps are rejected with LA_ERR_ALIAS.
 *  - Scratch memory is the caller's `ws` of `ws_bytes` bytes, at least
 *    la_workspace_size(...) (which may be 0; then ws may be NULL).  The
 *    library never allocates device memory.
 *  - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL = the default stream).  No host synchronisation (except the status
 *    query la_forward_wait_status), no other streams.
 *  - All arguments are validated before any launch; on error nothing is
 *    launched and a status is returned (la_last_error() gives details).  A
 *    failed launch returns LA_ERR_HIP with the HIP message.  No C++
 *    exception crosses this interface.  The library holds no device state.
 *  - phi is applied inside the kernels; gradients are with respect to the
 *    raw Q, K, V.  No epsilon is added to the denominator: phi > 0 keeps it
 *    positive for inputs above about -80 (below that exp underflows in fp32).
 */
#ifndef LA_H
#define LA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

typedef enum {
  LA_OK = 0,
  LA_ERR_NULL = 1,        /* a required pointer is NULL */
  LA_ERR_SHAPE = 2,       /* B, H < 1, N < 0, or sizes overflow */
  LA_ERR_DTYPE = 3,       /* dtype not LA_F32 / LA_BF16 */
  LA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  LA_ERR_ALIAS = 5,       /* an output overlaps an input or another output */
  LA_ERR_WORKSPACE = 6,   /* ws_bytes < la_workspace_size(...) or ws NULL */
  LA_ERR_UNSUPPORTED = 7, /* D or M not in {32, 64} */
  LA_ERR_HIP = 8,         /* a HIP launch failed */
  LA_ERR_ARG = 9,         /* inconsistent optional arguments */
  LA_ERR_WAIT = 10        /* a one-launch forward gave up waiting (see
                             la_forward_wait_status) */
} la_status;

typedef enum {
  LA_OP_FWD_CAUSAL = 0,
  LA_OP_FWD_NONCAUSAL = 1,
  LA_OP_BWD_CAUSAL = 2,
  LA_OP_DECODE = 3,
  LA_OP_BWD_NONCAUSAL = 4,
  LA_OP_FWD_DECAY = 5, /* la_forward_causal with logA */
  LA_OP_BWD_DECAY = 6  /* la_backward_causal with logA */
} la_op;

/* Feature map applied to Q and K by the attention entry points.
 *   LA_FEATURE_ELU1      phi(x) = elu(x) + 1 ("Transformers are RNNs -- part 2/3",
 *                        eq. 7); gradients are with respect to the raw Q, K.
 *   LA_FEATURE_IDENTITY  Q and K already hold feature vectors phi(q), phi(k)
 *                        of dimension D (another feature map: "Linear
 *                        Attention/zh", feature maps -- polynomial, positive
 *                        random features; see la_feature_*); they are used as
 *                        they are and the gradients are with respect to them.
 *                        The similarities phi(q).phi(k) summed into each
 *                        denominator must be positive. */
typedef enum { LA_FEATURE_ELU1 = 0, LA_FEATURE_IDENTITY = 1 } la_feature;

/* Form of the causal forward without a decay (results differ only in
 * rounding; both compute eq. 9-12 of "Transformers are RNNs -- part 2/3").
 *   LA_FORM_AUTO        the library's measured rule: one launch where the
 *                       segments allow it (at most four chunks, aggregates
 *                       summed by every workgroup), the state has D*M >= 2048
 *                       and every workgroup of the grid is resident at once;
 *                       two launches otherwise.
 *   LA_FORM_TWO_LAUNCH  a separate aggregate pass, then the forward.
 *   LA_FORM_ONE_LAUNCH  one launch wherever the segments allow it: each
 *                       workgroup walks its segment from a zero state,
 *                       publishes the segment's aggregate behind a flag in
 *                       `ws`, waits for the earlier segments' flags and adds
 *                       their aggregates at the end.  Where the grid is not
 *                       resident at once, progress relies on workgroups being
 *                       dispatched in index order (the lowest unfinished one
 *                       never waits); this order is not a documented
 *                       guarantee, hence the bounded waits below. */
typedef enum {
  LA_FORM_AUTO = 0,
  LA_FORM_TWO_LAUNCH = 1,
  LA_FORM_ONE_LAUNCH = 2
} la_form;

/* Per-call options.  Every entry point that plans segments takes a
 * `const la_options *opts`; NULL (or an all-zero struct) means the defaults.
 * The library keeps no state between calls: whatever a call depends on is in
 * its arguments, so concurrent calls from several host threads with
 * different options are independent (calls that share an output, a
 * workspace or a decode state still race, as with any buffer).
 *   segment_chunks  0: automatic segment length; > 0: segments of that many
 *                   64-token chunks (clamped to the sequence).  Results do
 *                   not depend on it beyond rounding.  A checkpoint is laid
 *                   out by it: la_checkpoint_size, la_forward_causal and the
 *                   la_backward_causal that reads the checkpoint must be
 *                   given the same value.
 *   forward_form    la_form (above).
 *   wait_polls      one-launch forward: polls (each waits for a device-scope
 *                   load, about a microsecond) before a workgroup waiting for
 *                   an earlier segment gives up; 0: the default 2^22 (a few
 *                   seconds); < 0: none at all, every wait gives up at once
 *                   (exercises the failure path: no wave spins).  A workgroup
 *                   that gives up makes its carry NaN, so its rows of O and
 *                   den, its checkpoint entries and the final state show the
 *                   failure instead of a wrong value, and sets the status
 *                   word of `ws` (la_forward_wait_status) and, when given,
 *                   *status.
 *   status          optional device pointer to one 32-bit word: the
 *                   one-launch forward ORs 1 into it when a wait gave up.
 *                   Never cleared by the library.
 *   timed_kernel    optional kernel name (see la_kernel_names): every launch
 *                   of that kernel in this call is bracketed by a pair of
 *                   caller-created HIP events recorded on the launch stream,
 *                   events[2 i] before and events[2 i + 1] after, for i =
 *                   *events_used, *events_used + 1, ... while i <
 *                   event_pairs; *events_used (host memory) is advanced by
 *                   one per recorded pair.  Reading the times is the
 *                   caller's (hipEventElapsedTime after a synchronisation). */
typedef struct la_options {
  int segment_chunks;
  int forward_form;
  int wait_polls;
  int event_pairs;
  unsigned *status;
  const char *timed_kernel;
  void **events;
  int *events_used;
} la_options;

/* Library version, as 10000*major + 100*minor + patch. */
int la_version(void);

/* Bytes of scratch memory the operation `op` needs for these sizes
 * (0 when none).  Returns 0 for invalid arguments. */
size_t la_workspace_size(int op, int B, int H, int N, int D, int M, int dtype,
                         const la_options *opts);

/* Bytes of the segment-state checkpoint written by la_forward_causal and
 * read by la_backward_causal: the float32 state (S, Z) before every segment
 * of the sequence and after the last one.  The sequence is cut into
 * segments of a fixed length chosen from (B, H, N, D, M) and
 * opts->segment_chunks only, so a checkpoint is valid for any call with the
 * same sizes and segment option.  Its size is
 * O(N * D * M / segment) per head, well inside the pages' linear-memory
 * bound; no per-token state S_i is ever stored ("Transformers are RNNs --
 * part 2/3", section 3.3.1).  The decayed recurrence (logA given) uses
 * longer segments and at most this many bytes.  For wide feature vectors
 * (D > 64) the states are those of the D/64 feature slices of every head
 * (the same memory as the heads' states). */
size_t la_checkpoint_size(int B, int H, int N, int D, int M,
                          const la_options *opts);

/* Sequence segment length (tokens) used for these sizes and options: the
 * spacing of the checkpoint entries.  By default about 1024 (short sequences
 * of small states) or 512 segments are planned over all heads, each a whole
 * number of 64-token chunks. */
int la_segment_length(int B, int H, int N, int D, int M,
                      const la_options *opts);

/* Status of the last one-launch causal forward that used this workspace
 * (same sizes and options): LA_ERR_WAIT when one of its workgroups gave up
 * waiting for an earlier segment's aggregate (its rows of O and den, its
 * checkpoint entries and the final state are then NaN), LA_OK otherwise
 * (also when the call took the two-launch form or needed no workspace).
 * Reads the status word of `ws` after synchronising `stream`: the only
 * call of this library that blocks the host. */
int la_forward_wait_status(const void *ws, size_t ws_bytes, int B, int H,
                           int N, int D, int M, int dtype, void *stream,
                           const la_options *opts);

/*
 * Causal forward, eq. 9-12 ("Transformers are RNNs -- part 2/3", section 3.3).
 *   Q, K, V     inputs.
 *   logA        optional [B,H,N] float32 log-decay per token and head
 *               ("Linear Attention/zh", variants and extensions: RetNet's
 *               decay, a constant per head, or a data-dependent gate):
 *               S_t = a_t S_{t-1} + phi(K_t) V_t^T and Z_t = a_t Z_{t-1} +
 *               phi(K_t) with a_t = exp(logA_t); values must be finite and
 *               <= 0 (a_t in (0, 1]).  NULL: the plain running sums.  The
 *               workspace is then la_workspace_size(LA_OP_FWD_DECAY, ...),
 *               and the checkpoint holds the decayed states (valid only for
 *               a backward with the same logA).
 *   O           output [B,H,N,M] in `dtype` (float32 values rounded to
 *               nearest even for bf16).
 *   den         optional output [B,H,N] float32: phi(Q_i)^T Z_i (needed by
 *               la_backward_causal).  NULL to skip.
 *   S0, Z0      optional initial state (both or neither): the state before
 *               token 1, so a sequence can be continued (eq. 16-19 with a
 *               non-zero s_0, z_0).
 *   S_out,Z_out optional final state S_N, Z_N (both or neither).
 *   ckpt        optional output of la_checkpoint_size(...) bytes: segment
 *               boundary states for la_backward_causal.  NULL to skip.
 *   ws          la_workspace_size(LA_OP_FWD_CAUSAL, ...) bytes: segment
 *               aggregates, their prefix states, and (one-launch form, see
 *               la_form) one 32-bit flag per segment plus the status word,
 *               cleared by the call itself, so any contents are
 *               accepted.  Wide feature vectors always take two launches
 *               (and a third that sums the slices' shares, kept in `ws`).  In the one-launch form the workgroups of a call
 *               exchange segment aggregates through `ws`: calls that overlap
 *               on one workspace race, as with any scratch buffer.
 */
int la_forward_causal(const void *Q, const void *K, const void *V,
                      const float *logA, void *O, float *den, const float *S0,
                      const float *Z0, float *S_out, float *Z_out,
                      float *ckpt, int B, int H, int N, int D, int M,
                      int dtype, int feature, void *ws, size_t ws_bytes,
                      void *stream, const la_options *opts);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the causal
 * forward of la_forward_causal with the same arguments and results, minus
 * `ws` and `ws_bytes`.  Its scratch (segment aggregates, prefix states, the
 * one-launch form's flags and status word) is a static array of
 * LA_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held from
 * the library's first use on that GPU until the process ends; the call
 * allocates nothing.  Sizes whose la_workspace_size(LA_OP_FWD_CAUSAL, ...)
 * (LA_OP_FWD_DECAY with logA) exceeds it are rejected with
 * LA_ERR_WORKSPACE before any launch.  Every call on one GPU shares that
 * GPU's array and leaves its contents behind (each call clears what must
 * start at zero itself): calls that overlap on one GPU -- on different
 * streams or host threads -- race; order them on one stream.
 * la_forward_wait_status does not apply (its status word lives in the
 * static array; pass opts->status to learn of a wait that gave up).
 */
#define LA_NOALLOC_SCRATCH_BYTES ((size_t)24 << 20)
int la_forward_causal_noalloc(const void *Q, const void *K, const void *V,
                              const float *logA, void *O, float *den,
                              const float *S0, const float *Z0, float *S_out,
                              float *Z_out, float *ckpt, int B, int H, int N,
                              int D, int M, int dtype, int feature,
                              void *stream, const la_options *opts);

/*
 * Non-causal forward (reading notes on "Transformers are RNNs", section 3.2,
 * eq. 5-6): S = sum_j phi(K_j) V_j^T and Z = sum_j phi(K_j) are formed once
 * per head and reused for every query, O_i = phi(Q_i)^T S / phi(Q_i)^T Z.
 *   S_out, Z_out optional outputs [B,H,D,M], [B,H,D] float32 (both or
 *               neither): the totals S, Z, which la_backward_noncausal can
 *               take instead of forming them again (zero for N = 0).
 */
int la_forward_noncausal(const void *Q, const void *K, const void *V, void *O,
                         float *S_out, float *Z_out, int B, int H, int N,
                         int D, int M, int dtype, int feature, void *ws,
                         size_t ws_bytes, void *stream,
                         const la_options *opts);

/*
 * Causal backward: gradients of a scalar loss with respect to the raw Q, K,
 * V given dO = dL/dO, by the cumulative sums of eq. 13-15 ("Transformers are
 * RNNs -- part 2/3", section 3.3.1): a forward-running sum of phi(K) V^T for
 * the query gradient and a backward-running sum of phi(Q) (dL/dnum)^T for
 * the key and value gradients, in linear time without any per-token state.
 * The denominator's share (left by the pages to automatic differentiation)
 * is the quotient rule: dL/dnum_i = dO_i / den_i, dL/dden_i =
 * -(dO_i . O_i) / den_i.
 *   logA        the forward's log-decay, or NULL (see la_forward_causal).
 *               With logA the workspace is la_workspace_size(
 *               LA_OP_BWD_DECAY, ...) and O, den are validated but not read
 *               (den_i and O_i . dO_i are recomputed in the order that keeps
 *               every decay factor <= 1).
 *   O, den      the forward's O and den (required when N > 0).
 *   S0, Z0      the initial state the forward started from (both or neither).
 *   ckpt        the forward's checkpoint (same sizes) or NULL: then the
 *               segment states are recomputed into `ws`.
 *   dS_N, dZ_N  optional gradients [B,H,D,M], [B,H,D] float32 of the loss
 *               with respect to the forward's final state S_out, Z_out (both
 *               or neither; NULL: the final state does not reach the loss).
 *               Every term phi(K_j) V_j^T is part of S_N, so they start the
 *               backward-running sum of eq. 14-15.
 *   dQ, dK, dV  outputs in `dtype`.
 *   dlogA       [B,H,N] float32 output, required with logA and NULL
 *               without: the gradient with respect to logA.
 *   dS0, dZ0    optional outputs [B,H,D,M], [B,H,D] float32 (both or
 *               neither): the gradient with respect to the initial state S0,
 *               Z0 (zero state when those were NULL), i.e. the
 *               backward-running sum carried through token 1.  With dS_N, dZ_N
 *               this chains a backward over consecutive pieces of a sequence.
 *               They must not overlap dS_N, dZ_N.  For N = 0 they receive
 *               dS_N, dZ_N (zero when NULL) and nothing else is read.
 */
int la_backward_causal(const void *Q, const void *K, const void *V,
                       const float *logA, const void *O, const float *den,
                       const void *dO, const float *S0, const float *Z0,
                       const float *ckpt, const float *dS_N,
                       const float *dZ_N, void *dQ, void *dK, void *dV,
                       float *dlogA, float *dS0, float *dZ0, int B, int H,
                       int N, int D, int M, int dtype, int feature, void *ws,
                       size_t ws_bytes, void *stream, const la_options *opts);

/*
 * Non-causal backward: gradients of a scalar loss with respect to the raw Q,
 * K, V of la_forward_noncausal given dO = dL/dO.  The causal backward's
 * quotient rule with the masks removed (reading notes on "Transformers are
 * RNNs", section 3.2, eq. 5-6): the running sums of eq. 13-15 become the
 * totals S = sum_j phi(K_j) V_j^T, Z = sum_j phi(K_j) (query side) and
 * R = sum_i phi(Q_i) g_i^T, r = sum_i c_i phi(Q_i) with g_i = dO_i / den_i,
 * c_i = -(dO_i . O_i) / den_i (key side):
 *   dphi(Q_i) = S g_i + c_i Z,  dphi(K_j) = R V_j + r,  dV_j = R^T phi(K_j).
 * den_i and dO_i . O_i are recomputed from S, Z, so neither O nor den is an
 * input.  Linear time, O(D M) state per head.
 *   Q, K, V, dO inputs [B,H,N,D] / [B,H,N,M] in `dtype` (Q, K feature-sliced
 *               for wide feature vectors).
 *   S_tot, Z_tot optional: the totals written by la_forward_noncausal for the
 *               same Q, K, V (both or neither); NULL: formed here again.
 *   dQ, dK, dV  outputs in `dtype`.
 *   ws          la_workspace_size(LA_OP_BWD_NONCAUSAL, ...) bytes (never 0
 *               for N > 0).
 */
int la_backward_noncausal(const void *Q, const void *K, const void *V,
                          const void *dO, const float *S_tot,
                          const float *Z_tot, void *dQ, void *dK, void *dV,
                          int B, int H, int N, int D, int M, int dtype,
                          int feature, void *ws, size_t ws_bytes,
                          void *stream, const la_options *opts);

/*
 * One RNN step of the attention ("Transformers are RNNs -- part 2/3",
 * section 3.4, eq. 18-20 without the projections, f_l and residual):
 *   S += phi(k) v^T;  Z += phi(k);  y = phi(q)^T S / phi(q)^T Z.
 *   logA        optional [B,H] float32 log-decay of this step (as in
 *               la_forward_causal): S = a S + phi(k) v^T, Z = a Z + phi(k).
 *   q, k [B,H,D], v [B,H,M], y [B,H,M] in `dtype`; S [B,H,D,M] and Z [B,H,D]
 *   float32, updated in place (the update comes first: masking is
 *   inclusive).  Wide feature vectors (D > 64): one workgroup per head
 *   streams its state; no logA.  Calls on one stream are ordered; overlapping calls on
 *   different streams that share S/Z race.
 */
int la_decode_step(const void *q, const void *k, const void *v,
                   const float *logA, float *S, float *Z, void *y, int B,
                   int H, int D, int M, int dtype, int feature, void *stream,
                   const la_options *opts);

/*
 * Positive random features ("Linear Attention/zh", feature maps: Performer's
 * phi(x) proportional to exp(W x - |x|^2 / 2); "The Transformer Family v2",
 * random feature attention): Phi[b,h,n,c] = exp(W[h,c,:] . X[b,h,n,:] -
 * |X[b,h,n,:]|^2 / 2) / sqrt(C), so phi(x) . phi(y) estimates exp(x . y)
 * without bias when the rows of W are standard normal.  Feed Phi of queries
 * and keys to the attention entry points with LA_FEATURE_IDENTITY.
 *   X    [B,H,N,Din] in `dtype`; W [H,C,Din] float32 (the random projection,
 *        owned by the caller); Phi output in `dtype`: [B,H,N,C] for C <= 64,
 *        feature-sliced [B,H,C/64,N,64] for wider maps.
 *   Din in {32, 64}; C in {32, 64} or a multiple of 64 up to 4096.  Same
 *   validation and error behaviour as the attention entry points;
 *   asynchronous on `stream`.
 */
int la_feature_random(const void *X, const float *W, void *Phi, int B, int H,
                      int N, int Din, int C, int dtype, void *stream);

/* Vector-Jacobian product of la_feature_random: dX = sum_c dPhi_c phi_c
 * (W_c - x), with phi recomputed in float32.  dPhi in the layout of Phi, dX
 * [B,H,N,Din] in `dtype`. */
int la_feature_random_vjp(const void *X, const float *W, const void *dPhi,
                          void *dX, int B, int H, int N, int Din, int C,
                          int dtype, void *stream);

/*
 * Degree-2 polynomial features ("Linear Attention/zh", feature maps:
 * phi(x) = (1, x, x (x) x) truncated; "Transformers are RNNs -- part 2/3",
 * section 3.2.1): Phi = (1, x_1 .. x_Din, x_a x_b for a, b = 1..Din
 * a-major, then zeros up to C), so phi(x) . phi(y) = 1 + x.y + (x.y)^2 > 0.
 *   X [B,H,N,Din], Phi in `dtype` ([B,H,N,C] for C <= 64, feature-sliced
 *   [B,H,C/64,N,64] for wider maps); C in {32, 64} or a multiple of 64 up
 *   to 4096, with 1 <= Din <= 64 and 1 + Din + Din^2 <= C (Din <= 5 for C =
 *   32, <= 7 for C = 64, C = 1088 for Din = 32).
 */
int la_feature_poly2(const void *X, void *Phi, int B, int H, int N, int Din,
                     int C, int dtype, void *stream);

/* Vector-Jacobian product of la_feature_poly2: dX_a = dPhi[1 + a] +
 * sum_b (dPhi[1 + Din + a Din + b] + dPhi[1 + Din + b Din + a]) x_b. */
int la_feature_poly2_vjp(const void *X, const void *dPhi, void *dX, int B,
                         int H, int N, int Din, int C, int dtype,
                         void *stream);

/* Name of a status code. */
const char *la_status_string(int status);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char *la_last_error(void);

/* Comma-separated names of the kernels the library launches. */
const char *la_kernel_names(void);

#ifdef __cplusplus
}
#endif

#endif /* LA_H */
