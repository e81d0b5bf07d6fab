/*
 * streamkl.h -- C ABI of the fused attention-KL primitive for MI355X (gfx950).
 *
 * What it computes.  For every query row r = (b, h, i) the forward KL divergence
 * between the teacher and the student attention distributions over the keys,
 * teacher first, in nats:
 *
 *     s_t[j] = tau_t * (Q_t[i] . K_t[j]),      s_s[j] = tau_s * (Q_s[i] . K_s[j])
 *     P_t = softmax_j(s_t),                    P_s = softmax_j(s_s)
 *     KL_r = sum_j P_t[j] * (log P_t[j] - log P_s[j])
 *
 * The quantity and its use as a distillation loss are those of "StreamKL: Fast
 * and Memory-Efficient KL Divergence for Boosting Attention Distillation"
 * (abstract: KL between two attention distributions, reduced without
 * materialising either N_Q x N_K matrix; forward in one streaming pass, backward
 * recomputing the probabilities tile by tile).  The direction (teacher in the
 * first slot), the natural log and the temperature reading tau = 1/(sqrt(d) T)
 * follow "Lecture 05 - Where It All Lands", section 3.1 (forward KL at
 * temperature T); a T^2 or alpha weighting (section 3.3) is applied by the caller
 * through the upstream gradient of streamkl_bwd.
 *
 * Causal masking, when requested, is bottom-right aligned: key j is allowed for
 * query i iff j <= i + (n_k - n_q).  Causal with n_q > n_k is rejected (it would
 * leave rows with no key).  Masked keys are excluded from both softmaxes.
 *
 * Conventions common to every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing, frees nothing, never synchronises, and keeps no mutable
 *    global state; it is safe to call from several host threads.
 *  - Inputs are [B, H, N, d] with the last dimension contiguous.  `strides`
 *    gives, in ELEMENTS, the batch, head and row strides of q_t, k_t, q_s, k_s in
 *    that order (12 values: q_t.b, q_t.h, q_t.n, k_t.b, ...); NULL means fully
 *    contiguous.  Every row must start on a 16-byte boundary, and the row
 *    stride times the element size must be below 2^26 bytes (64 MiB; the
 *    kernels address a 32-row tile with 32-bit offsets).
 *  - Teacher and student share dtype, B, H, n_q and n_k; d_t and d_s may differ.
 *  - Per-row outputs (kl_rows, lse_t, lse_s, grad_rows) are contiguous fp32
 *    [B, H, n_q].  Gradients dq_s / dk_s are contiguous [B, H, n_q | n_k, d_s]
 *    in the input dtype and are overwritten, not accumulated.
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *    enqueued on it and the call returns before the work completes; a fault
 *    during execution surfaces at the caller's next synchronisation.
 *  - Every argument is validated on the host before any HIP call is made; an
 *    error status means nothing was enqueued.
 */
#ifndef STREAMKL_H
#define STREAMKL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    STREAMKL_OK = 0,
    STREAMKL_ERR_INVALID = 1,     /* null pointer, bad size, bad tau, misalignment, causal with n_q > n_k,
                                     a row stride of 2^26 bytes or more, or a problem too large for one
                                     dispatch (B H (ceil(n_q/128) +
                                     ceil(n_k/128)) 256 >= 2^32, or n_q / n_k beyond 2^30 - 128) */
    STREAMKL_ERR_UNSUPPORTED = 2, /* (dtype, d_t, d_s) combination not built */
    STREAMKL_ERR_WORKSPACE = 3,   /* workspace too small (streamkl_fwd_split) */
    STREAMKL_ERR_HIP = 4          /* a HIP launch error was reported */
} streamkl_status;

typedef enum {
    STREAMKL_F32 = 0,  /* fp32 inputs, fp32 MFMA (v_mfma_f32_32x32x2_f32) */
    STREAMKL_BF16 = 1  /* bf16 inputs, bf16 MFMA with fp32 accumulation */
} streamkl_dtype;

/*
 * Forward.  One streaming pass over the key tiles of every query block keeps,
 * per query row, the teacher max m_t and normaliser l_t, the student max m_s and
 * normaliser l_s, and the teacher-weighted score accumulators, and finishes with
 *     KL = E_{P_t}[s_t - s_s] - LSE_t + LSE_s.
 *
 *   q_t, k_t  teacher queries [B,H,n_q,d_t] and keys [B,H,n_k,d_t]
 *   q_s, k_s  student queries [B,H,n_q,d_s] and keys [B,H,n_k,d_s]
 *   tau_t, tau_s  score scales (finite, >= 0; tau = 0 gives a uniform row)
 *   causal    0 or 1
 *   kl_rows   out, per-row KL (nats)
 *   lse_t, lse_s  out, per-row log-normalisers log sum_j exp(s[j]); needed by
 *             streamkl_bwd.  These 8 bytes per row are the only state kept
 *             between the passes.
 *   kl_sum    out, one fp32 device scalar = deterministic sum of kl_rows
 *             (fixed reduction order, fp64 accumulation); may be NULL.
 *
 * Supported (d_t, d_s): each of 64 and 128, for both dtypes.
 */
streamkl_status streamkl_fwd(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                             streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                             const int64_t *strides, float tau_t, float tau_s, int causal,
                             float *kl_rows, float *lse_t, float *lse_s, float *kl_sum,
                             void *stream);

/*
 * Split forward and its pieces.  The per-row online state has an associative
 * merge, so the forward can run over disjoint key ranges independently and be
 * combined afterwards: within one GPU to fill it when B H ceil(n_q / 128) is
 * small (split-K), across GPUs when the keys are sharded (context parallel).
 *
 * A row's partial state over a key subset J is STREAMKL_STATE_FLOATS floats
 *   [m_t, L, AT, AS, m_s, LS]
 * with reference values m_t, m_s (raw scores q.k; any finite value that keeps
 * the sums in range -- the kernels use them as running references), c = tau
 * log2(e), and over the allowed keys j in J
 *   L = sum 2^(c_t (x_t[j] - m_t)),  AT = sum 2^(c_t (x_t[j] - m_t)) x_t[j],
 *   AS = sum 2^(c_t (x_t[j] - m_t)) x_s[j],  LS = sum 2^(c_s (x_s[j] - m_s)),
 * x = q . k unscaled.  An empty subset has L = LS = 0.  The union of subsets
 * merges by rescaling to the larger references and adding; the finish is
 *   LSE_t = tau_t m_t + ln L,  LSE_s = tau_s m_s + ln LS,
 *   KL = (tau_t AT - tau_s AS) / L - LSE_t + LSE_s.
 */
#define STREAMKL_STATE_FLOATS 6

/* Partial forward over the keys [k_begin, k_end) (global key indices; the
 * causal mask, if any, is taken in global coordinates).  k_begin must be a
 * multiple of 32 and k_end a multiple of 32 or n_k.  state: out, device fp32
 * [B*H*n_q][STREAMKL_STATE_FLOATS], 16-byte aligned.  Other arguments as
 * streamkl_fwd. */
streamkl_status streamkl_fwd_partial(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                                     streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                                     const int64_t *strides, float tau_t, float tau_s, int causal,
                                     int k_begin, int k_end, float *state, void *stream);

/* Merge of n_states partial states per row, laid out [n_states][rows][6]
 * (device fp32), into kl_rows, lse_t, lse_s ([rows] fp32, as streamkl_fwd)
 * and, if kl_sum is not NULL, their deterministic sum. */
streamkl_status streamkl_fwd_merge(const float *states, int n_states, int64_t rows, float tau_t, float tau_s,
                                   float *kl_rows, float *lse_t, float *lse_s, float *kl_sum, void *stream);

/* Suggested number of key splits for streamkl_fwd_split on an MI355X (1 when
 * the unsplit forward already fills the GPU). */
int streamkl_fwd_split_count(int B, int H, int n_q, int n_k, int causal);

/* Workspace bytes streamkl_fwd_split needs: n_split * B * H * n_q * 6 * 4. */
size_t streamkl_fwd_split_workspace_size(int B, int H, int n_q, int n_split);

/* streamkl_fwd with the keys cut into n_split (1..64) equal ranges, one
 * launch over all of them (their states in the caller's workspace, 16-byte
 * aligned, at least streamkl_fwd_split_workspace_size bytes, else
 * STREAMKL_ERR_WORKSPACE), then the merge.  Same outputs as streamkl_fwd up to
 * rounding. */
streamkl_status streamkl_fwd_split(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                                   streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                                   const int64_t *strides, float tau_t, float tau_s, int causal, int n_split,
                                   void *workspace, size_t workspace_bytes, float *kl_rows, float *lse_t,
                                   float *lse_s, float *kl_sum, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * streamkl_fwd_split with the split states in a scratch array the library
 * holds on each GPU it runs on (STREAMKL_NOALLOC_SCRATCH_BYTES, a fixed
 * 16 MiB per GPU, kept until the process ends) instead of a caller workspace.
 * It allocates and frees nothing.  Arguments, outputs and errors as in
 * streamkl_fwd_split, except that STREAMKL_ERR_WORKSPACE means the states
 * (streamkl_fwd_split_workspace_size) would not fit in the scratch array, and
 * STREAMKL_ERR_HIP also covers a failure to locate the array on the current
 * device (the device the stream belongs to must be the current one).  Every
 * call on one GPU uses that GPU's single array: calls that overlap on one GPU
 * (on different streams, or from several host threads) race and must be
 * serialised by the caller; consecutive calls on one stream are safe. */
#define STREAMKL_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
streamkl_status streamkl_fwd_split_noalloc(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                                           streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                                           const int64_t *strides, float tau_t, float tau_s, int causal,
                                           int n_split, float *kl_rows, float *lse_t, float *lse_s, float *kl_sum,
                                           void *stream);

/*
 * Backward.  Gradients of L = sum_r g_r KL_r with respect to the student
 * queries and keys; the teacher is a fixed target and gets no gradient.  The
 * probabilities are recomputed tile by tile from the saved log-normalisers:
 *     dS[i][j] = g_r * tau_s * (P_s[j] - P_t[j])      (0 for masked keys)
 *     dq_s[i]  = sum_j dS[i][j] k_s[j],     dk_s[j] = sum_i dS[i][j] q_s[i]
 *
 *   q_t ... causal   exactly as passed to streamkl_fwd
 *   lse_t, lse_s     the forward's outputs for the same inputs
 *   grad_rows        [B,H,n_q] fp32 upstream gradient dL/dKL_r, or NULL to use
 *                    grad_scalar for every row (1.0 for L = kl_sum)
 *   dq_s, dk_s       out, input dtype, contiguous
 *
 * No workspace is used: one deterministic launch, with no atomics, holds both a
 * query-major block per 128 queries (dq_s) and a key-major block per 128 keys
 * (dk_s) of every head.  The query-major blocks recompute the scores, so no
 * dq_s partial sums cross blocks.  The alternative, key-major blocks only with
 * dq_s summed by fp32 atomics into a caller workspace, would need one atomic
 * add per query row, head-dimension element and 128-key block: 34 GB at
 * B=2, H=16, n_q=n_k=16384, d=128, which on MI355X takes about 25 ms on its
 * own, twice this whole backward.  So the call has no workspace arguments, and
 * streamkl_bwd_workspace_size (below) returns 0 for every shape.
 */
streamkl_status streamkl_bwd(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                             streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                             const int64_t *strides, float tau_t, float tau_s, int causal,
                             const float *lse_t, const float *lse_s,
                             const float *grad_rows, float grad_scalar,
                             void *dq_s, void *dk_s, void *stream);

/*
 * Backward with respect to the FIRST (teacher) distribution.  Gradients of the
 * same loss L = sum_r g_r KL_r with respect to the teacher queries and keys,
 * for callers that train the teacher as well, or that want the reverse
 * divergence.  From the forward-KL definition ("Lecture 05 - Where It All
 * Lands", section 3.1), with L_r[j] = log P_t[j] - log P_s[j]:
 *     dKL_r / ds_t[j] = P_t[j] (L_r[j] - KL_r)
 *     dS_t[i][j] = g_r * tau_t * P_t[j] * (s_t[j] - s_s[j] - LSE_t + LSE_s - KL_r)
 *     dq_t[i] = sum_j dS_t[i][j] k_t[j],     dk_t[j] = sum_i dS_t[i][j] q_t[i]
 * Reverse divergence: called with the two distributions swapped (student
 * tensors and tau_s in the teacher slots) after streamkl_fwd on the same
 * swapped arguments, it returns the student gradients of KL(P_s || P_t), the
 * mode-seeking direction of "Lecture 05", section 3.4.
 *
 *   q_t ... causal   exactly as passed to streamkl_fwd
 *   lse_t, lse_s,    the forward's outputs for the same inputs
 *   kl_rows
 *   grad_rows,       as in streamkl_bwd
 *   grad_scalar
 *   dq_t, dk_t       out, input dtype, contiguous [B,H,n_q,d_t] and [B,H,n_k,d_t]
 *
 * Same launch structure as streamkl_bwd (one deterministic launch, no
 * workspace, no atomics); errors as in streamkl_bwd, plus INVALID for a NULL
 * kl_rows.
 */
streamkl_status streamkl_bwd_teacher(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                                     streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                                     const int64_t *strides, float tau_t, float tau_s, int causal,
                                     const float *lse_t, const float *lse_s, const float *kl_rows,
                                     const float *grad_rows, float grad_scalar,
                                     void *dq_t, void *dk_t, void *stream);

/*
 * Grouped heads, per-batch lengths and packed sequences.  The pages define
 * the divergence per query row of one teacher and one student attention map
 * and say nothing of
 * how heads pair up when the two models, or the queries and keys of one
 * model, have different head counts; these entry points take the plainest
 * reading, the grouped-key convention.  There are H KL heads (the per-row
 * outputs are [B, H, n_q]); KL head h compares teacher query head
 * h / (H / heads_q_t) against student query head h / (H / heads_q_s), each
 * attending over its own model's key head h / (H / heads_k), so a model
 * with fewer query heads than H is broadcast over consecutive KL heads, and
 * keys are shared by consecutive query heads as in grouped-query attention.
 * Every heads_q divides H and every heads_k divides its model's heads_q.
 *
 * Tensors keep their own head counts: q_t [B, heads_q_t, n_q, d_t], k_t
 * [B, heads_k_t, n_k, d_t], q_s [B, heads_q_s, n_q, d_s], k_s [B, heads_k_s,
 * n_k, d_s]; default strides are contiguous in those shapes.  The gradient of
 * a shared head is the sum over the KL heads that read it: dq_s [B,
 * heads_q_s, n_q, d_s], dk_s [B, heads_k_s, n_k, d_s] (dq_t, dk_t likewise
 * with the teacher's counts).
 *
 * Padding: seqlen_q / seqlen_k (device int32 [B], NULL = n_q / n_k) give the
 * valid query rows and keys of each batch inside the padded n_q / n_k
 * (values are clamped to [0, n_q] / [0, n_k]).  Keys past seqlen_k[b] are
 * masked from both softmaxes; rows past seqlen_q[b] are empty.  The causal
 * mask is bottom-right aligned within the valid lengths
 * (j <= i + seqlen_k[b] - seqlen_q[b]).  An empty row (past the valid length,
 * or left with no allowed key) has KL 0 and LSEs 0, and contributes no
 * gradient; gradient rows past the valid lengths are written as 0.
 *
 * Packed sequences: cu_seqlens_q (device int32 [B + 1], NULL = padded) makes
 * the queries packed: batch b owns query rows cu_seqlens_q[b] ..
 * cu_seqlens_q[b + 1] - 1 of q_t [rows, heads_q_t, d_t] and q_s [rows,
 * heads_q_s, d_s] (n_q is then the longest sequence; a longer one is cut to
 * its first n_q rows, without an error: the offsets live in device memory
 * and are not read on the host), and dq_s / dq_t come back packed the same
 * way, contiguous.  Only the rows some sequence owns are written: rows before
 * cu_seqlens_q[0], past cu_seqlens_q[B], or past a cut sequence's n_q are
 * left as the caller allocated them (the Python binding passes zeroed
 * buffers, so they come back 0).  cu_seqlens_k does the same for the keys.  The batch
 * stride of a packed tensor is ignored (its rows are located by the
 * offsets); NULL strides mean contiguous [rows, heads, d].  A kind is either
 * packed or padded with lengths: seqlen_q together with cu_seqlens_q is
 * INVALID.  The per-row outputs (KL, LSEs, upstream gradients) stay padded
 * [B, H, n_q].
 */
typedef struct {
    int heads_q_t, heads_k_t, heads_q_s, heads_k_s;  /* 0 means H */
    const int32_t *seqlen_q, *seqlen_k;               /* device [B], 4-byte aligned, or NULL */
    const int32_t *cu_seqlens_q, *cu_seqlens_k;       /* device [B + 1], 4-byte aligned, or NULL */
} streamkl_layout;

/* streamkl_fwd with a layout (NULL layout = streamkl_fwd).  INVALID also for a
 * head count that is negative or breaks the divisibility above. */
streamkl_status streamkl_fwd_ex(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                                streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                                const int64_t *strides, const streamkl_layout *layout, float tau_t, float tau_s,
                                int causal, float *kl_rows, float *lse_t, float *lse_s, float *kl_sum,
                                void *stream);

/* Workspace bytes that streamkl_bwd_ex (first = 0) or streamkl_bwd_teacher_ex
 * (first = 1) can use for this shape and layout; 0 when none helps.  A
 * gradient block of a shared head loops over the KL heads that read it; when
 * such blocks are few (for instance one key head shared by every query head)
 * each group is split over several blocks that write fp32 partial sums here,
 * summed afterwards in a fixed order. */
size_t streamkl_bwd_ex_workspace_size(int B, int H, int n_q, int n_k, int d_t, int d_s,
                                      const streamkl_layout *layout, int first);

/* streamkl_bwd with a layout: dq_s, dk_s in the student's head counts.
 * workspace: device, 16-byte aligned, or NULL; with at least
 * streamkl_bwd_ex_workspace_size bytes long head groups are split (same
 * results up to rounding), otherwise they are not (no error). */
streamkl_status streamkl_bwd_ex(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                                streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                                const int64_t *strides, const streamkl_layout *layout, float tau_t, float tau_s,
                                int causal, const float *lse_t, const float *lse_s, const float *grad_rows,
                                float grad_scalar, void *dq_s, void *dk_s, void *workspace, size_t workspace_bytes,
                                void *stream);

/* streamkl_bwd_teacher with a layout: dq_t, dk_t in the teacher's head
 * counts; workspace as for streamkl_bwd_ex. */
streamkl_status streamkl_bwd_teacher_ex(const void *q_t, const void *k_t, const void *q_s, const void *k_s,
                                        streamkl_dtype dtype, int B, int H, int n_q, int n_k, int d_t, int d_s,
                                        const int64_t *strides, const streamkl_layout *layout, float tau_t,
                                        float tau_s, int causal, const float *lse_t, const float *lse_s,
                                        const float *kl_rows, const float *grad_rows, float grad_scalar, void *dq_t,
                                        void *dk_t, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Vocabulary-logit KL at temperature.  The distillation loss of "Lecture 05 -
 * Where It All Lands", section 3.1, applied to output logits: for every row r
 * of the teacher and student logit matrices z_t, z_s ([rows, V]),
 *
 *     p = softmax(z_t[r] / T),   q = softmax(z_s[r] / T),
 *     KL_r = sum_v p[v] (log p[v] - log q[v])   (nats, teacher first),
 *
 * in one streaming pass over each row with the same online (reference max,
 * normaliser, teacher-weighted accumulator) state as the attention forward; no
 * [rows, V] intermediate is written.  The T^2 factor of section 3.3 (and any
 * loss weight) is the caller's, through the upstream gradient.
 *
 * Conventions of the vocabulary entry points:
 *  - z_t, z_s: device pointers, dtype as `dtype` (shared), row r of z_t starts
 *    at z_t + r * ld_t elements (ld_t >= V), likewise z_s with ld_s; the V
 *    logits of a row are contiguous.  Pointers must be aligned to the element
 *    size.  16-byte aligned rows (base 16-byte aligned, ld and V multiples of 8)
 *    take the vectorised path; any other layout a slower element-wise path.
 *  - Logits must be finite (a vocabulary mask is expressed by a large negative
 *    finite logit, e.g. -1e4); temperature in [1e-4, 1e6].
 *  - Per-row outputs kl_rows, lse_t, lse_s (log-normalisers of z / T) and
 *    grad_rows are contiguous fp32 [rows]; gradients dz_s, dz_t are contiguous
 *    [rows, V] in the input dtype, overwritten.
 *  - rows >= 1, 1 <= V <= 2^30 (INVALID otherwise, as for a null pointer, a
 *    misaligned pointer or a bad temperature).  A row is owned by one wave
 *    (V < 4096, four rows per workgroup) or one workgroup; launches cover at
 *    most 2^20 rows each, so any row count is served by consecutive launches.
 *  - No workspace, no atomics, deterministic; stream and error behaviour as
 *    for the attention entry points.
 */

/* Forward: kl_rows, lse_t, lse_s (out, required) and, if kl_sum is not NULL,
 * their deterministic sum (one fp32 device scalar). */
streamkl_status streamkl_vocab_fwd(const void *z_t, const void *z_s, streamkl_dtype dtype, int64_t rows, int V,
                                   int64_t ld_t, int64_t ld_s, float temperature, float *kl_rows, float *lse_t,
                                   float *lse_s, float *kl_sum, void *stream);

/* Backward of L = sum_r g_r KL_r (g_r = grad_rows[r], or grad_scalar for
 * every row when grad_rows is NULL), recomputing p and q from the forward's
 * lse_t, lse_s:
 *     dz_s[r][v] = g_r / T * (q[v] - p[v])
 *     dz_t[r][v] = g_r / T * p[v] * ((z_t - z_s)[r][v] / T - LSE_t + LSE_s - KL_r)
 * dz_s: out, required.  dz_t: out, or NULL for student gradients only; when
 * given, kl_rows (the forward's) is required. */
streamkl_status streamkl_vocab_bwd(const void *z_t, const void *z_s, streamkl_dtype dtype, int64_t rows, int V,
                                   int64_t ld_t, int64_t ld_s, float temperature, const float *lse_t,
                                   const float *lse_s, const float *kl_rows, const float *grad_rows,
                                   float grad_scalar, void *dz_s, void *dz_t, void *stream);

/* Forward and backward in one launch, for callers that know the upstream
 * weights before the loss is computed (a plain sum or mean of the per-row KL,
 * with or without the T^2 factor): each row is read for the forward and again
 * for the gradients right after, while its logits are still in the caches.
 * Outputs as streamkl_vocab_fwd plus dz_s (required) and dz_t (optional) as
 * streamkl_vocab_bwd. */
streamkl_status streamkl_vocab_fwd_bwd(const void *z_t, const void *z_s, streamkl_dtype dtype, int64_t rows, int V,
                                       int64_t ld_t, int64_t ld_s, float temperature, const float *grad_rows,
                                       float grad_scalar, float *kl_rows, float *lse_t, float *lse_s,
                                       float *kl_sum, void *dz_s, void *dz_t, void *stream);

/* Bytes of device memory, beyond the caller's inputs and required outputs, that
 * the library needs for a call of this shape: always 0 here (the saved
 * log-normalisers are an output of streamkl_fwd). */
size_t streamkl_bwd_workspace_size(int B, int H, int n_q, int n_k, int d_t, int d_s,
                                   streamkl_dtype dtype, int causal);

/* Static, human-readable name of a status code. */
const char *streamkl_status_string(streamkl_status status);

/* 1 if (dtype, d_t, d_s) is built into this library, else 0. */
int streamkl_supported(streamkl_dtype dtype, int d_t, int d_s);

#ifdef __cplusplus
}
#endif

#endif /* STREAMKL_H */
