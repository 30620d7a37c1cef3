/*
 * kda.h - C ABI of the MI355X (gfx950) Kimi Delta Attention forward library.
 *
 * One call, kda_fwd(), runs the chunked KDA forward pass on the GPU: the
 * per-channel gated delta-rule recurrence over head dimension K = V = 128.
 * Per (sequence, head) chain and token t (state S is K x V, fp32):
 *
 *   a_t  = lower_bound * sigmoid(exp(A_log[h]) * (g_t + dt_bias[h,:]))
 *   S    = diag(exp(a_t)) S
 *   S    = S + sigmoid(beta_t) k_t (v_t - S^T k_t)^T
 *   o_t  = scale * S^T q_t
 *
 * Where each piece is defined (the FlashKDA pages):
 *   - the tensor contract, dtypes, shapes, contiguity, K = V = 128, the
 *     sigmoid on beta, the optional recurrent states and packed sequences:
 *     "FlashKDA Input Tensor Shapes and DTypes", all sections;
 *   - the gate, lower_bound in [-5, 0] and its log2 rescaling
 *     gate_scale = lower_bound * log2(e): "FlashKDA lower_bound Parameter",
 *     "Conversion to the Gate Scale Factor" and the FAQ on dt_bias;
 *   - the base-2 exponent: "Base-2 Exponent Optimization in FlashKDA",
 *     "Re-basing the Gate Activation";
 *   - chunks of 16 tokens and the 16x16 unit-triangular inverse:
 *     "How FlashKDA's CHUNK Size of 16 Improves Numerical Stability",
 *     "Efficient 16x16 Matrix Inversion".
 * The pages never write the delta-rule update or the place of A_log; the
 * library takes the reading above (A_log multiplies the biased gate inside
 * the sigmoid; decay, then write with the decayed state, then read).
 *
 * Ownership and threading: the caller owns every buffer.  All tensor
 * pointers are DEVICE pointers to contiguous row-major memory on the current
 * HIP device.  The library allocates nothing, reads no environment
 * variables, never synchronises and is safe to call from several host
 * threads; apart from kda_fwd_scan_static (one fixed scratch array per GPU,
 * shared by its calls, see there) it keeps no state between calls.  The
 * work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 * and completes asynchronously.
 */
#ifndef KDA_H
#define KDA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes.  Every argument error is detected on the host, before any
 * work is enqueued, and leaves every buffer untouched. */
typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL_POINTER = 1,  /* q, k, v, g, beta or out is NULL while T > 0,
                                  or a state pointer is given with dtype
                                  KDA_DTYPE_NONE */
    KDA_ERR_HEAD_DIM = 2,      /* K != 128 or V != 128 */
    KDA_ERR_LOWER_BOUND = 3,   /* lower_bound outside [-5, 0], or NaN */
    KDA_ERR_VARLEN_BATCH = 4,  /* cu_seqlens given with B != 1, or num_seqs < 0 */
    KDA_ERR_STATE_DTYPE = 5,   /* unknown state dtype, or initial_state and
                                  final_state both given with different dtypes */
    KDA_ERR_ALIAS = 6,         /* out or final_state overlaps an input, or
                                  final_state partly overlaps initial_state */
    KDA_ERR_SIZE = 7,          /* B < 1, H < 1, H > 65536, T < 0 or
                                  T > 2^31-1, sizes overflow int64, or more
                                  than 2^31-1 (sequence, head) chains */
    KDA_ERR_SCALE = 8,         /* scale is not finite */
    KDA_ERR_LAUNCH = 9,        /* the HIP runtime rejected the launch */
    KDA_ERR_WORKSPACE = 10,    /* kda_fwd_scan: workspace NULL, not 16-byte
                                  aligned, smaller than
                                  kda_fwd_scan_workspace_bytes(), or
                                  overlapping a tensor argument */
    KDA_ERR_ALIGNMENT = 11,    /* a non-NULL pointer is misaligned: q, k, v,
                                  g, out, initial_state and final_state need
                                  16 bytes, beta 2, A_log and dt_bias 4,
                                  cu_seqlens 8 (allocator memory and whole
                                  token rows of it always are) */
    KDA_ERR_OPTION = 12        /* kda_options: an unknown value, a non-zero
                                  reserved field, or a kernel / inverse /
                                  sigmoid combination that no kernel of the
                                  library implements for this call */
} kda_status;

/* Element type of initial_state / final_state. */
typedef enum kda_dtype {
    KDA_DTYPE_NONE = 0,
    KDA_DTYPE_BF16 = 1,
    KDA_DTYPE_FP32 = 2
} kda_dtype;

/*
 * Explicit choices for kda_fwd_ex and kda_fwd_scan (a NULL options pointer
 * means all defaults, which is what kda_fwd uses).  They change how the
 * same result is computed, never what is computed: the kernel, and two of
 * the pages' own design choices kept as ablations.
 *
 *   kernel   KDA_KERNEL_AUTO: decode-shaped calls (no cu_seqlens, at most
 *            16 tokens), where the state traffic dominates, take the token
 *            recurrence (at most 8 tokens) or the single-chunk kernel; all
 *            other calls the pipelined chunked kernel.  CHUNKED, RECURRENT
 *            and SINGLE force one kernel; SINGLE takes only calls without
 *            cu_seqlens of at most 16 tokens.
 *   inverse  how the chunked kernels form the unit lower-triangular 16x16
 *            inverse (I + A)^-1: fp32 forward substitution (default), or the
 *            fp16 Neumann-series product the chunk-size page describes under
 *            "Efficient 16x16 Matrix Inversion" (pipelined chunked kernel
 *            only).
 *   sigmoid  how the gate evaluates the logistic function: 1/(1 + 2^-x') with
 *            the hardware exp2 and reciprocal (default), or 1/2 + tanh(x/2)/2
 *            with a rational tanh, the tanh form the lower_bound page names
 *            (whole-chain calls of the chunked and single-chunk kernels,
 *            forward substitution only).
 *   reserved must be 0.
 *
 * With KDA_KERNEL_AUTO a non-default inverse or sigmoid restricts the choice
 * to the kernels that implement it; a forced kernel that does not implement
 * the requested combination, or cannot take the call, gives KDA_ERR_OPTION.
 */
typedef enum kda_kernel {
    KDA_KERNEL_AUTO = 0,
    KDA_KERNEL_CHUNKED = 1,
    KDA_KERNEL_RECURRENT = 2,
    KDA_KERNEL_SINGLE = 3
} kda_kernel;

typedef enum kda_inverse {
    KDA_INVERSE_SUBSTITUTION = 0,
    KDA_INVERSE_NEUMANN = 1
} kda_inverse;

typedef enum kda_sigmoid {
    KDA_SIGMOID_EXP2 = 0,
    KDA_SIGMOID_TANH = 1
} kda_sigmoid;

typedef struct kda_options {
    int32_t kernel;   /* kda_kernel */
    int32_t inverse;  /* kda_inverse */
    int32_t sigmoid;  /* kda_sigmoid */
    int32_t reserved; /* 0 */
} kda_options;

/*
 * kda_fwd - chunked KDA forward pass.
 *
 *   q, k, g      bf16 [B,T,H,K]; v bf16 [B,T,H,V]; channel index fastest.
 *   beta         bf16 [B,T,H], logits (the sigmoid is applied inside).
 *   scale        finite scalar applied to the read-out, o = scale * S^T q.
 *   out          bf16 [B,T,H,V], written (round to nearest even).  Rows of
 *                a packed batch that lie outside every sequence are not
 *                written.
 *   A_log        fp32 [H] or NULL (NULL acts as A_log = 0).
 *   dt_bias      fp32 [H,K] or NULL (NULL acts as 0).
 *   lower_bound  in [-5, 0]; 0 turns the decay off.
 *   initial_state  [N,H,V,K] of initial_state_dtype (bf16 or fp32), stored
 *                transposed: element [n,h,v,k] is S[k][v].  NULL = zero.
 *   final_state  [N,H,V,K] of final_state_dtype, written with the state
 *                after the last token of each sequence (bf16: round to
 *                nearest even).  NULL = not written.  It may be the same
 *                buffer as initial_state (in-place update) but must not
 *                partly overlap it.
 *   cu_seqlens   NULL for batch mode (N = B sequences of length T), or a
 *                device int64 [num_seqs+1] of sequence start offsets into
 *                the packed token axis (B must be 1; N = num_seqs).  Its
 *                contents are not read on the host: they should be
 *                nondecreasing from 0 to T; the kernels clamp every segment
 *                to [0, T], so bad contents give wrong results, never an
 *                out-of-bounds access.
 *   B, T, H      sizes; T may be 0 (then only final_state is written).
 *   K, V         head dimensions; must both be 128.
 *   stream       hipStream_t to enqueue on (NULL = default stream).
 *
 * Returns KDA_OK once the work is enqueued, or an error code (nothing
 * enqueued).  num_seqs is ignored in batch mode.
 */
kda_status kda_fwd(const void *q, const void *k, const void *v, const void *g,
                   const void *beta, double scale, void *out,
                   const float *A_log, const float *dt_bias, double lower_bound,
                   const void *initial_state, kda_dtype initial_state_dtype,
                   void *final_state, kda_dtype final_state_dtype,
                   const int64_t *cu_seqlens, int64_t num_seqs,
                   int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                   void *stream);

/*
 * kda_fwd_ex - kda_fwd with explicit options (NULL = the defaults, which is
 * exactly kda_fwd).  Same arguments, results and errors as kda_fwd, plus
 * KDA_ERR_OPTION.
 */
kda_status kda_fwd_ex(const void *q, const void *k, const void *v, const void *g,
                      const void *beta, double scale, void *out,
                      const float *A_log, const float *dt_bias, double lower_bound,
                      const void *initial_state, kda_dtype initial_state_dtype,
                      void *final_state, kda_dtype final_state_dtype,
                      const int64_t *cu_seqlens, int64_t num_seqs,
                      int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                      const kda_options *options, void *stream);

/*
 * kda_fwd_scan - the same forward pass as kda_fwd (same arguments, same
 * results up to rounding), computed with parallelism inside each sequence:
 * for workloads with few (sequence, head) chains, where kda_fwd leaves most
 * of the GPU idle.
 *
 * Each chain is cut into segments of seg_chunks chunks (16 tokens each).
 * The recurrence above is affine in the state, so a segment maps its start
 * state S to M S + b.  The call enqueues three steps on `stream`: one pass
 * that computes b for every segment but the last (segment 0 from the real
 * initial state, the others from zero) and M for the inner segments (the
 * state update with v set to zero, from an identity start), a combine step
 * that walks each chain's segments in order (start of segment s+1 =
 * M_s * start of s + b_s), and the output pass, every segment from its true
 * start state (two steps when no chain has more than two segments).  b and
 * the combined states stay fp32; M and the running state enter the combine
 * as hi + lo bf16 pairs (about 17 significant bits each), so the results
 * match kda_fwd's to within the rounding of the bf16 matrix operands both
 * forms use.  The first pass also keeps a copy of each chain's initial
 * state in the workspace, which the output pass reads: final_state may be
 * the initial_state buffer here too.
 *
 *   seg_chunks       chunks per segment, >= 1 (KDA_ERR_SIZE otherwise).  One
 *                    segment per chain (seg_chunks >= ceil(T / 16)) is exactly
 *                    kda_fwd.
 *   workspace        DEVICE scratch owned by the caller, 16-byte aligned, at
 *                    least kda_fwd_scan_workspace_bytes() bytes, not
 *                    overlapping any tensor argument.  Its contents on entry
 *                    are ignored and on return are unspecified; it must not be
 *                    used by other work until the call's work has completed
 *                    on `stream`.
 *   workspace_bytes  its size in bytes.
 *   options          as for kda_fwd_ex (NULL = defaults); the segmented
 *                    form runs the pipelined chunked kernel, so the kernel
 *                    must be AUTO or CHUNKED and the sigmoid EXP2
 *                    (KDA_ERR_OPTION otherwise).
 * Every other argument, the ownership rules and the error codes are those of
 * kda_fwd, plus KDA_ERR_WORKSPACE and KDA_ERR_OPTION.
 */
kda_status kda_fwd_scan(const void *q, const void *k, const void *v, const void *g,
                        const void *beta, double scale, void *out,
                        const float *A_log, const float *dt_bias, double lower_bound,
                        const void *initial_state, kda_dtype initial_state_dtype,
                        void *final_state, kda_dtype final_state_dtype,
                        const int64_t *cu_seqlens, int64_t num_seqs,
                        int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                        int64_t seg_chunks, void *workspace, int64_t workspace_bytes,
                        const kda_options *options, void *stream);

/*
 * kda_fwd_scan_static - kda_fwd_scan without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  The scratch the
 * segmented form needs (kda_fwd_scan_workspace_bytes() for these sizes) is
 * taken from a fixed device array of the library, KDA_SCAN_STATIC_BYTES per
 * GPU, which each GPU the library runs on holds until the process ends; the
 * call itself allocates nothing.  Calls whose scratch would exceed it return
 * KDA_ERR_WORKSPACE (nothing enqueued); the automatic segment length of the
 * Python binding keeps about 256 (chain, segment) pairs, i.e. 32 MiB.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, or different host threads without ordering)
 * race on it and give wrong results; calls ordered on one stream are safe.
 * Nothing in the array needs to start at zero (each call writes every slab
 * before reading it).  Same arguments (minus the workspace), results and
 * other errors as kda_fwd_scan; KDA_ERR_LAUNCH if the array's device address
 * cannot be looked up on the current device.
 */
#define KDA_SCAN_STATIC_BYTES (32ll << 20)
kda_status kda_fwd_scan_static(const void *q, const void *k, const void *v, const void *g,
                               const void *beta, double scale, void *out,
                               const float *A_log, const float *dt_bias, double lower_bound,
                               const void *initial_state, kda_dtype initial_state_dtype,
                               void *final_state, kda_dtype final_state_dtype,
                               const int64_t *cu_seqlens, int64_t num_seqs,
                               int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                               int64_t seg_chunks, const kda_options *options, void *stream);

/*
 * Bytes of workspace kda_fwd_scan needs for these sizes: two fp32 128x128
 * slabs per (chain, segment), with ceil(ceil(T/16) / seg_chunks) segments per
 * chain (every sequence has at most T tokens).  cu_seqlens is only tested for
 * NULL (batch mode: N = B chains per head) and never read.  Returns -1 for
 * seg_chunks < 1, negative sizes or overflow.
 */
int64_t kda_fwd_scan_workspace_bytes(const int64_t *cu_seqlens, int64_t num_seqs,
                                     int64_t B, int64_t T, int64_t H, int64_t seg_chunks);

/* Static, NUL-terminated description of a status code. */
const char *kda_status_string(kda_status status);

/*
 * Name of the kernel kda_fwd_ex runs for a call with T tokens per batch row
 * (varlen != 0: cu_seqlens given) and these options (NULL = defaults, i.e.
 * kda_fwd's choice): "recurrent" (the token recurrence itself), "single"
 * (the chunked stages for one chunk, one small workgroup per chain) or
 * "mfma" (the pipelined chunked kernel); see kda_options.  Returns NULL when
 * the options are invalid for such a call (kda_fwd_ex would return
 * KDA_ERR_OPTION).  A static string; pure host logic, no device work.
 * kda_fwd_scan always runs the chunked kernel.
 */
const char *kda_fwd_kernel(int64_t T, int varlen, const kda_options *options);

/* ABI version of this header (bumped on any signature change). */
#define KDA_ABI_VERSION 4
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
