// C-ABI front end of the KDA forward library: argument checks, the log2 gate
// scale, and the hand-off to the kernels.  Every check runs on the host
// before anything is enqueued; nothing here touches device memory.
#include "kda.h"

#include <cmath>
#include <cstdint>

#include "kda_internal.h"

namespace {

constexpr double kLog2e = 1.4426950408889634;  // 1 / ln 2

bool mul_ok(int64_t a, int64_t b, int64_t *r) { return !__builtin_mul_overflow(a, b, r); }

// Byte range [lo, hi) of a buffer.
struct Span {
    uintptr_t lo = 0, hi = 0;
    bool overlaps(const Span &o) const { return lo < o.hi && o.lo < hi; }
};

Span span(const void *p, int64_t bytes)
{
    Span s;
    if (p && bytes > 0) {
        s.lo = reinterpret_cast<uintptr_t>(p);
        s.hi = s.lo + static_cast<uintptr_t>(bytes);
    }
    return s;
}

bool valid_kind(kda_dtype d) { return d == KDA_DTYPE_BF16 || d == KDA_DTYPE_FP32; }

// Validated arguments of a forward call, and the byte ranges the alias
// checks need.
struct Checked {
    kda::FwdParams p;
    int64_t chains = 0;
    Span spans[11];  // inputs, out, final_state, initial_state
    int n_spans = 0;
};

kda_status check_args(const void *q, const void *k, const void *v, const void *g, const void *beta,
                      double scale, void *out, const float *A_log, const float *dt_bias,
                      double lower_bound, const void *initial_state, kda_dtype initial_state_dtype,
                      void *final_state, kda_dtype final_state_dtype, const int64_t *cu_seqlens,
                      int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                      Checked *c)
{
    if (K != kda::kHeadDim || V != kda::kHeadDim)
        return KDA_ERR_HEAD_DIM;
    // NaN fails both comparisons and is rejected too.
    if (!(lower_bound >= -5.0 && lower_bound <= 0.0))
        return KDA_ERR_LOWER_BOUND;
    if (!std::isfinite(scale))
        return KDA_ERR_SCALE;
    if (B < 1 || H < 1 || H > 65536 || T < 0 || T > INT32_MAX)
        return KDA_ERR_SIZE;
    if (cu_seqlens && (B != 1 || num_seqs < 0))
        return KDA_ERR_VARLEN_BATCH;
    if (initial_state && !valid_kind(initial_state_dtype))
        return initial_state_dtype == KDA_DTYPE_NONE ? KDA_ERR_NULL_POINTER : KDA_ERR_STATE_DTYPE;
    if (final_state && !valid_kind(final_state_dtype))
        return final_state_dtype == KDA_DTYPE_NONE ? KDA_ERR_NULL_POINTER : KDA_ERR_STATE_DTYPE;
    if (initial_state && final_state && initial_state_dtype != final_state_dtype)
        return KDA_ERR_STATE_DTYPE;

    const int64_t N = cu_seqlens ? num_seqs : B;
    // rows = B*T*H token-head rows; act_bytes = bytes of one bf16 [B,T,H,128]
    // tensor; state_f32_bytes = bytes of an fp32 [N,H,128,128] state.
    int64_t tokens, rows, act_bytes, beta_bytes, chains, state_f32_bytes;
    if (!mul_ok(B, T, &tokens) || !mul_ok(tokens, H, &rows) ||
        !mul_ok(rows, 128 * 2, &act_bytes) || !mul_ok(rows, 2, &beta_bytes) ||
        !mul_ok(N, H, &chains) || !mul_ok(chains, 128 * 128 * 4, &state_f32_bytes) ||
        chains > INT32_MAX)
        return KDA_ERR_SIZE;
    // Token tensors may be NULL only when they are empty (T == 0).
    if (rows > 0 && (!q || !k || !v || !g || !beta || !out))
        return KDA_ERR_NULL_POINTER;
    const int64_t init_bytes =
        initial_state ? state_f32_bytes / (initial_state_dtype == KDA_DTYPE_BF16 ? 2 : 1) : 0;
    const int64_t final_bytes =
        final_state ? state_f32_bytes / (final_state_dtype == KDA_DTYPE_BF16 ? 2 : 1) : 0;

    const Span inputs[] = {span(q, act_bytes), span(k, act_bytes), span(v, act_bytes),
                           span(g, act_bytes), span(beta, beta_bytes),
                           span(A_log, A_log ? H * 4 : 0), span(dt_bias, dt_bias ? H * 512 : 0),
                           span(cu_seqlens, cu_seqlens ? (N + 1) * 8 : 0)};
    const Span so = span(out, act_bytes), sf = span(final_state, final_bytes),
               si = span(initial_state, init_bytes);
    for (const Span &s : inputs) {
        if (so.overlaps(s) || sf.overlaps(s))
            return KDA_ERR_ALIAS;
    }
    if (so.overlaps(sf) || so.overlaps(si))
        return KDA_ERR_ALIAS;
    if (sf.overlaps(si) && final_state != initial_state)
        return KDA_ERR_ALIAS;
    // The kernels move q, k, v, g, out and the states in pieces of up to 16
    // bytes; beta, A_log, dt_bias and cu_seqlens are read element by element.
    const auto misaligned = [](const void *ptr, uintptr_t a) {
        return ptr != nullptr && reinterpret_cast<uintptr_t>(ptr) % a != 0;
    };
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(g, 16) ||
        misaligned(out, 16) || misaligned(initial_state, 16) || misaligned(final_state, 16) ||
        misaligned(beta, 2) || misaligned(A_log, 4) || misaligned(dt_bias, 4) ||
        misaligned(cu_seqlens, 8))
        return KDA_ERR_ALIGNMENT;
    for (const Span &s : inputs) c->spans[c->n_spans++] = s;
    c->spans[c->n_spans++] = so;
    c->spans[c->n_spans++] = sf;
    c->spans[c->n_spans++] = si;

    kda::FwdParams &p = c->p;
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.g = static_cast<const uint16_t *>(g);
    p.beta = static_cast<const uint16_t *>(beta);
    p.out = static_cast<uint16_t *>(out);
    p.A_log = A_log;
    p.dt_bias = dt_bias;
    p.init_state = initial_state;
    p.final_state = final_state;
    p.init_kind = initial_state ? static_cast<int>(initial_state_dtype) : kda::kStateNone;
    p.final_kind = final_state ? static_cast<int>(final_state_dtype) : kda::kStateNone;
    p.cu_seqlens = cu_seqlens;
    p.num_seqs = N;
    p.T = T;
    p.H = H;
    p.scale = static_cast<float>(scale);
    // The gate is carried in log2 units so that every decay is a plain exp2
    // (lower_bound page, "Conversion to the Gate Scale Factor").
    p.gate_scale = static_cast<float>(lower_bound * kLog2e);
    c->chains = chains;
    return KDA_OK;
}

// The kernel a kda_fwd_ex call with these options runs (kda::Kernel), or -1
// when the options are invalid for the call: an unknown value, a non-zero
// reserved field, or a combination no kernel implements.  Decode-shaped
// calls (no cu_seqlens, at most one chunk per sequence) go to the token
// recurrence up to kRecurrentMaxTokens tokens and to the single-chunk kernel
// up to 16; the rest to the pipelined chunked kernel.  The Neumann inverse
// exists in the chunked kernel only; the tanh-form sigmoid in the chunked
// (forward substitution) and single-chunk kernels.
int choose_kernel(const kda_options *options, int64_t T, bool varlen)
{
    const kda_options none = {KDA_KERNEL_AUTO, KDA_INVERSE_SUBSTITUTION, KDA_SIGMOID_EXP2, 0};
    const kda_options &o = options ? *options : none;
    if (o.reserved != 0 || (o.inverse != KDA_INVERSE_SUBSTITUTION && o.inverse != KDA_INVERSE_NEUMANN) ||
        (o.sigmoid != KDA_SIGMOID_EXP2 && o.sigmoid != KDA_SIGMOID_TANH))
        return -1;
    const bool neumann = o.inverse == KDA_INVERSE_NEUMANN, tanh_form = o.sigmoid == KDA_SIGMOID_TANH;
    if (neumann && tanh_form)
        return -1;
    const bool one_chunk = !varlen && T <= kda::kChunk;
    const bool recurrent_ok = !neumann && !tanh_form, single_ok = one_chunk && !neumann;
    switch (o.kernel) {
    case KDA_KERNEL_AUTO:
        if (recurrent_ok && !varlen && T <= kda::kRecurrentMaxTokens)
            return kda::kKernelRecurrent;
        return single_ok ? kda::kKernelSingle : kda::kKernelChunked;
    case KDA_KERNEL_CHUNKED: return kda::kKernelChunked;
    case KDA_KERNEL_RECURRENT: return recurrent_ok ? kda::kKernelRecurrent : -1;
    case KDA_KERNEL_SINGLE: return single_ok ? kda::kKernelSingle : -1;
    default: return -1;
    }
}

void apply_forms(const kda_options *options, kda::FwdParams *p)
{
    p->inverse = options && options->inverse == KDA_INVERSE_NEUMANN ? kda::kInverseNeumann : kda::kInverseSubst;
    p->sigmoid = options && options->sigmoid == KDA_SIGMOID_TANH ? kda::kSigmoidTanh : kda::kSigmoidExp;
}

// Segments per chain for segments of seg_chunks chunks: every sequence has
// at most T tokens.  -1 if seg_chunks < 1.
int64_t segments_per_chain(int64_t T, int64_t seg_chunks)
{
    if (seg_chunks < 1)
        return -1;
    const int64_t chunks = (T + kda::kChunk - 1) / kda::kChunk;
    return chunks > 0 ? (chunks + seg_chunks - 1) / seg_chunks : 1;
}

constexpr int64_t kSlabBytes = int64_t(kda::kHeadDim) * kda::kHeadDim * 4;  // one fp32 state

}  // namespace

extern "C" kda_status kda_fwd_ex(const void *q, const void *k, const void *v, const void *g,
                                 const void *beta, double scale, void *out, const float *A_log,
                                 const float *dt_bias, double lower_bound,
                                 const void *initial_state, kda_dtype initial_state_dtype,
                                 void *final_state, kda_dtype final_state_dtype,
                                 const int64_t *cu_seqlens, int64_t num_seqs, int64_t B,
                                 int64_t T, int64_t H, int64_t K, int64_t V,
                                 const kda_options *options, void *stream)
{
    Checked c;
    const kda_status st = check_args(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
                                     initial_state, initial_state_dtype, final_state,
                                     final_state_dtype, cu_seqlens, num_seqs, B, T, H, K, V, &c);
    if (st != KDA_OK)
        return st;
    const int kernel = choose_kernel(options, T, cu_seqlens != nullptr);
    if (kernel < 0)
        return KDA_ERR_OPTION;
    apply_forms(options, &c.p);
    if (c.chains == 0)
        return KDA_OK;
    hipError_t err = kda::launch_forward(c.p, kernel, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

extern "C" kda_status kda_fwd(const void *q, const void *k, const void *v, const void *g,
                              const void *beta, double scale, void *out, const float *A_log,
                              const float *dt_bias, double lower_bound,
                              const void *initial_state, kda_dtype initial_state_dtype,
                              void *final_state, kda_dtype final_state_dtype,
                              const int64_t *cu_seqlens, int64_t num_seqs, int64_t B,
                              int64_t T, int64_t H, int64_t K, int64_t V, void *stream)
{
    return kda_fwd_ex(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                      initial_state_dtype, final_state, final_state_dtype, cu_seqlens, num_seqs, B,
                      T, H, K, V, nullptr, stream);
}

extern "C" int64_t kda_fwd_scan_workspace_bytes(const int64_t *cu_seqlens, int64_t num_seqs,
                                                int64_t B, int64_t T, int64_t H,
                                                int64_t seg_chunks)
{
    const int64_t n_seg = segments_per_chain(T, seg_chunks);
    const int64_t N = cu_seqlens ? num_seqs : B;
    int64_t chains, slabs, bytes;
    if (n_seg < 0 || N < 0 || H < 1 || T < 0 || !mul_ok(N, H, &chains) ||
        !mul_ok(chains, n_seg, &slabs) || !mul_ok(slabs, 2 * kSlabBytes, &bytes))
        return -1;
    return bytes;
}

namespace {

// kda_fwd_scan's checks and launch, with the workspace given (workspace !=
// nullptr) or, for the static variant, taken from the library's fixed
// scratch (workspace == nullptr, capacity = its size).
kda_status fwd_scan(const void *q, const void *k, const void *v, const void *g, const void *beta,
                    double scale, void *out, const float *A_log, const float *dt_bias,
                    double lower_bound, const void *initial_state, kda_dtype initial_state_dtype,
                    void *final_state, kda_dtype final_state_dtype, const int64_t *cu_seqlens,
                    int64_t num_seqs, int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                    int64_t seg_chunks, void *workspace, int64_t workspace_bytes, bool use_static,
                    const kda_options *options, void *stream)
{
    Checked c;
    const kda_status st = check_args(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
                                     initial_state, initial_state_dtype, final_state,
                                     final_state_dtype, cu_seqlens, num_seqs, B, T, H, K, V, &c);
    if (st != KDA_OK)
        return st;
    // the segmented form runs the pipelined chunked kernel (exp2 sigmoid)
    if (options && ((options->kernel != KDA_KERNEL_AUTO && options->kernel != KDA_KERNEL_CHUNKED) ||
                    options->sigmoid != KDA_SIGMOID_EXP2 ||
                    choose_kernel(options, T, cu_seqlens != nullptr) < 0))
        return KDA_ERR_OPTION;
    apply_forms(options, &c.p);
    const int64_t n_seg = segments_per_chain(T, seg_chunks);
    int64_t blocks;
    // grids: chains * n_seg blocks for the map and output passes, chains * 8
    // for the combine step (run with more than two segments)
    if (n_seg < 0 || !mul_ok(c.chains, n_seg, &blocks) || blocks > INT32_MAX ||
        (n_seg > 2 && c.chains > INT32_MAX / 8))
        return KDA_ERR_SIZE;
    const int64_t need = blocks * 2 * kSlabBytes;
    if (use_static) {
        if (need > kda::kStaticScratchBytes)
            return KDA_ERR_WORKSPACE;
        if (c.chains == 0)
            return KDA_OK;
        if (kda::static_scratch(&workspace) != hipSuccess)
            return KDA_ERR_LAUNCH;
    } else {
        if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
            return KDA_ERR_WORKSPACE;
        const Span sw = span(workspace, need);
        for (int i = 0; i < c.n_spans; ++i) {
            if (sw.overlaps(c.spans[i]))
                return KDA_ERR_WORKSPACE;
        }
        if (c.chains == 0)
            return KDA_OK;
    }
    kda::FwdParams &p = c.p;
    p.seg_chunks = seg_chunks;
    p.n_seg = n_seg;
    p.seg_b = static_cast<float *>(workspace);
    p.seg_m = p.seg_b + blocks * (kSlabBytes / 4);
    hipError_t err = n_seg == 1 ? kda::launch_chunk_mfma(p, static_cast<hipStream_t>(stream))
                                : kda::launch_forward_scan(p, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace

extern "C" kda_status kda_fwd_scan(const void *q, const void *k, const void *v, const void *g,
                                   const void *beta, double scale, void *out, const float *A_log,
                                   const float *dt_bias, double lower_bound,
                                   const void *initial_state, kda_dtype initial_state_dtype,
                                   void *final_state, kda_dtype final_state_dtype,
                                   const int64_t *cu_seqlens, int64_t num_seqs, int64_t B,
                                   int64_t T, int64_t H, int64_t K, int64_t V, int64_t seg_chunks,
                                   void *workspace, int64_t workspace_bytes,
                                   const kda_options *options, void *stream)
{
    return fwd_scan(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                    initial_state_dtype, final_state, final_state_dtype, cu_seqlens, num_seqs, B, T,
                    H, K, V, seg_chunks, workspace, workspace_bytes, false, options, stream);
}

extern "C" kda_status kda_fwd_scan_static(const void *q, const void *k, const void *v, const void *g,
                                          const void *beta, double scale, void *out,
                                          const float *A_log, const float *dt_bias, double lower_bound,
                                          const void *initial_state, kda_dtype initial_state_dtype,
                                          void *final_state, kda_dtype final_state_dtype,
                                          const int64_t *cu_seqlens, int64_t num_seqs, int64_t B,
                                          int64_t T, int64_t H, int64_t K, int64_t V,
                                          int64_t seg_chunks, const kda_options *options,
                                          void *stream)
{
    return fwd_scan(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                    initial_state_dtype, final_state, final_state_dtype, cu_seqlens, num_seqs, B, T,
                    H, K, V, seg_chunks, nullptr, 0, true, options, stream);
}

extern "C" const char *kda_status_string(kda_status status)
{
    switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL_POINTER: return "a required pointer is NULL (or a state has no dtype)";
    case KDA_ERR_HEAD_DIM: return "K and V must both be 128";
    case KDA_ERR_LOWER_BOUND: return "lower_bound must lie in [-5, 0]";
    case KDA_ERR_VARLEN_BATCH: return "cu_seqlens requires B == 1 and num_seqs >= 0";
    case KDA_ERR_STATE_DTYPE: return "state dtype must be bf16 or fp32, and match between initial and final";
    case KDA_ERR_ALIAS: return "an output buffer overlaps an input buffer";
    case KDA_ERR_SIZE: return "bad size (B >= 1, 1 <= H <= 65536, 0 <= T < 2^31, no int64 overflow)";
    case KDA_ERR_SCALE: return "scale must be finite";
    case KDA_ERR_LAUNCH: return "the HIP runtime rejected the kernel launch";
    case KDA_ERR_WORKSPACE: return "workspace is NULL, not 16-byte aligned, too small, or overlaps a tensor";
    case KDA_ERR_ALIGNMENT: return "a tensor pointer is misaligned (q, k, v, g, out, states: 16 bytes; beta 2; A_log, dt_bias 4; cu_seqlens 8)";
    case KDA_ERR_OPTION: return "invalid options: unknown value, non-zero reserved field, or a kernel / inverse / sigmoid combination not implemented for this call";
    }
    return "unknown status";
}

extern "C" int kda_abi_version(void) { return KDA_ABI_VERSION; }

namespace kda {
hipError_t launch_forward(const FwdParams &p, int kernel, hipStream_t stream)
{
    switch (kernel) {
    case kKernelRecurrent: return launch_decode(p, stream);
    case kKernelSingle: return launch_chunk_single(p, stream);
    default: return launch_chunk_mfma(p, stream);
    }
}

// The segmented form: map (end states and, with more than two segments,
// transition matrices, in one pass), combine, output; three launches in
// order on one stream (two when no chain has more than two segments).
hipError_t launch_forward_scan(const FwdParams &p, hipStream_t stream)
{
    FwdParams s = p;
    s.phase = p.n_seg > 2 ? kPhaseMapBM : kPhaseMapB;
    hipError_t err = launch_chunk_mfma(s, stream);
    if (err == hipSuccess && p.n_seg > 2)
        err = launch_scan_combine(s, stream);
    if (err == hipSuccess) {
        s.phase = kPhaseOut;
        err = launch_chunk_mfma(s, stream);
    }
    return err;
}
}  // namespace kda

extern "C" const char *kda_fwd_kernel(int64_t T, int varlen, const kda_options *options)
{
    switch (choose_kernel(options, T, varlen != 0)) {
    case kda::kKernelRecurrent: return "recurrent";
    case kda::kKernelSingle: return "single";
    case kda::kKernelChunked: return "mfma";
    default: return nullptr;
    }
}
