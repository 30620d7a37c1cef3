// Recurrent KDA forward kernel for decode-shaped calls: a few tokens per
// sequence, the state carried in and out.
//
// Such a call is dominated by the state: 64 KiB of fp32 read and 64 KiB
// written per (sequence, head) chain, against 1 KiB of q, k, v, g per token.
// What matters is that the state traffic of many chains is in flight at once.
// The chunked kernel holds one chain per compute unit behind a five-stage
// pipeline whose fill alone outlasts a handful of tokens; this kernel runs the
// token recurrence directly, with one 256-thread workgroup and about 20 KiB of
// LDS per chain, so that several chains share a compute unit and the state
// loads and stores of one overlap the arithmetic of the others.
//
// The recurrence, per token i of a chain (decay first, the delta write with
// the decayed state, the read after the write; input-tensor page and
// lower_bound page, "Conversion to the Gate Scale Factor"):
//   S <- diag(alpha_i) S;  u = v_i - S^T k_i;  S <- S + beta_i k_i u^T;
//   o_i = scale S^T q_i
// with alpha_i = 2^(a_i) per channel, a_i in log2 units.  Within a pass of up
// to kPassTokens tokens the state is kept as S = diag(Gamma_i) Shat, Gamma_i
// the product of the pass's decays up to token i, so that a token costs three
// fp32 multiply-adds per state element instead of four:
//   u = v_i - Shat^T (Gamma_i k_i);  Shat += (beta_i k_i / Gamma_i) u^T;
//   o_i = Shat^T (scale Gamma_i q_i)
// and S = diag(Gamma_last) Shat at the end of the pass.  The decay of one
// token is at least 2^(lower_bound log2 e) >= 2^-7.22 (lower_bound >= -5), so
// 1 / Gamma stays below 2^58 over 8 tokens: far inside the fp32 range
// (chunk-size page, "bf16 Dynamic Range and Exponential Terms", for the same
// bound over 16 tokens).
//
// Thread t holds 4 columns (4 (t / 8) ..) of the state, each on the 16 rows
// 32 m + 4 (t % 8) + e (m, e < 4), in registers: every operand element a
// thread reads from LDS serves its 4 columns, and the dot products over the
// rows finish with a 3-step exchange among the 8 threads of a column group.
// The rows are interleaved so that the 8 threads of a group load and store
// each 128-byte line of a state row together.
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int D = kHeadDim;
constexpr int kThreads = 256;
constexpr int kPassTokens = 8;    // tokens per pass
constexpr int kLoadTokens = 16;   // tokens whose inputs load together (two passes)
static_assert(kThreads == 64 * kLoadTokens / 4, "each wave loads 4 tokens of every tensor");
static_assert(2 * D == kThreads, "two threads per channel prepare a pass");

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// Sum over the 8 lanes of an aligned group: quad permutations [1,0,3,2] and
// [2,3,0,1], then the half-row mirror (lane i <-> 7 - i) adds the other quad.
__device__ __forceinline__ float group8_sum(float x)
{
    x += dpp<0xb1>(x);
    x += dpp<0x4e>(x);
    return x + dpp<0x141>(x);
}

// Direct global-to-LDS load (global_load_lds_dwordx4): lane i's 16 bytes,
// read at base + voff, land at LDS byte address dst + 16 i (dst is
// wave-uniform, in M0).  Written as asm so that the compiler does not make
// unrelated LDS accesses wait for it; the caller waits (vmcnt) before the
// barrier that hands the data to the other threads.
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t dst)
{
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(dst) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmem()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Start loading the raw q, k, v, g rows of the (at most kLoadTokens) tokens
// from t0 into raw[4][kLoadTokens][D]: load r of wave w moves tensor r, tokens
// 4 w .. 4 w + 3 (lane i: token 4 w + i / 16, bytes 16 (i % 16) ..), one
// 16-byte piece per lane, in the tile's own order.  Tokens at or past `nl`
// read the first token instead (their rows are never used).
__device__ __forceinline__ void load_raw(const FwdParams &p, int64_t row, int64_t t0, int64_t h, int nl,
                                         uint32_t raw_lds, int tid)
{
    const int w = tid >> 6, lane = tid & 63;
    const int i = 4 * w + (lane >> 4);
    const uint32_t voff = static_cast<uint32_t>((i < nl ? i : 0) * p.H * D * 2 + 16 * (lane & 15));
    const int64_t first = ((row * p.T + t0) * p.H + h) * D;
    dma16(p.q + first, voff, raw_lds + 1024 * w);
    dma16(p.k + first, voff, raw_lds + 1024 * w + 1 * kLoadTokens * D * 2);
    dma16(p.v + first, voff, raw_lds + 1024 * w + 2 * kLoadTokens * D * 2);
    dma16(p.g + first, voff, raw_lds + 1024 * w + 3 * kLoadTokens * D * 2);
}

template <int INIT, int FINAL>
__global__ __launch_bounds__(kThreads, 4) void decode_kernel(FwdParams p)  // 4 chains per compute unit
{
    __shared__ __align__(16) uint16_t raw[4][kLoadTokens][D];  // q, k, v, g of two passes (bf16)
    __shared__ __align__(16) float kg[kPassTokens][D];         // Gamma_i k_i
    __shared__ __align__(16) float kh[kPassTokens][D];         // beta_i k_i / Gamma_i
    __shared__ __align__(16) float qg[kPassTokens][D];         // scale Gamma_i q_i
    __shared__ __align__(16) float gam_last[D];                // Gamma at the pass's last token
    __shared__ float bet[kLoadTokens];                         // beta_i

    const int tid = threadIdx.x;
    const int rg = tid & 7, col0 = 4 * (tid >> 3);  // rows 32 m + 4 rg + e; columns col0 ..
    const int64_t chain = blockIdx.x;
    const int64_t n = chain / p.H, h = chain - n * p.H;
    int64_t t_begin, t_end, row;
    chain_segment(p, n, &t_begin, &t_end, &row);

    // The inputs of the first two passes are requested before the state
    // (beta first: the compiler waits for it itself), so that the wait for
    // them below lets the state loads stay in flight.  Longer sequences load
    // 16 tokens at a time.
    const uint32_t raw_lds = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t *)&raw[0][0][0]));
    int nl = static_cast<int>(t_end - t_begin < kLoadTokens ? t_end - t_begin : kLoadTokens);
    float beta_logit = 0.f;
    if (tid < nl)
        beta_logit = bf16_to_f32(p.beta[(row * p.T + t_begin + tid) * p.H + h]);
    if (nl > 0)
        load_raw(p, row, t_begin, h, nl, raw_lds, tid);

    // s[cc][4 m + e] = S[32 m + 4 rg + e][col0 + cc]; the state is stored
    // [V][K], so the four rows 32 m + 4 rg .. of a column are 16 bytes.
    float s[4][16];
    const int64_t slab = chain * D * D + int64_t(col0) * D + 4 * rg;
    if constexpr (INIT == kStateFp32) {
        const float *src = static_cast<const float *>(p.init_state) + slab;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f32x4_t x = *reinterpret_cast<const f32x4_t *>(src + cc * D + 32 * m);
#pragma unroll
                for (int e = 0; e < 4; ++e) s[cc][4 * m + e] = x[e];
            }
    } else if constexpr (INIT == kStateBf16) {
        const uint16_t *src = static_cast<const uint16_t *>(p.init_state) + slab;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const u32x2_t x = *reinterpret_cast<const u32x2_t *>(src + cc * D + 32 * m);
                s[cc][4 * m] = __uint_as_float(x[0] << 16);
                s[cc][4 * m + 1] = __uint_as_float(x[0] & 0xffff0000u);
                s[cc][4 * m + 2] = __uint_as_float(x[1] << 16);
                s[cc][4 * m + 3] = __uint_as_float(x[1] & 0xffff0000u);
            }
    } else {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int j = 0; j < 16; ++j) s[cc][j] = 0.f;
    }

    // pass preparation: thread t takes channel t / 2, tokens 4 (t % 2) .. + 3
    const int pc = tid >> 1, part = tid & 1;
    const float head_neg = -(p.A_log ? expf(p.A_log[h]) : 1.0f) * kLog2eF;  // log2 units
    const float bias_neg = p.dt_bias ? head_neg * p.dt_bias[h * D + pc] : 0.f;

    for (int64_t tl = t_begin; tl < t_end; tl += kLoadTokens) {
        if (tl != t_begin) {
            nl = static_cast<int>(t_end - tl < kLoadTokens ? t_end - tl : kLoadTokens);
            if (tid < nl)
                beta_logit = bf16_to_f32(p.beta[(row * p.T + tl + tid) * p.H + h]);
            __syncthreads();  // the previous passes are done with the raw inputs
            load_raw(p, row, tl, h, nl, raw_lds, tid);
            wait_vmem<0>();
        } else {
            // 16 state loads (fp32 or bf16 initial state) follow the raw
            // loads; allowing 8 of them in flight still covers the raw loads
            wait_vmem<INIT == kStateNone ? 0 : 8>();
        }
        if (tid < nl)
            bet[tid] = sigmoid_f32(beta_logit);
        for (int pass = 0; pass * kPassTokens < nl; ++pass) {
            const int64_t t0 = tl + pass * kPassTokens;
            const int r0 = pass * kPassTokens;  // the pass's first token in the raw tile
            const int nb = nl - r0 < kPassTokens ? nl - r0 : kPassTokens;
            __syncthreads();  // raw inputs in LDS; the previous pass is done with the operands

            // Decays and factored operands.  The two threads of a channel each
            // take four tokens; the second scales its running products by the
            // first's total (exchanged within the lane pair).
            {
                const int i0 = 4 * part;
                float al[4], cum = 1.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float a = 1.0f;
                    if (i0 + i < nb) {
                        const float e = exp2_f32(fmaf(bf16_to_f32(raw[3][r0 + i0 + i][pc]), head_neg, bias_neg));
                        a = exp2_f32(p.gate_scale * __builtin_amdgcn_rcpf(1.0f + e));
                    }
                    cum *= a;
                    al[i] = cum;
                }
                const float first_total = dpp<0xa0>(cum);  // quad_perm [0,0,2,2]: the pair's even lane
                const float lead = part ? first_total : 1.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ti = i0 + i;
                    if (ti < nb) {
                        const float gam = lead * al[i];
                        const float kk = bf16_to_f32(raw[1][r0 + ti][pc]);
                        kg[ti][pc] = gam * kk;
                        kh[ti][pc] = bet[r0 + ti] * kk * __builtin_amdgcn_rcpf(gam);
                        qg[ti][pc] = p.scale * gam * bf16_to_f32(raw[0][r0 + ti][pc]);
                    }
                }
                // Gamma at the pass's last token: the second thread holds it
                // unless the pass has at most 4 tokens
                if (part == (nb > 4 ? 1 : 0))
                    gam_last[pc] = lead * cum;
            }
            __syncthreads();

            for (int i = 0; i < nb; ++i) {
                f32x4_t a[4], b[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) a[m] = *reinterpret_cast<const f32x4_t *>(&kg[i][32 * m + 4 * rg]);
                // u = v_i - Shat^T (Gamma_i k_i) for the 4 columns
                const u32x2_t vb = *reinterpret_cast<const u32x2_t *>(&raw[2][r0 + i][col0]);
                const float vcol[4] = {__uint_as_float(vb[0] << 16), __uint_as_float(vb[0] & 0xffff0000u),
                                       __uint_as_float(vb[1] << 16), __uint_as_float(vb[1] & 0xffff0000u)};
                float u[4];
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    float d0 = 0.f, d1 = 0.f;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        d0 = fmaf(s[cc][4 * m], a[m][0], d0);
                        d1 = fmaf(s[cc][4 * m + 1], a[m][1], d1);
                        d0 = fmaf(s[cc][4 * m + 2], a[m][2], d0);
                        d1 = fmaf(s[cc][4 * m + 3], a[m][3], d1);
                    }
                    u[cc] = vcol[cc] - group8_sum(d0 + d1);
                }
                // Shat += (beta_i k_i / Gamma_i) u^T
#pragma unroll
                for (int m = 0; m < 4; ++m) b[m] = *reinterpret_cast<const f32x4_t *>(&kh[i][32 * m + 4 * rg]);
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                    for (int m = 0; m < 4; ++m)
#pragma unroll
                        for (int e = 0; e < 4; ++e) s[cc][4 * m + e] = fmaf(b[m][e], u[cc], s[cc][4 * m + e]);
                // o_i = Shat^T (scale Gamma_i q_i)
#pragma unroll
                for (int m = 0; m < 4; ++m) a[m] = *reinterpret_cast<const f32x4_t *>(&qg[i][32 * m + 4 * rg]);
                float o[4];
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    float d0 = 0.f, d1 = 0.f;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        d0 = fmaf(s[cc][4 * m], a[m][0], d0);
                        d1 = fmaf(s[cc][4 * m + 1], a[m][1], d1);
                        d0 = fmaf(s[cc][4 * m + 2], a[m][2], d0);
                        d1 = fmaf(s[cc][4 * m + 3], a[m][3], d1);
                    }
                    o[cc] = group8_sum(d0 + d1);
                }
                if (rg == 0) {
                    const u32x2_t packed = {uint32_t(f32_to_bf16_rne(o[0])) | (uint32_t(f32_to_bf16_rne(o[1])) << 16),
                                            uint32_t(f32_to_bf16_rne(o[2])) | (uint32_t(f32_to_bf16_rne(o[3])) << 16)};
                    *reinterpret_cast<u32x2_t *>(p.out + ((row * p.T + t0 + i) * p.H + h) * D + col0) = packed;
                }
            }

            // S = diag(Gamma_last) Shat
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f32x4_t g = *reinterpret_cast<const f32x4_t *>(&gam_last[32 * m + 4 * rg]);
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[cc][4 * m + e] *= g[e];
            }
        }
    }

    if constexpr (FINAL == kStateFp32) {
        float *dst = static_cast<float *>(p.final_state) + slab;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int m = 0; m < 4; ++m)
                *reinterpret_cast<f32x4_t *>(dst + cc * D + 32 * m) =
                    f32x4_t{s[cc][4 * m], s[cc][4 * m + 1], s[cc][4 * m + 2], s[cc][4 * m + 3]};
    } else if constexpr (FINAL == kStateBf16) {
        uint16_t *dst = static_cast<uint16_t *>(p.final_state) + slab;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int m = 0; m < 4; ++m)
                *reinterpret_cast<u32x2_t *>(dst + cc * D + 32 * m) =
                    u32x2_t{uint32_t(f32_to_bf16_rne(s[cc][4 * m])) | (uint32_t(f32_to_bf16_rne(s[cc][4 * m + 1])) << 16),
                            uint32_t(f32_to_bf16_rne(s[cc][4 * m + 2])) | (uint32_t(f32_to_bf16_rne(s[cc][4 * m + 3])) << 16)};
    }
}

template <int INIT>
const void *decode_instance(int final_kind)
{
    switch (final_kind) {
    case kStateFp32: return reinterpret_cast<const void *>(&decode_kernel<INIT, kStateFp32>);
    case kStateBf16: return reinterpret_cast<const void *>(&decode_kernel<INIT, kStateBf16>);
    default: return reinterpret_cast<const void *>(&decode_kernel<INIT, kStateNone>);
    }
}

}  // namespace

hipError_t launch_decode(const FwdParams &p, hipStream_t stream)
{
    const int64_t blocks = p.num_seqs * p.H;
    if (blocks == 0)
        return hipSuccess;
    const int init = p.init_state ? p.init_kind : kStateNone;
    const int fin = p.final_state ? p.final_kind : kStateNone;
    const void *kernel = init == kStateFp32   ? decode_instance<kStateFp32>(fin)
                         : init == kStateBf16 ? decode_instance<kStateBf16>(fin)
                                              : decode_instance<kStateNone>(fin);
    FwdParams args = p;
    void *argv[] = {&args};
    return hipLaunchKernel(kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), argv, 0, stream);
}

}  // namespace kda
