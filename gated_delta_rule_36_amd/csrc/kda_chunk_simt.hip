// Straightforward chunked KDA forward kernel: fp32 vector ALU arithmetic, all
// tiles in LDS, one workgroup of 256 threads per (sequence, head) chain.
//
// Per chunk of 16 tokens (gate values a in log2 units, G = inclusive cumsum
// of a within the chunk, Gamma = 2^G, Gamma_C = 2^G at the chunk's end):
//   Qt = scale q Gamma, Kt = k Gamma, Kh = k / Gamma, Kb = k Gamma_C / Gamma
//   A  = diag(beta) Kt Kh^T (strictly lower), P = Qt Kh^T (lower)
//   T  = (I + A)^-1 (unit lower triangular, forward substitution)
//   W  = T diag(beta) Kt,  U~ = T diag(beta) V
//   U  = U~ - W S,  O = Qt S + P U,  S <- diag(Gamma_C) S + Kb^T U
// which is the token recurrence regrouped by chunk.  The chunk size of 16
// keeps 2^(+-G) inside the fp32/bf16 exponent range for lower_bound >= -5
// (chunk-size page, "bf16 Dynamic Range and Exponential Terms").
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int C = kChunk;
constexpr int D = kHeadDim;
constexpr int NT = 256;

template <int INIT, int FINAL>
__global__ __launch_bounds__(NT) void chunk_simt_kernel(FwdParams p)
{
    __shared__ float S[D][D];  // S[k][v], the fp32 state
    __shared__ float Qt[C][D], Kt[C][D], Kh[C][D], Kb[C][D], Vu[C][D], W[C][D], Ga[C][D];
    __shared__ float Am[C][C], Pm[C][C], Tm[C][C];
    __shared__ float bet[C], gam_end[D];

    const int tid = threadIdx.x;
    const int64_t chain = blockIdx.x;
    const int64_t H = p.H, T = p.T;
    const int64_t n = chain / H, h = chain % H;
    int64_t t_begin, t_end, row;
    chain_segment(p, n, &t_begin, &t_end, &row);

    for (int e = tid; e < D * D; e += NT) {
        const int vv = e / D, kk = e % D;
        S[kk][vv] = load_state<INIT>(p.init_state, chain * D * D + e);
    }
    const float head_mult = p.A_log ? expf(p.A_log[h]) : 1.0f;

    for (int64_t c0 = t_begin; c0 < t_end; c0 += C) {
        const int len = static_cast<int>(t_end - c0 < C ? t_end - c0 : C);
        __syncthreads();  // the previous chunk is done with every tile

        // stream in, gate activation; rows past the end act as no-ops
        for (int e = tid; e < C * D; e += NT) {
            const int i = e / D, c = e % D;
            float qv = 0.f, kv = 0.f, vv = 0.f, a = 0.f;
            if (i < len) {
                const int64_t idx = ((row * T + c0 + i) * H + h) * D + c;
                qv = bf16_to_f32(p.q[idx]);
                kv = bf16_to_f32(p.k[idx]);
                vv = bf16_to_f32(p.v[idx]);
                const float bias = p.dt_bias ? p.dt_bias[h * D + c] : 0.f;
                a = p.gate_scale * sigmoid_f32(head_mult * (bf16_to_f32(p.g[idx]) + bias));
            }
            Qt[i][c] = qv;
            Kt[i][c] = kv;
            Vu[i][c] = vv;
            Ga[i][c] = a;
        }
        if (tid < C)
            bet[tid] = tid < len ? sigmoid_f32(bf16_to_f32(p.beta[(row * T + c0 + tid) * H + h]))
                                 : 0.f;
        __syncthreads();

        // per-channel cumulative gate and the four decayed operands
        if (tid < D) {
            const int c = tid;
            float G[C];
            float run = 0.f;
            for (int i = 0; i < C; ++i) {
                run += Ga[i][c];
                G[i] = run;
            }
            for (int i = 0; i < C; ++i) {
                const float kv = Kt[i][c];
                const float up = exp2_f32(G[i]);
                Kt[i][c] = kv * up;
                Qt[i][c] = Qt[i][c] * p.scale * up;
                Kh[i][c] = kv * exp2_f32(-G[i]);
                Kb[i][c] = kv * exp2_f32(run - G[i]);
            }
            gam_end[c] = exp2_f32(run);
        }
        __syncthreads();

        // decay-masked Kt Kh^T and Qt Kh^T
        {
            const int i = tid / C, j = tid % C;
            float a = 0.f, pq = 0.f;
            if (j < i)
                for (int c = 0; c < D; ++c) a += Kt[i][c] * Kh[j][c];
            if (j <= i)
                for (int c = 0; c < D; ++c) pq += Qt[i][c] * Kh[j][c];
            Am[i][j] = bet[i] * a;
            Pm[i][j] = pq;
        }
        __syncthreads();

        // T = (I + A)^-1 by forward substitution, one column per thread
        if (tid < C) {
            const int j = tid;
            for (int i = 0; i < C; ++i) {
                float t = 0.f;
                if (i == j) {
                    t = 1.f;
                } else if (i > j) {
                    for (int m = j; m < i; ++m) t -= Am[i][m] * Tm[m][j];
                }
                Tm[i][j] = t;
            }
        }
        __syncthreads();

        // WY form: W = T diag(beta) Kt, U~ = T diag(beta) V; this thread owns
        // column c of rows i0..i0+7
        const int c = tid % D, i0 = (tid / D) * (C / 2);
        float u[C / 2];
        for (int ii = 0; ii < C / 2; ++ii) {
            const int i = i0 + ii;
            float w = 0.f, uu = 0.f;
            for (int j = 0; j <= i; ++j) {
                const float tb = Tm[i][j] * bet[j];
                w += tb * Kt[j][c];
                uu += tb * Vu[j][c];
            }
            W[i][c] = w;
            u[ii] = uu;
        }
        __syncthreads();

        // U = U~ - W S
        for (int ii = 0; ii < C / 2; ++ii) {
            const int i = i0 + ii;
            float acc = u[ii];
            for (int kk = 0; kk < D; ++kk) acc -= W[i][kk] * S[kk][c];
            u[ii] = acc;
        }
        for (int ii = 0; ii < C / 2; ++ii) Vu[i0 + ii][c] = u[ii];
        __syncthreads();

        // O = Qt S + P U
        for (int ii = 0; ii < C / 2; ++ii) {
            const int i = i0 + ii;
            float o = 0.f;
            for (int kk = 0; kk < D; ++kk) o += Qt[i][kk] * S[kk][c];
            for (int j = 0; j <= i; ++j) o += Pm[i][j] * Vu[j][c];
            if (i < len) p.out[((row * T + c0 + i) * H + h) * D + c] = f32_to_bf16_rne(o);
        }
        __syncthreads();

        // S <- diag(Gamma_C) S + Kb^T U; this thread owns column c, half the rows
        for (int kk = (tid / D) * (D / 2); kk < (tid / D + 1) * (D / 2); ++kk) {
            float s = gam_end[kk] * S[kk][c];
            for (int i = 0; i < C; ++i) s += Kb[i][kk] * Vu[i][c];
            S[kk][c] = s;
        }
    }
    __syncthreads();

    for (int e = tid; e < D * D; e += NT) {
        const int vv = e / D, kk = e % D;
        store_state<FINAL>(p.final_state, chain * D * D + e, S[kk][vv]);
    }
}

template <int INIT, int FINAL>
hipError_t launch(const FwdParams &p, hipStream_t stream)
{
    const int64_t chains = p.num_seqs * p.H;
    FwdParams args = p;
    void *argv[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void *>(&chunk_simt_kernel<INIT, FINAL>),
                           dim3(static_cast<unsigned>(chains)), dim3(NT), argv, 0, stream);
}

template <int INIT>
hipError_t launch_final(const FwdParams &p, hipStream_t stream)
{
    switch (p.final_kind) {
    case kStateBf16: return launch<INIT, kStateBf16>(p, stream);
    case kStateFp32: return launch<INIT, kStateFp32>(p, stream);
    default: return launch<INIT, kStateNone>(p, stream);
    }
}

}  // namespace

hipError_t launch_chunk_simt(const FwdParams &p, hipStream_t stream)
{
    switch (p.init_kind) {
    case kStateBf16: return launch_final<kStateBf16>(p, stream);
    case kStateFp32: return launch_final<kStateFp32>(p, stream);
    default: return launch_final<kStateNone>(p, stream);
    }
}

}  // namespace kda
