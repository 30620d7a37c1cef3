// Combine step of the segmented KDA forward pass (intra-sequence scan).
//
// The recurrence is affine in the state: a segment of chunks maps its start
// state S to M S + b, with M the product of the chunks' transition matrices
// diag(Gamma_C) - Kbar^T W (each chunk's state update with v set to zero)
// and b the segment's end state from a zero start.  The map kernels store,
// for every chain and segment s, b_s in seg_b[s] (stored [V][K] like every
// state) and M_s (the end state of an identity start, untransposed) in
// seg_m[s]; seg_b[0] already holds the true end state of segment 0.  This
// kernel walks the segments of each chain in order,
//   seg_b[s] <- M_s seg_b[s-1] + seg_b[s]      (s = 1 .. segments - 2),
// after which seg_b[s] is the true state at the end of segment s, i.e. the
// start state of segment s + 1.
//
// In the stored [V][K] layout (element [v][k] = S[k][v]) the update reads
// new[v][k] = sum_j cur[v][j] * M[k][j] + b[v][k], where the transition pass
// stored M itself, row-major ([k][j]): a [16 x 128] x [128 x 128] product per
// block of 16 value columns, on fp32 MFMA (v_mfma_f32_16x16x4f32), so the
// combine adds no rounding beyond fp32.  The contraction index is taken in
// the order j = 32 g + kk (MFMA step kk, K-slot g), so every lane's operands
// for one segment are 32 consecutive floats of one row of M and of cur; the
// next segment's operands load while the current one multiplies.
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;
constexpr int D = kHeadDim;
constexpr int kRows = 16;             // stored rows (value columns v) per block
constexpr int kBlocksPerChain = D / kRows;
constexpr int kCombineThreads = 256;  // 4 waves; wave w owns columns 32w .. 32w + 31

// One segment's operands held by a lane: row k = 32 w + 16 t + l16 of M,
// columns 32 g4 .. 32 g4 + 31 (t = 0, 1), and b at rows 4 g4 + r, column k.
struct StepRegs {
    f32x4_t m[2][8];
    f32x4_t b[2];
};

__device__ __forceinline__ void load_step(StepRegs &r, const float *ms, const float *bs, int wave,
                                          int l16, int g4)
{
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int k = 32 * wave + 16 * t + l16;
        const f32x4_t *row = reinterpret_cast<const f32x4_t *>(ms + k * D + 32 * g4);
#pragma unroll
        for (int q = 0; q < 8; ++q) r.m[t][q] = row[q];
#pragma unroll
        for (int i = 0; i < 4; ++i) r.b[t][i] = bs[(4 * g4 + i) * D + k];
    }
}

__global__ __launch_bounds__(kCombineThreads) void scan_combine_kernel(FwdParams p)
{
    // this block's rows of the running state, double-buffered: segment s
    // reads buffer (s - 1) % 2 and writes the other, so one barrier per segment
    __shared__ __align__(16) float cur[2][kRows][D + 4];
    const int chain = static_cast<int>(blockIdx.x) / kBlocksPerChain;
    const int vb = static_cast<int>(blockIdx.x) % kBlocksPerChain;
    int64_t t_begin, t_end, row;
    chain_segment(p, chain / p.H, &t_begin, &t_end, &row);
    const int64_t nc = (t_end - t_begin + C - 1) / C;
    const int segs = nc > 0 ? static_cast<int>((nc + p.seg_chunks - 1) / p.seg_chunks) : 1;
    if (segs <= 2)
        return;  // seg_b[0] is already the start state of the only later segment
    const int last = segs - 2;  // segments 1 .. last are combined

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
    const int64_t slab = int64_t(D) * D;
    float *const b_chain = p.seg_b + int64_t(chain) * p.n_seg * slab + int64_t(vb) * kRows * D;
    const float *const m_chain = p.seg_m + int64_t(chain) * p.n_seg * slab;

    for (int i = threadIdx.x; i < kRows * D; i += kCombineThreads)
        cur[0][i / D][i % D] = b_chain[i];

    // new = cur M^T + b for segment s, written to seg_b[s] and to the other
    // buffer of cur.  Four partial sums per tile (over q mod 4) keep eight
    // independent MFMA chains in flight instead of two.
    auto step = [&](int s, const StepRegs &r) {
        __syncthreads();  // the previous segment's result (or seg_b[0]) is in cur[(s - 1) % 2]
        const int rd = (s - 1) & 1;
        f32x4_t acc[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            acc[t][0] = r.b[t];
            acc[t][1] = acc[t][2] = acc[t][3] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        const f32x4_t *arow = reinterpret_cast<const f32x4_t *>(&cur[rd][l16][32 * g4]);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const f32x4_t a = arow[q];
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    acc[t][q & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], r.m[t][q][e], acc[t][q & 3], 0, 0, 0);
        }
        float *const bs = b_chain + s * slab;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const f32x4_t sum = (acc[t][0] + acc[t][1]) + (acc[t][2] + acc[t][3]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int v = 4 * g4 + i, k = 32 * wave + 16 * t + l16;
                cur[rd ^ 1][v][k] = sum[i];
                bs[v * D + k] = sum[i];
            }
        }
    };

    // two register sets: the operands of segment s + 1 load while s multiplies
    StepRegs ra, rb;
    load_step(ra, m_chain + slab, b_chain + slab, wave, l16, g4);
    for (int s = 1; s <= last; s += 2) {
        if (s + 1 <= last)
            load_step(rb, m_chain + (s + 1) * slab, b_chain + (s + 1) * slab, wave, l16, g4);
        step(s, ra);
        if (s + 1 > last)
            break;
        if (s + 2 <= last)
            load_step(ra, m_chain + (s + 2) * slab, b_chain + (s + 2) * slab, wave, l16, g4);
        step(s + 1, rb);
    }
}

}  // namespace

hipError_t launch_scan_combine(const FwdParams &p, hipStream_t stream)
{
    const int64_t blocks = p.num_seqs * p.H * kBlocksPerChain;
    FwdParams args = p;
    void *argv[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void *>(&scan_combine_kernel),
                           dim3(static_cast<unsigned>(blocks)), dim3(kCombineThreads), argv, 0, stream);
}

}  // namespace kda
