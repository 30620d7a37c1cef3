// Combine step of the segmented KDA forward pass (intra-sequence scan).
//
// The recurrence is affine in the state: a segment of chunks maps its start
// state S to M S + b, with M the product of the chunks' transition matrices
// diag(Gamma_C) - Kbar^T W (each chunk's state update with v set to zero)
// and b the segment's end state from a zero start.  The map kernels store,
// for every chain and segment s, b_s in seg_b[s] and M_s (as the end state
// of an identity start, i.e. transposed like every stored state) in
// seg_m[s]; seg_b[0] already holds the true end state of segment 0.  This
// kernel walks the segments of each chain in order,
//   seg_b[s] <- M_s seg_b[s-1] + seg_b[s]      (s = 1 .. segments - 2),
// after which seg_b[s] is the true state at the end of segment s, i.e. the
// start state of segment s + 1.
//
// In the stored [V][K] layout (element [v][k] = S[k][v]) the update reads
// new[v][k] = sum_j cur[v][j] * Mst[j][k] + b[v][k] with Mst[j][k] = M[k][j],
// the stored form of M: a [16 x 128] x [128 x 128] product per block of 16
// value columns, on fp32 MFMA (v_mfma_f32_16x16x4f32), so the combine adds
// no rounding beyond fp32.
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

__global__ __launch_bounds__(kCombineThreads) void scan_combine_kernel(FwdParams p)
{
    __shared__ float cur[kRows][D + 4];  // this block's rows of the running state (padded)
    const int chain = static_cast<int>(blockIdx.x) / kBlocksPerChain;
    const int vb = static_cast<int>(blockIdx.x) % kBlocksPerChain;
    int64_t t_begin, t_end, row;
    chain_segment(p, chain / p.H, &t_begin, &t_end, &row);
    const int64_t nc = (t_end - t_begin + C - 1) / C;
    const int segs = nc > 0 ? static_cast<int>((nc + p.seg_chunks - 1) / p.seg_chunks) : 1;
    if (segs <= 2)
        return;  // seg_b[0] is already the start state of the only later segment

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
    const int64_t slab = int64_t(D) * D;
    float *const b_chain = p.seg_b + int64_t(chain) * p.n_seg * slab + int64_t(vb) * kRows * D;
    const float *const m_chain = p.seg_m + int64_t(chain) * p.n_seg * slab;

    for (int i = threadIdx.x; i < kRows * D; i += kCombineThreads)
        cur[i / D][i % D] = b_chain[i];
    __syncthreads();

    for (int s = 1; s <= segs - 2; ++s) {
        float *const bs = b_chain + s * slab;
        const float *const ms = m_chain + s * slab;
        // accumulators start from b: lane (column l16 of tile t, g4) holds
        // rows 4 g4 .. 4 g4 + 3
        f32x4_t acc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[t][r] = bs[(4 * g4 + r) * D + 32 * wave + 16 * t + l16];
        // contraction over j in steps of 4: A[m][kk] = cur[m][4 kk + g4]
        // from lane (m = l16, g4), B[kk][n] = Mst[4 kk + g4][n] from lane
        // (n = l16, g4)
#pragma unroll 8
        for (int kk = 0; kk < D / 4; ++kk) {
            const float a = cur[l16][4 * kk + g4];
#pragma unroll
            for (int t = 0; t < 2; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                    a, ms[(4 * kk + g4) * D + 32 * wave + 16 * t + l16], acc[t], 0, 0, 0);
        }
        __syncthreads();  // every wave has finished reading cur
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int v = 4 * g4 + r, k = 32 * wave + 16 * t + l16;
                cur[v][k] = acc[t][r];
                bs[v * D + k] = acc[t][r];
            }
        __syncthreads();
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
