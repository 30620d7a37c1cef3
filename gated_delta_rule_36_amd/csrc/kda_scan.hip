// Combine step of the segmented KDA forward pass (intra-sequence scan).
//
// The recurrence is affine in the state: a segment of chunks maps its start
// state S to M S + b, with M the product of the chunks' transition matrices
// diag(Gamma_C) - Kbar^T W (each chunk's state update with v set to zero)
// and b the segment's end state from a zero start.  The map kernels store,
// for every chain and segment s, b_s in seg_b[s] (fp32, stored [V][K] like
// every state) and M_s in seg_m[s] as two bf16 planes, hi = bf16(M) and
// lo = bf16(M - hi), each row-major [k][j]; seg_b[0] already holds the true
// end state of segment 0.  This kernel walks the segments of each chain in
// order,
//   seg_b[s] <- M_s seg_b[s-1] + seg_b[s]      (s = 1 .. segments - 2),
// after which seg_b[s] is the true state at the end of segment s, i.e. the
// start state of segment s + 1.
//
// In the stored [V][K] layout (element [v][k] = S[k][v]) the update reads
// new[v][k] = sum_j cur[v][j] * M[k][j] + b[v][k].  A block owns 16 rows v
// of one chain; wave w computes columns k = 32 w .. 32 w + 31 (two 16 x 16
// tiles) with v_mfma_f32_16x16x32_bf16.  Both factors enter as hi + lo bf16
// pairs and the product as hi*hi + hi*lo + lo*hi: about 17 significant bits
// per factor and a dropped lo*lo term below 2^-17 of the product, so each
// step adds an error of the order of fp32 rounding, not of bf16.  The
// contraction index is taken in the order j = 32 g4 + 8 kt + e (lane group
// g4, MFMA step kt, element e), so every lane's operands are 16-byte pieces
// of one row of M and of cur.
//
// Operands for segment s + 1 are loaded straight into LDS (direct
// global-to-LDS loads, issued by each wave for its own rows of M and its own
// columns of b) while segment s multiplies; each wave waits for its own
// loads with an explicit vmcnt, so the only workgroup barrier per segment
// orders the running state, which every wave reads whole.
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int D = kHeadDim;
constexpr int kRows = 16;             // stored rows (value columns v) per block
constexpr int kBlocksPerChain = D / kRows;
constexpr int kCombineThreads = 256;  // 4 waves; wave w owns columns 32w .. 32w + 31
constexpr int kPlaneBytes = D * D * 2;  // one bf16 plane of M_s

// LDS, 160 KiB.  Rows of 16-byte pieces are stored XOR-swizzled (piece c of
// row r at position c ^ (r & 15)): the 16 lanes that one pass of a 128-bit
// read serves then hit 16 different bank groups.
struct CombineShared {
    // M_s rows 32 w .. 32 w + 31 of wave w, hi and lo planes: [buf][w][plane][row][256 B]
    uint8_t m[2][4][2][32][256];
    // b_s rows 16 vb .. 16 vb + 15, columns 32 w .. 32 w + 31 of wave w: [buf][w][row][32]
    float b[2][4][kRows][32];
    // running state rows (this block's 16), hi and lo planes: [buf][plane][row][256 B]
    uint8_t cur[2][2][kRows][256];
};
static_assert(sizeof(CombineShared) <= 160 * 1024, "LDS budget");

typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u8 *)p));
}
template <typename V>
__device__ __forceinline__ V lds_ld(uint32_t a)
{
    return *(const __attribute__((address_space(3))) V *)(uintptr_t)a;
}
template <typename V>
__device__ __forceinline__ void lds_st(uint32_t a, V v)
{
    *(__attribute__((address_space(3))) V *)(uintptr_t)a = v;
}
// Direct global-to-LDS load (global_load_lds_dwordx4): lane i's 16 bytes,
// read at base + voff, land at LDS byte address dst + 16 i (dst is
// wave-uniform and goes in M0).  Written as asm so that the compiler neither
// tracks it nor makes unrelated accesses wait for it; the issuing wave waits
// for it with wait_vmem.
__device__ __forceinline__ void dma16(const char *base, uint32_t voff, uint32_t dst)
{
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(dst) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmem()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x)); }

// Global stores of one segment step per lane: 2 tiles x 4 rows, one dword
// each.  The top of the next step waits for all but these many vector-memory
// operations, i.e. for the segment's direct loads issued before them.
constexpr int kStoresPerStep = 8;

__global__ __launch_bounds__(kCombineThreads) void scan_combine_kernel(FwdParams p)
{
    __shared__ CombineShared sh;
    // Workgroups go to the 8 XCDs round-robin (block b to XCD b mod 8); the
    // mapping below puts the 8 blocks of a chain on one XCD, so each M_s is
    // fetched into that XCD's L2 once instead of once per block.  Chains past
    // the last whole group of 8 keep the plain mapping.
    const int b = static_cast<int>(blockIdx.x);
    const int whole = static_cast<int>(p.num_seqs * p.H / 8) * 8 * kBlocksPerChain;
    int chain, vb;
    if (b < whole) {
        const int xcd = b % 8, i = b / 8;
        chain = 8 * (i / kBlocksPerChain) + xcd;
        vb = i % kBlocksPerChain;
    } else {
        chain = b / kBlocksPerChain;
        vb = b % kBlocksPerChain;
    }
    int64_t t_begin, t_end, row;
    chain_segment(p, chain / p.H, &t_begin, &t_end, &row);
    const int64_t nc = (t_end - t_begin + kChunk - 1) / kChunk;
    const int segs = nc > 0 ? static_cast<int>((nc + p.seg_chunks - 1) / p.seg_chunks) : 1;
    if (segs <= 2)
        return;  // seg_b[0] is already the start state of the only later segment
    const int last = segs - 2;  // segments 1 .. last are combined

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t slab_bytes = int64_t(D) * D * 4;
    const char *const m_chain = reinterpret_cast<const char *>(p.seg_m) + int64_t(chain) * p.n_seg * slab_bytes +
                                int64_t(32 * wave) * 256;
    char *const b_chain = reinterpret_cast<char *>(p.seg_b) + int64_t(chain) * p.n_seg * slab_bytes;
    const char *const b_rows = b_chain + int64_t(kRows * vb) * D * 4 + 32 * wave * 4;

    const uint32_t sh_m = lds_addr(&sh.m[0][wave][0][0][0]), sh_b = lds_addr(&sh.b[0][wave][0][0]),
                   sh_cur = lds_addr(&sh.cur[0][0][0][0]);
    constexpr uint32_t kMBuf = sizeof(sh.m[0]), kBBuf = sizeof(sh.b[0]), kCurBuf = sizeof(sh.cur[0]);
    constexpr uint32_t kMPlane = sizeof(sh.m[0][0][0]), kCurPlane = sizeof(sh.cur[0][0]);

    // Direct-load lane offsets.  M: load j (0..7) of a plane moves rows
    // 4 j + lane / 16 of this wave's 32, lane taking the piece that belongs
    // at position lane % 16.  b: load j (0..1) moves rows 8 j + lane / 8,
    // 128 bytes (this wave's 32 columns) each, unswizzled.
    const int mr = lane >> 4, mp = lane & 15;
    const uint32_t b_lane = static_cast<uint32_t>((lane >> 3) * D * 4 + 16 * (lane & 7));
    auto issue = [&](int s, int buf) {
        const char *ms = m_chain + int64_t(s) * slab_bytes;
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 4 * j + mr;  // row within the wave's 32; row k = 32 w + r, k & 15 = r & 15
                const uint32_t voff = static_cast<uint32_t>(r * 256 + 16 * (mp ^ (r & 15)));
                dma16(ms + pl * kPlaneBytes, voff, sh_m + buf * kMBuf + pl * kMPlane + j * 1024);
            }
        const char *bs = b_rows + int64_t(s) * slab_bytes;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            dma16(bs + j * 8 * D * 4, b_lane, sh_b + buf * kBBuf + j * 1024);
    };

    // segment 1's operands, then the running state from seg_b[0] (fp32, this
    // block's 16 rows) as hi / lo planes
    issue(1, 1);
    {
        const int v = threadIdx.x >> 4, c = threadIdx.x & 15;  // row v, piece c (columns 8 c .. 8 c + 7)
        const f32x4_t *src = reinterpret_cast<const f32x4_t *>(b_chain + (int64_t(kRows * vb + v) * D + 8 * c) * 4);
        const f32x4_t x0 = src[0], x1 = src[1];
        uint16_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = e < 4 ? x0[e] : x1[e - 4];
            hi[e] = bf16_bits(x);
            lo[e] = bf16_bits(x - bf16_to_f32(hi[e]));
        }
        u32x4_t h, l;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            h[q] = hi[2 * q] | (uint32_t(hi[2 * q + 1]) << 16);
            l[q] = lo[2 * q] | (uint32_t(lo[2 * q + 1]) << 16);
        }
        const uint32_t a = sh_cur + v * 256 + 16 * (c ^ v);
        lds_st(a, h);
        lds_st(a + kCurPlane, l);
    }

    // this lane's LDS read offsets: A (cur row l16, piece 4 g4 + kt) and B
    // (M row 16 t + l16 of the wave's, same piece), both at (4 g4 + kt) ^ l16
    const uint32_t rd_cur = sh_cur + l16 * 256, rd_m = sh_m + l16 * 256;
    const uint32_t rd_b = sh_b + (4 * g4) * 32 * 4 + l16 * 4;
    float *const st_base = reinterpret_cast<float *>(b_chain) + int64_t(kRows * vb + 4 * g4) * D + 32 * wave + l16;

    for (int s = 1; s <= last; ++s) {
        const int buf = s & 1, rd = (s - 1) & 1, wr = s & 1;
        // this wave's loads of segment s (issued one step earlier, before that
        // step's stores) have landed
        if (s == 1)
            wait_vmem<0>();
        else
            wait_vmem<kStoresPerStep>();
        lds_barrier();  // cur[rd] is complete; every wave is done with cur[wr]
        if (s < last)
            issue(s + 1, buf ^ 1);

        f32x4_t acc[2][3];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int x = 0; x < 3; ++x) acc[t][x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const uint32_t piece = 16 * ((4 * g4 + kt) ^ l16);
            const uint32_t ac = rd_cur + rd * kCurBuf + piece;
            const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, lds_ld<u32x4_t>(ac));
            const bf16x8_t al = __builtin_bit_cast(bf16x8_t, lds_ld<u32x4_t>(ac + kCurPlane));
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint32_t am = rd_m + buf * kMBuf + t * 16 * 256 + piece;
                const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, lds_ld<u32x4_t>(am));
                const bf16x8_t bl = __builtin_bit_cast(bf16x8_t, lds_ld<u32x4_t>(am + kMPlane));
                acc[t][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[t][0], 0, 0, 0);
                acc[t][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[t][1], 0, 0, 0);
                acc[t][2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[t][2], 0, 0, 0);
            }
        }
        // new[v][k] for v = 16 vb + 4 g4 + r, k = 32 w + 16 t + l16
        float *const st = st_base + int64_t(s) * D * D;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float bv = lds_ld<float>(rd_b + buf * kBBuf + r * 32 * 4 + t * 16 * 4);
                const float x = (acc[t][0][r] + (acc[t][1][r] + acc[t][2][r])) + bv;
                const int v = 4 * g4 + r, k = 32 * wave + 16 * t + l16;
                const uint16_t h = bf16_bits(x), l = bf16_bits(x - bf16_to_f32(h));
                const uint32_t a = sh_cur + wr * kCurBuf + v * 256 + 16 * ((k >> 3) ^ v) + 2 * (k & 7);
                lds_st(a, h);
                lds_st(a + kCurPlane, l);
                st[r * D + 16 * t] = x;
            }
    }
    wait_vmem<0>();  // no direct load may still be writing LDS when the wave ends
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
