// Chunked KDA forward kernel for gfx950: bf16 MFMA for every contraction,
// fp32 state held in accumulator registers, one workgroup of 8 waves per
// (sequence, head) chain.
//
// The chunk-of-16 form (gate a in log2 units, G = inclusive sum of a over
// the chunk, Gamma = 2^G, Gamma_C = its value at the chunk's last token):
//   Qt = scale q Gamma, Kt = k Gamma, Kbar = k Gamma_C / Gamma, Kh = Kbar / Gamma_C
//   A  = diag(beta) Kt Kh^T (strictly lower),  P = Qt Kh^T (lower)
//   T  = (I + A)^-1,  W = T diag(beta) Kt,  U~ = T diag(beta) V
//   U  = U~ - W S,  O = Qt S + P U,  S <- diag(Gamma_C) S + Kbar^T U
// The 16-token chunk keeps 2^(+-G) within the bf16/fp32 exponent range for
// lower_bound >= -5 (chunk-size page, "bf16 Dynamic Range and Exponential
// Terms"); the unit lower-triangular 16x16 inverse is the one the same page
// describes under "Efficient 16x16 Matrix Inversion" (solved here by forward
// substitution in fp32).
//
// Wave roles (64-lane waves; lane = 16 * g4 + l16):
//   waves 0-3  "state" waves.  Wave w owns the 128 x 32 slab S[:, 32w:32w+32]
//              of the state as 16 fp32 16x16 accumulator tiles and, per chunk,
//              computes U = U~ - W S, O = Qt S + P U (stores out) and the
//              state update.  S is the B operand of W S and Qt S through a
//              fixed permutation of the contraction index, so the fp32
//              accumulators convert to bf16 operands in place.
//   waves 4-7  "chunk" waves.  Wave p owns channels (and value columns)
//              32p..32p+31 and runs, for three different chunks at once:
//                G   stream in q/k/g/v (16-byte loads issued three chunks
//                    ahead), transpose to channel-major with an MFMA against
//                    a 0/1 selection matrix, gate, cumulative decay products,
//                    the decayed operands (written to LDS in the layouts the
//                    MFMAs read);
//                SOL A = diag(beta) Kt Kh^T, then four columns of T by
//                    forward substitution (and, wave 4 only, P);
//                WY  W and U~ for its 32 columns from T diag(beta) (split in
//                    two bf16 halves for precision).
// Iteration `it` runs G(it), SOL(it-1), WY(it-2) and the state update of
// chunk it-3; a single workgroup barrier per iteration orders every hand-off
// through LDS.
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;
constexpr int D = kHeadDim;
constexpr int kThreads = 768;  // 4 state waves, 4 gate waves, 4 solve/WY waves
constexpr int kRawSlots = 3;  // chunks staged in LDS: the one being read + 2 in flight

// LDS bank layout.  gfx950 serves 64-bit reads 32 lanes at a time from 64
// banks, 128-bit reads in four passes, and writes 16 lanes at a time into
// 32 banks.  The tiles below are placed (XOR swizzles measured conflict-free
// for the access patterns used here) so that lanes served together hit
// distinct banks:
//  * token-major tiles [16 tokens][128 channels] are read and written one
//    token row per lane; the 16-byte chunk c of row r is stored at c ^ r;
//  * 16-element bf16 rows (channel-major tiles, T diag(beta), P) are accessed
//    in 4-element chunks; chunk g of row r is stored at g ^ (bits 2-3 of r);
//  * 16-element fp32 rows (U~) likewise, at g ^ (bits 1-2 of r).
constexpr int AP = C + 4;  // padded row of the fp32 A matrix

__device__ __forceinline__ int tok_off(int r, int e) { return 8 * ((e >> 3) ^ (r & 15)) + (e & 7); }
__device__ __forceinline__ int chunk16(int r, int g) { return 4 * (g ^ ((r >> 2) & 3)); }
__device__ __forceinline__ int chunk32(int r, int g) { return 4 * (g ^ ((r >> 1) & 3)); }

struct __align__(16) Shared {
    uint16_t kt_row[2][C][D];  // Kt, token-major (bf16)
    uint16_t kh_row[2][C][D];  // Kh, token-major
    uint16_t qt_row[4][C][D];  // Qt (scale folded in), token-major
    uint16_t kt_col[3][D][C];  // Kt, channel-major
    uint16_t v_col[3][D][C];   // V, column-major
    uint16_t kb_col[4][D][C];  // Kbar, channel-major
    float gam_c[4][D];         // Gamma_C per channel
    float beta[2][C];          // sigmoid(beta logits), 0 on padding rows
    float amat[C][AP];         // A; every chunk wave writes the same values
    uint16_t tb_hi[2][C][C];   // T diag(beta) = hi + lo, two bf16 parts
    uint16_t tb_lo[2][C][C];
    uint16_t pmat[3][C][C];    // P
    uint16_t w_row[2][C][D];  // W, token-major
    float ut[2][D][C];         // U~, column-major
    // raw q, k, g, v of a chunk as fetched by each chunk wave (16 bytes per
    // lane, lane order), and the beta logits (zero-extended, chunk wave 0)
    u32x4_t raw[kRawSlots][4][4][64];
    uint32_t raw_beta[kRawSlots][64];
};

struct RawChunk {
    u32x4_t q, k, g, v;  // 8 bf16 each: one token, 8 consecutive channels
    uint32_t beta;       // bf16 logit in the low half (wave 4, lanes 0-15)
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ u32x2_t pack_bf16x4(f32x4_t x)
{
    return u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
}
__device__ __forceinline__ f32x4_t mfma32(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(u32x2_t a, u32x2_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                     __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8_t cat8(u32x2_t lo, u32x2_t hi)
{
    return __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
}
template <typename V>
__device__ __forceinline__ V lds_load(const void *p)
{
    return *static_cast<const V *>(p);
}
template <typename V>
__device__ __forceinline__ void lds_store(void *p, V v)
{
    *static_cast<V *>(p) = v;
}

// Workgroup barrier that orders LDS only.  Outstanding global loads (the
// prefetch) stay in flight across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS byte address of a __shared__ object, as a wave-uniform (scalar) value.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)(p))));
}

// Global -> LDS copies that bypass registers: every lane's 16 bytes (or its
// 2 bytes, zero-extended to 4) land at `lds` + lane * 16 (or * 4).  They are
// issued from inline assembly so that the compiler neither waits on them nor
// reorders them; completion is awaited explicitly with wait_vmem<N>() before
// the staged data is read.
__device__ __forceinline__ void dma_b128(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma_u16(const void *g, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_ushort %0, off" ::"v"(g), "s"(lds)
                 : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmem()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Broadcast lane `m` of each 16-lane row to the whole row.
template <int M>
__device__ __forceinline__ float row_bcast(float x)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + M, 0xF, 0xF, false));
}

// Every lane receives x from the lane with the same l16 in each of the four
// 16-lane rows (r0..r3 = rows 0..3).  v_permlane16_swap exchanges the odd
// rows of its first operand with the even rows of its second,
// v_permlane32_swap the upper 32 lanes of its first operand with the lower
// 32 of its second.  They are issued from inline assembly: with a register
// and its copy as operands the compiler folds the second result of the
// builtin into the first.  The s_nop covers the wait states a swap needs
// after a vector write of its operands.
__device__ __forceinline__ void swap_rows16(uint32_t &a, uint32_t &b)
{
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_rows32(uint32_t &a, uint32_t &b)
{
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void row_gather(float x, float &r0, float &r1, float &r2, float &r3)
{
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    swap_rows16(a, b);  // a: rows {0,0,2,2}, b: rows {1,1,3,3}
    uint32_t c = a, d = b;
    swap_rows32(a, c);  // a: {0,0,0,0}, c: {2,2,2,2}
    swap_rows32(b, d);  // b: {1,1,1,1}, d: {3,3,3,3}
    r0 = __builtin_bit_cast(float, a);
    r1 = __builtin_bit_cast(float, b);
    r2 = __builtin_bit_cast(float, c);
    r3 = __builtin_bit_cast(float, d);
}

// ---------------------------------------------------------------------------
// chunk waves
// ---------------------------------------------------------------------------

struct ChunkWave {
    const FwdParams &p;
    Shared &sh;
    int64_t t_begin, t_end;
    int nchunks;
    int pw;  // 0..3
    int lane, l16, g4;
    // Fetch addressing.  The bases and strides are wave-uniform (scalar
    // registers); only the lane offsets are per lane.
    const char *base_q, *base_k, *base_g, *base_v;  // channel 32 pw of token t_begin
    const char *base_beta;                          // beta of token t_begin
    int64_t chunk_bytes;       // between consecutive chunks of q/k/g/v: C * H * 256
    int64_t beta_chunk_bytes;  // between consecutive chunks of beta: C * H * 2
    int64_t lane_full;         // lane offset for token l16: l16 * H * 256 + 16 * g4
    int64_t lane_tail;         // lane offset for a row past the sequence end (token 0)
    int64_t beta_lane;         // beta lane offset for token `lane`: lane * H * 2
    uint32_t lds_raw;          // LDS address of raw[0][pw][0][0]
    uint32_t lds_raw_beta;     // LDS address of raw_beta[0][0]
    float head_neg;     // -exp(A_log[h]) * log2(e)
    float bias_neg[2];  // head_neg * dt_bias[h][ch] for the two 16-channel tiles
    bf16x8_t sel[2];    // 0/1 selection matrices for the channel-major transposes
    u32x2_t ident;      // 16x16 identity as an x16 B operand
    float grp_ge[3];    // (g4 >= 1), (g4 >= 2), (g4 >= 3)
    float grp_le[3];    // (g4 <= 0), (g4 <= 1), (g4 <= 2)
    float diag_one;     // (l16 == 4 pw + g4): row i equals column j of T
    float diag_below;   // (l16 >  4 pw + g4)

    __device__ int chunk_len(int x) const
    {
        const int64_t left = t_end - (t_begin + int64_t(x) * C);
        return static_cast<int>(left < C ? left : C);
    }

    // Copy chunk x into LDS slot `slot` (this wave's 32 channels of q, k, g,
    // v; chunk wave 0 also the 16 beta logits).  Every lane copies something
    // valid: rows past the sequence end re-read the chunk's first token and
    // are masked in the gate stage.  kDmaPerChunk copies per wave (+1 beta).
    static constexpr int kDmaPerChunk = 4;
    static constexpr uint32_t kSlotBytes = sizeof(Shared::raw[0]);
    static constexpr uint32_t kTensorBytes = sizeof(Shared::raw[0][0][0]);
    __device__ void fetch(int x, int slot) const
    {
        const int len = chunk_len(x);
        const int64_t off = l16 < len ? lane_full : lane_tail;
        const int64_t cb = int64_t(x) * chunk_bytes;
        const uint32_t m = lds_raw + static_cast<uint32_t>(slot) * kSlotBytes;
        dma_b128(base_q + cb + off, m);
        dma_b128(base_k + cb + off, m + kTensorBytes);
        dma_b128(base_g + cb + off, m + 2 * kTensorBytes);
        dma_b128(base_v + cb + off, m + 3 * kTensorBytes);
        if (pw == 0)
            dma_u16(base_beta + int64_t(x) * beta_chunk_bytes + (lane < len ? beta_lane : 0),
                    lds_raw_beta + static_cast<uint32_t>(slot) * sizeof(Shared::raw_beta[0]));
    }
    // Wait until the copies of the chunk fetched two fetches ago have landed.
    __device__ void wait_fetched() const
    {
        if (pw == 0)
            wait_vmem<2 * (kDmaPerChunk + 1)>();
        else
            wait_vmem<2 * kDmaPerChunk>();
    }
    __device__ RawChunk staged(int slot) const
    {
        RawChunk r;
        r.q = sh.raw[slot][pw][0][lane];
        r.k = sh.raw[slot][pw][1][lane];
        r.g = sh.raw[slot][pw][2][lane];
        r.v = sh.raw[slot][pw][3][lane];
        r.beta = sh.raw_beta[slot][lane];
        return r;
    }

    // G: gate, decay products and the decayed operands of chunk x.
    __device__ void gate_stage(int x, int s3, const RawChunk &r) const
    {
        const int len = chunk_len(x);
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        const int s2 = x & 1, s4 = x & 3;
        {
            const float b = sigmoid_f32(bf16_to_f32(static_cast<uint16_t>(r.beta)));
            if (pw == 0 && lane < C)
                sh.beta[s2][lane] = lane < len ? b : 0.f;
        }

#pragma unroll
        for (int t = 0; t < 2; ++t) {
            // channel-major tiles: lane (l16, g4) holds tokens 4*g4 + i of
            // channel 32*pw + 16*t + l16
            const f32x4_t cq = mfma32(__builtin_bit_cast(bf16x8_t, r.q), sel[t], zero);
            const f32x4_t ck = mfma32(__builtin_bit_cast(bf16x8_t, r.k), sel[t], zero);
            const f32x4_t cg = mfma32(__builtin_bit_cast(bf16x8_t, r.g), sel[t], zero);
            const f32x4_t cv = mfma32(__builtin_bit_cast(bf16x8_t, r.v), sel[t], zero);

            // Rows past the sequence end hold a copy of the chunk's first
            // token.  Only their decay needs masking (alpha = 1): their beta
            // is 0, which zeroes their rows and columns of T diag(beta) and so
            // of W, U~ and U; their A, P and output entries are never used.
            float al[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = exp2_f32(fmaf(cg[i], head_neg, bias_neg[t]));
                const float s = __builtin_amdgcn_rcpf(1.0f + e);
                const float a = exp2_f32(p.gate_scale * s);
                al[i] = (4 * g4 + i < len) ? a : 1.0f;
            }
            // products within the 4-token group, then across the 4 groups
            const float p0 = al[0], p1 = p0 * al[1], p2 = p1 * al[2], p3 = p2 * al[3];
            const float s3_ = 1.0f, s2_ = al[3], s1_ = al[2] * al[3], s0_ = al[1] * s1_;
            float P0, P1, P2, P3;
            row_gather(p3, P0, P1, P2, P3);
            const float gc = ((P0 * P1) * P2) * P3;
            // products of the group totals before and after this lane's group,
            // selected exactly with per-lane 0/1 factors f: f * P + (1 - f)
            // (no lane masks to keep live)
            const float pre = fmaf(grp_ge[0], P0, 1.0f - grp_ge[0]) *
                              fmaf(grp_ge[1], P1, 1.0f - grp_ge[1]) *
                              fmaf(grp_ge[2], P2, 1.0f - grp_ge[2]);
            const float suf = fmaf(grp_le[2], P3, 1.0f - grp_le[2]) *
                              fmaf(grp_le[1], P2, 1.0f - grp_le[1]) *
                              fmaf(grp_le[0], P1, 1.0f - grp_le[0]);
            const float inv_gc = __builtin_amdgcn_rcpf(gc);
            const float gam[4] = {pre * p0, pre * p1, pre * p2, pre * p3};
            const float gbar[4] = {s0_ * suf, s1_ * suf, s2_ * suf, s3_ * suf};

            f32x4_t kt, qt, kb, kh;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kt[i] = ck[i] * gam[i];
                qt[i] = cq[i] * (p.scale * gam[i]);
                kb[i] = ck[i] * gbar[i];
                kh[i] = kb[i] * inv_gc;
            }
            const int ch = 32 * pw + 16 * t + l16;
            const u32x2_t kt2 = pack_bf16x4(kt), qt2 = pack_bf16x4(qt), kb2 = pack_bf16x4(kb),
                          kh2 = pack_bf16x4(kh), v2 = pack_bf16x4(cv);
            const int cc = chunk16(ch, g4);
            lds_store(&sh.kt_col[s3][ch][cc], kt2);
            lds_store(&sh.v_col[s3][ch][cc], v2);
            lds_store(&sh.kb_col[s4][ch][cc], kb2);
            if (g4 == 0)
                sh.gam_c[s4][ch] = gc;
            // token-major copies: (X^T I) puts 4 consecutive channels of one
            // token in each lane
            const int col = tok_off(l16, 32 * pw + 16 * t + 4 * g4);
            lds_store(&sh.kt_row[s2][l16][col], pack_bf16x4(mfma16(kt2, ident, zero)));
            lds_store(&sh.kh_row[s2][l16][col], pack_bf16x4(mfma16(kh2, ident, zero)));
            lds_store(&sh.qt_row[s4][l16][col], pack_bf16x4(mfma16(qt2, ident, zero)));
        }
    }

    // SOL: A, four columns of T, and (wave 4) P for chunk x.
    __device__ void solve_stage(int x, int s3) const
    {
        const int s2 = x & 1, s4 = x & 3;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, pacc = acc;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const int col = tok_off(l16, 32 * kt + 8 * g4);
            const bf16x8_t a = lds_load<bf16x8_t>(&sh.kt_row[s2][l16][col]);
            const bf16x8_t b = lds_load<bf16x8_t>(&sh.kh_row[s2][l16][col]);
            acc = mfma32(a, b, acc);
            if (pw == 0) {
                const bf16x8_t q = lds_load<bf16x8_t>(&sh.qt_row[s4][l16][col]);
                pacc = mfma32(b, q, pacc);
            }
        }
        // acc: lane (j = l16, g4) holds (Kt Kh^T)[4*g4 + i][j]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row_i = 4 * g4 + i;
            sh.amat[row_i][l16] = l16 < row_i ? sh.beta[s2][row_i] * acc[i] : 0.f;
        }
        if (pw == 0) {
            // pacc: lane (i = l16, g4) holds P[i][4*g4 + e]
            f32x4_t pm;
#pragma unroll
            for (int e = 0; e < 4; ++e) pm[e] = (4 * g4 + e <= l16) ? pacc[e] : 0.f;
            lds_store(&sh.pmat[s3][l16][chunk16(l16, g4)], pack_bf16x4(pm));
        }

        // T[:, j] for j = 4*pw + g4; lane (g4, l16 = row i).  Right-looking
        // forward substitution: once t_m is known, every later row adds
        // A[i][m] t_m to its running sum.
        const int j = 4 * pw + g4, i = l16;
        float arow[C];  // A[i][:], zero from column i on
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4_t v = lds_load<f32x4_t>(&sh.amat[i][4 * q4]);
            arow[4 * q4 + 0] = v[0];
            arow[4 * q4 + 1] = v[1];
            arow[4 * q4 + 2] = v[2];
            arow[4 * q4 + 3] = v[3];
        }
        // Lane i keeps run = sum_m A[i][m] t_m; t_i = e_ij - g_ij * run where
        // e_ij = (i == j) and g_ij = (i > j).  Step m broadcasts t_m from lane
        // m of each 16-lane row; A[i][m] = 0 for m >= i, so the update needs no
        // condition.
        float run = 0.f;
        solve_steps(arow, run);
        const float t_i = fmaf(-diag_below, run, diag_one);
        const float tb = t_i * sh.beta[s2][j];
        const __bf16 hi = static_cast<__bf16>(tb);
        const __bf16 lo = static_cast<__bf16>(tb - static_cast<float>(hi));
        // element (i, j) lives in chunk j / 4 = pw at position j % 4 = g4
        sh.tb_hi[s2][i][chunk16(i, pw) + g4] = __builtin_bit_cast(uint16_t, hi);
        sh.tb_lo[s2][i][chunk16(i, pw) + g4] = __builtin_bit_cast(uint16_t, lo);
    }

    template <int M = 0>
    __device__ __forceinline__ void solve_steps(const float (&arow)[C], float &run) const
    {
        if constexpr (M < C) {
            const float tm = row_bcast<M>(fmaf(-diag_below, run, diag_one));
            run = fmaf(arow[M], tm, run);
            solve_steps<M + 1>(arow, run);
        }
    }

};

// WY: W and U~ for this wave's 32 columns of chunk x.
__device__ void wy_stage(Shared &sh, int x, int s3, int pw, int l16, int g4)
{
    const int s2 = x & 1;
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    // lane (l16, g4) holds (T diag(beta))[l16][4*g4 .. 4*g4+3]: the A operand
    // of T diag(beta) V and the B operand of Kt^T (T diag(beta))^T
    const u32x2_t th = lds_load<u32x2_t>(&sh.tb_hi[s2][l16][chunk16(l16, g4)]);
    const u32x2_t tl = lds_load<u32x2_t>(&sh.tb_lo[s2][l16][chunk16(l16, g4)]);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int ch = 32 * pw + 16 * t + l16;
        const u32x2_t ka = lds_load<u32x2_t>(&sh.kt_col[s3][ch][chunk16(ch, g4)]);
        f32x4_t w = mfma16(ka, th, zero);
        w = mfma16(ka, tl, w);  // lane (token l16, g4): W[l16][32pw+16t+4g4+i]
        lds_store(&sh.w_row[s2][l16][tok_off(l16, 32 * pw + 16 * t + 4 * g4)], pack_bf16x4(w));
        const u32x2_t vb = lds_load<u32x2_t>(&sh.v_col[s3][ch][chunk16(ch, g4)]);
        f32x4_t u = mfma16(th, vb, zero);
        u = mfma16(tl, vb, u);  // lane (vcol, g4): U~[4g4+i][vcol]
        lds_store(&sh.ut[s2][ch][chunk32(ch, g4)], u);
    }
}

// ---------------------------------------------------------------------------
// state waves
// ---------------------------------------------------------------------------

template <int INIT, int FINAL>
struct StateWave {
    const FwdParams &p;
    Shared &sh;
    int64_t t_begin, t_end, chain;
    int w, lane, l16, g4;
    uint16_t *dst_out;   // out at token t_begin, value column 32w + 4g4
    int64_t tok_stride;  // H * 128
    f32x4_t S[8][2];     // S[16mt + 4g4 + i][32w + 16nt + l16]

    __device__ int64_t state_index(int mt, int nt) const
    {
        return (chain * D + 32 * w + 16 * nt + l16) * D + 16 * mt + 4 * g4;
    }

    __device__ void load_state()
    {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int64_t idx = state_index(mt, nt);
                if constexpr (INIT == kStateFp32) {
                    S[mt][nt] = *reinterpret_cast<const f32x4_t *>(
                        static_cast<const float *>(p.init_state) + idx);
                } else if constexpr (INIT == kStateBf16) {
                    const u32x2_t b = *reinterpret_cast<const u32x2_t *>(
                        static_cast<const uint16_t *>(p.init_state) + idx);
                    S[mt][nt] = f32x4_t{__uint_as_float(b[0] << 16), __uint_as_float(b[0] & 0xffff0000u),
                                        __uint_as_float(b[1] << 16), __uint_as_float(b[1] & 0xffff0000u)};
                } else {
                    S[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
            }
    }

    __device__ void store_state() const
    {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int64_t idx = state_index(mt, nt);
                if constexpr (FINAL == kStateFp32) {
                    *reinterpret_cast<f32x4_t *>(static_cast<float *>(p.final_state) + idx) = S[mt][nt];
                } else if constexpr (FINAL == kStateBf16) {
                    *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(p.final_state) + idx) =
                        u32x2_t{uint32_t(f32_to_bf16_rne(S[mt][nt][0])) |
                                    (uint32_t(f32_to_bf16_rne(S[mt][nt][1])) << 16),
                                uint32_t(f32_to_bf16_rne(S[mt][nt][2])) |
                                    (uint32_t(f32_to_bf16_rne(S[mt][nt][3])) << 16)};
                }
            }
    }

    __device__ void chunk(int x, int s3)
    {
        const int s2 = x & 1, s4 = x & 3;
        const int64_t left = t_end - (t_begin + int64_t(x) * C);
        const int len = static_cast<int>(left < C ? left : C);

        // S as bf16 B operands; contraction slot 8*g4 + e maps to state row
        // 32kt + 4g4 + e (e < 4) and 32kt + 16 + 4g4 + (e - 4) (e >= 4), which
        // is exactly what this lane's accumulators of tiles 2kt, 2kt+1 hold.
        bf16x8_t sb[4][2];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                sb[kt][nt] = cat8(pack_bf16x4(S[2 * kt][nt]), pack_bf16x4(S[2 * kt + 1][nt]));

        // X = W S (lane (vcol, g4): rows 4g4..4g4+3) and Y^T = S^T Qt^T (lane
        // (token, g4): value columns 4g4..4g4+3 of the tile), from the same
        // operand registers with the roles of A and B swapped
        f32x4_t X[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4_t Y[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const int lo = tok_off(l16, 32 * kt + 4 * g4), hi = tok_off(l16, 32 * kt + 16 + 4 * g4);
            const bf16x8_t wa = cat8(lds_load<u32x2_t>(&sh.w_row[s2][l16][lo]),
                                     lds_load<u32x2_t>(&sh.w_row[s2][l16][hi]));
            const bf16x8_t qa = cat8(lds_load<u32x2_t>(&sh.qt_row[s4][l16][lo]),
                                     lds_load<u32x2_t>(&sh.qt_row[s4][l16][hi]));
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                X[nt] = mfma32(wa, sb[kt][nt], X[nt]);
                Y[nt] = mfma32(sb[kt][nt], qa, Y[nt]);
            }
        }

        // U = U~ - W S, as bf16 operands (lane (vcol, g4): tokens 4g4..4g4+3)
        u32x2_t ub[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int vc = 32 * w + 16 * nt + l16;
            const f32x4_t u = lds_load<f32x4_t>(&sh.ut[s2][vc][chunk32(vc, g4)]) - X[nt];
            ub[nt] = pack_bf16x4(u);
        }

        // O^T = Y^T + U^T P^T; lane (token l16, g4) then holds 4 consecutive
        // output values of its token and stores them directly
        const u32x2_t pa = lds_load<u32x2_t>(&sh.pmat[s3][l16][chunk16(l16, g4)]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const f32x4_t o = mfma16(ub[nt], pa, Y[nt]);
            if (l16 < len)
                *reinterpret_cast<u32x2_t *>(dst_out + (int64_t(x) * C + l16) * tok_stride + 16 * nt) =
                    pack_bf16x4(o);
        }

        // S <- diag(Gamma_C) S + Kbar^T U
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const f32x4_t gc = lds_load<f32x4_t>(&sh.gam_c[s4][16 * mt + 4 * g4]);
            const u32x2_t ka = lds_load<u32x2_t>(&sh.kb_col[s4][16 * mt + l16][chunk16(l16, g4)]);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) S[mt][nt] = mfma16(ka, ub[nt], S[mt][nt] * gc);
        }
    }
};

template <int INIT, int FINAL>
__global__ __launch_bounds__(kThreads, 1) void chunk_mfma_kernel(FwdParams p)
{
    __shared__ Shared sh;
    const int64_t chain = blockIdx.x;
    const int64_t n = chain / p.H, h = chain % p.H;
    int64_t t_begin, t_end, row;
    chain_segment(p, n, &t_begin, &t_end, &row);
    const int64_t nchunks = (t_end - t_begin + C - 1) / C;  // < 2^31 (T is bounded on the host)
    const int n_iter = nchunks > 0 ? static_cast<int>(nchunks) + 3 : 0;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t tok_stride = p.H * D;
    const int64_t first = (row * p.T + t_begin) * p.H + h;  // token-head row of t_begin

    if (wave < 4) {
        StateWave<INIT, FINAL> sw{p, sh, t_begin, t_end, chain, wave, lane, l16, g4,
                                  p.out + first * D + 32 * wave + 4 * g4, tok_stride, {}};
        sw.load_state();
        const int nc = static_cast<int>(nchunks);
        int s3 = 0, wy3 = 1;  // chunk index mod 3 of the updated and the WY chunk
        for (int it = 0; it < n_iter; ++it) {
            if (it >= 3) {
                sw.chunk(it - 3, s3);
                s3 = s3 == 2 ? 0 : s3 + 1;
            }
            // W and U~ of chunk it-2 for this wave's 32 channels / value columns
            if (it >= 2 && it - 2 < nc)
                wy_stage(sh, it - 2, wy3, wave, l16, g4);
            wy3 = wy3 == 2 ? 0 : wy3 + 1;
            lds_barrier();
        }
        sw.store_state();
        return;
    }

    // waves 4-7 stream chunks in and run the gate stage; waves 8-11 run the
    // solve and WY stages.  Both kinds own the 32 channels 32*pw..32*pw+31.
    const bool gate_wave = wave < 8;
    const int pw = gate_wave ? wave - 4 : wave - 8;
    const int64_t wave_off = (first * D + 32 * pw) * 2;  // bytes
    const int64_t tok_bytes = tok_stride * 2;
    ChunkWave cw{p, sh, t_begin, t_end, static_cast<int>(nchunks), pw, lane, l16, g4,
                 reinterpret_cast<const char *>(p.q) + wave_off,
                 reinterpret_cast<const char *>(p.k) + wave_off,
                 reinterpret_cast<const char *>(p.g) + wave_off,
                 reinterpret_cast<const char *>(p.v) + wave_off,
                 reinterpret_cast<const char *>(p.beta + first),
                 C * tok_bytes, C * p.H * 2,
                 l16 * tok_bytes + 16 * g4, 16 * g4, lane * p.H * 2,
                 lds_addr(&sh.raw[0][pw][0][0]), lds_addr(&sh.raw_beta[0][0])};
    const int nc = static_cast<int>(nchunks);

    if (!gate_wave) {
        cw.diag_one = l16 == 4 * pw + g4 ? 1.0f : 0.0f;
        cw.diag_below = l16 > 4 * pw + g4 ? 1.0f : 0.0f;
        int sol3 = 2;  // chunk index mod 3 of the SOL chunk
        for (int it = 0; it < n_iter; ++it) {
            if (it >= 1 && it - 1 < nc)
                cw.solve_stage(it - 1, sol3);
            sol3 = sol3 == 2 ? 0 : sol3 + 1;
            lds_barrier();
        }
        return;
    }

    const float head_mult = p.A_log ? expf(p.A_log[h]) : 1.0f;
    cw.head_neg = -head_mult * kLog2eF;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int ch = 32 * pw + 16 * t + l16;
        cw.bias_neg[t] = p.dt_bias ? cw.head_neg * p.dt_bias[h * D + ch] : 0.f;
        // selection matrix: element e of lane (l16, g4) is 1 when contraction
        // index 8*g4 + e equals channel 16*t + l16
        bf16x8_t sel;
#pragma unroll
        for (int e = 0; e < 8; ++e) sel[e] = static_cast<__bf16>((8 * g4 + e == 16 * t + l16) ? 1.0f : 0.0f);
        cw.sel[t] = sel;
    }
    {
        uint16_t idb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) idb[e] = (4 * g4 + e == l16) ? 0x3F80 : 0;
        cw.ident = u32x2_t{uint32_t(idb[0]) | (uint32_t(idb[1]) << 16),
                           uint32_t(idb[2]) | (uint32_t(idb[3]) << 16)};
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        cw.grp_ge[q] = g4 >= q + 1 ? 1.0f : 0.0f;
        cw.grp_le[q] = g4 <= q ? 1.0f : 0.0f;
    }
    if (n_iter == 0)
        return;

    // chunks 0 and 1 go to slots 0 and 1; iteration `it` fetches chunk it+2
    cw.fetch(0, 0);
    cw.fetch(nc > 1 ? 1 : 0, 1);
    int g3 = 0;  // chunk index mod 3 of the G chunk
    for (int it = 0; it < n_iter; ++it) {
        // G runs in every iteration: past the last chunk it only fills LDS
        // slots that no later stage reads.
        const int s_next = g3 == 0 ? 2 : g3 - 1;  // slot (it + 2) % 3
        cw.fetch(it + 2 < nc ? it + 2 : nc - 1, s_next);
        cw.wait_fetched();
        cw.gate_stage(it, g3, cw.staged(g3));
        g3 = g3 == 2 ? 0 : g3 + 1;
        lds_barrier();
    }
    // no copy may still be writing LDS when the wave ends
    wait_vmem<0>();
}

template <int INIT, int FINAL>
hipError_t launch(const FwdParams &p, hipStream_t stream)
{
    const int64_t chains = p.num_seqs * p.H;
    FwdParams args = p;
    void *argv[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void *>(&chunk_mfma_kernel<INIT, FINAL>),
                           dim3(static_cast<unsigned>(chains)), dim3(kThreads), argv, 0, stream);
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

hipError_t launch_chunk_mfma(const FwdParams &p, hipStream_t stream)
{
    switch (p.init_kind) {
    case kStateBf16: return launch_final<kStateBf16>(p, stream);
    case kStateFp32: return launch_final<kStateFp32>(p, stream);
    default: return launch_final<kStateNone>(p, stream);
    }
}

}  // namespace kda
