// Chunked KDA forward kernel for gfx950: bf16 MFMA for every contraction,
// fp32 state held in accumulator registers, one workgroup of 16 waves per
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
// Wave roles (64-lane waves; lane = 16 * g4 + l16; wave w runs on SIMD w % 4,
// so every SIMD holds one state wave, two gate waves and one solve wave):
//   waves 0-3    state waves.  Wave w owns the 128 x 32 slab S[:, 32w:32w+32]
//                of the state as 16 fp32 16x16 accumulator tiles.  Per chunk:
//                U = U~ - W S, O = Qt S + P U (stores out) and the state
//                update.  S is the B operand of W S and Qt S through a fixed
//                permutation of the contraction index, so the fp32
//                accumulators convert to bf16 operands in place.
//   waves 4-11   gate waves.  Wave 4 + c owns channels 16c..16c+15: it loads
//                q, k, g, v and beta straight into registers two chunks ahead,
//                transposes q, k, g to channel-major with an MFMA against the
//                identity, computes the gate, the cumulative decay products
//                and the decayed operands, and stores them channel-major (v
//                as loaded, token-major).
//   waves 12-15  solve waves.  Wave 12 forms A, wave 13 P (from the
//                channel-major tiles, read as token-major operands through
//                transposing LDS reads), waves 14 and 15 solve columns 0..7
//                and 8..15 of T; wave 12 + p then runs the WY stage (W and
//                U~) for channels / value columns 32p..32p+31.
// The state and solve waves run at raised issue priority: they carry the
// serial dependency chains of an iteration, and the gate waves (ample
// independent work) fill the issue slots they leave.
// Iteration `it` runs the gate stage of chunk it, A and P of chunk it-1, the
// solve of chunk it-2, WY of chunk it-3 and the state update of chunk it-4;
// one workgroup barrier per iteration orders every hand-off through LDS.
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;
constexpr int D = kHeadDim;
constexpr int kThreads = 1024;  // 4 state waves, 8 gate waves, 4 solve waves
constexpr int kStages = 4;      // iterations between the gate and the state stage of a chunk

// LDS bank layout.  gfx950 serves 64-bit reads 32 lanes at a time from 64
// banks, 128-bit reads in four passes, and writes 16 lanes at a time into
// 32 banks.  The tiles below are placed (XOR swizzles measured conflict-free
// for the access patterns used here) so that lanes served together hit
// distinct banks:
//  * token-major tiles [16 tokens][128 channels] are read and written one
//    token row per lane; the 16-byte chunk c of row r is stored at c ^ r;
//  * 16-element bf16 rows (channel-major tiles, T diag(beta), P) are accessed
//    in 4-element chunks; chunk g of row r is stored at g ^ (bits 2-3 of r);
//  * 16-element fp32 rows (U~) likewise, at g ^ (bits 1-2 of r);
//  * 16 x 16 fp32 matrices use a row pitch of 20 floats.
constexpr int AP = C + 4;

__device__ __forceinline__ int tok_off(int r, int e) { return 8 * ((e >> 3) ^ (r & 15)) + (e & 7); }
__device__ __forceinline__ int chunk16(int r, int g) { return 4 * (g ^ ((r >> 2) & 3)); }
__device__ __forceinline__ int chunk32(int r, int g) { return 4 * (g ^ ((r >> 1) & 3)); }

// Ring buffers between the stages; a tile written for chunk x lives in slot
// x mod (its ring size), which is sized to outlive its last reader.
struct __align__(16) Shared {
    uint16_t kt_col[4][D][C];  // Kt, channel-major; read by A and WY
    uint16_t kh_col[2][D][C];  // Kh, channel-major; read by A and P
    uint16_t qt_col[5][D][C];  // Qt (scale folded in), channel-major; read by P and the state stage
    uint16_t v_row[4][C][D];   // V as loaded, token-major; read by WY
    uint16_t kb_col[5][D][C];  // Kbar, channel-major; read by the state stage
    float gam_c[5][D];         // Gamma_C per channel
    float beta[3][C];          // sigmoid(beta logits), 0 on padding rows
    float amat[2][C][AP];      // -A = -diag(beta) Kt Kh^T, strictly lower
    uint16_t pmat[4][C][C];    // P (bf16), lower
    uint16_t tb_hi[2][C][C];   // T diag(beta) = hi + lo, two bf16 parts
    uint16_t tb_lo[2][C][C];
    uint16_t w_row[2][C][D];   // W, token-major
    float ut[2][D][C];         // U~, column-major
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

// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane row, lane
// L supplies the four bf16 at its address, X[L][0..3], and lane i receives
// X[4r + i/4][i%4] for r = 0..3.  With lane L of row g4 pointing at tokens
// 4(L%4)..4(L%4)+3 of channel c0 + 4 g4 + L/4 of a channel-major tile, lane
// (token i, g4) receives channels c0 + 4 g4 .. c0 + 4 g4 + 3 of token i: the
// token-major operand of an MFMA that contracts over channels.
__device__ __forceinline__ u32x2_t tok_operand(const uint16_t (&col)[D][C], int c0, int l16, int g4)
{
    const int c = c0 + 4 * g4 + (l16 >> 2);
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t *)(&col[c][chunk16(c, l16 & 3)]));
    return __builtin_bit_cast(u32x2_t, v);
}
// The same read on a token-major tile: with lane L of row g4 pointing at
// channels c0 + 4(L%4) .. c0 + 4(L%4) + 3 of token 4 g4 + L/4, lane (l16, g4)
// receives tokens 4 g4 .. 4 g4 + 3 of channel c0 + l16: the channel-major
// operand of an MFMA that contracts over tokens.
__device__ __forceinline__ u32x2_t chan_operand(const uint16_t (&row)[C][D], int c0, int l16, int g4)
{
    const int r = 4 * g4 + (l16 >> 2);
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t *)(&row[r][tok_off(r, c0 + 4 * (l16 & 3))]));
    return __builtin_bit_cast(u32x2_t, v);
}
// Eight channels per lane for a 16x16x32 operand over channels 32kt..32kt+31:
// contraction slot 8 g4 + e is channel 32kt + 4 g4 + e (e < 4) and
// 32kt + 16 + 4 g4 + (e - 4) (e >= 4).
__device__ __forceinline__ bf16x8_t tok_operand32(const uint16_t (&col)[D][C], int kt, int l16, int g4)
{
    return cat8(tok_operand(col, 32 * kt, l16, g4), tok_operand(col, 32 * kt + 16, l16, g4));
}

// Workgroup barrier that orders LDS only.  Outstanding global loads (the
// prefetch) stay in flight across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmem()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Cross-row swaps: v_permlane16_swap exchanges the odd rows (16 lanes each)
// of its first operand with the even rows of its second, v_permlane32_swap
// the upper 32 lanes of its first operand with the lower 32 of its second.
// (The results are copied out element by element: a __builtin_bit_cast of a
// vector element reads element 0 with this compiler.)
__device__ __forceinline__ void swap_rows16(uint32_t &a, uint32_t &b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    a = r0;
    b = r1;
}
__device__ __forceinline__ void swap_rows32(uint32_t &a, uint32_t &b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    a = r0;
    b = r1;
}

// Products over the four 16-lane rows r0..r3 of x (one value per row at the
// same l16): the total, and for this lane's row g4 the product of the rows
// before it (pre) and after it (suf).  fh = (g4 >= 2), fo = (g4 odd) as 0/1
// floats; f * y + (1 - f) selects y or 1 exactly.
__device__ __forceinline__ void row_products(float x, float fh, float fo, float &total, float &pre,
                                             float &suf)
{
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    swap_rows16(a, b);  // a: rows {r0,r0,r2,r2}, b: {r1,r1,r3,r3}
    const float fa = __builtin_bit_cast(float, a), fb = __builtin_bit_cast(float, b);
    uint32_t c = __builtin_bit_cast(uint32_t, fa * fb), d = c;  // r0 r1 | r2 r3
    swap_rows32(c, d);  // c: r0 r1 everywhere, d: r2 r3 everywhere
    const float lo = __builtin_bit_cast(float, c), hi = __builtin_bit_cast(float, d);
    total = lo * hi;
    pre = fmaf(fh, lo, 1.0f - fh) * fmaf(fo, fa, 1.0f - fo);
    suf = fmaf(1.0f - fh, hi, fh) * fmaf(1.0f - fo, fb, fo);
}

// ---------------------------------------------------------------------------
// gate waves
// ---------------------------------------------------------------------------

// One chunk of a gate wave's inputs, loaded straight into registers: per
// lane one token (l16) and 4 consecutive channels (16c + 4 g4 ..) of q, k,
// g, v, and (lane < 16) the bf16 beta logit of token `lane` in the low half
// of `beta`.
struct RawRegs {
    u32x2_t q, k, g, v;
    uint32_t beta;
};

// Plain loads: the compiler tracks them and waits (s_waitcnt vmcnt) right
// before the first use of each register set, leaving the loads of the other
// set in flight.
__device__ __forceinline__ u32x2_t gload_b64(const char *p)
{
    return *reinterpret_cast<const u32x2_t *>(p);
}
__device__ __forceinline__ uint32_t gload_u16(const char *p)
{
    return *reinterpret_cast<const uint16_t *>(p);
}

struct GateWave {
    const FwdParams &p;
    Shared &sh;
    int64_t t_begin, t_end;
    int gc16;  // 0..7: channels 16 gc16 .. 16 gc16 + 15, wave-uniform
    int lane, l16, g4;
    // Load addressing.  The bases and strides are wave-uniform (scalar
    // registers); only the lane offsets are per lane.
    const char *base_q, *base_k, *base_g, *base_v;  // channel 16 gc16 of token t_begin
    const char *base_beta;                          // beta of token t_begin
    int64_t chunk_bytes;       // between consecutive chunks of q/k/g/v: C * H * 256
    int64_t beta_chunk_bytes;  // between consecutive chunks of beta: C * H * 2
    int64_t lane_full;         // lane offset for token l16: l16 * H * 256 + 8 * g4
    int64_t lane_tail;         // lane offset for a row past the sequence end (token 0)
    int64_t beta_lane;         // beta lane offset for token `lane`: lane * H * 2
    float head_neg;  // -exp(A_log[h]) * log2(e)
    float bias_neg;  // head_neg * dt_bias[h][16 gc16 + l16]
    u32x2_t ident;   // 16x16 identity as an x16 operand
    float grp_hi;   // (g4 >= 2)
    float grp_odd;  // (g4 odd)

    __device__ int chunk_len(int x) const
    {
        const int64_t left = t_end - (t_begin + int64_t(x) * C);
        return static_cast<int>(left < C ? left : C);
    }

    // Start loading chunk x into r.  Every lane loads something valid: rows
    // past the sequence end re-read the chunk's first token and are masked
    // in the gate stage.
    __device__ void issue(RawRegs &r, int x) const
    {
        const int len = chunk_len(x);
        const int64_t off = (len >= C || l16 < len) ? lane_full : lane_tail;
        const int64_t cb = int64_t(x) * chunk_bytes;
        r.q = gload_b64(base_q + cb + off);
        r.k = gload_b64(base_k + cb + off);
        r.g = gload_b64(base_g + cb + off);
        r.v = gload_b64(base_v + cb + off);
        r.beta = gload_u16(base_beta + int64_t(x) * beta_chunk_bytes + (lane < len ? beta_lane : 0));
    }

    // Gate, decay products and decayed operands of chunk x for this wave's
    // 16 channels.  FULL: all 16 rows of the chunk lie in the sequence.
    __device__ void gate_stage(int x, const RawRegs &r) const
    {
        if (chunk_len(x) >= C)
            gate_rows<true>(x, r);
        else
            gate_rows<false>(x, r);
    }
    template <bool FULL>
    __device__ void gate_rows(int x, const RawRegs &r) const
    {
        const int len = chunk_len(x);
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        const int s2 = x & 1, s3 = x % 3, s4 = x & 3, s5 = x % 5;
        // beta (gate wave 0; every gate wave loads it, so that all of them
        // keep the same number of loads in flight)
        if (gc16 == 0) {
            const float b = sigmoid_f32(bf16_to_f32(static_cast<uint16_t>(r.beta)));
            if (lane < C)
                sh.beta[s3][lane] = (FULL || lane < len) ? b : 0.f;
        }

        // channel-major: (X I) with X token-major puts tokens 4 g4 .. 4 g4 + 3
        // of channel 16 gc16 + l16 in lane (l16, g4)
        const f32x4_t cq = mfma16(r.q, ident, zero);
        const f32x4_t ck = mfma16(r.k, ident, zero);
        const f32x4_t cg = mfma16(r.g, ident, zero);

        // Rows past the sequence end hold a copy of the chunk's first token.
        // Only their decay needs masking (alpha = 1): their beta is 0, which
        // zeroes their rows and columns of T diag(beta) and so of W, U~ and
        // U; their A, P and output entries are never used.
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float e = exp2_f32(fmaf(cg[i], head_neg, bias_neg));
            const float s = __builtin_amdgcn_rcpf(1.0f + e);
            const float a = exp2_f32(p.gate_scale * s);
            al[i] = (FULL || 4 * g4 + i < len) ? a : 1.0f;
        }
        // products within the 4-token group, then across the 4 groups
        const float p0 = al[0], p1 = p0 * al[1], p2 = p1 * al[2], p3 = p2 * al[3];
        const float s3_ = 1.0f, s2_ = al[3], s1_ = al[2] * al[3], s0_ = al[1] * s1_;
        // the group totals of the other rows: all four (gc), those before
        // this lane's group (pre) and those after it (suf)
        float gc, pre, suf;
        row_products(p3, grp_hi, grp_odd, gc, pre, suf);
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
        const int ch = 16 * gc16 + l16, cc = chunk16(ch, g4);
        lds_store(&sh.kt_col[s4][ch][cc], pack_bf16x4(kt));
        lds_store(&sh.kh_col[s2][ch][cc], pack_bf16x4(kh));
        lds_store(&sh.qt_col[s5][ch][cc], pack_bf16x4(qt));
        lds_store(&sh.v_row[s4][l16][tok_off(l16, 16 * gc16 + 4 * g4)], r.v);
        lds_store(&sh.kb_col[s5][ch][cc], pack_bf16x4(kb));
        if (g4 == 0)
            sh.gam_c[s5][ch] = gc;
    }
};

// ---------------------------------------------------------------------------
// solve waves
// ---------------------------------------------------------------------------

struct SolveWave {
    Shared &sh;
    int pw;  // 0..3, wave-uniform
    int l16, g4;

    // -A of chunk x: lane (j = l16, g4) gets (Kt Kh^T)[4 g4 + e][j].
    __device__ void a_stage(int x) const
    {
        const int s2 = x & 1, s3 = x % 3, s4 = x & 3;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
            acc = mfma32(tok_operand32(sh.kt_col[s4], kt, l16, g4),
                         tok_operand32(sh.kh_col[s2], kt, l16, g4), acc);
        const f32x4_t b = lds_load<f32x4_t>(&sh.beta[s3][4 * g4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * g4 + e;
            sh.amat[s2][i][l16] = l16 < i ? -b[e] * acc[e] : 0.f;  // stored negated
        }
    }

    // P of chunk x, as P^T = Kh Qt^T: lane (i = l16, g4) gets
    // P[i][4 g4 .. 4 g4 + 3], the layout the state stage reads.
    __device__ void p_stage(int x) const
    {
        const int s2 = x & 1, s4 = x & 3, s5 = x % 5;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
            acc = mfma32(tok_operand32(sh.kh_col[s2], kt, l16, g4),
                         tok_operand32(sh.qt_col[s5], kt, l16, g4), acc);
        f32x4_t pm;
#pragma unroll
        for (int e = 0; e < 4; ++e) pm[e] = (4 * g4 + e <= l16) ? acc[e] : 0.f;
        lds_store(&sh.pmat[s4][l16][chunk16(l16, g4)], pack_bf16x4(pm));
    }

    // Columns 8 (pw - 2) .. 8 (pw - 2) + 7 of T for chunk x (solve waves 2
    // and 3), stored as T diag(beta).
    __device__ void solve_stage(int x) const
    {
        const int s2 = x & 1, s3 = x % 3;
        // T[:, j] for j = j0, j0 + 1 with j0 = 8 (pw - 2) + 2 g4; lane
        // (g4, l16 = row i).  Right-looking forward substitution on
        // v = e_j - A t: lane i starts from v_i = (i == j); step m takes
        // t_m = v_m (final once the rows above m are done; zero for m < j)
        // from lane m of its 16-lane row and subtracts A[i][m] t_m from every
        // v_i.  A[i][m] = 0 for m >= i, so a row stops changing once it is
        // final.  The two columns run as independent chains.
        const int j0 = 8 * (pw - 2) + 2 * g4, i = l16;
        float nrow[C];  // -A[i][:], zero from column i on
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4_t v = lds_load<f32x4_t>(&sh.amat[s2][i][4 * q4]);
            nrow[4 * q4 + 0] = v[0];
            nrow[4 * q4 + 1] = v[1];
            nrow[4 * q4 + 2] = v[2];
            nrow[4 * q4 + 3] = v[3];
        }
        float v0 = i == j0 ? 1.0f : 0.0f, v1 = i == j0 + 1 ? 1.0f : 0.0f;
        solve_steps(nrow, v0, v1);
        const f32x2_t b2 = lds_load<f32x2_t>(&sh.beta[s3][j0]);
        const float tb0 = v0 * b2[0];
        const float tb1 = v1 * b2[1];
        const __bf16 hi0 = static_cast<__bf16>(tb0), hi1 = static_cast<__bf16>(tb1);
        const __bf16 lo0 = static_cast<__bf16>(tb0 - static_cast<float>(hi0));
        const __bf16 lo1 = static_cast<__bf16>(tb1 - static_cast<float>(hi1));
        // elements (i, j0), (i, j0 + 1): chunk j0 / 4, positions j0 % 4, + 1
        const int pos = chunk16(i, j0 >> 2) + (j0 & 3);
        lds_store(&sh.tb_hi[s2][i][pos], pack_bf16x2(static_cast<float>(hi0), static_cast<float>(hi1)));
        lds_store(&sh.tb_lo[s2][i][pos], pack_bf16x2(static_cast<float>(lo0), static_cast<float>(lo1)));
    }

    // One multiply-add per step and column, with t_m read straight from lane
    // m of the row through the DPP broadcast of the first source (the
    // compiler emits a separate move for the builtin form).  The s_nop gives
    // the two wait states a DPP read needs after the vector write of its
    // source.  Step 15 is skipped: A[i][15] = 0 for every row.
    template <int M = 0>
    __device__ __forceinline__ void solve_steps(const float (&nrow)[C], float &v0, float &v1) const
    {
        if constexpr (M < C - 1) {
            asm volatile("s_nop 1\n\t"
                         "v_fmac_f32_dpp %0, %0, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf\n\t"
                         "v_fmac_f32_dpp %1, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                         : "+v"(v0), "+v"(v1)
                         : "v"(nrow[M]), "n"(M));
            solve_steps<M + 1>(nrow, v0, v1);
        }
    }

    // WY: W and U~ for channels / value columns 32 pw .. 32 pw + 31 of chunk x.
    // T diag(beta) = T_hi + T_lo (two bf16 parts) enters one 16x16x32 MFMA
    // as the contraction [T_hi | T_lo] against [X; X].
    __device__ void wy_stage(int x) const
    {
        const int s2 = x & 1, s4 = x & 3;
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        // lane (l16, g4) holds (T diag(beta))[l16][4*g4 .. 4*g4+3]: the A
        // operand of T diag(beta) V and the B operand of Kt^T (T diag(beta))^T
        const u32x2_t th = lds_load<u32x2_t>(&sh.tb_hi[s2][l16][chunk16(l16, g4)]);
        const u32x2_t tl = lds_load<u32x2_t>(&sh.tb_lo[s2][l16][chunk16(l16, g4)]);
        const bf16x8_t t8 = cat8(th, tl);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int ch = 32 * pw + 16 * t + l16;
            const u32x2_t ka = lds_load<u32x2_t>(&sh.kt_col[s4][ch][chunk16(ch, g4)]);
            // lane (token l16, g4): W[l16][32pw+16t+4g4+i]
            const f32x4_t w = mfma32(cat8(ka, ka), t8, zero);
            lds_store(&sh.w_row[s2][l16][tok_off(l16, 32 * pw + 16 * t + 4 * g4)], pack_bf16x4(w));
            const u32x2_t vb = chan_operand(sh.v_row[s4], 32 * pw + 16 * t, l16, g4);
            // lane (vcol, g4): U~[4g4+i][vcol]
            const f32x4_t u = mfma32(t8, cat8(vb, vb), zero);
            lds_store(&sh.ut[s2][ch][chunk32(ch, g4)], u);
        }
    }
};

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

    __device__ void chunk(int x)
    {
        const int s2 = x & 1, s4 = x & 3, s5 = x % 5;
        const int64_t left = t_end - (t_begin + int64_t(x) * C);
        const int len = static_cast<int>(left < C ? left : C);

        // X = W S (lane (vcol, g4): rows 4g4..4g4+3) and Y^T = S^T Qt^T (lane
        // (token, g4): value columns 4g4..4g4+3 of the tile), from the same
        // operand registers with the roles of A and B swapped.  S enters as
        // bf16 B operands: contraction slot 8*g4 + e maps to state row
        // 32kt + 4g4 + e (e < 4) and 32kt + 16 + 4g4 + (e - 4) (e >= 4), which
        // is exactly what this lane's accumulators of tiles 2kt, 2kt+1 hold.
        f32x4_t X[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4_t Y[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const int lo = tok_off(l16, 32 * kt + 4 * g4), hi = tok_off(l16, 32 * kt + 16 + 4 * g4);
            const bf16x8_t wa = cat8(lds_load<u32x2_t>(&sh.w_row[s2][l16][lo]),
                                     lds_load<u32x2_t>(&sh.w_row[s2][l16][hi]));
            const bf16x8_t qa = tok_operand32(sh.qt_col[s5], kt, l16, g4);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const bf16x8_t sb = cat8(pack_bf16x4(S[2 * kt][nt]), pack_bf16x4(S[2 * kt + 1][nt]));
                X[nt] = mfma32(wa, sb, X[nt]);
                Y[nt] = mfma32(sb, qa, Y[nt]);
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
        const u32x2_t pa = lds_load<u32x2_t>(&sh.pmat[s4][l16][chunk16(l16, g4)]);

        // O^T = Y^T + U^T P^T; lane (token l16, g4) then holds 4 consecutive
        // output values of its token and stores them directly
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
            const f32x4_t gc = lds_load<f32x4_t>(&sh.gam_c[s5][16 * mt + 4 * g4]);
            const u32x2_t ka = lds_load<u32x2_t>(&sh.kb_col[s5][16 * mt + l16][chunk16(l16, g4)]);
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
    const int nc = static_cast<int>(nchunks);
    // even, so that the gate waves' two-set loop needs no exit in between
    const int n_iter = nc > 0 ? (nc + kStages + 1) & ~1 : 0;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t tok_stride = p.H * D;
    const int64_t first = (row * p.T + t_begin) * p.H + h;  // token-head row of t_begin

    if (wave < 4) {
        StateWave<INIT, FINAL> sw{p, sh, t_begin, t_end, chain, wave, lane, l16, g4,
                                  p.out + first * D + 32 * wave + 4 * g4, tok_stride, {}};
        __builtin_amdgcn_s_setprio(3);
        sw.load_state();
        for (int it = 0; it < n_iter; ++it) {
            if (it >= kStages && it - kStages < nc)
                sw.chunk(it - kStages);
            lds_barrier();
        }
        sw.store_state();
        return;
    }

    if (wave >= 12) {
        const int pw = wave - 12;
        const SolveWave sv{sh, pw, l16, g4};
        __builtin_amdgcn_s_setprio(3);
        for (int it = 0; it < n_iter; ++it) {
            if (pw < 2) {
                if (it >= 1 && it - 1 < nc) {
                    if (pw == 0)
                        sv.a_stage(it - 1);
                    else
                        sv.p_stage(it - 1);
                }
            } else if (it >= 2 && it - 2 < nc)
                sv.solve_stage(it - 2);
            if (it >= 3 && it - 3 < nc)
                sv.wy_stage(it - 3);
            lds_barrier();
        }
        return;
    }

    // gate waves
    const int gc16 = wave - 4;
    const int64_t wave_off = (first * D + 16 * gc16) * 2;  // bytes
    const int64_t tok_bytes = tok_stride * 2;
    GateWave gw{p, sh, t_begin, t_end, gc16, lane, l16, g4,
                reinterpret_cast<const char *>(p.q) + wave_off,
                reinterpret_cast<const char *>(p.k) + wave_off,
                reinterpret_cast<const char *>(p.g) + wave_off,
                reinterpret_cast<const char *>(p.v) + wave_off,
                reinterpret_cast<const char *>(p.beta + first),
                C * tok_bytes, C * p.H * 2,
                l16 * tok_bytes + 8 * g4, 8 * g4, lane * p.H * 2};
    const float head_mult = p.A_log ? expf(p.A_log[h]) : 1.0f;
    gw.head_neg = -head_mult * kLog2eF;
    gw.bias_neg = p.dt_bias ? gw.head_neg * p.dt_bias[h * D + 16 * gc16 + l16] : 0.f;
    {
        uint16_t idb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) idb[e] = (4 * g4 + e == l16) ? 0x3F80 : 0;
        gw.ident = u32x2_t{uint32_t(idb[0]) | (uint32_t(idb[1]) << 16),
                           uint32_t(idb[2]) | (uint32_t(idb[3]) << 16)};
    }
    gw.grp_hi = g4 >= 2 ? 1.0f : 0.0f;
    gw.grp_odd = (g4 & 1) ? 1.0f : 0.0f;
    if (n_iter == 0)
        return;

    // Two register sets alternate: iteration `it` uses the set holding chunk
    // it (loaded two iterations earlier), runs the gate stage on it and
    // reloads the set with chunk it + 2.  Past the last chunk the stage runs
    // on a repeat of it and fills only ring slots that no later stage reads.
    // The state and solve waves (priority 3) sit on the critical path; the
    // gate waves fill the issue slots they leave.
    __builtin_amdgcn_s_setprio(1);
    RawRegs ra{}, rb{};
    gw.issue(ra, 0);
    asm volatile("" ::: "memory");  // keep the two sets' loads in order
    gw.issue(rb, nc > 1 ? 1 : 0);
    for (int it = 0; it < n_iter; it += 2) {
        gw.gate_stage(it, ra);
        gw.issue(ra, it + 2 < nc ? it + 2 : nc - 1);
        lds_barrier();
        gw.gate_stage(it + 1, rb);
        gw.issue(rb, it + 3 < nc ? it + 3 : nc - 1);
        lds_barrier();
    }
    // no load may still be writing registers when the wave ends
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
