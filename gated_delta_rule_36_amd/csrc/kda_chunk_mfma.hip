// Chunked KDA forward kernels for gfx950: bf16 MFMA for every contraction,
// fp32 state held in accumulator registers; the pipelined kernel runs one
// workgroup of 16 waves per (sequence, head) chain.
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
//   waves 4-11   gate waves.  Loads: waves 4-7 each move half of q or k (8
//                token rows) of each chunk straight into LDS with direct
//                global-to-LDS loads two chunks ahead, whole 128-byte lines
//                per request, into a staging ring (g and v are loaded the
//                same way by wave 13, v into its ring for the WY stage; the
//                loads sit on the waves that finish their stage early, so
//                no wave at the end of an iteration waits for memory).
//                Compute: wave 4 + c
//                owns channels 16c..16c+15: it reads its q, k, g channel-major
//                through transposing LDS reads, computes the gate, the
//                cumulative decay products and the decayed operands, and
//                stores them channel-major.
//   waves 12-15  solve waves.  Wave 12 loads beta two chunks ahead and forms
//                A, wave 13 P (from the channel-major tiles, read as
//                token-major operands through transposing LDS reads), waves
//                14 and 15 solve columns 0..7 and 8..15 of T; wave 12 + p then
//                runs the WY stage (W and U~) for channels / value columns
//                32p..32p+31.
// The state and solve waves run at raised issue priority: they carry the
// serial dependency chains of an iteration, and the gate waves (ample
// independent work) fill the issue slots they leave.
// Iteration `it` runs the gate stage of chunk it, A and P of chunk it-1, the
// solve of chunk it-2, WY of chunk it-3 and the state update of chunk it-4;
// one workgroup barrier per iteration orders every hand-off through LDS.
//
// The same stage code also runs unpipelined, for a single chunk per chain
// (chunk_single_kernel, at the end of this file): the stage structs take the
// LDS layout as a template parameter.
#include <hip/hip_runtime.h>

#include <cstddef>

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
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

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
//  * 16 x 16 fp32 matrices use a row pitch of 20 floats;
//  * W rows are padded to 272 bytes instead (no swizzle), with the channels
//    of each 32-channel block kt stored in the order the state stage reads
//    them: 16-byte chunk 4 kt + g holds channels 32kt + 4g .. 32kt + 4g + 3
//    and 32kt + 16 + 4g .. 32kt + 16 + 4g + 3.
constexpr int AP = C + 4;
constexpr int kWPitch = D + 8;  // bf16 elements per W row

__device__ __forceinline__ int tok_off(int r, int e) { return 8 * ((e >> 3) ^ (r & 15)) + (e & 7); }
__device__ __forceinline__ int chunk16(int r, int g) { return 4 * (g ^ ((r >> 2) & 3)); }
__device__ __forceinline__ int chunk32(int r, int g) { return 4 * (g ^ ((r >> 1) & 3)); }

// Hot-loop LDS accesses go through 32-bit LDS byte addresses: a per-lane
// base computed once, plus the ring slot's offset (one add per chunk), plus
// a constant that the compiler folds into the instruction's offset field.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u8 *)p));
}
// A per-chunk base address (lane base + ring slot) kept in one register:
// without the empty asm the compiler re-associates base + slot + constant
// and keeps one hoisted base per constant, paying an add per access.
__device__ __forceinline__ uint32_t slot_base(uint32_t a)
{
    asm("" : "+v"(a));
    return a;
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
// Byte offset, within a channel-major bf16 tile, of the address lane
// (l16, g4) passes to the transposing read that yields the token-major
// operand of channels c0 .. c0 + 15 (c0 a multiple of 16; add c0 * 2 C).
__device__ __forceinline__ uint32_t tok_lane(int l16, int g4)
{
    return 2 * ((4 * g4 + (l16 >> 2)) * C + 4 * ((l16 & 3) ^ g4));
}
// Byte offset of lane (l16, g4)'s four elements in row l16 of a 16-wide
// bf16 tile (chunk16 swizzle); row 16 m + l16 adds 512 m.
__device__ __forceinline__ uint32_t row16_lane(int l16, int g4)
{
    return 2 * (l16 * C + chunk16(l16, g4));
}
// The same for 16-wide fp32 rows (chunk32 swizzle).
__device__ __forceinline__ uint32_t row32_lane(int l16, int g4)
{
    return 4 * (l16 * C + chunk32(l16, g4));
}

// Ring buffers between the stages; a tile written for chunk x lives in slot
// x mod (its ring size), which is sized to outlive its last reader.
struct __align__(16) SharedPipe {
    uint16_t kt_col[4][D][C];  // Kt, channel-major; read by A and WY
    uint16_t kh_col[2][D][C];  // Kh, channel-major; read by A and P
    uint16_t qt_col[5][D][C];  // Qt (scale folded in), channel-major; read by P and the state stage
    uint16_t v_row[6][C][D];   // V as loaded (DMA), token-major; read by WY
    uint16_t kb_col[5][D][C];  // Kbar, channel-major; read by the state stage
    float gam_c[5][D];         // Gamma_C per channel
    float beta[3][C];          // sigmoid(beta logits), 0 on padding rows
    float amat[2][C][AP];      // -A = -diag(beta) Kt Kh^T, strictly lower
    uint16_t pmat[4][C][C];    // P (bf16), lower
    uint16_t tb_hi[2][C][C];   // T diag(beta) = hi + lo, two bf16 parts
    uint16_t tb_lo[2][C][C];
    uint16_t w_row[2][C][kWPitch];  // -W, token-major, padded rows
    float ut[2][D][C];         // U~, column-major
    uint16_t stage[3][3][C][D];  // q, k, g as loaded (DMA), token-major; read by the gate stage
};

// The same tiles with one slot each, for a single chunk per workgroup (the
// single-chunk kernel below): W and U~ are written only after the gate stage
// has read the staging tiles, so they share that space.
struct __align__(16) SharedSingle {
    uint16_t kt_col[1][D][C];
    uint16_t kh_col[1][D][C];
    uint16_t qt_col[1][D][C];
    uint16_t v_row[1][C][D];
    uint16_t kb_col[1][D][C];
    float gam_c[1][D];
    float beta[1][C];
    float amat[1][C][AP];
    uint16_t pmat[1][C][C];
    uint16_t tb_hi[1][C][C];
    uint16_t tb_lo[1][C][C];
    union {
        uint16_t stage[1][3][C][D];
        struct {
            uint16_t w_row[1][C][kWPitch];
            float ut[1][D][C];
        } wu;
    };
};

// Byte offsets of the tiles within a layout's shared block.
struct PipeLayout {
    static constexpr uint32_t kOffKt = offsetof(SharedPipe, kt_col), kOffKh = offsetof(SharedPipe, kh_col);
    static constexpr uint32_t kOffQt = offsetof(SharedPipe, qt_col), kOffV = offsetof(SharedPipe, v_row);
    static constexpr uint32_t kOffKb = offsetof(SharedPipe, kb_col), kOffGam = offsetof(SharedPipe, gam_c);
    static constexpr uint32_t kOffBeta = offsetof(SharedPipe, beta), kOffA = offsetof(SharedPipe, amat);
    static constexpr uint32_t kOffP = offsetof(SharedPipe, pmat), kOffThi = offsetof(SharedPipe, tb_hi);
    static constexpr uint32_t kOffTlo = offsetof(SharedPipe, tb_lo), kOffW = offsetof(SharedPipe, w_row);
    static constexpr uint32_t kOffU = offsetof(SharedPipe, ut), kOffStage = offsetof(SharedPipe, stage);
};
struct SingleLayout {
    static constexpr uint32_t kOffKt = offsetof(SharedSingle, kt_col), kOffKh = offsetof(SharedSingle, kh_col);
    static constexpr uint32_t kOffQt = offsetof(SharedSingle, qt_col), kOffV = offsetof(SharedSingle, v_row);
    static constexpr uint32_t kOffKb = offsetof(SharedSingle, kb_col), kOffGam = offsetof(SharedSingle, gam_c);
    static constexpr uint32_t kOffBeta = offsetof(SharedSingle, beta), kOffA = offsetof(SharedSingle, amat);
    static constexpr uint32_t kOffP = offsetof(SharedSingle, pmat), kOffThi = offsetof(SharedSingle, tb_hi);
    static constexpr uint32_t kOffTlo = offsetof(SharedSingle, tb_lo), kOffW = offsetof(SharedSingle, wu.w_row);
    static constexpr uint32_t kOffU = offsetof(SharedSingle, wu.ut), kOffStage = offsetof(SharedSingle, stage);
};
// The stage structs below take the layout as a template parameter and see its
// offsets under these names.
#define KDA_LAYOUT_OFFSETS(L)                                                                     \
    static constexpr uint32_t kOffKt = L::kOffKt, kOffKh = L::kOffKh, kOffQt = L::kOffQt;         \
    static constexpr uint32_t kOffV = L::kOffV, kOffKb = L::kOffKb, kOffGam = L::kOffGam;         \
    static constexpr uint32_t kOffBeta = L::kOffBeta, kOffA = L::kOffA, kOffP = L::kOffP;         \
    static constexpr uint32_t kOffThi = L::kOffThi, kOffTlo = L::kOffTlo, kOffW = L::kOffW;       \
    static constexpr uint32_t kOffU = L::kOffU, kOffStage = L::kOffStage;
// The pipelined kernel's offsets, for its own address set-up.
constexpr uint32_t kOffKt = PipeLayout::kOffKt, kOffKh = PipeLayout::kOffKh, kOffQt = PipeLayout::kOffQt;
constexpr uint32_t kOffV = PipeLayout::kOffV, kOffKb = PipeLayout::kOffKb, kOffGam = PipeLayout::kOffGam;
constexpr uint32_t kOffBeta = PipeLayout::kOffBeta, kOffA = PipeLayout::kOffA, kOffP = PipeLayout::kOffP;
constexpr uint32_t kOffThi = PipeLayout::kOffThi, kOffTlo = PipeLayout::kOffTlo, kOffW = PipeLayout::kOffW;
constexpr uint32_t kOffU = PipeLayout::kOffU, kOffStage = PipeLayout::kOffStage;
constexpr uint32_t kTile = D * C * 2;          // bf16 [D][C] or [C][D] tile
constexpr uint32_t kTileW = C * kWPitch * 2;   // W tile
constexpr uint32_t kTileU = D * C * 4;         // U~ tile (fp32)
constexpr uint32_t kTileCC = C * C * 2;        // 16 x 16 bf16 (P, T parts)
constexpr uint32_t kTileA = C * AP * 4;        // -A (fp32)
constexpr uint32_t kTileGam = D * 4, kTileBeta = C * 4;
static_assert(kTileGam * 8 == kTile, "the Gamma_C ring offset is the tile ring offset / 8");

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ u32x2_t pack_bf16x4(f32x4_t x)
{
    return u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
}
__device__ __forceinline__ f32x4_t bf16x4_to_f32(u32x2_t t)
{
    const uint32_t a = t[0], b = t[1];
    return f32x4_t{__uint_as_float(a << 16), __uint_as_float(a & 0xffff0000u), __uint_as_float(b << 16),
                   __uint_as_float(b & 0xffff0000u)};
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

// Transposing LDS read (ds_read_b64_tr_b16) at LDS byte address a.  Within
// each 16-lane row, lane L supplies the four bf16 at its address, X[L][0..3],
// and lane i receives X[4r + i/4][i%4] for r = 0..3.
//  * On a channel-major tile, with lane L of row g4 pointing at tokens
//    4(L%4)..4(L%4)+3 of channel c0 + 4 g4 + L/4 (address tok_lane + 2 C c0),
//    lane (token i, g4) receives channels c0 + 4 g4 .. c0 + 4 g4 + 3 of token
//    i: the token-major operand of an MFMA that contracts over channels.
//  * On a token-major tile, with lane L of row g4 pointing at channels
//    c0 + 4(L%4) .. c0 + 4(L%4) + 3 of token 4 g4 + L/4, lane (l16, g4)
//    receives tokens 4 g4 .. 4 g4 + 3 of channel c0 + l16: the channel-major
//    operand of an MFMA that contracts over tokens.
__device__ __forceinline__ u32x2_t lds_tr(uint32_t a)
{
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                           (__attribute__((address_space(3))) s16x4_t *)(uintptr_t)a));
}
// Eight channels per lane for a 16x16x32 operand over channels c0..c0+31 of
// a channel-major tile (a = tile + tok_lane + 2 C c0): contraction slot
// 8 g4 + e is channel c0 + 4 g4 + e (e < 4) and c0 + 16 + 4 g4 + (e - 4).
__device__ __forceinline__ bf16x8_t lds_tr32(uint32_t a)
{
    return cat8(lds_tr(a), lds_tr(a + 32 * C));
}
// Lane part of the transposing read of channels c0 + 4(L%4).. of token
// 4 g4 + L/4 in a token-major [C][D] tile (tok_off swizzle).
__device__ __forceinline__ uint32_t chan_lane(int c0, int l16, int g4)
{
    const int r = 4 * g4 + (l16 >> 2);
    return 2 * (r * D + tok_off(r, c0 + 4 * (l16 & 3)));
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

// tanh(y) ~ y P(y^2) / Q(y^2) on |y| <= 9 (beyond, tanh = 1 to 2^-23), P and Q
// of degree 4 in y^2 with P(0) = Q(0) = 1: a rational fit of tanh by weighted
// least squares on the relative error (gated_delta_rule_36_amd/fit_tanh.py);
// in fp32, Horner order, the error is about 3e-7 on the whole line.  Used
// by the tanh form of the logistic function, sigma(x) = 1/2 + tanh(x/2)/2,
// which needs no exponential (the pages' sigmoid_tanh_approx; gfx950 has no
// tanh instruction).
constexpr float kTanhClamp = 9.0f;
constexpr float kTanhP1 = 0.13381032645702362f, kTanhP2 = 0.0034955963492393494f,
                kTanhP3 = 2.0609206330846064e-05f, kTanhP4 = 1.3354815919797147e-08f;
constexpr float kTanhQ1 = 0.4671434760093689f, kTanhQ2 = 0.02587701380252838f,
                kTanhQ3 = 0.0003285647835582495f, kTanhQ4 = 7.776625352562405e-07f;

// Plain load (the beta logits): the compiler tracks it and waits (s_waitcnt
// vmcnt) right before the first use of the register.
__device__ __forceinline__ uint32_t gload_u16(const char *p)
{
    return *reinterpret_cast<const uint16_t *>(p);
}

// Direct global-to-LDS load (global_load_lds_dwordx4): lane i's 16 bytes,
// read at base + voff, land at LDS byte address dst + 16 i (dst is
// wave-uniform and goes in M0).  Written as asm so that the compiler does not
// make later, unrelated LDS accesses wait for it; the issuing wave waits
// (vmcnt) before the barrier that hands the data to the other waves.  NT:
// the non-temporal hint (nt), for inputs read for the last time (a whole
// chain, or the segmented form's output pass); the map passes of the
// segmented form leave it off, since their inputs are read again by the
// output pass and may still be in the last-level cache then.
template <bool NT>
__device__ __forceinline__ void dma16(const char *base, uint32_t voff, uint32_t dst)
{
    if constexpr (NT)
        asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "{m0}"(dst) : "memory");
    else
        asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(dst) : "memory");
}

// Direct loads of 4 NJ token rows of one tensor per chunk into an LDS ring,
// 4 rows (1 KB) per load: lane i takes 16-byte chunk (i % 16) ^ r of row
// r = row0 + 4 j + i / 16, which lands at position i % 16 of the row: the
// swizzled token-major layout.  Rows past the sequence end take token 0's
// data.  The cursor (chunk, source, ring slot) advances one chunk per
// iteration up to the last chunk, so the loop needs no per-chunk multiplies
// or remainders.  Bases and strides are wave-uniform (scalar registers).
// NT: the non-temporal hint on the loads (dma16).
template <int NJ, bool NT = true>
struct Loader {
    const char *src;              // the tensor at chunk x
    int64_t chunk_bytes;          // between consecutive chunks: C * H * 256
    uint32_t full[NJ], tail[NJ];  // lane offsets; rows past a partial last chunk on token 0
    uint32_t dst, dst0, dst_end;  // LDS: chunk x's slot (row row0), the ring's first slot, its end
    uint32_t slot;                // bytes between ring slots
    int x, n_full;                // chunk being loaded; full chunks of the range

    __device__ __forceinline__ void init(const uint16_t *tensor, int64_t tok_bytes, int row0, int lane, int tail_len,
                         int nfull, uint32_t ring0, uint32_t slot_bytes, int ring)
    {
        src = reinterpret_cast<const char *>(tensor);
        chunk_bytes = C * tok_bytes;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int r = row0 + 4 * j + (lane >> 4), c = (lane & 15) ^ r;
            full[j] = static_cast<uint32_t>(r * tok_bytes + 16 * c);
            tail[j] = static_cast<uint32_t>((r < tail_len ? r : 0) * tok_bytes + 16 * c);
        }
        dst0 = ring0;
        dst = ring0 + 256 * row0;
        dst_end = ring0 + ring * slot_bytes;
        slot = slot_bytes;
        x = 0;
        n_full = nfull;
    }
    // Start loading chunk x (NJ loads; every lane loads something valid).
    __device__ __forceinline__ void issue() const
    {
        const bool f = x < n_full;
#pragma unroll
        for (int j = 0; j < NJ; ++j) dma16<NT>(src, f ? full[j] : tail[j], dst + 1024 * j);
    }
    __device__ __forceinline__ void advance(int nc)
    {
        if (x < nc - 1) {
            ++x;
            src += chunk_bytes;
            dst = dst + slot >= dst_end ? dst - (dst_end - dst0) + slot : dst + slot;
        }
    }
};

template <class L>
struct GateWave {
    KDA_LAYOUT_OFFSETS(L)
    const FwdParams &p;
    int gc16;  // 0..7: channels 16 gc16 .. 16 gc16 + 15, wave-uniform
    int lane, l16, g4;
    int n_full, tail;  // full chunks of the sequence; length of a partial last chunk (0: none)
    // LDS addresses (ring slot 0, without the ring's offset): this lane's
    // transposing read of channels 16 gc16 + 4 (l16 % 4) .. of token
    // 4 g4 + l16 / 4 in the stage tiles; its stores into the channel-major
    // tiles (channel 16 gc16 + l16, tokens 4 g4 ..) and of Gamma_C.
    uint32_t rd_stage, st_col, st_gam;
    float head_neg;  // -exp(A_log[h]) * log2(e)
    float bias_neg;  // head_neg * dt_bias[h][16 gc16 + l16]
    float grp_hi;   // (g4 >= 2)
    float grp_odd;  // (g4 odd)
    // tanh form: y = x / 2 = head_y g + bias_y; a = gs_half (1 + tanh y)
    float head_y, bias_y, gs_half;

    __device__ __forceinline__ int chunk_len(int x) const { return x < n_full ? C : tail; }

    // Gate, decay products and decayed operands of chunk x for this wave's
    // 16 channels.  FULL: all 16 rows of the chunk lie in the sequence.
    // o3, o5: offsets of chunk x's stage slot and of its Qt / Kbar ring slot
    // (x mod 3 and x mod 5 slots, kept as running offsets by the caller).
    // QT: form Qt (only the output needs it; without it q is never read).
    template <int SIG, bool QT = true>
    __device__ __forceinline__ void gate_stage(int x, uint32_t o3, uint32_t o5) const
    {
        if (x < n_full)
            gate_rows<true, SIG, QT>(x, o3, o5);
        else
            gate_rows<false, SIG, QT>(x, o3, o5);
    }
    template <bool FULL, int SIG, bool QT>
    __device__ __forceinline__ void gate_rows(int x, uint32_t o3, uint32_t o5) const
    {
        const int len = FULL ? C : tail;
        const uint32_t s2 = x & 1, s4 = x & 3;
        // channel-major: the transposing read of the token-major stage tiles
        // gives lane (l16, g4) tokens 4 g4 .. 4 g4 + 3 of channel 16 gc16 + l16
        const uint32_t ar = slot_base(rd_stage + o3);
        const f32x4_t cq = QT ? bf16x4_to_f32(lds_tr(ar)) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        const f32x4_t ck = bf16x4_to_f32(lds_tr(ar + kTile));
        const f32x4_t cg = bf16x4_to_f32(lds_tr(ar + 2 * kTile));

        // Rows past the sequence end hold a copy of the chunk's first token.
        // Only their decay needs masking (alpha = 1): their beta is 0 (set by
        // the solve wave that loads beta), which
        // zeroes their rows and columns of T diag(beta) and so of W, U~ and
        // U; their A, P and output entries are never used.
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float a;
            if constexpr (SIG == kSigmoidTanh) {
                const float y = __builtin_amdgcn_fmed3f(fmaf(cg[i], head_y, bias_y), -kTanhClamp, kTanhClamp);
                const float u = y * y;
                const float pn = fmaf(fmaf(fmaf(fmaf(kTanhP4, u, kTanhP3), u, kTanhP2), u, kTanhP1), u, 1.0f);
                const float qd = fmaf(fmaf(fmaf(fmaf(kTanhQ4, u, kTanhQ3), u, kTanhQ2), u, kTanhQ1), u, 1.0f);
                a = exp2_f32(fmaf(gs_half, y * pn * __builtin_amdgcn_rcpf(qd), gs_half));
            } else {
                const float e = exp2_f32(fmaf(cg[i], head_neg, bias_neg));
                const float s = __builtin_amdgcn_rcpf(1.0f + e);
                a = exp2_f32(p.gate_scale * s);
            }
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
        const uint32_t a5 = slot_base(st_col + o5);  // Qt and Kbar share the ring index
        lds_st(slot_base(st_col + s4 * kTile) + kOffKt, pack_bf16x4(kt));
        lds_st(slot_base(st_col + s2 * kTile) + kOffKh, pack_bf16x4(kh));
        if constexpr (QT)
            lds_st(a5 + kOffQt, pack_bf16x4(qt));
        lds_st(a5 + kOffKb, pack_bf16x4(kb));
        if (g4 == 0)
            lds_st(st_gam + (o5 >> 3), gc);
    }
};

// ---------------------------------------------------------------------------
// solve waves
// ---------------------------------------------------------------------------

template <class L>
struct SolveWave {
    KDA_LAYOUT_OFFSETS(L)
    int pw;  // 0..3, wave-uniform
    int l16, g4;
    // LDS addresses (ring slot 0, without the ring's offset) of this lane's
    // accesses: tok = sh + tok_lane; r16 = sh + row16_lane; amat_st: -A
    // entries (4 g4 + e, l16); amat_ld: row l16 of -A; bt: beta of tokens
    // 4 g4 .. 4 g4 + 3 (wave 0) or of the column pair j0, j0 + 1 (waves 2, 3);
    // tb_st: T diag(beta) entries (l16, j0 .. j0 + 1); wy_k: Kt channel
    // 32 pw + l16; wy_w: W row l16, chunk 4 pw + g4; wy_v0/1: V operands
    // of channels 32 pw and 32 pw + 16; wy_u: U~ column 32 pw + l16.
    uint32_t tok, r16, amat_st, amat_ld, bt, tb_st, wy_k, wy_w, wy_v0, wy_v1, wy_u;
    // Beta (wave 0): logits of token `lane` (lane < 16) of each chunk, loaded
    // two iterations ahead of their use; st_beta = the lane's LDS entry.
    int lane, n_full, tail;
    const char *base_beta;     // beta of token t_begin
    int64_t beta_chunk_bytes;  // C * H * 2
    uint32_t beta_lane;        // lane * H * 2 (lane < 16), else 0
    uint32_t st_beta;
    uint32_t bq;  // beta of tokens 4 g4 .. 4 g4 + 3 (the Neumann inverse)

    // The beta logits of chunk x (rows past the end read token 0).
    __device__ __forceinline__ uint32_t load_beta(int x) const
    {
        uint32_t off = beta_lane;
        if (x >= n_full)
            off = lane < tail ? beta_lane : 0u;
        return gload_u16(base_beta + int64_t(x) * beta_chunk_bytes + off);
    }
    // sigmoid(beta) of chunk x into its ring slot, 0 on rows past the end.
    __device__ __forceinline__ void put_beta(int x, uint32_t logit) const
    {
        const int len = x < n_full ? C : tail;
        const float b = sigmoid_f32(bf16_to_f32(static_cast<uint16_t>(logit)));
        if (lane < C)
            lds_st(st_beta + static_cast<uint32_t>(x % 3) * kTileBeta, lane < len ? b : 0.f);
    }

    // -A of chunk x: lane (j = l16, g4) gets (Kt Kh^T)[4 g4 + e][j].
    __device__ __forceinline__ void a_stage(int x) const
    {
        const uint32_t s2 = x & 1, s3 = x % 3, s4 = x & 3;
        const uint32_t ak = slot_base(tok + s4 * kTile + kOffKt), ah = slot_base(tok + s2 * kTile + kOffKh);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
            acc = mfma32(lds_tr32(ak + 64 * C * kt), lds_tr32(ah + 64 * C * kt), acc);
        const f32x4_t b = lds_ld<f32x4_t>(bt + s3 * kTileBeta);
        const uint32_t am = slot_base(amat_st + s2 * kTileA);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * g4 + e;
            lds_st(am + 4 * AP * e, l16 < i ? -b[e] * acc[e] : 0.f);  // stored negated
        }
    }

    // P of chunk x, as P^T = Kh Qt^T: lane (i = l16, g4) gets
    // P[i][4 g4 .. 4 g4 + 3], the layout the state stage reads.
    __device__ __forceinline__ void p_stage(int x) const
    {
        const uint32_t s2 = x & 1, s4 = x & 3, s5 = x % 5;
        const uint32_t ah = slot_base(tok + s2 * kTile + kOffKh), aq = slot_base(tok + s5 * kTile + kOffQt);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
            acc = mfma32(lds_tr32(ah + 64 * C * kt), lds_tr32(aq + 64 * C * kt), acc);
        f32x4_t pm;
#pragma unroll
        for (int e = 0; e < 4; ++e) pm[e] = (4 * g4 + e <= l16) ? acc[e] : 0.f;
        lds_st(r16 + s4 * kTileCC + kOffP, pack_bf16x4(pm));
    }

    // Columns 8 (pw - 2) .. 8 (pw - 2) + 7 of T for chunk x (solve waves 2
    // and 3), stored as T diag(beta).
    __device__ __forceinline__ void solve_stage(int x) const
    {
        const uint32_t s2 = x & 1, s3 = x % 3;
        // T[:, j] for j = j0, j0 + 1 with j0 = 8 (pw - 2) + 2 g4; lane
        // (g4, l16 = row i).  Right-looking forward substitution on
        // v = e_j - A t: lane i starts from v_i = (i == j); step m takes
        // t_m = v_m (final once the rows above m are done; zero for m < j)
        // from lane m of its 16-lane row and subtracts A[i][m] t_m from every
        // v_i.  A[i][m] = 0 for m >= i, so a row stops changing once it is
        // final.  The two columns run as independent chains.
        const int j0 = 8 * (pw - 2) + 2 * g4, i = l16;
        const uint32_t ar = slot_base(amat_ld + s2 * kTileA);
        float nrow[C];  // -A[i][:], zero from column i on
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4_t v = lds_ld<f32x4_t>(ar + 16 * q4);
            nrow[4 * q4 + 0] = v[0];
            nrow[4 * q4 + 1] = v[1];
            nrow[4 * q4 + 2] = v[2];
            nrow[4 * q4 + 3] = v[3];
        }
        float v0 = i == j0 ? 1.0f : 0.0f, v1 = i == j0 + 1 ? 1.0f : 0.0f;
        solve_steps(nrow, v0, v1);
        const f32x2_t b2 = lds_ld<f32x2_t>(bt + s3 * kTileBeta);
        const float tb0 = v0 * b2[0];
        const float tb1 = v1 * b2[1];
        const __bf16 hi0 = static_cast<__bf16>(tb0), hi1 = static_cast<__bf16>(tb1);
        const __bf16 lo0 = static_cast<__bf16>(tb0 - static_cast<float>(hi0));
        const __bf16 lo1 = static_cast<__bf16>(tb1 - static_cast<float>(hi1));
        const uint32_t at = slot_base(tb_st + s2 * kTileCC);
        lds_st(at + kOffThi, pack_bf16x2(static_cast<float>(hi0), static_cast<float>(hi1)));
        lds_st(at + kOffTlo, pack_bf16x2(static_cast<float>(lo0), static_cast<float>(lo1)));
    }

    // T of chunk x for the whole chunk in one wave (wave 14), as the product
    // (I + L)(I + L^2)(I + L^4)(I + L^8) with L = -A: A is strictly lower, so
    // L^16 = 0 and the product is the whole Neumann series -- the inverse the
    // chunk-size page describes under "Efficient 16x16 Matrix Inversion",
    // with fp16 MFMA operands and fp32 accumulation as there.  An MFMA result
    // (lane (j, g4) holding X[4 g4 + r][j]) is the B operand of X and the A
    // operand of X^T as it stands, so each power is also formed transposed
    // and no value moves between lanes; the last product gives T^T, i.e. row
    // l16 of T in lane (l16, g4), the layout T diag(beta) is stored in.
    __device__ __forceinline__ void solve_neumann(int x) const
    {
        const uint32_t s2 = x & 1, s3 = x % 3;
        f32x4_t eye;  // the identity in either layout: (l16 == 4 g4 + r)
#pragma unroll
        for (int r = 0; r < 4; ++r) eye[r] = (l16 == 4 * g4 + r) ? 1.0f : 0.0f;
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        auto h = [](f32x4_t v) { return __builtin_convertvector(v, f16x4_t); };
        auto mm = [&](f16x4_t a, f16x4_t b) { return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, zero, 0, 0, 0); };
        // L = -A as stored: row l16 (A operand), column l16 (B operand)
        const f32x4_t la = lds_ld<f32x4_t>(slot_base(amat_ld + s2 * kTileA) + 16 * g4);
        const uint32_t ac = slot_base(amat_st + s2 * kTileA);
        f32x4_t lb;
#pragma unroll
        for (int r = 0; r < 4; ++r) lb[r] = lds_ld<float>(ac + 4 * AP * r);
        const f16x4_t LA = h(la), LB = h(lb);
        const f32x4_t L2 = mm(LA, LB), L2T = mm(LB, LA);
        const f16x4_t L2h = h(L2), L2Th = h(L2T);
        const f32x4_t L4 = mm(L2Th, L2h), L4T = mm(L2h, L2Th);
        const f32x4_t L8 = mm(h(L4T), h(L4));
        const f32x4_t P = mm(h(L4T + eye), h(L8 + eye));  // (I + L^4)(I + L^8)
        const f32x4_t Q = mm(h(L2T + eye), h(P));         // (I + L^2) P
        const f32x4_t TT = mm(h(Q), h(la + eye));         // ((I + L) Q)^T
        const f32x4_t tb = TT * lds_ld<f32x4_t>(bq + s3 * kTileBeta);  // T diag(beta), row l16
        f32x4_t hi, lo;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            hi[r] = static_cast<float>(static_cast<__bf16>(tb[r]));
            lo[r] = tb[r] - hi[r];
        }
        const uint32_t at = slot_base(r16 + s2 * kTileCC);
        lds_st(at + kOffThi, pack_bf16x4(hi));
        lds_st(at + kOffTlo, pack_bf16x4(lo));
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
    // as the contraction [T_hi | T_lo] against [X; X].  The W tile receives
    // -W, so that the state waves accumulate U = U~ - W S onto U~.
    __device__ __forceinline__ void wy_stage(int x) const
    {
        const uint32_t s2 = x & 1, s4 = x & 3, s6 = x % 6;
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        // lane (l16, g4) holds (T diag(beta))[l16][4*g4 .. 4*g4+3]: the A
        // operand of T diag(beta) V and the B operand of Kt^T (T diag(beta))^T
        const uint32_t at = slot_base(r16 + s2 * kTileCC);
        const bf16x8_t t8 = cat8(lds_ld<u32x2_t>(at + kOffThi), lds_ld<u32x2_t>(at + kOffTlo));
        const uint32_t ak = slot_base(wy_k + s4 * kTile), aw = slot_base(wy_w + s2 * kTileW),
                       au = slot_base(wy_u + s2 * kTileU);
        const uint32_t av[2] = {slot_base(wy_v0 + s6 * kTile), slot_base(wy_v1 + s6 * kTile)};
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const u32x2_t ka = lds_ld<u32x2_t>(ak + 32 * C * t);
            // lane (token l16, g4): W[l16][32pw+16t+4g4+i], stored negated at
            // chunk 4 pw + g4, half t of the padded row
            const f32x4_t w = mfma32(cat8(ka, ka), t8, zero);
            lds_st(aw + 8 * t, pack_bf16x4(-w));
            const u32x2_t vb = lds_tr(av[t]);
            // lane (vcol, g4): U~[4g4+i][vcol]
            const f32x4_t u = mfma32(t8, cat8(vb, vb), zero);
            lds_st(au + 64 * C * t, u);
        }
    }
};

// ---------------------------------------------------------------------------
// state waves
// ---------------------------------------------------------------------------

// Where a state wave's state comes from and goes to (wave-uniform).
enum StateSrc : int { kSrcZero = 0, kSrcIdentity = 1, kSrcFp32 = 2, kSrcBf16 = 3 };
enum ChunkMode : int { kChunkFull = 0, kChunkState = 1, kChunkTransition = 2 };
// Kernel mode of the fused map pass: waves 0-3 carry the end state
// (kChunkState), waves 4-7 the transition matrix (kChunkTransition).
constexpr int kChunkMapBM = 3;
// kDstHiLoT: untransposed ([K][V]: element [k][v] = S[k][v]) as two bf16
// planes, hi = bf16(S) then lo = bf16(S - hi), in one fp32-sized slab.
enum StateDst : int { kDstNone = 0, kDstFp32 = 2, kDstBf16 = 3, kDstHiLoT = 4 };

template <class L>
struct StateWave {
    KDA_LAYOUT_OFFSETS(L)
    const FwdParams &p;
    int w, lane, l16, g4;
    int n_full, tail;          // full chunks of the range; length of a partial last chunk
    char *out_base;            // out at the range's first token, value column 32 w (wave-uniform)
    int64_t out_chunk_bytes;   // between consecutive chunks of out: C * H * 256
    uint32_t out_lane;         // lane offset: token l16, value column 4 g4
    // LDS addresses (ring slot 0) of this lane's reads: Qt operands
    // (tok_lane), W row l16 chunk g4, U~ column 32 w + l16, P row l16,
    // Gamma_C rows 4 g4 .., Kbar channel l16.
    uint32_t rd_q, rd_w, rd_u, rd_p, rd_g, rd_k;
    f32x4_t S[8][2];     // S[16mt + 4g4 + i][32w + 16nt + l16]

    // Element offset, within one [V][K] state slab, of this lane's tile (mt, nt).
    __device__ __forceinline__ int64_t slab_index(int mt, int nt) const
    {
        return int64_t(32 * w + 16 * nt + l16) * D + 16 * mt + 4 * g4;
    }

    // slab: element offset of the [V][K] slab in ptr.
    __device__ __forceinline__ void load_state(int src, const void *ptr, int64_t slab)
    {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int64_t idx = slab + slab_index(mt, nt);
                if (src == kSrcFp32) {
                    S[mt][nt] = *reinterpret_cast<const f32x4_t *>(static_cast<const float *>(ptr) + idx);
                } else if (src == kSrcBf16) {
                    const u32x2_t b = *reinterpret_cast<const u32x2_t *>(static_cast<const uint16_t *>(ptr) + idx);
                    S[mt][nt] = f32x4_t{__uint_as_float(b[0] << 16), __uint_as_float(b[0] & 0xffff0000u),
                                        __uint_as_float(b[1] << 16), __uint_as_float(b[1] & 0xffff0000u)};
                } else {
                    const int v = 32 * w + 16 * nt + l16;  // identity: S[k][v] = (k == v)
                    const float one = src == kSrcIdentity ? 1.0f : 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[mt][nt][i] = (16 * mt + 4 * g4 + i == v) ? one : 0.0f;
                }
            }
    }

    __device__ __forceinline__ void store_state(int dst, void *ptr, int64_t slab) const
    {
        if (dst == kDstNone)
            return;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int64_t idx = slab + slab_index(mt, nt);
                if (dst == kDstFp32) {
                    *reinterpret_cast<f32x4_t *>(static_cast<float *>(ptr) + idx) = S[mt][nt];
                } else if (dst == kDstHiLoT) {
                    uint16_t *const hi = static_cast<uint16_t *>(ptr) + 2 * slab + 32 * w + 16 * nt + l16;
                    uint16_t *const lo = hi + D * D;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x = S[mt][nt][i];
                        const uint16_t h = f32_to_bf16_rne(x);
                        hi[(16 * mt + 4 * g4 + i) * D] = h;
                        lo[(16 * mt + 4 * g4 + i) * D] = f32_to_bf16_rne(x - bf16_to_f32(h));
                    }
                } else {
                    *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(ptr) + idx) =
                        u32x2_t{uint32_t(f32_to_bf16_rne(S[mt][nt][0])) |
                                    (uint32_t(f32_to_bf16_rne(S[mt][nt][1])) << 16),
                                uint32_t(f32_to_bf16_rne(S[mt][nt][2])) |
                                    (uint32_t(f32_to_bf16_rne(S[mt][nt][3])) << 16)};
                }
            }
    }

    // MODE kChunkFull: outputs and state; kChunkState: the state only (no
    // Y, no output); kChunkTransition: the state with v ignored (U = -W S),
    // which carries an identity start to the range's transition matrix.
    template <int MODE>
    __device__ __forceinline__ void chunk(int x, uint32_t o5)
    {
        constexpr bool kOut = MODE == kChunkFull;
        const uint32_t s2 = x & 1, s4 = x & 3;
        const int len = x < n_full ? C : tail;

        // U = U~ - W S (lane (vcol, g4): rows 4g4..4g4+3), accumulated onto
        // U~ from the W tile's -W (U = -W S without v: the transition), and
        // Y^T = S^T Qt^T (lane (token, g4): value columns 4g4..4g4+3 of the
        // tile), from the same operand registers with the roles of A and B
        // swapped.  S enters as bf16 B operands: contraction slot 8*g4 + e
        // maps to state row 32kt + 4g4 + e (e < 4) and 32kt + 16 + 4g4 + (e - 4)
        // (e >= 4), which is exactly what this lane's accumulators of tiles
        // 2kt, 2kt+1 hold and what chunk 4 kt + g4 of a W row holds.
        const uint32_t aw = slot_base(rd_w + s2 * kTileW), aq = slot_base(rd_q + o5);
        f32x4_t X[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4_t Y[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        if constexpr (MODE != kChunkTransition) {
            const uint32_t au = slot_base(rd_u + s2 * kTileU);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) X[nt] = lds_ld<f32x4_t>(au + 64 * C * nt);
        }
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const bf16x8_t wa = __builtin_bit_cast(bf16x8_t, lds_ld<u32x4_t>(aw + 64 * kt));
            const bf16x8_t qa = lds_tr32(aq + 64 * C * kt);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const bf16x8_t sb = cat8(pack_bf16x4(S[2 * kt][nt]), pack_bf16x4(S[2 * kt + 1][nt]));
                X[nt] = mfma32(wa, sb, X[nt]);
                if constexpr (kOut)
                    Y[nt] = mfma32(sb, qa, Y[nt]);
            }
        }

        // U as bf16 operands (lane (vcol, g4): tokens 4g4..4g4+3)
        const u32x2_t ub[2] = {pack_bf16x4(X[0]), pack_bf16x4(X[1])};

        if constexpr (kOut) {
            // O^T = Y^T + U^T P^T; lane (token l16, g4) then holds 4
            // consecutive output values of its token in each tile: value
            // columns 16 nt + 4 g4 .. + 3, one 8-byte store per tile
            const u32x2_t pa = lds_ld<u32x2_t>(slot_base(rd_p + s4 * kTileCC));
            const u32x2_t o0 = pack_bf16x4(mfma16(ub[0], pa, Y[0]));
            const u32x2_t o1 = pack_bf16x4(mfma16(ub[1], pa, Y[1]));
            if (l16 < len) {
                char *const o = out_base + int64_t(x) * out_chunk_bytes + out_lane;
                *reinterpret_cast<u32x2_t *>(o) = o0;
                *reinterpret_cast<u32x2_t *>(o + 32) = o1;
            }
        }

        // S <- diag(Gamma_C) S + Kbar^T U
        const uint32_t ag = slot_base(rd_g + (o5 >> 3)), ak = slot_base(rd_k + o5);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const f32x4_t gc = lds_ld<f32x4_t>(ag + 64 * mt);
            const u32x2_t ka = lds_ld<u32x2_t>(ak + 32 * C * mt);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) S[mt][nt] = mfma16(ka, ub[nt], S[mt][nt] * gc);
        }
    }
};

template <int MODE, class L>
__device__ __forceinline__ void state_loop(StateWave<L> &sw, int n_iter, int nc)
{
    uint32_t o5 = 0;  // chunk x's Qt / Kbar ring slot (x mod 5), as a running offset
    for (int it = 0; it < n_iter; ++it) {
        if (it >= kStages && it - kStages < nc) {
            sw.template chunk<MODE>(it - kStages, o5);
            o5 = o5 == 4 * kTile ? 0 : o5 + kTile;
        }
        lds_barrier();
    }
}

// MODE: the state waves' chunk mode (kChunkFull for whole chains and the
// output pass, kChunkState for the segment end states), or kChunkMapBM for
// the fused map pass of the segmented form: eight state waves, 0-3 for the
// segment's end state from its start (kChunkState) and 4-7 for its
// transition matrix from the identity (kChunkTransition), and four gate
// waves of 32 channels each (8-11); the gate and solve work and the loads
// are shared by both states.
// INV: the inverse (Inverse); SIG: the gate's logistic function (Sigmoid).
template <int MODE, int INV, int SIG = kSigmoidExp>
__global__ __launch_bounds__(kThreads, 1) void chunk_mfma_kernel(FwdParams p)
{
    __shared__ SharedPipe sh;
    // Without outputs (the map passes of the segmented form) q, Qt and P are
    // not needed.
    constexpr bool kFused = MODE == kChunkMapBM;
    constexpr bool kOut = MODE == kChunkFull;
    constexpr int kStateWaves = kFused ? 8 : 4;
    // Block -> chain (and, in the segmented form, segment).  The grid is
    // below 2^31 blocks (checked on the host), so 32-bit arithmetic suffices;
    // readfirstlane keeps these wave-uniform values in scalar registers.
    const int n_seg = static_cast<int>(p.n_seg);
    int chain = blockIdx.x, seg = 0;
    if (p.phase != kPhaseWhole) {
        // chain c's segments on XCD c mod 8 (blocks go to XCD b mod 8), where
        // the combine step reads them
        const int b = static_cast<int>(blockIdx.x);
        const int whole = static_cast<int>(p.num_seqs * p.H / 8) * 8 * n_seg;
        if (b < whole) {
            const int i = b >> 3;
            chain = 8 * (i / n_seg) + (b & 7);
            seg = i % n_seg;
        } else {
            chain = b / n_seg;
            seg = b - chain * n_seg;
        }
    }
    chain = __builtin_amdgcn_readfirstlane(chain);
    seg = __builtin_amdgcn_readfirstlane(seg);
    const int H = static_cast<int>(p.H);
    const int64_t n = chain / H, h = chain - (chain / H) * H;
    int64_t t_begin, t_end, row;
    chain_segment(p, n, &t_begin, &t_end, &row);

    // Where this block's state starts and ends, and its token range (all
    // wave-uniform).
    int src = p.init_state ? (p.init_kind == kStateBf16 ? kSrcBf16 : kSrcFp32) : kSrcZero;
    const void *src_ptr = p.init_state;
    int64_t src_slab = int64_t(chain) * D * D;
    int dst = p.final_state ? (p.final_kind == kStateBf16 ? kDstBf16 : kDstFp32) : kDstNone;
    void *dst_ptr = p.final_state;
    int64_t dst_slab = int64_t(chain) * D * D;
    if (p.phase != kPhaseWhole) {
        const int64_t nc_chain = (t_end - t_begin + C - 1) / C;
        const int segs = static_cast<int>(nc_chain > 0 ? (nc_chain + p.seg_chunks - 1) / p.seg_chunks : 1);
        const int64_t scratch = (int64_t(chain) * n_seg + seg) * D * D;
        if (p.phase == kPhaseMapB || p.phase == kPhaseMapBM) {
            // b_s for segments 0 .. segs - 2: segment 0 from the real start,
            // later ones from zero (and, fused, M_s for 1 .. segs - 2 into
            // seg_m at the same slab index)
            if (seg >= segs - 1)
                return;
            if (seg > 0)
                src = kSrcZero;
            dst = kDstFp32;
            dst_ptr = p.seg_b;
            dst_slab = scratch;
        } else {
            // outputs of every segment from its true start state: the real
            // one for segment 0, seg_b[s - 1] (after the combine step) for
            // the others; the chain's last segment writes the final state.
            // With two or more segments, segment 0 reads the copy of the
            // initial state that the map pass left in its seg_m slab (which
            // holds no matrix): final_state may be the initial_state buffer,
            // and the last segment's workgroup may store it before segment
            // 0's workgroup has started.
            if (seg >= segs)
                return;
            if (seg > 0) {
                src = kSrcFp32;
                src_ptr = p.seg_b;
                src_slab = scratch - D * D;
            } else if (segs > 1 && src != kSrcZero) {
                src = kSrcFp32;
                src_ptr = p.seg_m;
                src_slab = scratch;
            }
            if (seg != segs - 1)
                dst = kDstNone;
        }
        t_begin += int64_t(seg) * p.seg_chunks * C;
        t_end = t_end < t_begin + p.seg_chunks * C ? t_end : t_begin + p.seg_chunks * C;
    }
    const int len_seq = static_cast<int>(t_end - t_begin);
    const int n_full = len_seq / C, tail = len_seq % C;
    const int nc = n_full + (tail > 0);
    // even, so that the gate waves' two-set loop needs no exit in between
    const int n_iter = nc > 0 ? (nc + kStages + 1) & ~1 : 0;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t tok_bytes = p.H * D * 2;                  // between consecutive tokens
    const int64_t first = (row * p.T + t_begin) * p.H + h;  // token-head row of t_begin
    const uint32_t sh0 = lds_addr(&sh);

    if (wave < kStateWaves) {
        const int w = wave & 3;  // value columns 32 w .. 32 w + 31
        StateWave<PipeLayout> sw{p, w, lane, l16, g4, n_full, tail,
                                  reinterpret_cast<char *>(p.out + first * D + 32 * w),
                                  C * tok_bytes,
                                  static_cast<uint32_t>(l16 * tok_bytes + 8 * g4),
                                  sh0 + kOffQt + tok_lane(l16, g4),
                                  sh0 + kOffW + 2 * kWPitch * l16 + 16 * g4,
                                  sh0 + kOffU + 128 * C * w + row32_lane(l16, g4),
                                  sh0 + kOffP + row16_lane(l16, g4),
                                  sh0 + kOffGam + 16 * g4,
                                  sh0 + kOffKb + row16_lane(l16, g4),
                                  {}};
        __builtin_amdgcn_s_setprio(3);
        if constexpr (kFused) {
            if (wave >= 4) {
                // M_s: from the identity, v ignored; segment 0 starts from a
                // known state, so its matrix is not stored
                sw.load_state(kSrcIdentity, nullptr, 0);
                if (n_iter > 0)
                    lds_barrier();  // the gate waves' first loads are in LDS
                state_loop<kChunkTransition, PipeLayout>(sw, n_iter, nc);
                sw.store_state(seg > 0 ? kDstHiLoT : kDstNone, p.seg_m, dst_slab);
                return;
            }
        }
        sw.load_state(src, src_ptr, src_slab);
        // map pass, segment 0: keep a copy of the chain's initial state (fp32)
        // in the segment's seg_m slab for the output pass
        if (p.phase != kPhaseWhole && p.phase != kPhaseOut && seg == 0 && src != kSrcZero)
            sw.store_state(kDstFp32, p.seg_m, dst_slab);
        if (n_iter > 0)
            lds_barrier();  // the gate waves' first loads are in LDS
        state_loop<kFused ? kChunkState : MODE, PipeLayout>(sw, n_iter, nc);
        sw.store_state(dst, dst_ptr, dst_slab);
        return;
    }

    if (wave >= 12) {
        const int pw = wave - 12;
        const int j0 = 8 * (pw - 2) + 2 * g4;  // the solve waves' column pair
        const SolveWave<PipeLayout> sv{pw, l16, g4,
                           sh0 + tok_lane(l16, g4),
                           sh0 + row16_lane(l16, g4),
                           sh0 + kOffA + 4 * (4 * g4 * AP + l16),
                           sh0 + kOffA + 4 * AP * l16,
                           sh0 + kOffBeta + (pw == 0 ? 16 * g4 : 4 * j0),
                           sh0 + 2 * (l16 * C + chunk16(l16, j0 >> 2) + (j0 & 3)),
                           sh0 + kOffKt + 64 * C * pw + row16_lane(l16, g4),
                           sh0 + kOffW + 2 * kWPitch * l16 + 16 * (4 * pw + g4),
                           sh0 + kOffV + chan_lane(32 * pw, l16, g4),
                           sh0 + kOffV + chan_lane(32 * pw + 16, l16, g4),
                           sh0 + kOffU + 128 * C * pw + row32_lane(l16, g4),
                           lane, n_full, tail,
                           reinterpret_cast<const char *>(p.beta + first),
                           C * p.H * 2,
                           lane < C ? static_cast<uint32_t>(lane * p.H * 2) : 0u,
                           sh0 + kOffBeta + 4 * lane,
                           sh0 + kOffBeta + 16 * g4};
        __builtin_amdgcn_s_setprio(3);
        if (pw == 0) {
            // A of chunk it - 1 and WY of chunk it - 3 each iteration; the beta
            // logits of chunk y are loaded at iteration y - 1 into register
            // set y % 2 and used at iteration y + 1, where they first go to
            // LDS for the solve of chunk y at iteration y + 2.
            uint32_t b_even = nc > 0 ? sv.load_beta(0) : 0u, b_odd = 0;  // no chunk: nothing to read
            if (n_iter > 0)
                lds_barrier();  // the gate waves' first loads are in LDS
            for (int it = 0; it < n_iter; it += 2) {
                if (it >= 1 && it - 1 < nc)  // chunk it - 1 (odd)
                    sv.put_beta(it - 1, b_odd);
                b_odd = sv.load_beta(it + 1 < nc ? it + 1 : nc - 1);
                if (it >= 1 && it - 1 < nc)
                    sv.a_stage(it - 1);
                if (it >= 3 && it - 3 < nc)
                    sv.wy_stage(it - 3);
                lds_barrier();
                if (it < nc)  // chunk it (even)
                    sv.put_beta(it, b_even);
                b_even = sv.load_beta(it + 2 < nc ? it + 2 : nc - 1);
                if (it < nc)
                    sv.a_stage(it);
                if (it >= 2 && it - 2 < nc)
                    sv.wy_stage(it - 2);
                lds_barrier();
            }
            wait_vmem<0>();  // no load may still be writing registers when the wave ends
            return;
        }
        if (pw == 1) {
            // P of chunk it - 1 and WY of chunk it - 3 each iteration; this
            // wave also loads all 16 rows of g and v two chunks ahead (g into
            // the stage ring, v into its ring for WY), like the gate waves'
            // loads of q and k.  Without outputs P is not needed.
            Loader<4, kOut> lg, lv;
            lg.init(p.g + first * D, tok_bytes, 0, lane, tail, n_full, sh0 + kOffStage + 2 * kTile, 3 * kTile, 3);
            lv.init(p.v + first * D, tok_bytes, 0, lane, tail, n_full, sh0 + kOffV, kTile, 6);
            if (n_iter > 0) {
                for (int c = 0; c < 2; ++c) {  // chunks 0 and min(1, nc - 1)
                    lg.issue();
                    lv.issue();
                    lg.advance(nc);
                    lv.advance(nc);
                }
                wait_vmem<8>();  // chunk 0
                lds_barrier();
            }
            for (int it = 0; it < n_iter; ++it) {
                lg.issue();  // chunk min(it + 2, nc - 1); slots as for the gate waves' loads
                lv.issue();
                lg.advance(nc);
                lv.advance(nc);
                if constexpr (kOut)
                    if (it >= 1 && it - 1 < nc)
                        sv.p_stage(it - 1);
                if (it >= 3 && it - 3 < nc)
                    sv.wy_stage(it - 3);
                wait_vmem<8>();  // chunk it + 1
                lds_barrier();
            }
            wait_vmem<0>();  // no load may still be writing LDS when the wave ends
            return;
        }
        if (n_iter > 0)
            lds_barrier();  // the first loads are in LDS
        for (int it = 0; it < n_iter; ++it) {
            if (it >= 2 && it - 2 < nc) {
                if constexpr (INV == kInverseNeumann) {
                    if (pw == 2)
                        sv.solve_neumann(it - 2);
                } else {
                    sv.solve_stage(it - 2);
                }
            }
            if (it >= 3 && it - 3 < nc)
                sv.wy_stage(it - 3);
            lds_barrier();
        }
        return;
    }

    // gate waves: channels 16 gc16 .. 16 gc16 + 15 (and, fused, 16 gc16 + 64 ..)
    const int gc16 = wave - kStateWaves;
    const float head_mult = p.A_log ? expf(p.A_log[h]) : 1.0f;
    auto gate_wave = [&](int gc) {
        GateWave<PipeLayout> g{p, gc, lane, l16, g4, n_full, tail,
                               sh0 + kOffStage + chan_lane(16 * gc, l16, g4),
                               sh0 + 512 * gc + row16_lane(l16, g4),
                               sh0 + kOffGam + 4 * (16 * gc + l16)};
        g.head_neg = -head_mult * kLog2eF;
        g.bias_neg = p.dt_bias ? g.head_neg * p.dt_bias[h * D + 16 * gc + l16] : 0.f;
        g.head_y = 0.5f * head_mult;  // x / 2 = exp(A_log) (g + dt_bias) / 2
        g.bias_y = p.dt_bias ? g.head_y * p.dt_bias[h * D + 16 * gc + l16] : 0.f;
        g.gs_half = 0.5f * p.gate_scale;
        g.grp_hi = g4 >= 2 ? 1.0f : 0.0f;
        g.grp_odd = (g4 & 1) ? 1.0f : 0.0f;
        return g;
    };
    const GateWave<PipeLayout> gw = gate_wave(gc16);
    const GateWave<PipeLayout> gw2 = gate_wave(kFused ? gc16 + 4 : gc16);
    if (n_iter == 0)
        return;

    // The stage ring holds three chunks: iteration `it` starts the loads of
    // chunk it + 2, runs the gate stage on chunk it and, before the barrier,
    // waits for the loads of chunk it + 1 (issued one iteration earlier), so
    // every chunk has two iterations to arrive.  Past the last chunk the
    // iterations that drain the pipeline load and gate nothing (the state
    // waves then have the SIMDs to themselves).  Waves 4-7 load rows
    // 8 (gc16 % 2) .. + 7 of q (waves 4, 5) or k (6, 7); waves 8-11 load
    // nothing.  The state and solve waves (priority 3) sit on the critical
    // path; the gate waves fill the issue slots they leave.
    // Fused, waves 8-9 load the rows of k (q is not needed).
    __builtin_amdgcn_s_setprio(1);
    const int tensor = kFused ? 1 : gc16 >> 1;  // 0: q, 1: k
    const bool loads = kFused ? gc16 < 2 : gc16 < 4 && (kOut || gc16 >= 2);  // q only for the output
    Loader<2, kOut> ld;
    ld.init((tensor == 0 ? p.q : p.k) + first * D, tok_bytes, 8 * (gc16 & 1), lane, tail, n_full,
            sh0 + kOffStage + tensor * kTile, 3 * kTile, 3);
    if (loads) {
        for (int c = 0; c < 2; ++c) {  // chunks 0 and min(1, nc - 1)
            ld.issue();
            ld.advance(nc);
        }
    }
    wait_vmem<2>();  // chunk 0 (a no-op for the waves that load nothing)
    lds_barrier();
    uint32_t o3 = 0, o5 = 0;  // chunk it's stage slot and Qt / Kbar slot
    auto gate = [&](int it) {
        gw.template gate_stage<SIG, kOut>(it, o3, o5);
        if constexpr (kFused)
            gw2.template gate_stage<SIG, false>(it, o3, o5);
        o3 = o3 == 2 * (3 * kTile) ? 0 : o3 + 3 * kTile;
        o5 = o5 == 4 * kTile ? 0 : o5 + kTile;
    };
    int it = 0;
    for (; it < nc - 2; ++it) {
        // slot of chunk it + 2 (stage: last read by the gate stage of chunk
        // it - 1; V: by WY of chunk it - 4, both before the last barrier)
        if (loads) {
            ld.issue();
            ld.advance(nc);
        }
        gate(it);
        wait_vmem<2>();  // chunk it + 1
        lds_barrier();
    }
    // the last two chunks (nothing left to load), then the drain
    for (; it < n_iter; ++it) {
        if (it < nc)
            gate(it);
        wait_vmem<0>();  // chunk nc - 1 (first pass only; later a no-op)
        lds_barrier();
    }
    // no load may still be writing LDS when the wave ends
    wait_vmem<0>();
}

// One chunk per workgroup: the stages of the pipelined kernel run in order
// for a single chunk of at most 16 tokens, by 4 waves with the tiles of
// SharedSingle (36 KiB, so four chains share a compute unit), one barrier
// between stages.  For decode-shaped calls (T <= 16, no cu_seqlens): the
// state's loads overlap the loads, gate and solve of the chunk, and four
// workgroups per compute unit overlap one another's state traffic.  Wave w
// loads tensor w (q, k, g into the staging tiles, v into the V tile), takes
// channel groups 2w and 2w + 1 of the gate stage, the solve roles of solve
// wave w (A for w = 0, P for 1, T for 2 and 3, then WY for channels / value
// columns 32w ..) and value columns 32w .. of the state.
template <int SIG>
__global__ __launch_bounds__(256, 4) void chunk_single_kernel(FwdParams p)
{
    using SL = SingleLayout;
    __shared__ SharedSingle sh;
    const int chain = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x));
    const int H = static_cast<int>(p.H);
    const int64_t n = chain / H, h = chain - (chain / H) * H;
    int64_t t_begin, t_end, row;
    chain_segment(p, n, &t_begin, &t_end, &row);
    const int src = p.init_state ? (p.init_kind == kStateBf16 ? kSrcBf16 : kSrcFp32) : kSrcZero;
    const int dst = p.final_state ? (p.final_kind == kStateBf16 ? kDstBf16 : kDstFp32) : kDstNone;
    const int64_t slab = int64_t(chain) * D * D;
    // the host sends only calls of at most one chunk per sequence
    const int len_seq = static_cast<int>(t_end - t_begin);
    const int n_full = len_seq / C, tail = len_seq % C;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t tok_bytes = p.H * D * 2;
    const int64_t first = (row * p.T + t_begin) * p.H + h;
    const uint32_t sh0 = lds_addr(&sh);

    StateWave<SL> sw{p, wave, lane, l16, g4, n_full, tail,
                     reinterpret_cast<char *>(p.out + first * D + 32 * wave),
                     C * tok_bytes,
                     static_cast<uint32_t>(l16 * tok_bytes + 8 * g4),
                     sh0 + SL::kOffQt + tok_lane(l16, g4),
                     sh0 + SL::kOffW + 2 * kWPitch * l16 + 16 * g4,
                     sh0 + SL::kOffU + 128 * C * wave + row32_lane(l16, g4),
                     sh0 + SL::kOffP + row16_lane(l16, g4),
                     sh0 + SL::kOffGam + 16 * g4,
                     sh0 + SL::kOffKb + row16_lane(l16, g4),
                     {}};
    if (len_seq == 0) {  // an empty sequence passes its state through
        sw.load_state(src, p.init_state, slab);
        sw.store_state(dst, p.final_state, slab);
        return;
    }

    // Loads: the chunk's rows first, then beta (wave 0) and the state, so
    // that the wait for the rows leaves the state loads in flight.
    Loader<4> ld;
    ld.init((wave == 0 ? p.q : wave == 1 ? p.k : wave == 2 ? p.g : p.v) + first * D, tok_bytes, 0, lane,
            tail, n_full, sh0 + (wave < 3 ? SL::kOffStage + wave * kTile : SL::kOffV), kTile, 1);
    ld.issue();
    const int pw = wave;
    const int j0 = 8 * (pw - 2) + 2 * g4;  // the T solve's column pair (waves 2, 3)
    const SolveWave<SL> sv{pw, l16, g4,
                           sh0 + tok_lane(l16, g4),
                           sh0 + row16_lane(l16, g4),
                           sh0 + SL::kOffA + 4 * (4 * g4 * AP + l16),
                           sh0 + SL::kOffA + 4 * AP * l16,
                           sh0 + SL::kOffBeta + (pw == 0 ? 16 * g4 : 4 * j0),
                           sh0 + 2 * (l16 * C + chunk16(l16, j0 >> 2) + (j0 & 3)),
                           sh0 + SL::kOffKt + 64 * C * pw + row16_lane(l16, g4),
                           sh0 + SL::kOffW + 2 * kWPitch * l16 + 16 * (4 * pw + g4),
                           sh0 + SL::kOffV + chan_lane(32 * pw, l16, g4),
                           sh0 + SL::kOffV + chan_lane(32 * pw + 16, l16, g4),
                           sh0 + SL::kOffU + 128 * C * pw + row32_lane(l16, g4),
                           lane, n_full, tail,
                           reinterpret_cast<const char *>(p.beta + first),
                           C * p.H * 2,
                           lane < C ? static_cast<uint32_t>(lane * p.H * 2) : 0u,
                           sh0 + SL::kOffBeta + 4 * lane,
                           sh0 + SL::kOffBeta + 16 * g4};
    const uint32_t logit = wave == 0 ? sv.load_beta(0) : 0u;
    sw.load_state(src, p.init_state, slab);
    // The 16 state loads (fp32 or bf16 initial state) come after the row
    // loads; allowing 8 of them in flight still covers the rows.
    if (src == kSrcFp32 || src == kSrcBf16)
        wait_vmem<8>();
    else
        wait_vmem<0>();
    if (wave == 0)
        sv.put_beta(0, logit);

    const float head_mult = p.A_log ? expf(p.A_log[h]) : 1.0f;
    auto gate = [&](int gc16) {
        GateWave<SL> gw{p, gc16, lane, l16, g4, n_full, tail,
                        sh0 + SL::kOffStage + chan_lane(16 * gc16, l16, g4),
                        sh0 + 512 * gc16 + row16_lane(l16, g4),
                        sh0 + SL::kOffGam + 4 * (16 * gc16 + l16)};
        gw.head_neg = -head_mult * kLog2eF;
        gw.bias_neg = p.dt_bias ? gw.head_neg * p.dt_bias[h * D + 16 * gc16 + l16] : 0.f;
        gw.grp_hi = g4 >= 2 ? 1.0f : 0.0f;
        gw.grp_odd = (g4 & 1) ? 1.0f : 0.0f;
        gw.head_y = 0.5f * head_mult;
        gw.bias_y = p.dt_bias ? gw.head_y * p.dt_bias[h * D + 16 * gc16 + l16] : 0.f;
        gw.gs_half = 0.5f * p.gate_scale;
        gw.template gate_stage<SIG>(0, 0, 0);
    };
    lds_barrier();  // rows and beta in LDS
    gate(2 * wave);
    gate(2 * wave + 1);
    lds_barrier();
    if (wave == 0)
        sv.a_stage(0);
    else if (wave == 1)
        sv.p_stage(0);
    lds_barrier();
    if (wave >= 2)
        sv.solve_stage(0);
    lds_barrier();
    sv.wy_stage(0);  // W and U~ overwrite the staging tiles, which the gate stage has read
    lds_barrier();
    sw.template chunk<kChunkFull>(0, 0);
    sw.store_state(dst, p.final_state, slab);
}

}  // namespace

hipError_t launch_chunk_mfma(const FwdParams &p, hipStream_t stream)
{
    const int64_t chains = p.num_seqs * p.H;
    const int64_t blocks = p.phase == kPhaseWhole ? chains : chains * p.n_seg;
    const void *kernel;
    if (p.inverse == kInverseNeumann)
        kernel = p.phase == kPhaseMapB    ? reinterpret_cast<const void *>(&chunk_mfma_kernel<kChunkState, kInverseNeumann>)
                 : p.phase == kPhaseMapBM ? reinterpret_cast<const void *>(&chunk_mfma_kernel<kChunkMapBM, kInverseNeumann>)
                                          : reinterpret_cast<const void *>(&chunk_mfma_kernel<kChunkFull, kInverseNeumann>);
    else
        kernel = p.phase == kPhaseMapB    ? reinterpret_cast<const void *>(&chunk_mfma_kernel<kChunkState, kInverseSubst>)
                 : p.phase == kPhaseMapBM ? reinterpret_cast<const void *>(&chunk_mfma_kernel<kChunkMapBM, kInverseSubst>)
                                          : reinterpret_cast<const void *>(&chunk_mfma_kernel<kChunkFull, kInverseSubst>);
    // the tanh-form gate is built for whole chains with the default inverse
    if (p.sigmoid == kSigmoidTanh && p.phase == kPhaseWhole && p.inverse == kInverseSubst)
        kernel = reinterpret_cast<const void *>(&chunk_mfma_kernel<kChunkFull, kInverseSubst, kSigmoidTanh>);
    FwdParams args = p;
    void *argv[] = {&args};
    return hipLaunchKernel(kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), argv, 0, stream);
}

hipError_t launch_chunk_single(const FwdParams &p, hipStream_t stream)
{
    const int64_t chains = p.num_seqs * p.H;
    if (chains == 0)
        return hipSuccess;
    const void *kernel = p.sigmoid == kSigmoidTanh ? reinterpret_cast<const void *>(&chunk_single_kernel<kSigmoidTanh>)
                                                   : reinterpret_cast<const void *>(&chunk_single_kernel<kSigmoidExp>);
    FwdParams args = p;
    void *argv[] = {&args};
    return hipLaunchKernel(kernel, dim3(static_cast<unsigned>(chains)), dim3(256), argv, 0, stream);
}

}  // namespace kda
