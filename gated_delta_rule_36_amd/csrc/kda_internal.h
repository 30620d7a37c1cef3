// Internal interface between the C-ABI front end (kda_api.cpp) and the HIP
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace kda {

constexpr int kChunk = 16;     // tokens per chunk (fixed, as on the chunk-size page)
constexpr int kHeadDim = 128;  // K = V = 128

enum StateKind : int { kStateNone = 0, kStateBf16 = 1, kStateFp32 = 2 };
enum Phase : int { kPhaseWhole = 0, kPhaseMapB = 1, kPhaseMapBM = 2, kPhaseOut = 3 };
// How the MFMA kernel forms T = (I + A)^-1: fp32 forward substitution (the
// default) or the fp16 Neumann product (an ablation; KDA_INVERSE_NEUMANN).
enum Inverse : int { kInverseSubst = 0, kInverseNeumann = 1 };
// How the gate evaluates the logistic function: 1/(1 + 2^-x') with the
// hardware exp2 and rcp (the default), or 1/2 + tanh(x/2)/2 with a rational
// tanh (an ablation; KDA_SIGMOID_TANH, whole-chain chunked calls only).
enum Sigmoid : int { kSigmoidExp = 0, kSigmoidTanh = 1 };

// Everything a launch needs.  Pointers are device pointers; sizes were
// validated by the front end.
struct FwdParams {
    const uint16_t *q, *k, *v, *g, *beta;  // bf16 bit patterns
    uint16_t *out;                         // bf16 bit patterns
    const float *A_log;                    // [H] or nullptr
    const float *dt_bias;                  // [H,K] or nullptr
    const void *init_state;                // [N,H,V,K] or nullptr
    void *final_state;                     // [N,H,V,K] or nullptr
    int init_kind, final_kind;             // StateKind
    const int64_t *cu_seqlens;             // [N+1] or nullptr
    int64_t num_seqs;                      // N (sequences)
    int64_t T, H;                          // token axis length, heads
    float scale;                           // read-out scale
    float gate_scale;                      // lower_bound * log2(e), in fp32
    int inverse = kInverseSubst;           // Inverse (MFMA kernel)
    int sigmoid = kSigmoidExp;             // Sigmoid (MFMA kernel, whole chains)

    // Intra-sequence scan (kda_fwd_scan).  Every chain is cut into segments
    // of seg_chunks chunks; segment s maps its start state S to M_s S + b_s
    // (the recurrence is affine in the state).  Phases: kPhaseWhole (whole
    // chains, kda_fwd); kPhaseMapB: b_s of segments 0 .. last-1 into seg_b
    // (segment 0 from the real initial state, the others from zero);
    // kPhaseMapBM: the same and, in the same pass, M_s of segments
    // 1 .. last-1 into seg_m (identity start, v ignored); then the combine
    // step turns seg_b[s] into the true start state of segment s + 1;
    // kPhaseOut: every segment from its true start state, writing outputs,
    // and the final state from the last segment.
    int phase = 0;
    int64_t seg_chunks = 0;  // chunks per segment (phase != kPhaseWhole)
    int64_t n_seg = 1;       // segments per chain, the longest chain's count
    float *seg_b = nullptr;  // fp32 [chains][n_seg][V][K]
    float *seg_m = nullptr;  // [chains][n_seg] fp32-sized slabs: M_s itself as bf16 hi, lo planes [K][K]
};

// The kernels kda_fwd_ex chooses between.
enum Kernel : int { kKernelChunked = 1, kKernelRecurrent = 2, kKernelSingle = 3 };

// Enqueue the whole forward pass on `stream` with kernel `kernel`.  Returns
// the launch status.
hipError_t launch_forward(const FwdParams &p, int kernel, hipStream_t stream);

// Enqueue the segmented form: map (phase 1), combine, output (phase 3).
// p.seg_chunks, p.n_seg, p.seg_b and p.seg_m must be set.
hipError_t launch_forward_scan(const FwdParams &p, hipStream_t stream);

// Individual kernel launchers (one per implementation).
hipError_t launch_chunk_mfma(const FwdParams &p, hipStream_t stream);
// The chunked stages for calls of at most one chunk (16 tokens) per sequence
// and no cu_seqlens: one 4-wave workgroup per chain, several per compute unit.
hipError_t launch_chunk_single(const FwdParams &p, hipStream_t stream);
// The token recurrence for decode-shaped calls (few tokens per sequence,
// state in and out): one small workgroup per chain.
hipError_t launch_decode(const FwdParams &p, hipStream_t stream);
// Calls without cu_seqlens of at most this many tokens per sequence take the
// recurrent kernel by default; up to one chunk (16 tokens), the single-chunk
// kernel; longer or packed calls, the pipelined chunked kernel.
constexpr int64_t kRecurrentMaxTokens = 8;
// Bytes of the fixed device scratch kda_fwd_scan_static uses instead of a
// caller workspace (KDA_SCAN_STATIC_BYTES in kda.h).
constexpr int64_t kStaticScratchBytes = int64_t(32) << 20;
// Device address of that scratch on the current device (looked up once per
// device with hipGetSymbolAddress).
hipError_t static_scratch(void **ptr);

// The combine step of the segmented form: for every chain and s >= 1,
// seg_b[c][s] <- M_s seg_b[c][s-1] + seg_b[c][s] (in stored [V][K] terms).
hipError_t launch_scan_combine(const FwdParams &p, hipStream_t stream);

}  // namespace kda
