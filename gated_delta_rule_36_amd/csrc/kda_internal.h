// Internal interface between the C-ABI front end (kda_api.cpp) and the HIP
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace kda {

constexpr int kChunk = 16;     // tokens per chunk (fixed, as on the chunk-size page)
constexpr int kHeadDim = 128;  // K = V = 128

enum StateKind : int { kStateNone = 0, kStateBf16 = 1, kStateFp32 = 2 };

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
};

// Enqueue the whole forward pass on `stream`.  Returns the launch status.
hipError_t launch_forward(const FwdParams &p, hipStream_t stream);

// Individual kernel launchers (one per implementation).
hipError_t launch_chunk_mfma(const FwdParams &p, hipStream_t stream);
hipError_t launch_chunk_simt(const FwdParams &p, hipStream_t stream);

}  // namespace kda
