// Host-side launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace kda {

struct PrefillParams {
    const void* q;
    const void* k;
    const void* v;
    const float* la;
    const float* beta;
    const float* S0;
    const int32_t* cu;      // device [n_seqs+1] or nullptr (equal lengths T)
    const int32_t* order;   // device [n_seqs] workspace for the longest-first order, or nullptr
    float* o;
    float* S_T;
    int64_t T;              // tokens per sequence (equal lengths) or total (packed)
    int32_t n_seqs, H, n_slices, n_units;
};

// Enqueue the prefill (and, when `sort`, the sequence-order pass first).
hipError_t launch_chunk_fwd(const PrefillParams& prm, bool bf16_in, int wcols, bool sort,
                            hipStream_t stream);

hipError_t launch_decode_step(const void* q, const void* k, const void* v, bool bf16_in,
                              const float* log_alpha, const float* beta, float* S,
                              int64_t n_states, float* o, hipStream_t stream);

}  // namespace kda
