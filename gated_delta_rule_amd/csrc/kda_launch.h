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
    // Equal lengths only: each sequence is cut into segments, segment 0 of
    // seg_first tokens (0: seg_len) and every later one of seg_len tokens
    // (the last one shorter); a launch runs segments seg_r0 .. seg_r0 +
    // seg_per_seq - 1 of every sequence as independent chains, chain
    // b * seg_per_seq + (r - seg_r0) for segment r of sequence b.
    // seg_per_seq = 1, seg_len = T, seg_first = seg_r0 = 0: no split.  The
    // pipelined kernel takes uniform segments only (seg_first 0 or seg_len,
    // seg_r0 0).
    int64_t seg_len;
    int32_t seg_per_seq;
    // Window mode (equal lengths, backward pass): seg_sel >= 0 runs only
    // segment seg_sel of each of the n_seqs sequences (chain n = sequence n),
    // and h_states / r_out / u_out use the window's compact layout: chunk j
    // of the window in slot n * (seg_len / 32) + j, token t of the window in
    // row n * seg_len + (t - window start).  -1 otherwise.
    int32_t seg_sel;
    // Transition pass: every chain starts from the identity state and reads
    // v as zero, so its final state is the chain's linear map S_in -> S_out.
    int32_t s0_identity;
    int32_t n_seqs, H, n_slices, n_units;   // n_seqs counts chains (segments)
    // Optional [slots, H, 128, 128]: the state at the start of every chunk
    // (unsplit sequences or window mode); chunk j of sequence n starting at
    // token t0 goes to slot t0 / 32 + n + j, which no other chunk uses (in
    // window mode: see seg_sel).
    float* h_states;
    // With h_states: V - K+ S and U of every chunk, token-major like o.
    float* r_out;
    float* u_out;
    // Two chains at once (launch_chunk_fwd_dual): the chain from S0 (or zero)
    // with the values v, whose final state goes to S_T, and the chain from the
    // identity with v read as zero, whose final state (the transition) goes
    // to S_T2.  o is not written.  nullptr otherwise.
    float* S_T2;
    // (segment plan, see seg_len)
    int64_t seg_first;
    int32_t seg_r0;
};

// The bf16 prefill with 16 value columns per consumer wave as a three-stage
// pipeline (scan, tiles, chain) with one workgroup barrier per chunk.  Same
// arguments, grid and outputs (h_states, r_out, u_out included).
hipError_t launch_chunk_fwd_pipe(const PrefillParams& p, hipStream_t stream);

// Enqueue the prefill (and, when `sort`, the sequence-order pass first).
hipError_t launch_chunk_fwd(const PrefillParams& prm, bool bf16_in, int wcols, bool sort,
                            hipStream_t stream);

// Both chains of a segment in one launch (one 32-column-per-wave workgroup
// per (segment, head); n_slices must be 1): the local final state from S0 or
// zero into S_T and the transition (identity start, v = 0) into S_T2.
hipError_t launch_chunk_fwd_dual(const PrefillParams& prm, bool bf16_in, hipStream_t stream);

// Incoming states of the segmented prefill's segments after the first:
// S_in[b, 0] = E[b] (the first segment's final state), S_in[b, j + 1] =
// F[b, j] S_in[b, j] + Sl[b, j] for the n_mid middle segments, whose
// transition F and zero-start final state Sl were computed.  S_in[b, j] for
// j < n_mid goes to S_mid[b, j], S_in[b, n_mid] (the last segment's) to
// S_last[b].  E and S_last [B, H, 128, 128]; F, Sl and S_mid
// [B * n_mid, H, 128, 128].
hipError_t launch_segment_merge(const float* F, const float* Sl, const float* E, float* S_mid,
                                float* S_last, int32_t B, int32_t n_mid, int32_t H,
                                hipStream_t stream);

// Multi-token recurrent decode: per state, apply the first n_replay[b]
// (NULL: all Tr) replay tokens, then T tokens with outputs; the state is
// stored after the replay (commit = 0) or after everything (commit = 1).
hipError_t launch_recurrent(const void* q, const void* k, const void* v, bool bf16_in,
                            const float* log_alpha, const float* beta, const void* rq,
                            const void* rk, const void* rv, const float* rlog_alpha,
                            const float* rbeta, const int32_t* n_replay, float* S,
                            int64_t n_states, int32_t H, int32_t T, int32_t Tr, int32_t commit,
                            float* o, hipStream_t stream);

// Layer prologue / epilogue (equal lengths: cu == nullptr, rows = n_seqs * T;
// packed: rows = T, cu [n_seqs + 1]).  cache [n_seqs, 3 tensors, 3 taps, H, 128]
// or nullptr.
struct LayerParams {
    const void* q_raw;
    const void* k_raw;
    const void* v_raw;
    const float* conv_w;    // [3, H, 128, 4]
    float* cache;
    const float* a;         // [rows, H, 128]
    const float* b;         // [rows, H]
    const int32_t* cu;
    void* q;
    void* k;
    void* v;
    float* log_alpha;
    float* beta;
    int64_t rows, T;
    int32_t n_seqs, H;
};
hipError_t launch_prologue(const LayerParams& p, bool bf16_in, hipStream_t stream);
hipError_t launch_epilogue(const float* o, const float* g, const float* w, float* out, int64_t items,
                           hipStream_t stream);

// Backward pass after a forward pass that stored the state at every chunk
// start in h (see PrefillParams::h_states; chunk j of sequence n in slot
// start_n / 32 + n + j).  Arrays: h, dsn [slots, H, 128, 128];
// tmp [slots, H, 15488] floats per (chunk, head): T^T, M^T, P [32][32],
// K_end^T, Q+^T, -(B_beta K+)^T [128][32] and e^{g_C} [128];
// w, r, u [tokens, H, 128].  Window mode (win_len > 0, equal lengths only):
// the pass covers tokens [win_idx * win_len, (win_idx + 1) * win_len) of
// every sequence, with the compact slots and rows of PrefillParams::seg_sel
// (slots = n_seqs * win_len / 32, rows = n_seqs * win_len); dS_T is the
// gradient at the window's end and dS0 receives the one at its start (the
// same array is allowed: each element is read before it is written, by the
// same thread).
struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const float* la;
    const float* beta;
    const int32_t* cu;      // device [n_seqs + 1] or nullptr (equal lengths T)
    const float* dO;
    const float* dS_T;      // or nullptr (zero)
    float* dq;
    float* dk;
    float* dv;
    float* dla;
    float* dbeta;
    float* dS0;             // or nullptr (not wanted)
    const float* h;
    const float* r;         // [tokens, H, 128]: V - K+ S of the forward pass
    const float* u;         // [tokens, H, 128]: U of the forward pass
    float* dsn;
    float* tmp;
    float* w;
    int64_t T;              // tokens per sequence (equal lengths) or total (packed)
    int64_t slots;
    int64_t win_len;        // window mode: tokens per window (a multiple of 32), else 0
    int32_t win_idx;        // window mode: which window
    int32_t n_seqs, H;
};
hipError_t launch_chunk_bwd(const BwdParams& p, bool bf16_in, hipStream_t stream);
// The same passes split at the point where they need the forward pass: the
// chunk matrices read only the inputs, so they may run beside it.
hipError_t launch_chunk_bwd_tmp(const BwdParams& p, bool bf16_in, hipStream_t stream);
hipError_t launch_chunk_bwd_walk_grad(const BwdParams& p, bool bf16_in, hipStream_t stream);

}  // namespace kda
