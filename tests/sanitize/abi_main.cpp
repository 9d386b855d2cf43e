// Sanitizer driver for the C ABI's host code (gated_delta_rule_amd/csrc/
// kda_abi.hip compiled as plain C++ with g++ and -fsanitize=address,undefined
// by tests/test_sanitizers.py; CPU only).  The kernel launchers are replaced
// by stubs that record what they were asked to launch and touch no memory,
// so every validation branch and every launch plan (packed batches, equal
// lengths, the sequence-parallel path, decode, recurrent, layer steps,
// backward) runs under the sanitizers without a GPU.  The pointers are fake
// device addresses that are never dereferenced.  The few HIP runtime calls
// the ABI makes itself (the backward's second stream and its events) are
// stubbed too and logged beside the launches, so the fork / join order of
// the backward's passes is checked as well.
#include <stdint.h>
#include <stdio.h>

#include "kda.h"
#include "kda_launch.h"

namespace {
int n_launch = 0, n_merge = 0, n_dual = 0, last_slices = 0, last_units = 0;
int fails = 0;
int fail_fwd_in = -1;   // > 0: the forward launch that many calls from now fails
// forward and backward launches in order, for the backward's window plan
struct Rec {
    char kind;                 // 'f' forward, 'd' dual-chain forward, 'm' merge,
                               // 't' chunk matrices, 'g' walk + gradients,
                               // 'r' event record, 'w' stream waits for event
    int seg_sel, win_idx;
    bool stores;               // forward keeps per-chunk values
    const float *S0, *S_T, *dS_T;
    float* dS0;
    int64_t seg_len, win_len, slots;
    hipStream_t stream;        // stream of the launch / record / wait
    hipEvent_t event;          // 'r', 'w'
    // forward launches ('f', and 'd' for the dual-chain pass): the segment plan
    int64_t seg_first = 0;
    int seg_r0 = 0, seg_per_seq = 0, n_seqs = 0, n_units = 0, n_slices = 0;
    bool has_o = false;
    const float* S_T2 = nullptr;
};
Rec recs[512];
int n_recs = 0;
void rec(const Rec& r) {
    if (n_recs < 512) recs[n_recs++] = r;
}
// the stubbed runtime's objects: fake handles, never dereferenced
hipStream_t const kSide = (hipStream_t)(uintptr_t)0x5100;
int n_events = 0, n_streams = 0;
#define CHECK(c)                                                               \
    do {                                                                       \
        if (!(c)) {                                                            \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);     \
            ++fails;                                                           \
        }                                                                      \
    } while (0)
}  // namespace

namespace kda {
hipError_t launch_chunk_fwd_pipe(const PrefillParams&, hipStream_t) { return hipSuccess; }
static void rec_fwd(char kind, const PrefillParams& p, hipStream_t stream) {
    Rec r{kind, p.seg_sel, 0, p.h_states != nullptr, p.S0, p.S_T, nullptr, nullptr, p.seg_len, 0, 0,
          stream, nullptr};
    r.seg_first = p.seg_first;
    r.seg_r0 = p.seg_r0;
    r.seg_per_seq = p.seg_per_seq;
    r.n_seqs = p.n_seqs;
    r.n_units = p.n_units;
    r.n_slices = p.n_slices;
    r.has_o = p.o != nullptr;
    r.S_T2 = p.S_T2;
    rec(r);
}
hipError_t launch_chunk_fwd(const PrefillParams& p, bool, int wcols, bool, hipStream_t stream) {
    ++n_launch;
    rec_fwd('f', p, stream);
    if (fail_fwd_in > 0 && --fail_fwd_in == 0) return hipErrorInvalidValue;
    CHECK(p.seg_sel < 0 || (!p.cu && p.seg_len % 32 == 0 && p.seg_len > 0));
    CHECK(!p.h_states || (p.r_out && p.u_out && !p.o));
    last_slices = p.n_slices;
    last_units = p.n_units;
    CHECK(wcols * 4 * p.n_slices == 128);
    CHECK(p.n_units == p.n_seqs * p.H);
    return hipSuccess;
}
hipError_t launch_chunk_fwd_dual(const PrefillParams& p, bool, hipStream_t stream) {
    ++n_launch;
    ++n_dual;
    rec_fwd('d', p, stream);
    CHECK(p.n_slices == 1 && p.S_T && p.S_T2 && !p.o && !p.S0);
    CHECK(p.n_units == p.n_seqs * p.H);
    return hipSuccess;
}
hipError_t launch_segment_merge(const float* F, const float* Sl, const float* E, float* S_mid,
                                float* S_last, int32_t B, int32_t n_mid, int32_t H, hipStream_t stream) {
    ++n_merge;
    // S0 = E, S_T = S_mid, dS_T = F, S_T2 = Sl, dS0 = S_last, seg_len = n_mid
    Rec r{'m', -1, -1, false, E, S_mid, F, S_last, n_mid, 0, 0, stream, nullptr};
    r.S_T2 = Sl;
    r.n_seqs = B;
    rec(r);
    CHECK(B >= 1 && n_mid >= 1 && H >= 1 && F && Sl && E && S_mid && S_last);
    return hipSuccess;
}
hipError_t launch_recurrent(const void*, const void*, const void*, bool, const float*, const float*,
                            const void*, const void*, const void*, const float*, const float*,
                            const int32_t*, float*, int64_t n_states, int32_t, int32_t T, int32_t Tr,
                            int32_t, float*, hipStream_t) {
    ++n_launch;
    CHECK(n_states >= 1 && T >= 0 && T <= 64 && Tr >= 0 && Tr <= 64);
    return hipSuccess;
}
hipError_t launch_prologue(const LayerParams& p, bool, hipStream_t) {
    ++n_launch;
    CHECK(p.rows >= 1);
    return hipSuccess;
}
hipError_t launch_epilogue(const float*, const float*, const float*, float*, int64_t items,
                           hipStream_t) {
    ++n_launch;
    CHECK(items >= 1);
    return hipSuccess;
}
static void bwd_checks(const BwdParams& p) {
    CHECK(p.slots >= 1);
    CHECK(p.win_len == 0 || (!p.cu && p.win_len % 32 == 0 && p.slots * 32 == p.n_seqs * p.win_len));
}
hipError_t launch_chunk_bwd_tmp(const BwdParams& p, bool, hipStream_t stream) {
    ++n_launch;
    bwd_checks(p);
    rec(Rec{'t', -1, p.win_idx, false, nullptr, nullptr, p.dS_T, p.dS0, 0, p.win_len, p.slots, stream,
            nullptr});
    return hipSuccess;
}
hipError_t launch_chunk_bwd_walk_grad(const BwdParams& p, bool, hipStream_t stream) {
    ++n_launch;
    bwd_checks(p);
    rec(Rec{'g', -1, p.win_idx, false, nullptr, nullptr, p.dS_T, p.dS0, 0, p.win_len, p.slots, stream,
            nullptr});
    return hipSuccess;
}
}  // namespace kda

// HIP runtime calls of the ABI itself
hipError_t hipGetDevice(int* d) {
    *d = 0;
    return hipSuccess;
}
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned int) {
    ++n_streams;
    *s = kSide;
    return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
    *e = (hipEvent_t)(uintptr_t)(0xe000 + 16 * ++n_events);
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s) {
    rec(Rec{'r', -1, -1, false, nullptr, nullptr, nullptr, nullptr, 0, 0, 0, s, e});
    return hipSuccess;
}
hipError_t hipStreamWaitEvent(hipStream_t s, hipEvent_t e, unsigned int) {
    rec(Rec{'w', -1, -1, false, nullptr, nullptr, nullptr, nullptr, 0, 0, 0, s, e});
    return hipSuccess;
}

// 1 TiB apart, so no two of them overlap at these sizes
static const void* P(int i) { return (const void*)(uintptr_t)((1ull << 44) + (uint64_t)i * (1ull << 40)); }
static float* F(int i) { return (float*)P(i); }

int main() {
    // equal lengths, enough pairs for one slice per head
    CHECK(kda_chunk_fwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), nullptr, nullptr, 3, 45, 96, 128,
                        128, F(5), F(6), nullptr, 0, nullptr) == KDA_OK);
    CHECK(last_slices == 1 && last_units == 288);
    // few pairs: two slices per head
    CHECK(kda_chunk_fwd(P(0), P(1), P(2), KDA_F32, F(3), F(4), F(7), nullptr, 1, 8192, 96, 128, 128,
                        F(5), F(7), nullptr, 0, nullptr) == KDA_OK);
    CHECK(last_slices == 2);
    // packed batch with its order workspace
    CHECK(kda_chunk_fwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), nullptr, (const int32_t*)P(8), 32,
                        270000, 96, 128, 128, F(5), nullptr, (void*)P(9), 128, nullptr) == KDA_OK);
    // sequence-parallel path.  Pass 1: segment 0 from S0 (writing o) on the
    // second stream beside the dual-chain pass over the middle segments; the
    // merge from segment 0's final state; pass 2: the last segment (from its
    // incoming state, writing o and S_T) on the second stream beside the
    // rerun of the middle segments.  The segments of the plan (the kernels'
    // mapping from chain index to tokens, restated here) tile every sequence
    // exactly, and both passes fit the 256 compute units.
    hipStream_t const kMainF = (hipStream_t)(uintptr_t)0x3400;
    auto seg_range = [](const Rec& f, int64_t T, int64_t n, int64_t* t0, int64_t* t1) {
        const int64_t b = n / f.seg_per_seq, r = f.seg_r0 + (n - b * f.seg_per_seq);
        const int64_t first = f.seg_first > 0 ? f.seg_first : f.seg_len;
        const int64_t len = r == 0 ? first : f.seg_len, e = (b + 1) * T;
        *t0 = b * T + (r == 0 ? 0 : first + (r - 1) * f.seg_len);
        if (*t0 > e) *t0 = e;
        *t1 = e - *t0 > len ? *t0 + len : e;
    };
    auto seq_parallel_plan = [&](int n_seqs, int64_t T, int H, const float* S0, float* S_T,
                                 int expect_P, int dtype = KDA_BF16) {
        const size_t ws = kda_chunk_fwd_workspace_bytes(n_seqs, T, H, 128, 128, 0);
        const int64_t units = (int64_t)n_seqs * H;
        CHECK(ws == (size_t)(3 * expect_P - 4) * units * 65536);
        n_recs = 0;
        CHECK(kda_chunk_fwd(P(0), P(1), P(2), dtype, F(3), F(4), S0, nullptr, n_seqs, T, H, 128,
                            128, F(5), S_T, (void*)P(9), ws, kMainF) == KDA_OK);
        // launches in order, with the fork / join state at each
        const Rec* L[8] = {};
        bool forked[8] = {}, side_joined = false;
        int nl = 0, joins = 0;
        hipEvent_t fork_ev = nullptr, join_ev = nullptr;
        bool fork_open = false;
        for (int i = 0; i < n_recs; ++i) {
            const Rec& r = recs[i];
            if (r.kind == 'r' && r.stream == kMainF) { fork_ev = r.event; fork_open = false; }
            else if (r.kind == 'w' && r.stream == kSide) fork_open = r.event == fork_ev && fork_ev;
            else if (r.kind == 'r' && r.stream == kSide) join_ev = r.event;
            else if (r.kind == 'w' && r.stream == kMainF) { CHECK(r.event == join_ev && join_ev); ++joins; side_joined = true; }
            else if (nl < 8 && r.kind != 'r' && r.kind != 'w') {
                forked[nl] = r.stream == kSide && fork_open;
                L[nl++] = &r;
                if (r.stream == kSide) side_joined = false;
            }
        }
        CHECK(nl == 5 && joins == 2 && side_joined);
        if (nl != 5) return;
        const Rec &f0 = *L[0], &fd = *L[1], &fm = *L[2], &fl = *L[3], &fc = *L[4];
        CHECK(f0.kind == 'f' && forked[0] && fd.kind == 'd' && fd.stream == kMainF);
        CHECK(fm.kind == 'm' && fm.stream == kMainF);
        CHECK(fl.kind == 'f' && forked[3] && fc.kind == 'f' && fc.stream == kMainF);
        const int Pn = fd.seg_per_seq + 2;
        CHECK(Pn == expect_P);
        // segment 0: from S0, writes o and its final state E (one uniform
        // segment: the pipelined kernel's plain mapping)
        CHECK(f0.seg_r0 == 0 && f0.seg_per_seq == 1 && f0.n_seqs == n_seqs && f0.has_o &&
              f0.S0 == S0 && f0.S_T && f0.n_slices == 2 && f0.n_units == units && f0.seg_first == 0);
        // dual pass over the middle segments: no o, from zero and from I
        CHECK(fd.seg_r0 == 1 && fd.n_seqs == n_seqs * (Pn - 2) && fd.n_slices == 1 && !fd.has_o);
        // the merge: E -> incoming states (middle segments, last segment)
        CHECK(fm.S0 == f0.S_T && fm.dS_T == fd.S_T2 && fm.S_T2 == fd.S_T &&
              fm.seg_len == Pn - 2 && fm.n_seqs == n_seqs);
        // the middle segments rerun from their incoming states, write o
        CHECK(fc.seg_r0 == 1 && fc.seg_per_seq == Pn - 2 && fc.n_seqs == n_seqs * (Pn - 2) &&
              fc.has_o && fc.S0 == fm.S_T && fc.S_T == nullptr && fc.n_slices == 1);
        CHECK(fc.seg_len == fd.seg_len && fc.seg_first == fd.seg_first && f0.seg_len == fd.seg_first);
        // the last segment: from its incoming state, writes o and S_T
        CHECK(fl.seg_r0 == 1 && fl.seg_per_seq == 1 && fl.n_seqs == n_seqs && fl.n_slices == 2 &&
              fl.has_o && fl.S_T == S_T && fl.S0 == fm.dS0 && fl.seg_len >= T);
        CHECK(units * Pn <= 256);
        for (int64_t b = 0; b < n_seqs; ++b) {
            int64_t t0, t1, at = b * T;
            seg_range(f0, T, b, &t0, &t1);
            CHECK(t0 == at && t1 > t0 && (t1 - t0) % 32 == 0);
            at = t1;
            for (int r = 1; r < Pn - 1; ++r) {
                int64_t c0, c1, d0, d1;
                seg_range(fc, T, b * (Pn - 2) + (r - 1), &c0, &c1);
                seg_range(fd, T, b * (Pn - 2) + (r - 1), &d0, &d1);
                CHECK(c0 == at && c1 > c0 && (c1 - c0) % 32 == 0 && d0 == c0 && d1 == c1);
                at = c1;
            }
            seg_range(fl, T, b, &t0, &t1);
            CHECK(t0 == at && t1 == (b + 1) * T && t1 - t0 >= 32);
        }
    };
    seq_parallel_plan(1, 1 << 20, 16, nullptr, F(6), 16);   // 1M tokens, 16 heads
    seq_parallel_plan(1, 1 << 20, 16, F(7), F(7), 16);      // S_T == S0
    seq_parallel_plan(2, 7000, 3, F(7), F(6), 3);           // ragged last segment
    seq_parallel_plan(1, 8192, 64, F(7), nullptr, 4);       // rerun on 192 one-slice chains
    seq_parallel_plan(1, 8192, 4, nullptr, F(6), 4);        // 12 rerun chains
    seq_parallel_plan(3, 100000, 1, F(7), F(6), 48);
    seq_parallel_plan(1, 1 << 22, 1, nullptr, F(6), 256);
    for (int64_t T = 6144; T < 6144 + 40; ++T) seq_parallel_plan(1, T, 5, nullptr, F(6), 3);
    for (int64_t T = 6144; T < 6144 + 40; ++T) seq_parallel_plan(1, T, 5, nullptr, F(6), 3, KDA_F32);
    seq_parallel_plan(1, 1 << 18, 16, F(7), F(6), 16, KDA_F32);
    for (int P = 3; P <= 256; P += 23) seq_parallel_plan(1, 2048 * P, 1, nullptr, F(6), P);
    for (int P = 3; P <= 256; P += 23) seq_parallel_plan(1, 2048 * P + 2047, 1, F(7), F(6), P, KDA_F32);
    // too short for three segments: the sequential path, no workspace
    CHECK(kda_chunk_fwd_workspace_bytes(2, 6000, 3, 128, 128, 0) == 0);
    CHECK(kda_chunk_fwd_workspace_bytes(1, 8192, 96, 128, 128, 0) == 0);
    // error paths
    CHECK(kda_chunk_fwd(P(0), P(1), P(2), 9, F(3), F(4), nullptr, nullptr, 1, 8, 4, 128, 128, F(5),
                        nullptr, nullptr, 0, nullptr) == KDA_ERR_BAD_DTYPE);
    CHECK(kda_chunk_fwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), nullptr, nullptr, 1, 8,
                        KDA_MAX_HEADS + 1, 128, 128, F(5), nullptr, nullptr, 0,
                        nullptr) == KDA_ERR_TOO_LARGE);
    CHECK(kda_chunk_fwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), nullptr, nullptr, 0x7fffffff,
                        (int64_t)1 << 40, 4, 128, 128, F(5), nullptr, nullptr, 0,
                        nullptr) == KDA_ERR_TOO_LARGE);
    CHECK(kda_chunk_fwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), nullptr, (const int32_t*)P(8), 2, 64,
                        4, 128, 128, F(5), nullptr, nullptr, 0, nullptr) == KDA_ERR_WORKSPACE);
    CHECK(kda_chunk_fwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), nullptr, nullptr, 2, 64, 4, 128, 128,
                        (float*)P(0), nullptr, nullptr, 0, nullptr) == KDA_ERR_ALIASING);
    // decode, recurrent
    CHECK(kda_decode_step(P(0), P(1), P(2), KDA_BF16, F(3), F(4), F(6), 256, 96, 128, 128, F(5),
                          nullptr) == KDA_OK);
    CHECK(kda_decode_step(P(0), P(1), P(2), KDA_BF16, F(3), F(4), F(6), 4, 4, 128, 128, F(6),
                          nullptr) == KDA_ERR_ALIASING);
    CHECK(kda_recurrent_fwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), P(10), P(11), P(12), F(13), F(14),
                            (const int32_t*)P(15), F(6), 8, 4, 4, 4, 128, 128, 0, F(5),
                            nullptr) == KDA_OK);
    CHECK(kda_recurrent_fwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), nullptr, nullptr, nullptr, nullptr,
                            nullptr, nullptr, F(6), 8, 65, 0, 4, 128, 128, 1, F(5),
                            nullptr) == KDA_ERR_BAD_SHAPE);
    // layer steps
    CHECK(kda_prologue(P(0), P(1), P(2), KDA_BF16, F(3), F(16), F(4), F(17), (const int32_t*)P(8), 3,
                       100, 4, 128, (void*)P(5), (void*)P(6), (void*)P(7), F(9), F(10),
                       nullptr) == KDA_OK);
    CHECK(kda_epilogue(F(0), F(1), F(2), 64, 4, 128, F(0), nullptr) == KDA_OK);
    CHECK(kda_epilogue(F(0), F(1), F(2), 64, 4, 128, F(1), nullptr) == KDA_ERR_ALIASING);
    // backward: equal lengths run in windows, the last first
    // The launches of the last call, without the event records and waits,
    // and a check that every chunk-matrix pass runs on the second stream
    // after a fork from the caller's stream and is joined before the walk
    // that reads it.
    hipStream_t const kMain = (hipStream_t)(uintptr_t)0x3300;
    auto launches = [&](Rec* out, int cap) {
        int n = 0;
        for (int i = 0; i < n_recs && n < cap; ++i)
            if (recs[i].kind != 'r' && recs[i].kind != 'w') out[n++] = recs[i];
        return n;
    };
    auto check_fork_join = [&]() {
        hipEvent_t fork_ev = nullptr, join_ev = nullptr;
        bool side_waited = false;   // the side stream waits for the latest fork record
        bool pending = false;       // a chunk-matrix pass not yet joined
        for (int i = 0; i < n_recs; ++i) {
            const Rec& r = recs[i];
            if (r.kind == 'r' && r.stream == kMain) { fork_ev = r.event; side_waited = false; }
            else if (r.kind == 'w' && r.stream == kSide) CHECK(side_waited = (r.event == fork_ev));
            else if (r.kind == 'r' && r.stream == kSide) join_ev = r.event;
            else if (r.kind == 'w' && r.stream == kMain) { CHECK(r.event == join_ev && join_ev); pending = false; }
            else if (r.kind == 't') { CHECK(r.stream == kSide && side_waited); pending = true; }
            else if (r.kind == 'g') { CHECK(r.stream == kMain && !pending); }
            else if (r.kind == 'f') CHECK(r.stream == kMain);
        }
        CHECK(!pending);
    };
    auto bwd_plan = [&](int n_seqs, int64_t T, size_t ws, const float* S0, const float* gST,
                        float* gS0, int expect_windows, int64_t expect_win_len) {
        n_recs = 0;
        CHECK(kda_chunk_bwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), S0, nullptr, n_seqs, T, 96, 128,
                            128, F(20), gST, F(21), F(22), F(23), F(24), F(25), gS0, (void*)P(27), ws,
                            kMain) == KDA_OK);
        check_fork_join();
        Rec L[512];
        const int n = launches(L, 512);
        const int K = expect_windows;
        // the last window's chunk matrices, the K - 1 window-start passes,
        // then per window (last first) its chunk matrices (all but the
        // first), the forward keeping values, the walk and gradients
        CHECK(n == 1 + (K - 1) + 3 * K - 1);
        if (n != 1 + (K - 1) + 3 * K - 1) return;
        CHECK(L[0].kind == 't' && L[0].win_idx == K - 1);
        // the states at the window starts: forward over windows 0 .. K-2
        const float* prev_end = nullptr;
        for (int w = 0; w + 1 < K; ++w) {
            const Rec& r = L[1 + w];
            CHECK(r.kind == 'f' && r.seg_sel == w && !r.stores && r.S_T && r.seg_len == expect_win_len);
            CHECK(w == 0 ? r.S0 == S0 : r.S0 == prev_end);
            prev_end = r.S_T;
        }
        const float* carry = nullptr;
        int at = K;
        for (int i = 0; i < K; ++i) {
            const int w = K - 1 - i;
            if (i > 0) {
                const Rec& t = L[at++];
                CHECK(t.kind == 't' && t.win_idx == w && t.win_len == expect_win_len);
            }
            const Rec& f = L[at++];
            const Rec& b = L[at++];
            CHECK(f.kind == 'f' && f.seg_sel == w && f.stores && f.seg_len == expect_win_len);
            CHECK(w == 0 ? f.S0 == S0 : f.S0 == L[w].S_T);
            CHECK(b.kind == 'g' && b.win_idx == w && b.win_len == expect_win_len);
            CHECK(b.slots == n_seqs * expect_win_len / 32);
            CHECK(w == K - 1 ? b.dS_T == gST : b.dS_T == carry);
            if (w == 0) CHECK(b.dS0 == gS0);
            else CHECK(b.dS0 != nullptr && (w == K - 1 || b.dS0 == carry));
            carry = b.dS0;
        }
    };
    {
        const size_t ws = kda_chunk_bwd_workspace_bytes(1, 8192, 96, 128, 128, 0);
        CHECK(ws > 0 && ws == kda_chunk_bwd_workspace_bytes_window(1, 8192, 96, 128, 128, KDA_BWD_WINDOW));
        bwd_plan(1, 8192, ws, nullptr, nullptr, F(26), 4, 2048);
        bwd_plan(1, 8192, ws, F(7), F(8), F(26), 4, 2048);
        // a little less workspace: the next shorter window
        bwd_plan(1, 8192, ws - 1, nullptr, nullptr, F(26), 8, 1024);
        // one window, as large as the sequence
        const size_t one = kda_chunk_bwd_workspace_bytes_window(1, 8192, 96, 128, 128, 8192);
        CHECK(one > ws && one == kda_chunk_bwd_workspace_bytes_window(1, 8192, 96, 128, 128, 1 << 30));
        bwd_plan(1, 8192, one, F(7), F(8), F(8), 1, 8192);
        // a ragged last window, three sequences
        const size_t w3 = kda_chunk_bwd_workspace_bytes_window(3, 300, 96, 128, 128, 64);
        bwd_plan(3, 300, w3, F(7), F(8), F(26), 5, 64);
        // nothing to run but the gradient hand-through
        bwd_plan(2, 0, kda_chunk_bwd_workspace_bytes(2, 0, 96, 128, 128, 0), F(7), F(8), F(26), 1, 32);
        CHECK(kda_chunk_bwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), nullptr, nullptr, 1, 8192, 96, 128,
                            128, F(20), nullptr, F(21), F(22), F(23), F(24), F(25), F(26), (void*)P(27),
                            1000, nullptr) == KDA_ERR_WORKSPACE);
        // packed batches: one forward, one backward over every chunk
        n_recs = 0;
        const size_t wp = kda_chunk_bwd_workspace_bytes(4, 5000, 96, 128, 128, 1);
        CHECK(kda_chunk_bwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), nullptr, (const int32_t*)P(28), 4,
                            5000, 96, 128, 128, F(20), nullptr, F(21), F(22), F(23), F(24), F(25), F(26),
                            (void*)P(27), wp, kMain) == KDA_OK);
        check_fork_join();
        Rec L[8];
        CHECK(launches(L, 8) == 3 && L[0].kind == 't' && L[0].win_len == 0 && L[0].slots == 5000 / 32 + 4 &&
              L[1].kind == 'f' && L[1].seg_sel < 0 && L[1].stores && L[2].kind == 'g' &&
              L[2].win_len == 0 && L[2].slots == 5000 / 32 + 4);
        CHECK(kda_chunk_bwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), nullptr, (const int32_t*)P(28), 4,
                            5000, 96, 128, 128, F(20), nullptr, F(21), F(22), F(23), F(24), F(25), F(26),
                            (void*)P(27), wp - 1, nullptr) == KDA_ERR_WORKSPACE);
        // a forward launch that fails while a chunk-matrix pass is on the
        // second stream: the call reports KDA_ERR_HIP and joins that stream
        // back into the caller's before it returns (windowed: the first
        // window-start pass, and the storing forward of the third window
        // from the end; packed: its one forward)
        for (int at : {1, 5}) {
            n_recs = 0;
            fail_fwd_in = at;
            CHECK(kda_chunk_bwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), nullptr, nullptr, 1, 8192, 96,
                                128, 128, F(20), nullptr, F(21), F(22), F(23), F(24), F(25), F(26),
                                (void*)P(27), ws, kMain) == KDA_ERR_HIP);
            CHECK(fail_fwd_in == 0 && n_recs > 0 && recs[n_recs - 1].kind == 'w' &&
                  recs[n_recs - 1].stream == kMain);
            check_fork_join();
        }
        n_recs = 0;
        fail_fwd_in = 1;
        CHECK(kda_chunk_bwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), nullptr, (const int32_t*)P(28), 4,
                            5000, 96, 128, 128, F(20), nullptr, F(21), F(22), F(23), F(24), F(25), F(26),
                            (void*)P(27), wp, kMain) == KDA_ERR_HIP);
        CHECK(fail_fwd_in == 0 && n_recs > 0 && recs[n_recs - 1].kind == 'w' &&
              recs[n_recs - 1].stream == kMain);
        check_fork_join();
        fail_fwd_in = -1;
    }
    // one second stream and two events for the whole process
    CHECK(n_streams == 1 && n_events == 2);
    for (int s = -1; s <= 9; ++s) CHECK(kda_status_str(s) != nullptr);
    CHECK(kda_abi_version() == KDA_ABI_VERSION);
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("ABI sanitizer driver: all checks passed (%d launches planned)\n", n_launch);
    return 0;
}
