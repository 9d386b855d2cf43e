// Sanitizer driver for the C ABI's host code (gated_delta_rule_amd/csrc/
// kda_abi.hip compiled as plain C++ with g++ and -fsanitize=address,undefined
// by tests/test_sanitizers.py; CPU only).  The kernel launchers are replaced
// by stubs that record what they were asked to launch and touch no memory,
// so every validation branch and every launch plan (packed batches, equal
// lengths, the sequence-parallel path, decode, recurrent, layer steps,
// backward) runs under the sanitizers without a GPU.  The pointers are fake
// device addresses that are never dereferenced.
#include <stdint.h>
#include <stdio.h>

#include "kda.h"
#include "kda_launch.h"

namespace {
int n_launch = 0, n_merge = 0, n_dual = 0, last_slices = 0, last_units = 0;
int fails = 0;
// forward and backward launches in order, for the backward's window plan
struct Rec {
    char kind;                 // 'f' forward, 'b' backward passes
    int seg_sel, win_idx;
    bool stores;               // forward keeps per-chunk values
    const float *S0, *S_T, *dS_T;
    float* dS0;
    int64_t seg_len, win_len, slots;
};
Rec recs[256];
int n_recs = 0;
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
hipError_t launch_chunk_fwd(const PrefillParams& p, bool, int wcols, bool, hipStream_t) {
    ++n_launch;
    if (n_recs < 256)
        recs[n_recs++] = Rec{'f', p.seg_sel, 0, p.h_states != nullptr, p.S0, p.S_T, nullptr, nullptr,
                             p.seg_len, 0, 0};
    CHECK(p.seg_sel < 0 || (!p.cu && p.seg_len % 32 == 0 && p.seg_len > 0));
    CHECK(!p.h_states || (p.r_out && p.u_out && !p.o));
    last_slices = p.n_slices;
    last_units = p.n_units;
    CHECK(wcols * 4 * p.n_slices == 128);
    CHECK(p.n_units == p.n_seqs * p.H);
    return hipSuccess;
}
hipError_t launch_chunk_fwd_dual(const PrefillParams& p, bool, hipStream_t) {
    ++n_launch;
    ++n_dual;
    CHECK(p.n_slices == 1 && p.S_T && p.S_T2 && !p.o);
    CHECK(p.n_units == p.n_seqs * p.H && p.n_units >= 256);
    return hipSuccess;
}
hipError_t launch_segment_merge(const float*, const float*, const float*, float*, float*, int32_t B,
                                int32_t P, int32_t H, hipStream_t) {
    ++n_merge;
    CHECK(B >= 1 && P >= 2 && H >= 1);
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
hipError_t launch_chunk_bwd(const BwdParams& p, bool, hipStream_t) {
    ++n_launch;
    CHECK(p.slots >= 1);
    CHECK(p.win_len == 0 || (!p.cu && p.win_len % 32 == 0 && p.slots * 32 == p.n_seqs * p.win_len));
    if (n_recs < 256)
        recs[n_recs++] = Rec{'b', -1, p.win_idx, false, nullptr, nullptr, p.dS_T, p.dS0, 0,
                             p.win_len, p.slots};
    return hipSuccess;
}
}  // namespace kda

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
    // sequence-parallel path with 256 segment chains: one launch for both
    // chains of every segment, the merge, the rerun
    {
        const size_t ws = kda_chunk_fwd_workspace_bytes(1, 1 << 20, 16, 128, 128, 0);
        CHECK(ws == (size_t)3 * 16 * 16 * 65536);
        const int before = n_launch, mb = n_merge, db = n_dual;
        CHECK(kda_chunk_fwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), nullptr, nullptr, 1, 1 << 20, 16,
                            128, 128, F(5), F(6), (void*)P(9), ws, nullptr) == KDA_OK);
        CHECK(n_launch - before == 2 && n_merge - mb == 1 && n_dual - db == 1);
    }
    // ... and with fewer chains (two workgroups per chain): the two chains
    // as separate launches
    {
        const size_t ws = kda_chunk_fwd_workspace_bytes(2, 6000, 3, 128, 128, 0);
        CHECK(ws == (size_t)3 * 2 * 2 * 3 * 65536);
        const int before = n_launch, mb = n_merge, db = n_dual;
        CHECK(kda_chunk_fwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), nullptr, nullptr, 2, 6000, 3,
                            128, 128, F(5), F(6), (void*)P(9), ws, nullptr) == KDA_OK);
        CHECK(n_launch - before == 3 && n_merge - mb == 1 && n_dual == db);
    }
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
    auto bwd_plan = [&](int n_seqs, int64_t T, size_t ws, const float* S0, const float* gST,
                        float* gS0, int expect_windows, int64_t expect_win_len) {
        n_recs = 0;
        CHECK(kda_chunk_bwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), S0, nullptr, n_seqs, T, 96, 128,
                            128, F(20), gST, F(21), F(22), F(23), F(24), F(25), gS0, (void*)P(27), ws,
                            nullptr) == KDA_OK);
        const int K = expect_windows;
        CHECK(n_recs == (K - 1) + 2 * K);
        if (n_recs != (K - 1) + 2 * K) return;
        // the states at the window starts: forward over windows 0 .. K-2
        const float* prev_end = nullptr;
        for (int w = 0; w + 1 < K; ++w) {
            const Rec& r = recs[w];
            CHECK(r.kind == 'f' && r.seg_sel == w && !r.stores && r.S_T && r.seg_len == expect_win_len);
            CHECK(w == 0 ? r.S0 == S0 : r.S0 == prev_end);
            prev_end = r.S_T;
        }
        // then per window, last first: forward keeping values, backward passes
        const float* carry = nullptr;
        for (int i = 0; i < K; ++i) {
            const int w = K - 1 - i;
            const Rec& f = recs[K - 1 + 2 * i];
            const Rec& b = recs[K + 2 * i];
            CHECK(f.kind == 'f' && f.seg_sel == w && f.stores && f.seg_len == expect_win_len);
            CHECK(w == 0 ? f.S0 == S0 : f.S0 == recs[w - 1].S_T);
            CHECK(b.kind == 'b' && b.win_idx == w && b.win_len == expect_win_len);
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
                            (void*)P(27), wp, nullptr) == KDA_OK);
        CHECK(n_recs == 2 && recs[0].kind == 'f' && recs[0].seg_sel < 0 && recs[0].stores &&
              recs[1].kind == 'b' && recs[1].win_len == 0 && recs[1].slots == 5000 / 32 + 4);
        CHECK(kda_chunk_bwd(P(0), P(1), P(2), KDA_BF16, F(3), F(4), nullptr, (const int32_t*)P(28), 4,
                            5000, 96, 128, 128, F(20), nullptr, F(21), F(22), F(23), F(24), F(25), F(26),
                            (void*)P(27), wp - 1, nullptr) == KDA_ERR_WORKSPACE);
    }
    for (int s = -1; s <= 9; ++s) CHECK(kda_status_str(s) != nullptr);
    CHECK(kda_abi_version() == KDA_ABI_VERSION);
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("ABI sanitizer driver: all checks passed (%d launches planned)\n", n_launch);
    return 0;
}
